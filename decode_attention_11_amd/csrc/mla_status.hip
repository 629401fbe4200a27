// Status strings of the C ABI.
#include "mla_decode.h"

extern "C" const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}
