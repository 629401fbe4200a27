// Paged latent-KV write at rank-local slots, gfx950.
//
// Stores new 576-wide bf16 KV rows at the slots cp_local_slot gave their
// positions and writes nothing for the pad slot: under decode context
// parallelism a rank must not touch the slots other ranks own (PR #52188
// page, key source snippets, cp_local_slot, and risks).  Slot s is row
// s % block_size of block s / block_size; with the cache laid out
// [num_blocks, block_size, 576] that is simply cache row s.  Slots that are
// negative or past the cache write nothing, so no input can make the kernel
// store outside the cache.
//
// Bandwidth-bound copy: each 1152-byte row is 72 chunks of 16 bytes; a
// thread moves one chunk.  The row's slot is read by the 72 threads of the
// row (one cache line, served from L1/L2 after the first).
#include <hip/hip_runtime.h>
#include <cstdint>

#include "mla_decode.h"

namespace {

constexpr int kChunks = MLA_D_QK * 2 / 16;  // 16-byte chunks per row

struct KvWriteArgs {
  const uint4* rows;    // [n, 72] chunks
  const int64_t* slots; // [n]
  uint4* cache;         // [num_blocks * block_size, 72] chunks
  int64_t n_rows;
  int64_t cache_rows;
};

__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / kChunks;
  if (row >= a.n_rows) return;
  const int c = (int)(idx - row * kChunks);
  const int64_t slot = a.slots[row];
  if (slot < 0 || slot >= a.cache_rows) return;
  a.cache[slot * kChunks + c] = a.rows[row * kChunks + c];
}

}  // namespace

extern "C" int mla_kv_write(const void* kv_new, const int64_t* slots, int64_t n_rows, void* kv_cache,
                            int num_blocks, int block_size, hipStream_t stream) {
  if (n_rows < 0 || num_blocks < 1 || block_size < 1) return MLA_ERR_INVALID_ARG;
  if (n_rows == 0) return MLA_OK;
  if (!kv_new || !slots || !kv_cache) return MLA_ERR_INVALID_ARG;
  // rows move as 16-byte chunks
  if ((reinterpret_cast<uintptr_t>(kv_new) | reinterpret_cast<uintptr_t>(kv_cache)) & 15) return MLA_ERR_INVALID_ARG;
  const int64_t threads = n_rows * kChunks;
  if (n_rows > (int64_t(1) << 40)) return MLA_ERR_INVALID_ARG;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MLA_ERR_INVALID_ARG;
  KvWriteArgs a{static_cast<const uint4*>(kv_new), slots, static_cast<uint4*>(kv_cache), n_rows,
                (int64_t)num_blocks * block_size};
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}
