// LSE-weighted merge of partial attention results (one per rank's shard), gfx950.
//
// The pages require the cross-rank merge of (out, lse) pairs and that the
// LSE bases agree before merging (PR #54012 page, implementation breakdown;
// PR #48180 page, implementation breakdown) but do not print the formula;
// this is the standard log-sum-exp combine stated in include/mla_decode.h.
// Bandwidth-bound: each (row, head) item reads n_parts x (1 KiB + 4 B) and
// writes 1 KiB + 4 B.  One wave per item, 8 output columns per lane with
// 16-byte loads and stores.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "mla_decode.h"
#include "mla_device.h"

using namespace mla;

namespace {

constexpr int kMaxParts = 64;

struct MergeArgs {
  const uint16_t* part[kMaxParts];
  const float* lse_in[kMaxParts];
  int n_parts;
  int64_t items;   // rows * H
  float to_log2;   // 1/ln2 for base e, 1 for base 2
  float from_log2; // ln2 for base e, 1 for base 2
  uint16_t* out;
  float* lse;
};

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.items) return;
  // every lane reads all the LSEs of its item (they are in cache after the first)
  float M = NEG_INF;
  for (int i = 0; i < a.n_parts; ++i) M = fmaxf(M, a.lse_in[i][item] * a.to_log2);
  uint16_t* op = a.out + item * D_V + lane * 8;
  if (M == NEG_INF) {
    *reinterpret_cast<uint4*>(op) = uint4{0u, 0u, 0u, 0u};
    if (a.lse && lane == 0) a.lse[item] = NEG_INF;
    return;
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int i = 0; i < a.n_parts; ++i) {
    const float li = a.lse_in[i][item] * a.to_log2;
    const float w = (li == NEG_INF) ? 0.f : fast_exp2(li - M);
    wsum += w;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(a.part[i] + item * D_V + lane * 8);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += w * (float)v[c];
  }
  const float inv = 1.f / wsum;
  bf16x8 r;
#pragma unroll
  for (int c = 0; c < 8; c += 2) {
    const bf16x2 pr = to_bf16x2(acc[c] * inv, acc[c + 1] * inv);
    r[c] = pr[0];
    r[c + 1] = pr[1];
  }
  *reinterpret_cast<bf16x8*>(op) = r;
  if (a.lse && lane == 0) a.lse[item] = (M + __log2f(wsum)) * a.from_log2;
}

}  // namespace

extern "C" int mla_merge_lse(const void* const* partials, const float* const* lses, int n_parts,
                             int rows, int H, int lse_base, void* out, float* lse, hipStream_t stream) {
  if (n_parts < 1 || n_parts > kMaxParts || rows < 0 || H < 1 ||
      (lse_base != MLA_LSE_BASE_E && lse_base != MLA_LSE_BASE_2) || !partials || !lses)
    return MLA_ERR_INVALID_ARG;
  if (rows == 0) return MLA_OK;
  if (!out) return MLA_ERR_INVALID_ARG;
  MergeArgs a{};
  for (int i = 0; i < n_parts; ++i) {
    if (!partials[i] || !lses[i]) return MLA_ERR_INVALID_ARG;
    a.part[i] = static_cast<const uint16_t*>(partials[i]);
    a.lse_in[i] = lses[i];
  }
  a.n_parts = n_parts;
  a.items = (int64_t)rows * H;
  a.to_log2 = (lse_base == MLA_LSE_BASE_E) ? LOG2E : 1.f;
  a.from_log2 = (lse_base == MLA_LSE_BASE_E) ? LN2 : 1.f;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  const int64_t blocks = (a.items + 3) / 4;
  if (blocks > 0x7FFFFFFF) return MLA_ERR_INVALID_ARG;
  if (launch(merge_kernel, dim3((unsigned)blocks), dim3(256), stream, a) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}
