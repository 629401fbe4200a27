// Paged absorbed-MLA decode for gfx950: plan, partial attention, split combine.
//
// What one call computes is stated in include/mla_decode.h (per-row causal
// bounds from the global lengths, round-robin rank-local keys, softmax over
// 576-wide scores, 512-wide values, LSE in base e or 2).
//
// Work decomposition.  The rows of request b are its q_len*H (query token,
// head) pairs, row = j*H + h, cut into row tiles.  Each (request, row tile)
// group must attend to n_b keys, n_b being the bound of its last query row.
// All groups' keys are laid end to end (units ordered by request, row tile,
// key) and cut into G equal ranges, one per workgroup, so every CU gets the
// same number of keys whatever the length mix (a balanced split-KV).  A
// range that crosses group boundaries is processed as several pieces.  Each
// piece writes an fp32 partial (unnormalised O^T, running max in log2 units,
// softmax denominator) to the workspace; a combine kernel merges the pieces
// of each group and writes bf16 out and the LSE.  The idea of splitting keys
// across workgroups with a workspace is the split-KV of the trtllm-gen path
// (PR #54012 page, implementation breakdown: the non-DCP call keeps its
// multi-CTA KV counter buffer); the balanced range split is this library's.
//
// Kernel family R16 (this file): 16 rows per tile; four waves of a
// workgroup take turns over 16-key subtiles of the piece, each keeping its
// own online-softmax state for the 16 rows, and the four states are merged
// in LDS at the end of the piece.  Scores are S^T = K * Q^T on
// v_mfma_f32_16x16x32_bf16 (K rows as the A operand straight from HBM into
// registers, Q^T resident in registers), so each lane holds 4 keys of one
// row; P*V is O^T += V^T * P^T on v_mfma_f32_16x16x16_bf16 with V^T read
// from LDS by ds_read_b64_tr_b16, so P never leaves registers and each lane
// owns one row of O^T.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "mla_decode.h"
#include "mla_device.h"

using namespace mla;

namespace {

struct DecodeArgs {
  const uint8_t* q;        // bf16 [B, Q, H, 576]
  const uint8_t* kv;       // bf16 [num_blocks, bs, 576]
  const int32_t* bt;       // [B, max_blocks]
  const int32_t* seq_lens; // [B]
  const int32_t* glob;     // [B] or null
  int B, Q, H, R;          // R = Q*H rows per request
  int num_blocks, bs, max_blocks;
  int W, rank, causal;
  float scale_log2;        // softmax scale times log2(e)
  int lse_base;
  int n_rt;                // row tiles per request
  int G;                   // partial workgroups
  int64_t* prefix;         // [B+1] unit offsets of the requests
  float* partials;         // [G + B*n_rt] slots
  uint16_t* out;           // bf16 [B*R, 512]
  float* lse;              // [B*R] or null
};

__device__ __forceinline__ int request_tot(const DecodeArgs& a, int b, int seq) {
  return a.glob ? a.glob[b] : seq;
}

// Keys of the largest row of request b (row j = q_len-1 has the longest prefix).
__device__ __forceinline__ int request_keys(const DecodeArgs& a, int b) {
  int seq = a.seq_lens[b];
  return row_bound(seq, request_tot(a, b, seq), a.Q, a.Q - 1, a.W, a.rank, a.causal);
}

// ---------------------------------------------------------------- plan
// prefix[b] = sum over earlier requests of n_rt * keys: one block-wide scan.
__global__ __launch_bounds__(256) void plan_kernel(DecodeArgs a) {
  __shared__ int64_t wsum[4];
  __shared__ int64_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { carry = 0; a.prefix[0] = 0; }
  __syncthreads();
  for (int base = 0; base < a.B; base += 256) {
    const int b = base + tid;
    int64_t v = (b < a.B) ? (int64_t)a.n_rt * request_keys(a, b) : 0;
    for (int off = 1; off < 64; off <<= 1) {
      int64_t y = __shfl_up(v, off, 64);
      if (lane >= off) v += y;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int64_t add = carry;
    for (int w = 0; w < wave; ++w) add += wsum[w];
    if (b < a.B) a.prefix[b + 1] = add + v;
    __syncthreads();
    if (tid == 255) carry = add + v;
    __syncthreads();
  }
}

// ---------------------------------------------------------------- R16 partial
constexpr int R16_ROWS = 16;
constexpr int R16_SUB = 16;          // keys per subtile
constexpr int R16_VROW = 1056;       // LDS bytes per key row of a V stage (1024 + 32 pad)
constexpr int R16_VSTAGE = R16_SUB * R16_VROW;
constexpr int R16_MRG_LD = 17;       // padded row stride of the LDS merge buffer [dv][row]
constexpr int R16_SLOT = R16_ROWS * D_V + 2 * R16_ROWS;  // floats per partial slot
constexpr int R16_SMEM = 4 * R16_VSTAGE;                 // V stages; the merge buffer aliases them

static_assert(D_V * R16_MRG_LD * 4 <= R16_SMEM, "merge buffer must fit in the V stages");

struct R16Piece {
  int b, rt, k0, k1;
};

// Loads the 16 keys of one subtile as MFMA A-operand fragments: lane (li, g)
// gets key k0 + 16*s + li, 16-byte chunks 4*kk + g of its 576-wide row.
__device__ __forceinline__ void r16_load(bf16x8 (&kb)[18], const DecodeArgs& a, const int32_t* btr,
                                         int k0, int k1, int nsub, int s, int li, int g) {
  const int t = k0 + R16_SUB * s + li;
  bool valid = (s < nsub) && (t < k1);
  const uint8_t* rowp = nullptr;
  if (valid) {
    const int vb = t / a.bs;
    const int blk = (vb < a.max_blocks) ? btr[vb] : -1;
    valid = (unsigned)blk < (unsigned)a.num_blocks;
    rowp = a.kv + ((int64_t)blk * a.bs + (t - vb * a.bs)) * ROW_BYTES;
  }
  if (valid) {
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) kb[kk] = load_bf16x8(rowp + (4 * kk + g) * 16);
  } else {
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) kb[kk] = zero_bf16x8();
  }
}

__device__ __forceinline__ void r16_compute(const bf16x8 (&kb)[18], const bf16x8 (&qf)[18], f32x4 (&o)[32],
                                            float& m, float& l, uint8_t* vs, float scale_log2,
                                            int kbase, int k1, int nrow, int li, int g) {
  // S^T[t][row] for the 16 keys of the subtile: lane holds t = 4g+i, row = li.
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 18; kk += 2) {
    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk], qf[kk], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk + 1], qf[kk + 1], sb, 0, 0, 0);
  }
  // the V part (first 512 columns) of this subtile goes to LDS for the transposed read
#pragma unroll
  for (int kk = 0; kk < 16; ++kk)
    *reinterpret_cast<bf16x8*>(vs + li * R16_VROW + (4 * kk + g) * 16) = kb[kk];

  float p[4];
  float mx = NEG_INF;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = kbase + 4 * g + i;
    float v = (sa[i] + sb[i]) * scale_log2;
    v = (t < k1 && t < nrow) ? v : NEG_INF;
    p[i] = v;
    mx = fmaxf(mx, v);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mnew = fmaxf(m, mx);
  float alpha = 1.f;
  if (mnew != NEG_INF) {
    alpha = fast_exp2(m - mnew);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(p[i] - mnew);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = 0.f;
  }
  float rs = (p[0] + p[1]) + (p[2] + p[3]);
  rs += __shfl_xor(rs, 16, 64);
  rs += __shfl_xor(rs, 32, 64);
  l = l * alpha + rs;
  m = mnew;
  const bf16x4 pf = to_bf16x4(p[0], p[1], p[2], p[3]);
  // O^T[dv][row] += V^T[dv][t] * P^T[t][row]; the tr read gives lane (li, g)
  // V[4g+e][16*mt+li] for e = 0..3 when lane (q, g) points at row 4g+q/4,
  // columns 16*mt + 4*(q%4).
  const uint8_t* vread = vs + (4 * g + (li >> 2)) * R16_VROW + (li & 3) * 8;
#pragma unroll
  for (int mt = 0; mt < 32; ++mt) {
    o[mt] *= alpha;
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(vread + mt * 32));
    o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, v), pf, o[mt], 0, 0, 0);
  }
}

__global__ __launch_bounds__(256, 1) void attn_r16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[R16_SMEM];
  __shared__ float mrg_m[4][R16_ROWS];
  __shared__ float mrg_l[R16_ROWS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int64_t T = a.prefix[a.B];
  const int w = blockIdx.x;
  int64_t u = (int64_t)w * T / a.G;
  const int64_t uend = (int64_t)(w + 1) * T / a.G;
  if (u >= uend) return;

  // request holding unit u: the largest b with prefix[b] <= u
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.prefix[mid] <= u) lo = mid; else hi = mid;
  }
  int b = lo;
  uint8_t* vs = smem + wave * R16_VSTAGE;
  float* mrg_o = reinterpret_cast<float*>(smem);

  while (u < uend) {
    const int64_t pb = a.prefix[b], pb1 = a.prefix[b + 1];
    if (pb1 <= u) { ++b; continue; }
    const int nb = (int)((pb1 - pb) / a.n_rt);
    const int rt = (int)((u - pb) / nb);
    const int k0 = (int)((u - pb) - (int64_t)rt * nb);
    const int64_t left = uend - u;
    const int k1 = (int)((int64_t)(nb - k0) < left ? nb : k0 + left);

    // this lane's row (as the S^T / O^T column)
    const int my_row = rt * R16_ROWS + li;
    const bool row_ok = my_row < a.R;
    const int seq = a.seq_lens[b];
    const int nrow = row_ok ? row_bound(seq, request_tot(a, b, seq), a.Q, my_row / a.H, a.W, a.rank, a.causal) : 0;

    bf16x8 qf[18];
    {
      const uint8_t* qrow = a.q + ((int64_t)b * a.R + (row_ok ? my_row : 0)) * ROW_BYTES;
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) qf[kk] = row_ok ? load_bf16x8(qrow + (4 * kk + g) * 16) : zero_bf16x8();
    }
    f32x4 o[32];
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = NEG_INF, l = 0.f;

    const int32_t* btr = a.bt + (int64_t)b * a.max_blocks;
    const int nsub = (k1 - k0 + R16_SUB - 1) / R16_SUB;
    bf16x8 kb0[18], kb1[18];
    r16_load(kb0, a, btr, k0, k1, nsub, wave, li, g);
    r16_load(kb1, a, btr, k0, k1, nsub, wave + 4, li, g);
    for (int s = wave; s < nsub; s += 8) {
      r16_compute(kb0, qf, o, m, l, vs, a.scale_log2, k0 + R16_SUB * s, k1, nrow, li, g);
      r16_load(kb0, a, btr, k0, k1, nsub, s + 8, li, g);
      if (s + 4 < nsub) {
        r16_compute(kb1, qf, o, m, l, vs, a.scale_log2, k0 + R16_SUB * (s + 4), k1, nrow, li, g);
        r16_load(kb1, a, btr, k0, k1, nsub, s + 12, li, g);
      }
    }

    // merge the four waves' states of the 16 rows in LDS, in a fixed wave
    // order so that the result does not depend on timing
    __syncthreads();
    if (g == 0) mrg_m[wave][li] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(mrg_m[0][li], mrg_m[1][li]), fmaxf(mrg_m[2][li], mrg_m[3][li]));
    const float f = (m == NEG_INF) ? 0.f : fast_exp2(m - M);
    for (int wv = 0; wv < 4; ++wv) {
      if (wave == wv) {
#pragma unroll
        for (int mt = 0; mt < 32; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* dst = &mrg_o[(16 * mt + 4 * g + i) * R16_MRG_LD + li];
            *dst = (wv == 0 ? 0.f : *dst) + o[mt][i] * f;
          }
        if (g == 0) mrg_l[li] = (wv == 0 ? 0.f : mrg_l[li]) + l * f;
      }
      __syncthreads();
    }
    const int slot = w + b * a.n_rt + rt;
    float* ps = a.partials + (int64_t)slot * R16_SLOT;
    for (int e = tid; e < D_V * R16_ROWS; e += 256)
      ps[e] = mrg_o[(e >> 4) * R16_MRG_LD + (e & 15)];
    if (tid < R16_ROWS) {
      const float Mt = fmaxf(fmaxf(mrg_m[0][tid], mrg_m[1][tid]), fmaxf(mrg_m[2][tid], mrg_m[3][tid]));
      ps[D_V * R16_ROWS + tid] = Mt;
      ps[D_V * R16_ROWS + R16_ROWS + tid] = mrg_l[tid];
    }
    __syncthreads();
    u += k1 - k0;
  }
}

// ---------------------------------------------------------------- combine
// One workgroup per (request, row tile): merge the partial slots of the
// workgroups that covered it, write bf16 out and the LSE.
template <int ROWS>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  constexpr int TPR = 256 / ROWS;          // threads per row
  constexpr int DV_PER = D_V / TPR;        // output columns per thread
  constexpr int SLOT = ROWS * D_V + 2 * ROWS;
  const int grp = blockIdx.x;
  const int b = grp / a.n_rt, rt = grp - b * a.n_rt;
  const int row = threadIdx.x % ROWS, part = threadIdx.x / ROWS;
  const int row_idx = rt * ROWS + row;
  if (row_idx >= a.R) return;
  const int64_t T = a.prefix[a.B];
  const int64_t pb = a.prefix[b], pb1 = a.prefix[b + 1];
  const int nb = (int)((pb1 - pb) / a.n_rt);
  int w0 = 0, w1 = -1;
  if (nb > 0) {
    const int64_t u0 = pb + (int64_t)rt * nb;
    w0 = range_owner(u0, T, a.G);
    w1 = range_owner(u0 + nb - 1, T, a.G);
  }
  float M = NEG_INF;
  for (int w = w0; w <= w1; ++w) {
    const float* ps = a.partials + (int64_t)(w + grp) * SLOT;
    M = fmaxf(M, ps[ROWS * D_V + row]);
  }
  const int64_t orow = (int64_t)b * a.R + row_idx;
  uint16_t* op = a.out + orow * D_V;
  if (M == NEG_INF) {
    for (int c = 0; c < DV_PER; c += 8) {
      uint4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<uint4*>(op + part * DV_PER + c) = z;
    }
    if (a.lse && part == 0) a.lse[orow] = NEG_INF;
    return;
  }
  float L = 0.f;
  for (int w = w0; w <= w1; ++w) {
    const float* ps = a.partials + (int64_t)(w + grp) * SLOT;
    const float mw = ps[ROWS * D_V + row];
    const float f = (mw == NEG_INF) ? 0.f : fast_exp2(mw - M);
    L += f * ps[ROWS * D_V + ROWS + row];
  }
  const float inv = 1.f / L;
  for (int c0 = 0; c0 < DV_PER; c0 += 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int w = w0; w <= w1; ++w) {
      const float* ps = a.partials + (int64_t)(w + grp) * SLOT;
      const float mw = ps[ROWS * D_V + row];
      const float f = (mw == NEG_INF) ? 0.f : fast_exp2(mw - M);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] += f * ps[(part * DV_PER + c0 + c) * ROWS + row];
    }
    bf16x8 r;
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
      const bf16x2 pr = to_bf16x2(acc[c] * inv, acc[c + 1] * inv);
      r[c] = pr[0];
      r[c + 1] = pr[1];
    }
    *reinterpret_cast<bf16x8*>(op + part * DV_PER + c0) = r;
  }
  if (a.lse && part == 0) {
    const float l2 = M + __log2f(L);
    a.lse[orow] = (a.lse_base == MLA_LSE_BASE_E) ? l2 * LN2 : l2;
  }
}

// ---------------------------------------------------------------- host side
struct Plan {
  int rows_tile;
  int n_rt;
  int G;
  size_t prefix_off, partial_off, bytes;
};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

Plan make_plan(int B, int q_len, int H, int max_seq_len, int cus) {
  Plan p{};
  const int64_t R = (int64_t)q_len * H;
  p.rows_tile = R16_ROWS;
  p.n_rt = (int)((R + p.rows_tile - 1) / p.rows_tile);
  const int64_t units = (int64_t)B * p.n_rt * (max_seq_len > 0 ? max_seq_len : 1);
  int64_t G = (units + 255) / 256;  // at least 256 keys per workgroup
  if (G > cus) G = cus;
  if (G < 1) G = 1;
  p.G = (int)G;
  const size_t slot = (size_t)(p.rows_tile * D_V + 2 * p.rows_tile) * sizeof(float);
  p.prefix_off = 0;
  p.partial_off = align_up((size_t)(B + 1) * sizeof(int64_t));
  p.bytes = p.partial_off + align_up(((size_t)p.G + (size_t)B * p.n_rt) * slot);
  return p;
}

thread_local hipEvent_t tl_prof_start = nullptr;
thread_local hipEvent_t tl_prof_stop = nullptr;

}  // namespace

extern "C" int mla_profile_attention_events(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return MLA_ERR_INVALID_ARG;
  tl_prof_start = start;
  tl_prof_stop = stop;
  return MLA_OK;
}

extern "C" size_t mla_decode_workspace_size(int B, int q_len, int H, int max_seq_len) {
  if (B <= 0 || q_len < 1 || H < 1 || max_seq_len < 0) return 0;
  return make_plan(B, q_len, H, max_seq_len, device_cu_count()).bytes;
}

extern "C" int mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                          const int32_t* seq_lens, const int32_t* causal_seqlens_global,
                          int B, int q_len, int H, int num_blocks, int block_size, int max_blocks,
                          int max_seq_len, int cp_world, int cp_rank, int causal, float scale,
                          int lse_base, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (B < 0 || q_len < 1 || H < 1 || num_blocks < 1 || block_size < 1 || max_blocks < 1 ||
      max_seq_len < 0 || cp_world < 1 || cp_rank < 0 || cp_rank >= cp_world ||
      (causal != 0 && causal != 1) || (lse_base != MLA_LSE_BASE_E && lse_base != MLA_LSE_BASE_2) ||
      !std::isfinite(scale))
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)q_len * H > (1 << 24)) return MLA_ERR_INVALID_ARG;
  if (causal && cp_world > 1 && causal_seqlens_global == nullptr) return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!q || !kv_cache || !block_table || !seq_lens || !out) return MLA_ERR_INVALID_ARG;
  const Plan p = make_plan(B, q_len, H, max_seq_len, device_cu_count());
  if (workspace_bytes < p.bytes || workspace == nullptr) return MLA_ERR_INVALID_ARG;

  DecodeArgs a{};
  a.q = static_cast<const uint8_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv_cache);
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.glob = causal_seqlens_global;
  a.B = B; a.Q = q_len; a.H = H; a.R = q_len * H;
  a.num_blocks = num_blocks; a.bs = block_size; a.max_blocks = max_blocks;
  a.W = cp_world; a.rank = cp_rank; a.causal = causal;
  a.scale_log2 = scale * LOG2E;
  a.lse_base = lse_base;
  a.n_rt = p.n_rt;
  a.G = p.G;
  a.prefix = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(workspace) + p.prefix_off);
  a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + p.partial_off);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;

  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, a);
  if (tl_prof_start) (void)hipEventRecord(tl_prof_start, stream);
  hipLaunchKernelGGL(attn_r16_kernel, dim3(p.G), dim3(256), 0, stream, a);
  if (tl_prof_stop) (void)hipEventRecord(tl_prof_stop, stream);
  hipLaunchKernelGGL(combine_kernel<R16_ROWS>, dim3(B * p.n_rt), dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}
