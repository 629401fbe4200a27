// Device-side helpers shared by the gfx950 kernels of libmla_decode.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int D_QK = 576;
constexpr int D_V = 512;
constexpr int ROW_BYTES = D_QK * 2;  // one latent KV row / one query head: 1152 bytes
constexpr float NEG_INF = -__builtin_inff();
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// floor(x / d) for x >= 0, d >= 1.  Below 2^52 one correctly rounded double
// division gives it exactly: x/d is either an integer (then representable) or
// at least 1/d from the next integer, while the rounded quotient is within
// 2^-53 * x/d of it, and x < 2^53 keeps that below 1/d.  Larger values take
// the 64-bit integer division (a long instruction sequence on the GPU).
__device__ __forceinline__ int64_t floordiv(int64_t x, int64_t d) {
  constexpr int64_t kExact = int64_t(1) << 52;
  if (x < kExact && d < kExact) return (int64_t)((double)x / (double)d);
  return x / d;
}

// Two floats to packed bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}

__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  return __builtin_convertvector(v, bf16x4);
}

// acc + the sum of the 8 bf16 values (v_dot2c_f32_bf16 against ones, fp32
// accumulation): the denominator that matches P as the P*V product sees it.
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), ones, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), ones, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), ones, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), ones, acc, false);
  return acc;
}

typedef __attribute__((address_space(1))) const bf16x8 global_bf16x8;
typedef __attribute__((address_space(1))) const int32_t global_i32;

// 16-byte load through the global address space (global_load_dwordx4; a
// generic pointer would become a flat load, which also counts against the
// LDS wait counter).
__device__ __forceinline__ bf16x8 gload_bf16x8(const uint8_t* p) {
  return *(global_bf16x8*)(p);
}

__device__ __forceinline__ int32_t gload_i32(const int32_t* p) {
  return *(global_i32*)(p);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

// Rank-local visible key count of query row j of a request: causal rows see
// the global prefix G = tot - (q_len-1-j); positions go to the ranks in
// segments of I (segment k to rank k mod W), so rank r holds
// (G / (I*W))*I + min(max(G % (I*W) - r*I, 0), I) of them (with I = 1:
// ceil(max(G - r, 0) / W)), capped by its local length (PR #52188 page, key
// source snippets: the per-row prefix and the rank-local length).
// Non-causal rows see the whole local length.
__device__ __forceinline__ int row_bound(int seq, int tot, int q_len, int j, int W, int r, int I, int causal) {
  if (seq < 0) seq = 0;
  if (!causal) return seq;
  int64_t g = (int64_t)tot - (q_len - 1 - j);
  if (g < 0) g = 0;
  const int64_t span = (int64_t)I * W;
  const int64_t rounds = floordiv(g, span);
  int64_t rem = g - rounds * span - (int64_t)r * I;
  rem = rem < 0 ? 0 : (rem > I ? I : rem);
  const int64_t n = rounds * I + rem;
  return n < seq ? (int)n : seq;
}

// The lane's index in its wave, computed afresh from the execution mask
// (two instructions).  Code that runs once per piece, between long loops
// that need every register, takes it from here: a lane index or anything
// derived from it that is kept across such a loop is spilled, and each
// reload waits for all vector-memory operations in flight.  The opaque zero
// keeps the compiler from hoisting the computation out of the loop.
__device__ __forceinline__ int lane_id_fresh() {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, z));
}

// Lane shuffles whose source lane is derived from lane_id_fresh() at the
// point of use (ds_bpermute reads lane addr/4 of its source).
__device__ __forceinline__ float shfl_xor_fresh(float x, int off) {
  const int src = lane_id_fresh() ^ off;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}
__device__ __forceinline__ int64_t shfl_i64(int64_t v, int src) {
  const int lo = __builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)v);
  const int hi = __builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Work ranges: T units are cut into G ranges, the first G/2 of weight wa
// and the rest of weight wb (wa = wb: equal ranges).  Range w starts at
// floor(T * W(w) / Wt), with W(w) = wa min(w, G/2) + wb max(w - G/2, 0) and
// Wt = W(G).  All in 64-bit integers: T * Wt stays far below 2^63.
__device__ __forceinline__ int64_t range_weight(int64_t w, int G, int wa, int wb) {
  const int64_t h = G / 2;
  return w <= h ? wa * w : wa * h + wb * (w - h);
}
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t T, int G, int wa, int wb) {
  return floordiv(T * range_weight(w, G, wa, wb), range_weight(G, G, wa, wb));
}

// The range that holds unit u (0 <= u < T): the largest w whose start is at
// most u.  start(w) <= u  <=>  T W(w) <= (u + 1) Wt - 1  <=>  W(w) <= Wmax.
__device__ __forceinline__ int range_owner(int64_t u, int64_t T, int G, int wa, int wb) {
  const int64_t wmax = floordiv((u + 1) * range_weight(G, G, wa, wb) - 1, T);
  const int64_t h = G / 2;
  const int64_t w = wmax <= wa * h ? wmax / wa : h + (wmax - wa * h) / wb;
  return (int)(w < G - 1 ? w : G - 1);
}

// Whether range w holds any unit: with fewer units than ranges some are empty
// (and can lie between the owners of two units).
__device__ __forceinline__ bool range_nonempty(int w, int64_t T, int G, int wa, int wb) {
  return range_start(w, T, G, wa, wb) < range_start(w + 1, T, G, wa, wb);
}

// Launch a kernel that takes one argument struct and return the runtime's
// status for this launch itself (hipGetLastError would also report a
// sticky error left behind by earlier, unrelated work).  With events given,
// the runtime records them at the kernel's own start and end.
template <class A>
inline hipError_t launch(void (*kernel)(A), dim3 grid, dim3 block, hipStream_t stream, A& args,
                         hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
  void* argv[] = {&args};
  if (start != nullptr)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream, start, stop, 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
}

}  // namespace mla
