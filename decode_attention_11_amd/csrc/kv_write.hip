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
#include <cmath>
#include <cstdint>

#include "mla_decode.h"
#include "mla_device.h"

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

// ---- FP8 cache: rows quantised to E4M3 on the way in.
//
// Each bf16 value is divided by the cache scale in fp32 (HIP's default fp32
// division is correctly rounded) and replaced by the nearest E4M3 code,
// ties to the even code; magnitudes from 448 up (infinities too) saturate to
// +-448, NaN becomes 0x7F.  The encoding is done on the fp32 bits: below
// 2^-6 the code counts 2^-9 steps (rint: half to even); above, adding
// 0x7FFFF plus the lowest kept bit to the magnitude's bits rounds the 23-bit
// mantissa to 3 bits half to even, a carry moving into the exponent, and the
// exponent is rebiased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80;
  const float ax = __builtin_fabsf(x);
  if (!(ax == ax)) return 0x7F;
  if (ax >= 448.f) return sign | 0x7E;
  if (ax < 0.015625f) return sign | (uint32_t)__builtin_rintf(ax * 512.f);
  const uint32_t a = __builtin_bit_cast(uint32_t, ax);
  const uint32_t r = a + 0x7FFFF + ((a >> 20) & 1);
  return sign | ((((r >> 23) - 120) << 3) | ((r >> 20) & 7));
}

constexpr int kCodeChunks = MLA_D_QK / 16;  // 16-code chunks per row

struct KvWriteF8Args {
  const uint4* rows;    // [n, 72] chunks of 8 bf16 values
  const int64_t* slots; // [n]
  uint4* cache;         // [num_blocks * block_size, 36] chunks of 16 codes
  int64_t n_rows;
  int64_t cache_rows;
  float scale;
};

// one thread per 16 values: 32 bytes in, 16 bytes out
__global__ __launch_bounds__(256) void kv_write_fp8_kernel(KvWriteF8Args a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / kCodeChunks;
  if (row >= a.n_rows) return;
  const int c = (int)(idx - row * kCodeChunks);
  const int64_t slot = a.slots[row];
  if (slot < 0 || slot >= a.cache_rows) return;
  const uint4 v0 = a.rows[row * kChunks + 2 * c], v1 = a.rows[row * kChunks + 2 * c + 1];
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) << 16;  // bf16 -> fp32, exact
    out[e >> 2] |= e4m3_code(__builtin_bit_cast(float, bits) / a.scale) << (8 * (e & 3));
  }
  a.cache[slot * kCodeChunks + c] = uint4{out[0], out[1], out[2], out[3]};
}

}  // namespace

extern "C" int mla_kv_write_fp8(const void* kv_new, const int64_t* slots, int64_t n_rows, float kv_scale,
                                void* kv_cache, int num_blocks, int block_size, hipStream_t stream) {
  if (n_rows < 0 || num_blocks < 1 || block_size < 1 || !(std::isfinite(kv_scale) && kv_scale > 0.f))
    return MLA_ERR_INVALID_ARG;
  if (n_rows == 0) return MLA_OK;
  if (!kv_new || !slots || !kv_cache) return MLA_ERR_INVALID_ARG;
  // rows are read and written as 16-byte chunks
  if ((reinterpret_cast<uintptr_t>(kv_new) | reinterpret_cast<uintptr_t>(kv_cache)) & 15) return MLA_ERR_INVALID_ARG;
  if (n_rows > (int64_t(1) << 40)) return MLA_ERR_INVALID_ARG;
  const int64_t blocks = (n_rows * kCodeChunks + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MLA_ERR_INVALID_ARG;
  KvWriteF8Args a{static_cast<const uint4*>(kv_new), slots, static_cast<uint4*>(kv_cache), n_rows,
                  (int64_t)num_blocks * block_size, kv_scale};
  if (mla::launch(kv_write_fp8_kernel, dim3((unsigned)blocks), dim3(256), stream, a) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

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
  if (mla::launch(kv_write_kernel, dim3((unsigned)blocks), dim3(256), stream, a) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}
