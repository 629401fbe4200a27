// A bare bf16 MFMA loop: the achievable matrix rate of this GPU, against
// which the attention kernels' rates are reported beside the published peak.
// Not part of the decode path.
#include "mla_decode.h"
#include "mla_device.h"

using namespace mla;

namespace {

// Four independent accumulation chains per wave (v_mfma_f32_32x32x16_bf16 on
// operands of ones: each MFMA adds 16 to every accumulator element), so the
// matrix pipe never waits on a result.  Thread t writes the sum of its four
// chains' first elements, 64 * iters.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)1.0f;
    b[i] = (__bf16)1.0f;
  }
  asm volatile("" : "+v"(a), "+v"(b));
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = c0[0] + c1[0] + c2[0] + c3[0];
}

}  // namespace

extern "C" int mla_probe_mfma(int workgroups, int iters, float* out, hipStream_t stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 20) || out == nullptr)
    return MLA_ERR_INVALID_ARG;
  int a_iters = iters;
  float* a_out = out;
  void* argv[] = {&a_iters, &a_out};
  if (hipLaunchKernel(reinterpret_cast<const void*>(mfma_loop_kernel), dim3(workgroups), dim3(256), argv, 0,
                      stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}
