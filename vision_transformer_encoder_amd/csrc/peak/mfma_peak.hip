// Measurement probe, not part of the tower: dense MFMA issue rate of the
// two matrix instructions the tower's kernels use, v_mfma_f32_32x32x16_bf16
// (attention, bf16 GEMMs) and the FP8 v_mfma_f32_32x32x64_f8f6f4 (block-
// scaled GEMMs), on every compute unit at once.  The benchmark divides the
// FLOPs by the kernel's time to get the peak the chip reaches under load
// (its clock then), next to the published one.
//
// Each wave runs four independent accumulator chains (enough to cover the
// MFMA latency) for `iters` steps; two 256-thread workgroups per compute
// unit give two waves per SIMD.  The accumulators are summed into `out`
// (one float per thread) so that nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* __restrict__ out) {
  const int t = threadIdx.x;
  f32x16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16_t{};
  if constexpr (KIND == 0) {
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(float)((t + e) & 7);
      b[e] = (__bf16)(float)((t * 3 + e) & 7);
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
  } else {
    i32x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x38383838 + ((t + e) & 3);  // E4M3 values near 1
      b[e] = 0x30303030 + ((t * 3 + e) & 3);
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[blockIdx.x * 256 + t] = s;
}
}  // namespace

extern "C" {

// FLOPs one launch performs: 2 * M * N * K per MFMA, 4 MFMAs per step per
// wave, 4 waves per workgroup.
double vit_peak_mfma_flops(int kind, int iters, int workgroups) {
  const double per = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  return per * 4.0 * iters * 4.0 * workgroups;
}

// kind 0: bf16, 1: FP8.  out: workgroups * 256 floats of device memory.
// Returns a hipError_t value (0 on success).
int vit_peak_mfma(int kind, int iters, int workgroups, float* out, void* stream) {
  if ((kind != 0 && kind != 1) || iters < 1 || workgroups < 1 || !out) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    mfma_peak_kernel<0><<<workgroups, 256, 0, s>>>(iters, out);
  else
    mfma_peak_kernel<1><<<workgroups, 256, 0, s>>>(iters, out);
  return (int)hipGetLastError();
}

}  // extern "C"
