// 2D rotate_half rotary embedding of Q and K, in place (FlashRT
// "Qwen3-VL-8B on RTX 5090" page, section 3: "2D rotate_half RoPE", kernel
// rope_neox_qk_bf16; spark_model "layers/vision_encoder.rs" page: head_dim/4
// inverse frequencies).  Per head: dims [0, hd/2) rotate by the patch row,
// dims [hd/2, hd) by the patch column; inside each half, dims i and i+hd/4
// form a pair turned by angle p * theta^(-2i/(hd/2)).
//
// HBM-bound (read + write of Q and K).  A 256-thread workgroup handles 4
// tokens: it first evaluates the 2 * hd/4 distinct angles of each token once
// into LDS (all heads and both of Q, K share them), then each wave rotates
// one token: one lane per (q|k, head, axis) unit of hd/2 contiguous values.
#include "common.h"
#include "kernels.h"

namespace vit {

template <int HD>
__global__ __launch_bounds__(256) void rope2d_kernel(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                                     int64_t ld, const int32_t* __restrict__ pos, int T,
                                                     int heads, float log2_theta) {
  constexpr int Q4 = HD / 4;
  constexpr int HALF = HD / 2;
  __shared__ float cs[4][2][Q4][2];  // [token][axis][i][cos|sin]
  const int t0 = blockIdx.x * 4;
  for (int e = threadIdx.x; e < 4 * 2 * Q4; e += 256) {
    const int tok = e / (2 * Q4), axis = (e / Q4) & 1, i = e % Q4;
    const int t = t0 + tok;
    float c = 1.0f, s = 0.0f;
    if (t < T) {
      const float f = exp2f(-(2.0f * (float)i / (float)HALF) * log2_theta);
      const float ang = (float)pos[2 * t + axis] * f;
      sincosf(ang, &s, &c);
    }
    cs[tok][axis][i][0] = c;
    cs[tok][axis][i][1] = s;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, tok = threadIdx.x >> 6;
  const int t = t0 + tok;
  if (t >= T) return;
  for (int u = lane; u < 4 * heads; u += 64) {
    const int which = u / (2 * heads);
    const int h = (u >> 1) % heads;
    const int axis = u & 1;
    uint16_t* p = (which ? k : q) + (int64_t)t * ld + h * HD + axis * HALF;
    float x[HALF];
    if constexpr (HALF % 4 == 0) {
#pragma unroll
      for (int j = 0; j < HALF / 4; ++j) {
        const uint2 w = reinterpret_cast<const uint2*>(p)[j];
        x[4 * j + 0] = bf_lo(w.x);
        x[4 * j + 1] = bf_hi(w.x);
        x[4 * j + 2] = bf_lo(w.y);
        x[4 * j + 3] = bf_hi(w.y);
      }
    } else {
#pragma unroll
      for (int j = 0; j < HALF; ++j) x[j] = bf2f(p[j]);
    }
    float y[HALF];
#pragma unroll
    for (int i = 0; i < Q4; ++i) {
      const float c = cs[tok][axis][i][0], s = cs[tok][axis][i][1];
      y[i] = x[i] * c - x[i + Q4] * s;
      y[i + Q4] = x[i + Q4] * c + x[i] * s;
    }
    if constexpr (HALF % 4 == 0) {
#pragma unroll
      for (int j = 0; j < HALF / 4; ++j) {
        uint2 w;
        w.x = pack_bf16x2(y[4 * j + 0], y[4 * j + 1]);
        w.y = pack_bf16x2(y[4 * j + 2], y[4 * j + 3]);
        reinterpret_cast<uint2*>(p)[j] = w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < HALF; ++j) p[j] = f2bf(y[j]);
    }
  }
}

hipError_t launch_rope2d(uint16_t* q, uint16_t* k, int64_t ld, const int32_t* pos, int T,
                         int heads, int head_dim, float theta, hipStream_t stream) {
  const float l2t = log2f(theta);
  const dim3 grid((T + 3) / 4);
  switch (head_dim) {
    case 72:
      rope2d_kernel<72><<<grid, 256, 0, stream>>>(q, k, ld, pos, T, heads, l2t);
      break;
    case 64:
      rope2d_kernel<64><<<grid, 256, 0, stream>>>(q, k, ld, pos, T, heads, l2t);
      break;
    case 80:
      rope2d_kernel<80><<<grid, 256, 0, stream>>>(q, k, ld, pos, T, heads, l2t);
      break;
    case 128:
      rope2d_kernel<128><<<grid, 256, 0, stream>>>(q, k, ld, pos, T, heads, l2t);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vit
