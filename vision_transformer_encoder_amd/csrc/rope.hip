// 2D rotate_half rotary embedding of Q and K, in place (FlashRT
// "Qwen3-VL-8B on RTX 5090" page, section 3: "2D rotate_half RoPE", kernel
// rope_neox_qk_bf16; spark_model "layers/vision_encoder.rs" page: head_dim/4
// inverse frequencies).  Per head: dims [0, hd/2) rotate by the patch row,
// dims [hd/2, hd) by the patch column; inside each half, dims i and i+hd/4
// form a pair turned by angle p * theta^(-2i/(hd/2)).
//
// HBM-bound (read + write of Q and K).  A 256-thread workgroup handles a
// few tokens.  Their Q and K rows are fetched into LDS with 16-byte loads on
// consecutive lanes (whole cache lines), the 2 * hd/4 distinct angles of each
// token are evaluated once into LDS (all heads and both of Q, K share them),
// every lane then rotates one (q|k, head, axis) unit of hd/2 values in LDS,
// and the rows go back with 16-byte stores.  A second kernel, the same
// per-unit rotation on global memory directly, serves rows that are not
// 16-byte aligned.
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

// Angles of token t into cs[axis][i][cos|sin]: pair i of an axis half turns
// by p * theta^(-2i/(hd/2)), p = the patch row (axis 0) or column (axis 1).
template <int HD>
__device__ __forceinline__ void rope_angles(float (*cs)[HD / 4][2], int e, const int32_t* __restrict__ pos, int t,
                                            int T, float log2_theta) {
  constexpr int Q4 = HD / 4;
  constexpr int HALF = HD / 2;
  const int axis = e / Q4, i = e % Q4;
  float c = 1.0f, sn = 0.0f;
  if (t < T) {
    const float f = exp2f(-(2.0f * (float)i / (float)HALF) * log2_theta);
    const float ang = (float)pos[2 * t + axis] * f;
    sincosf(ang, &sn, &c);
  }
  cs[axis][i][0] = c;
  cs[axis][i][1] = sn;
}

// Coalesced variant: TPB tokens per workgroup, rows staged in dynamic LDS
// ([token][q|k][heads * HD] bf16).  Needs heads * HD % 8 == 0 and 16-byte
// aligned rows (checked by the launcher).  NPT = 16-byte chunks per thread:
// every thread issues all its loads before the first wait (addresses
// clamped into the rows, so no load is conditional), then writes them to
// LDS; the write-back likewise reads all its chunks before storing.  A loop
// of load / wait / LDS store would cost one memory round trip per chunk.
template <int HD, int NPT>
__global__ __launch_bounds__(256) void rope2d_rows_kernel(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                                          int64_t ld, const int32_t* __restrict__ pos, int T,
                                                          int heads, int tpb, float log2_theta) {
  constexpr int Q4 = HD / 4;
  constexpr int HALF = HD / 2;
  extern __shared__ uint4 rows[];
  __shared__ __attribute__((aligned(16))) float cs[8][2][Q4][2];  // [token][axis][i][cos|sin]
  static_assert(Q4 % 2 == 0 && HALF % 4 == 0, "pairs are read two at a time, values four at a time");
  const int W = heads * HD, nch = W >> 3;
  const int t0 = blockIdx.x * tpb;
  const int total = tpb * 2 * nch;
  // chunk c = tid + 256 i is (row r, column chunk ch) = divmod(c, nch),
  // stepped per i without a division; chunks past the end take the last one
  const int tid = threadIdx.x;
  const int dr = 256 / nch, dch = 256 - dr * nch;
  const int r0 = tid / nch, ch0 = tid - r0 * nch;
  uint4 buf[NPT];
  {
    int r = r0, ch = ch0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const bool in = tid + 256 * i < total;
      const int rr = in ? r : 2 * tpb - 1, cc = in ? ch : nch - 1;
      const int t = min(t0 + (rr >> 1), T - 1);
      buf[i] = *reinterpret_cast<const uint4*>(((rr & 1) ? k : q) + (int64_t)t * ld + cc * 8);
      r += dr;
      ch += dch;
      if (ch >= nch) {
        ch -= nch;
        ++r;
      }
    }
  }
  // unconditional, so the loads stay ahead of the first wait: a thread past
  // the end rewrites chunk total - 1 with the value its owner writes
#pragma unroll
  for (int i = 0; i < NPT; ++i) rows[min(tid + 256 * i, total - 1)] = buf[i];
  for (int e = threadIdx.x; e < tpb * 2 * Q4; e += 256)
    rope_angles<HD>(cs[e / (2 * Q4)], e % (2 * Q4), pos, t0 + e / (2 * Q4), T, log2_theta);
  __syncthreads();
  // one lane per (token, q|k, head, axis) unit of HALF values, rotated in LDS
  uint16_t* xl = reinterpret_cast<uint16_t*>(rows);
  const int units = tpb * 4 * heads;
  for (int u = threadIdx.x; u < units; u += 256) {
    const int axis = u & 1, h = (u >> 1) % heads, r = (u >> 1) / heads;  // r = 2 * token + (q|k)
    const int tok = r >> 1;
    if (t0 + tok >= T) continue;
    uint2* p = reinterpret_cast<uint2*>(xl + (int64_t)r * W + h * HD + axis * HALF);
    float x[HALF];
#pragma unroll
    for (int j = 0; j < HALF / 4; ++j) {
      const uint2 w = p[j];
      x[4 * j + 0] = bf_lo(w.x);
      x[4 * j + 1] = bf_hi(w.x);
      x[4 * j + 2] = bf_lo(w.y);
      x[4 * j + 3] = bf_hi(w.y);
    }
    const float4* csp = reinterpret_cast<const float4*>(&cs[tok][axis][0][0]);
    float y[HALF];
#pragma unroll
    for (int i2 = 0; i2 < Q4 / 2; ++i2) {
      const float4 c2 = csp[i2];  // cos, sin of pairs 2 i2 and 2 i2 + 1
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int i = 2 * i2 + d;
        const float c = d ? c2.z : c2.x, sn = d ? c2.w : c2.y;
        y[i] = x[i] * c - x[i + Q4] * sn;
        y[i + Q4] = x[i + Q4] * c + x[i] * sn;
      }
    }
#pragma unroll
    for (int j = 0; j < HALF / 4; ++j) {
      uint2 w;
      w.x = pack_bf16x2(y[4 * j + 0], y[4 * j + 1]);
      w.y = pack_bf16x2(y[4 * j + 2], y[4 * j + 3]);
      p[j] = w;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NPT; ++i) buf[i] = rows[min(tid + 256 * i, total - 1)];
  int r = r0, ch = ch0;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int t = t0 + (r >> 1);
    if (tid + 256 * i < total && t < T)
      *reinterpret_cast<uint4*>(((r & 1) ? k : q) + (int64_t)t * ld + ch * 8) = buf[i];
    r += dr;
    ch += dch;
    if (ch >= nch) {
      ch -= nch;
      ++r;
    }
  }
}

template <int HD>
static hipError_t launch_rope2d_hd(uint16_t* q, uint16_t* k, int64_t ld, const int32_t* pos, int T, int heads,
                                   float l2t, hipStream_t stream) {
  const int W = heads * HD;
  const bool aligned = W % 8 == 0 && ld % 8 == 0 && reinterpret_cast<uintptr_t>(q) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(k) % 16 == 0;
  if (aligned) {
    // tokens per workgroup: 8 while the staged rows stay within 40 KB of LDS
    const int tpb = (size_t)8 * 2 * W * 2 <= 40960 ? 8 : ((size_t)4 * 2 * W * 2 <= 40960 ? 4 : 0);
    if (tpb > 0) {
      const size_t lds = (size_t)tpb * 2 * W * 2;
      const int npt = (tpb * 2 * (W / 8) + 255) / 256;  // <= 10: the rows fit in 40 KB
      const dim3 grid((T + tpb - 1) / tpb);
#define VIT_ROPE_ROWS(N)                                                                      \
  case N:                                                                                     \
    rope2d_rows_kernel<HD, N><<<grid, 256, lds, stream>>>(q, k, ld, pos, T, heads, tpb, l2t); \
    return hipGetLastError();
      switch (npt) {
        VIT_ROPE_ROWS(1) VIT_ROPE_ROWS(2) VIT_ROPE_ROWS(3) VIT_ROPE_ROWS(4) VIT_ROPE_ROWS(5)
        VIT_ROPE_ROWS(6) VIT_ROPE_ROWS(7) VIT_ROPE_ROWS(8) VIT_ROPE_ROWS(9) VIT_ROPE_ROWS(10)
        default:
          break;
      }
#undef VIT_ROPE_ROWS
    }
  }
  rope2d_kernel<HD><<<(T + 3) / 4, 256, 0, stream>>>(q, k, ld, pos, T, heads, l2t);
  return hipGetLastError();
}

hipError_t launch_rope2d(uint16_t* q, uint16_t* k, int64_t ld, const int32_t* pos, int T,
                         int heads, int head_dim, float theta, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const float l2t = log2f(theta);
  switch (head_dim) {
    case 72:
      return launch_rope2d_hd<72>(q, k, ld, pos, T, heads, l2t, stream);
    case 64:
      return launch_rope2d_hd<64>(q, k, ld, pos, T, heads, l2t, stream);
    case 80:
      return launch_rope2d_hd<80>(q, k, ld, pos, T, heads, l2t, stream);
    case 128:
      return launch_rope2d_hd<128>(q, k, ld, pos, T, heads, l2t, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace vit
