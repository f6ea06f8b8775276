// FP8 block-128 quantisation kernels (FlashRT "Qwen3-VL-8B on RTX 5090"
// page, section 1 "FP8 block-128 ViT GEMMs" and section 3: per-token /
// per-128-K-block FP8 activation quant fused into the producing LayerNorm;
// scale = amax / 448 as in TensorRT-Model-Connect PR #2106, Implementation).
//
// All of these are HBM-bound: one pass over the bf16 input, one over the
// codes.  Rows are handled by one 64-lane wave each so every reduction is a
// register shuffle; a 128-column block maps onto 16 lanes x 8 elements, so
// one 16-byte load per lane per block and 16-lane shuffles for the amax.
#include "common.h"
#include "kernels.h"

namespace vit {

// ---------------------------------------------------------------- per row
// One wave per row; blocks of 128 columns, four per wave iteration.
template <int NI>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                         int rows, int cols, int Cp,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + (int64_t)row * ldx;
  const int nblk = Cp >> 7;
  // pass it covers blocks 4 it .. 4 it + 3, 16 lanes each.  With cols % 8 == 0
  // (rows 16-byte aligned) every pass's chunk is loaded before the first
  // reduction, addresses clamped into the row and values past it zeroed: a
  // load under a branch would be followed by a full wait at its end.
  float v[NI][8];
  if ((cols & 7) == 0) {
    uint4 w[NI];
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int b = min(4 * it + (lane >> 4), nblk - 1);
      w[it] = *reinterpret_cast<const uint4*>(xr + min(b * 128 + (lane & 15) * 8, cols - 8));
    }
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int b = 4 * it + (lane >> 4), c = b * 128 + (lane & 15) * 8;
      const bool live = b < nblk && c < cols;
      const float t[8] = {bf_lo(w[it].x), bf_hi(w[it].x), bf_lo(w[it].y), bf_hi(w[it].y),
                          bf_lo(w[it].z), bf_hi(w[it].z), bf_lo(w[it].w), bf_hi(w[it].w)};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[it][i] = live ? t[i] : 0.0f;
    }
  } else {
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int b = 4 * it + (lane >> 4);
      if (b < nblk) {
        load8_bf16(xr, b * 128 + (lane & 15) * 8, cols, v[it]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[it][i] = 0.0f;
      }
    }
  }
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int b = 4 * it + (lane >> 4);
    const int c = b * 128 + (lane & 15) * 8;
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[it][i]));
    am = group16_max(am);
    float s, inv;
    block_scale(am, s, inv);
    if (b < nblk) {
      uint2 o;
      o.x = e4m3x4(v[it][0] * inv, v[it][1] * inv, v[it][2] * inv, v[it][3] * inv);
      o.y = e4m3x4(v[it][4] * inv, v[it][5] * inv, v[it][6] * inv, v[it][7] * inv);
      *reinterpret_cast<uint2*>(codes + (int64_t)row * Cp + c) = o;
      if ((lane & 15) == 0) scales[(int64_t)row * nblk + b] = s;
    }
  }
}

// Rows wider than 64 blocks: the same work as a loop of passes.
__global__ __launch_bounds__(256) void quant_rows_wide_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                              int rows, int cols, int Cp,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + (int64_t)row * ldx;
  const int nblk = Cp >> 7;
  for (int b0 = 0; b0 < nblk; b0 += 4) {
    const int b = b0 + (lane >> 4);
    const int c = b * 128 + (lane & 15) * 8;
    float v[8];
    if (b < nblk) {
      load8_bf16(xr, c, cols, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
    am = group16_max(am);
    float s, inv;
    block_scale(am, s, inv);
    if (b < nblk) {
      uint2 o;
      o.x = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      o.y = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
      *reinterpret_cast<uint2*>(codes + (int64_t)row * Cp + c) = o;
      if ((lane & 15) == 0) scales[(int64_t)row * nblk + b] = s;
    }
  }
}

// ---------------------------------------------------------------- 128x128
// One 256-thread workgroup per 128x128 block: thread t covers row t/2 and
// the 64 columns (t%2)*64 .. +64 of the block.
__global__ __launch_bounds__(256) void quant_blocks128_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                              int rows, int cols, int Cp,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  __shared__ float red[4];
  const int bc = blockIdx.x, br = blockIdx.y;
  const int t = threadIdx.x;
  const int r = br * 128 + (t >> 1);
  const int c0 = bc * 128 + (t & 1) * 64;
  float v[64];
  const bool live = r < rows;
  const uint16_t* xr = x + (int64_t)(live ? r : 0) * ldx;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (live) {
      load8_bf16(xr, c0 + 8 * j, cols, v + 8 * j);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[8 * j + i] = 0.0f;
    }
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) am = fmaxf(am, fabsf(v[i]));
  am = wave_max(am);
  if ((t & 63) == 0) red[t >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s, inv;
  block_scale(am, s, inv);
  uint8_t* out = codes + (int64_t)r * Cp + c0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint2 o;
    o.x = e4m3x4(v[8 * j + 0] * inv, v[8 * j + 1] * inv, v[8 * j + 2] * inv, v[8 * j + 3] * inv);
    o.y = e4m3x4(v[8 * j + 4] * inv, v[8 * j + 5] * inv, v[8 * j + 6] * inv, v[8 * j + 7] * inv);
    *reinterpret_cast<uint2*>(out + 8 * j) = o;
  }
  if (t == 0) scales[(int64_t)br * (Cp >> 7) + bc] = s;
}

// ---------------------------------------------------------------- encoder
__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float* __restrict__ x,
                                                          uint8_t* __restrict__ codes, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    float4 v = *reinterpret_cast<const float4*>(x + i);
    *reinterpret_cast<uint32_t*>(codes + i) = e4m3x4_sat(v.x, v.y, v.z, v.w);
  } else {
    for (int64_t j = i; j < n; ++j) codes[j] = (uint8_t)(e4m3x4_sat(x[j], 0.0f, 0.0f, 0.0f) & 0xff);
  }
}

// ---------------------------------------------------------------- LN + quant
// One wave per row of D = 512*NC or fewer columns (D % 128 == 0).  Chunk
// i*64+lane holds columns 8*(i*64+lane) .. +8; a 128-column block is 16
// consecutive chunks, i.e. 16 consecutive lanes of one iteration.
// OUT_BF16: the normalised row is stored in bf16 (out, row stride ldo)
// instead of being quantised (the bf16-GEMM blocks).
template <int NC, bool OUT_BF16>
__global__ __launch_bounds__(256) void layernorm_quant_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                              const uint16_t* __restrict__ gamma,
                                                              const uint16_t* __restrict__ beta, float eps,
                                                              int M, int D, uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales,
                                                              float* __restrict__ prequant,
                                                              uint16_t* __restrict__ out, int64_t ldo) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int nchunk = D >> 3;
  const uint16_t* xr = x + (int64_t)row * ldx;
  // gamma and beta travel with the row (one memory round trip, not two)
  uint4 gw[NC], bw[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int ch = min(i * 64 + lane, nchunk - 1);
    gw[i] = *reinterpret_cast<const uint4*>(gamma + ch * 8);
    bw[i] = *reinterpret_cast<const uint4*>(beta + ch * 8);
  }
  // every lane loads a chunk (lanes past the row re-read its last chunk and
  // zero the values afterwards), so all of a lane's loads are in flight
  // together: a load under a branch is followed by a full wait at its end
  uint4 xw[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) xw[i] = *reinterpret_cast<const uint4*>(xr + min(i * 64 + lane, nchunk - 1) * 8);
  float v[NC][8];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const bool live = i * 64 + lane < nchunk;
    const float t[8] = {bf_lo(xw[i].x), bf_hi(xw[i].x), bf_lo(xw[i].y), bf_hi(xw[i].y),
                        bf_lo(xw[i].z), bf_hi(xw[i].z), bf_lo(xw[i].w), bf_hi(xw[i].w)};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[i][j] = live ? t[j] : 0.0f;
      sum += v[i][j];
    }
  }
  const float mean = wave_sum(sum) / (float)D;
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (i * 64 + lane < nchunk) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = v[i][j] - mean;
        sq += d * d;
      }
    }
  }
  const float var = wave_sum(sq) / (float)D;
  const float rstd = 1.0f / sqrtf(var + eps);
  const int nblk = D >> 7;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int ch = i * 64 + lane;
    const bool live = ch < nchunk;
    float y[8];
    if (live) {
      const float g[8] = {bf_lo(gw[i].x), bf_hi(gw[i].x), bf_lo(gw[i].y), bf_hi(gw[i].y),
                          bf_lo(gw[i].z), bf_hi(gw[i].z), bf_lo(gw[i].w), bf_hi(gw[i].w)};
      const float bb[8] = {bf_lo(bw[i].x), bf_hi(bw[i].x), bf_lo(bw[i].y), bf_hi(bw[i].y),
                           bf_lo(bw[i].z), bf_hi(bw[i].z), bf_lo(bw[i].w), bf_hi(bw[i].w)};
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = (v[i][j] - mean) * rstd * g[j] + bb[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = 0.0f;
    }
    if constexpr (OUT_BF16) {
      if (live) {
        uint4 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        o.z = pack_bf16x2(y[4], y[5]);
        o.w = pack_bf16x2(y[6], y[7]);
        *reinterpret_cast<uint4*>(out + (int64_t)row * ldo + ch * 8) = o;
      }
      continue;
    }
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(y[j]));
    am = group16_max(am);
    float s, inv;
    block_scale(am, s, inv);
    if (live) {
      uint2 o;
      o.x = e4m3x4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
      o.y = e4m3x4(y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv);
      *reinterpret_cast<uint2*>(codes + (int64_t)row * D + ch * 8) = o;
      if ((lane & 15) == 0) scales[(int64_t)row * nblk + (ch >> 4)] = s;
      if (prequant) {
        float4* p = reinterpret_cast<float4*>(prequant + (int64_t)row * D + ch * 8);
        p[0] = make_float4(y[0], y[1], y[2], y[3]);
        p[1] = make_float4(y[4], y[5], y[6], y[7]);
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_quant_rows(const uint16_t* x, int64_t ldx, int rows, int cols, uint8_t* codes,
                             float* scales, hipStream_t stream) {
  const int Cp = (cols + 127) / 128 * 128;
  const int ni = (Cp / 128 + 3) / 4;  // passes of four 128-column blocks
  const dim3 grid((rows + 3) / 4);
#define VIT_QR_CASE(N)                                                                      \
  case N:                                                                                   \
    quant_rows_kernel<N><<<grid, 256, 0, stream>>>(x, ldx, rows, cols, Cp, codes, scales); \
    break;
  switch (ni) {
    VIT_QR_CASE(1) VIT_QR_CASE(2) VIT_QR_CASE(3) VIT_QR_CASE(4) VIT_QR_CASE(5) VIT_QR_CASE(6)
    VIT_QR_CASE(7) VIT_QR_CASE(8) VIT_QR_CASE(9) VIT_QR_CASE(10) VIT_QR_CASE(11) VIT_QR_CASE(12)
    VIT_QR_CASE(13) VIT_QR_CASE(14) VIT_QR_CASE(15) VIT_QR_CASE(16)
    default:
      quant_rows_wide_kernel<<<grid, 256, 0, stream>>>(x, ldx, rows, cols, Cp, codes, scales);
  }
#undef VIT_QR_CASE
  return hipGetLastError();
}

hipError_t launch_quant_blocks128(const uint16_t* x, int64_t ldx, int rows, int cols,
                                  uint8_t* codes, float* scales, hipStream_t stream) {
  const int Cp = (cols + 127) / 128 * 128;
  dim3 grid(Cp / 128, (rows + 127) / 128);
  quant_blocks128_kernel<<<grid, 256, 0, stream>>>(x, ldx, rows, cols, Cp, codes, scales);
  return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream) {
  const int64_t groups = (n + 3) / 4;
  e4m3_encode_kernel<<<(unsigned)((groups + 255) / 256), 256, 0, stream>>>(x, codes, n);
  return hipGetLastError();
}

template <bool OUT_BF16>
static hipError_t launch_layernorm(const uint16_t* x, int64_t ldx, const uint16_t* gamma, const uint16_t* beta,
                                   float eps, int M, int D, uint8_t* codes, float* scales, float* prequant,
                                   uint16_t* out, int64_t ldo, hipStream_t stream) {
  const int nc = (D / 8 + 63) / 64;
  const dim3 grid((M + 3) / 4), block(256);
#define VIT_LNQ_CASE(N)                                                                               \
  case N:                                                                                            \
    layernorm_quant_kernel<N, OUT_BF16><<<grid, block, 0, stream>>>(x, ldx, gamma, beta, eps, M, D, \
                                                                    codes, scales, prequant, out, ldo); \
    break;
  switch (nc) {
    VIT_LNQ_CASE(1)
    VIT_LNQ_CASE(2)
    VIT_LNQ_CASE(3)
    VIT_LNQ_CASE(4)
    VIT_LNQ_CASE(5)
    VIT_LNQ_CASE(6)
    VIT_LNQ_CASE(7)
    VIT_LNQ_CASE(8)
    VIT_LNQ_CASE(9)
    VIT_LNQ_CASE(10)
    VIT_LNQ_CASE(11)
    VIT_LNQ_CASE(12)
    VIT_LNQ_CASE(13)
    VIT_LNQ_CASE(14)
    VIT_LNQ_CASE(15)
    VIT_LNQ_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef VIT_LNQ_CASE
  return hipGetLastError();
}

hipError_t launch_layernorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                                  const uint16_t* beta, float eps, int M, int D, uint8_t* codes,
                                  float* scales, float* prequant, hipStream_t stream) {
  return launch_layernorm<false>(x, ldx, gamma, beta, eps, M, D, codes, scales, prequant, nullptr, 0, stream);
}

hipError_t launch_layernorm_bf16(const uint16_t* x, int64_t ldx, const uint16_t* gamma, const uint16_t* beta,
                                 float eps, int M, int D, uint16_t* out, int64_t ldo, hipStream_t stream) {
  return launch_layernorm<true>(x, ldx, gamma, beta, eps, M, D, nullptr, nullptr, nullptr, out, ldo, stream);
}

}  // namespace vit
