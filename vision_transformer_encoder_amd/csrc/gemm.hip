// GEMMs of the tower (FlashRT "Qwen3-VL-8B on RTX 5090" page):
//  * block-scaled FP8 W8A8 (section 1 "FP8 block-128 ViT GEMMs"; bias adds
//    fused into the GEMM; section 3: GELU fused with the FP8 quant of the fc2
//    input) for qkv / proj / fc1 / fc2;
//  * bf16 (section 4: patch embed and mergers stay bf16) for the patch
//    embedding (fp32 pixels rounded on load) and the merger MLPs.
// Weights are [N, K] row-major (spark_model "layers/vision_encoder.rs":
// C[M,N] = A[M,K] @ B[N,K]^T + bias), activations [M, K]; both K-contiguous.
//
// gfx950 design: 256 threads = 4 waves on a 128 (n) x 128 (m) output tile,
// 2 x 2 waves of 64 x 64, v_mfma_f32_32x32x64_f8f6f4 (FP8) or
// v_mfma_f32_32x32x16_bf16.  The WEIGHT is the MFMA A operand and the
// ACTIVATION the B operand, so in the 32x32 accumulator layout a lane holds
// one token row (lane % 32) and 4 runs of 4 consecutive output features:
// epilogue stores are 8-byte runs, the per-row FP8 requant amax is mostly
// in-lane, and the per-row activation scale is one register per m-tile.
// FP8 block scaling: each 128-deep K block is one MFMA chain started from
// zero (the MFMA's internal sum is not fp32-exact, so partial sums are
// promoted every 128 K), then acc += partial * sA[m, kb] * sW[n/128, kb]
// in fp32 VALU.  Tiles of A and W are double-buffered in LDS with a
// 144-byte row stride (conflict-free 16-byte operand reads); the next K
// block's global loads are in flight during the current block's MFMAs.
#include "common.h"
#include "kernels.h"

namespace vit {

namespace {
constexpr int kBM = 128;   // tokens per tile
constexpr int kBN = 128;   // output features per tile
constexpr int kRowB = 128; // bytes of K per tile row per step
constexpr int kLS = 144;   // LDS row stride in bytes
constexpr int kTileB = 128 * kLS;
}  // namespace

__device__ __forceinline__ i32x8_t lds_read32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  i32x8_t r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

// ============================================================ FP8 block-128
template <int EPI>
__global__ __launch_bounds__(256) void fp8_gemm_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scales, const uint8_t* __restrict__ w,
    const float* __restrict__ w_scales, int M, int N, int Np, int Kp, int n_tiles,
    const uint16_t* __restrict__ bias, const uint16_t* residual, uint16_t* out,
    uint8_t* __restrict__ out_codes, float* __restrict__ out_scales, float* __restrict__ prequant) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2 * kTileB];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[2 * kTileB];
  __shared__ float sa_lds[2][kBM];
  __shared__ float red[2][2][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int n_tile = blockIdx.x % n_tiles, m_tile = blockIdx.x / n_tiles;
  const int n0 = n_tile * kBN, m0 = m_tile * kBM;
  const int Kb = Kp >> 7;

  uint4 ra[4], rw[4];
  float rs = 0.0f;
  const int lrow = tid >> 3, lcol = (tid & 7) * 16;
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      const int am = min(m0 + row, M - 1);
      ra[i] = *reinterpret_cast<const uint4*>(a + (int64_t)am * Kp + kb * kRowB + lcol);
      rw[i] = *reinterpret_cast<const uint4*>(w + (int64_t)(n0 + row) * Kp + kb * kRowB + lcol);
    }
    if (tid < kBM) rs = a_scales[(int64_t)min(m0 + tid, M - 1) * Kb + kb];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      *reinterpret_cast<uint4*>(a_lds + buf * kTileB + row * kLS + lcol) = ra[i];
      *reinterpret_cast<uint4*>(w_lds + buf * kTileB + row * kLS + lcol) = rw[i];
    }
    if (tid < kBM) sa_lds[buf][tid] = rs;
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kb = 0; kb < Kb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < Kb) gload(kb + 1);
    const float sw = w_scales[(int64_t)n_tile * Kb + kb];
    const uint8_t* wl = w_lds + buf * kTileB;
    const uint8_t* al = a_lds + buf * kTileB;
    i32x8_t wop[2][2], aop[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        wop[t][kh] = lds_read32(wl + (64 * wn + 32 * t + l32) * kLS + 64 * kh + 32 * g);
        aop[t][kh] = lds_read32(al + (64 * wm + 32 * t + l32) * kLS + 64 * kh + 32 * g);
      }
    }
    float coef[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) coef[mt] = sa_lds[buf][64 * wm + 32 * mt + l32] * sw;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16_t part = f32x16_t{};
        part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wop[nt][0], aop[mt][0], part, 0, 0, 0, 0, 0, 0);
        part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wop[nt][1], aop[mt][1], part, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nt][mt][r] = fmaf(part[r], coef[mt], acc[nt][mt][r]);
      }
    }
    if (kb + 1 < Kb) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // lane holds m = m0 + 64wm + 32mt + l32 and n = n0 + 64wn + 32nt + 8rg + 4g + j
  if constexpr (EPI == 0 || EPI == 1) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int m = m0 + 64 * wm + 32 * mt + l32;
      if (m >= M) continue;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = n0 + 64 * wn + 32 * nt + 8 * rg + 4 * g;
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = acc[nt][mt][4 * rg + j];
          if (n + 4 <= N && (N & 3) == 0) {
            if (bias) {
              const uint2 b = *reinterpret_cast<const uint2*>(bias + n);
              y[0] += bf_lo(b.x); y[1] += bf_hi(b.x); y[2] += bf_lo(b.y); y[3] += bf_hi(b.y);
            }
            uint16_t* op = out + (int64_t)m * N + n;
            if constexpr (EPI == 1) {
              const uint2 rr = *reinterpret_cast<const uint2*>(residual + (int64_t)m * N + n);
              y[0] += bf_lo(rr.x); y[1] += bf_hi(rr.x); y[2] += bf_lo(rr.y); y[3] += bf_hi(rr.y);
            }
            uint2 o2;
            o2.x = pack_bf16x2(y[0], y[1]);
            o2.y = pack_bf16x2(y[2], y[3]);
            *reinterpret_cast<uint2*>(op) = o2;
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (n + j < N) {
                float v = y[j] + (bias ? bf2f(bias[n + j]) : 0.0f);
                if constexpr (EPI == 1) v += bf2f(residual[(int64_t)m * N + n + j]);
                out[(int64_t)m * N + n + j] = f2bf(v);
              }
            }
          }
        }
      }
    }
  } else {
    // bias + GELU, then FP8 requant per row and 128 columns (= this n tile)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = n0 + 64 * wn + 32 * nt + 8 * rg + 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float b = (bias && n + j < N) ? bf2f(bias[n + j]) : 0.0f;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const float v = acc[nt][mt][4 * rg + j] + b;
            acc[nt][mt][4 * rg + j] = (n + j < N) ? gelu_tanh(v) : 0.0f;
          }
        }
      }
    }
    float amax[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float am = 0.0f;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) am = fmaxf(am, fabsf(acc[nt][mt][r]));
      am = fmaxf(am, __shfl_xor(am, 32));
      if (g == 0) red[wm][wn][32 * mt + l32] = am;
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) amax[mt] = fmaxf(red[wm][0][32 * mt + l32], red[wm][1][32 * mt + l32]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int m = m0 + 64 * wm + 32 * mt + l32;
      if (m >= M) continue;
      float s, inv;
      block_scale(amax[mt], s, inv);
      if (wn == 0 && g == 0) out_scales[(int64_t)m * (Np >> 7) + n_tile] = s;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = n0 + 64 * wn + 32 * nt + 8 * rg + 4 * g;
          const float y[4] = {acc[nt][mt][4 * rg + 0], acc[nt][mt][4 * rg + 1], acc[nt][mt][4 * rg + 2],
                              acc[nt][mt][4 * rg + 3]};
          *reinterpret_cast<uint32_t*>(out_codes + (int64_t)m * Np + n) =
              e4m3x4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
          if (prequant) {
            *reinterpret_cast<float4*>(prequant + (int64_t)m * Np + n) = make_float4(y[0], y[1], y[2], y[3]);
          }
        }
      }
    }
  }
}

hipError_t launch_fp8_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w,
                           const float* w_scales, int M, int N, int K, const uint16_t* bias,
                           const uint16_t* residual, int epilogue, uint16_t* out,
                           uint8_t* out_codes, float* out_scales, float* prequant,
                           hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int Kp = (K + 127) / 128 * 128;
  const int Np = (N + 127) / 128 * 128;
  const int n_tiles = Np / kBN, m_tiles = (M + kBM - 1) / kBM;
  const dim3 grid(n_tiles * m_tiles);
  switch (epilogue) {
    case 0:
      fp8_gemm_kernel<0><<<grid, 256, 0, stream>>>(a, a_scales, w, w_scales, M, N, Np, Kp, n_tiles, bias,
                                                   residual, out, out_codes, out_scales, prequant);
      break;
    case 1:
      fp8_gemm_kernel<1><<<grid, 256, 0, stream>>>(a, a_scales, w, w_scales, M, N, Np, Kp, n_tiles, bias,
                                                   residual, out, out_codes, out_scales, prequant);
      break;
    case 2:
      fp8_gemm_kernel<2><<<grid, 256, 0, stream>>>(a, a_scales, w, w_scales, M, N, Np, Kp, n_tiles, bias,
                                                   residual, out, out_codes, out_scales, prequant);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ============================================================ bf16
// Same tiling; K steps of 64 elements (128 bytes per row), 4 MFMAs of K=16
// per step accumulated directly.  A_F32: A is fp32 (rounded to bf16 as it
// is staged into LDS).
template <int EPI, bool A_F32>
__global__ __launch_bounds__(256) void bf16_gemm_kernel(const void* __restrict__ a_ptr,
                                                        const uint16_t* __restrict__ w, int M, int N,
                                                        int K, int n_tiles,
                                                        const uint16_t* __restrict__ bias,
                                                        const uint16_t* __restrict__ add,
                                                        uint16_t* __restrict__ out, int64_t ld_out) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2 * kTileB];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[2 * kTileB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int n_tile = blockIdx.x % n_tiles, m_tile = blockIdx.x / n_tiles;
  const int n0 = n_tile * kBN, m0 = m_tile * kBM;
  const int ksteps = (K + 63) / 64;

  // bf16 A / W: chunk = 8 elements (16 B); row = tid/8 + 32i, col = (tid%8)*8
  // fp32 A: chunk = 4 elements (16 B in, 8 B out); row = tid/16 + 16i, col = (tid%16)*4
  uint4 rw[4];
  uint4 ra16[4];
  float4 ra32[8];
  auto gload = [&](int ks) {
    const int k0 = ks * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      const int kc = k0 + (tid & 7) * 8;
      const int wr = min(n0 + row, N - 1);
      rw[i] = kc < K ? *reinterpret_cast<const uint4*>(w + (int64_t)wr * K + kc) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (A_F32) {
      const float* a = reinterpret_cast<const float*>(a_ptr);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 4) + 16 * i;
        const int kc = k0 + (tid & 15) * 4;
        const int ar = min(m0 + row, M - 1);
        ra32[i] = kc < K ? *reinterpret_cast<const float4*>(a + (int64_t)ar * K + kc) : make_float4(0, 0, 0, 0);
      }
    } else {
      const uint16_t* a = reinterpret_cast<const uint16_t*>(a_ptr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        const int kc = k0 + (tid & 7) * 8;
        const int ar = min(m0 + row, M - 1);
        ra16[i] = kc < K ? *reinterpret_cast<const uint4*>(a + (int64_t)ar * K + kc) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(w_lds + buf * kTileB + row * kLS + (tid & 7) * 16) = rw[i];
    }
    if constexpr (A_F32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 4) + 16 * i;
        uint2 p;
        p.x = pack_bf16x2(ra32[i].x, ra32[i].y);
        p.y = pack_bf16x2(ra32[i].z, ra32[i].w);
        *reinterpret_cast<uint2*>(a_lds + buf * kTileB + row * kLS + (tid & 15) * 8) = p;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        *reinterpret_cast<uint4*>(a_lds + buf * kTileB + row * kLS + (tid & 7) * 16) = ra16[i];
      }
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < ksteps) gload(ks + 1);
    const uint8_t* wl = w_lds + buf * kTileB;
    const uint8_t* al = a_lds + buf * kTileB;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t wop[2], aop[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        wop[t] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                  wl + (64 * wn + 32 * t + l32) * kLS + 32 * kk + 16 * g));
        aop[t] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                  al + (64 * wm + 32 * t + l32) * kLS + 32 * kk + 16 * g));
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop[nt], aop[mt], acc[nt][mt], 0, 0, 0);
    }
    if (ks + 1 < ksteps) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int m = m0 + 64 * wm + 32 * mt + l32;
    if (m >= M) continue;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = n0 + 64 * wn + 32 * nt + 8 * rg + 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (n + j < N) {
            float v = acc[nt][mt][4 * rg + j] + (bias ? bf2f(bias[n + j]) : 0.0f);
            if constexpr (EPI == 1) v = gelu_tanh(v);
            if constexpr (EPI == 2) v += add ? bf2f(add[(int64_t)m * N + n + j]) : 0.0f;
            out[(int64_t)m * ld_out + n + j] = f2bf(v);
          }
        }
      }
    }
  }
}

hipError_t launch_bf16_gemm(const void* a, bool a_f32, const uint16_t* w, int M, int N, int K,
                            const uint16_t* bias, const uint16_t* add, int epilogue,
                            uint16_t* out, int64_t ld_out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int n_tiles = (N + kBN - 1) / kBN, m_tiles = (M + kBM - 1) / kBM;
  const dim3 grid(n_tiles * m_tiles);
#define VIT_BG(E, F)                                                                                   \
  bf16_gemm_kernel<E, F><<<grid, 256, 0, stream>>>(a, w, M, N, K, n_tiles, bias, add, out, ld_out)
  if (a_f32) {
    switch (epilogue) {
      case 0: VIT_BG(0, true); break;
      case 1: VIT_BG(1, true); break;
      case 2: VIT_BG(2, true); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (epilogue) {
      case 0: VIT_BG(0, false); break;
      case 1: VIT_BG(1, false); break;
      case 2: VIT_BG(2, false); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef VIT_BG
  return hipGetLastError();
}

}  // namespace vit
