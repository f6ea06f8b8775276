// GEMMs of the tower (FlashRT "Qwen3-VL-8B on RTX 5090" page):
//  * block-scaled FP8 W8A8 (section 1 "FP8 block-128 ViT GEMMs"; bias adds
//    fused into the GEMM; section 3: GELU fused with the FP8 quant of the fc2
//    input) for qkv / proj / fc1 / fc2;
//  * bf16 (section 4: patch embed and mergers stay bf16) for the patch
//    embedding (fp32 pixels rounded on load) and the merger MLPs; shapes
//    with bf16 activations, N % 256 == 0 and K % 192 == 0 (the mergers) go
//    to the kernel of gemm_wide.hip (256 x 128 tiles, 64 x 64 for small M).
// Weights are [N, K] row-major (spark_model "layers/vision_encoder.rs":
// C[M,N] = A[M,K] @ B[N,K]^T + bias), activations [M, K]; both K-contiguous.
//
// gfx950 design: 256 threads = 4 waves on a 128 (n) x 128 (m) output tile,
// 2 x 2 waves of 64 x 64, v_mfma_f32_32x32x64_f8f6f4 (FP8) or
// v_mfma_f32_32x32x16_bf16, the weight as MFMA A operand and the activation
// as B operand.  When M is small enough that 128-token tiles would give at
// most one workgroup per CU, the FP8 GEMM takes 128 x 64 tiles (waves of
// 64 x 32) instead: each output is the same chain of MFMAs and FMAs.
//  * FP8 block scaling: each 128-deep K block is one MFMA chain started from
//    zero (the MFMA's internal sum is not fp32-exact, so partial sums are
//    promoted every 128 K), then acc += partial * sA[m, kb] * sW[n/128, kb]
//    in fp32 VALU (one FMA per output per K block).
//  * K loop: A and W tiles (128 rows x 128 bytes each step) double-buffered
//    in LDS with a 144-byte row stride (conflict-free 16-byte operand
//    reads); the next step's global loads are in flight during the current
//    step's MFMAs; load addresses are fixed per thread outside the loop.
//  * Epilogue through LDS: the fp32 tile is parked in LDS, then every row is
//    finished by 16 consecutive threads (8 columns each): bias, residual,
//    GELU and the per-row 128-column FP8 requant amax (16-lane shuffle)
//    all happen there, and every global store is a full 16-byte run, so
//    rows are written with whole cache lines.
//  * Tile order is XCD-aware: workgroups are dealt round-robin to the 8
//    XCDs, so block id b is remapped to a logical tile index such that each
//    XCD owns a contiguous range of the tile order, and that order walks the
//    N tiles in groups of at most 12 (every M tile of one group, then the
//    next group): the workgroups resident on one XCD share a few activation
//    tiles and one group's weight slice in its L2.
#include "common.h"
#include "kernels.h"

namespace vit {

namespace {
constexpr int kBM = 128;   // tokens per tile
constexpr int kBN = 128;   // output features per tile
constexpr int kRowB = 128; // bytes of K per tile row per step
constexpr int kLS = 144;   // LDS row stride in bytes
constexpr int kTileB = 128 * kLS;
constexpr int kCS = 132;   // fp32 row stride of the parked C tile (floats)
}  // namespace

__device__ __forceinline__ i32x8_t lds_read32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  i32x8_t r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

// Park the 64 x 32 MT fp32 accumulators of this wave in the LDS C tile
// (row = m local, column = n local).
template <int MT>
__device__ __forceinline__ void park_acc(float* c_lds, const f32x16_t acc[2][MT], int wn, int wm, int l32, int g) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ml = 32 * MT * wm + 32 * mt + l32;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int nl = 64 * wn + 32 * nt + 8 * rg + 4 * g;
        *reinterpret_cast<float4*>(c_lds + ml * kCS + nl) =
            make_float4(acc[nt][mt][4 * rg + 0], acc[nt][mt][4 * rg + 1], acc[nt][mt][4 * rg + 2],
                        acc[nt][mt][4 * rg + 3]);
      }
    }
  }
}

// Workgroup barrier over LDS only: this wave's LDS traffic is complete; its
// global loads in flight are not waited for (their registers are tracked by
// the compiler as usual).
__device__ __forceinline__ void tile_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ============================================================ FP8 block-128
// BM = 128 or 64 tokens per tile: 2 x 2 waves of 64 (n) x BM / 2 (m).  The
// 64-token tiles are for small M, where 128-token tiles would leave CUs
// idle; every output sees the same MFMAs, promotions and epilogue either way.
template <int EPI, int BM>
__global__ __launch_bounds__(256) void fp8_gemm_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scales, const uint8_t* __restrict__ w,
    const float* __restrict__ w_scales, int M, int N, int Np, int Kp, int n_tiles, int nblocks, int group_n,
    const uint16_t* __restrict__ bias, const uint16_t* residual, uint16_t* out,
    uint8_t* __restrict__ out_codes, float* __restrict__ out_scales, float* __restrict__ prequant) {
  constexpr int MT = BM / 64;             // 32-row m sub-tiles per wave
  constexpr int NA = BM / 32;             // A rows loaded per thread and step
  constexpr int kTileA = BM * kLS;
  constexpr int kPasses = BM / 16;        // epilogue rows per thread
  // A x2, W x2; the C tile after the loop
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kTileA + 2 * kTileB];
  __shared__ float sa_lds[2][BM];
  uint8_t* a_lds = smem;
  uint8_t* w_lds = smem + 2 * kTileA;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int lb = xcd_logical_block(blockIdx.x, nblocks);
  int m_tile, n_tile;
  grouped_tile(lb, nblocks / n_tiles, n_tiles, group_n, m_tile, n_tile);
  const int n0 = n_tile * kBN, m0 = m_tile * BM;
  const int Kb = Kp >> 7;

  // per-thread load slots: rows lrow + 32i, 16 bytes at lcol, as 32-bit
  // offsets from the tile's first row (< 128 Kp); the tile bases are 64-bit
  const int lrow = tid >> 3, lcol = (tid & 7) * 16;
  const uint8_t* a_tile = a + (size_t)m0 * Kp;
  const uint8_t* w_tile = w + (size_t)n0 * Kp;
  uint32_t a_off[NA], w_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < NA) a_off[i] = (uint32_t)(min(m0 + lrow + 32 * i, M - 1) - m0) * (uint32_t)Kp + lcol;
    w_off[i] = (uint32_t)(lrow + 32 * i) * (uint32_t)Kp + lcol;
  }
  const float* sa_ptr = a_scales + (size_t)min(m0 + (tid & (BM - 1)), M - 1) * Kb;
  const float* sw_ptr = w_scales + (size_t)n_tile * Kb;

  u32x4_t ra[NA], rw[4];
  float rs = 0.0f;
  auto gload = [&](int kb) {
    const uint8_t* ak = a_tile + kb * kRowB;
    const uint8_t* wk = w_tile + kb * kRowB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < NA) ra[i] = *reinterpret_cast<const u32x4_t*>(ak + a_off[i]);
      rw[i] = *reinterpret_cast<const u32x4_t*>(wk + w_off[i]);
    }
    rs = sa_ptr[kb];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      if (i < NA) *reinterpret_cast<u32x4_t*>(a_lds + buf * kTileA + row * kLS + lcol) = ra[i];
      *reinterpret_cast<u32x4_t*>(w_lds + buf * kTileB + row * kLS + lcol) = rw[i];
    }
    if (tid < BM) sa_lds[buf][tid] = rs;
  };

  f32x16_t acc[2][MT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = f32x16_t{};

  // one 128-deep K block from LDS buffer buf
  auto mma_block = [&](int buf, int kb) {
    const float sw = sw_ptr[kb];
    const uint8_t* wl = w_lds + buf * kTileB + (64 * wn + l32) * kLS + 32 * g;
    const uint8_t* al = a_lds + buf * kTileA + (32 * MT * wm + l32) * kLS + 32 * g;
    i32x8_t wop[2][2], aop[MT][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        wop[t][kh] = lds_read32(wl + 32 * t * kLS + 64 * kh);
        if (t < MT) aop[t][kh] = lds_read32(al + 32 * t * kLS + 64 * kh);
      }
    }
    f32x16_t part[2][MT];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        part[nt][mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wop[nt][0], aop[mt][0], f32x16_t{}, 0, 0,
                                                                       0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        part[nt][mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wop[nt][1], aop[mt][1], part[nt][mt], 0,
                                                                       0, 0, 0, 0, 0);
      }
    }
    float coef[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) coef[mt] = sa_lds[buf][32 * MT * wm + 32 * mt + l32] * sw;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nt][mt][r] = fmaf(part[nt][mt][r], coef[mt], acc[nt][mt][r]);
  };

  if constexpr (BM == 128) {
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kb = 0; kb < Kb; ++kb) {
      const int buf = kb & 1;
      if (kb + 1 < Kb) gload(kb + 1);
      mma_block(buf, kb);
      if (kb + 1 < Kb) lstore(buf ^ 1);
      __syncthreads();
    }
  } else {
    // 64-token tiles run about one workgroup per CU, with nothing to hide a
    // step's global loads behind: they are issued two K blocks ahead, into
    // two register sets (block k in set k % 2).  Step k loads block k + 2
    // into the set whose block went to LDS at step k - 1, computes block k
    // and stores block k + 1 (loaded at step k - 1).  The last steps load
    // and store the final block again rather than branch around the loads.
    u32x4_t ra2[2][NA], rw2[2][4];
    float rs2[2];
    const int last = Kb - 1;
    auto gload2 = [&](int set, int kb) {
      const uint8_t* ak = a_tile + kb * kRowB;
      const uint8_t* wk = w_tile + kb * kRowB;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < NA) ra2[set][i] = *reinterpret_cast<const u32x4_t*>(ak + a_off[i]);
        rw2[set][i] = *reinterpret_cast<const u32x4_t*>(wk + w_off[i]);
      }
      rs2[set] = sa_ptr[kb];
    };
    auto lstore2 = [&](int set, int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = lrow + 32 * i;
        if (i < NA) *reinterpret_cast<u32x4_t*>(a_lds + buf * kTileA + row * kLS + lcol) = ra2[set][i];
        *reinterpret_cast<u32x4_t*>(w_lds + buf * kTileB + row * kLS + lcol) = rw2[set][i];
      }
      if (tid < BM) sa_lds[buf][tid] = rs2[set];
    };
    auto step = [&](int kb, int set) {
      gload2(set, min(kb + 2, last));
      mma_block(set, kb);
      lstore2(set ^ 1, set ^ 1);
      __syncthreads();
    };
    gload2(0, 0);
    lstore2(0, 0);
    gload2(1, min(1, last));
    __syncthreads();
    int kb = 0;
    for (; kb + 2 <= Kb; kb += 2) {
      step(kb, 0);
      step(kb + 1, 1);
    }
    if (kb < Kb) {
      mma_block(0, kb);
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------- epilogue
  // thread -> (row = tid/16 + 16 pass, 8 columns at (tid%16)*8).  The bias
  // and residual loads are issued before the tile is parked, so their
  // latency overlaps the LDS round trip, and all eight rows are read from
  // LDS before the first is finished.
  const int cc = (tid & 15) * 8;
  const int n = n0 + cc;
  const bool vec = n + 8 <= N && (N & 7) == 0;
  float b8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b8[j] = 0.0f;
  if (bias) {
    if (vec) {
      load8_bf16(bias, n, N, b8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) b8[j] = (n + j < N) ? bf2f(bias[n + j]) : 0.0f;
    }
  }
  uint4 res8[kPasses];
  if constexpr (EPI == 1) {
    if (vec) {
#pragma unroll
      for (int pass = 0; pass < kPasses; ++pass) {
        const int m = min(m0 + (tid >> 4) + 16 * pass, M - 1);
        res8[pass] = *reinterpret_cast<const uint4*>(residual + (int64_t)m * N + n);
      }
    }
  }
  float* c_lds = reinterpret_cast<float*>(smem);
  park_acc<MT>(c_lds, acc, wn, wm, l32, g);
  tile_barrier();
  float4 cv[kPasses][2];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int ml = (tid >> 4) + 16 * pass;
    cv[pass][0] = *reinterpret_cast<const float4*>(c_lds + ml * kCS + cc);
    cv[pass][1] = *reinterpret_cast<const float4*>(c_lds + ml * kCS + cc + 4);
  }
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int m = m0 + (tid >> 4) + 16 * pass;
    const float4 c0 = cv[pass][0], c1 = cv[pass][1];
    float y[8] = {c0.x + b8[0], c0.y + b8[1], c0.z + b8[2], c0.w + b8[3],
                  c1.x + b8[4], c1.y + b8[5], c1.z + b8[6], c1.w + b8[7]};
    if constexpr (EPI == 0 || EPI == 1) {
      if (m < M) {
        if constexpr (EPI == 1) {
          float r8[8];
          if (vec) {
            const uint4 w4 = res8[pass];
            r8[0] = bf_lo(w4.x); r8[1] = bf_hi(w4.x); r8[2] = bf_lo(w4.y); r8[3] = bf_hi(w4.y);
            r8[4] = bf_lo(w4.z); r8[5] = bf_hi(w4.z); r8[6] = bf_lo(w4.w); r8[7] = bf_hi(w4.w);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) r8[j] = (n + j < N) ? bf2f(residual[(int64_t)m * N + n + j]) : 0.0f;
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] += r8[j];
        }
        if (vec) {
          uint4 o;
          o.x = pack_bf16x2(y[0], y[1]);
          o.y = pack_bf16x2(y[2], y[3]);
          o.z = pack_bf16x2(y[4], y[5]);
          o.w = pack_bf16x2(y[6], y[7]);
          *reinterpret_cast<uint4*>(out + (int64_t)m * N + n) = o;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (n + j < N) out[(int64_t)m * N + n + j] = f2bf(y[j]);
        }
      }
    } else {
      // GELU, then FP8 requant of this row's 128 columns (16 lanes x 8);
      // columns past N are zero
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float gj = gelu_tanh(y[j]);
        y[j] = (n + j < N) ? gj : 0.0f;
        am = fmaxf(am, fabsf(y[j]));
      }
      am = row16_max(am);
      float s, inv;
      block_scale(am, s, inv);
      if (m < M) {
        uint2 cw;
        cw.x = e4m3x4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
        cw.y = e4m3x4(y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv);
        *reinterpret_cast<uint2*>(out_codes + (int64_t)m * Np + n) = cw;
        if ((tid & 15) == 0) out_scales[(int64_t)m * (Np >> 7) + n_tile] = s;
        if (prequant) {
          float4* p = reinterpret_cast<float4*>(prequant + (int64_t)m * Np + n);
          p[0] = make_float4(y[0], y[1], y[2], y[3]);
          p[1] = make_float4(y[4], y[5], y[6], y[7]);
        }
      }
    }
  }
}

// n tiles per group of the tile order (grouped_tile): groups of at most 12
// tiles, of near-equal size
static int gemm_group_n(int n_tiles) {
  constexpr int kGroupN = 12;
  const int groups = (n_tiles + kGroupN - 1) / kGroupN;
  return (n_tiles + groups - 1) / groups;
}

hipError_t launch_fp8_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w,
                           const float* w_scales, int M, int N, int K, const uint16_t* bias,
                           const uint16_t* residual, int epilogue, uint16_t* out,
                           uint8_t* out_codes, float* out_scales, float* prequant,
                           hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int Kp = (K + 127) / 128 * 128;
  const int Np = (N + 127) / 128 * 128;
  const int n_tiles = Np / kBN;
  // 64-token tiles when 128-token tiles would give at most one workgroup per
  // CU: twice the workgroups, two per CU, for the same bytes
  const bool small = n_tiles * ((M + 127) / 128) <= device_cu_count();
  const int m_tiles = small ? (M + 63) / 64 : (M + 127) / 128;
  const int nblocks = n_tiles * m_tiles;
  const int group_n = gemm_group_n(n_tiles);
  const dim3 grid(nblocks);
#define VIT_FP8_GEMM_LAUNCH(E, B)                                                                              \
  fp8_gemm_kernel<E, B><<<grid, 256, 0, stream>>>(a, a_scales, w, w_scales, M, N, Np, Kp, n_tiles, nblocks, \
                                                  group_n, bias, residual, out, out_codes, out_scales, prequant)
  switch (epilogue * 2 + (small ? 1 : 0)) {
    case 0: VIT_FP8_GEMM_LAUNCH(0, 128); break;
    case 1: VIT_FP8_GEMM_LAUNCH(0, 64); break;
    case 2: VIT_FP8_GEMM_LAUNCH(1, 128); break;
    case 3: VIT_FP8_GEMM_LAUNCH(1, 64); break;
    case 4: VIT_FP8_GEMM_LAUNCH(2, 128); break;
    case 5: VIT_FP8_GEMM_LAUNCH(2, 64); break;
    default:
      return hipErrorInvalidValue;
  }
#undef VIT_FP8_GEMM_LAUNCH
  return hipGetLastError();
}

// ============================================================ bf16
// Same tiling; K steps of 64 elements (128 bytes per row), 4 MFMAs of K=16
// per step accumulated directly.  A_F32: A is fp32 (rounded to bf16 as it
// is staged into LDS).
template <int EPI, bool A_F32>
__global__ __launch_bounds__(256) void bf16_gemm_kernel(const void* __restrict__ a_ptr,
                                                        const uint16_t* __restrict__ w, int M, int N,
                                                        int K, int n_tiles, int nblocks, int group_n,
                                                        const uint16_t* __restrict__ bias,
                                                        const uint16_t* add,  // may be out (in-place add)
                                                        uint16_t* out, int64_t ld_out) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kTileB];
  uint8_t* a_lds = smem;
  uint8_t* w_lds = smem + 2 * kTileB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int lb = xcd_logical_block(blockIdx.x, nblocks);
  int m_tile, n_tile;
  grouped_tile(lb, nblocks / n_tiles, n_tiles, group_n, m_tile, n_tile);
  const int n0 = n_tile * kBN, m0 = m_tile * kBM;
  const int ksteps = (K + 63) / 64;

  // bf16 A / W: chunk = 8 elements (16 B); row = tid/8 + 32i, col = (tid%8)*8
  // fp32 A: chunk = 4 elements (16 B in, 8 B out); row = tid/16 + 16i, col = (tid%16)*4
  // element offsets from the tile's first row (< 128 K, 32-bit); the tile
  // bases are 64-bit
  const int wcol = (tid & 7) * 8;
  const uint16_t* w_tile = w + (size_t)n0 * K;
  uint32_t w_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w_off[i] = (uint32_t)(min(n0 + (tid >> 3) + 32 * i, N - 1) - n0) * (uint32_t)K + wcol;
  constexpr int NA = A_F32 ? 8 : 4;
  const int acol = A_F32 ? (tid & 15) * 4 : (tid & 7) * 8;
  uint32_t a_off[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = A_F32 ? (tid >> 4) + 16 * i : (tid >> 3) + 32 * i;
    a_off[i] = (uint32_t)(min(m0 + row, M - 1) - m0) * (uint32_t)K + acol;
  }

  u32x4_t rw[4];
  u32x4_t ra16[4];
  f32x4_t ra32[8];
  auto gload = [&](int ks) {
    const int k0 = ks * 64;
    const uint16_t* wk = w_tile + k0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rw[i] = (k0 + wcol < K) ? *reinterpret_cast<const u32x4_t*>(wk + w_off[i]) : u32x4_t{0, 0, 0, 0};
    if constexpr (A_F32) {
      const float* ak = reinterpret_cast<const float*>(a_ptr) + (size_t)m0 * K + k0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        ra32[i] = (k0 + acol < K) ? *reinterpret_cast<const f32x4_t*>(ak + a_off[i]) : f32x4_t{0, 0, 0, 0};
    } else {
      const uint16_t* ak = reinterpret_cast<const uint16_t*>(a_ptr) + (size_t)m0 * K + k0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ra16[i] = (k0 + acol < K) ? *reinterpret_cast<const u32x4_t*>(ak + a_off[i]) : u32x4_t{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4_t*>(w_lds + buf * kTileB + row * kLS + (tid & 7) * 16) = rw[i];
    }
    if constexpr (A_F32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 4) + 16 * i;
        uint2 p;
        p.x = pack_bf16x2(ra32[i][0], ra32[i][1]);
        p.y = pack_bf16x2(ra32[i][2], ra32[i][3]);
        *reinterpret_cast<uint2*>(a_lds + buf * kTileB + row * kLS + (tid & 15) * 8) = p;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        *reinterpret_cast<u32x4_t*>(a_lds + buf * kTileB + row * kLS + (tid & 7) * 16) = ra16[i];
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
    const uint8_t* wl = w_lds + buf * kTileB + (64 * wn + l32) * kLS + 16 * g;
    const uint8_t* al = a_lds + buf * kTileB + (64 * wm + l32) * kLS + 16 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t wop[2], aop[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        wop[t] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(wl + 32 * t * kLS + 32 * kk));
        aop[t] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(al + 32 * t * kLS + 32 * kk));
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

  // epilogue: bias and the added rows are loaded before the tile is parked,
  // and all eight rows of a thread are read from LDS before the first is
  // finished (as in the FP8 kernel)
  const int cc = (tid & 15) * 8;
  const int n = n0 + cc;
  float b8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b8[j] = (bias && n + j < N) ? bf2f(bias[n + j]) : 0.0f;
  const bool vec = n + 8 <= N && (N & 7) == 0 && (ld_out & 7) == 0;
  uint4 add8[8];
  if constexpr (EPI == 2) {
    if (add && vec) {
#pragma unroll
      for (int pass = 0; pass < 8; ++pass) {
        const int m = min(m0 + (tid >> 4) + 16 * pass, M - 1);
        add8[pass] = *reinterpret_cast<const uint4*>(add + (int64_t)m * N + n);
      }
    }
  }
  float* c_lds = reinterpret_cast<float*>(smem);
  park_acc<2>(c_lds, acc, wn, wm, l32, g);
  tile_barrier();
  float4 cv[8][2];
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const int ml = (tid >> 4) + 16 * pass;
    cv[pass][0] = *reinterpret_cast<const float4*>(c_lds + ml * kCS + cc);
    cv[pass][1] = *reinterpret_cast<const float4*>(c_lds + ml * kCS + cc + 4);
  }
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const int m = m0 + (tid >> 4) + 16 * pass;
    const float4 c0 = cv[pass][0], c1 = cv[pass][1];
    float y[8] = {c0.x + b8[0], c0.y + b8[1], c0.z + b8[2], c0.w + b8[3],
                  c1.x + b8[4], c1.y + b8[5], c1.z + b8[6], c1.w + b8[7]};
    if constexpr (EPI == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = gelu_tanh(y[j]);
    }
    if (m < M) {
      if constexpr (EPI == 2) {
        if (add) {
          if (vec) {
            const uint4 u = add8[pass];
            y[0] += bf_lo(u.x); y[1] += bf_hi(u.x); y[2] += bf_lo(u.y); y[3] += bf_hi(u.y);
            y[4] += bf_lo(u.z); y[5] += bf_hi(u.z); y[6] += bf_lo(u.w); y[7] += bf_hi(u.w);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] += (n + j < N) ? bf2f(add[(int64_t)m * N + n + j]) : 0.0f;
          }
        }
      }
      if (vec) {
        uint4 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        o.z = pack_bf16x2(y[4], y[5]);
        o.w = pack_bf16x2(y[6], y[7]);
        *reinterpret_cast<uint4*>(out + (int64_t)m * ld_out + n) = o;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (n + j < N) out[(int64_t)m * ld_out + n + j] = f2bf(y[j]);
      }
    }
  }
}

hipError_t launch_bf16_gemm(const void* a, bool a_f32, const uint16_t* w, int M, int N, int K,
                            const uint16_t* bias, const uint16_t* add, int epilogue,
                            uint16_t* out, int64_t ld_out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (!a_f32 && epilogue != 2 && bf16_gemm_wide_fits(N, K, ld_out, out, bias))
    return launch_bf16_gemm_wide(static_cast<const uint16_t*>(a), w, M, N, K, bias, epilogue, out, ld_out, stream);
  const int n_tiles = (N + kBN - 1) / kBN, m_tiles = (M + kBM - 1) / kBM;
  const int nblocks = n_tiles * m_tiles;
  const dim3 grid(nblocks);
#define VIT_BG(E, F)                                                                                        \
  bf16_gemm_kernel<E, F><<<grid, 256, 0, stream>>>(a, w, M, N, K, n_tiles, nblocks, gemm_group_n(n_tiles), bias, \
                                                   add, out, ld_out)
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
