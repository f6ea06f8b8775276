// bf16 GEMM with 256-wide tiles for the merger MLPs (FlashRT "Qwen3-VL-8B
// on RTX 5090" page, section 4: the mergers stay bf16; spark_model
// "layers/vision_encoder.rs": C[M,N] = A[M,K] @ W[N,K]^T + bias): bf16
// activations with N % 256 == 0 and K % 192 == 0, the other cases go to
// bf16_gemm_kernel (gemm.hip).  For small M the same kernel runs on 64 x 64
// tiles (below).
//
// gfx950 design: 256 (n) x 128 (m) tiles, 8 waves of 64 (n) x 64 (m) (two
// per SIMD, 4 x 2 over the tile) on v_mfma_f32_16x16x32_bf16 (operand lane
// l: row l % 16, k 8 (l / 16) .. +8; result lane l: rows n 4 (l / 16) +
// 0..3 of column m l % 16).  A tile takes a quarter fewer global bytes per
// multiply-add than a 128 x 128 one.  The 1564 x 4608 merger fc1 is 234
// tiles, one workgroup per CU: the latency of the global loads is hidden by
// depth, each 64-deep K step being copied global -> LDS directly (buffer
// loads with the LDS as destination, no registers) two steps before it is
// used, into a ring of three stages, and the LDS reads of one wave hide
// behind the MFMAs of the other wave on its SIMD.  An XOR swizzle chosen on
// the global side keeps the 16-byte operand reads conflict-free in 128-byte
// rows.  The epilogue writes from the accumulators (four features of a
// token per 8-byte store).
#include "common.h"
#include "kernels.h"

namespace vit {

namespace {
constexpr int kRowB = 128;         // bytes per tile row and K step (64 bf16)
}  // namespace

// Tile shapes.  Wide: 256 (n) x 128 (m), 8 waves of 64 x 64 (4 x 2).
// Small, for M so small that wide tiles would leave most CUs idle (the
// mergers of images up to about 2000 patches): 64 x 64, 4 waves of 32 x 32
// (2 x 2), three to a CU.  Both compute every 16 x 16 output block as the
// same chain of 16x16x32 MFMAs over K, so they write the same bytes.
template <int WT, int NW, int MW>
struct WideShape {
  static constexpr int kWT = WT;               // wave tile (n and m)
  static constexpr int kNW = NW, kMW = MW;     // waves along n and m
  static constexpr int kWaves = NW * MW;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBN = WT * NW;          // output features per tile
  static constexpr int kBM = WT * MW;          // tokens per tile
  static constexpr int kSub = WT / 16;         // 16 x 16 blocks per wave and axis
  static constexpr int kCopyW = kBN / (8 * kWaves), kCopyA = kBM / (8 * kWaves);
  static constexpr int kStageW = kBN * kRowB, kStageA = kBM * kRowB;
};
using WideTile = WideShape<64, 4, 2>;
using SmallTile = WideShape<32, 2, 2>;

// Global -> LDS copy of one K step of a tile: wave instruction j of wave w
// fills LDS bytes [1024 (w + W j), +1024), i.e. rows 8 (w + W j) .. +8, for
// W waves.  Lane l lands at row 8 (w + W j) + l / 8, 16-byte slot p = l % 8,
// and loads the row's chunk p ^ ((row / 2) % 8) (the same 128-byte line):
// slot p of row r holds chunk p ^ ((r / 2) % 8).
__device__ __forceinline__ uint32_t swz_off(int row, int lane, int K) {
  const int p = lane & 7;
  return ((uint32_t)row * (uint32_t)K + 8 * (p ^ ((row >> 1) & 7))) * 2;
}

// Operand read: 16 bytes of k chunk c (0..7) of tile row r.
__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* stage, int r, int c) {
  return __builtin_bit_cast(bf16x8_t,
                            *reinterpret_cast<const uint4*>(stage + r * kRowB + 16 * (c ^ ((r >> 1) & 7))));
}

template <int EPI, class S>
__global__ __launch_bounds__(S::kThreads) void bf16_gemm_wide_kernel(const uint16_t* __restrict__ a,
                                                                const uint16_t* __restrict__ w, int M, int N, int K,
                                                                int n_tiles, int nblocks, int group_n,
                                                                const uint16_t* __restrict__ bias, uint16_t* out,
                                                                int64_t ld_out) {
  constexpr int kBN = S::kBN, kBM = S::kBM, kWaves = S::kWaves, kSub = S::kSub, kWT = S::kWT;
  constexpr int kCopyW = S::kCopyW, kCopyA = S::kCopyA;
  // three stages as separate arrays, so that the compiler's wait before a
  // read covers only the copies into that stage
  __shared__ __attribute__((aligned(16))) uint8_t w_s0[S::kStageW], w_s1[S::kStageW], w_s2[S::kStageW];
  __shared__ __attribute__((aligned(16))) uint8_t a_s0[S::kStageA], a_s1[S::kStageA], a_s2[S::kStageA];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % S::kNW, wm = wave / S::kNW;
  const int l16 = lane & 15, lg = lane >> 4;
  const int lb = xcd_logical_block(blockIdx.x, nblocks);
  int m_tile, n_tile;
  grouped_tile(lb, nblocks / n_tiles, n_tiles, group_n, m_tile, n_tile);
  const int n0 = n_tile * kBN, m0 = m_tile * kBM;
  const int ksteps = K / 64;

  // buffer descriptors of the two operand tiles; A rows past M re-read row M - 1
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w + (size_t)n0 * K), (short)0, kBN * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a + (size_t)m0 * K), (short)0, min(M - m0, kBM) * K * 2, 0x00020000);
  uint32_t w_off[kCopyW], a_off[kCopyA];
#pragma unroll
  for (int j = 0; j < kCopyW; ++j) w_off[j] = swz_off(8 * (wave + kWaves * j) + (lane >> 3), lane, K);
#pragma unroll
  for (int j = 0; j < kCopyA; ++j) {
    const int r = 8 * (wave + kWaves * j) + (lane >> 3);
    const int rc = min(m0 + r, M - 1) - m0;
    a_off[j] = ((uint32_t)rc * (uint32_t)K + 8 * ((lane & 7) ^ ((r >> 1) & 7))) * 2;
  }
  auto copy_step = [&](uint8_t* ws, uint8_t* as, int ks) {
#pragma unroll
    for (int j = 0; j < kCopyW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, ws + 1024 * (wave + kWaves * j), 16, (int)w_off[j], ks * 128,
                                               0, 0);
#pragma unroll
    for (int j = 0; j < kCopyA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, as + 1024 * (wave + kWaves * j), 16, (int)a_off[j], ks * 128,
                                               0, 0);
  };

  f32x4_t acc[kSub][kSub];
#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int j = 0; j < kSub; ++j) acc[i][j] = f32x4_t{};
  // one K step from a stage: per 32 k, the A fragments, then the W
  // fragments, each read kFA - 1 = 2 ahead of its MFMAs
  constexpr int kFA = 3;
  auto compute = [&](const uint8_t* ws, const uint8_t* as) {
    const int wr = kWT * wn + l16, ar = kWT * wm + l16;
    // i = kSub kk + ns
    auto w_frag = [&](int i) { return lds_frag(ws, wr + 16 * (i % kSub), 4 * (i / kSub) + lg); };
    bf16x8_t wf[kFA];
#pragma unroll
    for (int i = 0; i < kFA - 1; ++i) wf[i] = w_frag(i);
    bf16x8_t aop[2][kSub];
#pragma unroll
    for (int ms = 0; ms < kSub; ++ms) aop[0][ms] = lds_frag(as, ar + 16 * ms, lg);
#pragma unroll
    for (int i = 0; i < 2 * kSub; ++i) {
      const int kk = i / kSub, ns = i % kSub;
      if (i + kFA - 1 < 2 * kSub) wf[(i + kFA - 1) % kFA] = w_frag(i + kFA - 1);
      if (i == 1) {
#pragma unroll
        for (int ms = 0; ms < kSub; ++ms) aop[1][ms] = lds_frag(as, ar + 16 * ms, 4 + lg);
      }
#pragma unroll
      for (int ms = 0; ms < kSub; ++ms)
        acc[ns][ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i % kFA], aop[kk][ms], acc[ns][ms], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Step s reads stage s % 3.  Its copy was issued two steps earlier; each
  // wave waits for its own copy (all but the copies of step s + 1: 6 per
  // wave for the wide tile, 4 for the small one) and for its LDS reads of
  // step s - 1, then the barrier: the stage is whole, and stage (s + 2) % 3,
  // read at step s - 1, is free for the next copy.
  // K steps come in threes (K % 192 == 0), so every step has the same shape:
  // the last two steps copy the final K step once more into their free stage
  // rather than branch (a branch around the copies costs a full wait).
  const int last = ksteps - 1;
  copy_step(w_s0, a_s0, 0);
  copy_step(w_s1, a_s1, 1);
  auto step = [&](int ks, const uint8_t* ws, const uint8_t* as, uint8_t* wn2, uint8_t* an2) {
    if constexpr (kCopyW + kCopyA == 6)
      asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    copy_step(wn2, an2, min(ks + 2, last));
    compute(ws, as);
  };
  for (int ks = 0; ks < ksteps; ks += 3) {
    step(ks, w_s0, a_s0, w_s2, a_s2);
    step(ks + 1, w_s1, a_s1, w_s0, a_s0);
    step(ks + 2, w_s2, a_s2, w_s1, a_s1);
  }
  // the surplus copies land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue from the accumulators: lane holds features n0 + WT wn + 16 ns
  // + 4 (lane / 16) + 0..3 of token m0 + WT wm + 16 ms + lane % 16; four
  // consecutive features are one 8-byte store (the 16 lanes of a token
  // row group write 32 contiguous bytes per instruction)
#pragma unroll
  for (int ns = 0; ns < kSub; ++ns) {
    const int n = n0 + kWT * wn + 16 * ns + 4 * lg;
    float b4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (bias) {
      const uint2 bw = *reinterpret_cast<const uint2*>(bias + n);
      b4[0] = bf_lo(bw.x);
      b4[1] = bf_hi(bw.x);
      b4[2] = bf_lo(bw.y);
      b4[3] = bf_hi(bw.y);
    }
#pragma unroll
    for (int ms = 0; ms < kSub; ++ms) {
      const int m = m0 + kWT * wm + 16 * ms + l16;
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[r] = acc[ns][ms][r] + b4[r];
        if constexpr (EPI == 1) y[r] = gelu_tanh(y[r]);
      }
      if (m < M)
        *reinterpret_cast<uint2*>(out + (int64_t)m * ld_out + n) = make_uint2(pack_bf16x2(y[0], y[1]),
                                                                              pack_bf16x2(y[2], y[3]));
    }
  }
}

bool bf16_gemm_wide_fits(int N, int K, int64_t ld_out, const void* out, const void* bias) {
  return N % WideTile::kBN == 0 && K % 192 == 0 && K > 0 && (ld_out & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0 &&
         (reinterpret_cast<uintptr_t>(bias) & 7) == 0;
}

hipError_t launch_bf16_gemm_wide(const uint16_t* a, const uint16_t* w, int M, int N, int K, const uint16_t* bias,
                                 int epilogue, uint16_t* out, int64_t ld_out, hipStream_t stream) {
  if (epilogue != 0 && epilogue != 1) return hipErrorInvalidValue;
  // 64 x 64 tiles (8 per wide tile) while there are at most 2.25 of them per
  // CU: a CU takes about twice as long per output on them as on wide tiles,
  // so they pay off only where wide tiles leave most CUs idle (the merger
  // fc2, N 4096 and K 4608, one box: 21 against 53 us at M = 243, 31
  // against 55 at 456, 65 against 58 at 972)
  const int wide_tiles = N / WideTile::kBN * ((M + WideTile::kBM - 1) / WideTile::kBM);
  if (4 * 8 * wide_tiles > 9 * device_cu_count()) {
    const int n_tiles = N / WideTile::kBN, m_tiles = (M + WideTile::kBM - 1) / WideTile::kBM;
    const int nblocks = n_tiles * m_tiles;
    // groups of 4 n tiles: the tiles one XCD holds at a time span about as
    // many W bytes (4 x 256 rows) as A bytes (7-8 x 128 rows)
    const int group_n = min(4, n_tiles);
    if (epilogue == 0)
      bf16_gemm_wide_kernel<0, WideTile><<<nblocks, WideTile::kThreads, 0, stream>>>(
          a, w, M, N, K, n_tiles, nblocks, group_n, bias, out, ld_out);
    else
      bf16_gemm_wide_kernel<1, WideTile><<<nblocks, WideTile::kThreads, 0, stream>>>(
          a, w, M, N, K, n_tiles, nblocks, group_n, bias, out, ld_out);
  } else {
    // walked in groups of 16 n tiles (1024 W rows) over every m tile
    const int n_tiles = N / SmallTile::kBN, m_tiles = (M + SmallTile::kBM - 1) / SmallTile::kBM;
    const int nblocks = n_tiles * m_tiles;
    const int group_n = min(16, n_tiles);
    if (epilogue == 0)
      bf16_gemm_wide_kernel<0, SmallTile><<<nblocks, SmallTile::kThreads, 0, stream>>>(
          a, w, M, N, K, n_tiles, nblocks, group_n, bias, out, ld_out);
    else
      bf16_gemm_wide_kernel<1, SmallTile><<<nblocks, SmallTile::kThreads, 0, stream>>>(
          a, w, M, N, K, n_tiles, nblocks, group_n, bias, out, ld_out);
  }
  return hipGetLastError();
}

}  // namespace vit
