// Full bidirectional attention over cu_seqlens windows, head_dim 72, bf16
// MFMA with an fp32 online softmax (FlashRT "Qwen3-VL-8B on RTX 5090" page,
// section 3: "FA2 (full, bidirectional)"; section 5: every image is its own
// cu_seqlens attention window; section 1: this attention is the largest cost
// of the tower and is compute-bound).
//
// gfx950 design (not the page's sm_120 kernel):
//  * Persistent stream-K grid: one 512-thread workgroup (8 waves, two per
//    SIMD) per CU.  The unit of work is one 64-key tile of one work item
//    (head, window, 256-query tile); the whole ordered list of key tiles is
//    cut into equal contiguous ranges, one per workgroup, so the load is
//    even whatever the window lengths.  An item cut by a range boundary
//    leaves fp32 partials (O, l, m) that a small second kernel merges in key
//    order, so the result does not depend on timing.
//  * Each wave owns 32 queries of the item for its whole key range.
//    Everything is computed transposed, S^T = K Q^T and O^T = V^T P^T, with
//    v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane holds
//    one column (lane % 32) and 16 rows, so every lane owns ONE query: the
//    row max and the rescale of O stay in the lane's registers, plus one
//    cross-half exchange (v_permlane32_swap) per tile.
//  * P never leaves registers: the 16 key-rows a lane holds in S^T are, in
//    order, the 8+8 k-slots of the B operand of two PV MFMAs (the key order
//    inside an MFMA is a free permutation as long as V^T uses the same one).
//  * head_dim 72 is padded to 80 for Q K^T (5 MFMAs of K=16) and to 96 rows
//    for V^T (3 row tiles of 32).  Of the third V^T tile, row 72 is all ones:
//    its output row is the softmax denominator (sum of the bf16 P actually
//    multiplied), accumulated and rescaled by the MFMA for free; rows 73..95
//    are zero.  Q's padding column 72 is 1.0, which turns K's column 72 into
//    an additive key mask inside the MFMA (no VALU masking).
//  * Software pipeline across key tiles: while the VALU turns S(j) into P(j)
//    (exp2 with the scale folded in), the MFMA unit already computes S(j+1);
//    then the PV MFMAs of tile j run, interleaved by hand with the row max
//    of S(j+1).  K and V^T tiles live in a 6-buffer LDS ring with one
//    barrier per two tiles; a tile is stored three steps before its K is
//    read, and its global loads are issued two steps before that (two
//    register sets).  Half the barriers of a 4-buffer ring with one barrier
//    per tile: 2-3 % off the kernel.
//  * The two waves that share a SIMD run opposite phases: waves 4..7 take
//    each barrier between their QK/exp phase (VALU-heavy) and their PV phase
//    (MFMA-heavy), waves 0..3 after the PV phase, so one wave's exp work
//    overlaps the other's PV MFMAs.
//  * The running max is only raised (and O rescaled) when a row max grows
//    by more than 2^8 over it: exact after the final division by the row
//    sum, and it removes the per-tile rescale of 48 accumulators.
//  * Row strides in LDS (88 bf16 for K, 68 for V^T) keep the ds_read_b128 /
//    ds_read_b64 operand fetches and the staging writes bank-conflict free.
//  * K/V tiles are fetched with buffer loads whose descriptor starts at the
//    tile's first row and ends at the last token: per-thread offsets are
//    fixed for the whole loop (no per-tile address arithmetic), and rows
//    past the last token read as zero in hardware, so no clamping is needed
//    (rows of the next window inside the batch are finite and masked).
//  * Items are ordered head-major and cut into one range per workgroup
//    (a range holds about 1.5 items at 6256 tokens, so at most one cut per
//    range boundary), with ids mapped so that each XCD takes a contiguous
//    run of the order: an XCD's 32 workgroups share two heads' K/V in its
//    L2.  Two rounds of half-size ranges would give each XCD one head at a
//    time (a third of the L2 misses) but cut nearly every item: the kernel
//    time is the same and the combine takes half again as long.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace vit {

namespace {
constexpr int kHD = 72;
constexpr int kThreads = 512;     // 8 waves: two per SIMD (one wave per SIMD cannot overlap its
                                  // own MFMA and VALU work well enough)
constexpr int kBQ = 256;          // queries per workgroup: 32 per wave
constexpr int kBK = 64;           // keys per tile
constexpr int kKS = 88;           // K row stride in LDS (bf16): 80 used
constexpr int kVS = 68;           // V^T row stride in LDS (bf16): 64 used
constexpr int kKBuf = kBK * kKS;  // elements per K buffer
constexpr int kVRows = kHD + 2;  // V^T rows 0..71, row 72 = ones, row 73 = zeros
constexpr int kVBuf = kVRows * kVS;
// Key tiles per workgroup barrier: two.  A tile is stored kAhead = 3 steps
// before the step whose QK phase reads it, and its stage is reused kStages = 6
// tiles later: between two barriers (after the odd steps) an interval reads
// tiles j-1 .. j+2 and writes tiles j+3, j+4.  (One barrier per tile with a
// 4-stage ring was 2-3 % slower.)
constexpr int kAhead = 3;
constexpr int kStages = 6;
constexpr float kLazy = 8.0f;     // rescale only when the max grows by > 2^8
constexpr int kFragAhead = 2;     // LDS operand fragments read this many MFMAs ahead
}  // namespace

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// Workgroup barrier for the LDS ring: this wave's LDS writes are complete,
// its global loads in flight are not waited for (they only feed registers).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Staging of one K/V tile.  K: 64 rows x 9 chunks of 16 B = 576 chunks,
// thread t owns chunks t, t + kThreads, ... (below 576).  V: 16 groups of 4 keys
// x 9 chunks of 8 d = 144 items on threads 64..207 (v thread vt = t - 64),
// 4 x 16 B each, transposed into V^T on the way to LDS.  All offsets are
// fixed per thread.
// V item mapping: lane group vt/16 picks the d chunk, vt%16 the key group,
// with chunks ordered 0,2,1,3,4,6,5,7,8 so that the two 16-lane halves of
// every 32-lane LDS write phase hit V^T rows 16 apart: with the 34-dword row
// stride those are 32 banks apart, and each phase writes 64 distinct banks.
constexpr int kVThread0 = 64;

constexpr int kKChunks = (576 + kThreads - 1) / kThreads;  // K chunks per thread

struct KVRegs {
  u32x4_t k[kKChunks];
  u32x4_t v[4];
};

struct KVPlan {
  uint32_t kgoff[kKChunks];  // byte offsets of the K chunks within a tile
  int klds[kKChunks];        // their LDS element offsets
  uint32_t vgoff;     // byte offset of key 4*vkg, chunk vc within a tile
  uint32_t vstride;   // bytes per row
  int vlds;           // V^T LDS offset of row 8*vc, column 4*vkg
};

__device__ __forceinline__ KVPlan make_plan(int tid, int64_t ld, int64_t hoff) {
  KVPlan p;
#pragma unroll
  for (int i = 0; i < kKChunks; ++i) {
    // 16 consecutive chunks = 16 consecutive rows of one column: the 16 lanes
    // of each ds_write_b128 phase hit distinct banks (44-dword row stride)
    const int c = min(tid + kThreads * i, 575);
    const int blk = c >> 4;
    const int row = (blk / 9) * 16 + (c & 15), col = blk % 9;
    p.kgoff[i] = (uint32_t)((row * ld + hoff + col * 8) * 2);
    p.klds[i] = row * kKS + col * 8;
  }
  const int vt = min(max(tid - kVThread0, 0), 143);
  const int vgrp = vt >> 4;
  const int vc = (vgrp == 1 || vgrp == 5) ? vgrp + 1 : ((vgrp == 2 || vgrp == 6) ? vgrp - 1 : vgrp);
  const int vkg = vt & 15;
  p.vgoff = (uint32_t)((4 * vkg * ld + hoff + vc * 8) * 2);
  p.vstride = (uint32_t)(ld * 2);
  p.vlds = 8 * vc * kVS + 4 * vkg;
  return p;
}

// Buffer descriptor over rows [row0, total) of a [total, ld] bf16 array.  Its
// record count is clamped to 2^31 - 1 bytes: loads reach at most one 64-row
// tile past row0, so the clamp only matters where the end of the array is
// far beyond every load (a window of more than 2^31 bytes of rows).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int64_t ld, int row0, int total) {
  const uint16_t* p = base + (int64_t)row0 * ld;
  const int64_t bytes = min((int64_t)(total - row0) * ld * 2, (int64_t)0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, (int)(bytes > 0 ? bytes : 0),
                                           0x00020000);
}

__device__ __forceinline__ u32x4_t buf_ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ void load_kv(KVRegs& r, const KVPlan& p, const uint16_t* __restrict__ k,
                                        const uint16_t* __restrict__ v, int64_t ld, int row0, int total,
                                        int tid) {
  const __amdgpu_buffer_rsrc_t kr = rows_rsrc(k, ld, row0, total);
  const __amdgpu_buffer_rsrc_t vr = rows_rsrc(v, ld, row0, total);
#pragma unroll
  for (int i = 0; i < kKChunks; ++i)
    if (tid + kThreads * i < 576) r.k[i] = buf_ld(kr, p.kgoff[i]);
  if (tid >= kVThread0 && tid < kVThread0 + 144) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = buf_ld(vr, p.vgoff + i * p.vstride);
  }
}

__device__ __forceinline__ void store_kv(const KVRegs& r, const KVPlan& p, uint16_t* __restrict__ ks,
                                         uint16_t* __restrict__ vt, int tid) {
#pragma unroll
  for (int i = 0; i < kKChunks; ++i)
    if (tid + kThreads * i < 576) *reinterpret_cast<u32x4_t*>(ks + p.klds[i]) = r.k[i];
  if (tid >= kVThread0 && tid < kVThread0 + 144) {
    // r.v[i] holds d = 8vc..8vc+7 of key 4vkg+i (dword j = d 8vc+2j, 8vc+2j+1);
    // write V^T[8vc+2j (+1)][4vkg .. 4vkg+3] with byte permutes.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 lo, hi;
      lo.x = __builtin_amdgcn_perm(r.v[1][j], r.v[0][j], 0x05040100u);
      lo.y = __builtin_amdgcn_perm(r.v[3][j], r.v[2][j], 0x05040100u);
      hi.x = __builtin_amdgcn_perm(r.v[1][j], r.v[0][j], 0x07060302u);
      hi.y = __builtin_amdgcn_perm(r.v[3][j], r.v[2][j], 0x07060302u);
      *reinterpret_cast<uint2*>(vt + p.vlds + 2 * j * kVS) = lo;
      *reinterpret_cast<uint2*>(vt + p.vlds + (2 * j + 1) * kVS) = hi;
    }
  }
}

// S^T tile (64 keys x 32 queries) = K Q^T from the K buffer.
__device__ __forceinline__ void qk_tile(f32x16_t s[2], const uint16_t* __restrict__ ks, const bf16x8_t qf[5],
                                        int l32, int g) {
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    s[jt] = f32x16_t{};
    const uint16_t* kr = ks + (32 * jt + l32) * kKS + 8 * g;
#pragma unroll
    for (int kc = 0; kc < 5; ++kc)
      s[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(kr + 16 * kc), qf[kc], s[jt], 0, 0, 0);
  }
}

// max of x over lanes l and l ^ 32 (v_permlane32_swap: a VALU exchange of
// the two wave halves; the pair returned holds the lane's own value and its
// partner's)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// Softmax numerators of one S^T tile: P = exp2(S * scale - m) as the bf16
// B operands of the PV MFMAs.
__device__ __forceinline__ void exp_tile(bf16x8_t pb[2][2], const f32x16_t s[2], float scale_log2, float m) {
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(s[jt][8 * h + j], scale_log2, -m));
      u32x4_t w;
      w[0] = pack_bf16x2(p[0], p[1]);
      w[1] = pack_bf16x2(p[2], p[3]);
      w[2] = pack_bf16x2(p[4], p[5]);
      w[3] = pack_bf16x2(p[6], p[7]);
      pb[jt][h] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
}

// V^T fragment of PV MFMA i (i % 3 = row tile dt, i / 3 = 16-key slot).
__device__ __forceinline__ bf16x8_t v_frag(const uint16_t* __restrict__ vt, int i, int l32, int g, int vrow2) {
  const int dt = i % 3, ksl = i / 3;
  const uint16_t* vr = vt + (dt < 2 ? 32 * dt + l32 : vrow2) * kVS + 4 * g + 16 * ksl;
  const uint2 a0 = *reinterpret_cast<const uint2*>(vr);
  const uint2 a1 = *reinterpret_cast<const uint2*>(vr + 8);
  return __builtin_bit_cast(bf16x8_t, u32x4_t{a0.x, a0.y, a1.x, a1.y});
}

// O^T += V^T P^T for one key tile (V^T stage `vt`), not interleaved.
__device__ __forceinline__ void pv_tile(f32x16_t acc[3], const uint16_t* __restrict__ vt, const bf16x8_t pb[2][2],
                                        int l32, int g, int vrow2) {
#pragma unroll
  for (int i = 0; i < 12; ++i)
    acc[i % 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(vt, i, l32, g, vrow2), pb[(i / 3) >> 1][(i / 3) & 1],
                                                         acc[i % 3], 0, 0, 0);
}

// Scaled row max (log2 units) of one S^T tile: each lane owns one query.
__device__ __forceinline__ float tile_max(const f32x16_t s[2], float scale_log2) {
  float a = fmaxf(s[0][0], s[0][1]), b = fmaxf(s[1][0], s[1][1]);
#pragma unroll
  for (int rr = 2; rr < 16; ++rr) {
    a = fmaxf(a, s[0][rr]);
    b = fmaxf(b, s[1][rr]);
  }
  return halves_max(fmaxf(a, b)) * scale_log2;
}

// The steady-state work of one key tile, interleaved by hand.  A wave issues
// in order, so a long run of VALU work with no MFMA in it leaves the matrix
// core idle; here every slot issues one MFMA followed by the VALU work that
// fits under it:
//   phase 1: the 10 MFMAs of S(j+1) = K(j+1) Q^T, each with 1-2 pairs of the
//            exp2 of P(j);
//   phase 2: the 12 MFMAs of O^T += V^T(j) P(j)^T, each with a share of the
//            row max of S(j+1).
// Consecutive MFMAs write different accumulators, LDS operand fragments are
// read two MFMAs ahead, and sched_barrier keeps the compiler from regrouping
// the slots.  Returns the scaled row max of S(j+1).
template <class Stage>
__device__ __forceinline__ float tile_step(f32x16_t s_nxt[2], f32x16_t acc[3], const f32x16_t s_cur[2],
                                           const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vt,
                                           const bf16x8_t qf[5], float scale_log2, float m, int l32, int g,
                                           int vrow2, Stage&& stage) {
  // K fragment i: key half jt = i & 1, d chunk kc = i >> 1
  const uint16_t* kr = ks + l32 * kKS + 8 * g;
  auto k_frag = [&](int i) { return ld_bf16x8(kr + (i & 1) * 32 * kKS + 16 * (i >> 1)); };

  u32x4_t pw[4];  // P(j) as bf16 pairs: pw[ksl] holds keys 16 ksl .. 16 ksl + 15
  constexpr int PF = kFragAhead;
  bf16x8_t kf[PF + 1];
#pragma unroll
  for (int i = 0; i < PF; ++i) kf[i] = k_frag(i);
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i + PF < 10) kf[(i + PF) % (PF + 1)] = k_frag(i + PF);
    const int jt = i & 1, kc = i >> 1;
    s_nxt[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % (PF + 1)], qf[kc], kc == 0 ? f32x16_t{} : s_nxt[jt], 0,
                                                        0, 0);
#pragma unroll
    for (int e2 = 16 * i / 10; e2 < 16 * (i + 1) / 10; ++e2) {
      const int e = 2 * e2, jc = e >> 4, rr = e & 15;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s_cur[jc][rr], scale_log2, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s_cur[jc][rr + 1], scale_log2, -m));
      pw[e >> 3][(e & 7) >> 1] = pack_bf16x2(p0, p1);
    }
    stage(i);
    __builtin_amdgcn_sched_barrier(0);
  }

  bf16x8_t vf[PF + 1];
#pragma unroll
  for (int i = 0; i < PF; ++i) vf[i] = v_frag(vt, i, l32, g, vrow2);
  float ma = -INFINITY, mb = -INFINITY;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    if (i + PF < 12) vf[(i + PF) % (PF + 1)] = v_frag(vt, i + PF, l32, g, vrow2);
    acc[i % 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % (PF + 1)], __builtin_bit_cast(bf16x8_t, pw[i / 3]),
                                                         acc[i % 3], 0, 0, 0);
#pragma unroll
    for (int e = 32 * i / 12; e < 32 * (i + 1) / 12; ++e) {
      if (e & 1)
        mb = fmaxf(mb, s_nxt[e >> 4][e & 15]);
      else
        ma = fmaxf(ma, s_nxt[e >> 4][e & 15]);
    }
    // keep this slot's share of the max here (IR passes would otherwise
    // sink the whole reduction past the last MFMA)
    asm volatile("" : "+v"(ma), "+v"(mb));
    stage(10 + i);
    __builtin_amdgcn_sched_barrier(0);
  }
  return halves_max(fmaxf(ma, mb)) * scale_log2;
}

// Key masking costs no VALU work: Q carries 1.0 in padding column 72 and K
// carries 0 there, except for the key rows of the last tile that lie past
// the window, whose column 72 holds the most negative finite bf16.  Their
// scores come out of the MFMA near -3.4e38 and their P underflows to 0.
constexpr uint32_t kMaskedKey = 0xff7fu;  // bf16 -3.39e38

// Partial result of a segment that does not cover its item's whole key
// range: rows 0..71 unnormalised O^T, row 72 the row sum l, row 73 the
// running max m (log2 units), one column per query of the 256-query tile, fp32.
constexpr int kSlotRows = kHD + 2;
constexpr int kSlotFloats = kSlotRows * kBQ;
constexpr int kMaxWorkgroups = kAttnMaxRanges;
// The work order is cut into one range per workgroup; a range can leave at
// most two partial slots (an item cut at its start, one cut at its end).
constexpr int kMaxRanges = kMaxWorkgroups;

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  const int32_t* cu;
  float* partial;         // [2 * num_ranges][kSlotRows][kBQ]
  int64_t ld, ldo;
  int64_t work_per_head;  // sum over windows of (q tiles x key tiles)
  int64_t work;           // work_per_head * heads
  int num_seqs, heads, total, num_wgs, num_ranges;
  float scale_log2;
  AttnRangeStart start[kAttnMaxRanges];  // where each range starts (host plan)
};

// Work item = (head, window, q tile); its key tiles are the unit of work.
// Items are ordered head-major, so the contiguous ranges that the XCD
// mapping gives each XCD touch one or two heads' K/V.
struct Segment {
  int head, win, seq_begin, seq_len, qtile, kt, nq, nk;  // kt: first key tile of the segment
};

__device__ __forceinline__ int64_t range_start(const AttnParams& a, int r) {
  return (int64_t)r * a.work / a.num_ranges;
}

// Key tile `rem` (q tile rem / nk, key tile rem % nk) of window `win`, head `head`.
__device__ __forceinline__ Segment segment_at(const AttnParams& a, int head, int win, int rem) {
  Segment s;
  s.head = head;
  s.win = win;
  s.seq_begin = a.cu[win];
  s.seq_len = a.cu[win + 1] - s.seq_begin;
  s.nq = (s.seq_len + kBQ - 1) / kBQ;
  s.nk = (s.seq_len + kBK - 1) / kBK;
  s.qtile = rem / max(s.nk, 1);
  s.kt = rem - s.qtile * s.nk;
  return s;
}

// First segment of range r: its window and position come from the host's
// plan, its head from the range's start in the work order.
__device__ __forceinline__ Segment range_first(const AttnParams& a, int r) {
  const int head = (int)(range_start(a, r) / a.work_per_head);
  return segment_at(a, head, a.start[r].win, a.start[r].rem);
}

// The item after the one s belongs to (its first key tile): the next q tile
// of the window, else the next non-empty window, else window 0 of the next
// head.  Only called while work remains, so a non-empty window follows.
__device__ __forceinline__ Segment next_item(const AttnParams& a, const Segment& s) {
  if (s.qtile + 1 < s.nq) return segment_at(a, s.head, s.win, (s.qtile + 1) * s.nk);
  int head = s.head, w = s.win + 1;
  for (;;) {
    if (w >= a.num_seqs) {
      w = 0;
      ++head;
    }
    if (a.cu[w + 1] > a.cu[w]) break;
    ++w;
  }
  return segment_at(a, head, w, 0);
}

// Key tiles [s.kt, kt_end) of one item: the pipelined flash loop.  With
// slot == nullptr the segment covers the whole key range and writes the
// normalised bf16 output, otherwise its partial (O, l, m) goes to slot.
template <bool kLate>
__device__ __forceinline__ void run_segment(const AttnParams& a, const Segment& s, int kt_end, float* slot,
                                            uint16_t* __restrict__ ks_mem, uint16_t* __restrict__ vt_mem) {
  // an opaque copy of the thread id: addresses derived from it are rebuilt
  // per segment instead of being hoisted out of the segment loop, where they
  // would stay live in registers across the whole flash loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const float scale_log2 = a.scale_log2;
  const int64_t ld = a.ld;
  const int64_t hoff = (int64_t)s.head * kHD;
  const int ntiles = kt_end - s.kt;
  const int row0 = s.seq_begin + s.kt * kBK;
  const int last_valid = s.seq_len - (s.nk - 1) * kBK;  // valid keys in the window's last tile

  // the previous segment's readers of every stage are done past this point
  __syncthreads();
  // K padding columns 72..79 back to zero (a previous segment may have
  // masked keys there); thread 64 st + r owns row r of stage st.
  if (tid < kStages * kBK)
    *reinterpret_cast<u32x4_t*>(ks_mem + (tid / kBK) * kKBuf + (tid % kBK) * kKS + 72) = u32x4_t{0, 0, 0, 0};
  // mask the keys past the window in its last tile (global tile t in stage st)
  auto mask_last = [&](int t, int st) {
    if (t == s.nk - 1 && last_valid < kBK && tid >= kBK * st && tid < kBK * (st + 1) && tid - kBK * st >= last_valid)
      *reinterpret_cast<uint32_t*>(ks_mem + st * kKBuf + (tid - kBK * st) * kKS + 72) = kMaskedKey;
  };

  // ---- Q^T operand: lane holds query q_row, d = 16kc + 8g .. +8; d = 72 is
  // the constant 1.0 that picks up the key mask, d = 73..79 are zero
  const int q_local = s.qtile * kBQ + wave * 32 + l32;
  const int q_row = min(q_local, s.seq_len - 1);
  bf16x8_t qf[5];
  {
    const uint16_t* qp = a.q + (int64_t)(s.seq_begin + q_row) * ld + hoff;
#pragma unroll
    for (int kc = 0; kc < 5; ++kc) {
      const int d = 16 * kc + 8 * g;
      qf[kc] = d < kHD ? ld_bf16x8(qp + d) : __builtin_bit_cast(bf16x8_t, u32x4_t{0x3f80u, 0, 0, 0});
    }
  }

  // third V^T row tile: rows 64..71 real (lanes l32 < 8), row 72 = ones
  // (softmax denominator, lane 8), rows 73..95 = the zero row (a broadcast).
  const int vrow2 = l32 < 8 ? 64 + l32 : (l32 == 8 ? 72 : 73);

  f32x16_t acc[3];
#pragma unroll
  for (int dt = 0; dt < 3; ++dt) acc[dt] = f32x16_t{};
  float m_run = -INFINITY;  // running max of scaled scores (log2 units)

  // ---- prologue: the segment's tiles 0 .. kAhead-1 into stages 0 .. kAhead-1,
  // tile kAhead into registers (loads past the window are harmless: see load_kv)
  const KVPlan plan = make_plan(tid, ld, hoff);
  {
    KVRegs pre[kAhead];
#pragma unroll
    for (int t = 0; t < kAhead; ++t) load_kv(pre[t], plan, a.k, a.v, ld, row0 + t * kBK, a.total, tid);
#pragma unroll
    for (int t = 0; t < kAhead; ++t) {
      store_kv(pre[t], plan, ks_mem + t * kKBuf, vt_mem + t * kVBuf, tid);
      mask_last(s.kt + t, t);
    }
  }
  // two register sets: a tile's global load is issued two tile steps before
  // its LDS store
  KVRegs r_a, r_b;
  load_kv(r_a, plan, a.k, a.v, ld, row0 + kAhead * kBK, a.total, tid);
  load_kv(r_b, plan, a.k, a.v, ld, row0 + (kAhead + 1) * kBK, a.total, tid);
  __syncthreads();

  f32x16_t s_a[2], s_b[2];
  qk_tile(s_a, ks_mem, qf, l32, g);
  float mx = tile_max(s_a, scale_log2);  // scaled row max of the current S tile

  auto rescale = [&]() {
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < 3; ++dt) acc[dt] *= alpha;
    }
  };

  int bv = 0;  // stage holding tile j
  auto next_stage = [](int st, int n) { return st + n >= kStages ? st + n - kStages : st + n; };
  // Tile j (j < ntiles - 1).  Tile j+kAhead goes from registers r to LDS and
  // tile j+kAhead+2 is fetched into r (past the segment these are harmless
  // extra loads into a free stage).  Then the interleaved MFMA/VALU work of
  // the tile, with this wave group's barrier after its QK or its PV phase.
  auto body = [&](int j, f32x16_t (&s_cur)[2], f32x16_t (&s_nxt)[2], KVRegs& r, bool sync) {
    const int bk = next_stage(bv, 1);       // stage of tile j+1
    const int bw = next_stage(bv, kAhead);  // stage for tile j+kAhead
    rescale();
    store_kv(r, plan, ks_mem + bw * kKBuf, vt_mem + bw * kVBuf, tid);
    mask_last(s.kt + j + kAhead, bw);
    load_kv(r, plan, a.k, a.v, ld, row0 + (j + kAhead + 2) * kBK, a.total, tid);
    auto hook = [&](int slot) {
      if (kLate && sync && slot == 9) lds_barrier();
    };
    mx = tile_step(s_nxt, acc, s_cur, ks_mem + bk * kKBuf, vt_mem + bv * kVBuf, qf, scale_log2, m_run, l32, g,
                   vrow2, hook);
    if (!kLate && sync) lds_barrier();
    bv = bk;
  };
  // Last tile: P and PV only.
  auto tail = [&](f32x16_t (&s_cur)[2]) {
    rescale();
    bf16x8_t pb[2][2];
    exp_tile(pb, s_cur, scale_log2, m_run);
    pv_tile(acc, vt_mem + bv * kVBuf, pb, l32, g, vrow2);
  };

  // two tiles per trip with the S registers and the staging register sets
  // swapping roles: no copies
  int j = 0;
  for (; j + 2 < ntiles; j += 2) {
    body(j, s_a, s_b, r_a, false);
    body(j + 1, s_b, s_a, r_b, true);
  }
  if (j + 1 < ntiles) {
    body(j, s_a, s_b, r_a, false);
    tail(s_b);
  } else {
    tail(s_a);
  }

  // ---- results: lane holds query q_local, O^T rows d = 32dt + 8(rr/4) + 4g + rr%4;
  // row 72 (the row sum) sits in acc[2][4] of the g == 0 half.
  if (slot) {
    const int qi = wave * 32 + l32;
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int d = 32 * dt + 8 * (rr >> 2) + 4 * g + (rr & 3);
        if (d <= kHD) slot[d * kBQ + qi] = acc[dt][rr];
      }
    }
    if (g == 0) slot[(kHD + 1) * kBQ + qi] = m_run;
    return;
  }
  const float l_tot = __shfl(acc[2][4], l32);
  const float inv_l = 1.0f / l_tot;
  if (q_local < s.seq_len) {
    uint16_t* op = a.o + (int64_t)(s.seq_begin + q_local) * a.ldo + hoff;
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = 32 * dt + 8 * rg + 4 * g;
        if (d < kHD) {
          uint2 w;
          w.x = pack_bf16x2(acc[dt][4 * rg + 0] * inv_l, acc[dt][4 * rg + 1] * inv_l);
          w.y = pack_bf16x2(acc[dt][4 * rg + 2] * inv_l, acc[dt][4 * rg + 3] * inv_l);
          *reinterpret_cast<uint2*>(op + d) = w;
        }
      }
    }
  }
}

// Persistent stream-K grid: workgroup g (logical, XCD-grouped) takes the
// key tiles [g W / G, (g+1) W / G) of the whole work order, so every
// workgroup gets the same number of key tiles however the (window, q tile,
// head) items divide into the resident slots.  Items cut by a range
// boundary leave partials that attention_combine_kernel merges.
__global__ __launch_bounds__(kThreads, 1) void attention_kernel(AttnParams a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks_mem[kStages * kKBuf];
  __shared__ __attribute__((aligned(16))) uint16_t vt_mem[kStages * kVBuf];

  // V^T row 72 is all ones, row 73 all zeros, in every stage (never overwritten)
  for (int i = threadIdx.x; i < kStages * 2 * (kVS / 2); i += kThreads) {
    const int st = i / kVS, rem = i % kVS;  // kVS dwords cover the two rows
    const int row = 72 + rem / (kVS / 2), col = 2 * (rem % (kVS / 2));
    *reinterpret_cast<uint32_t*>(vt_mem + st * kVBuf + row * kVS + col) = row == 72 ? 0x3f803f80u : 0u;
  }

  // waves 4..7 are the "late" group: one wave of each SIMD takes the barrier
  // of a key tile between its QK/exp and its PV phase, so the two waves that
  // share a SIMD run opposite phases (one VALU-heavy, one MFMA-heavy)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool late = wave >= 4;
  const int lg = xcd_logical_block(blockIdx.x, a.num_wgs);
  for (int rg = lg; rg < a.num_ranges; rg += a.num_wgs) {
    int64_t p = range_start(a, rg);
    const int64_t end = range_start(a, rg + 1);
    Segment s = range_first(a, rg);
    while (p < end) {
      if (s.nk == 0) break;  // only if the device windows disagree with the host's copy
      const int kt_end = (int)min((int64_t)s.nk, s.kt + (end - p));
      // a segment that starts inside its item uses slot 2 rg, one that starts
      // the item but stops short of its end slot 2 rg + 1
      float* slot = (s.kt == 0 && kt_end == s.nk)
                        ? nullptr
                        : a.partial + (size_t)(2 * rg + (s.kt != 0 ? 0 : 1)) * kSlotFloats;
      if (late)
        run_segment<true>(a, s, kt_end, slot, ks_mem, vt_mem);
      else
        run_segment<false>(a, s, kt_end, slot, ks_mem, vt_mem);
      p += kt_end - s.kt;
      if (p < end) s = next_item(a, s);  // the segment ran to its item's end
    }
  }
}

// Merge the partials of every item that the stream-K ranges cut.  The
// block of the range that holds an item's last key tile does it, reading the
// item's segments in key order (deterministic):
//   m = max_s m_s,  l = sum_s 2^(m_s - m) l_s,  O = sum_s 2^(m_s - m) O_s / l.
// Thread (query, half) merges 36 of the query's 72 values; the bf16 tile is
// parked in LDS and written back as whole 144-byte head rows, 16 bytes per
// lane on consecutive lanes.
__global__ __launch_bounds__(2 * kBQ) void attention_combine_kernel(AttnParams a) {
  constexpr int kHalf = kHD / 2;
  constexpr int kRowU4 = kHD / 8;  // 16-byte chunks per query row (9)
  __shared__ uint4 tile[kBQ * kRowU4];
  const int lg = blockIdx.x;  // range
  const int64_t p = range_start(a, lg), end = range_start(a, lg + 1);
  if (p >= end) return;
  const Segment s = range_first(a, lg);
  if (s.nk == 0 || s.kt == 0 || s.kt + (end - p) < s.nk) return;  // not an item's last segment
  const int64_t p0 = p - s.kt;                        // the item's first key tile
  int g0 = (int)(p0 * a.num_ranges / a.work);
  while (g0 + 1 < a.num_ranges && range_start(a, g0 + 1) <= p0) ++g0;
  while (g0 > 0 && range_start(a, g0) > p0) --g0;

  const int tid = threadIdx.x, qi = tid & (kBQ - 1), half = tid / kBQ;
  const int rows = min(kBQ, s.seq_len - s.qtile * kBQ);  // queries of this tile inside the window
  if (qi < rows) {
    auto slot_of = [&](int gg) -> const float* {
      return a.partial + (size_t)(gg == g0 ? 2 * gg + 1 : 2 * gg) * kSlotFloats;
    };
    float m = -INFINITY;
    float o[kHalf];
    float l = 0.0f;
    if (lg == g0 + 1) {
      // two segments, the usual cut: every value loaded before the first
      // wait (a loop with a run-time trip count waits once per iteration);
      // the same operations in the same order as the loop below
      const float* s0 = slot_of(g0);
      const float* s1 = slot_of(lg);
      float o0[kHalf], o1[kHalf];
      const float m0 = s0[(kHD + 1) * kBQ + qi], m1 = s1[(kHD + 1) * kBQ + qi];
      const float l0 = s0[kHD * kBQ + qi], l1 = s1[kHD * kBQ + qi];
#pragma unroll
      for (int i = 0; i < kHalf; ++i) {
        o0[i] = s0[(half * kHalf + i) * kBQ + qi];
        o1[i] = s1[(half * kHalf + i) * kBQ + qi];
      }
      m = fmaxf(fmaxf(m, m0), m1);
      const float w0 = __builtin_amdgcn_exp2f(m0 - m), w1 = __builtin_amdgcn_exp2f(m1 - m);
      l = fmaf(w1, l1, fmaf(w0, l0, 0.0f));
#pragma unroll
      for (int i = 0; i < kHalf; ++i) o[i] = fmaf(w1, o1[i], fmaf(w0, o0[i], 0.0f));
    } else if (lg - g0 < 4) {
      // three or four segments (short ranges, small windows): the same,
      // with the values of a fourth segment loaded from the last one again
      // and not used
      constexpr int kS = 4;
      const int ns = lg - g0 + 1;
      float mv[kS], lv[kS], ov[kS][kHalf];
#pragma unroll
      for (int j = 0; j < kS; ++j) {
        const float* sl = slot_of(min(g0 + j, lg));
        mv[j] = sl[(kHD + 1) * kBQ + qi];
        lv[j] = sl[kHD * kBQ + qi];
#pragma unroll
        for (int i = 0; i < kHalf; ++i) ov[j][i] = sl[(half * kHalf + i) * kBQ + qi];
      }
#pragma unroll
      for (int j = 0; j < kS; ++j) m = j < ns ? fmaxf(m, mv[j]) : m;
#pragma unroll
      for (int i = 0; i < kHalf; ++i) o[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < kS; ++j) {
        const float w = __builtin_amdgcn_exp2f(mv[j] - m);
        l = j < ns ? fmaf(w, lv[j], l) : l;
#pragma unroll
        for (int i = 0; i < kHalf; ++i) o[i] = j < ns ? fmaf(w, ov[j][i], o[i]) : o[i];
      }
    } else {
      for (int gg = g0; gg <= lg; ++gg) m = fmaxf(m, slot_of(gg)[(kHD + 1) * kBQ + qi]);
#pragma unroll
      for (int i = 0; i < kHalf; ++i) o[i] = 0.0f;
      for (int gg = g0; gg <= lg; ++gg) {
        const float* sl = slot_of(gg);
        const float w = __builtin_amdgcn_exp2f(sl[(kHD + 1) * kBQ + qi] - m);
        l = fmaf(w, sl[kHD * kBQ + qi], l);
#pragma unroll
        for (int i = 0; i < kHalf; ++i) o[i] = fmaf(w, sl[(half * kHalf + i) * kBQ + qi], o[i]);
      }
    }
    const float inv_l = 1.0f / l;
    uint2* trow = reinterpret_cast<uint2*>(tile + qi * kRowU4) + half * (kHalf / 4);
#pragma unroll
    for (int i = 0; i < kHalf; i += 4) {
      uint2 w;
      w.x = pack_bf16x2(o[i] * inv_l, o[i + 1] * inv_l);
      w.y = pack_bf16x2(o[i + 2] * inv_l, o[i + 3] * inv_l);
      trow[i / 4] = w;
    }
  }
  __syncthreads();
  uint16_t* obase = a.o + (int64_t)(s.seq_begin + s.qtile * kBQ) * a.ldo + (int64_t)s.head * kHD;
  for (int c = tid; c < rows * kRowU4; c += 2 * kBQ) {
    const int q = c / kRowU4, ch = c - q * kRowU4;
    *reinterpret_cast<uint4*>(obase + (int64_t)q * a.ldo + ch * 8) = tile[c];
  }
}

size_t attention_partial_bytes() { return (size_t)2 * kMaxRanges * kSlotFloats * sizeof(float); }

// ---------------------------------------------------------------- no-allocation variant
// The partials of vit_attention_noalloc live in this file-scope array, one
// copy per device (38.8 MB: two slots of [74][256] fp32 for each of the at
// most 256 stream-K ranges; the need does not grow with the input).  Host
// code never uses its name as an address: the device address of each copy
// is taken once per device with hipGetSymbolAddress and kept below.
static __device__ __align__(256) float scratch[2 * kMaxRanges * kSlotFloats];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
float* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

size_t attention_scratch_bytes() { return sizeof(scratch); }

hipError_t attention_scratch(hipStream_t stream, float** ptr) {
  static_assert(sizeof(scratch) >= (size_t)2 * kMaxRanges * kSlotFloats * sizeof(float), "scratch too small");
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    // with that device current; the caller's current device is restored
    int cur = -1;
    hipError_t r = hipGetDevice(&cur);
    if (r == hipSuccess && cur != dev) r = hipSetDevice(dev);
    void* p = nullptr;
    if (r == hipSuccess) r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t r2 = hipSetDevice(cur);
      if (r == hipSuccess) r = r2;
    }
    g_scratch_err[dev] = r;
    g_scratch_ptr[dev] = r == hipSuccess ? static_cast<float*>(p) : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// Compute units of the current device (256 if the query fails), cached per
// device.
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Resident slots of the current device: one 512-thread workgroup per CU,
// at most kMaxWorkgroups.
static int attention_slots() { return std::min(device_cu_count(), kMaxWorkgroups); }

// Host plan of the stream-K split.  The work order of one head lists, per
// window, its q tiles x key tiles; the whole order is heads x that list,
// cut into one equal range per workgroup.  For each range the window and
// the position inside that window's list where it starts are found in one
// sweep over the windows (the ranges visited in order of their in-head
// position), so the kernels locate every segment in constant time.
void plan_attention(const int32_t* cu_host, int num_seqs, int heads, AttnPlan* plan) {
  int64_t wph = 0;
  for (int w = 0; w < num_seqs; ++w) {
    const int64_t len = cu_host[w + 1] - cu_host[w];
    wph += ((len + kBQ - 1) / kBQ) * ((len + kBK - 1) / kBK);
  }
  plan->work_per_head = wph;
  plan->num_ranges = 0;
  if (wph == 0) return;
  const int64_t work = wph * heads;
  const int R = (int)std::min<int64_t>(attention_slots(), work);
  plan->num_ranges = R;
  int64_t rel[kAttnMaxRanges];
  int order[kAttnMaxRanges];
  for (int r = 0; r < R; ++r) {
    const int64_t p = (int64_t)r * work / R;
    rel[r] = p - (p / wph) * wph;
    order[r] = r;
  }
  std::sort(order, order + R, [&](int x, int y) { return rel[x] < rel[y]; });
  int64_t acc = 0;
  int i = 0;
  for (int w = 0; w < num_seqs && i < R; ++w) {
    const int64_t len = cu_host[w + 1] - cu_host[w];
    const int64_t span = ((len + kBQ - 1) / kBQ) * ((len + kBK - 1) / kBK);
    while (i < R && rel[order[i]] < acc + span) {
      plan->start[order[i]].win = w;
      plan->start[order[i]].rem = (int32_t)(rel[order[i]] - acc);
      ++i;
    }
    acc += span;
  }
}

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_qkv, uint16_t* o,
                            int64_t ld_o, const int32_t* cu, int num_seqs, int total_tokens, const AttnPlan& plan,
                            int heads, float scale, float* partial, hipStream_t stream) {
  if (plan.work_per_head == 0) return hipSuccess;
  AttnParams a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.cu = cu;
  a.partial = partial;
  a.ld = ld_qkv;
  a.ldo = ld_o;
  a.work_per_head = plan.work_per_head;
  a.work = plan.work_per_head * heads;
  a.num_seqs = num_seqs;
  a.heads = heads;
  a.total = total_tokens;
  a.num_wgs = plan.num_ranges;
  a.num_ranges = plan.num_ranges;
  a.scale_log2 = scale * 1.4426950408889634f;
  std::copy(plan.start, plan.start + plan.num_ranges, a.start);
  attention_kernel<<<a.num_wgs, kThreads, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attention_combine_kernel<<<a.num_ranges, 2 * kBQ, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace vit
