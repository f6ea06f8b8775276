// Full bidirectional attention over cu_seqlens windows, head_dim 72, bf16
// MFMA with an fp32 online softmax (FlashRT "Qwen3-VL-8B on RTX 5090" page,
// section 3: "FA2 (full, bidirectional)"; section 5: every image is its own
// cu_seqlens attention window; section 1: this attention is the largest cost
// of the tower and is compute-bound).
//
// gfx950 design (not the page's sm_120 kernel):
//  * One 256-thread workgroup = 4 waves = 128 queries of one (window, head);
//    each wave owns 32 queries for the whole key loop.
//  * Everything is computed transposed, S^T = K Q^T and O^T = V^T P^T, with
//    v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane holds
//    one column (lane % 32) and 16 rows, so every lane owns ONE query: the
//    row max and the rescale of O stay in the lane's registers, plus one
//    cross-half exchange (lane ^ 32) per tile.
//  * P never leaves registers: the 16 key-rows a lane holds in S^T are, in
//    order, the 8+8 k-slots of the B operand of two PV MFMAs (the key order
//    inside an MFMA is a free permutation as long as V^T uses the same one).
//  * head_dim 72 is padded to 80 for Q K^T (5 MFMAs of K=16) and to 96 rows
//    for V^T (3 row tiles of 32).  Of the third V^T tile, row 72 is all ones:
//    its output row is the softmax denominator (sum of the bf16 P actually
//    multiplied), accumulated and rescaled by the MFMA for free; rows 73..95
//    are zero.  These rows come from registers, not LDS.
//  * Software pipeline across key tiles: while the VALU turns S(j) into P(j)
//    (exp2 with the scale folded in), the MFMA unit already computes S(j+1);
//    then the PV MFMAs of tile j run.  K and V^T tiles live in a 3-buffer LDS
//    ring (tile j: V^T read, tile j+1: K read, tile j+2: being written), one
//    barrier per tile; global loads of tile j+2 are in flight during tile j.
//  * The running max is only raised (and O rescaled) when a row max grows
//    by more than 2^8 over it: exact after the final division by the row
//    sum, and it removes the per-tile rescale of 48 accumulators.
//  * Row strides in LDS (88 bf16 for K, 68 for V^T) keep the ds_read_b128 /
//    ds_read_b64 operand fetches bank-conflict free.
//  * K/V tiles are fetched with buffer loads whose descriptor starts at the
//    tile's first row and ends at the last token: per-thread offsets are
//    fixed for the whole loop (no per-tile address arithmetic), and rows
//    past the last token read as zero in hardware, so no clamping is needed
//    (rows of the next window inside the batch are finite and masked).
//  * Workgroup id -> (q tile, head) with head fastest: ids that share a head
//    are congruent mod 8, so each XCD (ids round-robin over 8 XCDs) serves
//    two heads and keeps their K/V in its own L2.
#include "common.h"
#include "kernels.h"

namespace vit {

namespace {
constexpr int kHD = 72;
constexpr int kBQ = 128;          // queries per workgroup
constexpr int kBK = 64;           // keys per tile
constexpr int kKS = 88;           // K row stride in LDS (bf16): 80 used
constexpr int kVS = 68;           // V^T row stride in LDS (bf16): 64 used
constexpr int kKBuf = kBK * kKS;  // elements per K buffer
constexpr int kVRows = kHD + 2;  // V^T rows 0..71, row 72 = ones, row 73 = zeros
constexpr int kVBuf = kVRows * kVS;
constexpr int kStages = 3;
constexpr float kLazy = 8.0f;     // rescale only when the max grows by > 2^8
}  // namespace

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// Staging of one K/V tile.  K: 64 rows x 9 chunks of 16 B = 576 chunks,
// thread t owns chunks t, t+256 and (t < 64) t+512.  V: 16 groups of 4 keys
// x 9 chunks of 8 d = 144 items (threads 0..143), 4 x 16 B each, transposed
// into V^T on the way to LDS.  All offsets are fixed per thread.
// V item mapping: lane group tid/16 picks the d chunk, tid%16 the key group,
// with chunks ordered 0,2,1,3,4,6,5,7,8 so that the two 16-lane halves of
// every 32-lane LDS write phase hit V^T rows 16 apart: with the 34-dword row
// stride those are 32 banks apart, and each phase writes 64 distinct banks.
struct KVRegs {
  u32x4_t k0, k1, k2;
  u32x4_t v[4];
};

struct KVPlan {
  uint32_t kgoff[3];  // byte offsets of the three K chunks within a tile
  int klds[3];        // their LDS element offsets
  uint32_t vgoff;     // byte offset of key 4*vkg, chunk vc within a tile
  uint32_t vstride;   // bytes per row
  int vlds;           // V^T LDS offset of row 8*vc, column 4*vkg
};

__device__ __forceinline__ KVPlan make_plan(int tid, int64_t ld, int64_t hoff) {
  KVPlan p;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    // 16 consecutive chunks = 16 consecutive rows of one column: the 16 lanes
    // of each ds_write_b128 phase hit distinct banks (44-dword row stride)
    const int c = min(tid + 256 * i, 575);
    const int blk = c >> 4;
    const int row = (blk / 9) * 16 + (c & 15), col = blk % 9;
    p.kgoff[i] = (uint32_t)((row * ld + hoff + col * 8) * 2);
    p.klds[i] = row * kKS + col * 8;
  }
  const int vgrp = min(tid >> 4, 8);
  const int vc = (vgrp == 1 || vgrp == 5) ? vgrp + 1 : ((vgrp == 2 || vgrp == 6) ? vgrp - 1 : vgrp);
  const int vkg = tid & 15;
  p.vgoff = (uint32_t)((4 * vkg * ld + hoff + vc * 8) * 2);
  p.vstride = (uint32_t)(ld * 2);
  p.vlds = 8 * vc * kVS + 4 * vkg;
  return p;
}

// Buffer descriptor over rows [row0, total) of a [total, ld] bf16 array.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int64_t ld, int row0, int total) {
  const uint16_t* p = base + (int64_t)row0 * ld;
  const int64_t bytes = (int64_t)(total - row0) * ld * 2;
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
  r.k0 = buf_ld(kr, p.kgoff[0]);
  r.k1 = buf_ld(kr, p.kgoff[1]);
  if (tid < 64) r.k2 = buf_ld(kr, p.kgoff[2]);
  if (tid < 144) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = buf_ld(vr, p.vgoff + i * p.vstride);
  }
}

__device__ __forceinline__ void store_kv(const KVRegs& r, const KVPlan& p, uint16_t* __restrict__ ks,
                                         uint16_t* __restrict__ vt, int tid) {
  *reinterpret_cast<u32x4_t*>(ks + p.klds[0]) = r.k0;
  *reinterpret_cast<u32x4_t*>(ks + p.klds[1]) = r.k1;
  if (tid < 64) *reinterpret_cast<u32x4_t*>(ks + p.klds[2]) = r.k2;
  if (tid < 144) {
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

__device__ __forceinline__ void mask_tile(f32x16_t s[2], int key0, int nkeys, int g) {
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = key0 + 32 * jt + 8 * (rr >> 2) + 4 * g + (rr & 3);
      if (key >= nkeys) s[jt][rr] = -INFINITY;
    }
  }
}

__global__ __launch_bounds__(256, 2) void attention_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, int64_t ld,
                                                           uint16_t* __restrict__ o, int64_t ldo,
                                                           const int32_t* __restrict__ cu, int num_seqs,
                                                           int heads, float scale_log2, int total) {
  __shared__ __attribute__((aligned(16))) uint16_t ks_mem[kStages * kKBuf];
  __shared__ __attribute__((aligned(16))) uint16_t vt_mem[kStages * kVBuf];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  // ---- which (window, q tile, head)
  const int head = blockIdx.x % heads;
  int tile = blockIdx.x / heads;
  int seq_begin = 0, seq_len = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int b = cu[s], e = cu[s + 1];
    const int nt = (e - b + kBQ - 1) / kBQ;
    if (tile < nt) {
      seq_begin = b;
      seq_len = e - b;
      break;
    }
    tile -= nt;
  }
  if (seq_len == 0) return;  // cannot happen for a correctly sized grid

  const int64_t hoff = (int64_t)head * kHD;

  // ---- constant parts of every stage (never overwritten): K padding columns
  // 72..79 are zero; V^T row 72 is all ones, row 73 all zeros.
  for (int i = tid; i < kStages * kBK; i += 256)
    *reinterpret_cast<uint4*>(ks_mem + (i / kBK) * kKBuf + (i % kBK) * kKS + 72) = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < kStages * 2 * (kVS / 2); i += 256) {
    const int st = i / kVS, rem = i % kVS;  // kVS dwords cover the two rows
    const int row = 72 + rem / (kVS / 2), col = 2 * (rem % (kVS / 2));
    *reinterpret_cast<uint32_t*>(vt_mem + st * kVBuf + row * kVS + col) = row == 72 ? 0x3f803f80u : 0u;
  }

  // ---- Q^T operand: lane holds query q_row, d = 16kc + 8g .. +8 (zero past 72)
  const int q_local = tile * kBQ + wave * 32 + l32;
  const int q_row = min(q_local, seq_len - 1);
  bf16x8_t qf[5];
  {
    const uint16_t* qp = q + (int64_t)(seq_begin + q_row) * ld + hoff;
#pragma unroll
    for (int kc = 0; kc < 5; ++kc) {
      const int d = 16 * kc + 8 * g;
      qf[kc] = d < kHD ? ld_bf16x8(qp + d) : __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
    }
  }

  // third V^T row tile: rows 64..71 real (lanes l32 < 8), row 72 = ones
  // (softmax denominator, lane 8), rows 73..95 = the zero row (a broadcast).
  const int vrow2 = l32 < 8 ? 64 + l32 : (l32 == 8 ? 72 : 73);

  f32x16_t acc[3];
#pragma unroll
  for (int dt = 0; dt < 3; ++dt) acc[dt] = f32x16_t{};
  float m_run = -INFINITY;  // running max of scaled scores (log2 units)

  const int ntiles = (seq_len + kBK - 1) / kBK;
  const KVPlan plan = make_plan(tid, ld, hoff);
  KVRegs r;
  load_kv(r, plan, k, v, ld, seq_begin, total, tid);
  store_kv(r, plan, ks_mem, vt_mem, tid);
  if (ntiles > 1) {
    load_kv(r, plan, k, v, ld, seq_begin + kBK, total, tid);
    store_kv(r, plan, ks_mem + kKBuf, vt_mem + kVBuf, tid);
  }
  __syncthreads();

  f32x16_t s_a[2], s_b[2];
  qk_tile(s_a, ks_mem, qf, l32, g);
  if (seq_len < kBK) mask_tile(s_a, 0, seq_len, g);

  int bv = 0;  // stage holding tile it
  // One key tile: softmax of s_cur (tile it) on the VALU while the MFMA unit
  // computes s_nxt (tile it+1), then O += P V of tile it.
  auto step = [&](int it, f32x16_t (&s_cur)[2], f32x16_t (&s_nxt)[2]) {
    const int bk = bv == kStages - 1 ? 0 : bv + 1;  // stage of tile it+1
    const int bw = bk == kStages - 1 ? 0 : bk + 1;  // stage for tile it+2
    const bool more2 = it + 2 < ntiles;
    if (more2) load_kv(r, plan, k, v, ld, seq_begin + (it + 2) * kBK, total, tid);

    // ---- S(it+1) is queued on the MFMA unit first: it depends on nothing
    // below and runs while the VALU does the softmax of S(it)
    qk_tile(s_nxt, ks_mem + bk * kKBuf, qf, l32, g);

    // ---- row max of S(it); lazy rescale of O
    float mx = fmaxf(s_cur[0][0], s_cur[0][1]);
#pragma unroll
    for (int rr = 2; rr < 16; ++rr) mx = fmaxf(mx, s_cur[0][rr]);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s_cur[1][rr]);
    mx = halves_max(mx) * scale_log2;
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < 3; ++dt) acc[dt] *= alpha;
    }

    // ---- P(it) = exp2(S * scale - m)
    bf16x8_t pb[2][2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(s_cur[jt][8 * h + j], scale_log2, -m_run));
        uint4 w;
        w.x = pack_bf16x2(p[0], p[1]);
        w.y = pack_bf16x2(p[2], p[3]);
        w.z = pack_bf16x2(p[4], p[5]);
        w.w = pack_bf16x2(p[6], p[7]);
        pb[jt][h] = __builtin_bit_cast(bf16x8_t, w);
      }
    }

    // ---- O^T += V^T P^T (tile it)
    const uint16_t* vt = vt_mem + bv * kVBuf;
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
      const uint16_t* vr = vt + (dt < 2 ? 32 * dt + l32 : vrow2) * kVS + 4 * g;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kb = 32 * jt + 16 * h;
          const uint2 a0 = *reinterpret_cast<const uint2*>(vr + kb);
          const uint2 a1 = *reinterpret_cast<const uint2*>(vr + kb + 8);
          const uint4 w = make_uint4(a0.x, a0.y, a1.x, a1.y);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pb[jt][h], acc[dt],
                                                           0, 0, 0);
        }
      }
    }

    if ((it + 2) * kBK > seq_len && it + 1 < ntiles) mask_tile(s_nxt, (it + 1) * kBK, seq_len, g);
    if (more2) store_kv(r, plan, ks_mem + bw * kKBuf, vt_mem + bw * kVBuf, tid);
    __syncthreads();
    bv = bk;
  };

  // two tiles per trip with the S registers swapping roles: no copies
  for (int it = 0; it < ntiles; it += 2) {
    step(it, s_a, s_b);
    if (it + 1 < ntiles) step(it + 1, s_b, s_a);
  }

  // ---- normalise and store: lane holds query q_local, d = 32dt + 8(rr/4) + 4g + rr%4;
  // the row sum sits in acc[2][4] of the g == 0 half (row 72 of O^T).
  const float l_lo = acc[2][4];
  const float l_tot = __shfl(l_lo, l32);
  const float inv_l = 1.0f / l_tot;
  if (q_local < seq_len) {
    uint16_t* op = o + (int64_t)(seq_begin + q_local) * ldo + hoff;
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

int attention_q_tiles(const int32_t* cu_host, int num_seqs) {
  int n = 0;
  for (int s = 0; s < num_seqs; ++s) n += (cu_host[s + 1] - cu_host[s] + kBQ - 1) / kBQ;
  return n;
}

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            int64_t ld_qkv, uint16_t* o, int64_t ld_o, const int32_t* cu,
                            int num_seqs, int total_tokens, int total_q_tiles, int heads, float scale,
                            hipStream_t stream) {
  if (total_q_tiles == 0) return hipSuccess;
  const float scale_log2 = scale * 1.4426950408889634f;
  attention_kernel<<<total_q_tiles * heads, 256, 0, stream>>>(q, k, v, ld_qkv, o, ld_o, cu, num_seqs,
                                                             heads, scale_log2, total_tokens);
  return hipGetLastError();
}

}  // namespace vit
