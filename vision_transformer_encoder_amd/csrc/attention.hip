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
//    row max / row sum of the softmax and the rescale of O stay in the
//    lane's registers, plus one cross-half exchange (lane ^ 32) per tile.
//  * P never leaves registers: the 16 key-rows a lane holds in S^T are, in
//    order, the 8+8 k-slots of the B operand of two PV MFMAs (the key order
//    inside an MFMA is a free permutation as long as V^T uses the same one).
//  * head_dim 72 is padded to 80 for Q K^T (5 MFMAs of K=16) and to 96 rows
//    for V^T (3 row tiles of 32); the pad lanes read zeros kept in LDS.
//  * K tiles (64 keys x 80) and V^T tiles (96 x 64) are double-buffered in
//    LDS; the next tile's global loads are issued before the current
//    tile's MFMAs.  Row strides (88 and 68 bf16) make the ds_read_b128 /
//    ds_read_b64 operand fetches bank-conflict free.
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
constexpr int kVRows = 96;        // V^T rows (head_dim padded to 3 x 32)
constexpr int kKBuf = kBK * kKS;  // elements per K buffer
constexpr int kVBuf = kVRows * kVS;
}  // namespace

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// Loads of one K/V tile into registers.  K: 64 rows x 9 chunks of 16 B = 576
// chunks, up to 3 per thread.  V: 16 groups of 4 keys x 9 chunks of 8 d =
// 144 items (threads 0..143), 4 x 16 B each.  Keys past the window end are
// clamped to its last key (finite data; their scores are masked).
struct KVRegs {
  uint4 k[3];
  uint4 v[4];
};

__device__ __forceinline__ void load_kv(KVRegs& r, const uint16_t* __restrict__ kbase,
                                        const uint16_t* __restrict__ vbase, int64_t ld, int key0,
                                        int nkeys, int tid) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int c = tid + 256 * i;
    if (c < 576) {
      const int row = c / 9, col = c % 9;
      const int key = min(key0 + row, nkeys - 1);
      r.k[i] = *reinterpret_cast<const uint4*>(kbase + (int64_t)key * ld + col * 8);
    }
  }
  if (tid < 144) {
    const int c = tid % 9, kg = tid / 9;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(key0 + 4 * kg + i, nkeys - 1);
      r.v[i] = *reinterpret_cast<const uint4*>(vbase + (int64_t)key * ld + c * 8);
    }
  }
}

__device__ __forceinline__ void store_kv(const KVRegs& r, uint16_t* __restrict__ ks,
                                         uint16_t* __restrict__ vt, int tid) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int c = tid + 256 * i;
    if (c < 576) {
      const int row = c / 9, col = c % 9;
      *reinterpret_cast<uint4*>(ks + row * kKS + col * 8) = r.k[i];
    }
  }
  if (tid < 144) {
    const int c = tid % 9, kg = tid / 9;
    // r.v[i] holds d = 8c..8c+7 of key 4kg+i; write V^T[8c+j][4kg .. 4kg+3].
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r.v[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r.v[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r.v[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r.v[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // d = 8c + 2j (low halves) and 8c + 2j + 1 (high halves)
      uint2 lo, hi;
      lo.x = (w0[j] & 0xffffu) | (w1[j] << 16);
      lo.y = (w2[j] & 0xffffu) | (w3[j] << 16);
      hi.x = (w0[j] >> 16) | (w1[j] & 0xffff0000u);
      hi.y = (w2[j] >> 16) | (w3[j] & 0xffff0000u);
      *reinterpret_cast<uint2*>(vt + (8 * c + 2 * j) * kVS + 4 * kg) = lo;
      *reinterpret_cast<uint2*>(vt + (8 * c + 2 * j + 1) * kVS + 4 * kg) = hi;
    }
  }
}

__global__ __launch_bounds__(256) void attention_kernel(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, int64_t ld,
                                                        uint16_t* __restrict__ o, int64_t ldo,
                                                        const int32_t* __restrict__ cu, int num_seqs,
                                                        int heads, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint16_t ks_mem[2 * kKBuf];
  __shared__ __attribute__((aligned(16))) uint16_t vt_mem[2 * kVBuf];

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
  const uint16_t* kbase = k + (int64_t)seq_begin * ld + hoff;
  const uint16_t* vbase = v + (int64_t)seq_begin * ld + hoff;

  // ---- zero the padding of both LDS buffers (K cols 72..79, V^T rows 72..95)
  for (int i = tid; i < 2 * kBK; i += 256) {
    *reinterpret_cast<uint4*>(ks_mem + (i / kBK) * kKBuf + (i % kBK) * kKS + 72) = make_uint4(0, 0, 0, 0);
  }
  for (int i = tid; i < 2 * 24 * (kVS / 4); i += 256) {
    const int b = i / (24 * (kVS / 4)), rem = i % (24 * (kVS / 4));
    *reinterpret_cast<uint2*>(vt_mem + b * kVBuf + (72 + rem / (kVS / 4)) * kVS + 4 * (rem % (kVS / 4))) =
        make_uint2(0, 0);
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
      if (d < kHD) {
        qf[kc] = ld_bf16x8(qp + d);
      } else {
        qf[kc] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
      }
    }
  }

  f32x16_t acc[3];
#pragma unroll
  for (int dt = 0; dt < 3; ++dt) acc[dt] = f32x16_t{};
  float m_run = -INFINITY;  // running max of scaled scores (log2 units)
  float l_run = 0.0f;       // lane-partial running sum

  const int ntiles = (seq_len + kBK - 1) / kBK;
  KVRegs r;
  load_kv(r, kbase, vbase, ld, 0, seq_len, tid);
  store_kv(r, ks_mem, vt_mem, tid);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const uint16_t* ks = ks_mem + buf * kKBuf;
    const uint16_t* vt = vt_mem + buf * kVBuf;
    if (it + 1 < ntiles) load_kv(r, kbase, vbase, ld, (it + 1) * kBK, seq_len, tid);

    // ---- S^T = K Q^T for 2 x 32 keys
    f32x16_t s[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      s[jt] = f32x16_t{};
      const uint16_t* kr = ks + (32 * jt + l32) * kKS + 8 * g;
#pragma unroll
      for (int kc = 0; kc < 5; ++kc) {
        s[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(kr + 16 * kc), qf[kc], s[jt], 0, 0, 0);
      }
    }
    // ---- mask keys past the window end (last tile only)
    const int key0 = it * kBK;
    if (key0 + kBK > seq_len) {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = key0 + 32 * jt + 8 * (rr >> 2) + 4 * g + (rr & 3);
          if (key >= seq_len) s[jt][rr] = -INFINITY;
        }
      }
    }
    // ---- online softmax, one query per lane
    float mx = s[0][0];
#pragma unroll
    for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, s[0][rr]);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[1][rr]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.0f;
    bf16x8_t pb[2][2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = __builtin_amdgcn_exp2f(fmaf(s[jt][8 * h + j], scale_log2, -m_new));
          psum += p[j];
        }
        uint4 w;
        w.x = pack_bf16x2(p[0], p[1]);
        w.y = pack_bf16x2(p[2], p[3]);
        w.z = pack_bf16x2(p[4], p[5]);
        w.w = pack_bf16x2(p[6], p[7]);
        pb[jt][h] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) acc[dt] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
      const uint16_t* vr = vt + (32 * dt + l32) * kVS + 4 * g;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kb = 32 * jt + 16 * h;
          uint4 w;
          const uint2 a0 = *reinterpret_cast<const uint2*>(vr + kb);
          const uint2 a1 = *reinterpret_cast<const uint2*>(vr + kb + 8);
          w.x = a0.x; w.y = a0.y; w.z = a1.x; w.w = a1.y;
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pb[jt][h],
                                                           acc[dt], 0, 0, 0);
        }
      }
    }

    if (it + 1 < ntiles) store_kv(r, ks_mem + (buf ^ 1) * kKBuf, vt_mem + (buf ^ 1) * kVBuf, tid);
    __syncthreads();
  }

  // ---- normalise and store: lane holds query q_local, d = 32dt + 8(rr/4) + 4g + rr%4
  const float l_tot = l_run + __shfl_xor(l_run, 32);
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
                            int num_seqs, int total_q_tiles, int heads, float scale,
                            hipStream_t stream) {
  if (total_q_tiles == 0) return hipSuccess;
  const float scale_log2 = scale * 1.4426950408889634f;
  attention_kernel<<<total_q_tiles * heads, 256, 0, stream>>>(q, k, v, ld_qkv, o, ld_o, cu, num_seqs,
                                                             heads, scale_log2);
  return hipGetLastError();
}

}  // namespace vit
