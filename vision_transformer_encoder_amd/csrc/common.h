// Device helpers shared by the gfx950 kernels of libvit: vector types, bf16
// and OCP E4M3FN conversion, wave reductions, block-128 scale computation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vit {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
// Plain vector (not HIP's uint4 struct) so register arrays of it stay in
// registers instead of being demoted to scratch.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;
// Block maxima below 2^-116 give a zero scale; from 2^-116 up, amax / 448
// (>= 2^-124.8) and 448 / amax (<= 2^124.8) are normal, finite fp32 values.
constexpr float kTinyAmax = 0x1p-116f;

__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two bf16 packed in one dword: low half = element 0.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f2bf(float a) { return (uint16_t)(pack_bf16x2(a, 0.0f) & 0xffffu); }

// fp32 -> OCP E4M3FN, nearest-even (v_cvt_pk_fp8_f32 on gfx950).  The
// conversion itself gives 448 up to 464 (where the next E4M3 step would lie)
// and the NaN code above it, so e4m3x4 is exact saturation only for inputs of
// magnitude at most 464.  The block quantisers feed it x * (448 / amax) with
// |x| <= amax, at most 448 (1 + 2^-23) after the two roundings.  Arbitrary
// values go through e4m3x4_sat, which clamps to +-448 first.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}
__device__ __forceinline__ float e4m3_clamp(float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); }
__device__ __forceinline__ uint32_t e4m3x4_sat(float a, float b, float c, float d) {
  return e4m3x4(e4m3_clamp(a), e4m3_clamp(b), e4m3_clamp(c), e4m3_clamp(d));
}

// Block-128 scale: s = amax / 448 and inv = 448 / amax, both correctly
// rounded fp32 divisions; zero for a (near-)zero block.  For amax in
// [2^-116, 2^126) each quotient is the product with a reciprocal (1/448
// rounded, or v_rcp_f32 of amax) followed by one correction step with the
// exact FMA residual, which on gfx950 gives the correctly rounded quotient
// for every fp32 mantissa at every exponent of that range (compared bit for
// bit with the IEEE division over all 2^23 mantissas of each exponent); at
// 2^126 and above v_rcp_f32 is subnormal, so those blocks (and NaN) take the
// IEEE division itself.
__device__ __forceinline__ void block_scale(float amax, float& s, float& inv) {
  if (amax < kTinyAmax) {
    s = 0.0f;
    inv = 0.0f;
  } else if (amax < 0x1p126f) {
    constexpr float c = 1.0f / kE4M3Max;
    const float q = amax * c;
    s = fmaf(fmaf(-q, kE4M3Max, amax), c, q);
    const float y = __builtin_amdgcn_rcpf(amax);
    const float p = kE4M3Max * y;
    inv = fmaf(fmaf(-p, amax, kE4M3Max), y, p);
  } else {
    s = amax / kE4M3Max;
    inv = kE4M3Max / amax;
  }
}

// Cross-lane reductions without LDS round trips.  A row of 16 lanes is
// reduced with DPP (quad swaps xor 1 and xor 2, then the half-row and row
// mirrors); rows are then combined with the 16- and 32-lane swaps, whose
// result pair holds the lane's own value and its partner's.  Every step adds
// the same two values in every lane that receives them (a + b = b + a), so
// the result is bit-identical across the lanes it covers.
template <int CTRL>
__device__ __forceinline__ float dpp_peer(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

// max over each row of 16 lanes, in every lane of the row
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_peer<kDppXor1>(v));
  v = fmaxf(v, dpp_peer<kDppXor2>(v));
  v = fmaxf(v, dpp_peer<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_peer<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float group16_max(float v) { return row16_max(v); }

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_peer<kDppXor1>(v);
  v += dpp_peer<kDppXor2>(v);
  v += dpp_peer<kDppHalfMirror>(v);
  v += dpp_peer<kDppMirror>(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = __int_as_float(r16[0]) + __int_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r32[0]) + __int_as_float(r32[1]);
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = fmaxf(__int_as_float(r16[0]), __int_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(r32[0]), __int_as_float(r32[1]));
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8).  Logical index
// of workgroup `bid` such that XCD x owns the contiguous logical range
// [x*q + min(x, r), ...), nblocks = 8q + r: neighbouring logical tiles share
// an XCD and its L2.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int x = bid & 7, i = bid >> 3;
  return x * q + min(x, r) + i;
}

// Output tile (m_tile, n_tile) of logical tile index lb when the n tiles are
// walked in groups of group_n: every m tile of one group, then the next
// group.  With XCD-contiguous logical indices, the workgroups resident on
// one XCD at a time then share one group's weight slice in its L2 instead
// of streaming the whole weight.  group_n >= n_tiles is plain m-major order.
__device__ __forceinline__ void grouped_tile(int lb, int m_tiles, int n_tiles, int group_n, int& m_tile,
                                             int& n_tile) {
  const int g = lb / (m_tiles * group_n);
  const int n0 = g * group_n;
  const int gn = min(group_n, n_tiles - n0);
  const int rem = lb - g * m_tiles * group_n;
  m_tile = rem / gn;
  n_tile = n0 + rem % gn;
}

// tanh-form GELU in fp32, evaluated through the identity
// 0.5 x (1 + tanh(u)) = x / (1 + e^(-2u)),  u = sqrt(2/pi) (x + 0.044715 x^3):
// one exp2 and one reciprocal instead of a tanh, and no cancellation in
// 1 + tanh(u) for negative x (where that form loses most of its relative
// precision).  The exponent -2 log2(e) u is x (c0 + c1 x^2) with
// c0 = -2 log2(e) sqrt(2/pi) and c1 = 0.044715 c0: one FMA and one multiply.
// e^(-2u) overflows to +inf for very negative x, giving -0.
__device__ __forceinline__ float gelu_tanh(float x) {
  constexpr float c0 = -2.302208198144325f;
  constexpr float c1 = -0.1029432395800235f;
  const float e = __builtin_amdgcn_exp2f(x * fmaf(c1, x * x, c0));
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// Image of packed position t: the last j in [0, n) with cu[j] <= t (cu[0..n]
// non-decreasing token offsets; empty images are skipped).  Binary search.
__device__ __forceinline__ int image_of(const int32_t* __restrict__ cu, int n, int t) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// 8 bf16 (one 16-byte load) as fp32.
__device__ __forceinline__ void unpack8_bf16(uint4 w, float v[8]) {
  v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
  v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
}

// Load 8 bf16 starting at column c of a row as fp32; columns >= cols read 0.
// The full-vector path needs the row 16-byte aligned and c % 8 == 0.
__device__ __forceinline__ void load8_bf16(const uint16_t* __restrict__ row, int c, int cols, float v[8]) {
  if (c + 8 <= cols) {
    uint4 w = *reinterpret_cast<const uint4*>(row + c);
    v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
    v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (c + i < cols) ? bf2f(row[c + i]) : 0.0f;
  }
}

}  // namespace vit
