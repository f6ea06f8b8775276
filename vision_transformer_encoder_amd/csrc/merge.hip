// 2x2 spatial merge fused with the merger LayerNorm, and the per-token
// geometry of packed images (FlashRT "Qwen3-VL-8B on RTX 5090" page,
// section 3: "2x2 patch merger -> image_embeds"; spark_model
// "layers/vision_encoder.rs" page: spatial_merge_size 2, kernel
// vision_spatial_merge).  The merged row of image j at (R, C) concatenates
// the tokens (2R, 2C), (2R, 2C+1), (2R+1, 2C), (2R+1, 2C+1) of that image,
// tokens being in raster order.  HBM-bound: the gather reads each token once.
#include "common.h"
#include "kernels.h"

namespace vit {

// One wave per merged row; the 4*D features are NC chunks of 8 per lane.
template <int NC>
__global__ __launch_bounds__(256) void merge_layernorm_kernel(const uint16_t* __restrict__ x, int D,
                                                              const int32_t* __restrict__ grid_hw,
                                                              const int32_t* __restrict__ cu,
                                                              int num_images, int TM,
                                                              const uint16_t* __restrict__ gamma,
                                                              const uint16_t* __restrict__ beta,
                                                              float eps, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int mrow = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (mrow >= TM) return;
  // the image of this merged row: image j's merged rows start at cu[j] / 4
  const int j = image_of(cu, num_images, 4 * mrow);
  const int tok0 = cu[j], w = max(grid_hw[2 * j + 1], 2);
  const int local = mrow - tok0 / 4;
  const int R = local / (w / 2), C = local % (w / 2);
  // clamped into the batch (only matters if the device grids disagreed with
  // the validated host copy)
  const int last = 4 * TM - 1;
  const int src[4] = {min(tok0 + 2 * R * w + 2 * C, last), min(tok0 + 2 * R * w + 2 * C + 1, last),
                      min(tok0 + (2 * R + 1) * w + 2 * C, last), min(tok0 + (2 * R + 1) * w + 2 * C + 1, last)};
  const int D4 = 4 * D;
  const int nchunk = D4 >> 3, cpd = D >> 3;
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
  for (int i = 0; i < NC; ++i) {
    const int ch = min(i * 64 + lane, nchunk - 1);
    const int slot = ch / cpd, cc = ch - slot * cpd;
    xw[i] = *reinterpret_cast<const uint4*>(x + (int64_t)src[slot] * D + cc * 8);
  }
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
  const float mean = wave_sum(sum) / (float)D4;
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
  const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D4 + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int ch = i * 64 + lane;
    if (ch < nchunk) {
      const float gg[8] = {bf_lo(gw[i].x), bf_hi(gw[i].x), bf_lo(gw[i].y), bf_hi(gw[i].y),
                           bf_lo(gw[i].z), bf_hi(gw[i].z), bf_lo(gw[i].w), bf_hi(gw[i].w)};
      const float bb[8] = {bf_lo(bw[i].x), bf_hi(bw[i].x), bf_lo(bw[i].y), bf_hi(bw[i].y),
                           bf_lo(bw[i].z), bf_hi(bw[i].z), bf_lo(bw[i].w), bf_hi(bw[i].w)};
      uint4 o;
      o.x = pack_bf16x2((v[i][0] - mean) * rstd * gg[0] + bb[0], (v[i][1] - mean) * rstd * gg[1] + bb[1]);
      o.y = pack_bf16x2((v[i][2] - mean) * rstd * gg[2] + bb[2], (v[i][3] - mean) * rstd * gg[3] + bb[3]);
      o.z = pack_bf16x2((v[i][4] - mean) * rstd * gg[4] + bb[4], (v[i][5] - mean) * rstd * gg[5] + bb[5]);
      o.w = pack_bf16x2((v[i][6] - mean) * rstd * gg[6] + bb[6], (v[i][7] - mean) * rstd * gg[7] + bb[7]);
      *reinterpret_cast<uint4*>(out + (int64_t)mrow * D4 + ch * 8) = o;
    }
  }
}

hipError_t launch_merge_layernorm(const uint16_t* x, int D, const int32_t* grid_hw, const int32_t* cu,
                                  int num_images, int T, const uint16_t* gamma,
                                  const uint16_t* beta, float eps, uint16_t* out,
                                  hipStream_t stream) {
  const int TM = T / 4;
  if (TM == 0) return hipSuccess;
  const int nc = (4 * D / 8 + 63) / 64;
  const dim3 grid((TM + 3) / 4);
#define VIT_ML(N)                                                                                      \
  case N:                                                                                             \
    merge_layernorm_kernel<N><<<grid, 256, 0, stream>>>(x, D, grid_hw, cu, num_images, TM, gamma, beta, \
                                                        eps, out);                                 \
    break;
  switch (nc) {
    VIT_ML(1) VIT_ML(2) VIT_ML(3) VIT_ML(4) VIT_ML(5) VIT_ML(6) VIT_ML(7) VIT_ML(8)
    VIT_ML(9) VIT_ML(10) VIT_ML(11) VIT_ML(12) VIT_ML(13) VIT_ML(14) VIT_ML(15) VIT_ML(16)
    default:
      return hipErrorInvalidValue;
  }
#undef VIT_ML
  return hipGetLastError();
}

// ---------------------------------------------------------------- geometry
__global__ void cu_from_grids_kernel(const int32_t* __restrict__ grid_hw, int n, int32_t* __restrict__ cu) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    int acc = 0;
    cu[0] = 0;
    for (int j = 0; j < n; ++j) {
      acc += grid_hw[2 * j] * grid_hw[2 * j + 1];
      cu[j + 1] = acc;
    }
  }
}

__global__ __launch_bounds__(256) void positions_kernel(const int32_t* __restrict__ grid_hw,
                                                        const int32_t* __restrict__ cu, int n, int T,
                                                        int32_t* __restrict__ pos) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int lo = image_of(cu, n, t);
  const int w = grid_hw[2 * lo + 1];
  const int local = t - cu[lo];
  pos[2 * t] = local / w;
  pos[2 * t + 1] = local % w;
}

hipError_t launch_geometry(const int32_t* grid_hw, int num_images, int T, int32_t* cu,
                           int32_t* pos, hipStream_t stream) {
  cu_from_grids_kernel<<<1, 64, 0, stream>>>(grid_hw, num_images, cu);
  if (T > 0) positions_kernel<<<(T + 255) / 256, 256, 0, stream>>>(grid_hw, cu, num_images, T, pos);
  return hipGetLastError();
}

// ---------------------------------------------------------------- position table
// Learned position embedding resampled to each image's grid (FlashRT page,
// section 3: "patch_embed -> +interpolated pos_embed"; spark_model page,
// struct VisionEncoder: a [G*G, 1152] bf16 table, G = num_grid_per_side =
// 48, with an f32 host copy).  Corner-aligned bilinear samples: token (r, c)
// of an h x w image reads the table at y = (G-1) r / (h-1), x = (G-1) c /
// (w-1) (0 for a single row or column), in f32 with every operation rounded
// in this order and nothing contracted into an FMA:
//   w00 = (1-dy)(1-dx), w01 = (1-dy) dx, w10 = dy (1-dx), w11 = dy dx,
//   v = ((w00 T[y0,x0] + w01 T[y0,x1]) + w10 T[y1,x0]) + w11 T[y1,x1],
// stored as bf16.  One wave per token, 8 features per lane per step; the four
// table rows of a token are contiguous 16-byte loads.
// NC = 16-byte chunks per lane: all of a lane's loads (four table rows per
// chunk) are issued before the first wait.  NC = 0: rows wider than 8192,
// one chunk per loop trip.
template <int NC>
__global__ __launch_bounds__(256) void pos_interp_kernel(const uint16_t* __restrict__ table, int G, int D,
                                                         const int32_t* __restrict__ grid_hw,
                                                         const int32_t* __restrict__ cu, int num_images,
                                                         int T, uint16_t* __restrict__ out, int64_t ldo) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int j = image_of(cu, num_images, t);
  const int h = max(grid_hw[2 * j], 1), w = max(grid_hw[2 * j + 1], 1);
  // (r, c) clamped into the table's sample range (only matters if the device
  // grids disagreed with the validated host copy)
  const int local = t - cu[j], r = min(local / w, h - 1), c = local % w;
  // (G-1) i is an exact f32 integer; the division is correctly rounded
  const float y = h > 1 ? ((float)(G - 1) * (float)r) / (float)(h - 1) : 0.0f;
  const float x = w > 1 ? ((float)(G - 1) * (float)c) / (float)(w - 1) : 0.0f;
  const int y0 = (int)floorf(y), x0 = (int)floorf(x);
  const int y1 = min(y0 + 1, G - 1), x1 = min(x0 + 1, G - 1);
  const float dy = y - (float)y0, dx = x - (float)x0;
  const float w00 = (1.0f - dy) * (1.0f - dx), w01 = (1.0f - dy) * dx;
  const float w10 = dy * (1.0f - dx), w11 = dy * dx;
  const uint16_t* r00 = table + (int64_t)(y0 * G + x0) * D;
  const uint16_t* r01 = table + (int64_t)(y0 * G + x1) * D;
  const uint16_t* r10 = table + (int64_t)(y1 * G + x0) * D;
  const uint16_t* r11 = table + (int64_t)(y1 * G + x1) * D;
  uint16_t* orow = out + (int64_t)t * ldo;
  const int nch = D >> 3;
  if constexpr (NC == 0) {
    for (int ch = lane; ch < nch; ch += 64) {
      float a[8], b[8], e[8], f[8];
      load8_bf16(r00, ch * 8, D, a);
      load8_bf16(r01, ch * 8, D, b);
      load8_bf16(r10, ch * 8, D, e);
      load8_bf16(r11, ch * 8, D, f);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float s01 = w00 * a[i] + w01 * b[i];
        const float s2 = s01 + w10 * e[i];
        v[i] = s2 + w11 * f[i];
      }
      uint4 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      o.z = pack_bf16x2(v[4], v[5]);
      o.w = pack_bf16x2(v[6], v[7]);
      *reinterpret_cast<uint4*>(orow + ch * 8) = o;
    }
    return;
  }
  constexpr int kNC = NC > 0 ? NC : 1;
  uint4 q[kNC][4];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int ch = min(i * 64 + lane, nch - 1);  // lanes past the row re-read its last chunk
    q[i][0] = *reinterpret_cast<const uint4*>(r00 + ch * 8);
    q[i][1] = *reinterpret_cast<const uint4*>(r01 + ch * 8);
    q[i][2] = *reinterpret_cast<const uint4*>(r10 + ch * 8);
    q[i][3] = *reinterpret_cast<const uint4*>(r11 + ch * 8);
  }
  // every chunk is computed and stored, lanes past the row on their clamped
  // copy (the same value the owning lane writes there): with no branch, the
  // compiler keeps the loads ahead of the first wait
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int ch = i * 64 + lane;
    float a[8], b[8], e[8], f[8];
    unpack8_bf16(q[i][0], a);
    unpack8_bf16(q[i][1], b);
    unpack8_bf16(q[i][2], e);
    unpack8_bf16(q[i][3], f);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s01 = w00 * a[i] + w01 * b[i];
      const float s2 = s01 + w10 * e[i];
      v[i] = s2 + w11 * f[i];
    }
    uint4 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    o.z = pack_bf16x2(v[4], v[5]);
    o.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(orow + min(ch, nch - 1) * 8) = o;
  }
}

hipError_t launch_pos_interp(const uint16_t* table, int G, int D, const int32_t* grid_hw, const int32_t* cu,
                             int num_images, int T, uint16_t* out, int64_t ldo, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4);
#define VIT_PI(N)                                                                                  \
  case N:                                                                                          \
    pos_interp_kernel<N><<<grid, 256, 0, stream>>>(table, G, D, grid_hw, cu, num_images, T, out, ldo); \
    break;
  switch ((D / 8 + 63) / 64) {
    VIT_PI(1) VIT_PI(2) VIT_PI(3) VIT_PI(4) VIT_PI(5) VIT_PI(6) VIT_PI(7) VIT_PI(8)
    VIT_PI(9) VIT_PI(10) VIT_PI(11) VIT_PI(12) VIT_PI(13) VIT_PI(14) VIT_PI(15) VIT_PI(16)
    default:
      pos_interp_kernel<0><<<grid, 256, 0, stream>>>(table, G, D, grid_hw, cu, num_images, T, out, ldo);
  }
#undef VIT_PI
  return hipGetLastError();
}

}  // namespace vit
