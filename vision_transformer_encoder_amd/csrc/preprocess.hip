// Image / video frames -> the tower's patch input (FlashRT "Qwen3-VL-8B on
// RTX 5090" page: section 1, image preprocessing on the GPU and max_pixels
// through the processor's smart_resize, which rounds to the patch grid;
// section 5, each image or video frame group is its own attention window;
// spark_model "layers/vision_encoder.rs" page, PATCH_DIM doc: a patch is
// C x temporal_patch_size x patch_size^2 = 3 x 2 x 16 x 16 = 1536 values).
//
// Frames [F, H, W, 3] u8 (RGB, row-major) are resized to H' x W' with
// bilinear half-pixel-centre sampling, normalised per channel and cut into
// 16 x 16 patches: frames 2g and 2g+1 form temporal group g (a missing last
// frame repeats the one before), group g is a window of (H'/16) x (W'/16)
// patches in raster order, and a patch row holds [channel][frame of the
// pair][row][col].  All arithmetic is f32 with every operation rounded in a
// fixed order (nothing contracted into an FMA):
//   s = (o + 1/2) (H / H') - 1/2, clamped at 0;  i0 = floor(s),
//   i1 = min(i0 + 1, H - 1), l = s - i0, h = 1 - l (the same along x);
//   v = hy (hx P00 + lx P01) + ly (hx P10 + lx P11);  y = v a_c + b_c,
// with a_c = 1 / (255 std_c) and b_c = -mean_c / std_c rounded to f32.
//
// HBM-bound: one workgroup per patch row writes its 1536 floats with
// consecutive lanes on consecutive columns; the four source bytes of each
// output come from the same few frame rows, which stay in L1/L2.
#include "common.h"
#include "kernels.h"

namespace vit {

struct PreParams {
  const uint8_t* frames;
  float* out;
  int F, H, W, Ho, Wo, gw, per_group;  // per_group = (Ho/16) * (Wo/16)
  float sy, sx;                        // H / Ho, W / Wo in f32
  float a[3], b[3];
};

__global__ __launch_bounds__(256) void preprocess_kernel(PreParams p) {
#pragma clang fp contract(off)
  // each thread owns columns tid + 256 k of the patch row (k < 6); all 24 of
  // its source bytes are loaded before the first wait
  constexpr int kPer = 1536 / 256;
  const int row = blockIdx.x;
  const int g = row / p.per_group, local = row - g * p.per_group;
  const int pr = local / p.gw, pc = local - pr * p.gw;
  float* orow = p.out + (int64_t)row * 1536;
  float px4[kPer][4], ly[kPer], lx[kPer];
  int cch[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int col = threadIdx.x + 256 * k;
    const int c = col >> 9, t = (col >> 8) & 1, py = (col >> 4) & 15, px = col & 15;
    const int f = min(2 * g + t, p.F - 1);
    const int oy = pr * 16 + py, ox = pc * 16 + px;
    float ys = ((float)oy + 0.5f) * p.sy - 0.5f;
    float xs = ((float)ox + 0.5f) * p.sx - 0.5f;
    ys = fmaxf(ys, 0.0f);
    xs = fmaxf(xs, 0.0f);
    // s < n - 1/2 for every output, so floor(s) <= n - 1; the clamp only
    // guards the loads
    const int y0 = min((int)floorf(ys), p.H - 1), x0 = min((int)floorf(xs), p.W - 1);
    const int y1 = min(y0 + 1, p.H - 1), x1 = min(x0 + 1, p.W - 1);
    ly[k] = ys - (float)y0;
    lx[k] = xs - (float)x0;
    cch[k] = c;
    const uint8_t* fr = p.frames + (int64_t)f * p.H * p.W * 3;
    px4[k][0] = (float)fr[((int64_t)y0 * p.W + x0) * 3 + c];
    px4[k][1] = (float)fr[((int64_t)y0 * p.W + x1) * 3 + c];
    px4[k][2] = (float)fr[((int64_t)y1 * p.W + x0) * 3 + c];
    px4[k][3] = (float)fr[((int64_t)y1 * p.W + x1) * 3 + c];
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const float hy = 1.0f - ly[k], hx = 1.0f - lx[k];
    const float top = hx * px4[k][0] + lx[k] * px4[k][1];
    const float bot = hx * px4[k][2] + lx[k] * px4[k][3];
    const float v = hy * top + ly[k] * bot;
    const int c = cch[k];
    orow[threadIdx.x + 256 * k] = v * p.a[c] + p.b[c];
  }
}

hipError_t launch_preprocess(const uint8_t* frames, int F, int H, int W, int Ho, int Wo, const float a[3],
                             const float b[3], float* out, hipStream_t stream) {
  PreParams p;
  p.frames = frames;
  p.out = out;
  p.F = F;
  p.H = H;
  p.W = W;
  p.Ho = Ho;
  p.Wo = Wo;
  p.gw = Wo / 16;
  p.per_group = (Ho / 16) * (Wo / 16);
  p.sy = (float)H / (float)Ho;
  p.sx = (float)W / (float)Wo;
  for (int c = 0; c < 3; ++c) {
    p.a[c] = a[c];
    p.b[c] = b[c];
  }
  const int64_t rows = (int64_t)((F + 1) / 2) * p.per_group;
  if (rows == 0) return hipSuccess;
  preprocess_kernel<<<(unsigned)rows, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace vit
