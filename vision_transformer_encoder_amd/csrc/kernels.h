// Internal launchers of libvit's kernels.  Arguments are validated by the
// C ABI layer (abi.cpp) before any of these is called; each launcher only
// enqueues work on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vit {

hipError_t launch_quant_rows(const uint16_t* x, int64_t ldx, int rows, int cols, uint8_t* codes,
                             float* scales, hipStream_t stream);
hipError_t launch_quant_blocks128(const uint16_t* x, int64_t ldx, int rows, int cols,
                                  uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_e4m3_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream);
hipError_t launch_layernorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                                  const uint16_t* beta, float eps, int M, int D, uint8_t* codes,
                                  float* scales, float* prequant, hipStream_t stream);
// LayerNorm with the normalised row stored in bf16 (same kernel, no quant).
hipError_t launch_layernorm_bf16(const uint16_t* x, int64_t ldx, const uint16_t* gamma, const uint16_t* beta,
                                 float eps, int M, int D, uint16_t* out, int64_t ldo, hipStream_t stream);

// Compute units of the current device, cached per device (attention.hip).
int device_cu_count();

hipError_t launch_fp8_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w,
                           const float* w_scales, int M, int N, int K, const uint16_t* bias,
                           const uint16_t* residual, int epilogue, uint16_t* out,
                           uint8_t* out_codes, float* out_scales, float* prequant,
                           hipStream_t stream);

hipError_t launch_bf16_gemm(const void* a, bool a_f32, const uint16_t* w, int M, int N, int K,
                            const uint16_t* bias, const uint16_t* add, int epilogue,
                            uint16_t* out, int64_t ld_out, hipStream_t stream);

// The bf16 GEMM of gemm_wide.hip (256 x 128 tiles, 64 x 64 ones for small
// M) for bf16 A: usable when bf16_gemm_wide_fits(); epilogue 0 (bias) or 1
// (bias + GELU).
bool bf16_gemm_wide_fits(int N, int K, int64_t ld_out, const void* out, const void* bias);
hipError_t launch_bf16_gemm_wide(const uint16_t* a, const uint16_t* w, int M, int N, int K, const uint16_t* bias,
                                 int epilogue, uint16_t* out, int64_t ld_out, hipStream_t stream);

hipError_t launch_rope2d(uint16_t* q, uint16_t* k, int64_t ld, const int32_t* pos, int T,
                         int heads, int head_dim, float theta, hipStream_t stream);

// Stream-K plan of one attention launch, from the host copy of cu_seqlens:
// the work per head (sum over windows of 256-query tiles x 64-key tiles),
// one range of the work order per workgroup, and where each range starts
// (its window and the position inside that window's (q tile, key tile)
// list), so that the kernels never search the windows.
constexpr int kAttnMaxRanges = 256;
struct AttnRangeStart {
  int32_t win;
  int32_t rem;
};
struct AttnPlan {
  int64_t work_per_head;
  int num_ranges;
  AttnRangeStart start[kAttnMaxRanges];
};
void plan_attention(const int32_t* cu_host, int num_seqs, int heads, AttnPlan* plan);

// Stream-K attention: `partial` is device memory of attention_partial_bytes()
// for the partials of items that the per-workgroup ranges cut; the launch
// enqueues the main kernel and the combine kernel.
hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            int64_t ld_qkv, uint16_t* o, int64_t ld_o, const int32_t* cu,
                            int num_seqs, int total_tokens, const AttnPlan& plan, int heads,
                            float scale, float* partial, hipStream_t stream);
size_t attention_partial_bytes();
// Device address (for the device `stream` runs on) of the library's own
// copy of the attention partials, used by vit_attention_noalloc; set up on
// the first call per device.
hipError_t attention_scratch(hipStream_t stream, float** ptr);
size_t attention_scratch_bytes();

// grid_hw [n][2] and cu [n + 1] (the token offsets of the images) describe
// the same packing.
hipError_t launch_merge_layernorm(const uint16_t* x, int D, const int32_t* grid_hw, const int32_t* cu,
                                  int num_images, int T, const uint16_t* gamma,
                                  const uint16_t* beta, float eps, uint16_t* out,
                                  hipStream_t stream);

// cu[0..n] and (row, col) per token from the packed image grids.
hipError_t launch_geometry(const int32_t* grid_hw, int num_images, int T, int32_t* cu,
                           int32_t* pos, hipStream_t stream);

hipError_t launch_preprocess(const uint8_t* frames, int F, int H, int W, int Ho, int Wo, const float a[3],
                             const float b[3], float* out, hipStream_t stream);

hipError_t launch_pos_interp(const uint16_t* table, int G, int D, const int32_t* grid_hw, const int32_t* cu,
                             int num_images, int T, uint16_t* out, int64_t ldo, hipStream_t stream);

}  // namespace vit
