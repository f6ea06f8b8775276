/*
 * vit.h - C ABI of libvit.so: the forward pass of a Qwen3-VL-style ViT
 * vision tower on one AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources):
 *  - FlashRT doc "Qwen3-VL-8B on RTX 5090 (NVFP4 language stack + FP8 ViT)",
 *    section 3 Inference architecture: patch_embed; 27 pre-norm blocks of
 *    LayerNorm -> qkv -> 2D rotate_half RoPE -> full bidirectional attention
 *    -> proj -> residual -> LayerNorm -> fc1 -> GELU(tanh) -> fc2 ->
 *    residual, hidden 1152, 16 heads x head_dim 72; DeepStack taps at layers
 *    8/16/24; 2x2 patch merger to out_hidden 4096; FFN 4304 zero-padded to
 *    4352.  Section 1: FP8 block-128 W8A8 GEMMs, bias adds fused.  Section 3:
 *    FP8 activation quant fused into LayerNorm and GELU.  Section 5: each
 *    image is an independent cu_seqlens attention window.
 *  - spark_model page "layers/vision_encoder.rs": weight list of struct
 *    ViTBlock / MergerLayer / VisionEncoder, PATCH_DIM = 1536, DeepStack
 *    indexes [8, 16, 24] after the Nth block plus the last block.
 *  - TensorRT-Model-Connect PR #2106, section Implementation: FP8 scale
 *    = amax / 448.
 *
 * Conventions for every entry point:
 *  - bf16 tensors are passed as uint16_t bit patterns, FP8 tensors as
 *    uint8_t OCP E4M3FN codes, scales as float.  Row-major throughout.
 *  - Every pointer argument is a DEVICE pointer unless its name ends in
 *    _host.  Device pointers must be 16-byte aligned (VIT_ERR_ALIGN).
 *  - The caller owns all memory it passes.  No entry point allocates, and
 *    the library is safe to call from several threads.  Its process-wide
 *    state: a cache of each device's compute-unit count (atomic, written on
 *    the first attention or GEMM launch on that device, which size their
 *    grids from it; every later call reads the same value) and, for
 *    vit_attention_noalloc only, one scratch array per device held in the
 *    code object, whose address is taken on the first such call on that
 *    device (see that entry point).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and runs asynchronously; no call synchronises with the host.
 *    Buffers must stay valid until that work has finished.
 *  - Arguments are validated on the host before anything is enqueued.  On
 *    any error the call returns a nonzero status, enqueues nothing and
 *    leaves every output untouched.  VIT_ERR_HIP means a launch failed
 *    after validation (outputs are then undefined).  Nothing aborts,
 *    prints or throws.
 *  - Outputs must not overlap inputs, except where a call documents an
 *    in-place operand.
 */
#ifndef VIT_H
#define VIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VIT_ABI_VERSION 5

/* Model dimensions (FlashRT section 3; spark_model struct VisionEncoder). */
#define VIT_HIDDEN 1152
#define VIT_HEADS 16
#define VIT_HEAD_DIM 72
#define VIT_MLP 4304
#define VIT_MLP_PADDED 4352
#define VIT_PATCH_DIM 1536
#define VIT_DEPTH 27
#define VIT_OUT_HIDDEN 4096
#define VIT_MERGED_DIM 4608
#define VIT_NUM_TAPS 4

typedef enum vit_status {
  VIT_OK = 0,
  VIT_ERR_NULL = 1,        /* a required pointer is NULL */
  VIT_ERR_ALIGN = 2,       /* a pointer or leading dimension is misaligned */
  VIT_ERR_SHAPE = 3,       /* a size is negative, too large or inconsistent */
  VIT_ERR_UNSUPPORTED = 4, /* valid request outside what the kernels implement */
  VIT_ERR_SEQLENS = 5,     /* cu_seqlens / image grids are not a valid packing */
  VIT_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required */
  VIT_ERR_ALIAS = 7,       /* an output overlaps an input it must not */
  VIT_ERR_HIP = 8          /* the HIP runtime reported an error */
} vit_status;

typedef void* vit_stream_t; /* hipStream_t */

int vit_abi_version(void);
const char* vit_status_string(int status);

/* ---------------------------------------------------------------------
 * FP8 block-128 quantiser (FlashRT section 1 "FP8 block-128"; section 3
 * "per-token / per-128-K-block FP8 activation quant"; PR #2106: scale
 * amax/448).  For each block of block_rows x 128 elements of x:
 *   amax = max |x|;  s = amax / 448, inv = 448 / amax (fp32, correctly
 *   rounded; both 0 when amax < 2^-116);  code = E4M3(x * inv), nearest
 *   with ties to even, saturating at +-448, -0 kept.
 * x: [rows, ld_x] bf16 (cols <= ld_x used, ld_x % 8 == 0).
 * block_rows: 1 (activations: per row, per 128 columns) or 128 (weights).
 * codes: [Rp, Cp] with Cp = ceil128(cols) and Rp = rows (block_rows 1) or
 *        ceil128(rows) (block_rows 128); padding codes are written as 0.
 * scales: [ceil(rows / block_rows), Cp / 128] float.
 * Ragged last blocks take their amax over the real elements only.
 * rows == 0 is a no-op.
 * ------------------------------------------------------------------- */
int vit_quant_fp8_block128(const uint16_t* x, int64_t ld_x, int rows, int cols,
                           int block_rows, uint8_t* codes, float* scales,
                           vit_stream_t stream);

/* The E4M3 encoder the quantising kernels use, exposed for testing:
 * codes[i] = E4M3(x[i]) (nearest, ties to even, saturating, -0 kept).
 * n >= 0, any n. */
int vit_e4m3_encode(const float* x, uint8_t* codes, int64_t n, vit_stream_t stream);

/* ---------------------------------------------------------------------
 * LayerNorm fused with the FP8 activation quant
 * (FlashRT section 3, layer_norm_to_fp8_block128_bf16: the normalised
 * activation goes straight to FP8 without a bf16 round trip).
 *   y = (x - mean) / sqrt(var + eps) * gamma + beta   (biased variance, fp32)
 *   codes, scales = block quant of y per row, per 128 columns (as above,
 *   from the fp32 value of y).
 * x: [M, ld_x] bf16; gamma, beta: [D] bf16; D % 128 == 0, D <= 8192.
 * codes: [M, D]; scales: [M, D/128]; prequant_debug: NULL or [M, D] fp32
 * receiving y before quantisation (for verification).
 * ------------------------------------------------------------------- */
int vit_layernorm_quant_fp8(const uint16_t* x, int64_t ld_x, const uint16_t* gamma,
                            const uint16_t* beta, float eps, int M, int D,
                            uint8_t* codes, float* scales, float* prequant_debug,
                            vit_stream_t stream);

/* ---------------------------------------------------------------------
 * LayerNorm with a bf16 result: the normalisation of the blocks that run
 * their GEMMs in bf16 (FlashRT section 4: "the first 3 blocks stay bf16").
 *   out = bf16((x - mean) / sqrt(var + eps) * gamma + beta)  (fp32 math)
 * x: [M, ld_x] bf16; gamma, beta: [D] bf16; D % 128 == 0, D <= 8192;
 * out: [M, ld_out] bf16, ld_out >= D.  out must not overlap x.
 * ------------------------------------------------------------------- */
int vit_layernorm(const uint16_t* x, int64_t ld_x, const uint16_t* gamma, const uint16_t* beta,
                  float eps, int M, int D, uint16_t* out, int64_t ld_out, vit_stream_t stream);

/* ---------------------------------------------------------------------
 * Block-scaled FP8 W8A8 GEMM with fused epilogues (FlashRT section 1:
 * FP8 block-128 ViT GEMMs, bias adds fused; section 3: GELU fused with the
 * FP8 quant of the fc2 input).
 *   C[m, n] = sum_kb a_scales[m, kb] * w_scales[n/128, kb]
 *                    * sum_{k in kb} E4M3(a[m, k]) * E4M3(w[n, k])
 * accumulated in fp32.  Kp = ceil128(K), Np = ceil128(N).
 * a: [M, Kp] codes (columns >= K must be zero codes); a_scales: [M, Kp/128].
 * w: [Np, Kp] codes (rows >= N zero); w_scales: [Np/128, Kp/128].
 * epilogue:
 *   VIT_EPI_BIAS:          out[m, n] = bf16(C + bias[n])            out [M, N]
 *   VIT_EPI_BIAS_RESIDUAL: out[m, n] = bf16(C + bias[n] + residual[m, n]);
 *                          residual [M, N] may be the same pointer as out
 *                          (in-place residual add), no other overlap.
 *   VIT_EPI_BIAS_GELU_FP8: y = GELU_tanh(C + bias[n]) for n < N, 0 for
 *                          N <= n < Np; out_codes [M, Np], out_scales
 *                          [M, Np/128] = block quant of y per row, per 128
 *                          columns; prequant_debug NULL or [M, Np] fp32 y.
 * bias: [N] bf16 or NULL (zero).  Unused output pointers may be NULL.
 * All leading dimensions are the logical widths (packed rows).  M <= 2^24,
 * N, K <= 2^20 (VIT_ERR_SHAPE).  M == 0 is a no-op.
 * ------------------------------------------------------------------- */
#define VIT_EPI_BIAS 0
#define VIT_EPI_BIAS_RESIDUAL 1
#define VIT_EPI_BIAS_GELU_FP8 2
int vit_fp8_block128_gemm(const uint8_t* a, const float* a_scales,
                          const uint8_t* w, const float* w_scales,
                          int M, int N, int K,
                          const uint16_t* bias, const uint16_t* residual, int epilogue,
                          uint16_t* out, uint8_t* out_codes, float* out_scales,
                          float* prequant_debug, vit_stream_t stream);

/* ---------------------------------------------------------------------
 * bf16 GEMM for the patch embedding and the merger MLPs (FlashRT section 4:
 * patch embed and mergers stay bf16).  C = A * W^T in fp32 with
 *   VIT_BEPI_BIAS:      out = bf16(C + bias)
 *   VIT_BEPI_BIAS_GELU: out = bf16(GELU_tanh(C + bias))
 *   VIT_BEPI_BIAS_ADD:  out = bf16(C + bias + add[m, n])   (position table)
 * a: [M, K] bf16, or fp32 when a_is_f32 (rounded to bf16, nearest even,
 * as it is loaded: the fp32 pixel buffer of the patch embedding).
 * w: [N, K] bf16; bias: [N] bf16 or NULL; add: [M, N] bf16 (BIAS_ADD only,
 * NULL = no add); out: [M, ld_out] bf16, ld_out >= N.
 * K % 8 == 0; M <= 2^24, N, K <= 2^20.  M == 0 is a no-op.
 * ------------------------------------------------------------------- */
#define VIT_BEPI_BIAS 0
#define VIT_BEPI_BIAS_GELU 1
#define VIT_BEPI_BIAS_ADD 2
int vit_bf16_gemm(const void* a, int a_is_f32, const uint16_t* w, int M, int N, int K,
                  const uint16_t* bias, const uint16_t* add, int epilogue,
                  uint16_t* out, int64_t ld_out, vit_stream_t stream);

/* ---------------------------------------------------------------------
 * 2D rotate_half rotary embedding, in place on Q and K (FlashRT section 3
 * "2D rotate_half RoPE", kernel rope_neox_qk_bf16; spark_model page:
 * head_dim/4 inverse frequencies).  For token t at (row, col) = pos_rc[t],
 * every head h, and axis a in {row, col} covering dims [a*hd/2, (a+1)*hd/2):
 *   f_i = theta^(-2i / (hd/2)), i < hd/4;  angle = p_a * f_i;
 *   (x[i], x[i + hd/4]) -> (x[i] cos - x[i+hd/4] sin, x[i+hd/4] cos + x[i] sin)
 * computed in fp32, stored bf16.
 * q, k: element (t, h, d) at [t*ld + h*head_dim + d]; ld % 4 == 0.
 * pos_rc: [T, 2] int32.  head_dim in {64, 72, 80, 128} (VIT_ERR_UNSUPPORTED
 * otherwise).  q and k must not overlap; they may interleave inside rows of
 * one buffer (q = qkv, k = qkv + H*hd with ld = 3*H*hd).
 * ------------------------------------------------------------------- */
int vit_rope2d(uint16_t* q, uint16_t* k, int64_t ld, const int32_t* pos_rc, int T,
               int num_heads, int head_dim, float theta, vit_stream_t stream);

/* ---------------------------------------------------------------------
 * Full bidirectional attention, varlen-packed (FlashRT section 3 "FA2
 * (full, bidirectional)"; section 5: each image its own cu_seqlens window).
 * For each window j = [cu[j], cu[j+1]) and head h:
 *   O_h = softmax(Q_h K_h^T * softmax_scale) V_h   (fp32 softmax, bf16 MMA)
 * q, k, v: element (t, h, d) at [t*ld_qkv + h*head_dim + d] (they may point
 * into one [T, 3*H*hd] qkv buffer); o: [t*ld_o + h*head_dim + d].
 * cu_seqlens_dev / cu_seqlens_host: the same num_seqs+1 int32 offsets on the
 * device and on the host (the host copy is read for validation and launch
 * sizing only); cu[0] = 0, non-decreasing, cu[num_seqs] = total_tokens.
 * head_dim must be 72 (VIT_ERR_UNSUPPORTED otherwise); ld_qkv, ld_o % 8 == 0
 * and <= 2^24; total_tokens <= 2^22.
 * workspace: >= vit_attention_workspace_size() bytes of device memory,
 * 16-byte aligned, not overlapping q, k, v or o (VIT_ERR_WORKSPACE if
 * missing or too small).  It holds fp32 partial results of (window, head,
 * 256-query) items whose key range is split between workgroups; its
 * contents on entry do not matter.  Two calls in flight at once (on
 * different streams) need different workspaces.
 * ------------------------------------------------------------------- */
size_t vit_attention_workspace_size(void);
int vit_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_qkv,
                  uint16_t* o, int64_t ld_o,
                  const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                  int num_seqs, int total_tokens, int num_heads, int head_dim,
                  float softmax_scale, void* workspace, size_t workspace_bytes,
                  vit_stream_t stream);

/* ---------------------------------------------------------------------
 * vit_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and errors as vit_attention,
 * without the workspace.  The partial results live in the library's own
 * array of vit_attention_noalloc_scratch_size() bytes (38.8 MB), one copy
 * per device, taken from the code object when the library is first used
 * on that device and held until the process ends; the need does not grow
 * with the input (it holds the partials of at most 256 ranges), so no
 * input is too large for it.  No call allocates (no hipMalloc / hipFree).
 * Calls that overlap in time on one device share that array and race:
 * serialise them (one stream, or events).  Nothing in the array needs to
 * be zero on entry.  The first call on a device may return VIT_ERR_HIP if
 * the array's address cannot be obtained there.
 * ------------------------------------------------------------------- */
size_t vit_attention_noalloc_scratch_size(void);
int vit_attention_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          int64_t ld_qkv, uint16_t* o, int64_t ld_o,
                          const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                          int num_seqs, int total_tokens, int num_heads, int head_dim,
                          float softmax_scale, vit_stream_t stream);

/* ---------------------------------------------------------------------
 * 2x2 spatial merge fused with the merger LayerNorm (FlashRT section 3
 * "2x2 patch merger"; spark_model page: spatial_merge_size 2).  For image j
 * with grid (h, w) = grid_hw[j] starting at token cu[j], merged row
 * cu[j]/4 + R*(w/2) + C is LayerNorm over the 4*D concatenation of tokens
 * (2R, 2C), (2R, 2C+1), (2R+1, 2C), (2R+1, 2C+1) (raster order).
 * x: [T, D] bf16 (D % 8 == 0); gamma, beta: [4D]; out: [T/4, 4D] bf16.
 * grid_hw_dev: [num_images, 2] int32 on the device, grid_hw_host the same
 * on the host (validation: h, w even, sum h*w == T).  cu_seqlens_dev:
 * [num_images + 1] int32 on the device, the token offsets of the images
 * (0, h0*w0, h0*w0 + h1*w1, ...; the cu_seqlens of the packing), which the
 * kernel binary-searches for each merged row's image; it must agree with
 * the grids (device data is not validated; a mismatch gives wrong values,
 * never an access outside x).
 * Errors: SHAPE, SEQLENS (grids), NULL, ALIGN (16-byte pointers), ALIAS
 * (out overlapping x, the grids or cu_seqlens_dev); nothing enqueued.
 * ------------------------------------------------------------------- */
int vit_merge2x2_layernorm(const uint16_t* x, int D, const int32_t* grid_hw_dev,
                           const int32_t* cu_seqlens_dev, const int32_t* grid_hw_host,
                           int num_images, int T, const uint16_t* gamma,
                           const uint16_t* beta, float eps, uint16_t* out,
                           vit_stream_t stream);

/* ---------------------------------------------------------------------
 * Learned position embedding resampled to each image's patch grid
 * (FlashRT section 3: "patch_embed -> +interpolated pos_embed"; spark_model
 * struct VisionEncoder: a [G*G, 1152] bf16 table with num_grid_per_side
 * G = 48).  The pages do not give the rule; this computes corner-aligned
 * bilinear samples: token (r, c) of an h x w image reads the table at
 * y = (G-1) r / (h-1), x = (G-1) c / (w-1) (0 for a single row / column),
 * in f32 with each operation rounded in the order
 *   ((w00 T[y0,x0] + w01 T[y0,x1]) + w10 T[y1,x0]) + w11 T[y1,x1],
 * w00 = (1-dy)(1-dx), w01 = (1-dy) dx, w10 = dy (1-dx), w11 = dy dx, and
 * stores bf16.
 * table: [G*G, dim] bf16 (1 <= G <= 1024, dim % 8 == 0).  grid_hw_dev /
 * grid_hw_host: [num_images, 2] int32 (h, w >= 1, sum h*w == T), tokens in
 * raster order per image, images packed in order.  cu_seqlens_dev:
 * [num_images + 1] int32 on the device, the images' token offsets, which
 * the kernel binary-searches for each token's image (it must agree with
 * the grids; a mismatch gives wrong values, never an access outside the
 * table or out).  out: [T, ld_out] bf16 (ld_out >= dim, ld_out % 8 == 0),
 * written in columns [0, dim).
 * Errors: SHAPE for out-of-range sizes, SEQLENS for grids that do not
 * sum to T, NULL / ALIGN (16-byte pointers) / ALIAS (out overlapping the
 * table, the grids or cu_seqlens_dev); nothing is enqueued on error.
 * ------------------------------------------------------------------- */
int vit_pos_embed_interp(const uint16_t* table, int grid_side, int dim,
                         const int32_t* grid_hw_dev, const int32_t* cu_seqlens_dev,
                         const int32_t* grid_hw_host, int num_images, int T,
                         uint16_t* out, int64_t ld_out, vit_stream_t stream);

/* ---------------------------------------------------------------------
 * Input preparation (FlashRT section 1: image preprocessing runs on the GPU
 * and max_pixels applies the processor's smart_resize, which rounds to the
 * patch grid; section 5: each image or video frame group is its own
 * attention window; spark_model PATCH_DIM doc: a patch is 3 x 2 x 16 x 16).
 *
 * vit_smart_resize (host only, no GPU work): the resized (height, width)
 * for an image, multiples of factor (32 = patch 16 x merge 2): each side
 * rounded to the nearest multiple (ties to even, at least factor); if the
 * area exceeds max_pixels (> 0), both sides are scaled by
 * sqrt(height * width / max_pixels) and floored to multiples; if it is
 * below min_pixels (> 0), scaled up by sqrt(min_pixels / (height * width))
 * and ceiled.  The 2172 x 724 image gives 736 x 2176 (6256 patches), and at
 * max_pixels 1e6 / 5e5 / 2.5e5 gives 3888 / 1824 / 972 patches.
 * Errors: NULL for missing outputs, SHAPE for sizes < 1 or > 2^20.
 *
 * vit_preprocess_frames: frames [num_frames, height, width, 3] u8 RGB on the
 * device -> pixels [ceil(num_frames/2) * (out_height/16) * (out_width/16),
 * 1536] f32 on the device, the input of vit_encoder_forward with one grid
 * (out_height/16, out_width/16) per frame pair.  Bilinear resize with
 * half-pixel centres, y = v / (255 std_c) - mean_c / std_c, patch rows in
 * raster order per frame pair, each laid out [channel][frame of the
 * pair][row][col]; a still image is one frame, and an odd last frame is
 * paired with itself.  mean_host / std_host: 3 floats on the host (std > 0).
 * out_height, out_width: multiples of 16 (of 32 for the encoder's 2x2
 * merge), e.g. from vit_smart_resize.  Errors: SHAPE, NULL, ALIGN (pixels
 * 16-byte aligned), ALIAS (pixels overlapping the frames).
 * ------------------------------------------------------------------- */
int vit_smart_resize(int height, int width, int factor, int64_t min_pixels, int64_t max_pixels,
                     int* out_height, int* out_width);
int vit_preprocess_frames(const uint8_t* frames, int num_frames, int height, int width,
                          int out_height, int out_width, const float* mean_host,
                          const float* std_host, float* pixels, vit_stream_t stream);

/* ---------------------------------------------------------------------
 * Weights of one block (spark_model struct ViTBlock).  FP8 weights are
 * 128x128-block quantised with vit_quant_fp8_block128(block_rows = 128).
 * Precision switch (FlashRT section 4: the first 3 blocks stay bf16): when
 * qkv_w, proj_w, fc1_w and fc2_w are all set, the block runs LayerNorm and
 * its four GEMMs in bf16 from them and the FP8 codes / scales may be NULL;
 * when they are all NULL, it runs the FP8 recipe.  Mixed sets are rejected.
 * ------------------------------------------------------------------- */
typedef struct vit_block_weights {
  const uint16_t* ln1_gamma;  /* [1152] bf16 */
  const uint16_t* ln1_beta;   /* [1152] */
  const uint8_t* qkv_codes;   /* [3456, 1152]: rows [q | k | v], each (head, dim) */
  const float* qkv_scales;    /* [27, 9] */
  const uint16_t* qkv_bias;   /* [3456] */
  const uint8_t* proj_codes;  /* [1152, 1152] */
  const float* proj_scales;   /* [9, 9] */
  const uint16_t* proj_bias;  /* [1152] */
  const uint16_t* ln2_gamma;  /* [1152] */
  const uint16_t* ln2_beta;   /* [1152] */
  const uint8_t* fc1_codes;   /* [4352, 1152], rows >= 4304 zero */
  const float* fc1_scales;    /* [34, 9] */
  const uint16_t* fc1_bias;   /* [4304] (entries beyond 4304 are not read) */
  const uint8_t* fc2_codes;   /* [1152, 4352], columns >= 4304 zero */
  const float* fc2_scales;    /* [9, 34] */
  const uint16_t* fc2_bias;   /* [1152] */
  const uint16_t* qkv_w;      /* [3456, 1152] bf16, or NULL */
  const uint16_t* proj_w;     /* [1152, 1152] bf16, or NULL */
  const uint16_t* fc1_w;      /* [4304, 1152] bf16, or NULL */
  const uint16_t* fc2_w;      /* [1152, 4304] bf16, or NULL */
} vit_block_weights;

/* Weights of one 2x2 merger MLP (spark_model struct MergerLayer), bf16.
 * Precision switch ("merger FP8", FlashRT section 1): when fc1_codes,
 * fc1_scales, fc2_codes and fc2_scales are all set (128x128-block
 * quantised like the block weights), the merger quantises its LayerNorm
 * output per token and 128 columns and runs both linears as block-scaled
 * FP8 GEMMs (GELU + requant fused into fc1); fc1_w / fc2_w may then be
 * NULL.  When they are all NULL, it runs in bf16.  Mixed sets are rejected. */
typedef struct vit_merger_weights {
  const uint16_t* ln_gamma;   /* [4608] */
  const uint16_t* ln_beta;    /* [4608] */
  const uint16_t* fc1_w;      /* [4608, 4608] */
  const uint16_t* fc1_b;      /* [4608] */
  const uint16_t* fc2_w;      /* [4096, 4608] */
  const uint16_t* fc2_b;      /* [4096] */
  const uint8_t* fc1_codes;   /* [4608, 4608] E4M3, or NULL */
  const float* fc1_scales;    /* [36, 36], or NULL */
  const uint8_t* fc2_codes;   /* [4096, 4608] E4M3, or NULL */
  const float* fc2_scales;    /* [32, 36], or NULL */
} vit_merger_weights;

typedef struct vit_encoder_weights {
  const uint16_t* patch_w;    /* [1152, 1536] bf16 */
  const uint16_t* patch_b;    /* [1152] */
  vit_block_weights blocks[VIT_DEPTH];
  vit_merger_weights mergers[VIT_NUM_TAPS]; /* DeepStack after 8, 16, 24; final after 27 */
  const uint16_t* pos_table;  /* [pos_grid_side^2, 1152] bf16, or NULL (no learned table) */
  int pos_grid_side;          /* G of pos_table (48), 1..1024; ignored when pos_table is NULL */
} vit_encoder_weights;

/* ---------------------------------------------------------------------
 * One pre-norm ViT block, in place on x (FlashRT section 3, "per block").
 *   a = Q(LN1(x));  qkv = bf16(a W_qkv^T + b);  q, k = RoPE2D(q, k);
 *   o = Attn(q, k, v; cu);  x = bf16(x + Q(o) W_proj^T + b);
 *   h = Q(GELU(Q(LN2(x)) W_fc1^T + b));  x = bf16(x + h W_fc2^T + b)
 * x_inout: [T, 1152] bf16.  pos_rc: [T, 2] int32 device.  cu_seqlens as
 * for vit_attention.  workspace: >= vit_block_workspace_size(T) bytes of
 * device memory, 256-byte aligned; its contents on entry do not matter.
 * ------------------------------------------------------------------- */
size_t vit_block_workspace_size(int T);
int vit_block_forward(const vit_block_weights* w, uint16_t* x_inout, int T,
                      const int32_t* pos_rc, const int32_t* cu_seqlens_dev,
                      const int32_t* cu_seqlens_host, int num_seqs,
                      void* workspace, size_t workspace_bytes, vit_stream_t stream);

/* ---------------------------------------------------------------------
 * The whole tower (FlashRT section 3): patch embed (bf16 GEMM, K = 1536,
 * plus a position embedding), 27 blocks, and after blocks 8, 16, 24 and 27
 * the 2x2 merger MLPs.  The position embedding added by the patch-embed
 * epilogue is either w->pos_table resampled to the grids (as by
 * vit_pos_embed_interp, into the workspace) or a precomputed [T, 1152]
 * table pos_embed; giving both is a SHAPE error, giving neither adds none.
 * w: host pointer to the weight table (its members are device pointers).
 * pixels: [T, 1536] fp32.  pos_embed: [T, 1152] bf16 or NULL.
 * grid_hw_dev / grid_hw_host: [num_images, 2] int32 patch grids (rows,
 * cols), each even; images are packed in order, T = sum h*w.
 * out: [4, T/4, 4096] bf16 (DeepStack 8, 16, 24, then final), merged rows
 * of the images in order.  last_hidden: NULL or [T, 1152] bf16 receiving
 * the output of block 27.
 * workspace: >= vit_encoder_workspace_size(T, num_images) bytes.
 * ------------------------------------------------------------------- */
size_t vit_encoder_workspace_size(int T, int num_images);
int vit_encoder_forward(const vit_encoder_weights* w, const float* pixels,
                        const uint16_t* pos_embed, const int32_t* grid_hw_dev,
                        const int32_t* grid_hw_host, int num_images, int T,
                        uint16_t* out, uint16_t* last_hidden,
                        void* workspace, size_t workspace_bytes, vit_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VIT_H */
