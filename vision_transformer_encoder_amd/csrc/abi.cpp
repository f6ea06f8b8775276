// C ABI of libvit.so (declared in include/vit.h): host-side argument
// validation, workspace layout and the orchestration of the block and of the
// whole tower.  Every entry point validates all of its arguments before it
// enqueues anything; on error it returns a status and touches nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>
#include <cstdint>

#include "kernels.h"
#include "vit.h"

namespace {

using vit::launch_attention;

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? VIT_OK : VIT_ERR_HIP; }

// Byte ranges [a, a + na) and [b, b + nb) overlap (empty ranges never do).
inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

inline size_t rup(size_t n, size_t a = 256) { return (n + a - 1) / a * a; }
inline int ceil128(int n) { return (n + 127) / 128 * 128; }

constexpr int kMaxTokens = 1 << 22;  // 4M tokens
constexpr int kMaxDim = 1 << 20;

// Validate a packing cu[0..n]: starts at 0, non-decreasing, ends at total.
inline bool valid_cu(const int32_t* cu, int n, int total) {
  if (cu[0] != 0) return false;
  for (int i = 0; i < n; ++i)
    if (cu[i + 1] < cu[i]) return false;
  return cu[n] == total;
}

// Image grids: every (h, w) even and >= 2, sum h*w == T.
inline bool valid_grids(const int32_t* g, int n, int T) {
  int64_t acc = 0;
  for (int j = 0; j < n; ++j) {
    const int h = g[2 * j], w = g[2 * j + 1];
    if (h < 2 || w < 2 || (h & 1) || (w & 1)) return false;
    acc += (int64_t)h * w;
    if (acc > T) return false;
  }
  return acc == T;
}

// ---------------------------------------------------------------- workspace
struct BlockWs {
  uint16_t* qkv;     // [T, 3456]
  uint16_t* o;       // [T, 1152]
  float* attn_part;  // attention partials (attention_partial_bytes())
  uint8_t* a_codes;  // [T, 1152]
  float* a_scales;   // [T, 9]
  uint8_t* h_codes;  // [T, 4352]
  float* h_scales;   // [T, 34]
  size_t bytes;
};

BlockWs block_ws_layout(void* base, int T) {
  BlockWs w{};
  size_t off = 0;
  auto take = [&](size_t n) {
    void* p = base ? static_cast<uint8_t*>(base) + off : nullptr;
    off += rup(n);
    return p;
  };
  const size_t t = (size_t)T;
  w.qkv = static_cast<uint16_t*>(take(t * 3 * VIT_HIDDEN * 2));
  w.o = static_cast<uint16_t*>(take(t * VIT_HIDDEN * 2));
  w.attn_part = static_cast<float*>(take(vit::attention_partial_bytes()));
  w.a_codes = static_cast<uint8_t*>(take(t * VIT_HIDDEN));
  w.a_scales = static_cast<float*>(take(t * (VIT_HIDDEN / 128) * 4));
  w.h_codes = static_cast<uint8_t*>(take(t * VIT_MLP_PADDED));
  w.h_scales = static_cast<float*>(take(t * (VIT_MLP_PADDED / 128) * 4));
  w.bytes = off;
  return w;
}

struct EncoderWs {
  BlockWs blk;
  uint16_t* x;      // [T, 1152] (used when last_hidden is NULL)
  int32_t* cu;      // [n + 1]
  int32_t* pos;     // [T, 2]
  uint16_t* m_ln;   // [T/4, 4608]  (inside blk.qkv: free between blocks)
  uint16_t* m_h;    // [T/4, 4608]
  size_t bytes;
};

EncoderWs encoder_ws_layout(void* base, int T, int n) {
  EncoderWs e{};
  e.blk = block_ws_layout(base, T);
  size_t off = e.blk.bytes;
  auto take = [&](size_t nb) {
    void* p = base ? static_cast<uint8_t*>(base) + off : nullptr;
    off += rup(nb);
    return p;
  };
  const size_t t = (size_t)T;
  e.x = static_cast<uint16_t*>(take(t * VIT_HIDDEN * 2));
  e.cu = static_cast<int32_t*>(take((size_t)(n + 1) * 4));
  e.pos = static_cast<int32_t*>(take(t * 2 * 4));
  e.bytes = off;
  // merger scratch reuses the qkv region: T/4 * 4608 * 2 bytes each, two of
  // them fit in T * 3456 * 2 bytes.
  const size_t mbytes = rup((t / 4) * VIT_MERGED_DIM * 2);
  e.m_ln = e.blk.qkv;
  e.m_h = base ? reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(e.blk.qkv) + mbytes) : nullptr;
  return e;
}

// ---------------------------------------------------------------- checks
// Pointers of `req` must all be set; of the two optional sets, exactly the
// one `use_a` selects must be complete (the other is ignored when complete
// and rejected when partly set).  Every set pointer must be 16-byte aligned.
template <size_t NR, size_t NA, size_t NB>
int check_weight_sets(const void* const (&req)[NR], const void* const (&a)[NA], const void* const (&b)[NB],
                      bool& use_a) {
  auto count = [](auto& arr) {
    int n = 0;
    for (const void* p : arr) n += p != nullptr;
    return n;
  };
  for (const void* p : req)
    if (!p) return VIT_ERR_NULL;
  const int na = count(a), nb = count(b);
  if ((na != 0 && na != (int)NA) || (na == 0 && nb != (int)NB)) return VIT_ERR_NULL;
  use_a = na == (int)NA;
  for (const void* p : req)
    if (!al16(p)) return VIT_ERR_ALIGN;
  for (const void* p : a)
    if (p && !al16(p)) return VIT_ERR_ALIGN;
  for (const void* p : b)
    if (p && !al16(p)) return VIT_ERR_ALIGN;
  return VIT_OK;
}

// bf16 is set when the block runs its GEMMs in bf16
int check_block_weights(const vit_block_weights* w, bool* bf16 = nullptr) {
  if (!w) return VIT_ERR_NULL;
  const void* const req[] = {w->ln1_gamma, w->ln1_beta, w->qkv_bias, w->proj_bias,
                             w->ln2_gamma, w->ln2_beta, w->fc1_bias, w->fc2_bias};
  const void* const bf[] = {w->qkv_w, w->proj_w, w->fc1_w, w->fc2_w};
  const void* const f8[] = {w->qkv_codes, w->qkv_scales, w->proj_codes, w->proj_scales,
                            w->fc1_codes, w->fc1_scales, w->fc2_codes, w->fc2_scales};
  bool use_bf = false;
  const int st = check_weight_sets(req, bf, f8, use_bf);
  if (bf16) *bf16 = use_bf;
  return st;
}

// fp8 is set when the merger runs its linears in FP8
int check_merger_weights(const vit_merger_weights* m, bool* fp8 = nullptr) {
  const void* const req[] = {m->ln_gamma, m->ln_beta, m->fc1_b, m->fc2_b};
  const void* const f8[] = {m->fc1_codes, m->fc1_scales, m->fc2_codes, m->fc2_scales};
  const void* const bf[] = {m->fc1_w, m->fc2_w};
  bool use_f8 = false;
  const int st = check_weight_sets(req, f8, bf, use_f8);
  if (fp8) *fp8 = use_f8;
  return st;
}

// ---------------------------------------------------------------- block
// The bf16-GEMM block (FlashRT section 4: the first 3 blocks stay bf16).
// Workspace reuse: the LayerNorm outputs [T, 1152] bf16 live in the region
// of the FP8 activation and hidden codes (unused here), the GELU output
// [T, 4304] bf16 in the qkv + o regions, dead once proj has read o.
hipError_t block_forward_bf16_impl(const vit_block_weights* w, uint16_t* x, int T, const int32_t* pos,
                                   const int32_t* cu_dev, int num_seqs, const vit::AttnPlan& plan, const BlockWs& ws,
                                   hipStream_t s) {
  constexpr int H = VIT_HIDDEN;
  const size_t t = (size_t)T;
  uint16_t* y = reinterpret_cast<uint16_t*>(ws.a_codes);
  uint16_t* h = ws.qkv;
  if ((size_t)(reinterpret_cast<uint8_t*>(ws.attn_part) - reinterpret_cast<uint8_t*>(ws.qkv)) <
          t * VIT_MLP * 2 ||
      (size_t)(reinterpret_cast<uint8_t*>(ws.h_scales) + t * (VIT_MLP_PADDED / 128) * 4 - ws.a_codes) < t * H * 2)
    return hipErrorInvalidValue;  // the layout no longer has room: a build error, not a caller's
  hipError_t e;
  if ((e = vit::launch_layernorm_bf16(x, H, w->ln1_gamma, w->ln1_beta, 1e-6f, T, H, y, H, s)) != hipSuccess)
    return e;
  if ((e = vit::launch_bf16_gemm(y, false, w->qkv_w, T, 3 * H, H, w->qkv_bias, nullptr, VIT_BEPI_BIAS, ws.qkv,
                                 3 * H, s)) != hipSuccess) return e;
  if ((e = vit::launch_rope2d(ws.qkv, ws.qkv + H, 3 * H, pos, T, VIT_HEADS, VIT_HEAD_DIM, 10000.0f, s)) !=
      hipSuccess) return e;
  if ((e = launch_attention(ws.qkv, ws.qkv + H, ws.qkv + 2 * H, 3 * H, ws.o, H, cu_dev, num_seqs, T, plan,
                            VIT_HEADS, 1.0f / std::sqrt((float)VIT_HEAD_DIM), ws.attn_part, s)) != hipSuccess)
    return e;
  // x = bf16(x + o W_proj^T + b), in place (each element read before it is written)
  if ((e = vit::launch_bf16_gemm(ws.o, false, w->proj_w, T, H, H, w->proj_bias, x, VIT_BEPI_BIAS_ADD, x, H, s)) !=
      hipSuccess) return e;
  if ((e = vit::launch_layernorm_bf16(x, H, w->ln2_gamma, w->ln2_beta, 1e-6f, T, H, y, H, s)) != hipSuccess)
    return e;
  if ((e = vit::launch_bf16_gemm(y, false, w->fc1_w, T, VIT_MLP, H, w->fc1_bias, nullptr, VIT_BEPI_BIAS_GELU, h,
                                 VIT_MLP, s)) != hipSuccess) return e;
  return vit::launch_bf16_gemm(h, false, w->fc2_w, T, H, VIT_MLP, w->fc2_bias, x, VIT_BEPI_BIAS_ADD, x, H, s);
}

hipError_t block_forward_impl(const vit_block_weights* w, uint16_t* x, int T, const int32_t* pos,
                              const int32_t* cu_dev, int num_seqs, const vit::AttnPlan& plan, const BlockWs& ws,
                              hipStream_t s) {
  constexpr int H = VIT_HIDDEN;
  if (w->qkv_w) return block_forward_bf16_impl(w, x, T, pos, cu_dev, num_seqs, plan, ws, s);
  hipError_t e;
  // LN1 -> FP8 (per token, per 128 columns)
  if ((e = vit::launch_layernorm_quant(x, H, w->ln1_gamma, w->ln1_beta, 1e-6f, T, H, ws.a_codes,
                                       ws.a_scales, nullptr, s)) != hipSuccess) return e;
  // qkv = bf16(a W^T + b)
  if ((e = vit::launch_fp8_gemm(ws.a_codes, ws.a_scales, w->qkv_codes, w->qkv_scales, T, 3 * H, H,
                                w->qkv_bias, nullptr, VIT_EPI_BIAS, ws.qkv, nullptr, nullptr, nullptr,
                                s)) != hipSuccess) return e;
  // RoPE on q and k in place
  if ((e = vit::launch_rope2d(ws.qkv, ws.qkv + H, 3 * H, pos, T, VIT_HEADS, VIT_HEAD_DIM, 10000.0f, s)) !=
      hipSuccess) return e;
  // attention
  if ((e = launch_attention(ws.qkv, ws.qkv + H, ws.qkv + 2 * H, 3 * H, ws.o, H, cu_dev, num_seqs, T, plan,
                            VIT_HEADS, 1.0f / std::sqrt((float)VIT_HEAD_DIM), ws.attn_part, s)) != hipSuccess)
    return e;
  // proj: x = bf16(x + Q(o) W^T + b)
  if ((e = vit::launch_quant_rows(ws.o, H, T, H, ws.a_codes, ws.a_scales, s)) != hipSuccess) return e;
  if ((e = vit::launch_fp8_gemm(ws.a_codes, ws.a_scales, w->proj_codes, w->proj_scales, T, H, H,
                                w->proj_bias, x, VIT_EPI_BIAS_RESIDUAL, x, nullptr, nullptr, nullptr, s)) !=
      hipSuccess) return e;
  // LN2 -> FP8; fc1 + GELU -> FP8; fc2 + residual
  if ((e = vit::launch_layernorm_quant(x, H, w->ln2_gamma, w->ln2_beta, 1e-6f, T, H, ws.a_codes,
                                       ws.a_scales, nullptr, s)) != hipSuccess) return e;
  if ((e = vit::launch_fp8_gemm(ws.a_codes, ws.a_scales, w->fc1_codes, w->fc1_scales, T, VIT_MLP, H,
                                w->fc1_bias, nullptr, VIT_EPI_BIAS_GELU_FP8, nullptr, ws.h_codes,
                                ws.h_scales, nullptr, s)) != hipSuccess) return e;
  return vit::launch_fp8_gemm(ws.h_codes, ws.h_scales, w->fc2_codes, w->fc2_scales, T, H, VIT_MLP,
                              w->fc2_bias, x, VIT_EPI_BIAS_RESIDUAL, x, nullptr, nullptr, nullptr, s);
}

hipError_t merger_forward_impl(const vit_merger_weights* m, const uint16_t* x, const int32_t* grid_dev,
                               const int32_t* cu_dev, int n, int T, uint16_t* out, const EncoderWs& ws,
                               hipStream_t s) {
  hipError_t e;
  const int TM = T / 4;
  if ((e = vit::launch_merge_layernorm(x, VIT_HIDDEN, grid_dev, cu_dev, n, T, m->ln_gamma, m->ln_beta, 1e-6f,
                                       ws.m_ln, s)) != hipSuccess) return e;
  if (m->fc1_codes) {
    // "merger FP8" (FlashRT section 1): the block recipe on the 4608-wide
    // merged rows.  Codes [T/4, 4608] and scales [T/4, 36] fit the block's
    // activation and hidden code regions exactly (T/4 * 4608 = T * 1152).
    const BlockWs& b = ws.blk;
    if ((e = vit::launch_quant_rows(ws.m_ln, VIT_MERGED_DIM, TM, VIT_MERGED_DIM, b.a_codes, b.a_scales, s)) !=
        hipSuccess) return e;
    if ((e = vit::launch_fp8_gemm(b.a_codes, b.a_scales, m->fc1_codes, m->fc1_scales, TM, VIT_MERGED_DIM,
                                  VIT_MERGED_DIM, m->fc1_b, nullptr, VIT_EPI_BIAS_GELU_FP8, nullptr, b.h_codes,
                                  b.h_scales, nullptr, s)) != hipSuccess) return e;
    return vit::launch_fp8_gemm(b.h_codes, b.h_scales, m->fc2_codes, m->fc2_scales, TM, VIT_OUT_HIDDEN,
                                VIT_MERGED_DIM, m->fc2_b, nullptr, VIT_EPI_BIAS, out, nullptr, nullptr, nullptr, s);
  }
  if ((e = vit::launch_bf16_gemm(ws.m_ln, false, m->fc1_w, TM, VIT_MERGED_DIM, VIT_MERGED_DIM, m->fc1_b,
                                 nullptr, VIT_BEPI_BIAS_GELU, ws.m_h, VIT_MERGED_DIM, s)) != hipSuccess)
    return e;
  return vit::launch_bf16_gemm(ws.m_h, false, m->fc2_w, TM, VIT_OUT_HIDDEN, VIT_MERGED_DIM, m->fc2_b,
                               nullptr, VIT_BEPI_BIAS, out, VIT_OUT_HIDDEN, s);
}

}  // namespace

extern "C" {

int vit_abi_version(void) { return VIT_ABI_VERSION; }

const char* vit_status_string(int status) {
  switch (status) {
    case VIT_OK: return "ok";
    case VIT_ERR_NULL: return "required pointer is NULL";
    case VIT_ERR_ALIGN: return "pointer or leading dimension misaligned";
    case VIT_ERR_SHAPE: return "invalid size";
    case VIT_ERR_UNSUPPORTED: return "unsupported configuration";
    case VIT_ERR_SEQLENS: return "invalid cu_seqlens or image grids";
    case VIT_ERR_WORKSPACE: return "workspace missing or too small";
    case VIT_ERR_ALIAS: return "output overlaps an input";
    case VIT_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int vit_quant_fp8_block128(const uint16_t* x, int64_t ld_x, int rows, int cols, int block_rows,
                           uint8_t* codes, float* scales, vit_stream_t stream) {
  if (rows < 0 || cols < 1 || rows > kMaxTokens * 4 || cols > kMaxDim) return VIT_ERR_SHAPE;
  if (block_rows != 1 && block_rows != 128) return VIT_ERR_UNSUPPORTED;
  if (ld_x < cols) return VIT_ERR_SHAPE;
  if (rows == 0) return VIT_OK;
  if (!x || !codes || !scales) return VIT_ERR_NULL;
  if (!al16(x) || !al16(codes) || !al16(scales) || (ld_x & 7)) return VIT_ERR_ALIGN;
  const int Cp = ceil128(cols);
  const int Rp = block_rows == 1 ? rows : ceil128(rows);
  const size_t xb = ((size_t)(rows - 1) * ld_x + cols) * 2;
  const size_t cb = (size_t)Rp * Cp;
  const size_t sb = (size_t)((rows + block_rows - 1) / block_rows) * (Cp / 128) * 4;
  if (overlap(x, xb, codes, cb) || overlap(x, xb, scales, sb) || overlap(codes, cb, scales, sb))
    return VIT_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(block_rows == 1 ? vit::launch_quant_rows(x, ld_x, rows, cols, codes, scales, s)
                                    : vit::launch_quant_blocks128(x, ld_x, rows, cols, codes, scales, s));
}

int vit_e4m3_encode(const float* x, uint8_t* codes, int64_t n, vit_stream_t stream) {
  if (n < 0 || n > ((int64_t)1 << 40)) return VIT_ERR_SHAPE;
  if (n == 0) return VIT_OK;
  if (!x || !codes) return VIT_ERR_NULL;
  if (!al16(x) || !al16(codes)) return VIT_ERR_ALIGN;
  if (overlap(x, (size_t)n * 4, codes, (size_t)n)) return VIT_ERR_ALIAS;
  return hip_status(vit::launch_e4m3_encode(x, codes, n, static_cast<hipStream_t>(stream)));
}

int vit_layernorm_quant_fp8(const uint16_t* x, int64_t ld_x, const uint16_t* gamma, const uint16_t* beta,
                            float eps, int M, int D, uint8_t* codes, float* scales, float* prequant_debug,
                            vit_stream_t stream) {
  if (M < 0 || M > kMaxTokens * 4 || D < 128 || D > 8192 || (D % 128) || ld_x < D) return VIT_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return VIT_ERR_SHAPE;
  if (M == 0) return VIT_OK;
  if (!x || !gamma || !beta || !codes || !scales) return VIT_ERR_NULL;
  if (!al16(x) || !al16(gamma) || !al16(beta) || !al16(codes) || !al16(scales) ||
      (prequant_debug && !al16(prequant_debug)) || (ld_x & 7))
    return VIT_ERR_ALIGN;
  const size_t xb = ((size_t)(M - 1) * ld_x + D) * 2, cb = (size_t)M * D, sb = (size_t)M * (D / 128) * 4;
  const size_t pb = prequant_debug ? (size_t)M * D * 4 : 0;
  if (overlap(x, xb, codes, cb) || overlap(x, xb, scales, sb) || overlap(codes, cb, scales, sb) ||
      overlap(prequant_debug, pb, x, xb) || overlap(prequant_debug, pb, codes, cb) ||
      overlap(prequant_debug, pb, scales, sb))
    return VIT_ERR_ALIAS;
  return hip_status(vit::launch_layernorm_quant(x, ld_x, gamma, beta, eps, M, D, codes, scales, prequant_debug,
                                                static_cast<hipStream_t>(stream)));
}

int vit_layernorm(const uint16_t* x, int64_t ld_x, const uint16_t* gamma, const uint16_t* beta, float eps, int M,
                  int D, uint16_t* out, int64_t ld_out, vit_stream_t stream) {
  if (M < 0 || M > kMaxTokens * 4 || D < 128 || D > 8192 || (D % 128) || ld_x < D || ld_out < D)
    return VIT_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return VIT_ERR_SHAPE;
  if (M == 0) return VIT_OK;
  if (!x || !gamma || !beta || !out) return VIT_ERR_NULL;
  if (!al16(x) || !al16(gamma) || !al16(beta) || !al16(out) || (ld_x & 7) || (ld_out & 7)) return VIT_ERR_ALIGN;
  const size_t xb = ((size_t)(M - 1) * ld_x + D) * 2, ob = ((size_t)(M - 1) * ld_out + D) * 2;
  if (overlap(x, xb, out, ob)) return VIT_ERR_ALIAS;
  return hip_status(vit::launch_layernorm_bf16(x, ld_x, gamma, beta, eps, M, D, out, ld_out,
                                               static_cast<hipStream_t>(stream)));
}

int vit_fp8_block128_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w, const float* w_scales,
                          int M, int N, int K, const uint16_t* bias, const uint16_t* residual, int epilogue,
                          uint16_t* out, uint8_t* out_codes, float* out_scales, float* prequant_debug,
                          vit_stream_t stream) {
  if (M < 0 || N < 1 || K < 1 || M > kMaxTokens * 4 || N > kMaxDim || K > kMaxDim) return VIT_ERR_SHAPE;
  if (epilogue < VIT_EPI_BIAS || epilogue > VIT_EPI_BIAS_GELU_FP8) return VIT_ERR_UNSUPPORTED;
  if (M == 0) return VIT_OK;
  if (!a || !a_scales || !w || !w_scales) return VIT_ERR_NULL;
  if ((epilogue == VIT_EPI_BIAS || epilogue == VIT_EPI_BIAS_RESIDUAL) && !out) return VIT_ERR_NULL;
  if (epilogue == VIT_EPI_BIAS_RESIDUAL && !residual) return VIT_ERR_NULL;
  if (epilogue == VIT_EPI_BIAS_GELU_FP8 && (!out_codes || !out_scales)) return VIT_ERR_NULL;
  const void* all[] = {a, a_scales, w, w_scales, bias, residual, out, out_codes, out_scales, prequant_debug};
  for (const void* p : all)
    if (p && !al16(p)) return VIT_ERR_ALIGN;
  // operand offsets are 32-bit only inside a 128-row tile (< 128 * Kp)
  const int Kp = ceil128(K), Np = ceil128(N);
  const size_t ab = (size_t)M * Kp, asb = (size_t)M * (Kp / 128) * 4, wb = (size_t)Np * Kp,
               wsb = (size_t)(Np / 128) * (Kp / 128) * 4, bb = bias ? (size_t)N * 2 : 0;
  const size_t rb = (size_t)M * N * 2;
  const void* ins[] = {a, a_scales, w, w_scales, bias};
  const size_t inb[] = {ab, asb, wb, wsb, bb};
  if (epilogue != VIT_EPI_BIAS_GELU_FP8) {
    for (int i = 0; i < 5; ++i)
      if (overlap(out, rb, ins[i], inb[i])) return VIT_ERR_ALIAS;
    if (epilogue == VIT_EPI_BIAS_RESIDUAL && residual != out && overlap(out, rb, residual, rb))
      return VIT_ERR_ALIAS;
  } else {
    const size_t cb = (size_t)M * Np, sb = (size_t)M * (Np / 128) * 4, pb = prequant_debug ? (size_t)M * Np * 4 : 0;
    for (int i = 0; i < 5; ++i)
      if (overlap(out_codes, cb, ins[i], inb[i]) || overlap(out_scales, sb, ins[i], inb[i]) ||
          overlap(prequant_debug, pb, ins[i], inb[i]))
        return VIT_ERR_ALIAS;
    if (overlap(out_codes, cb, out_scales, sb) || overlap(out_codes, cb, prequant_debug, pb) ||
        overlap(out_scales, sb, prequant_debug, pb))
      return VIT_ERR_ALIAS;
  }
  if ((int64_t)(Np / 128) * ((M + 127) / 128) >= (int64_t)1 << 31) return VIT_ERR_SHAPE;
  return hip_status(vit::launch_fp8_gemm(a, a_scales, w, w_scales, M, N, K, bias, residual, epilogue, out,
                                         out_codes, out_scales, prequant_debug, static_cast<hipStream_t>(stream)));
}

int vit_bf16_gemm(const void* a, int a_is_f32, const uint16_t* w, int M, int N, int K, const uint16_t* bias,
                  const uint16_t* add, int epilogue, uint16_t* out, int64_t ld_out, vit_stream_t stream) {
  if (M < 0 || N < 1 || K < 8 || (K % 8) || M > kMaxTokens * 4 || N > kMaxDim || K > kMaxDim || ld_out < N)
    return VIT_ERR_SHAPE;
  if (epilogue < VIT_BEPI_BIAS || epilogue > VIT_BEPI_BIAS_ADD) return VIT_ERR_UNSUPPORTED;
  if (M == 0) return VIT_OK;
  if (!a || !w || !out) return VIT_ERR_NULL;
  const void* all[] = {a, w, bias, add, out};
  for (const void* p : all)
    if (p && !al16(p)) return VIT_ERR_ALIGN;
  const size_t ob = ((size_t)(M - 1) * ld_out + N) * 2;
  if (overlap(out, ob, a, (size_t)M * K * (a_is_f32 ? 4 : 2)) || overlap(out, ob, w, (size_t)N * K * 2) ||
      overlap(out, ob, bias, bias ? (size_t)N * 2 : 0) ||
      overlap(out, ob, add, (add && epilogue == VIT_BEPI_BIAS_ADD) ? (size_t)M * N * 2 : 0))
    return VIT_ERR_ALIAS;
  return hip_status(vit::launch_bf16_gemm(a, a_is_f32 != 0, w, M, N, K, bias,
                                          epilogue == VIT_BEPI_BIAS_ADD ? add : nullptr, epilogue, out, ld_out,
                                          static_cast<hipStream_t>(stream)));
}

int vit_rope2d(uint16_t* q, uint16_t* k, int64_t ld, const int32_t* pos_rc, int T, int num_heads, int head_dim,
               float theta, vit_stream_t stream) {
  if (T < 0 || T > kMaxTokens || num_heads < 1 || num_heads > 256) return VIT_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 72 && head_dim != 80 && head_dim != 128) return VIT_ERR_UNSUPPORTED;
  const int64_t width = (int64_t)num_heads * head_dim;
  if (ld < width) return VIT_ERR_SHAPE;
  if (!(theta > 0.0f) || !std::isfinite(theta)) return VIT_ERR_SHAPE;
  if (T == 0) return VIT_OK;
  if (!q || !k || !pos_rc) return VIT_ERR_NULL;
  if (!al16(q) || !al16(k) || !al16(pos_rc) || (ld & 3)) return VIT_ERR_ALIGN;
  // q and k rows must be disjoint: either whole ranges apart, or interleaved
  // inside one row of stride ld.
  const int64_t d = (reinterpret_cast<intptr_t>(k) - reinterpret_cast<intptr_t>(q)) / 2;
  const size_t span = ((size_t)(T - 1) * ld + width) * 2;
  const bool apart = !overlap(q, span, k, span);
  const bool interleaved = (d >= width && d + width <= ld) || (-d >= width && -d + width <= ld);
  if (!apart && !interleaved) return VIT_ERR_ALIAS;
  if (overlap(pos_rc, (size_t)T * 8, q, span) || overlap(pos_rc, (size_t)T * 8, k, span)) return VIT_ERR_ALIAS;
  return hip_status(vit::launch_rope2d(q, k, ld, pos_rc, T, num_heads, head_dim, theta,
                                       static_cast<hipStream_t>(stream)));
}

size_t vit_attention_workspace_size(void) { return vit::attention_partial_bytes(); }

}  // extern "C"

namespace {
// Validation shared by vit_attention and vit_attention_noalloc (everything
// but the workspace).  VIT_OK with *nothing = true: nothing to enqueue.
int check_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_qkv, const uint16_t* o,
                    int64_t ld_o, const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                    int total_tokens, int num_heads, int head_dim, float softmax_scale, bool* nothing) {
  *nothing = true;
  if (num_seqs < 0 || num_seqs > (1 << 20) || total_tokens < 0 || total_tokens > kMaxTokens || num_heads < 1 ||
      num_heads > 256)
    return VIT_ERR_SHAPE;
  if (head_dim != VIT_HEAD_DIM) return VIT_ERR_UNSUPPORTED;
  const int64_t width = (int64_t)num_heads * head_dim;
  if (ld_qkv < width || ld_o < width || ld_qkv > (1 << 24) || ld_o > (1 << 24)) return VIT_ERR_SHAPE;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return VIT_ERR_SHAPE;
  if (!cu_seqlens_host) return VIT_ERR_NULL;
  if (num_seqs == 0) return total_tokens == 0 ? VIT_OK : VIT_ERR_SEQLENS;
  if (!valid_cu(cu_seqlens_host, num_seqs, total_tokens)) return VIT_ERR_SEQLENS;
  if (total_tokens == 0) return VIT_OK;
  if (!q || !k || !v || !o || !cu_seqlens_dev) return VIT_ERR_NULL;
  if (!al16(q) || !al16(k) || !al16(v) || !al16(o) || !al16(cu_seqlens_dev) || (ld_qkv & 7) || (ld_o & 7))
    return VIT_ERR_ALIGN;
  const size_t ib = ((size_t)(total_tokens - 1) * ld_qkv + width) * 2;
  const size_t ob = ((size_t)(total_tokens - 1) * ld_o + width) * 2;
  if (overlap(o, ob, q, ib) || overlap(o, ob, k, ib) || overlap(o, ob, v, ib)) return VIT_ERR_ALIAS;
  *nothing = false;
  return VIT_OK;
}
}  // namespace

extern "C" {

int vit_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_qkv, uint16_t* o,
                  int64_t ld_o, const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                  int total_tokens, int num_heads, int head_dim, float softmax_scale, void* workspace,
                  size_t workspace_bytes, vit_stream_t stream) {
  bool nothing = true;
  const int st = check_attention(q, k, v, ld_qkv, o, ld_o, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                 total_tokens, num_heads, head_dim, softmax_scale, &nothing);
  if (st != VIT_OK || nothing) return st;
  const int64_t width = (int64_t)num_heads * head_dim;
  const size_t ib = ((size_t)(total_tokens - 1) * ld_qkv + width) * 2;
  const size_t ob = ((size_t)(total_tokens - 1) * ld_o + width) * 2;
  const size_t wb = vit::attention_partial_bytes();
  if (!workspace || workspace_bytes < wb) return VIT_ERR_WORKSPACE;
  if (!al16(workspace)) return VIT_ERR_ALIGN;
  if (overlap(workspace, wb, q, ib) || overlap(workspace, wb, k, ib) || overlap(workspace, wb, v, ib) ||
      overlap(workspace, wb, o, ob))
    return VIT_ERR_ALIAS;
  vit::AttnPlan plan;
  vit::plan_attention(cu_seqlens_host, num_seqs, num_heads, &plan);
  return hip_status(launch_attention(q, k, v, ld_qkv, o, ld_o, cu_seqlens_dev, num_seqs, total_tokens, plan,
                                     num_heads, softmax_scale, static_cast<float*>(workspace),
                                     static_cast<hipStream_t>(stream)));
}

size_t vit_attention_noalloc_scratch_size(void) { return vit::attention_scratch_bytes(); }

int vit_attention_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_qkv, uint16_t* o,
                          int64_t ld_o, const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                          int num_seqs, int total_tokens, int num_heads, int head_dim, float softmax_scale,
                          vit_stream_t stream) {
  bool nothing = true;
  const int st = check_attention(q, k, v, ld_qkv, o, ld_o, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                 total_tokens, num_heads, head_dim, softmax_scale, &nothing);
  if (st != VIT_OK || nothing) return st;
  // the partials need at most attention_partial_bytes(), whatever the input
  if (vit::attention_partial_bytes() > vit::attention_scratch_bytes()) return VIT_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* scratch = nullptr;
  if (vit::attention_scratch(s, &scratch) != hipSuccess || !scratch) return VIT_ERR_HIP;
  vit::AttnPlan plan;
  vit::plan_attention(cu_seqlens_host, num_seqs, num_heads, &plan);
  return hip_status(launch_attention(q, k, v, ld_qkv, o, ld_o, cu_seqlens_dev, num_seqs, total_tokens, plan,
                                     num_heads, softmax_scale, scratch, s));
}

int vit_merge2x2_layernorm(const uint16_t* x, int D, const int32_t* grid_hw_dev, const int32_t* cu_seqlens_dev,
                           const int32_t* grid_hw_host, int num_images, int T, const uint16_t* gamma,
                           const uint16_t* beta, float eps, uint16_t* out, vit_stream_t stream) {
  if (D < 8 || (D % 8) || 4 * D > 8192 || T < 0 || T > kMaxTokens || num_images < 0 || num_images > (1 << 20))
    return VIT_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return VIT_ERR_SHAPE;
  if (num_images > 0 && !grid_hw_host) return VIT_ERR_NULL;
  if (num_images == 0) return T == 0 ? VIT_OK : VIT_ERR_SEQLENS;
  if (!valid_grids(grid_hw_host, num_images, T)) return VIT_ERR_SEQLENS;
  if (!x || !grid_hw_dev || !cu_seqlens_dev || !gamma || !beta || !out) return VIT_ERR_NULL;
  if (!al16(x) || !al16(grid_hw_dev) || !al16(cu_seqlens_dev) || !al16(gamma) || !al16(beta) || !al16(out))
    return VIT_ERR_ALIGN;
  const size_t ob = (size_t)T * D * 2;
  if (overlap(out, ob, x, ob) || overlap(out, ob, grid_hw_dev, (size_t)num_images * 8) ||
      overlap(out, ob, cu_seqlens_dev, (size_t)(num_images + 1) * 4))
    return VIT_ERR_ALIAS;
  return hip_status(vit::launch_merge_layernorm(x, D, grid_hw_dev, cu_seqlens_dev, num_images, T, gamma, beta, eps,
                                                out, static_cast<hipStream_t>(stream)));
}

size_t vit_block_workspace_size(int T) {
  if (T < 0 || T > kMaxTokens) return 0;
  return block_ws_layout(nullptr, T).bytes;
}

int vit_block_forward(const vit_block_weights* w, uint16_t* x_inout, int T, const int32_t* pos_rc,
                      const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs, void* workspace,
                      size_t workspace_bytes, vit_stream_t stream) {
  if (T < 0 || T > kMaxTokens || num_seqs < 0 || num_seqs > (1 << 20)) return VIT_ERR_SHAPE;
  int st = check_block_weights(w);
  if (st != VIT_OK) return st;
  if (!cu_seqlens_host) return VIT_ERR_NULL;
  if (num_seqs == 0) return T == 0 ? VIT_OK : VIT_ERR_SEQLENS;
  if (!valid_cu(cu_seqlens_host, num_seqs, T)) return VIT_ERR_SEQLENS;
  if (T == 0) return VIT_OK;
  if (!x_inout || !pos_rc || !cu_seqlens_dev || !workspace) return VIT_ERR_NULL;
  if (!al16(x_inout) || !al16(pos_rc) || !al16(cu_seqlens_dev) || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return VIT_ERR_ALIGN;
  const BlockWs ws = block_ws_layout(workspace, T);
  if (workspace_bytes < ws.bytes) return VIT_ERR_WORKSPACE;
  if (overlap(workspace, ws.bytes, x_inout, (size_t)T * VIT_HIDDEN * 2) ||
      overlap(workspace, ws.bytes, pos_rc, (size_t)T * 8))
    return VIT_ERR_ALIAS;
  vit::AttnPlan plan;
  vit::plan_attention(cu_seqlens_host, num_seqs, VIT_HEADS, &plan);
  return hip_status(block_forward_impl(w, x_inout, T, pos_rc, cu_seqlens_dev, num_seqs, plan, ws,
                                       static_cast<hipStream_t>(stream)));
}

int vit_smart_resize(int height, int width, int factor, int64_t min_pixels, int64_t max_pixels, int* out_height,
                     int* out_width) {
  if (!out_height || !out_width) return VIT_ERR_NULL;
  constexpr int kMaxSide = 1 << 20;
  if (height < 1 || width < 1 || height > kMaxSide || width > kMaxSide || factor < 1 || factor > kMaxSide)
    return VIT_ERR_SHAPE;
  const double f = factor;
  // nearest multiple, ties to even (the default rounding mode)
  int64_t h = std::max<int64_t>(factor, (int64_t)std::nearbyint(height / f) * factor);
  int64_t w = std::max<int64_t>(factor, (int64_t)std::nearbyint(width / f) * factor);
  const double area = (double)height * (double)width;
  if (max_pixels > 0 && h * w > max_pixels) {
    const double beta = std::sqrt(area / (double)max_pixels);
    h = std::max<int64_t>(factor, (int64_t)std::floor(height / beta / f) * factor);
    w = std::max<int64_t>(factor, (int64_t)std::floor(width / beta / f) * factor);
  } else if (min_pixels > 0 && h * w < min_pixels) {
    const double beta = std::sqrt((double)min_pixels / area);
    h = (int64_t)std::ceil(height * beta / f) * factor;
    w = (int64_t)std::ceil(width * beta / f) * factor;
  }
  if (h > kMaxSide || w > kMaxSide) return VIT_ERR_SHAPE;
  *out_height = (int)h;
  *out_width = (int)w;
  return VIT_OK;
}

int vit_preprocess_frames(const uint8_t* frames, int num_frames, int height, int width, int out_height,
                          int out_width, const float* mean_host, const float* std_host, float* pixels,
                          vit_stream_t stream) {
  constexpr int kMaxSide = 1 << 15;
  if (num_frames < 1 || num_frames > (1 << 16) || height < 1 || width < 1 || height > kMaxSide ||
      width > kMaxSide || out_height < 16 || out_width < 16 || out_height > kMaxSide || out_width > kMaxSide ||
      (out_height % 16) || (out_width % 16))
    return VIT_ERR_SHAPE;
  if (!mean_host || !std_host) return VIT_ERR_NULL;
  float a[3], b[3];
  for (int c = 0; c < 3; ++c) {
    const double m = mean_host[c], sd = std_host[c];
    if (!std::isfinite(m) || !std::isfinite(sd) || !(sd > 0.0)) return VIT_ERR_SHAPE;
    a[c] = (float)(1.0 / (255.0 * sd));
    b[c] = (float)(-m / sd);
  }
  const int64_t rows = (int64_t)((num_frames + 1) / 2) * (out_height / 16) * (out_width / 16);
  if (rows > (int64_t)kMaxTokens) return VIT_ERR_SHAPE;
  if (!frames || !pixels) return VIT_ERR_NULL;
  if (!al16(pixels)) return VIT_ERR_ALIGN;
  const size_t fb = (size_t)num_frames * height * width * 3, pb = (size_t)rows * VIT_PATCH_DIM * 4;
  if (overlap(frames, fb, pixels, pb)) return VIT_ERR_ALIAS;
  return hip_status(vit::launch_preprocess(frames, num_frames, height, width, out_height, out_width, a, b, pixels,
                                           static_cast<hipStream_t>(stream)));
}

int vit_pos_embed_interp(const uint16_t* table, int grid_side, int dim, const int32_t* grid_hw_dev,
                         const int32_t* cu_seqlens_dev, const int32_t* grid_hw_host, int num_images, int T,
                         uint16_t* out, int64_t ld_out, vit_stream_t stream) {
  if (grid_side < 1 || grid_side > 1024 || dim < 8 || (dim % 8) || dim > kMaxDim || T < 0 || T > kMaxTokens ||
      num_images < 0 || num_images > (1 << 20) || ld_out < dim || (ld_out & 7))
    return VIT_ERR_SHAPE;
  if (num_images > 0 && !grid_hw_host) return VIT_ERR_NULL;
  int64_t total = 0;
  for (int j = 0; j < num_images; ++j) {
    const int h = grid_hw_host[2 * j], w = grid_hw_host[2 * j + 1];
    if (h < 1 || w < 1 || h > kMaxTokens || w > kMaxTokens) return VIT_ERR_SEQLENS;
    total += (int64_t)h * w;
    if (total > T) return VIT_ERR_SEQLENS;
  }
  if (total != T) return VIT_ERR_SEQLENS;
  if (T == 0) return VIT_OK;
  if (!table || !grid_hw_dev || !cu_seqlens_dev || !out) return VIT_ERR_NULL;
  if (!al16(table) || !al16(grid_hw_dev) || !al16(cu_seqlens_dev) || !al16(out)) return VIT_ERR_ALIGN;
  const size_t tb = (size_t)grid_side * grid_side * dim * 2;
  const size_t ob = ((size_t)(T - 1) * ld_out + dim) * 2;
  if (overlap(out, ob, table, tb) || overlap(out, ob, grid_hw_dev, (size_t)num_images * 8) ||
      overlap(out, ob, cu_seqlens_dev, (size_t)(num_images + 1) * 4))
    return VIT_ERR_ALIAS;
  return hip_status(vit::launch_pos_interp(table, grid_side, dim, grid_hw_dev, cu_seqlens_dev, num_images, T, out,
                                           ld_out, static_cast<hipStream_t>(stream)));
}

size_t vit_encoder_workspace_size(int T, int num_images) {
  if (T < 0 || T > kMaxTokens || num_images < 0 || num_images > (1 << 20)) return 0;
  return encoder_ws_layout(nullptr, T, num_images).bytes;
}

int vit_encoder_forward(const vit_encoder_weights* w, const float* pixels, const uint16_t* pos_embed,
                        const int32_t* grid_hw_dev, const int32_t* grid_hw_host, int num_images, int T,
                        uint16_t* out, uint16_t* last_hidden, void* workspace, size_t workspace_bytes,
                        vit_stream_t stream) {
  if (T < 0 || T > kMaxTokens || num_images < 0 || num_images > (1 << 20)) return VIT_ERR_SHAPE;
  if (!w) return VIT_ERR_NULL;
  if (!w->patch_w || !w->patch_b) return VIT_ERR_NULL;
  if (!al16(w->patch_w) || !al16(w->patch_b)) return VIT_ERR_ALIGN;
  for (int b = 0; b < VIT_DEPTH; ++b) {
    const int st = check_block_weights(&w->blocks[b]);
    if (st != VIT_OK) return st;
  }
  for (int m = 0; m < VIT_NUM_TAPS; ++m) {
    const int st = check_merger_weights(&w->mergers[m]);
    if (st != VIT_OK) return st;
  }
  if (w->pos_table && (pos_embed || w->pos_grid_side < 1 || w->pos_grid_side > 1024)) return VIT_ERR_SHAPE;
  if (w->pos_table && !al16(w->pos_table)) return VIT_ERR_ALIGN;
  if (num_images > 0 && !grid_hw_host) return VIT_ERR_NULL;
  if (num_images == 0) return T == 0 ? VIT_OK : VIT_ERR_SEQLENS;
  if (!valid_grids(grid_hw_host, num_images, T)) return VIT_ERR_SEQLENS;
  if (!pixels || !grid_hw_dev || !out || !workspace) return VIT_ERR_NULL;
  if (!al16(pixels) || !al16(grid_hw_dev) || !al16(out) || (pos_embed && !al16(pos_embed)) ||
      (last_hidden && !al16(last_hidden)) || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return VIT_ERR_ALIGN;
  const EncoderWs ws = encoder_ws_layout(workspace, T, num_images);
  if (workspace_bytes < ws.bytes) return VIT_ERR_WORKSPACE;
  const size_t outb = (size_t)VIT_NUM_TAPS * (T / 4) * VIT_OUT_HIDDEN * 2, xb = (size_t)T * VIT_HIDDEN * 2;
  if (overlap(out, outb, workspace, ws.bytes) || overlap(out, outb, pixels, (size_t)T * VIT_PATCH_DIM * 4) ||
      overlap(last_hidden, last_hidden ? xb : 0, workspace, ws.bytes) ||
      overlap(last_hidden, last_hidden ? xb : 0, out, outb) ||
      overlap(last_hidden, last_hidden ? xb : 0, pixels, (size_t)T * VIT_PATCH_DIM * 4) ||
      overlap(out, outb, pos_embed, pos_embed ? xb : 0) ||
      overlap(last_hidden, last_hidden ? xb : 0, pos_embed, pos_embed ? xb : 0))
    return VIT_ERR_ALIAS;

  // attention plan of the packing (the same for every block), from the host
  // copy of the grids
  std::vector<int32_t> cu_host(num_images + 1, 0);
  for (int j = 0; j < num_images; ++j) cu_host[j + 1] = cu_host[j] + grid_hw_host[2 * j] * grid_hw_host[2 * j + 1];
  vit::AttnPlan plan;
  vit::plan_attention(cu_host.data(), num_images, VIT_HEADS, &plan);

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* x = last_hidden ? last_hidden : ws.x;
  hipError_t e;
  if ((e = vit::launch_geometry(grid_hw_dev, num_images, T, ws.cu, ws.pos, s)) != hipSuccess) return VIT_ERR_HIP;
  // the learned table resampled to the grids goes to the qkv region, which
  // the blocks only use later
  const uint16_t* pos_add = pos_embed;
  if (w->pos_table) {
    if ((e = vit::launch_pos_interp(w->pos_table, w->pos_grid_side, VIT_HIDDEN, grid_hw_dev, ws.cu, num_images, T,
                                    ws.blk.qkv, VIT_HIDDEN, s)) != hipSuccess)
      return VIT_ERR_HIP;
    pos_add = ws.blk.qkv;
  }
  if ((e = vit::launch_bf16_gemm(pixels, true, w->patch_w, T, VIT_HIDDEN, VIT_PATCH_DIM, w->patch_b, pos_add,
                                 pos_add ? VIT_BEPI_BIAS_ADD : VIT_BEPI_BIAS, x, VIT_HIDDEN, s)) != hipSuccess)
    return VIT_ERR_HIP;
  static const int taps[VIT_NUM_TAPS] = {8, 16, 24, 27};
  int ti = 0;
  const size_t tap_elems = (size_t)(T / 4) * VIT_OUT_HIDDEN;
  for (int b = 0; b < VIT_DEPTH; ++b) {
    if ((e = block_forward_impl(&w->blocks[b], x, T, ws.pos, ws.cu, num_images, plan, ws.blk, s)) != hipSuccess)
      return VIT_ERR_HIP;
    if (ti < VIT_NUM_TAPS && b + 1 == taps[ti]) {
      if ((e = merger_forward_impl(&w->mergers[ti], x, grid_hw_dev, ws.cu, num_images, T, out + ti * tap_elems, ws,
                                   s)) != hipSuccess)
        return VIT_ERR_HIP;
      ++ti;
    }
  }
  return VIT_OK;
}

}  // extern "C"
