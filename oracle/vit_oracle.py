"""fp64 numpy oracle of the ViT vision-tower forward (test infrastructure only).

See ``oracle/__init__.py`` for the sources.  Conventions used throughout:

* all arrays are numpy float64 unless stated; a "bf16 value" or "fp32 value"
  is a float64 that is exactly representable in that format;
* a "storage point" is a place where the GPU path keeps a tensor in bf16 in
  memory; ``mode="storage"`` rounds there, ``mode="pure"`` does not (FP8
  quantisation points are rounded in both modes, they are part of the method);
* activations are [tokens, features] row-major, weights are [out, in]
  (the ``C = A @ W^T + b`` convention of the spark_model page, kernel handle
  ``vision_gemm_bias`` in struct VisionEncoder).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# Model dimensions.  FlashRT page section 3 (ViT tower: 27 blocks, hidden
# 1152, 16 heads x head_dim 72, out_hidden 4096); spark_model page struct
# VisionEncoder (intermediate_size 4304, spatial_merge_size 2, PATCH_DIM
# 1536 = 3 x 2 x 16 x 16); FlashRT section 3 (4304 zero-padded to 4352).
# --------------------------------------------------------------------------
HIDDEN = 1152
HEADS = 16
HEAD_DIM = 72
MLP = 4304
MLP_PADDED = 4352
PATCH_DIM = 1536
DEPTH = 27
OUT_HIDDEN = 4096
MERGE = 2
MERGED_DIM = HIDDEN * MERGE * MERGE  # 4608
# DeepStack taps: after the 8th, 16th and 24th block (1-indexed; spark_model
# page, field deepstack_indexes) plus the final block 27 (module doc there).
TAPS = (8, 16, 24, 27)
LN_EPS = 1e-6
ROPE_THETA = 10000.0

E4M3_MAX = 448.0
BLOCK = 128
# amax below this gives a zero scale: 448/amax would overflow fp32.
TINY_AMAX = 2.0 ** -116


# ==========================================================================
# Number formats
# ==========================================================================

def round_to_float_format(x, frac_bits: int, emin: int, max_finite: float,
                          saturate: bool) -> np.ndarray:
    """Round float64 values to a binary floating-point format, ties to even.

    The format has ``frac_bits`` stored fraction bits, minimum normal exponent
    ``emin`` (subnormals below it, gradual underflow) and largest finite value
    ``max_finite``.  A result above ``max_finite`` becomes ``max_finite`` when
    ``saturate`` else infinity (IEEE overflow).  Sign (including -0) is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)          # ax = m * 2**e with m in [0.5, 1)
    e = np.maximum(e - 1, emin)  # exponent of the binade, floored at emin
    quantum = np.ldexp(1.0, e - frac_bits)
    r = np.rint(ax / quantum) * quantum  # exact scaling; rint = ties to even
    over = r > max_finite
    if saturate:
        r = np.where(over, max_finite, r)
    else:
        r = np.where(over, np.inf, r)
    r = np.where(np.isnan(x), np.nan, r)
    return np.copysign(r, x)


def bf16(x) -> np.ndarray:
    """Round to bfloat16 (8 exponent bits, 7 fraction bits), ties to even."""
    return round_to_float_format(x, 7, -126, float.fromhex("0x1.fep127"), False)


def f32(x) -> np.ndarray:
    """Round to IEEE binary32 (numpy's conversion is round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# --- OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits, no inf,
# --- S.1111.111 is NaN, largest finite 448.  The pages call the format
# --- "FP8 block-128" with scale amax/448 (FlashRT section 1; PR #2106).

def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes, from the closed form."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        f = c & 0x7
        if e == 0xF and f == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (f / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + f / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_decode_table()
_E4M3_POS = _E4M3[:0x7F]  # codes 0x00..0x7E: +0 .. 448, strictly increasing


def e4m3_decode(codes) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(t) -> np.ndarray:
    """Encode finite values to E4M3FN: nearest, ties to even, saturating at
    +-448, zero keeps its sign (-0 -> 0x80)."""
    t = np.asarray(t, dtype=np.float64)
    r = round_to_float_format(np.abs(t), 3, -6, E4M3_MAX, True)
    # code of the grid value r: normal r = (1 + f/8) 2^E -> (E + 7) * 8 + f,
    # subnormal r = f 2^-9 -> f; checked against the decode table below.
    m, e = np.frexp(r)
    normal = (e - 1 + 7) * 8 + np.rint((2.0 * m - 1.0) * 8.0)
    sub = np.rint(r * 512.0)
    mag = np.where(r >= 2.0 ** -6, normal, sub).astype(np.uint8)
    assert np.all(_E4M3_POS[mag] == r)
    sign = np.signbit(t).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


# ==========================================================================
# Block-128 FP8 quantiser (FlashRT section 1 "FP8 block-128 ViT GEMMs",
# section 3 "per-token / per-128-K-block FP8 activation quant"; scale
# amax/448 as in PR #2106 Implementation).  Activations use 1 x 128 blocks
# (per token, per 128 columns), weights 128 x 128 blocks.
# ==========================================================================

def block_scale(amax: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(scale, inverse) for block maxima given as fp32 values.

    scale = fp32(amax / 448), inverse = fp32(448 / amax); both 0 for an
    all-zero (or vanishing) block.  Rounding the float64 quotient once to
    fp32 equals the correctly rounded fp32 division.
    """
    amax = np.asarray(amax, dtype=np.float64)
    zero = amax < TINY_AMAX
    safe = np.where(zero, 1.0, amax)
    s = np.where(zero, 0.0, f32(safe / E4M3_MAX))
    inv = np.where(zero, 0.0, f32(E4M3_MAX / safe))
    return s, inv


def ceil_to(n: int, m: int) -> int:
    return (n + m - 1) // m * m


def quantize_block128(x, block_rows: int) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise a [R, C] tensor of fp32 values in blocks of block_rows x 128.

    Returns codes [Rp, Cp] uint8 and scales [ceil(R/block_rows), Cp/128]
    (fp32 values in float64), Cp = ceil128(C), Rp = R for block_rows == 1
    else ceil128(R).  Ragged last blocks hold only the real elements; the
    padding codes are +0.  code = encode(fp32(x * inverse)).
    """
    x = f32(x)
    assert x.ndim == 2 and block_rows in (1, BLOCK)
    R, C = x.shape
    Cp = ceil_to(max(C, 1), BLOCK)
    Rp = R if block_rows == 1 else ceil_to(max(R, 1), BLOCK)
    xp = np.zeros((Rp, Cp), dtype=np.float64)
    xp[:R, :C] = x
    nbr = (R + block_rows - 1) // block_rows
    nbc = Cp // BLOCK
    blocks = xp[:nbr * block_rows].reshape(nbr, block_rows, nbc, BLOCK)
    amax = np.abs(blocks).max(axis=(1, 3))          # [nbr, nbc]
    s, inv = block_scale(amax)
    t = f32(blocks * inv[:, None, :, None])          # exact product, one rounding
    codes = np.zeros((Rp, Cp), dtype=np.uint8)
    codes[:nbr * block_rows] = e4m3_encode(t).reshape(nbr * block_rows, Cp)
    codes[R:] = 0
    return codes, s


def dequantize_block128(codes, scales, block_rows: int) -> np.ndarray:
    """decode(code) * scale of its block, [Rp, Cp]."""
    v = e4m3_decode(codes)
    Rp, Cp = v.shape
    s = np.repeat(np.repeat(scales, block_rows, axis=0)[:Rp], BLOCK, axis=1)
    return v * s[:Rp, :Cp]


# ==========================================================================
# Elementwise / row operations
# ==========================================================================

def layernorm(x, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """Biased-variance LayerNorm over the last axis with affine gamma, beta
    (spark_model page: kernel handle vision_layer_norm, "biased"; FlashRT
    section 3: LayerNorm before qkv and before fc1).  eps = 1e-6."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def gelu_tanh(x) -> np.ndarray:
    """GELU, tanh form (FlashRT section 3 "GELU(tanh)"); the published
    approximation 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def rope_inv_freq(head_dim: int = HEAD_DIM, theta: float = ROPE_THETA) -> np.ndarray:
    """head_dim/4 inverse frequencies (spark_model page, field rope_inv_freq
    "[head_dim / 4]"): f_i = theta^(-2i / (head_dim/2)), i < head_dim/4."""
    half = head_dim // 2
    i = np.arange(head_dim // 4, dtype=np.float64)
    return theta ** (-2.0 * i / half)


def rope2d(x, pos_rc, num_heads: int = HEADS, head_dim: int = HEAD_DIM,
           theta: float = ROPE_THETA) -> np.ndarray:
    """2D rotate_half rotary embedding of Q or K (FlashRT section 3 "2D
    rotate_half RoPE", kernel rope_neox_qk_bf16).

    x: [T, num_heads*head_dim]; pos_rc: [T, 2] integer (row, col) per token.
    Reading: the first head_dim/2 dims of each head rotate by the row index,
    the second half by the column index; inside each half, dims i and
    i + head_dim/4 form a rotate_half pair turned by angle p * f_i:
    (u, v) -> (u cos - v sin, v cos + u sin).
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    y = x.reshape(T, num_heads, head_dim).copy()
    f = rope_inv_freq(head_dim, theta)
    q4 = head_dim // 4
    for axis in (0, 1):
        ang = np.asarray(pos_rc, dtype=np.float64)[:, axis:axis + 1] * f[None, :]  # [T, q4]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        base = axis * (head_dim // 2)
        u = y[:, :, base:base + q4].copy()
        v = y[:, :, base + q4:base + 2 * q4].copy()
        y[:, :, base:base + q4] = u * c - v * s
        y[:, :, base + q4:base + 2 * q4] = v * c + u * s
    return y.reshape(T, num_heads * head_dim)


def attention(q, k, v, cu_seqlens: Sequence[int], num_heads: int = HEADS,
              head_dim: int = HEAD_DIM, scale: Optional[float] = None) -> np.ndarray:
    """Full bidirectional attention per image window (FlashRT section 3
    "FA2 (full, bidirectional)"; section 5: each image is its own cu_seqlens
    attention window).  O_h = softmax(Q_h K_h^T * scale) V_h, scale 1/sqrt(72).

    q, k, v: [T, num_heads*head_dim]; returns [T, num_heads*head_dim].
    """
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T = q.shape[0]
    out = np.zeros((T, num_heads * head_dim), dtype=np.float64)
    for j in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[j]), int(cu_seqlens[j + 1])
        if b == a:
            continue
        for h in range(num_heads):
            sl = slice(h * head_dim, (h + 1) * head_dim)
            s = (q[a:b, sl] @ k[a:b, sl].T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[a:b, sl] = p @ v[a:b, sl]
    return out


# ==========================================================================
# GEMMs
# ==========================================================================

def fp8_block128_gemm(a_codes, a_scales, w_codes, w_scales) -> np.ndarray:
    """Block-scaled FP8 W8A8 product (FlashRT section 1 "FP8 block-128 ViT
    GEMMs").  C[m, n] = sum over K blocks kb of
        sA[m, kb] * sW[n // 128, kb] * sum_{k in kb} dec(a[m, k]) dec(w[n, k]).
    a_codes [M, Kp], a_scales [M, Kp/128], w_codes [Np, Kp],
    w_scales [Np/128, Kp/128].  Returns float64 [M, Np].  The inner sums of
    128 E4M3 products are exact in float64.
    """
    A = e4m3_decode(a_codes)
    W = e4m3_decode(w_codes)
    M, Kp = A.shape
    Np = W.shape[0]
    assert W.shape[1] == Kp and Kp % BLOCK == 0 and Np % BLOCK == 0
    C = np.zeros((M, Np), dtype=np.float64)
    sw_cols = np.repeat(np.asarray(w_scales, dtype=np.float64), BLOCK, axis=0)  # [Np, Kb]
    for kb in range(Kp // BLOCK):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        part = A[:, ks] @ W[:, ks].T
        C += np.asarray(a_scales, dtype=np.float64)[:, kb:kb + 1] * sw_cols[None, :, kb] * part
    return C


def bf16_gemm(a, w, bias=None) -> np.ndarray:
    """Plain product a @ w^T (+ bias) of bf16-valued operands, float64 result
    (patch embed and mergers stay bf16: FlashRT section 4)."""
    c = np.asarray(a, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    if bias is not None:
        c = c + np.asarray(bias, dtype=np.float64)[None, :]
    return c


# FP8 GEMM epilogues (bias fused into the GEMM: FlashRT section 1, "ViT bias
# adds fused into adjacent kernels"; GELU + quant fused: section 3).
EPI_BIAS = 0
EPI_BIAS_RESIDUAL = 1
EPI_BIAS_GELU_FP8 = 2


def fp8_gemm_epilogue(C, N: int, epilogue: int, bias=None, residual=None,
                      storage: bool = True):
    """Apply an epilogue to the float64 product C [M, Np] whose first N
    columns are real.

    EPI_BIAS:          bf16(C + b)                -> [M, N]
    EPI_BIAS_RESIDUAL: bf16(C + b + residual)     -> [M, N]
    EPI_BIAS_GELU_FP8: Q_1x128(fp32(gelu(C + b))) -> (codes [M, Np],
                       scales [M, Np/128], prequant [M, Np]); columns >= N
                       are zero (a zero-padded weight row and bias).
    ``storage=False`` skips the bf16 rounding of the first two.
    """
    M, Np = C.shape
    b = np.zeros(Np) if bias is None else np.pad(np.asarray(bias, np.float64)[:N], (0, Np - N))
    if epilogue == EPI_BIAS:
        y = C[:, :N] + b[None, :N]
        return bf16(y) if storage else y
    if epilogue == EPI_BIAS_RESIDUAL:
        y = C[:, :N] + b[None, :N] + np.asarray(residual, np.float64)
        return bf16(y) if storage else y
    if epilogue == EPI_BIAS_GELU_FP8:
        pre = gelu_tanh(C + b[None, :])
        pre[:, N:] = 0.0
        pre32 = f32(pre)
        codes, scales = quantize_block128(pre32, 1)
        return codes, scales, pre
    raise ValueError(epilogue)


# ==========================================================================
# Weights
# ==========================================================================

@dataclass
class Fp8Weight:
    codes: np.ndarray   # [Np, Kp] uint8
    scales: np.ndarray  # [Np/128, Kp/128]


@dataclass
class BlockWeights:
    """One ViT block (spark_model page, struct ViTBlock: norm1 w/b, qkv w/b,
    proj w/b, norm2 w/b, fc1 w/b, fc2 w/b).  Linear weights as bf16 values
    [out, in]; their FP8 forms are derived by quantize_block128(., 128)."""
    ln1_g: np.ndarray
    ln1_b: np.ndarray
    qkv_w: np.ndarray   # [3456, 1152]
    qkv_b: np.ndarray
    proj_w: np.ndarray  # [1152, 1152]
    proj_b: np.ndarray
    ln2_g: np.ndarray
    ln2_b: np.ndarray
    fc1_w: np.ndarray   # [4304, 1152]
    fc1_b: np.ndarray
    fc2_w: np.ndarray   # [1152, 4304]
    fc2_b: np.ndarray
    _q: Dict[str, Fp8Weight] = field(default_factory=dict, repr=False)

    def fp8(self, name: str) -> Fp8Weight:
        if name not in self._q:
            codes, scales = quantize_block128(getattr(self, name + "_w"), BLOCK)
            self._q[name] = Fp8Weight(codes, scales)
        return self._q[name]


@dataclass
class MergerWeights:
    """One 2x2 merger MLP (spark_model page, struct MergerLayer: norm w/b,
    fc1 w/b, fc2 w/b), bf16 (FlashRT section 4: mergers stay bf16); the FP8
    variant ("merger FP8", FlashRT section 1 prefill history) uses
    quantize_block128(., 128) of the same bf16 weights."""
    ln_g: np.ndarray    # [4608]
    ln_b: np.ndarray
    fc1_w: np.ndarray   # [4608, 4608]
    fc1_b: np.ndarray
    fc2_w: np.ndarray   # [4096, 4608]
    fc2_b: np.ndarray
    _q: Dict[str, Fp8Weight] = field(default_factory=dict, repr=False)

    def fp8(self, name: str) -> Fp8Weight:
        if name not in self._q:
            codes, scales = quantize_block128(getattr(self, name + "_w"), BLOCK)
            self._q[name] = Fp8Weight(codes, scales)
        return self._q[name]


@dataclass
class EncoderWeights:
    patch_w: np.ndarray  # [1152, 1536] bf16 (spark_model page: patch_embed_w)
    patch_b: np.ndarray  # [1152]
    blocks: List[BlockWeights]
    mergers: List[MergerWeights]  # DeepStack 8, 16, 24, then the final merger


# ==========================================================================
# Geometry
# ==========================================================================

def cu_seqlens_from_grids(grids: Sequence[Tuple[int, int]]) -> np.ndarray:
    """Packed token offsets of images with patch grids (h, w): each image is
    its own attention window (FlashRT section 5)."""
    cu = [0]
    for h, w in grids:
        cu.append(cu[-1] + h * w)
    return np.asarray(cu, dtype=np.int64)


def positions_from_grids(grids: Sequence[Tuple[int, int]]) -> np.ndarray:
    """(row, col) of each token, 0-based per image, tokens in row-major
    raster order inside each image."""
    out = []
    for h, w in grids:
        r, c = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
        out.append(np.stack([r.ravel(), c.ravel()], axis=1))
    return np.concatenate(out, axis=0).astype(np.int64) if out else np.zeros((0, 2), np.int64)


def merge2x2(x, grids: Sequence[Tuple[int, int]]) -> np.ndarray:
    """2x2 spatial merge (FlashRT section 3 "2x2 patch merger"; spark_model
    page: spatial_merge_size 2, kernel vision_spatial_merge): for image j
    with grid (h, w) the merged row R*(w/2)+C concatenates the tokens at
    (2R, 2C), (2R, 2C+1), (2R+1, 2C), (2R+1, 2C+1).  [T, D] -> [T/4, 4D]."""
    x = np.asarray(x)
    D = x.shape[1]
    rows = []
    off = 0
    for h, w in grids:
        assert h % 2 == 0 and w % 2 == 0
        img = x[off:off + h * w].reshape(h, w, D)
        for R in range(h // 2):
            for C in range(w // 2):
                rows.append(np.concatenate([img[2 * R, 2 * C], img[2 * R, 2 * C + 1],
                                            img[2 * R + 1, 2 * C], img[2 * R + 1, 2 * C + 1]]))
        off += h * w
    return np.stack(rows, axis=0) if rows else np.zeros((0, 4 * D), x.dtype)


# ==========================================================================
# Block, merger, encoder
# ==========================================================================

def _rb(x, storage):
    return bf16(x) if storage else np.asarray(x, dtype=np.float64)


def block_forward_bf16(x, w: BlockWeights, pos_rc, cu_seqlens, mode: str = "storage",
                       trace: Optional[dict] = None) -> np.ndarray:
    """One pre-norm ViT block with bf16 GEMMs and no FP8 anywhere: the
    precision FlashRT section 4 keeps for the first 3 blocks ("patch embed,
    the mergers and the first 3 blocks stay bf16").  Same chain as
    block_forward; the LayerNorm outputs and the GELU output, which feed
    GEMMs, are stored in bf16 (there is no quantiser to take fp32).
    """
    storage = mode == "storage"
    x = np.asarray(x, dtype=np.float64)
    y1 = _rb(layernorm(x, w.ln1_g, w.ln1_b), storage)
    qkv = _rb(bf16_gemm(y1, w.qkv_w, w.qkv_b), storage)
    q, k, v = qkv[:, :HIDDEN], qkv[:, HIDDEN:2 * HIDDEN], qkv[:, 2 * HIDDEN:]
    q = _rb(rope2d(q, pos_rc), storage)
    k = _rb(rope2d(k, pos_rc), storage)
    o = _rb(attention(q, k, v, cu_seqlens), storage)
    x1 = _rb(bf16_gemm(o, w.proj_w, w.proj_b) + x, storage)
    y2 = _rb(layernorm(x1, w.ln2_g, w.ln2_b), storage)
    h = _rb(gelu_tanh(bf16_gemm(y2, w.fc1_w, w.fc1_b)), storage)
    x2 = _rb(bf16_gemm(h, w.fc2_w, w.fc2_b) + x1, storage)
    if trace is not None:
        trace.update(dict(y1=y1, qkv=qkv, q=q, k=k, o=o, x1=x1, y2=y2, h=h, x2=x2))
    return x2


def block_forward(x, w: BlockWeights, pos_rc, cu_seqlens, mode: str = "storage",
                  trace: Optional[dict] = None) -> np.ndarray:
    """One pre-norm ViT block (FlashRT section 3 "per block: LayerNorm -> qkv
    -> 2D rotate_half RoPE -> FA2 (full, bidirectional) -> proj -> residual ->
    LayerNorm -> fc1 -> GELU(tanh) -> fc2 -> residual"), with FP8 block-128
    W8A8 GEMMs whose activation quant is fused into LayerNorm / GELU
    (section 3, layer_norm_to_fp8_block128_bf16 / gelu_tanh_to_fp8_block128).

    Storage points (mode="storage"): qkv, rotated q/k, attention output and
    the two residual sums are bf16; quantised activations come from fp32.
    """
    storage = mode == "storage"
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    # LN1 -> FP8 (per token, per 128 columns)
    pre1 = f32(layernorm(x, w.ln1_g, w.ln1_b))
    a1, s1 = quantize_block128(pre1, 1)
    qw = w.fp8("qkv")
    qkv = fp8_gemm_epilogue(fp8_block128_gemm(a1, s1, qw.codes, qw.scales),
                            3 * HIDDEN, EPI_BIAS, bias=w.qkv_b, storage=storage)
    q, k, v = qkv[:, :HIDDEN], qkv[:, HIDDEN:2 * HIDDEN], qkv[:, 2 * HIDDEN:]
    q = _rb(rope2d(q, pos_rc), storage)
    k = _rb(rope2d(k, pos_rc), storage)
    o = _rb(attention(q, k, v, cu_seqlens), storage)
    a2, s2 = quantize_block128(f32(o), 1)
    pw = w.fp8("proj")
    x1 = fp8_gemm_epilogue(fp8_block128_gemm(a2, s2, pw.codes, pw.scales),
                           HIDDEN, EPI_BIAS_RESIDUAL, bias=w.proj_b, residual=x, storage=storage)
    pre2 = f32(layernorm(x1, w.ln2_g, w.ln2_b))
    a3, s3 = quantize_block128(pre2, 1)
    f1 = w.fp8("fc1")
    hc, hs, _ = fp8_gemm_epilogue(fp8_block128_gemm(a3, s3, f1.codes, f1.scales),
                                  MLP, EPI_BIAS_GELU_FP8, bias=w.fc1_b)
    f2 = w.fp8("fc2")
    hcp = np.zeros((T, f2.codes.shape[1]), dtype=np.uint8)
    hcp[:, :hc.shape[1]] = hc
    hsp = np.zeros((T, f2.codes.shape[1] // BLOCK))
    hsp[:, :hs.shape[1]] = hs
    x2 = fp8_gemm_epilogue(fp8_block128_gemm(hcp, hsp, f2.codes, f2.scales),
                           HIDDEN, EPI_BIAS_RESIDUAL, bias=w.fc2_b, residual=x1, storage=storage)
    if trace is not None:
        trace.update(dict(pre1=pre1, a1=a1, s1=s1, qkv=qkv, q=q, k=k, o=o, a2=a2, s2=s2,
                          x1=x1, pre2=pre2, a3=a3, s3=s3, h_codes=hc, h_scales=hs, x2=x2))
    return x2


def merger_forward(x, m: MergerWeights, grids, mode: str = "storage", fp8: bool = False) -> np.ndarray:
    """2x2 merge -> LayerNorm(4608) -> fc1 (+b) -> GELU(tanh) -> fc2 (+b),
    bf16 (FlashRT section 3 "2x2 patch merger -> image_embeds (out_hidden
    4096)"; spark_model page struct MergerLayer).  Readings: LayerNorm over
    the concatenated 4608 features for all four mergers, tanh-GELU.

    fp8=True is the "merger FP8" of FlashRT section 1 with the blocks' W8A8
    recipe: the bf16 LayerNorm output is quantised per token and 128
    columns, fc1 + bias + GELU is requantised the same way (from fp32),
    fc2 + bias is stored in bf16; weights quantised in 128 x 128 blocks."""
    storage = mode == "storage"
    y = merge2x2(x, grids)
    y = _rb(layernorm(y, m.ln_g, m.ln_b), storage)
    if not fp8:
        h = _rb(gelu_tanh(bf16_gemm(y, m.fc1_w, m.fc1_b)), storage)
        return _rb(bf16_gemm(h, m.fc2_w, m.fc2_b), storage)
    a, sa = quantize_block128(y, 1)
    f1, f2 = m.fp8("fc1"), m.fp8("fc2")
    hc, hs, _ = fp8_gemm_epilogue(fp8_block128_gemm(a, sa, f1.codes, f1.scales), MERGED_DIM,
                                  EPI_BIAS_GELU_FP8, bias=m.fc1_b)
    return fp8_gemm_epilogue(fp8_block128_gemm(hc, hs, f2.codes, f2.scales), OUT_HIDDEN, EPI_BIAS,
                             bias=m.fc2_b, storage=storage)


def patch_embed(pixels, w: EncoderWeights, pos_embed=None, mode: str = "storage") -> np.ndarray:
    """Patch embedding as a GEMM with K = PATCH_DIM = 3*2*16*16 (spark_model
    page, PATCH_DIM doc), in bf16 (FlashRT section 4); fp32 pixels are
    rounded to bf16 first.  Optional additive position table [T, 1152]."""
    c = bf16_gemm(bf16(pixels), w.patch_w, w.patch_b)
    if pos_embed is not None:
        c = c + np.asarray(pos_embed, dtype=np.float64)
    return _rb(c, mode == "storage")


# Learned position table: num_grid_per_side = 48, i.e. [2304, 1152]
# (spark_model page, struct VisionEncoder fields pos_embed and
# num_grid_per_side).
POS_GRID = 48


def pos_embed_interp(table, grids: Sequence[Tuple[int, int]], grid_side: int = POS_GRID) -> np.ndarray:
    """Per-token position embedding resampled from the learned [G*G, D] table
    (FlashRT section 3, "patch_embed -> +interpolated pos_embed"; spark_model
    page, struct VisionEncoder: a [2304, 1152] bf16 table with
    num_grid_per_side 48, kept on the host as f32 for the per-prompt
    geometry).  Returns [T, D] bf16 values, tokens in raster order per image,
    images packed in order.

    The pages do not state the resampling rule.  Reading taken: bilinear
    interpolation with corner-aligned samples, in f32 arithmetic (the page's
    host copy is f32), each operation rounded to f32 in this order:
      y = ((G-1) r) / (h-1) (0 when h = 1), y0 = floor(y), y1 = min(y0+1, G-1),
      dy = y - y0, and the same along the columns (x, x0, x1, dx);
      w00 = (1-dy)(1-dx), w01 = (1-dy) dx, w10 = dy (1-dx), w11 = dy dx;
      v = ((w00 T[y0,x0] + w01 T[y0,x1]) + w10 T[y1,x0]) + w11 T[y1,x1],
    then v is stored as bf16 (the operand the patch embedding adds)."""
    G = int(grid_side)
    tab = np.asarray(table, dtype=np.float64)
    if tab.ndim != 2 or tab.shape[0] != G * G:
        raise ValueError("table must be [G*G, D]")
    t32 = tab.astype(np.float32)
    if not np.array_equal(t32.astype(np.float64), tab):
        raise ValueError("table values must be f32 (bf16) values")
    f = np.float32
    out = []
    for h, w in grids:
        def axis(n):
            i = np.arange(n, dtype=np.float32)
            y = (f(G - 1) * i) / f(n - 1) if n > 1 else np.zeros(n, dtype=np.float32)
            y0 = np.floor(y).astype(np.int64)
            y1 = np.minimum(y0 + 1, G - 1)
            return y0, y1, (y - y0.astype(np.float32)).astype(np.float32)
        y0, y1, dy = axis(h)
        x0, x1, dx = axis(w)
        dy, dx = dy[:, None], dx[None, :]
        one = f(1.0)
        w00 = ((one - dy) * (one - dx))[..., None]
        w01 = ((one - dy) * dx)[..., None]
        w10 = (dy * (one - dx))[..., None]
        w11 = (dy * dx)[..., None]
        t00 = t32[(y0[:, None] * G + x0[None, :])]
        t01 = t32[(y0[:, None] * G + x1[None, :])]
        t10 = t32[(y1[:, None] * G + x0[None, :])]
        t11 = t32[(y1[:, None] * G + x1[None, :])]
        v = ((w00 * t00 + w01 * t01) + w10 * t10) + w11 * t11
        assert v.dtype == np.float32
        out.append(v.reshape(h * w, -1).astype(np.float64))
    return bf16(np.concatenate(out, axis=0))


def encoder_forward(pixels, w: EncoderWeights, grids, pos_embed=None,
                    mode: str = "storage", depth: int = DEPTH,
                    taps: Sequence[int] = TAPS, trace: Optional[dict] = None,
                    bf16_blocks: int = 0, fp8_mergers: bool = False):
    """Whole vision tower (FlashRT section 3): patch embed, blocks 1..27, the
    DeepStack taps after blocks 8/16/24 and the final block, each fed to its
    2x2 merger MLP.  Returns (out [len(taps), T/4, 4096], last hidden).
    Precision variants (FlashRT section 4 and section 1): the first
    ``bf16_blocks`` blocks with bf16 GEMMs, FP8 mergers."""
    cu = cu_seqlens_from_grids(grids)
    pos = positions_from_grids(grids)
    x = patch_embed(pixels, w, pos_embed, mode)
    outs = []
    ti = 0
    if trace is not None:
        trace["x0"] = x
    for b in range(1, depth + 1):
        fwd = block_forward_bf16 if b <= bf16_blocks else block_forward
        x = fwd(x, w.blocks[b - 1], pos, cu, mode)
        if trace is not None:
            trace[f"x{b}"] = x
        if ti < len(taps) and b == taps[ti]:
            outs.append(merger_forward(x, w.mergers[ti], grids, mode, fp8=fp8_mergers))
            ti += 1
    return np.stack(outs, axis=0), x


# ==========================================================================
# Algorithmic work (FLOPs), used to express measured times as throughput.
# ==========================================================================

def attention_flops(seq_lens: Sequence[int], hidden: int = HIDDEN) -> int:
    """4 * sum_i P_i^2 * hidden per block: QK^T and PV, 2 flops per MAC."""
    return int(sum(4 * int(p) * int(p) * hidden for p in seq_lens))


def block_gemm_flops(T: int) -> int:
    return 2 * T * HIDDEN * (3 * HIDDEN + HIDDEN + MLP + MLP)


def encoder_flops(seq_lens: Sequence[int], depth: int = DEPTH, n_mergers: int = 4) -> Dict[str, int]:
    T = int(sum(seq_lens))
    tm = T // 4
    merger = 2 * tm * MERGED_DIM * (MERGED_DIM + OUT_HIDDEN)
    d = dict(attention=depth * attention_flops(seq_lens), gemm=depth * block_gemm_flops(T),
             patch=2 * T * PATCH_DIM * HIDDEN, mergers=n_mergers * merger)
    d["total"] = sum(d.values())
    return d
