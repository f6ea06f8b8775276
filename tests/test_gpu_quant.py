"""GPU parity of the FP8 format and quantisers: the E4M3 encoder at every
rounding decision point, the block-128 quantiser for activations (1 x 128)
and weights (128 x 128), and LayerNorm fused with the quant.  Codes and
scales are bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
import vision_transformer_encoder_amd as vit
from gpu_util import announce, assert_close, dev_bf16, host_f64, host_u8

pytestmark = pytest.mark.gpu


def _decision_points() -> np.ndarray:
    """fp32 values at and around every E4M3 rounding boundary in every binade
    from 2^-13 to 2^9, plus a strided sweep of all mantissas, both signs,
    zeros, fp32 subnormals and out-of-range values (saturate)."""
    vals = []
    for e in range(-13, 10):
        base = np.uint32((e + 127) << 23)
        # boundaries of 3 kept fraction bits lie at multiples of 2^19 in the
        # fp32 fraction (representable values and midpoints alike)
        b = (np.arange(0, 1 << 23, 1 << 19, dtype=np.int64)[:, None] + np.arange(-3, 4)[None, :]).ravel()
        b = b[(b >= 0) & (b < (1 << 23))].astype(np.uint32)
        vals.append((base | b).view(np.float32))
        vals.append((base | np.arange(0, 1 << 23, 4099, dtype=np.uint32)).view(np.float32))
    v = np.concatenate(vals)
    extra = np.array([0.0, 1e-40, 3e-39, 448.0, 449.0, 464.0, 480.0, 1e6, 3e38], np.float32)
    v = np.concatenate([v, extra])
    v = np.concatenate([v, -v])
    return v.astype(np.float32)


def test_e4m3_encoder_decision_points(gpu):
    x = _decision_points()
    announce(f"vit_e4m3_encode n={x.size}")
    codes = host_u8(vit.vit_e4m3_encode(torch.from_numpy(x).to(gpu)))
    ref = O.e4m3_encode(x.astype(np.float64))
    bad = np.nonzero(codes != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[:5]]} gpu={codes[bad[:5]]} ref={ref[bad[:5]]}"
    # negative zero keeps its sign
    assert codes[np.nonzero((x == 0) & np.signbit(x))[0][0]] == 0x80


@pytest.mark.parametrize("rows,cols", [(1, 128), (7, 200), (300, 1152), (6256, 1152), (5, 4608), (3, 9000)])
def test_quant_rows_bit_exact(gpu, rows, cols):
    bits = synth.normal_bf16(2, "a", rows * 7 + cols, (rows, cols))
    bits[:, :3] = 0  # some structure: zero columns
    if rows > 2:
        bits[2] = 0  # an all-zero row (zero scale)
    announce(f"vit_quant_fp8_block128 rows={rows} cols={cols}")
    codes, scales = vit.vit_quant_fp8_block128(dev_bf16(bits, gpu), block_rows=1)
    rc, rs = O.quantize_block128(synth.bf16_bits_to_f64(bits), 1)
    assert np.array_equal(host_u8(codes), rc)
    assert np.array_equal(host_f64(scales), rs)


@pytest.mark.parametrize("shape", [(3456, 1152), (1152, 1152), (4304, 1152), (1152, 4304), (130, 200)])
def test_quant_weight_blocks_bit_exact(gpu, shape):
    bits = synth.normal_bf16(2, "w", shape[0] + shape[1], shape, std=0.02)
    announce(f"vit_quant_fp8_block128 weights {shape}")
    codes, scales = vit.vit_quant_fp8_block128(dev_bf16(bits, gpu), block_rows=128)
    rc, rs = O.quantize_block128(synth.bf16_bits_to_f64(bits), 128)
    assert codes.shape == rc.shape and scales.shape == rs.shape
    assert np.array_equal(host_u8(codes), rc)
    assert np.array_equal(host_f64(scales), rs)


@pytest.mark.parametrize("M", [1, 256, 6256])
def test_layernorm_quant(gpu, M):
    x = synth.normal_bf16(0, "x", M, (M, 1152))
    g = synth.normal_bf16(0, "ln1_g", M, (1152,), std=0.02, mean=1.0)
    b = synth.normal_bf16(0, "ln1_b", M, (1152,), std=0.01)
    announce(f"vit_layernorm_quant_fp8 M={M}")
    codes, scales, pre = vit.vit_layernorm_quant_fp8(dev_bf16(x, gpu), dev_bf16(g, gpu), dev_bf16(b, gpu),
                                                     1e-6, prequant=True)
    xf, gf, bf = (synth.bf16_bits_to_f64(t) for t in (x, g, b))
    ref = O.layernorm(xf, gf, bf)
    pre_h = host_f64(pre)
    assert_close(pre_h, ref, 1e-5, 0.99999999, f"LN prequant M={M}")
    # the oracle's quantiser applied to the GPU's own fp32 pre-quant values
    rc, rs = O.quantize_block128(pre_h, 1)
    assert np.array_equal(host_u8(codes), rc)
    assert np.array_equal(host_f64(scales), rs)
    # codes taken independently from the fp64 LayerNorm differ by at most
    # one E4M3 step, and only rarely
    oc, _ = O.quantize_block128(O.f32(ref), 1)
    diff = np.abs(O.e4m3_decode(host_u8(codes)) - O.e4m3_decode(oc))
    flips = int((diff > 0).sum())
    announce(f"LN-quant code flips vs fp64 pre-quant: {flips} of {codes.numel()}")
    assert flips <= max(4, codes.numel() // 2000)


@pytest.mark.parametrize("block_rows", [1, 128])
def test_quant_zero_scale_threshold(gpu, block_rows):
    """Blocks whose amax lies just below 2^-116 (zero scale, signed-zero
    codes), exactly at it and just above it (normal scale), with bf16
    inputs: 2^-116 (1 - 2^-8), 2^-116 and 2^-116 (1 + 2^-7)."""
    t = 2.0 ** -116
    amaxes = (t * (1 - 2.0 ** -8), t, t * (1 + 2.0 ** -7), 0.0)
    g = np.random.default_rng(12)
    rows = 4 if block_rows == 1 else 512
    x = np.zeros((rows, 256))
    for i, amax in enumerate(amaxes):
        # block i: rows i (1 x 128 blocks) or rows 128 i .. 128 i + 127
        r = slice(i, i + 1) if block_rows == 1 else slice(128 * i, 128 * (i + 1))
        blk = O.bf16(g.uniform(-1, 1, (x[r].shape[0], 256)) * amax)
        blk[0, 3] = -amax
        blk[0, 200] = amax
        x[r] = blk
    bits = synth.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f64(bits), x)
    announce(f"vit_quant_fp8_block128 zero-scale threshold, block_rows={block_rows}")
    codes, scales = vit.vit_quant_fp8_block128(dev_bf16(bits, gpu), block_rows=block_rows)
    rc, rs = O.quantize_block128(x, block_rows)
    assert np.array_equal(host_u8(codes), rc)
    assert np.array_equal(host_f64(scales), rs)
    s = host_f64(scales)
    assert np.all(s[0] == 0) and np.all(s[1] > 0) and np.all(s[2] > 0)


def test_quant_scales_over_every_bf16_block_max(gpu):
    """Every positive bf16 value from 2^-116 to the largest finite one as the
    maximum of a 1 x 128 block (31232 blocks; the other values of a block
    are bf16 fractions of it, both signs): codes and scales bit-exact against
    the oracle, i.e. the kernels' amax / 448 and 448 / amax equal the
    correctly rounded fp32 quotients over the whole range, including the
    top two binades where the kernels keep the plain division."""
    biased = np.arange(127 - 116, 255, dtype=np.uint32)          # exponents -116 .. 127
    mant = np.arange(128, dtype=np.uint32)
    amax_bits = ((biased[:, None] << 7) | mant[None, :]).ravel().astype(np.uint16)
    amax = synth.bf16_bits_to_f64(amax_bits)
    g = np.random.default_rng(21)
    x = O.bf16(g.uniform(-1.0, 1.0, (amax.size, 128)) * amax[:, None])
    col = g.integers(0, 128, amax.size)
    x[np.arange(amax.size), col] = np.where(g.random(amax.size) < 0.5, -amax, amax)
    assert np.array_equal(np.abs(x).max(axis=1), amax)
    bits = synth.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f64(bits), x)
    announce(f"vit_quant_fp8_block128 over every bf16 block maximum, {amax.size} blocks")
    codes, scales = vit.vit_quant_fp8_block128(dev_bf16(bits, gpu), block_rows=1)
    rc, rs = O.quantize_block128(x, 1)
    assert np.array_equal(host_f64(scales), rs)
    assert np.array_equal(host_u8(codes), rc)


@pytest.mark.parametrize("k", [-100, -40, 40, 100, 125])
def test_layernorm_quant_scaled_gamma(gpu, k):
    """LayerNorm-quant with gamma and beta scaled by 2^k, so that the fp32
    block maxima (every mantissa, not only bf16 ones) lie near 2^(k+2): the
    quantiser on the GPU's own pre-quant values is bit-exact against the
    oracle's at each scale, up to the top binade (k = 125), where the
    kernels keep the plain division."""
    M = 1024
    x = synth.normal_bf16(0, "x", 500 + k, (M, 1152))
    gf = O.bf16(np.ldexp(1.0 + 0.02 * np.random.default_rng(k + 400).standard_normal(1152), k))
    bf = O.bf16(np.ldexp(0.01 * np.random.default_rng(k + 600).standard_normal(1152), k))
    g = synth.f32_to_bf16_bits(gf.astype(np.float32))
    b = synth.f32_to_bf16_bits(bf.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f64(g), gf) and np.array_equal(synth.bf16_bits_to_f64(b), bf)
    announce(f"vit_layernorm_quant_fp8 gamma x 2^{k}")
    codes, scales, pre = vit.vit_layernorm_quant_fp8(dev_bf16(x, gpu), dev_bf16(g, gpu), dev_bf16(b, gpu), 1e-6,
                                                     prequant=True)
    pre_h = host_f64(pre)
    ref = O.layernorm(synth.bf16_bits_to_f64(x), gf, bf)
    assert_close(pre_h, ref, 1e-5, 0.99999999, f"LN prequant, gamma x 2^{k}")
    rc, rs = O.quantize_block128(pre_h, 1)
    assert np.array_equal(host_f64(scales), rs)
    assert np.array_equal(host_u8(codes), rc)
    amax = np.abs(pre_h).reshape(M, 9, 128).max(axis=2)
    assert amax.min() >= 2.0 ** (k - 1) and amax.max() < 2.0 ** (k + 4)
