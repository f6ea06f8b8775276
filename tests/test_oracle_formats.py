"""Pins of the oracle's number formats: bf16 rounding, E4M3FN codec and the
block-128 quantiser.  Checked against hand-derived points, closed forms and
torch's own format conversions (independent library routines)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def torch_e4m3_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------- bf16

def test_bf16_matches_torch_on_fp32_values():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(200000).astype(np.float32) * 10,
                        (g.standard_normal(10000) * 1e-38).astype(np.float32),   # subnormal range
                        g.standard_normal(10000).astype(np.float32) * 1e30])
    # exact ties: fp32 values whose low 16 bits are 0x8000
    u = (g.integers(0x3F000000, 0x4F000000, 5000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, u.view(np.float32)])
    assert np.array_equal(O.bf16(x.astype(np.float64)), torch_bf16(x))


def test_bf16_hand_points():
    assert O.bf16(1 + 2.0 ** -8) == 1.0                      # tie -> even
    assert O.bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6        # tie -> even (up)
    assert O.bf16(1 + 2.0 ** -8 + 2.0 ** -30) == 1 + 2.0 ** -7
    mx = float.fromhex("0x1.fep127")
    assert O.bf16(mx) == mx
    assert np.isinf(O.bf16(float.fromhex("0x1.ffp127")))     # tie above max -> inf
    assert np.signbit(O.bf16(-0.0))


def test_bf16_single_rounding_from_fp64():
    # A value just above a bf16 midpoint whose fp32 rounding lands exactly on
    # the midpoint: direct rounding from fp64 must go up.
    x = 1 + 2.0 ** -8 + 2.0 ** -40
    assert O.bf16(x) == 1 + 2.0 ** -7


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_closed_form_and_torch():
    t = O.e4m3_decode_table()
    finite = ~np.isnan(t)
    assert finite.sum() == 254
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0
    pos = t[1:0x7F]
    assert pos.min() == 2.0 ** -9 and np.all(np.diff(t[:0x7F]) > 0)
    assert t[0x08] == 2.0 ** -6 and t[0x07] == 7 * 2.0 ** -9
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ref), ~finite)
    assert np.array_equal(ref[finite], t[finite])


def test_e4m3_round_trip_all_finite_codes():
    t = O.e4m3_decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert np.array_equal(O.e4m3_encode(t[codes]), codes)


def test_e4m3_hand_points():
    cases = json.load(open(os.path.join(GOLDEN, "e4m3_points.json")))["cases"]
    for expr, code in cases:
        v = float(eval(expr, {"__builtins__": {}}))
        assert int(O.e4m3_encode(np.array([v]))[0]) == code, expr


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(1)
    x = np.concatenate([g.uniform(-448, 448, 300000), g.standard_normal(100000) * 1e-2,
                        g.standard_normal(100000) * 2.0 ** -8]).astype(np.float32)
    # every midpoint between neighbouring codes, and its fp32 neighbours
    t = O.e4m3_decode_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000), -mids])
    x = x[np.abs(x) <= 448]
    assert np.array_equal(O.e4m3_encode(x.astype(np.float64)), torch_e4m3_codes(x))


# ---------------------------------------------------------------- quantiser

def test_quantize_amax_maps_to_448_and_scale():
    g = np.random.default_rng(2)
    x = O.f32(g.standard_normal((64, 300)) * g.uniform(0.01, 100, (64, 1)))
    codes, s = O.quantize_block128(x, 1)
    assert codes.shape == (64, 384) and s.shape == (64, 3)
    for b in range(3):
        blk = x[:, b * 128:(b + 1) * 128]
        amax = np.abs(blk).max(axis=1)
        # scale * 448 equals amax to within one fp32 ulp
        assert np.all(np.abs(s[:, b] * 448 - amax) <= np.spacing(amax.astype(np.float32)).astype(np.float64))
        idx = np.abs(blk).argmax(axis=1)
        c = codes[np.arange(64), b * 128 + idx]
        assert np.all((c & 0x7F) == 0x7E)


def test_quantize_error_bound():
    g = np.random.default_rng(3)
    x = O.f32(g.standard_normal((32, 256)))
    codes, s = O.quantize_block128(x, 1)
    deq = O.dequantize_block128(codes, s, 1)
    sb = np.repeat(s, 128, axis=1)
    # |x - deq| <= half an E4M3 step (relative 2^-4 in the normal range,
    # absolute 2^-10 * s in the subnormal range), plus fp32 rounding of x*inv
    err = np.abs(x - deq)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * sb) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quantize_power_of_two_is_exact():
    g = np.random.default_rng(4)
    grid = O.e4m3_decode_table()[:0x7F]
    for k in (-5, 0, 3):
        vals = g.choice(grid, size=(4, 128)) * g.choice([-1.0, 1.0], size=(4, 128))
        vals[:, 7] = 448.0
        x = vals * 2.0 ** k
        codes, s = O.quantize_block128(x, 1)
        assert np.all(s == 2.0 ** k)
        assert np.array_equal(O.dequantize_block128(codes, s, 1), x)


def test_quantize_zero_block_and_signed_zero():
    x = np.zeros((2, 128))
    x[1] = -0.0
    codes, s = O.quantize_block128(x, 1)
    assert np.all(s == 0) and np.all(codes[0] == 0) and np.all(codes[1] == 0x80)


def test_quantize_ragged_equals_zero_padded():
    g = np.random.default_rng(5)
    x = O.f32(g.standard_normal((200, 200)))
    xp = np.zeros((256, 256))
    xp[:200, :200] = x
    for br in (1, 128):
        c1, s1 = O.quantize_block128(x, br)
        c2, s2 = O.quantize_block128(xp, br)
        R = c1.shape[0]
        assert np.array_equal(c1, c2[:R]) and np.array_equal(s1, s2[:s1.shape[0]])


def test_quantize_weight_blocks_independent_library():
    # 128x128 blocks, checked with torch's E4M3 conversion of x * inv
    g = np.random.default_rng(6)
    w = O.f32(g.standard_normal((256, 384)) * 0.02)
    codes, s = O.quantize_block128(w, 128)
    assert s.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128].astype(np.float32)
            amax = np.abs(blk).max()
            inv = np.float32(448.0) / amax
            assert s[i, j] == np.float32(amax) / np.float32(448.0)
            ref = torch_e4m3_codes(blk * inv)
            assert np.array_equal(codes[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128], ref)


def test_quantize_zero_scale_threshold_boundary():
    """Blocks whose amax sits just below and just above 2^-116.  Below, the
    block gets scale 0 and its codes are signed zeros.  Above, scale and
    inverse are normal, finite fp32 values (2^-116 / 448 > 2^-126, the
    smallest normal; 448 / 2^-116 < 2^128), the amax element maps to 448 and
    the half-step error bound holds.  A mistake in the threshold's
    comparison, its exponent or the zero path fails one side."""
    t = 2.0 ** -116
    below, above = O.f32(t * (1 - 2.0 ** -20)), O.f32(t * (1 + 2.0 ** -20))
    assert below < t < above  # both are fp32 values on either side of 2^-116
    g = np.random.default_rng(7)
    x = np.zeros((3, 128))
    for r, amax in enumerate((below, above, t)):
        x[r] = O.f32(g.uniform(-1, 1, 128) * amax)
        x[r, 5] = -amax
    codes, s = O.quantize_block128(x, 1)
    # below the threshold: scale 0, every code a zero of the element's sign
    assert s[0, 0] == 0.0
    assert np.all((codes[0] & 0x7F) == 0)
    assert np.array_equal(codes[0] >> 7, np.signbit(x[0]).astype(np.uint8))
    # at and above it: normal finite scale, amax -> 448 (code 0xFE for -amax)
    for r in (1, 2):
        amax = np.abs(x[r]).max()
        sv = np.float32(s[r, 0])
        assert np.isfinite(sv) and sv >= np.finfo(np.float32).tiny
        assert sv == np.float32(np.float32(amax) / np.float32(448.0))
        inv = np.float32(448.0) / np.float32(amax)
        assert np.isfinite(inv) and inv < np.finfo(np.float32).max
        assert codes[r, 5] == 0xFE
        deq = O.dequantize_block128(codes[r:r + 1], s[r:r + 1], 1)[0]
        bound = np.maximum(np.abs(x[r]) * 2.0 ** -4, 2.0 ** -10 * s[r, 0]) * (1 + 1e-6)
        assert np.all(np.abs(x[r] - deq) <= bound)
