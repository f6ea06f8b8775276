"""Pins of the oracle's operations: LayerNorm, GELU, 2D RoPE, attention,
the FP8 and bf16 GEMMs and the 2x2 merge.  Each is checked against an
independent library routine, a closed form, an invariant or brute force."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


# ---------------------------------------------------------------- LayerNorm

def test_layernorm_matches_torch():
    g = np.random.default_rng(0)
    x = g.standard_normal((33, 1152)) * 3 + 1
    gam, bet = 1 + 0.02 * g.standard_normal(1152), 0.01 * g.standard_normal(1152)
    ref = F.layer_norm(torch.from_numpy(x), (1152,), torch.from_numpy(gam), torch.from_numpy(bet), eps=1e-6)
    assert np.allclose(O.layernorm(x, gam, bet), ref.numpy(), rtol=0, atol=1e-12)


def test_layernorm_moments_and_affine_invariance():
    g = np.random.default_rng(1)
    x = g.standard_normal((5, 256))
    y = O.layernorm(x, 1.0, 0.0)
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose(y.var(axis=1), var / (var + 1e-6), rtol=1e-12)
    y2 = O.layernorm(7.0 * x - 3.0, 1.0, 0.0, eps=0.0)
    assert np.allclose(O.layernorm(x, 1.0, 0.0, eps=0.0), y2, atol=1e-12)


def test_layernorm_brute_force_small():
    x = [[1.0, 2.0, 4.0, 7.0]]
    mu = sum(x[0]) / 4
    var = sum((v - mu) ** 2 for v in x[0]) / 4
    exp = [[(v - mu) / math.sqrt(var + 1e-6) * 2.0 + 0.5 for v in x[0]]]
    assert np.allclose(O.layernorm(np.array(x), 2.0, 0.5), exp, atol=1e-14)


# ---------------------------------------------------------------- GELU

def test_gelu_tanh_matches_torch_and_identities():
    x = np.linspace(-12, 12, 20001)
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.allclose(O.gelu_tanh(x), ref, rtol=0, atol=1e-14)
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(O.gelu_tanh(x) - O.gelu_tanh(-x), x, atol=1e-12)
    assert np.allclose(O.gelu_tanh(np.array([30.0, -30.0])), [30.0, 0.0], atol=1e-12)


# ---------------------------------------------------------------- RoPE

def _pos(T, g):
    return g.integers(0, 140, size=(T, 2))


def test_rope_preserves_pair_norms_and_identity_at_origin():
    g = np.random.default_rng(2)
    x = g.standard_normal((20, 1152))
    pos = _pos(20, g)
    y = O.rope2d(x, pos)
    xh, yh = x.reshape(20, 16, 72), y.reshape(20, 16, 72)
    for base in (0, 36):
        n0 = xh[..., base:base + 18] ** 2 + xh[..., base + 18:base + 36] ** 2
        n1 = yh[..., base:base + 18] ** 2 + yh[..., base + 18:base + 36] ** 2
        assert np.allclose(n0, n1, rtol=1e-12)
    assert np.array_equal(O.rope2d(x, np.zeros((20, 2), int)), x)


def test_rope_complex_form():
    # Each rotate_half pair is the complex number u + i v multiplied by
    # exp(i * p * f): an independent formulation of the same rotation.
    g = np.random.default_rng(3)
    x = g.standard_normal((7, 1152))
    pos = _pos(7, g)
    y = O.rope2d(x, pos).reshape(7, 16, 72)
    xh = x.reshape(7, 16, 72)
    f = 10000.0 ** (-np.arange(0, 36, 2) / 36.0)
    for axis, base in ((0, 0), (1, 36)):
        z = xh[..., base:base + 18] + 1j * xh[..., base + 18:base + 36]
        zr = z * np.exp(1j * pos[:, axis, None, None] * f[None, None, :])
        assert np.allclose(y[..., base:base + 18], zr.real, atol=1e-12)
        assert np.allclose(y[..., base + 18:base + 36], zr.imag, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    g = np.random.default_rng(4)
    q = g.standard_normal((1, 1152))
    k = g.standard_normal((1, 1152))
    p1, p2 = np.array([[3, 40]]), np.array([[10, 5]])
    s = (O.rope2d(q, p1) * O.rope2d(k, p2)).reshape(16, 72).sum(1)
    shift = np.array([[17, 29]])
    s2 = (O.rope2d(q, p1 + shift) * O.rope2d(k, p2 + shift)).reshape(16, 72).sum(1)
    assert np.allclose(s, s2, atol=1e-10)
    # but not invariant to a shift of one side only
    s3 = (O.rope2d(q, p1 + shift) * O.rope2d(k, p2)).reshape(16, 72).sum(1)
    assert not np.allclose(s, s3, atol=1e-3)


def test_rope_row_axis_uses_first_half():
    # moving only the column leaves dims 0..35 of every head untouched
    g = np.random.default_rng(5)
    x = g.standard_normal((1, 1152))
    a = O.rope2d(x, np.array([[4, 0]])).reshape(16, 72)
    b = O.rope2d(x, np.array([[4, 9]])).reshape(16, 72)
    assert np.array_equal(a[:, :36], b[:, :36]) and not np.allclose(a[:, 36:], b[:, 36:])


def test_rope_equals_hf_layout_after_fixed_permutation():
    """The library (transformers) Qwen-VL vision rotary uses another layout:
    per token the angles [row f_0..f_17, col f_0..f_17] duplicated to 72 and
    one rotate_half over the whole head, pairs (i, i + 36).  The reading taken
    here (dims 0..35 rotate by the row, 36..71 by the column, pairs (i, i + 18)
    inside each half) is that rotation after a fixed per-head permutation of
    the dims, the same for q and k, so q.k scores agree: a weight-load
    permutation of the q and k rows of the qkv weight switches layouts."""
    from transformers.models.qwen3_vl.modeling_qwen3_vl import (Qwen3VLVisionRotaryEmbedding,
                                                                 apply_rotary_pos_emb_vision)
    g = np.random.default_rng(6)
    T = 40
    pos = _pos(T, g)
    q = g.standard_normal((T, 16, 72)).astype(np.float32).astype(np.float64)
    k = g.standard_normal((T, 16, 72)).astype(np.float32).astype(np.float64)
    ang = Qwen3VLVisionRotaryEmbedding(36)(torch.from_numpy(pos))        # [T, 36]
    emb = torch.cat([ang, ang], dim=-1)
    qh, kh = apply_rotary_pos_emb_vision(torch.from_numpy(q), torch.from_numpy(k), emb.cos(), emb.sin())
    qh, kh = qh.double().numpy(), kh.double().numpy()
    # HF dim of each dim of this layout: row pair halves, then column pair halves
    perm = np.concatenate([np.arange(0, 18), np.arange(36, 54), np.arange(18, 36), np.arange(54, 72)])
    qr = O.rope2d(q[:, :, perm].reshape(T, 1152), pos).reshape(T, 16, 72)
    kr = O.rope2d(k[:, :, perm].reshape(T, 1152), pos).reshape(T, 16, 72)
    tol = 1e-4 * np.abs(q).max()  # the library rotates in fp32 (angles up to ~140 rad)
    assert np.allclose(qr, qh[:, :, perm], atol=tol, rtol=0)
    assert np.allclose(kr, kh[:, :, perm], atol=tol, rtol=0)
    s_r = np.einsum("thd,uhd->htu", qr, kr)
    s_h = np.einsum("thd,uhd->htu", qh, kh)
    assert np.allclose(s_r, s_h, atol=1e-3, rtol=0)
    # without the permutation the two layouts genuinely differ
    assert not np.allclose(O.rope2d(q.reshape(T, 1152), pos).reshape(T, 16, 72), qh, atol=1e-2)


# ---------------------------------------------------------------- attention

def test_attention_matches_torch_sdpa_per_window():
    g = np.random.default_rng(6)
    cu = [0, 5, 37, 40]
    T = cu[-1]
    q, k, v = (g.standard_normal((T, 1152)) for _ in range(3))
    out = O.attention(q, k, v, cu)
    for j in range(3):
        a, b = cu[j], cu[j + 1]
        tq = torch.from_numpy(q[a:b].reshape(b - a, 16, 72).transpose(1, 0, 2).copy())
        tk = torch.from_numpy(k[a:b].reshape(b - a, 16, 72).transpose(1, 0, 2).copy())
        tv = torch.from_numpy(v[a:b].reshape(b - a, 16, 72).transpose(1, 0, 2).copy())
        ref = F.scaled_dot_product_attention(tq, tk, tv).numpy().transpose(1, 0, 2).reshape(b - a, 1152)
        assert np.allclose(out[a:b], ref, atol=1e-12)


def test_attention_invariants():
    g = np.random.default_rng(7)
    T = 24
    q, k = g.standard_normal((T, 1152)), g.standard_normal((T, 1152))
    # constant V -> V
    v = np.tile(g.standard_normal((1, 1152)), (T, 1))
    assert np.allclose(O.attention(q, k, v, [0, T]), v, atol=1e-12)
    # Q = 0 -> mean of V
    v = g.standard_normal((T, 1152))
    assert np.allclose(O.attention(np.zeros_like(q), k, v, [0, T]), np.tile(v.mean(0), (T, 1)), atol=1e-12)
    # one-key window -> that V
    assert np.allclose(O.attention(q[:1], k[:1], v[:1], [0, 1]), v[:1])
    # rows of P sum to one: with V = all-ones per head the output is ones
    assert np.allclose(O.attention(q, k, np.ones_like(v), [0, T]), 1.0, atol=1e-12)
    # permutation equivariance inside a window
    perm = g.permutation(T)
    assert np.allclose(O.attention(q[perm], k[perm], v[perm], [0, T]), O.attention(q, k, v, [0, T])[perm], atol=1e-12)


def test_attention_brute_force_tiny():
    g = np.random.default_rng(8)
    T = 4
    q, k, v = (g.standard_normal((T, 1152)) for _ in range(3))
    out = O.attention(q, k, v, [0, T])
    h, i, d = 5, 2, 17
    sl = slice(72 * h, 72 * h + 72)
    sc = [sum(q[i, sl][e] * k[j, sl][e] for e in range(72)) / math.sqrt(72) for j in range(T)]
    m = max(sc)
    p = [math.exp(s - m) for s in sc]
    z = sum(p)
    assert abs(out[i, 72 * h + d] - sum(p[j] / z * v[j, 72 * h + d] for j in range(T))) < 1e-12


def test_attention_varlen_equals_separate():
    g = np.random.default_rng(9)
    cu = [0, 9, 30]
    q, k, v = (g.standard_normal((30, 1152)) for _ in range(3))
    packed = O.attention(q, k, v, cu)
    a = O.attention(q[:9], k[:9], v[:9], [0, 9])
    b = O.attention(q[9:], k[9:], v[9:], [0, 21])
    assert np.array_equal(packed, np.concatenate([a, b]))


# ---------------------------------------------------------------- GEMMs

def _rand_codes(g, shape):
    c = g.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x00  # no NaN codes
    return c


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (3, 128, 256), (5, 256, 384)])
def test_fp8_gemm_brute_force(M, N, K):
    g = np.random.default_rng(M * 1000 + K)
    a, w = _rand_codes(g, (M, K)), _rand_codes(g, (N, K))
    sa = O.f32(g.uniform(0.001, 2, (M, K // 128)))
    sw = O.f32(g.uniform(0.001, 2, (N // 128, K // 128)))
    C = O.fp8_block128_gemm(a, sa, w, sw)
    t = O.e4m3_decode_table()
    for m in range(M):
        for n in range(0, N, 37):
            acc = 0.0
            for kb in range(K // 128):
                part = 0.0
                for kk in range(kb * 128, kb * 128 + 128):
                    part += t[a[m, kk]] * t[w[n, kk]]
                acc += sa[m, kb] * sw[n // 128, kb] * part
            assert abs(C[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_fp8_gemm_unit_scales_equal_plain_product_and_pow2_exact():
    g = np.random.default_rng(10)
    a, w = _rand_codes(g, (16, 512)), _rand_codes(g, (256, 512))
    t = O.e4m3_decode_table()
    C = O.fp8_block128_gemm(a, np.ones((16, 4)), w, np.ones((2, 4)))
    assert np.array_equal(C, t[a] @ t[w].T)
    sa = 2.0 ** g.integers(-8, 8, (16, 4)).astype(float)
    sw = 2.0 ** g.integers(-8, 8, (2, 4)).astype(float)
    C2 = O.fp8_block128_gemm(a, sa, w, sw)
    deqa = t[a] * np.repeat(sa, 128, axis=1)
    deqw = t[w] * np.repeat(np.repeat(sw, 128, axis=0), 128, axis=1)
    exact = np.zeros((16, 256))
    for kb in range(4):  # power-of-two scaled products are exact per block
        ks = slice(kb * 128, kb * 128 + 128)
        exact += deqa[:, ks] @ deqw[:, ks].T
    assert np.array_equal(C2, exact)


def test_fp8_gemm_ragged_k_equals_padded():
    g = np.random.default_rng(11)
    x = O.f32(g.standard_normal((8, 200)))
    w = O.f32(g.standard_normal((130, 200)) * 0.02)
    ac, as_ = O.quantize_block128(x, 1)
    wc, ws = O.quantize_block128(w, 128)
    xp = np.zeros((8, 256)); xp[:, :200] = x
    wp = np.zeros((256, 256)); wp[:130, :200] = w
    ac2, as2 = O.quantize_block128(xp, 1)
    wc2, ws2 = O.quantize_block128(wp, 128)
    assert np.array_equal(O.fp8_block128_gemm(ac, as_, wc, ws), O.fp8_block128_gemm(ac2, as2, wc2, ws2))


def test_fp8_gemm_close_to_exact_product():
    # quantisation error only: relative to the exact fp64 GEMM
    g = np.random.default_rng(12)
    x = O.f32(g.standard_normal((64, 1152)))
    w = O.f32(g.standard_normal((256, 1152)) * 0.02)
    ac, as_ = O.quantize_block128(x, 1)
    wc, ws = O.quantize_block128(w, 128)
    C = O.fp8_block128_gemm(ac, as_, wc, ws)
    ref = x @ w.T
    cos = (C * ref).sum() / np.linalg.norm(C) / np.linalg.norm(ref)
    assert cos > 0.998


def test_epilogues():
    g = np.random.default_rng(13)
    C = g.standard_normal((4, 256))
    b = g.standard_normal(200)
    r = g.standard_normal((4, 200))
    assert np.array_equal(O.fp8_gemm_epilogue(C, 200, O.EPI_BIAS, bias=b), O.bf16(C[:, :200] + b))
    assert np.array_equal(O.fp8_gemm_epilogue(C, 200, O.EPI_BIAS_RESIDUAL, bias=b, residual=r),
                          O.bf16(C[:, :200] + b + r))
    codes, s, pre = O.fp8_gemm_epilogue(C, 200, O.EPI_BIAS_GELU_FP8, bias=b)
    assert codes.shape == (4, 256) and s.shape == (4, 2)
    assert np.all(pre[:, 200:] == 0) and np.all(codes[:, 200:] == 0)
    assert np.allclose(pre[:, :200], F.gelu(torch.from_numpy(C[:, :200] + b), approximate="tanh").numpy())


def test_bf16_gemm_matches_torch():
    g = np.random.default_rng(14)
    a = O.bf16(g.standard_normal((9, 64)))
    w = O.bf16(g.standard_normal((40, 64)))
    b = g.standard_normal(40)
    ref = F.linear(torch.from_numpy(a), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    assert np.allclose(O.bf16_gemm(a, w, b), ref, atol=1e-12)


# ---------------------------------------------------------------- merge

@pytest.mark.parametrize("grids", [[(2, 2)], [(4, 6)], [(6, 4)], [(2, 2), (4, 6), (6, 4)]])
def test_merge_brute_force(grids):
    # token t carries its own (image, row, col) code in every feature slot
    rows = []
    for j, (h, w) in enumerate(grids):
        for r in range(h):
            for c in range(w):
                rows.append([1000 * j + 100 * r + c] * 3)
    x = np.array(rows, dtype=np.float64)
    y = O.merge2x2(x, grids)
    k = 0
    for j, (h, w) in enumerate(grids):
        for R in range(h // 2):
            for C in range(w // 2):
                exp = []
                for (dr, dc) in ((0, 0), (0, 1), (1, 0), (1, 1)):
                    exp += [1000 * j + 100 * (2 * R + dr) + (2 * C + dc)] * 3
                assert list(y[k]) == exp
                k += 1
    assert k == y.shape[0] == sum(h * w for h, w in grids) // 4


def test_positions_and_cu():
    grids = [(2, 3), (4, 2)]
    assert list(O.cu_seqlens_from_grids(grids)) == [0, 6, 14]
    pos = O.positions_from_grids(grids)
    assert pos[:6].tolist() == [[0, 0], [0, 1], [0, 2], [1, 0], [1, 1], [1, 2]]
    assert pos[6:].tolist() == [[r, c] for r in range(4) for c in range(2)]
