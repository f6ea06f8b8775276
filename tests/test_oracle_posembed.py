"""Pins of the oracle's interpolated position embedding (pos_embed_interp):
corner-aligned bilinear resampling of the learned 48 x 48 table, in f32,
stored as bf16.  Checked against two independent library resamplers (torch
bilinear with aligned corners, scipy's regular-grid linear interpolator), a
closed form (a table linear in row and column is reproduced at the sample
points), exact identities (the 48 x 48 grid, the corners, a 1 x 1 image) and
the packing of several images."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.interpolate import RegularGridInterpolator

import oracle as O


def _table(G, D, seed=0, std=0.02):
    g = np.random.default_rng(seed)
    return O.bf16(g.standard_normal((G * G, D)) * std)


def _bf16_close(got, ref, table_max, G=O.POS_GRID):
    # the oracle works in f32 and rounds once to bf16.  Against an fp64
    # resampler: one bf16 rounding (2^-8 relative), the f32 rounding of the
    # sample position y ~ (G-1) r/(h-1) (2^-24 (G-1) absolute) times the
    # table's step between neighbours (at most 2 max|T|), and the f32
    # rounding of the weights and the four-term sum (under 2^-21 max|T|,
    # which also covers cancellation near zero)
    atol = (2.0 ** -24 * 2 * (G - 1) + 2.0 ** -21) * table_max
    return np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + atol)


@pytest.mark.parametrize("hw", [(46, 136), (18, 54), (36, 108), (24, 76), (48, 38), (2, 2), (96, 96), (3, 7)])
def test_matches_torch_bilinear_align_corners(hw):
    G, D = O.POS_GRID, 64
    t = _table(G, D)
    h, w = hw
    got = O.pos_embed_interp(t, [hw])
    img = torch.from_numpy(t.reshape(G, G, D)).permute(2, 0, 1)[None]  # [1, D, G, G], fp64
    ref = F.interpolate(img, size=(h, w), mode="bilinear", align_corners=True)[0].permute(1, 2, 0)
    ref = ref.reshape(h * w, D).numpy()
    assert _bf16_close(got, ref, np.abs(t).max())


@pytest.mark.parametrize("hw", [(46, 136), (5, 3), (1, 9)])
def test_matches_scipy_regular_grid(hw):
    G, D = 8, 16
    t = _table(G, D, seed=3, std=1.0)
    h, w = hw
    got = O.pos_embed_interp(t, [hw], grid_side=G)
    ys = np.arange(h) * (G - 1) / (h - 1) if h > 1 else np.zeros(1)
    xs = np.arange(w) * (G - 1) / (w - 1) if w > 1 else np.zeros(1)
    f = RegularGridInterpolator((np.arange(G), np.arange(G)), t.reshape(G, G, D), method="linear")
    pts = np.stack(np.meshgrid(ys, xs, indexing="ij"), axis=-1).reshape(-1, 2)
    assert _bf16_close(got, f(pts), np.abs(t).max(), G)


def test_full_grid_is_the_table():
    G = O.POS_GRID
    t = _table(G, 32, seed=1)
    assert np.array_equal(O.pos_embed_interp(t, [(G, G)]), t)


@pytest.mark.parametrize("hw", [(46, 136), (2, 2), (17, 5), (48, 48)])
def test_corners_are_table_corners(hw):
    G = O.POS_GRID
    t = _table(G, 16, seed=2)
    h, w = hw
    o = O.pos_embed_interp(t, [hw]).reshape(h, w, -1)
    assert np.array_equal(o[0, 0], t[0])
    assert np.array_equal(o[0, w - 1], t[G - 1])
    assert np.array_equal(o[h - 1, 0], t[(G - 1) * G])
    assert np.array_equal(o[h - 1, w - 1], t[G * G - 1])


def test_single_patch_takes_the_first_entry():
    t = _table(O.POS_GRID, 16, seed=4)
    assert np.array_equal(O.pos_embed_interp(t, [(1, 1)]), t[:1])


def test_linear_table_is_reproduced():
    # T[r, c, d] = a_d r + b_d c + g_d (exact small dyadic values): bilinear
    # interpolation returns a_d y + b_d x + g_d at the sample point (y, x)
    G, D = O.POS_GRID, 8
    a = np.arange(D) / 64.0
    b = -np.arange(D) / 128.0
    g0 = np.full(D, 0.5)
    r, c = np.meshgrid(np.arange(G), np.arange(G), indexing="ij")
    t = (r[..., None] * a + c[..., None] * b + g0).reshape(G * G, D)
    h, w = 46, 136
    o = O.pos_embed_interp(t, [(h, w)]).reshape(h, w, D)
    y = np.arange(h) * (G - 1) / (h - 1)
    x = np.arange(w) * (G - 1) / (w - 1)
    ref = y[:, None, None] * a + x[None, :, None] * b + g0
    assert np.all(np.abs(o - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


def test_images_are_packed_in_order():
    t = _table(O.POS_GRID, 24, seed=5)
    grids = [(18, 54), (36, 108), (24, 76)]
    whole = O.pos_embed_interp(t, grids)
    parts = np.concatenate([O.pos_embed_interp(t, [g]) for g in grids])
    assert np.array_equal(whole, parts)
    assert whole.shape == (sum(h * w for h, w in grids), 24)


def test_transposed_table_gives_transposed_output():
    G = O.POS_GRID
    t = _table(G, 16, seed=6)
    tt = t.reshape(G, G, -1).transpose(1, 0, 2).reshape(G * G, -1)
    h, w = 20, 34
    o = O.pos_embed_interp(t, [(h, w)]).reshape(h, w, -1)
    ot = O.pos_embed_interp(tt, [(w, h)]).reshape(w, h, -1)
    assert _bf16_close(ot.transpose(1, 0, 2), o, np.abs(t).max())


def test_rejects_a_table_of_the_wrong_size():
    with pytest.raises(ValueError):
        O.pos_embed_interp(np.zeros((10, 8)), [(2, 2)], grid_side=4)
