"""Pins of the oracle's input preprocessing (oracle.preprocess): the
smart_resize sizes against the page's resolution table, the bilinear
resize against torch's (half-pixel centres, no antialias) and exact
identities, the normalisation against its closed form, and the patch layout
and temporal pairing against brute-force index loops."""

import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import preprocess as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    return json.load(open(os.path.join(GOLDEN, "pages_facts.json")))["smart_resize_rows"]


def test_smart_resize_reproduces_the_resolution_table():
    f = _facts()
    H, W = f["image_height"], f["image_width"]
    grids = []
    for max_pixels, patches in f["rows"]:
        h, w = P.smart_resize(H, W, max_pixels=max_pixels)
        assert h % 32 == 0 and w % 32 == 0
        assert (h // 16) * (w // 16) == patches, (max_pixels, h, w)
        grids.append((h // 16, w // 16))
    assert grids == [(46, 136), (36, 108), (24, 76), (18, 54)]


@pytest.mark.parametrize("hw", [(100, 100), (17, 900), (4000, 3000), (31, 33), (64, 96)])
@pytest.mark.parametrize("limits", [(0, None), (0, 250000), (200000, None), (3136, 1000000)])
def test_smart_resize_bounds(hw, limits):
    lo, hi = limits
    h, w = P.smart_resize(*hw, min_pixels=lo, max_pixels=hi)
    assert h % 32 == 0 and w % 32 == 0 and h >= 32 and w >= 32
    if hi is not None and (hw[0] * hw[1] >= 4 * 32 * 32):
        assert h * w <= hi
    if lo and (hi is None or P.smart_resize(*hw)[0] * P.smart_resize(*hw)[1] <= hi):
        assert h * w >= lo


def test_smart_resize_keeps_grid_sizes():
    assert P.smart_resize(736, 2176) == (736, 2176)
    # ties go to even multiples, as Python's round does
    assert P.smart_resize(48, 48) == (64, 64)   # 1.5 -> 2
    assert P.smart_resize(80, 80) == (64, 64)   # 2.5 -> 2


def test_resize_identity_and_constant():
    g = np.random.default_rng(0)
    img = g.integers(0, 256, (37, 53, 3), dtype=np.uint8)
    assert np.array_equal(P.resize_bilinear(img, 37, 53), img.astype(np.float32))
    const = np.full((20, 30, 3), 77, dtype=np.uint8)
    assert np.all(P.resize_bilinear(const, 48, 64) == 77.0)


@pytest.mark.parametrize("out", [(736, 2176), (64, 96), (16, 16), (35, 5)])
def test_resize_matches_torch_bilinear(out):
    g = np.random.default_rng(1)
    img = g.integers(0, 256, (61, 173, 3), dtype=np.uint8)
    got = P.resize_bilinear(img, *out)
    t = torch.from_numpy(img.astype(np.float64)).permute(2, 0, 1)[None]
    ref = F.interpolate(t, size=out, mode="bilinear", align_corners=False, antialias=False)
    ref = ref[0].permute(1, 2, 0).numpy()
    # the oracle works in f32: its source coordinate (i + 1/2) H/H' - 1/2
    # carries a few ulps of the source extent (at most 4 x 2^-24 x max(H, W)),
    # times a pixel step of at most 255, plus the f32 rounding of the
    # weighted sum (a few ulps of 255)
    tol = 255 * 4 * 2.0 ** -24 * max(img.shape[:2]) + 255 * 2.0 ** -20
    assert np.abs(got - ref).max() <= tol


def test_normalisation_closed_form():
    mean, std = (0.48, 0.46, 0.41), (0.27, 0.26, 0.28)
    frame = np.zeros((1, 1, 1, 3), dtype=np.uint8)
    frame[0, 0, 0] = (10, 128, 255)
    px, grids = P.preprocess_frames(frame, 16, 16, mean, std)
    assert grids == [(1, 1)] and px.shape == (1, 1536)
    v = px.reshape(3, 2, 16, 16)
    for c, raw in enumerate((10, 128, 255)):
        ref = (raw / 255.0 - mean[c]) / std[c]
        assert np.all(np.abs(v[c] - ref) <= 4 * 2.0 ** -24 * (abs(ref) + 4))


@pytest.mark.parametrize("F_", [1, 2, 3, 4])
def test_patch_layout_and_temporal_pairs(F_):
    # identity resize, mean 0 and std 1: every output value is the raw pixel
    # times f32(1/255), so each output names its source pixel
    g = np.random.default_rng(2)
    h, w = 32, 48
    frames = g.integers(0, 256, (F_, h, w, 3), dtype=np.uint8)
    px, grids = P.preprocess_frames(frames, h, w, (0.0, 0.0, 0.0), (1.0, 1.0, 1.0))
    inv255 = np.float32(1.0 / 255.0)
    G = (F_ + 1) // 2
    gh, gw = h // 16, w // 16
    assert grids == [(gh, gw)] * G and px.shape == (G * gh * gw, 1536)
    for gi in range(G):
        for pr in range(gh):
            for pc in range(gw):
                row = gi * gh * gw + pr * gw + pc
                for c in range(3):
                    for t in range(2):
                        f = min(2 * gi + t, F_ - 1)
                        for py in range(0, 16, 5):
                            for pxx in range(0, 16, 3):
                                col = ((c * 2 + t) * 16 + py) * 16 + pxx
                                src = np.float32(frames[f, pr * 16 + py, pc * 16 + pxx, c])
                                assert px[row, col] == np.float32(src * inv255)
