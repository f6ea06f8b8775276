"""Pins of the oracle's block, merger and encoder wiring, and of its
constants against the numbers printed on the source pages."""

import json
import os

import numpy as np
import pytest

import oracle as O
import synth
from oracle import inputs as OI

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def facts():
    return json.load(open(os.path.join(GOLDEN, "pages_facts.json")))


def test_constants_match_pages(facts):
    d = facts["tower_dims"]
    assert (O.DEPTH, O.HIDDEN, O.HEADS, O.HEAD_DIM, O.OUT_HIDDEN) == \
        (d["depth"], d["hidden"], d["heads"], d["head_dim"], d["out_hidden"])
    assert list(O.TAPS[:3]) == d["deepstack_layers"] == facts["encoder_struct"]["deepstack_indexes_1based"]
    assert list(O.TAPS) == facts["encoder_struct"]["module_doc_taps"]
    assert (O.MLP, O.MLP_PADDED) == (facts["ffn_padding"]["intermediate"], facts["ffn_padding"]["padded"])
    assert O.MLP_PADDED % 128 == 0 and O.MLP_PADDED - O.MLP < 128
    e = facts["encoder_struct"]
    assert O.PATCH_DIM == e["patch_dim"] == e["channels"] * e["temporal_patch"] * e["patch"] ** 2
    assert len(O.rope_inv_freq()) == e["rope_freqs"] == O.HEAD_DIM // 4
    assert O.MERGED_DIM == O.HIDDEN * e["spatial_merge"] ** 2


def test_workload_grids_reproduce_page_token_counts(facts):
    p = facts["patches_to_llm_tokens"]
    grid_of = {6256: (46, 136), 3888: (36, 108), 1824: (24, 76), 972: (18, 54)}
    for patches, llm_tokens in p["rows"]:
        h, w = grid_of[patches]
        assert h * w == patches
        x = np.zeros((patches, 1))
        merged = O.merge2x2(x, [(h, w)]).shape[0]
        assert merged + p["text_tokens"] == llm_tokens
    assert O.merge2x2(np.zeros((6256, 1)), [(46, 136)]).shape[0] == p["full_image_vision_tokens"]
    # the varlen batch of the three capped sizes
    grids = synth.grids_of(4)
    assert list(O.cu_seqlens_from_grids(grids)) == [0, 972, 4860, 6684]


def _small_block(cfg=0, idx=0):
    return synth.block_params(cfg, idx)


def _x(T, cfg=0):
    return synth.bf16_bits_to_f64(synth.normal_bf16(cfg, "x", 0, (T, 1152)))


def test_block_with_zero_weights_is_identity():
    p = OI.zero_like_block(_small_block(), keep=["ln1_g", "ln1_b", "ln2_g", "ln2_b"])
    w = OI.block_weights(p)
    grids = [(4, 4)]
    x = _x(16)
    y = O.block_forward(x, w, O.positions_from_grids(grids), O.cu_seqlens_from_grids(grids))
    assert np.array_equal(y, x)


def test_block_residual_wiring():
    # proj and fc2 zero: both branches add exactly their bias
    p = _small_block()
    p = dict(p)
    for n in ("proj_w", "fc2_w"):
        p[n] = np.zeros_like(p[n])
    w = OI.block_weights(p)
    grids = [(4, 4)]
    x = _x(16)
    y = O.block_forward(x, w, O.positions_from_grids(grids), O.cu_seqlens_from_grids(grids))
    x1 = O.bf16(x + w.proj_b)
    assert np.array_equal(y, O.bf16(x1 + w.fc2_b))


def test_block_varlen_packed_equals_separate():
    w = OI.block_weights(_small_block())
    grids = [(2, 4), (4, 6)]
    T = 32
    x = _x(T)
    packed = O.block_forward(x, w, O.positions_from_grids(grids), O.cu_seqlens_from_grids(grids))
    a = O.block_forward(x[:8], w, O.positions_from_grids(grids[:1]), [0, 8])
    b = O.block_forward(x[8:], w, O.positions_from_grids(grids[1:]), [0, 24])
    assert np.array_equal(packed, np.concatenate([a, b]))


def test_block_storage_vs_pure_close():
    w = OI.block_weights(_small_block())
    grids = [(4, 4)]
    x = _x(16)
    pos, cu = O.positions_from_grids(grids), O.cu_seqlens_from_grids(grids)
    tr = {}
    a = O.block_forward(x, w, pos, cu, "storage", trace=tr)
    b = O.block_forward(x, w, pos, cu, "pure")
    assert np.abs(a - b).max() / np.abs(b).max() < 2e-2
    # quantised FC1 activations carry the FP8 zero padding 4304..4351
    assert tr["h_codes"].shape == (16, 4352) and np.all(tr["h_codes"][:, 4304:] == 0)


# ---- precision variants: bf16 blocks (FlashRT section 4), FP8 mergers
# (FlashRT section 1)

def _cos_rel(a, b):
    a, b = np.ravel(a), np.ravel(b)
    return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b)), float(np.abs(a - b).max() / np.abs(b).max())


def test_bf16_block_with_zero_weights_is_identity():
    p = OI.zero_like_block(_small_block(), keep=["ln1_g", "ln1_b", "ln2_g", "ln2_b"])
    w = OI.block_weights(p)
    grids = [(4, 4)]
    x = _x(16)
    y = O.block_forward_bf16(x, w, O.positions_from_grids(grids), O.cu_seqlens_from_grids(grids))
    assert np.array_equal(y, x)


def test_bf16_block_residual_wiring():
    # proj and fc2 zero: both branches add exactly their bias
    p = dict(_small_block())
    for n in ("proj_w", "fc2_w"):
        p[n] = np.zeros_like(p[n])
    w = OI.block_weights(p)
    grids = [(4, 4)]
    x = _x(16)
    y = O.block_forward_bf16(x, w, O.positions_from_grids(grids), O.cu_seqlens_from_grids(grids))
    assert np.array_equal(y, O.bf16(O.bf16(x + w.proj_b) + w.fc2_b))


def test_bf16_block_varlen_packed_equals_separate():
    w = OI.block_weights(_small_block())
    grids = [(2, 4), (4, 6)]
    x = _x(32)
    packed = O.block_forward_bf16(x, w, O.positions_from_grids(grids), O.cu_seqlens_from_grids(grids))
    a = O.block_forward_bf16(x[:8], w, O.positions_from_grids(grids[:1]), [0, 8])
    b = O.block_forward_bf16(x[8:], w, O.positions_from_grids(grids[1:]), [0, 24])
    assert np.array_equal(packed, np.concatenate([a, b]))


def test_bf16_block_agrees_with_fp8_block():
    # The two precisions compute the same block: their updates x2 - x agree
    # to within FP8 quantisation noise (a dropped or mis-signed term in
    # either path would not).  Larger weights make the update visible.
    p = dict(_small_block())
    for n in ("qkv_w", "proj_w", "fc1_w", "fc2_w"):
        p[n] = synth.normal_bf16(0, n, 99, p[n].shape, std=0.05)
    w = OI.block_weights(p)
    grids = [(4, 8)]
    x = _x(32)
    pos, cu = O.positions_from_grids(grids), O.cu_seqlens_from_grids(grids)
    p16 = O.block_forward_bf16(x, w, pos, cu, "pure")
    d16 = p16 - x
    d8 = O.block_forward(x, w, pos, cu, "pure") - x
    # E4M3 keeps 3 mantissa bits: four quantised GEMMs put about 10 % rms
    # noise on the update
    cos, _ = _cos_rel(d8, d16)
    rms = float(np.linalg.norm(d8 - d16) / np.linalg.norm(d16))
    assert cos > 0.99 and rms < 0.15, (cos, rms)
    # the bf16 storage points move the block output by bf16 rounding only
    s16 = O.block_forward_bf16(x, w, pos, cu, "storage")
    assert np.abs(s16 - p16).max() / np.abs(p16).max() < 2e-2


def test_fp8_merger_zero_weights_gives_bias():
    m = OI.merger_weights(synth.merger_params(0, 0))
    m.fc1_w = np.zeros_like(m.fc1_w)
    m.fc2_w = np.zeros_like(m.fc2_w)
    grids = [(2, 4)]
    x = _x(8)
    y = O.merger_forward(x, m, grids, fp8=True)
    assert np.array_equal(y, np.broadcast_to(O.bf16(m.fc2_b), (2, 4096)))


def test_fp8_merger_agrees_with_bf16_merger():
    m = OI.merger_weights(synth.merger_params(0, 0))
    grids = [(4, 4), (2, 6)]
    x = _x(28)
    y8 = O.merger_forward(x, m, grids, "pure", fp8=True)
    y16 = O.merger_forward(x, m, grids, "pure")
    # the bias dominates the synthetic merger output: compare without it
    d8, d16 = y8 - m.fc2_b, y16 - m.fc2_b
    cos, _ = _cos_rel(d8, d16)
    rms = float(np.linalg.norm(d8 - d16) / np.linalg.norm(d16))
    assert cos > 0.99 and rms < 0.15, (cos, rms)


def test_encoder_precision_variants_route_blocks_and_mergers():
    ep = synth.EncoderParams(patch=synth.patch_params(0),
                             blocks=[synth.block_params(0, b) for b in range(4)],
                             mergers=[synth.merger_params(0, m) for m in range(2)])
    W = OI.encoder_weights(ep)
    grids = [(2, 4)]
    px = synth.pixels(0, 8).astype(np.float64)
    pos, cu = O.positions_from_grids(grids), O.cu_seqlens_from_grids(grids)
    tr = {}
    out, last = O.encoder_forward(px, W, grids, depth=4, taps=(1, 4), trace=tr, bf16_blocks=2, fp8_mergers=True)
    assert np.array_equal(tr["x1"], O.block_forward_bf16(tr["x0"], W.blocks[0], pos, cu))
    assert np.array_equal(tr["x2"], O.block_forward_bf16(tr["x1"], W.blocks[1], pos, cu))
    assert np.array_equal(tr["x3"], O.block_forward(tr["x2"], W.blocks[2], pos, cu))
    assert np.array_equal(out[0], O.merger_forward(tr["x1"], W.mergers[0], grids, fp8=True))
    assert np.array_equal(out[1], O.merger_forward(tr["x4"], W.mergers[1], grids, fp8=True))


def test_encoder_taps_are_block_outputs():
    # Short tower (depth 4, taps after blocks 1 and 4) built from the same
    # functions; the taps must be the mergers of those blocks' outputs.
    ep = synth.EncoderParams(patch=synth.patch_params(0),
                             blocks=[synth.block_params(0, b) for b in range(4)],
                             mergers=[synth.merger_params(0, m) for m in range(2)])
    W = OI.encoder_weights(ep)
    grids = [(2, 4)]
    px = synth.pixels(0, 8).astype(np.float64)
    tr = {}
    out, last = O.encoder_forward(px, W, grids, depth=4, taps=(1, 4), trace=tr)
    assert out.shape == (2, 2, 4096)
    assert np.array_equal(out[0], O.merger_forward(tr["x1"], W.mergers[0], grids))
    assert np.array_equal(out[1], O.merger_forward(tr["x4"], W.mergers[1], grids))
    assert np.array_equal(last, tr["x4"])
    # the patch embed is the bf16 GEMM of bf16-rounded pixels
    assert np.array_equal(tr["x0"], O.bf16(O.bf16(px) @ W.patch_w.T + W.patch_b))


def test_flop_counts():
    f = O.encoder_flops([6256])
    assert abs(f["attention"] / 1e9 - 4869.3) < 0.1
    assert abs(f["gemm"] / 1e9 - 5143.3) < 0.1
    assert abs(f["total"] / 1e9 - 10536.6) < 0.2
