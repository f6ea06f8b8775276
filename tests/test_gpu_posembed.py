"""GPU parity of the interpolated position embedding (vit_pos_embed_interp)
against the oracle, bit for bit (both evaluate the same f32 operations in
the same order and round once to bf16), and its use inside the tower: the
encoder given the learned table equals the encoder given the resampled
table as a precomputed input, and the whole tower stays within the oracle's
noise envelope."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
import vision_transformer_encoder_amd as vit
from gpu_util import announce, check_within, dev_bf16, host_f64, implementation_noise, metrics

pytestmark = pytest.mark.gpu


def _table(G=O.POS_GRID, D=1152, cfg=4):
    return synth.normal_bf16(cfg, "pos_table", G, (G * G, D), std=0.02)


@pytest.mark.parametrize("grids", [[(46, 136)], [(48, 48)], [(18, 54), (36, 108), (24, 76)],
                                   [(1, 1), (3, 5), (2, 97), (96, 1)]],
                         ids=["46x136", "48x48", "varlen3", "ragged"])
def test_interp_bit_exact(gpu, grids):
    bits = _table()
    T = sum(h * w for h, w in grids)
    announce(f"vit_pos_embed_interp G=48 D=1152 T={T} grids={grids}")
    got = vit.vit_pos_embed_interp(dev_bf16(bits, gpu), grids)
    ref = O.pos_embed_interp(synth.bf16_bits_to_f64(bits), grids)
    g = host_f64(got)
    assert g.shape == ref.shape
    assert np.array_equal(g, ref), f"{int((g != ref).sum())} of {ref.size} values differ"


def test_interp_rows_wider_than_8192(gpu):
    # more than 16 chunks per lane: the one-chunk-per-trip variant
    G, D = 3, 8200
    bits = _table(G, D, cfg=6)
    grids = [(2, 3), (1, 4)]
    announce(f"vit_pos_embed_interp G={G} D={D} grids={grids}")
    got = vit.vit_pos_embed_interp(dev_bf16(bits, gpu), grids)
    ref = O.pos_embed_interp(synth.bf16_bits_to_f64(bits), grids, grid_side=G)
    g = host_f64(got)
    assert np.array_equal(g, ref), f"{int((g != ref).sum())} of {ref.size} values differ"


def test_interp_other_table_and_strided_output(gpu):
    G, D = 7, 64
    bits = _table(G, D, cfg=5)
    grids = [(10, 3), (2, 2)]
    T = 34
    wide = torch.zeros((T, 96), dtype=torch.bfloat16, device=gpu)
    announce("vit_pos_embed_interp G=7 D=64 into columns 0..63 of a [34, 96] buffer")
    vit.vit_pos_embed_interp(dev_bf16(bits, gpu), grids, out=wide[:, :D])
    ref = O.pos_embed_interp(synth.bf16_bits_to_f64(bits), grids, grid_side=G)
    w = host_f64(wide)
    assert np.array_equal(w[:, :D], ref)
    assert np.all(w[:, D:] == 0), "columns past dim must be untouched"


def test_encoder_with_learned_table(gpu):
    ep = synth.encoder_params(0)
    bits = _table()
    W = vit.EncoderWeights(ep.patch, ep.blocks, ep.mergers, gpu, pos_table=bits)
    grids = [(8, 8), (4, 6)]
    T = sum(h * w for h, w in grids)
    px_h = synth.pixels(0, T)
    px = torch.from_numpy(px_h).to(gpu)
    announce(f"vit_encoder_forward with the 48x48 table, T={T}")
    out_t, last_t = vit.vit_encoder_forward(W, px, grids, want_last_hidden=True)
    # the same forward with the resampled table passed in as an input
    pos = vit.vit_pos_embed_interp(W.pos_table, grids)
    W_plain = vit.EncoderWeights(ep.patch, ep.blocks, ep.mergers, gpu)
    out_p, last_p = vit.vit_encoder_forward(W_plain, px, grids, pos_embed=pos, want_last_hidden=True)
    out_n, _ = vit.vit_encoder_forward(W_plain, px, grids)
    torch.cuda.synchronize()
    assert torch.equal(out_t.view(torch.int16), out_p.view(torch.int16))
    assert torch.equal(last_t.view(torch.int16), last_p.view(torch.int16))
    assert not torch.equal(out_t.view(torch.int16), out_n.view(torch.int16)), "the table had no effect"
    # whole tower against the oracle, within its noise envelope
    import oracle.inputs as OI
    ow = OI.encoder_weights(ep)
    opos = O.pos_embed_interp(synth.bf16_bits_to_f64(bits), grids)
    ref_out, ref_last = O.encoder_forward(px_h.astype(np.float64), ow, grids, pos_embed=opos)
    with implementation_noise(200):
        eo, el = O.encoder_forward(px_h.astype(np.float64), ow, grids, pos_embed=opos)
    got = host_f64(out_t)
    for i, name in enumerate(("deepstack8", "deepstack16", "deepstack24", "final")):
        check_within(got[i], ref_out[i], metrics(eo[i], ref_out[i]), f"tower with table {name}")
    check_within(host_f64(last_t), ref_last, metrics(el, ref_last), "tower with table last hidden")
