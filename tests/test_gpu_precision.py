"""GPU parity of the precision variants against the oracle's: blocks that run
LayerNorm and their GEMMs in bf16 (the FlashRT page, section 4, keeps the
first 3 blocks so) and mergers that run their linears as block-scaled FP8
GEMMs ("merger FP8", section 1)."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
import vision_transformer_encoder_amd as vit
from oracle import inputs as OI
from gpu_util import announce, assert_close, check_within, dev_bf16, host_f64, host_u8, implementation_noise, metrics

pytestmark = pytest.mark.gpu

MAX_REL, MIN_COS = 2e-2, 0.9995


@pytest.mark.parametrize("M,D", [(6256, 1152), (300, 4608), (1, 128)])
def test_layernorm_bf16(gpu, M, D):
    x = synth.normal_bf16(3, "x", 7, (M, D))
    g = synth.normal_bf16(3, "ln1_g", 7, (D,), std=0.02, mean=1.0)
    b = synth.normal_bf16(3, "ln1_b", 7, (D,), std=0.01)
    announce(f"vit_layernorm M={M} D={D}")
    out = vit.vit_layernorm(dev_bf16(x, gpu), dev_bf16(g, gpu), dev_bf16(b, gpu))
    ref = O.bf16(O.layernorm(synth.bf16_bits_to_f64(x), synth.bf16_bits_to_f64(g), synth.bf16_bits_to_f64(b)))
    # fp32 statistics against fp64: results differ only where bf16 rounding ties break
    assert_close(host_f64(out), ref, 2.0 ** -7, 0.99999, f"layernorm bf16 M={M} D={D}")


@pytest.mark.parametrize("cfg,grids", [(0, [(16, 16)]), (4, [(18, 54), (36, 108), (24, 76)])],
                         ids=["p256", "varlen_6684"])
def test_block_bf16_parity(gpu, cfg, grids):
    T = sum(h * w for h, w in grids)
    params = synth.block_params(cfg, 0)
    x_bits = synth.normal_bf16(cfg, "x", 0, (T, 1152))
    announce(f"vit_block_forward bf16 cfg={cfg} T={T}")
    w = vit.BlockWeights(params, gpu, precision="bf16")
    x = dev_bf16(x_bits, gpu).clone()
    pos = torch.from_numpy(synth.positions(grids)).to(gpu)
    vit.vit_block_forward(w, x, pos, synth.cu_seqlens(grids))
    torch.cuda.synchronize()
    got = host_f64(x)
    x0 = synth.bf16_bits_to_f64(x_bits)
    ref = O.block_forward_bf16(x0, OI.block_weights(params), synth.positions(grids), synth.cu_seqlens(grids))
    assert_close(got, ref, MAX_REL, MIN_COS, f"bf16 block T={T}")
    # the residual stream carries most of the output: compare the update too
    # (no FP8 requantisation here, so it meets the stated tolerance itself)
    assert_close(got - x0, ref - x0, 2e-2, 0.9995, f"bf16 block update T={T}")


def test_fp8_merger_parity(gpu):
    """The FP8 merger as the library runs it (merge + LayerNorm, per-token
    quant, fc1 + GELU + requant, fc2), one C-ABI call per step."""
    grids = [(46, 136)]
    T = 6256
    mp = synth.merger_params(3, 0)
    W = vit.MergerWeights(mp, gpu, precision="fp8")
    om = OI.merger_weights(mp)
    for n in ("fc1", "fc2"):  # the device weight codes are the oracle's, bit for bit
        assert np.array_equal(host_u8(W.q[n][0]), om.fp8(n).codes), n
    x_bits = synth.normal_bf16(3, "x", 3, (T, 1152))
    announce(f"FP8 merger T={T}")
    t = W.t
    y = vit.vit_merge2x2_layernorm(dev_bf16(x_bits, gpu), grids, t["m_ln_g"], t["m_ln_b"])
    a_c, a_s = vit.vit_quant_fp8_block128(y)
    h_c, h_s = vit.vit_fp8_block128_gemm(a_c, a_s, W.q["fc1"][0], W.q["fc1"][1], 4608, 4608, bias=t["m_fc1_b"],
                                         epilogue=vit.EPI_BIAS_GELU_FP8)
    out = vit.vit_fp8_block128_gemm(h_c, h_s, W.q["fc2"][0], W.q["fc2"][1], 4096, 4608, bias=t["m_fc2_b"],
                                    epilogue=vit.EPI_BIAS)
    ref = O.merger_forward(synth.bf16_bits_to_f64(x_bits), om, grids, fp8=True)
    got = host_f64(out)
    assert_close(got, ref, MAX_REL, MIN_COS, "FP8 merger")
    assert_close(got - om.fc2_b, ref - om.fc2_b, 5e-2, 0.999, "FP8 merger without its bias")


def test_encoder_precision_variants(gpu):
    """The whole tower with the first 3 blocks in bf16 and FP8 mergers:
    teacher-forced blocks 1..4 (bf16, bf16, bf16, FP8), then the
    free-running tower, held like the all-FP8 tower to the stated tolerance
    or twice the oracle's implementation-noise envelope."""
    ep = synth.encoder_params(0)
    W = vit.EncoderWeights(ep.patch, ep.blocks, ep.mergers, gpu, bf16_blocks=3, fp8_mergers=True)
    ow = OI.encoder_weights(ep)
    grids = [(8, 8), (4, 6)]
    T = sum(h * w for h, w in grids)
    px = synth.pixels(0, T)
    pos = torch.from_numpy(synth.positions(grids)).to(gpu)
    cu = synth.cu_seqlens(grids)
    opos, ocu = synth.positions(grids), synth.cu_seqlens(grids)
    tr = {}
    ref_out, ref_last = O.encoder_forward(px.astype(np.float64), ow, grids, trace=tr, bf16_blocks=3,
                                          fp8_mergers=True)
    for b in range(1, 5):
        fwd = O.block_forward_bf16 if b <= 3 else O.block_forward
        x = torch.from_numpy(tr[f"x{b - 1}"]).to(gpu).to(torch.bfloat16)
        vit.vit_block_forward(W.blocks[b - 1], x, pos, cu)
        with implementation_noise(b):
            xe = fwd(tr[f"x{b - 1}"], ow.blocks[b - 1], opos, ocu)
        check_within(host_f64(x), tr[f"x{b}"], metrics(xe, tr[f"x{b}"]), f"block {b} teacher-forced")
    announce(f"vit_encoder_forward bf16_blocks=3 fp8_mergers T={T}")
    out, last = vit.vit_encoder_forward(W, torch.from_numpy(px).to(gpu), grids, want_last_hidden=True)
    torch.cuda.synchronize()
    with implementation_noise(200):
        eo, el = O.encoder_forward(px.astype(np.float64), ow, grids, bf16_blocks=3, fp8_mergers=True)
    got = host_f64(out)
    for i, name in enumerate(("deepstack8", "deepstack16", "deepstack24", "final")):
        check_within(got[i], ref_out[i], metrics(eo[i], ref_out[i]), f"free-running {name}")
    check_within(host_f64(last), ref_last, metrics(el, ref_last), "free-running last hidden")
