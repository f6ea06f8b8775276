"""GPU parity of the 2x2 merge + LayerNorm, of one ViT block and of the whole
27-block tower with its four DeepStack/final mergers, against the
storage-emulating fp64 oracle (bf16 at the same storage points, FP8 codes
from the same quantiser)."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
import vision_transformer_encoder_amd as vit
from oracle import inputs as OI
from gpu_util import announce, assert_close, check_within, dev_bf16, host_f64, implementation_noise, metrics

pytestmark = pytest.mark.gpu

MAX_REL, MIN_COS = 2e-2, 0.9995


@pytest.mark.parametrize("grids", [[(46, 136)], [(18, 54), (36, 108), (24, 76)], [(2, 2), (4, 6)]],
                         ids=["p6256", "varlen", "tiny"])
def test_merge_layernorm(gpu, grids):
    T = sum(h * w for h, w in grids)
    x = synth.normal_bf16(3, "x", T, (T, 1152))
    g = synth.normal_bf16(3, "m_ln_g", 0, (4608,), std=0.02, mean=1.0)
    b = synth.normal_bf16(3, "m_ln_b", 0, (4608,), std=0.01)
    announce(f"vit_merge2x2_layernorm T={T}")
    out = vit.vit_merge2x2_layernorm(dev_bf16(x, gpu), grids, dev_bf16(g, gpu), dev_bf16(b, gpu))
    ref = O.bf16(O.layernorm(O.merge2x2(synth.bf16_bits_to_f64(x), grids), synth.bf16_bits_to_f64(g),
                             synth.bf16_bits_to_f64(b)))
    assert_close(host_f64(out), ref, 1e-2, 0.99999, f"merge+LN T={T}")


def _block_case(gpu, cfg, grids, block_index=0):
    T = sum(h * w for h, w in grids)
    params = synth.block_params(cfg, block_index)
    x_bits = synth.normal_bf16(cfg, "x", block_index, (T, 1152))
    return T, params, x_bits


@pytest.mark.parametrize("cfg,grids", [(0, [(16, 16)]), (4, [(18, 54), (36, 108), (24, 76)]), (3, [(46, 136)])],
                         ids=["p256", "varlen_6684", "p6256"])
def test_block_parity(gpu, cfg, grids):
    T, params, x_bits = _block_case(gpu, cfg, grids)
    announce(f"vit_block_forward cfg={cfg} T={T}")
    w = vit.BlockWeights(params, gpu)
    x = dev_bf16(x_bits, gpu).clone()
    pos = torch.from_numpy(synth.positions(grids)).to(gpu)
    cu = synth.cu_seqlens(grids)
    vit.vit_block_forward(w, x, pos, cu)
    torch.cuda.synchronize()
    got = host_f64(x)
    ow = OI.block_weights(params)
    ref = O.block_forward(synth.bf16_bits_to_f64(x_bits), ow, synth.positions(grids), cu)
    # the device weight codes are the oracle's, bit for bit
    for n in ("qkv", "proj", "fc1", "fc2"):
        assert np.array_equal(w.q[n][0].cpu().numpy(), ow.fp8(n).codes), n
    assert_close(got, ref, MAX_REL, MIN_COS, f"block T={T}")
    # the residual stream carries most of the output: compare the update too.
    # The update goes through the FP8 requantisation of the bf16 attention
    # output and of the LayerNorm / GELU outputs, where rounding-level
    # differences flip codes; it is held to the stated tolerance or to twice
    # the oracle's own drift under implementation-size noise, whichever is
    # wider (the rule of the free-running tower).
    x0 = synth.bf16_bits_to_f64(x_bits)
    with implementation_noise(7):
        noisy = O.block_forward(x0, ow, synth.positions(grids), cu)
    check_within(got - x0, ref - x0, metrics(noisy - x0, ref - x0), f"block update T={T}")


def test_block_deterministic_and_packed_matches_separate(gpu):
    grids = [(18, 54), (24, 76)]
    T, params, x_bits = _block_case(gpu, 4, grids, block_index=2)
    w = vit.BlockWeights(params, gpu)
    cu = synth.cu_seqlens(grids)
    pos = torch.from_numpy(synth.positions(grids)).to(gpu)
    x1 = dev_bf16(x_bits, gpu).clone()
    x2 = dev_bf16(x_bits, gpu).clone()
    vit.vit_block_forward(w, x1, pos, cu)
    vit.vit_block_forward(w, x2, pos, cu)
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16)), "two runs differ"
    a = int(cu[1])
    xa = dev_bf16(x_bits[:a], gpu).clone()
    xb = dev_bf16(x_bits[a:], gpu).clone()
    vit.vit_block_forward(w, xa, pos[:a].contiguous(), [0, a])
    vit.vit_block_forward(w, xb, pos[a:].contiguous(), [0, T - a])
    # the attention's stream-K split depends on the whole packing, so packed
    # and separate runs differ by fp32 rounding of the attention output,
    # which the FP8 requantisation before the projection can turn into
    # one-code flips: held to the block-update bound of the oracle parity test
    x0 = synth.bf16_bits_to_f64(x_bits)
    upd_packed = host_f64(x1) - x0
    upd_sep = np.concatenate([host_f64(xa), host_f64(xb)]) - x0
    assert_close(upd_packed, upd_sep, 5e-2, 0.999, "block packed vs separate (update)")


def test_block_zero_weights_identity(gpu):
    grids = [(16, 16)]
    T, params, x_bits = _block_case(gpu, 0, grids, block_index=5)
    p = OI.zero_like_block(params, keep=["ln1_g", "ln1_b", "ln2_g", "ln2_b"])
    w = vit.BlockWeights(p, gpu)
    x = dev_bf16(x_bits, gpu).clone()
    vit.vit_block_forward(w, x, torch.from_numpy(synth.positions(grids)).to(gpu), synth.cu_seqlens(grids))
    assert torch.equal(x.view(torch.int16), dev_bf16(x_bits, gpu).view(torch.int16))


@pytest.mark.parametrize("grids", [[(6, 8), (12, 21)], [(18, 54), (36, 108), (24, 76)]], ids=["two_images_300",
                                                                                              "varlen_6684"])
def test_block_forward_bit_exact_with_its_entry_points(gpu, grids):
    """The FP8 block forward is the chain of its C-ABI steps, byte for byte:
    LayerNorm-quant, QKV GEMM, RoPE, attention, row quantisation, projection
    + residual, LayerNorm-quant, FC1 + GELU-quant, FC2 + residual."""
    T = sum(h * w for h, w in grids)
    params = synth.block_params(4, 1)
    w = vit.BlockWeights(params, gpu)
    t = w.t
    x_bits = synth.normal_bf16(4, "x", 1, (T, 1152))
    pos = torch.from_numpy(synth.positions(grids)).to(gpu)
    cu = synth.cu_seqlens(grids)
    cu_dev = torch.from_numpy(cu).to(gpu)
    announce(f"vit_block_forward vs its entry points T={T}")
    x_blk = dev_bf16(x_bits, gpu).clone()
    vit.vit_block_forward(w, x_blk, pos, cu, cu_seqlens_dev=cu_dev)

    x = dev_bf16(x_bits, gpu).clone()
    c1, s1 = vit.vit_layernorm_quant_fp8(x, t["ln1_g"], t["ln1_b"])
    qkv = vit.vit_fp8_block128_gemm(c1, s1, w.q["qkv"][0], w.q["qkv"][1], 3456, 1152, bias=t["qkv_b"])
    vit.vit_rope2d(qkv[:, :1152], qkv[:, 1152:2304], pos)
    # the block's softmax scale is the fp32 1 / sqrtf(72), one ulp above the
    # binding's default (1 / sqrt(72) rounded from double)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(72.0)))
    o = vit.vit_attention(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], cu, cu_seqlens_dev=cu_dev,
                          softmax_scale=scale)
    oc, os_ = vit.vit_quant_fp8_block128(o, block_rows=1)
    vit.vit_fp8_block128_gemm(oc, os_, w.q["proj"][0], w.q["proj"][1], 1152, 1152, bias=t["proj_b"], residual=x,
                              epilogue=vit.EPI_BIAS_RESIDUAL, out=x)
    c2, s2 = vit.vit_layernorm_quant_fp8(x, t["ln2_g"], t["ln2_b"])
    hc, hs = vit.vit_fp8_block128_gemm(c2, s2, w.q["fc1"][0], w.q["fc1"][1], 4304, 1152, bias=t["fc1_b"],
                                       epilogue=vit.EPI_BIAS_GELU_FP8)
    vit.vit_fp8_block128_gemm(hc, hs, w.q["fc2"][0], w.q["fc2"][1], 1152, 4304, bias=t["fc2_b"], residual=x,
                              epilogue=vit.EPI_BIAS_RESIDUAL, out=x)
    torch.cuda.synchronize()
    n = int((x_blk.view(torch.int16) != x.view(torch.int16)).sum())
    assert n == 0, f"block forward and its entry points differ in {n} of {x.numel()} elements"


@pytest.fixture(scope="module")
def small_tower(gpu):
    ep = synth.encoder_params(0)
    return ep, vit.EncoderWeights(ep.patch, ep.blocks, ep.mergers, gpu)


@pytest.fixture(scope="module")
def oracle_tower():
    ow = OI.encoder_weights(synth.encoder_params(0))
    for b in ow.blocks:  # quantise once for every test of the module
        for n in ("qkv", "proj", "fc1", "fc2"):
            b.fp8(n)
    return ow


def _gpu_merger(W, m, x_dev, grids):
    """One merger through the C ABI: merge + LayerNorm, fc1 + GELU, fc2."""
    t = W.mergers[m].t
    y = vit.vit_merge2x2_layernorm(x_dev, grids, t["m_ln_g"], t["m_ln_b"])
    h = vit.vit_bf16_gemm(y, t["m_fc1_w"], bias=t["m_fc1_b"], epilogue=vit.BEPI_BIAS_GELU)
    return vit.vit_bf16_gemm(h, t["m_fc2_w"], bias=t["m_fc2_b"], epilogue=vit.BEPI_BIAS)


def test_encoder_parity_small(gpu, small_tower, oracle_tower):
    """Whole tower, all 27 blocks and 4 mergers, on two small images:
    (1) teacher-forced: every GPU block and merger fed the oracle's input;
    (2) free-running whole tower.  Each is held to the stated tolerance or,
    where the oracle's own implementation-noise envelope is wider, to twice
    that."""
    from gpu_util import metrics
    ep, W = small_tower
    grids = [(8, 8), (4, 6)]
    T = sum(h * w for h, w in grids)
    px = synth.pixels(0, T)
    pos = torch.from_numpy(synth.positions(grids)).to(gpu)
    cu = synth.cu_seqlens(grids)
    opos, ocu = synth.positions(grids), synth.cu_seqlens(grids)
    tr = {}
    ref_out, ref_last = O.encoder_forward(px.astype(np.float64), oracle_tower, grids, trace=tr)
    # (1) teacher-forced, block by block and merger by merger
    for b in range(1, 28):
        x = torch.from_numpy(tr[f"x{b - 1}"]).to(gpu).to(torch.bfloat16)
        vit.vit_block_forward(W.blocks[b - 1], x, pos, cu)
        with implementation_noise(b):
            xe = O.block_forward(tr[f"x{b - 1}"], oracle_tower.blocks[b - 1], opos, ocu)
        check_within(host_f64(x), tr[f"x{b}"], metrics(xe, tr[f"x{b}"]), f"block {b} teacher-forced")
    for m, tap in enumerate((8, 16, 24, 27)):
        x = torch.from_numpy(tr[f"x{tap}"]).to(gpu).to(torch.bfloat16)
        assert_close(host_f64(_gpu_merger(W, m, x, grids)), ref_out[m], MAX_REL, MIN_COS,
                     f"merger {m} teacher-forced")
    # (2) free-running whole tower
    announce(f"vit_encoder_forward T={T}")
    out, last = vit.vit_encoder_forward(W, torch.from_numpy(px).to(gpu), grids, want_last_hidden=True)
    torch.cuda.synchronize()
    with implementation_noise(100):
        eo, el = O.encoder_forward(px.astype(np.float64), oracle_tower, grids)
    got = host_f64(out)
    for i, name in enumerate(("deepstack8", "deepstack16", "deepstack24", "final")):
        check_within(got[i], ref_out[i], metrics(eo[i], ref_out[i]), f"free-running {name}")
    check_within(host_f64(last), ref_last, metrics(el, ref_last), "free-running last hidden")


def test_encoder_pos_embed_and_workspace_reuse(gpu, small_tower, oracle_tower):
    ep, W = small_tower
    grids = [(4, 4)]
    T = 16
    px = torch.from_numpy(synth.pixels(1, T)).to(gpu)
    pos = dev_bf16(synth.normal_bf16(1, "pos_embed", 0, (T, 1152)), gpu)
    ws = torch.empty(vit.vit_encoder_workspace_size(T, 1), dtype=torch.uint8, device=gpu)
    ws.fill_(0x7F)  # workspace contents on entry must not matter
    o1, _ = vit.vit_encoder_forward(W, px, grids, pos_embed=pos, workspace=ws)
    ws.fill_(0xFF)
    o2, _ = vit.vit_encoder_forward(W, px, grids, pos_embed=pos, workspace=ws)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    o3, _ = vit.vit_encoder_forward(W, px, grids)
    assert not torch.equal(o1.view(torch.int16), o3.view(torch.int16)), "position table had no effect"
    # the position table enters through the patch-embed epilogue: check x0
    x0 = torch.empty((T, 1152), dtype=torch.bfloat16, device=gpu)
    vit.vit_bf16_gemm(px, W.patch["patch_w"], bias=W.patch["patch_b"], add=pos, epilogue=vit.BEPI_BIAS_ADD, out=x0)
    ref0 = O.patch_embed(synth.pixels(1, T).astype(np.float64), oracle_tower, pos_embed=host_f64(pos))
    assert_close(host_f64(x0), ref0, 1e-2, 0.99999, "patch embed + position table")
