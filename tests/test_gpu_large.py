"""GPU parity at the largest sizes the entry points accept and with many
attention windows.

* A block over 1,048,576 tokens (4096 images of 16 x 16): the qkv rows of
  the attention pass 2^32 bytes from token 621,378 and the FC2 operand
  offsets pass 2^32 from token 986,895.  The input is one seeded 8-image
  batch repeated on the device; images are independent (per-token FP8
  scales, per-window attention), so every copy must match the oracle's
  output for the base batch.
* The patch-embed GEMM (fp32 pixels, K = 1536) over 2,883,584 rows, whose
  operand offsets pass 2^32 elements from row 2,796,203.
* Attention over 300 windows of mixed length with empty windows between
  and after them: the stream-K ranges start and continue across many
  windows and across heads.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth
import vision_transformer_encoder_amd as vit
from oracle import inputs as OI
from gpu_util import announce, assert_close, dev_bf16, host_f64

pytestmark = pytest.mark.gpu

MAX_REL, MIN_COS = 2e-2, 0.9995


def _copies_close(got: torch.Tensor, ref: np.ndarray, copies, what, max_rel, min_cos):
    """got: [copies * R, C] bf16 on the device; ref: [R, C] float64.  The
    sampled copies are compared on the host; every copy's max abs error is
    computed on the device against the same bound."""
    R = ref.shape[0]
    scale = np.abs(ref).max()
    for c in copies:
        assert_close(host_f64(got[c * R:(c + 1) * R]), ref, max_rel, min_cos, f"{what} copy {c}")
    ref_dev = torch.from_numpy(ref.astype(np.float32)).to(got.device)
    n = got.shape[0] // R
    worst = 0.0
    for c0 in range(0, n, 64):
        c1 = min(n, c0 + 64)
        d = (got[c0 * R:c1 * R].float().view(c1 - c0, R, -1) - ref_dev[None]).abs().amax(dim=(1, 2))
        worst = max(worst, float(d.max()))
    announce(f"{what}: max abs error over all {n} copies {worst:.3e} (bound {max_rel * scale:.3e})")
    assert worst <= max_rel * scale


def test_block_one_million_tokens(gpu):
    base = [(16, 16)] * 8
    Tb = 2048
    copies = 512
    T = Tb * copies
    params = synth.block_params(0, 3)
    xb = synth.normal_bf16(0, "x", 77, (Tb, 1152))
    w = vit.BlockWeights(params, gpu)
    announce(f"vit_block_forward T={T} ({copies * 8} images of 16x16)")
    x = dev_bf16(xb, gpu).repeat(copies, 1)
    pos = torch.from_numpy(synth.positions(base)).to(gpu).repeat(copies, 1)
    cu = (np.arange(copies * 8 + 1) * 256).astype(np.int32)
    vit.vit_block_forward(w, x, pos, cu)
    torch.cuda.synchronize()
    ref = O.block_forward(synth.bf16_bits_to_f64(xb), OI.block_weights(params), synth.positions(base),
                          synth.cu_seqlens(base))
    # copy 303 holds token 621,378, copy 482 lies past token 986,895
    _copies_close(x, ref, [0, 303, 482, copies - 1], "block T=1048576", MAX_REL, MIN_COS)
    del x
    torch.cuda.empty_cache()


def test_patch_embed_past_2e32_operand_elements(gpu):
    Mb = 1024
    copies = 2816
    M = Mb * copies
    p = synth.patch_params(0)
    px = synth.pixels(5, Mb)
    announce(f"vit_bf16_gemm fp32 A M={M} K=1536")
    a = torch.from_numpy(px).to(gpu).repeat(copies, 1)
    wt = dev_bf16(p["patch_w"], gpu)
    bias = dev_bf16(p["patch_b"], gpu)
    out = vit.vit_bf16_gemm(a, wt, bias=bias, epilogue=vit.BEPI_BIAS)
    torch.cuda.synchronize()
    del a
    ref = O.bf16(O.bf16_gemm(O.bf16(px.astype(np.float64)), synth.bf16_bits_to_f64(p["patch_w"]),
                             synth.bf16_bits_to_f64(p["patch_b"])))
    # copy 2731 lies past row 2,796,203
    _copies_close(out, ref, [0, 2731, copies - 1], "patch embed M=2883584", 1e-2, 0.99999)
    del out
    torch.cuda.empty_cache()


def test_attention_many_windows_with_empty_ones(gpu):
    g = np.random.default_rng(21)
    lens = g.integers(1, 400, size=300)
    lens[::17] = 0          # empty windows between others
    lens[-3:] = 0           # and after the last one
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    qb, kb, vb = [synth.normal_bf16(1, t, 31, (T, 1152)) for t in ("q", "k", "v")]
    qkv = torch.cat([dev_bf16(qb, gpu), dev_bf16(kb, gpu), dev_bf16(vb, gpu)], dim=1).contiguous()
    announce(f"vit_attention {len(lens)} windows ({int((lens == 0).sum())} empty), T={T}")
    o = host_f64(vit.vit_attention(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], cu))
    ref = O.attention(*(synth.bf16_bits_to_f64(b) for b in (qb, kb, vb)), cu)
    assert_close(o, ref, MAX_REL, MIN_COS, "attention, 300 windows")
