"""GPU parity of the block-scaled FP8 GEMM (all three epilogues) and of the
bf16 GEMM (patch embedding, merger MLP), on the tower's shapes at M = 6256
and on small ragged shapes."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
import vision_transformer_encoder_amd as vit
from gpu_util import announce, assert_close, dev_bf16, host_f64, host_u8

pytestmark = pytest.mark.gpu

TOL_GEMM = 1e-2


def _operands(gpu, M, N, K, seed):
    """Seeded bf16 activations / weights / bias / residual, quantised on the
    GPU (the quantisers are checked bit-exact elsewhere) and by the oracle."""
    a_bits = synth.normal_bf16(2, "a", seed, (M, K))
    w_bits = synth.normal_bf16(2, "w", seed, (N, K), std=0.02)
    b_bits = synth.normal_bf16(2, "bias", seed, (N,), std=0.01)
    r_bits = synth.normal_bf16(2, "residual", seed, (M, N))
    a_c, a_s = vit.vit_quant_fp8_block128(dev_bf16(a_bits, gpu), block_rows=1)
    w_c, w_s = vit.vit_quant_fp8_block128(dev_bf16(w_bits, gpu), block_rows=128)
    ra_c, ra_s = O.quantize_block128(synth.bf16_bits_to_f64(a_bits), 1)
    rw_c, rw_s = O.quantize_block128(synth.bf16_bits_to_f64(w_bits), 128)
    assert np.array_equal(host_u8(a_c), ra_c) and np.array_equal(host_u8(w_c), rw_c)
    return dict(a_c=a_c, a_s=a_s, w_c=w_c, w_s=w_s, b=dev_bf16(b_bits, gpu), r=dev_bf16(r_bits, gpu),
                C=O.fp8_block128_gemm(ra_c, ra_s, rw_c, rw_s),
                bf=synth.bf16_bits_to_f64(b_bits), rf=synth.bf16_bits_to_f64(r_bits))


SHAPES = [  # (name, M, N, K, epilogue)
    ("qkv", 6256, 3456, 1152, O.EPI_BIAS),
    ("proj", 6256, 1152, 1152, O.EPI_BIAS_RESIDUAL),
    ("fc1", 6256, 4304, 1152, O.EPI_BIAS_GELU_FP8),
    ("fc2", 6256, 1152, 4304, O.EPI_BIAS_RESIDUAL),
    ("ragged_a", 1, 128, 128, O.EPI_BIAS),
    ("ragged_b", 130, 200, 200, O.EPI_BIAS_RESIDUAL),
    ("ragged_c", 77, 130, 384, O.EPI_BIAS_GELU_FP8),
    ("ragged_d", 257, 256, 136, O.EPI_BIAS),
]


@pytest.mark.parametrize("name,M,N,K,epi", SHAPES, ids=[s[0] for s in SHAPES])
def test_fp8_gemm(gpu, name, M, N, K, epi):
    announce(f"vit_fp8_block128_gemm {name} M={M} N={N} K={K} epilogue={epi}")
    d = _operands(gpu, M, N, K, M + N + K)
    if epi == O.EPI_BIAS_GELU_FP8:
        codes, scales, pre = vit.vit_fp8_block128_gemm(d["a_c"], d["a_s"], d["w_c"], d["w_s"], N, K,
                                                       bias=d["b"], epilogue=epi, prequant=True)
        rc, rs, rpre = O.fp8_gemm_epilogue(d["C"], N, epi, bias=d["bf"])
        pre_h = host_f64(pre)
        assert_close(pre_h, rpre, TOL_GEMM, 0.9999, f"{name} prequant")
        assert np.all(pre_h[:, N:] == 0)
        gc, gs = O.quantize_block128(pre_h, 1)
        assert np.array_equal(host_u8(codes), gc), "codes differ from the oracle quantiser on GPU pre-quant"
        assert np.array_equal(host_f64(scales), gs)
    else:
        out = vit.vit_fp8_block128_gemm(d["a_c"], d["a_s"], d["w_c"], d["w_s"], N, K, bias=d["b"],
                                        residual=d["r"] if epi == O.EPI_BIAS_RESIDUAL else None, epilogue=epi)
        ref = O.fp8_gemm_epilogue(d["C"], N, epi, bias=d["bf"], residual=d["rf"])
        assert_close(host_f64(out), ref, TOL_GEMM, 0.9999, name)


def test_fp8_gemm_residual_in_place(gpu):
    M, N, K = 300, 1152, 1152
    d = _operands(gpu, M, N, K, 99)
    x = d["r"].clone()
    announce("vit_fp8_block128_gemm in-place residual")
    vit.vit_fp8_block128_gemm(d["a_c"], d["a_s"], d["w_c"], d["w_s"], N, K, bias=d["b"], residual=x,
                              epilogue=O.EPI_BIAS_RESIDUAL, out=x)
    ref = O.fp8_gemm_epilogue(d["C"], N, O.EPI_BIAS_RESIDUAL, bias=d["bf"], residual=d["rf"])
    assert_close(host_f64(x), ref, TOL_GEMM, 0.9999, "in-place residual")


def test_fp8_gemm_deterministic(gpu):
    d = _operands(gpu, 6256, 1152, 1152, 5)
    o1 = vit.vit_fp8_block128_gemm(d["a_c"], d["a_s"], d["w_c"], d["w_s"], 1152, 1152, bias=d["b"])
    o2 = vit.vit_fp8_block128_gemm(d["a_c"], d["a_s"], d["w_c"], d["w_s"], 1152, 1152, bias=d["b"])
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


BF16_SHAPES = [  # (name, M, N, K, a_f32, epilogue)
    ("patch_embed", 6256, 1152, 1536, True, 0),
    ("patch_embed_pos", 300, 1152, 1536, True, 2),
    ("merger_fc1", 1564, 4608, 4608, False, 1),
    ("merger_fc2", 1564, 4096, 4608, False, 0),
    ("ragged", 77, 130, 72, False, 1),
    # the 256-wide tile path (bf16 A, N % 256 == 0, K % 192 == 0): a ragged
    # last row tile, one round of three K steps, and no bias
    ("wide_ragged_m", 77, 512, 384, False, 1),
    ("wide_three_k_steps", 300, 256, 192, False, 0),
]


@pytest.mark.parametrize("name,M,N,K,a_f32,epi", BF16_SHAPES, ids=[s[0] for s in BF16_SHAPES])
def test_bf16_gemm(gpu, name, M, N, K, a_f32, epi):
    announce(f"vit_bf16_gemm {name} M={M} N={N} K={K} f32={a_f32} epilogue={epi}")
    seed = M + N + K
    if a_f32:
        a32 = synth.uniform_f32(3, "pixels", seed, (M, K), -1.0, 1.0)
        a_dev = torch.from_numpy(a32).to(gpu)
        a_val = O.bf16(a32.astype(np.float64))
    else:
        a_bits = synth.normal_bf16(3, "a", seed, (M, K))
        a_dev = dev_bf16(a_bits, gpu)
        a_val = synth.bf16_bits_to_f64(a_bits)
    w_bits = synth.normal_bf16(3, "w", seed, (N, K), std=0.02)
    b_bits = synth.normal_bf16(3, "bias", seed, (N,), std=0.01)
    add_bits = synth.normal_bf16(3, "pos_embed", seed, (M, N)) if epi == 2 else None
    if name == "wide_three_k_steps":
        b_bits = np.zeros_like(b_bits)
    out = vit.vit_bf16_gemm(a_dev, dev_bf16(w_bits, gpu), bias=None if name == "wide_three_k_steps" else dev_bf16(b_bits, gpu),
                            add=dev_bf16(add_bits, gpu) if add_bits is not None else None, epilogue=epi)
    c = O.bf16_gemm(a_val, synth.bf16_bits_to_f64(w_bits), synth.bf16_bits_to_f64(b_bits))
    if epi == 1:
        c = O.gelu_tanh(c)
    if epi == 2:
        c = c + synth.bf16_bits_to_f64(add_bits)
    assert_close(host_f64(out), O.bf16(c), TOL_GEMM, 0.9999, name)


@pytest.mark.parametrize("pad", [24, 2], ids=["wide_path", "fallback_path"])
def test_bf16_gemm_into_row_strided_output(gpu, pad):
    """bf16 GEMM into the first N columns of a wider buffer: a row stride the
    256-wide tile path takes (a multiple of 4) and one it leaves to the
    128 x 128 kernel; the columns past N keep their contents."""
    M, N, K = 200, 512, 192
    a_bits = synth.normal_bf16(3, "a", 11, (M, K))
    w_bits = synth.normal_bf16(3, "w", 11, (N, K), std=0.02)
    b_bits = synth.normal_bf16(3, "bias", 11, (N,), std=0.01)
    buf = torch.full((M, N + pad), 7.0, dtype=torch.bfloat16, device=gpu)
    announce(f"vit_bf16_gemm into a row stride of {N + pad}")
    vit.vit_bf16_gemm(dev_bf16(a_bits, gpu), dev_bf16(w_bits, gpu), bias=dev_bf16(b_bits, gpu),
                      epilogue=vit.BEPI_BIAS_GELU, out=buf[:, :N])
    c = O.gelu_tanh(O.bf16_gemm(synth.bf16_bits_to_f64(a_bits), synth.bf16_bits_to_f64(w_bits),
                                synth.bf16_bits_to_f64(b_bits)))
    assert_close(host_f64(buf[:, :N]), O.bf16(c), TOL_GEMM, 0.9999, f"row stride {N + pad}")
    assert torch.all(buf[:, N:] == 7.0)


# Small M takes other tilings (64-token FP8 tiles when 128-token ones would
# give at most one workgroup per CU; 64 x 64 bf16 tiles when the 256 x 128
# ones would fill at most half the CUs).  Every output is the same chain of
# MFMAs and FMAs in either tiling, so the rows of a small-M call equal, byte
# for byte, the same rows of a large-M call on the same operands.
FP8_TILE_SHAPES = [  # (name, N, K, epilogue)
    ("qkv", 3456, 1152, O.EPI_BIAS),
    ("proj", 1152, 1152, O.EPI_BIAS_RESIDUAL),
    ("fc1", 4304, 1152, O.EPI_BIAS_GELU_FP8),
    ("fc2", 1152, 4304, O.EPI_BIAS_RESIDUAL),
    # odd numbers of 128-deep K blocks (3 and 5): the tails of the 64-token
    # tiles' loop, which works on K blocks in pairs
    ("k3_gelu", 4304, 384, O.EPI_BIAS_GELU_FP8),
    ("k5", 1152, 640, O.EPI_BIAS_RESIDUAL),
]


@pytest.mark.parametrize("name,N,K,epi", FP8_TILE_SHAPES, ids=[s[0] for s in FP8_TILE_SHAPES])
def test_fp8_gemm_tilings_agree(gpu, name, N, K, epi):
    M = 6256
    d = _operands(gpu, M, N, K, 4000 + N + K)
    res = d["r"] if epi == O.EPI_BIAS_RESIDUAL else None

    def run(m):
        if epi == O.EPI_BIAS_GELU_FP8:
            c, s, p = vit.vit_fp8_block128_gemm(d["a_c"][:m], d["a_s"][:m], d["w_c"], d["w_s"], N, K, bias=d["b"],
                                                epilogue=epi, prequant=True)
            return [host_u8(c), host_f64(s), host_f64(p)]
        o = vit.vit_fp8_block128_gemm(d["a_c"][:m], d["a_s"][:m], d["w_c"], d["w_s"], N, K, bias=d["b"],
                                      residual=None if res is None else res[:m], epilogue=epi)
        return [o.view(torch.int16).cpu().numpy()]

    announce(f"vit_fp8_block128_gemm {name} tilings: M={M} against M=601, 64, 1")
    full = run(M)
    for m in (601, 64, 1):
        for got, ref in zip(run(m), full):
            assert np.array_equal(got, ref[:m]), f"{name}: rows of M={m} differ from the same rows at M={M}"


BF16_TILE_SHAPES = [("merger_fc1", 4608, 4608, 1), ("merger_fc2", 4096, 4608, 0)]


@pytest.mark.parametrize("name,N,K,epi", BF16_TILE_SHAPES, ids=[s[0] for s in BF16_TILE_SHAPES])
def test_bf16_gemm_tilings_agree(gpu, name, N, K, epi):
    M = 1564
    a = dev_bf16(synth.normal_bf16(3, "a", 5000 + N, (M, K)), gpu)
    w = dev_bf16(synth.normal_bf16(3, "w", 5000 + N, (N, K), std=0.02), gpu)
    b = dev_bf16(synth.normal_bf16(3, "bias", 5000 + N, (N,), std=0.01), gpu)
    announce(f"vit_bf16_gemm {name} tilings: M={M} against M=451, 243, 1")
    full = vit.vit_bf16_gemm(a, w, bias=b, epilogue=epi).view(torch.int16).cpu().numpy()
    for m in (451, 243, 1):
        got = vit.vit_bf16_gemm(a[:m], w, bias=b, epilogue=epi).view(torch.int16).cpu().numpy()
        assert np.array_equal(got, full[:m]), f"{name}: rows of M={m} differ from the same rows at M={M}"
