"""vit_attention_noalloc (the attention for callers that cannot allocate:
its partials live in the library's own per-device array) against
vit_attention with a caller workspace: two calls in a row through the C
ABI, the second on a smaller packing, each bit-identical to the
workspace entry point and within the attention tolerance of the oracle."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
import vision_transformer_encoder_amd as vit
from gpu_util import announce, assert_close, dev_bf16, host_f64

pytestmark = pytest.mark.gpu


def _case(gpu, grids, seed):
    T = sum(h * w for h, w in grids)
    q, k, v = [synth.normal_bf16(1, t, seed, (T, 1152)) for t in ("q", "k", "v")]
    qkv = torch.cat([dev_bf16(q, gpu), dev_bf16(k, gpu), dev_bf16(v, gpu)], dim=1).contiguous()
    cu = synth.cu_seqlens(grids)
    return T, cu, qkv, [synth.bf16_bits_to_f64(b) for b in (q, k, v)]


def test_noalloc_matches_workspace_entry_point(gpu):
    assert vit.vit_attention_noalloc_scratch_size() >= vit.vit_attention_workspace_size()
    for grids, seed in (([(46, 136)], 41), ([(18, 54), (24, 76)], 42)):
        T, cu, qkv, (q, k, v) = _case(gpu, grids, seed)
        cu_dev = torch.from_numpy(cu).to(gpu)
        out = torch.full((T, 1152), float("nan"), dtype=torch.bfloat16, device=gpu)
        announce(f"vit_attention_noalloc T={T} cu={list(cu)}")
        vit.vit_attention_noalloc(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], cu, cu_dev, out)
        ref_ws = vit.vit_attention(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], cu, cu_seqlens_dev=cu_dev)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_ws.view(torch.int16)), "differs from vit_attention"
        assert_close(host_f64(out), O.attention(q, k, v, cu), 2e-2, 0.9995, f"noalloc attention T={T}")
