"""GPU parity of 2D RoPE and of varlen full attention (head_dim 72) against
the fp64 oracle, with the edge cases of the window packing."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
import vision_transformer_encoder_amd as vit
from gpu_util import announce, assert_close, dev_bf16, host_f64

pytestmark = pytest.mark.gpu

MAX_REL, MIN_COS = 2e-2, 0.9995


def _qkv_bits(cfg, T, seed=0):
    return [synth.normal_bf16(cfg, t, seed, (T, 1152)) for t in ("q", "k", "v")]


# row stride 3456 takes the staged 16-byte path; 3460 (rows not 16-byte
# aligned) the one-lane-per-unit path
@pytest.mark.parametrize("ld", [3456, 3460])
@pytest.mark.parametrize("grids", [[(48, 38)], [(18, 54), (36, 108), (24, 76)], [(3, 5)]],
                         ids=["48x38", "varlen3", "3x5"])
def test_rope2d(gpu, grids, ld):
    T = sum(h * w for h, w in grids)
    q, k, _ = _qkv_bits(1, T)
    qkv = torch.zeros((T, ld), dtype=torch.bfloat16, device=gpu)
    qkv[:, :1152] = dev_bf16(q, gpu)
    qkv[:, 1152:2304] = dev_bf16(k, gpu)
    pos = synth.positions(grids)
    announce(f"vit_rope2d T={T}")
    vit.vit_rope2d(qkv[:, :1152], qkv[:, 1152:2304], torch.from_numpy(pos).to(gpu))
    res = host_f64(qkv)
    for name, src, sl in (("q", q, slice(0, 1152)), ("k", k, slice(1152, 2304))):
        ref = O.rope2d(synth.bf16_bits_to_f64(src), pos)
        assert_close(res[:, sl], O.bf16(ref), 1e-2, 0.99999, f"rope {name}")
        # GPU result is within one bf16 rounding of the exact rotation, plus
        # the fp32 angle error (|p f| 2^-23 scale) times the pair's norm
        src64 = synth.bf16_bits_to_f64(src).reshape(T, 16, 2, 2, 18)
        pair = np.sqrt(src64[:, :, :, 0, :] ** 2 + src64[:, :, :, 1, :] ** 2)
        pair = np.stack([pair, pair], axis=3).reshape(T, 1152)
        assert np.all(np.abs(res[:, sl] - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-4 * pair)
    assert np.all(res[:, 2304:] == 0), "v slice must be untouched"


# other head counts and widths take other chunks-per-thread variants of the
# staged kernel (1, 3 with a partial last pass, 8), with a ragged last group
# of tokens (T % 8 != 0)
@pytest.mark.parametrize("heads,hd", [(2, 64), (4, 72), (8, 128)], ids=["2x64", "4x72", "8x128"])
def test_rope2d_other_shapes(gpu, heads, hd):
    grids = [(3, 5), (6, 7)]
    T = sum(h * w for h, w in grids)
    W = heads * hd
    q = synth.normal_bf16(1, "q", 7, (T, W))
    k = synth.normal_bf16(1, "k", 7, (T, W))
    qk = torch.zeros((T, 2 * W), dtype=torch.bfloat16, device=gpu)
    qk[:, :W] = dev_bf16(q, gpu)
    qk[:, W:] = dev_bf16(k, gpu)
    pos = synth.positions(grids)
    announce(f"vit_rope2d T={T} heads={heads} head_dim={hd}")
    vit.vit_rope2d(qk[:, :W], qk[:, W:], torch.from_numpy(pos).to(gpu), num_heads=heads, head_dim=hd)
    res = host_f64(qk)
    for name, src, sl in (("q", q, slice(0, W)), ("k", k, slice(W, 2 * W))):
        ref = O.rope2d(synth.bf16_bits_to_f64(src), pos, num_heads=heads, head_dim=hd)
        assert_close(res[:, sl], O.bf16(ref), 1e-2, 0.99999, f"rope {name} {heads}x{hd}")


def _attention_case(gpu, grids, cfg=1):
    T = sum(h * w for h, w in grids)
    q0, k0, v = _qkv_bits(cfg, T)
    pos = synth.positions(grids)
    # q, k = bf16(RoPE(q0, k0)) from the oracle: attention isolated from RoPE
    q = O.bf16(O.rope2d(synth.bf16_bits_to_f64(q0), pos))
    k = O.bf16(O.rope2d(synth.bf16_bits_to_f64(k0), pos))
    vf = synth.bf16_bits_to_f64(v)
    qkv = torch.empty((T, 3456), dtype=torch.bfloat16, device=gpu)
    qkv[:, :1152] = torch.from_numpy(q).to(gpu).to(torch.bfloat16)
    qkv[:, 1152:2304] = torch.from_numpy(k).to(gpu).to(torch.bfloat16)
    qkv[:, 2304:] = dev_bf16(v, gpu)
    return T, qkv, q, k, vf


@pytest.mark.parametrize("grids", [[(48, 38)], [(18, 54), (36, 108), (24, 76)], [(46, 136)]],
                         ids=["p1824", "varlen_6684", "p6256"])
def test_attention_parity(gpu, grids):
    T, qkv, q, k, vf = _attention_case(gpu, grids)
    cu = synth.cu_seqlens(grids)
    announce(f"vit_attention T={T} cu={list(cu)}")
    o = vit.vit_attention(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], cu)
    torch.cuda.synchronize()
    ref = O.attention(q, k, vf, cu)
    assert_close(host_f64(o), ref, MAX_REL, MIN_COS, f"attention T={T}")


def test_attention_window_edge_cases(gpu):
    # windows of 1, 63, 64, 65, 127, 128, 129 and 200 tokens plus an empty one
    lens = [1, 63, 64, 65, 0, 127, 128, 129, 200]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    qb, kb, vb = _qkv_bits(1, T, seed=3)
    q, k, v = (synth.bf16_bits_to_f64(b) for b in (qb, kb, vb))
    qkv = torch.cat([dev_bf16(qb, gpu), dev_bf16(kb, gpu), dev_bf16(vb, gpu)], dim=1).contiguous()
    announce(f"vit_attention edge windows {lens}")
    o = host_f64(vit.vit_attention(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], cu))
    ref = O.attention(q, k, v, cu)
    assert_close(o, ref, MAX_REL, MIN_COS, "edge windows")
    # a one-token window returns its own V exactly (softmax of one score is 1)
    assert np.array_equal(o[0], v[0])


def test_attention_packed_equals_separate(gpu):
    """Windows packed in one call give what separate calls give.  The
    stream-K split of the key ranges depends on the whole packing, so the
    two agree to the attention tolerance rather than bit for bit."""
    grids = [(18, 54), (24, 76)]
    T, qkv, _, _, _ = _attention_case(gpu, grids)
    cu = synth.cu_seqlens(grids)
    packed = vit.vit_attention(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], cu)
    a = int(cu[1])
    first = vit.vit_attention(qkv[:a, :1152], qkv[:a, 1152:2304], qkv[:a, 2304:], [0, a])
    second_qkv = qkv[a:].clone()
    second = vit.vit_attention(second_qkv[:, :1152], second_qkv[:, 1152:2304], second_qkv[:, 2304:], [0, T - a])
    sep = torch.cat([first, second])
    assert_close(host_f64(packed), host_f64(sep), 1e-2, 0.99999, "packed vs separate")


def test_attention_constant_v_and_deterministic(gpu):
    T = 300
    qb, kb, _ = _qkv_bits(1, T, seed=9)
    vrow = synth.normal_bf16(1, "v", 9, (1, 1152))
    vb = np.repeat(vrow, T, axis=0)
    qkv = torch.cat([dev_bf16(qb, gpu), dev_bf16(kb, gpu), dev_bf16(vb, gpu)], dim=1).contiguous()
    o1 = vit.vit_attention(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], [0, T])
    o2 = vit.vit_attention(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], [0, T])
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # softmax weights sum to one: constant V comes back up to rounding
    vv = synth.bf16_bits_to_f64(vrow)
    assert np.allclose(host_f64(o1), np.repeat(vv, T, 0), rtol=1e-2, atol=1e-2)


def _peaky_case(gpu, grids, kind):
    """q, k with scores spanning tens of log2 units and each query's row max
    in a late key tile of its window.  Per head a random unit direction u is
    added to every query (weight cq) and to the keys, with a weight that
    ramps up along the window ("ramp": the max climbs by ~40 log2 units
    over the window's key tiles) or only on the window's last three keys
    ("spike": a jump of ~30 log2 units in the last tile).  The generic part
    of q is scaled by 3 so that scores are peaky everywhere."""
    T, _, q, k, vf = _attention_case(gpu, grids)
    g = np.random.default_rng(11)
    u = g.standard_normal((16, 72))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    cu = synth.cu_seqlens(grids)
    w = np.zeros(T)
    for j in range(len(cu) - 1):
        a, b = int(cu[j]), int(cu[j + 1])
        if kind == "ramp":
            w[a:b] = np.arange(b - a) / (b - a)
        else:
            w[b - 3:b] = 1.0
    cq, ck = (16.0, 16.0) if kind == "ramp" else (12.0, 18.0)
    qh = 3.0 * q.reshape(T, 16, 72) + cq * u[None]
    kh = k.reshape(T, 16, 72) + ck * w[:, None, None] * u[None]
    qp, kp = O.bf16(qh.reshape(T, 1152)), O.bf16(kh.reshape(T, 1152))
    qkv = torch.empty((T, 3456), dtype=torch.bfloat16, device=gpu)
    qkv[:, :1152] = torch.from_numpy(qp).to(gpu).to(torch.bfloat16)
    qkv[:, 1152:2304] = torch.from_numpy(kp).to(gpu).to(torch.bfloat16)
    qkv[:, 2304:] = torch.from_numpy(vf).to(gpu).to(torch.bfloat16)
    return T, cu, qkv, qp, kp, vf


@pytest.mark.parametrize("kind", ["ramp", "spike"])
@pytest.mark.parametrize("grids", [[(46, 136)], [(18, 54), (36, 108), (24, 76)]], ids=["p6256", "varlen_6684"])
def test_attention_peaky_logits(gpu, grids, kind):
    T, cu, qkv, q, k, v = _peaky_case(gpu, grids, kind)
    # how peaky the scores are (first window, head 0): the spread of a row
    # in log2 units, how far its first key tile's max lies below the row max
    # (the running max must climb by more than the 2^8 lazy-rescale margin),
    # and how many rows have their max in the last tenth of the window
    a, b = int(cu[0]), int(cu[1])
    s = (q[a:b, :72] @ k[a:b, :72].T) / math.sqrt(72) * math.log2(math.e)
    spread = float(np.median(s.max(axis=1) - s.min(axis=1)))
    climb = float(np.median(s.max(axis=1) - s[:, :64].max(axis=1)))
    late = float(np.mean(s.argmax(axis=1) >= 0.9 * (b - a)))
    announce(f"vit_attention peaky ({kind}) T={T}: median row spread {spread:.1f} log2 units, "
             f"row max {climb:.1f} above the first key tile's, {100 * late:.0f}% of row maxima in the last tenth")
    assert spread > 20.0 and climb > 16.0 and late > 0.8
    o = vit.vit_attention(qkv[:, :1152], qkv[:, 1152:2304], qkv[:, 2304:], cu)
    torch.cuda.synchronize()
    ref = O.attention(q, k, v, cu)
    assert_close(host_f64(o), ref, MAX_REL, MIN_COS, f"attention peaky {kind} T={T}")


@pytest.mark.parametrize("shards", [2, 8, 16], ids=["8_heads", "2_heads", "1_head"])
def test_attention_head_shard(gpu, shards):
    """Attention on a head shard: the share of one of `shards` GPUs in a head
    split of the 16 heads (q, k, v and o as column slices of the full
    [T, 3456] / [T, 1152] buffers, num_heads = 16 / shards).  Every shard is
    compared with the oracle on its heads, and the shards put together with
    the oracle on all 16."""
    grids = [(46, 136)]
    T, qkv, q, k, vf = _attention_case(gpu, grids)
    cu = synth.cu_seqlens(grids)
    H = 16 // shards
    W = 72 * H
    out = torch.empty((T, 1152), dtype=torch.bfloat16, device=gpu)
    announce(f"vit_attention head shards: {shards} x {H} heads, T={T}")
    for s in range(shards):
        c = slice(s * W, (s + 1) * W)
        vit.vit_attention(qkv[:, c], qkv[:, 1152 + s * W:1152 + (s + 1) * W], qkv[:, 2304 + s * W:2304 + (s + 1) * W],
                          cu, num_heads=H, out=out[:, c])
    torch.cuda.synchronize()
    got = host_f64(out)
    for s in (0, shards - 1):
        c = slice(s * W, (s + 1) * W)
        ref = O.attention(q[:, c], k[:, c], vf[:, c], cu, num_heads=H)
        assert_close(got[:, c], ref, MAX_REL, MIN_COS, f"attention shard {s} of {shards}")
    assert_close(got, O.attention(q, k, vf, cu), MAX_REL, MIN_COS, f"attention, {shards} shards put together")
