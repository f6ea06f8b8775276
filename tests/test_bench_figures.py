"""The benchmark's algorithmic work figures, which its roofline fractions
divide by, checked on the CPU against what the workloads are made of: GEMM
FLOPs from the weight shapes of the synthetic tower, attention FLOPs from
the windows and the head layout, quantiser and RoPE bytes from the arrays
the kernels read and write.  Also the source guard of the HBM traffic
lookup and the one-GPU refusal."""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle as O
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gemm(rows: int, shape) -> int:
    """2 FLOPs per multiply-add of rows x shape[1] times shape[1] x shape[0]."""
    return 2 * rows * shape[0] * shape[1]


def _attention(seq) -> int:
    """Per head and ordered (query, key) pair of a window: the q.k dot product
    and the p.v update, head_dim multiply-adds each."""
    return sum(p * p for p in seq) * synth.HEADS * 2 * (2 * synth.HEAD_DIM)


@pytest.mark.parametrize("cfg", [3, 4], ids=["encoder_p6256", "encoder_varlen_6684"])
def test_encoder_flops_from_the_tower(cfg):
    seq = [h * w for h, w in synth.grids_of(cfg)]
    T = sum(seq)
    S, Ms = synth.BLOCK_SHAPES, synth.MERGER_SHAPES
    blocks = synth.DEPTH * sum(_gemm(T, S[n]) for n in ("qkv_w", "proj_w", "fc1_w", "fc2_w"))
    attn = synth.DEPTH * _attention(seq)
    patch = _gemm(T, (synth.HIDDEN, synth.PATCH_DIM))
    mergers = 4 * sum(_gemm(T // 4, Ms[n]) for n in ("m_fc1_w", "m_fc2_w"))
    d = bench.encoder_flops(seq)
    assert (d["gemm"], d["attention"], d["patch"], d["mergers"]) == (blocks, attn, patch, mergers)
    assert d["total"] == blocks + attn + patch + mergers


def test_kernel_work_from_the_arrays():
    grids = synth.grids_of(3)
    seq = [h * w for h, w in grids]
    T = sum(seq)
    H = synth.HIDDEN
    w = bench.kernel_work(T, seq)
    # LayerNorm-quant and the row quantiser: read a bf16 row block, write the
    # codes and the fp32 scales the quantiser returns
    codes, scales = O.quantize_block128(np.zeros((T, H)), 1)
    quant_bytes = T * H * 2 + codes.astype(np.uint8).nbytes + scales.astype(np.float32).nbytes
    assert w["layernorm_quant"] == (quant_bytes, "B", 2 * synth.DEPTH)
    assert w["quant_rows"] == (quant_bytes, "B", synth.DEPTH)
    # RoPE: q and k read and written in place, plus the int32 positions
    assert w["rope2d"] == (2 * 2 * T * H * 2 + synth.positions(grids).nbytes, "B", synth.DEPTH)
    for name, wname in (("fp8_gemm_qkv", "qkv_w"), ("fp8_gemm_proj", "proj_w"),
                        ("fp8_gemm_fc1_gelu_quant", "fc1_w"), ("fp8_gemm_fc2", "fc2_w")):
        assert w[name] == (_gemm(T, synth.BLOCK_SHAPES[wname]), "F8", synth.DEPTH)
    assert w["attention"] == (_attention(seq), "F16", synth.DEPTH)
    assert w["patch_embed_bf16"] == (_gemm(T, (H, synth.PATCH_DIM)), "F16", 1)
    # 2 x 2 merge with its LayerNorm: the tap read once, the merged rows written
    assert w["merge_layernorm"] == (T * H * 2 + (T // 4) * synth.MERGED_DIM * 2, "B", 4)
    assert w["merger_fc1_bf16"] == (_gemm(T // 4, synth.MERGER_SHAPES["m_fc1_w"]), "F16", 4)
    assert w["merger_fc2_bf16"] == (_gemm(T // 4, synth.MERGER_SHAPES["m_fc2_w"]), "F16", 4)
    # the figures quoted for the roofline: 180.35 GFLOP per attention launch
    assert round(w["attention"][0] / 1e9, 2) == 180.35


def test_traffic_lookup_follows_the_sources(monkeypatch):
    t = bench.traffic_from_profiles("attention")
    assert t is None or t > 0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0000000000000000")
    assert bench.traffic_from_profiles("attention") is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2, r.stdout + r.stderr
    assert "one GPU" in r.stdout + r.stderr
