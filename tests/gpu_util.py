"""Helpers shared by the GPU parity tests: moving seeded bf16 bit patterns to
the device and back, and the comparison metrics used for parity.

Metrics: normwise max relative error ||gpu - ref||_inf / ||ref||_inf and the
cosine of the flattened tensors, both in float64."""

from __future__ import annotations

import sys

import numpy as np
import torch

import synth


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def dev_bf16(bits: np.ndarray, device="cuda:0") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 value of a device tensor (bf16 / fp32 / fp64)."""
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().astype(np.uint8)


def metrics(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    rel = np.abs(gpu - ref).max() / max(np.abs(ref).max(), 1e-300)
    cos = float(gpu @ ref / max(np.linalg.norm(gpu) * np.linalg.norm(ref), 1e-300))
    return float(rel), cos


def assert_close(gpu, ref, max_rel: float, min_cos: float, what: str = "") -> None:
    rel, cos = metrics(gpu, ref)
    announce(f"{what}: max_rel={rel:.3e} cos={cos:.7f}")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert rel <= max_rel and cos >= min_cos, f"{what}: max_rel={rel:.3e} (<= {max_rel}) cos={cos:.7f} (>= {min_cos})"


class implementation_noise:
    """Context in which the oracle runs with noise of the size of the
    precision the method's design computes in: half an fp32 ulp (2^-24) on
    every LayerNorm and GELU output (the quantiser inputs) and half a bf16
    ulp (2^-8) on every attention probability (the bf16 P of an FA2-style
    attention, as the FlashRT page's "BF16 attention" does).  The tower amplifies the FP8
    code flips such noise causes at rounding ties; how far the oracle moves
    under it is the envelope an fp32/bf16 implementation is held to against
    the fp64 oracle where it is wider than the stated tolerance."""

    def __init__(self, seed=0):
        self.rng = np.random.default_rng(seed)

    def _noise(self, y, ulp):
        return y * (1 + self.rng.choice([-1.0, 1.0], size=y.shape) * ulp)

    def __enter__(self):
        import math
        import oracle.vit_oracle as V
        self.V = V
        self.orig = (V.layernorm, V.gelu_tanh, V.attention)
        ln, gelu, _ = self.orig
        V.layernorm = lambda *a, **k: self._noise(ln(*a, **k), 2.0 ** -24)
        V.gelu_tanh = lambda *a, **k: self._noise(gelu(*a, **k), 2.0 ** -24)

        def attention(q, k, v, cu_seqlens, num_heads=16, head_dim=72, scale=None):
            scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
            out = np.zeros((q.shape[0], num_heads * head_dim))
            for j in range(len(cu_seqlens) - 1):
                a, b = int(cu_seqlens[j]), int(cu_seqlens[j + 1])
                for h in range(num_heads):
                    sl = slice(h * head_dim, (h + 1) * head_dim)
                    sc = (q[a:b, sl] @ k[a:b, sl].T) * scale
                    p = self._noise(np.exp(sc - sc.max(axis=1, keepdims=True)), 2.0 ** -8)
                    out[a:b, sl] = (p @ v[a:b, sl]) / p.sum(axis=1, keepdims=True)
            return out

        V.attention = attention
        return self

    def __exit__(self, *exc):
        self.V.layernorm, self.V.gelu_tanh, self.V.attention = self.orig
        return False


def check_within(got, ref, env, what, max_rel=2e-2, min_cos=0.9995):
    """max_rel <= max(2e-2, 2 * envelope max_rel) and 1 - cos <= max(5e-4,
    2 * (1 - envelope cos)); both printed."""
    rel, cos = metrics(got, ref)
    erel, ecos = env
    announce(f"{what}: gpu rel={rel:.3e} cos={cos:.7f} | oracle envelope rel={erel:.3e} cos={ecos:.7f}")
    assert np.all(np.isfinite(got)), what
    assert rel <= max(max_rel, 2 * erel), f"{what}: rel {rel:.3e}"
    assert 1 - cos <= max(1 - min_cos, 2 * (1 - ecos)), f"{what}: cos {cos:.7f}"
