"""Helpers shared by the GPU parity tests: moving seeded bf16 bit patterns to
the device and back, and the comparison metrics used for parity.

Metrics: normwise max relative error ||gpu - ref||_inf / ||ref||_inf and the
cosine of the flattened tensors, both in float64."""

from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from oracle.envelope import implementation_noise  # noqa: F401  (re-exported for the tests)


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


def check_within(got, ref, env, what, max_rel=2e-2, min_cos=0.9995):
    """max_rel <= max(2e-2, 2 * envelope max_rel) and 1 - cos <= max(5e-4,
    2 * (1 - envelope cos)); both printed."""
    rel, cos = metrics(got, ref)
    erel, ecos = env
    announce(f"{what}: gpu rel={rel:.3e} cos={cos:.7f} | oracle envelope rel={erel:.3e} cos={ecos:.7f}")
    assert np.all(np.isfinite(got)), what
    assert rel <= max(max_rel, 2 * erel), f"{what}: rel {rel:.3e}"
    assert 1 - cos <= max(1 - min_cos, 2 * (1 - ecos)), f"{what}: cos {cos:.7f}"
