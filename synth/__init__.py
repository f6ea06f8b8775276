"""Seeded synthetic inputs shared by the CPU oracle checks and the GPU path.

This module draws numbers and stores them in the formats both sides read
(bf16 bit patterns, fp32, int32 geometry).  It holds none of the method's
arithmetic: no normalisation, rotation, attention, quantisation or GEMM.

Every tensor comes from numpy's PCG64 seeded with
``SeedSequence([config_id, tensor_tag, index])``; values are drawn in fp32
and rounded to bf16 (nearest, ties to even) where the tensor is bf16.
Distributions follow the workloads described for this tower: activations
~N(0, 1), GEMM weights ~N(0, 0.02), biases ~N(0, 0.01), LayerNorm gamma
1 + N(0, 0.02) and beta ~N(0, 0.01), pixels ~U(-1, 1); the learned 48 x 48
position table ~N(0, 0.02) like the other weights.
"""

from __future__ import annotations

from dataclasses import dataclass
from functools import lru_cache
from typing import Dict, List, Sequence, Tuple

import numpy as np

HIDDEN, HEADS, HEAD_DIM, MLP, MLP_PADDED = 1152, 16, 72, 4304, 4352
PATCH_DIM, DEPTH, OUT_HIDDEN, MERGED_DIM = 1536, 27, 4096, 4608

# Tensor tags (stable integers: changing one changes every derived input).
TAGS = {
    "x": 1, "q": 2, "k": 3, "v": 4, "a": 5, "w": 6, "bias": 7, "residual": 8,
    "pixels": 9, "pos_embed": 10, "pos_table": 11, "frames": 12,
    "ln1_g": 20, "ln1_b": 21, "qkv_w": 22, "qkv_b": 23, "proj_w": 24, "proj_b": 25,
    "ln2_g": 26, "ln2_b": 27, "fc1_w": 28, "fc1_b": 29, "fc2_w": 30, "fc2_b": 31,
    "patch_w": 40, "patch_b": 41,
    "m_ln_g": 50, "m_ln_b": 51, "m_fc1_w": 52, "m_fc1_b": 53, "m_fc2_w": 54, "m_fc2_b": 55,
}

# Workloads.  Patch grids (rows, cols) of the image sizes the tower is run
# at: 6256 = 46 x 136 (one 2172x724 image), 3888 = 36 x 108, 1824 = 24 x 76
# (the varlen batch) or 48 x 38 (the attention-only case), 972 = 18 x 54.
CONFIGS = {
    0: dict(name="block_p256", grids=[(16, 16)]),
    1: dict(name="attention_p1824", grids=[(48, 38)]),
    2: dict(name="gemm_sweep_m6256", M=6256),
    3: dict(name="encoder_p6256", grids=[(46, 136)]),
    4: dict(name="encoder_varlen_972_3888_1824", grids=[(18, 54), (36, 108), (24, 76)]),
}


def rng(config_id: int, tag: str, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, TAGS[tag], index])))


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, nearest with ties to even (finite input)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    """Exact value of bf16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def normal_bf16(config_id: int, tag: str, index: int, shape, std: float = 1.0,
                mean: float = 0.0) -> np.ndarray:
    g = rng(config_id, tag, index)
    x = g.standard_normal(size=shape, dtype=np.float32) * np.float32(std) + np.float32(mean)
    return f32_to_bf16_bits(x)


def uniform_f32(config_id: int, tag: str, index: int, shape, lo: float, hi: float) -> np.ndarray:
    g = rng(config_id, tag, index)
    return (g.random(size=shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def frames_u8(config_id: int, index: int, shape) -> np.ndarray:
    """uint8 RGB frames [F, H, W, 3]: a smooth per-frame gradient plus
    uniform noise, so resampling sees both structure and texture."""
    g = rng(config_id, "frames", index)
    F_, H, W, C = shape
    yy, xx = np.meshgrid(np.linspace(0, 1, H, dtype=np.float32), np.linspace(0, 1, W, dtype=np.float32),
                         indexing="ij")
    base = np.stack([yy, xx, 1 - yy], axis=-1)[None] * np.float32(160)
    shift = g.uniform(0, 40, size=(F_, 1, 1, C)).astype(np.float32)
    noise = g.uniform(0, 56, size=shape).astype(np.float32)
    return np.clip(base + shift + noise, 0, 255).astype(np.uint8)


def grids_of(config_id: int) -> List[Tuple[int, int]]:
    return list(CONFIGS[config_id]["grids"])


def cu_seqlens(grids: Sequence[Tuple[int, int]]) -> np.ndarray:
    cu = [0]
    for h, w in grids:
        cu.append(cu[-1] + h * w)
    return np.asarray(cu, dtype=np.int32)


def positions(grids: Sequence[Tuple[int, int]]) -> np.ndarray:
    """(row, col) int32 per token, raster order within each image."""
    out = []
    for h, w in grids:
        r, c = np.meshgrid(np.arange(h, dtype=np.int32), np.arange(w, dtype=np.int32), indexing="ij")
        out.append(np.stack([r.ravel(), c.ravel()], axis=1))
    return np.concatenate(out, axis=0).astype(np.int32)


BLOCK_SHAPES = {
    "ln1_g": (HIDDEN,), "ln1_b": (HIDDEN,),
    "qkv_w": (3 * HIDDEN, HIDDEN), "qkv_b": (3 * HIDDEN,),
    "proj_w": (HIDDEN, HIDDEN), "proj_b": (HIDDEN,),
    "ln2_g": (HIDDEN,), "ln2_b": (HIDDEN,),
    "fc1_w": (MLP, HIDDEN), "fc1_b": (MLP,),
    "fc2_w": (HIDDEN, MLP), "fc2_b": (HIDDEN,),
}

MERGER_SHAPES = {
    "m_ln_g": (MERGED_DIM,), "m_ln_b": (MERGED_DIM,),
    "m_fc1_w": (MERGED_DIM, MERGED_DIM), "m_fc1_b": (MERGED_DIM,),
    "m_fc2_w": (OUT_HIDDEN, MERGED_DIM), "m_fc2_b": (OUT_HIDDEN,),
}


def _param(config_id: int, name: str, index: int, shape) -> np.ndarray:
    if name.endswith("_g"):
        return normal_bf16(config_id, name, index, shape, std=0.02, mean=1.0)
    if name.endswith("_b") and ("ln" in name):
        return normal_bf16(config_id, name, index, shape, std=0.01)
    if name.endswith("_b"):
        return normal_bf16(config_id, name, index, shape, std=0.01)
    return normal_bf16(config_id, name, index, shape, std=0.02)


def block_params(config_id: int, block_index: int) -> Dict[str, np.ndarray]:
    """bf16 bit patterns of one block's 12 tensors."""
    return {n: _param(config_id, n, block_index, s) for n, s in BLOCK_SHAPES.items()}


def merger_params(config_id: int, merger_index: int) -> Dict[str, np.ndarray]:
    return {n: _param(config_id, n, merger_index, s) for n, s in MERGER_SHAPES.items()}


def patch_params(config_id: int) -> Dict[str, np.ndarray]:
    return {"patch_w": normal_bf16(config_id, "patch_w", 0, (HIDDEN, PATCH_DIM), std=0.02),
            "patch_b": normal_bf16(config_id, "patch_b", 0, (HIDDEN,), std=0.01)}


def pixels(config_id: int, T: int) -> np.ndarray:
    return uniform_f32(config_id, "pixels", 0, (T, PATCH_DIM), -1.0, 1.0)


@dataclass
class EncoderParams:
    patch: Dict[str, np.ndarray]
    blocks: List[Dict[str, np.ndarray]]
    mergers: List[Dict[str, np.ndarray]]


@lru_cache(maxsize=2)
def encoder_params(config_id: int, depth: int = DEPTH) -> EncoderParams:
    return EncoderParams(patch=patch_params(config_id),
                         blocks=[block_params(config_id, b) for b in range(depth)],
                         mergers=[merger_params(config_id, m) for m in range(4)])
