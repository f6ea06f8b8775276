"""Turn the seeded synthetic tensors (bf16 bit patterns) into oracle weights.

Test infrastructure only (see ``oracle/__init__.py``).  Pure format
decoding: a bf16 bit pattern b has the value of the fp32 bit pattern b << 16.
"""

from __future__ import annotations

from typing import Dict, List

import numpy as np

import synth

from .vit_oracle import BlockWeights, EncoderWeights, MergerWeights


def dec(bits) -> np.ndarray:
    return synth.bf16_bits_to_f64(bits)


def block_weights(p: Dict[str, np.ndarray]) -> BlockWeights:
    return BlockWeights(**{k: dec(v) for k, v in p.items()})


def merger_weights(p: Dict[str, np.ndarray]) -> MergerWeights:
    return MergerWeights(ln_g=dec(p["m_ln_g"]), ln_b=dec(p["m_ln_b"]),
                         fc1_w=dec(p["m_fc1_w"]), fc1_b=dec(p["m_fc1_b"]),
                         fc2_w=dec(p["m_fc2_w"]), fc2_b=dec(p["m_fc2_b"]))


def encoder_weights(ep: "synth.EncoderParams") -> EncoderWeights:
    return EncoderWeights(patch_w=dec(ep.patch["patch_w"]), patch_b=dec(ep.patch["patch_b"]),
                          blocks=[block_weights(b) for b in ep.blocks],
                          mergers=[merger_weights(m) for m in ep.mergers])


def zero_like_block(p: Dict[str, np.ndarray], keep: List[str] = ()) -> Dict[str, np.ndarray]:
    """Copy of block parameters with every tensor not in ``keep`` set to 0."""
    return {k: (v if k in keep else np.zeros_like(v)) for k, v in p.items()}
