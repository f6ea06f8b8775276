"""Implementation-noise envelope of the oracle (test infrastructure only,
like the rest of this package).

The fp64 oracle is the reference; an implementation that computes in the
precisions the method's design uses (fp32 LayerNorm, GELU and softmax
statistics, bf16 attention probabilities) differs from it by rounding, and
the 27-block FP8 tower amplifies such differences wherever they flip an FP8
code at a rounding tie.  ``implementation_noise`` re-runs the oracle with
noise of exactly that size; how far the oracle itself then moves is the
envelope a GPU result is held to where it is wider than the stated
tolerance.
"""

from __future__ import annotations

import numpy as np


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


def within_envelope(got, ref, noisy, max_rel: float = 2e-2, min_cos: float = 0.9995):
    """(ok, (rel, cos), (env_rel, env_cos)): ``got`` is within max_rel /
    min_cos of ``ref``, or within twice the oracle's own drift ``noisy``
    under implementation noise, whichever is wider."""

    def metrics(a, b):
        a = np.asarray(a, np.float64).ravel()
        b = np.asarray(b, np.float64).ravel()
        rel = float(np.abs(a - b).max() / np.abs(b).max())
        cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
        return rel, cos

    rel, cos = metrics(got, ref)
    erel, ecos = metrics(noisy, ref)
    ok = bool(np.all(np.isfinite(got))) and rel <= max(max_rel, 2 * erel) and 1 - cos <= max(1 - min_cos,
                                                                                            2 * (1 - ecos))
    return ok, (rel, cos), (erel, ecos)
