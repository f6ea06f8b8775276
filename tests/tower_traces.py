"""Oracle traces of the whole 27-block tower at full size, computed in child
processes so that they run beside the other GPU tests (test infrastructure
only: this file calls ``oracle/`` and ``synth`` and nothing of the HIP
library).

A trace is the fp64 storage-mode oracle run once over a workload: the
residual stream after patch embed and after every block (x0 .. x27) and the
four merger outputs (DeepStack 8, 16, 24 and final).  Every one of these is
a bf16 storage point of the oracle, so it is saved exactly as bf16 bit
patterns.  The "noisy" run is the same forward under
``oracle.envelope.implementation_noise`` (its outputs set the envelope of
the free-running comparison).

Run as a script (one workload, one mode) it writes an ``.npz`` and prints a
progress line per block on stderr.  ``start``/``wait`` manage a set of such
children from the test session.
"""

from __future__ import annotations

import os
import subprocess
import sys
import time
from typing import Dict, List, Tuple

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# full-size workloads: one 46 x 136 image (6256 patches) and the packed
# 18 x 54 + 36 x 108 + 24 x 76 batch (972 + 3888 + 1824 = 6684 patches)
WORKLOADS = {3: "encoder_p6256", 4: "encoder_varlen_6684"}
THREADS_PER_CHILD = 4


def _bits(x: np.ndarray) -> np.ndarray:
    import oracle as O
    import synth
    x = np.asarray(x, np.float64)
    assert np.array_equal(O.bf16(x), x), "trace value is not a bf16 storage point"
    return synth.f32_to_bf16_bits(x.astype(np.float32))


def compute(cfg: int, noisy: bool, path: str) -> None:
    import oracle as O
    import oracle.vit_oracle as V
    import synth
    from oracle import inputs as OI
    from oracle.envelope import implementation_noise

    grids = synth.grids_of(cfg)
    T = sum(h * w for h, w in grids)
    ow = OI.encoder_weights(synth.encoder_params(cfg))
    px = synth.pixels(cfg, T).astype(np.float64)
    tag = f"[oracle {WORKLOADS[cfg]} {'noisy' if noisy else 'trace'}]"
    t0 = time.perf_counter()

    # progress line per block: wrap block_forward for the duration of the run
    orig = V.block_forward
    count = [0]

    def block_forward(*a, **k):
        y = orig(*a, **k)
        count[0] += 1
        sys.stderr.write(f"{tag} block {count[0]}/27 {time.perf_counter() - t0:.0f}s\n")
        sys.stderr.flush()
        return y

    V.block_forward = block_forward
    try:
        if noisy:
            with implementation_noise(100):
                out, last = O.encoder_forward(px, ow, grids)
            arrays = {"out": _bits(out), "last": _bits(last)}
        else:
            tr: Dict[str, np.ndarray] = {}
            out, last = O.encoder_forward(px, ow, grids, trace=tr)
            xs = np.stack([_bits(tr[f"x{b}"]) for b in range(28)])
            arrays = {"x": xs, "out": _bits(out), "last": _bits(last)}
    finally:
        V.block_forward = orig
    tmp = path + ".tmp.npz"
    np.savez(tmp, **arrays)
    os.replace(tmp, path)
    sys.stderr.write(f"{tag} done in {time.perf_counter() - t0:.0f}s\n")
    sys.stderr.flush()


class Children:
    """Background oracle runs, one child process per (workload, mode)."""

    def __init__(self, jobs: List[Tuple[int, bool]], directory: str):
        self.dir = directory
        self.procs: Dict[Tuple[int, bool], subprocess.Popen] = {}
        env = dict(os.environ)
        for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
            env[v] = str(THREADS_PER_CHILD)
        env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
        # the children never touch the GPU
        env["HIP_VISIBLE_DEVICES"] = ""
        for cfg, noisy in jobs:
            args = [sys.executable, os.path.abspath(__file__), str(cfg), "noisy" if noisy else "trace",
                    self.path(cfg, noisy)]
            self.procs[(cfg, noisy)] = subprocess.Popen(args, env=env, cwd=ROOT, stdin=subprocess.DEVNULL)

    def path(self, cfg: int, noisy: bool) -> str:
        return os.path.join(self.dir, f"tower_{cfg}_{'noisy' if noisy else 'trace'}.npz")

    def result(self, cfg: int, noisy: bool, timeout_s: float = 1500.0) -> Dict[str, np.ndarray]:
        p = self.procs[(cfg, noisy)]
        rc = p.wait(timeout=timeout_s)
        if rc != 0:
            raise RuntimeError(f"oracle child for workload {cfg} ({'noisy' if noisy else 'trace'}) exited {rc}")
        with np.load(self.path(cfg, noisy), allow_pickle=False) as z:
            return {k: z[k] for k in z.files}

    def stop(self) -> None:
        for p in self.procs.values():
            if p.poll() is None:
                p.kill()
                p.wait()


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    compute(int(sys.argv[1]), sys.argv[2] == "noisy", sys.argv[3])
