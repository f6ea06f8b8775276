"""Benchmark of the ViT vision-tower forward on one MI355X.

One step = one whole forward of the 27-block tower with its four mergers
(patch embed, 27 x [LN-quant, QKV FP8 GEMM, RoPE, attention, quant, proj,
LN-quant, FC1 (+GELU, requant), FC2], 4 x [merge + LN, fc1 + GELU, fc2]) on
one synthetic image of 46 x 136 = 6256 patches, inputs resident in HBM.

Prints ONE JSON line.  `value` is milliseconds per image (lower is better).
The `roofline` object is the attention kernel (the tower's largest cost):
algorithmic FLOPs per launch (4 * P^2 * 1152) over its average launch
duration, measured here with HIP events on the stream it runs on, at the
launch configuration the tower uses; its fraction is given against the
published bf16 peak and against the peak a dense-MFMA loop reaches on this
chip in the same run (`measured_peaks`).  `kernels` gives the same for
every kernel of the step.  `sizes` repeats the forward at 972, 1824, 3888
and 6256 patches and on the packed 972 + 3888 + 1824 batch (eager and as
one HIP graph), with the attention alone at each size.  `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of each workload (the
per-config figures state what was timed and what was scaled).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload encoder_p6256]
                       [--no-cpu-baseline] [--no-kernels] [--no-sizes]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published

METRIC = "ViT fwd ms/image @6256 patches; attention TFLOP/s as % of MI355X bf16 MFMA peak"

WORKLOADS = {
    "encoder_p6256": dict(grids=[(46, 136)], cfg=3,
                          desc="27-block ViT tower + 4 mergers, 1 image of 46x136 = 6256 patches"),
    "encoder_varlen_6684": dict(grids=[(18, 54), (36, 108), (24, 76)], cfg=4,
                                desc="27-block ViT tower + 4 mergers, 3 packed images of 972 + 3888 + 1824 patches"),
    "encoder_p3888": dict(grids=[(36, 108)], cfg=3, desc="27-block ViT tower + 4 mergers, 1 image of 3888 patches"),
    "encoder_p1824": dict(grids=[(24, 76)], cfg=3, desc="27-block ViT tower + 4 mergers, 1 image of 1824 patches"),
    "encoder_p972": dict(grids=[(18, 54)], cfg=3, desc="27-block ViT tower + 4 mergers, 1 image of 972 patches"),
}


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and layout are left out,
    so that a comment edit does not orphan counters taken on the same code."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "vision_transformer_encoder_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            text = open(os.path.join(csrc, f), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(f.encode() + b"\0" + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_hash") != kernel_source_hash():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def encoder_flops(seq_lens, depth=27, n_mergers=4):
    """Algorithmic FLOPs of one forward (2 per multiply-add; no padding)."""
    H, MLP, PD, MD, OUT = 1152, 4304, 1536, 4608, 4096
    T = sum(seq_lens)
    d = dict(attention=depth * sum(4 * p * p * H for p in seq_lens),
             gemm=depth * 2 * T * H * (3 * H + H + MLP + MLP),
             patch=2 * T * PD * H, mergers=n_mergers * 2 * (T // 4) * MD * (MD + OUT))
    d["total"] = sum(d.values())
    return d


def _host_info():
    """Cores this process may run on, the BLAS numpy calls (vendor, version,
    threads) and the CPU model."""
    info = {"affinity_cores": len(os.sched_getaffinity(0))}
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(blas[0].get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return info


def cpu_baseline(grids, cfg):
    """The fp64 oracle (storage-emulating and pure modes) timed on the host
    on a bounded sample of each workload, about 20-30 s of CPU work:
    the single block (256 patches) and the attention-only case (1824
    patches) whole; the FP8 GEMM sweep at M = 6256 whole (storage mode);
    for the two full towers the patch embed, one block and one merger,
    scaled to 27 blocks and 4 mergers (pure mode of the packed batch scaled
    from its storage time by the single image's pure / storage ratio)."""
    import numpy as np
    import oracle as O
    import synth
    from oracle import inputs as OI

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    def block_w(c, i):
        w = OI.block_weights(synth.block_params(c, i))
        for n in ("qkv", "proj", "fc1", "fc2"):
            w.fp8(n)  # weight preparation is not part of a forward
        return w

    per = {}
    t_all = time.perf_counter()
    # one block on a 16 x 16 grid (256 patches)
    g0 = [(16, 16)]
    x0 = synth.bf16_bits_to_f64(synth.normal_bf16(0, "x", 0, (256, 1152)))
    w0 = block_w(0, 0)
    p0, c0 = O.positions_from_grids(g0), O.cu_seqlens_from_grids(g0)
    per["block_p256"] = {m: round(1e3 * timed(lambda: O.block_forward(x0, w0, p0, c0, mode=m)), 1)
                         for m in ("storage", "pure")}
    per["block_p256"].update(unit="ms per block", timed="whole")
    # attention alone on a 48 x 38 grid (1824 patches; the same in both modes)
    g1 = [(48, 38)]
    q1, k1, v1 = (synth.bf16_bits_to_f64(synth.normal_bf16(1, t, 0, (1824, 1152))) for t in ("q", "k", "v"))
    ta = timed(lambda: O.attention(q1, k1, v1, O.cu_seqlens_from_grids(g1)))
    per["attention_p1824"] = {"storage": round(1e3 * ta, 1), "pure": round(1e3 * ta, 1),
                              "unit": "ms per call", "timed": "whole (attention has no storage points)"}
    # the four FP8 GEMMs of a block at M = 6256 with their epilogues
    a_c, a_s = O.quantize_block128(synth.bf16_bits_to_f64(synth.normal_bf16(2, "a", 0, (6256, 1152))), 1)
    h_c, h_s = O.quantize_block128(synth.bf16_bits_to_f64(synth.normal_bf16(2, "a", 1, (6256, 4352))), 1)
    wb = block_w(2, 0)
    res = synth.bf16_bits_to_f64(synth.normal_bf16(2, "residual", 0, (6256, 1152)))

    def sweep():
        for n, (ac, as_), N, epi in (("qkv", (a_c, a_s), 3456, O.EPI_BIAS), ("proj", (a_c, a_s), 1152,
                                                                              O.EPI_BIAS_RESIDUAL),
                                     ("fc1", (a_c, a_s), 4304, O.EPI_BIAS_GELU_FP8),
                                     ("fc2", (h_c, h_s), 1152, O.EPI_BIAS_RESIDUAL)):
            f = wb.fp8(n)
            O.fp8_gemm_epilogue(O.fp8_block128_gemm(ac, as_, f.codes, f.scales), N, epi,
                                bias=getattr(wb, n + "_b"), residual=res)
    per["gemm_sweep_m6256"] = {"storage": round(1e3 * timed(sweep), 1), "unit": "ms per sweep (4 GEMMs)",
                               "timed": "whole, storage mode (pure differs only in the bf16 rounding of "
                                        "the outputs; not timed separately)"}
    # the towers (one 46 x 136 image; the 972 + 3888 + 1824 batch), sampled
    for name, c, gr in (("encoder_p6256", 3, [(46, 136)]), ("encoder_varlen_6684", 4, [(18, 54), (36, 108),
                                                                                      (24, 76)])):
        T = sum(h * w for h, w in gr)
        pos, cu = O.positions_from_grids(gr), O.cu_seqlens_from_grids(gr)
        pp = synth.patch_params(c)
        ew = O.EncoderWeights(patch_w=OI.dec(pp["patch_w"]), patch_b=OI.dec(pp["patch_b"]), blocks=[], mergers=[])
        px = synth.pixels(c, T).astype(np.float64)
        bw = block_w(c, 0)
        mw = OI.merger_weights(synth.merger_params(c, 0))
        rec = {"unit": "ms per image", "images": len(gr)}
        for m in (("storage", "pure") if c == 3 else ("storage",)):
            box = {}
            tp = timed(lambda: box.update(x=O.patch_embed(px, ew, mode=m)))
            tb = timed(lambda: box.update(x=O.block_forward(box["x"], bw, pos, cu, mode=m)))
            tm = timed(lambda: O.merger_forward(box["x"], mw, gr, mode=m))
            total = tp + 27 * tb + 4 * tm
            rec[m] = round(1e3 * total / len(gr), 1)
            rec[m + "_measured_s"] = {"patch_embed": round(tp, 2), "block": round(tb, 2), "merger": round(tm, 2)}
        rec["timed"] = "patch embed + 1 of 27 blocks + 1 of 4 mergers, scaled to 27 blocks + 4 mergers"
        per[name] = rec
    v = per["encoder_varlen_6684"]
    s3 = per["encoder_p6256"]
    v["pure"] = round(v["storage"] * s3["pure"] / s3["storage"], 1)
    v["timed"] += "; pure mode scaled by the 6256-patch pure / storage ratio"
    measured = time.perf_counter() - t_all
    info = _host_info()
    used = min(info["affinity_cores"], info.get("blas_threads", info["affinity_cores"]))
    head = per["encoder_p6256"]
    return {"value": head["storage"], "unit": "ms/image", "cores": used, "kind": "oracle",
            "sample": ("27-block tower at 6256 patches, storage-emulating fp64 oracle: patch embed + 1 of 27 "
                       "blocks + 1 of 4 mergers timed, scaled to 27 blocks + 4 mergers; every workload in "
                       "per_config"),
            "measured_s": round(measured, 1), "per_config": per, **info,
            "threads_note": "BLAS calls use blas_threads threads; numpy's elementwise work runs on one"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="encoder_p6256", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel event timings")
    ap.add_argument("--no-sizes", action="store_true",
                    help="skip the forward at the other image sizes (972 / 1824 / 3888 patches, varlen batch)")
    ap.add_argument("--bf16-blocks", type=int, default=0,
                    help="precision variant: the first N blocks run LayerNorm and GEMMs in bf16 (the pages keep 3)")
    ap.add_argument("--fp8-mergers", action="store_true", help="precision variant: FP8 merger linears")
    ap.add_argument("--pos-table", action="store_true",
                    help="add the learned 48x48 position table, resampled to the grid, after the patch embedding")
    ap.add_argument("--graph", action="store_true",
                    help="capture the whole forward once as a HIP graph and time its replays")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--kernel", default=None,
                    help="only launch this kernel of the step (eagerly, --kernel-reps times) and report its "
                         "timing: the program the per-kernel counter profiles run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs the tower on one GPU; --gpus {args.gpus} is not supported "
              "(a packed batch would shard by image across GPUs with no exchange)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import vision_transformer_encoder_amd as vit

    vit.require_library()
    dev = torch.device("cuda:0")
    wl = WORKLOADS[args.workload]
    grids, cfg = wl["grids"], wl["cfg"]
    T = sum(h * w for h, w in grids)
    nimg = len(grids)

    print(f"[bench] workload {args.workload}: T={T}, images={nimg}", file=sys.stderr, flush=True)
    if args.kernel:
        # weights of one block and one merger suffice for a single kernel
        ep = synth.EncoderParams(patch=synth.patch_params(cfg), blocks=[synth.block_params(cfg, 0)] * 27,
                                 mergers=[synth.merger_params(cfg, 0)] * 4)
        W = vit.EncoderWeights(ep.patch, ep.blocks, ep.mergers, dev)
        k = time_kernels(vit, W, T, grids, dev, args.kernel_reps, [h * w for h, w in grids],
                         only=args.kernel, eager=True)
        print(json.dumps({"kernel": args.kernel, "workload": args.workload, **k[args.kernel]}), flush=True)
        return 0
    ep = synth.encoder_params(cfg)
    pos_table = synth.normal_bf16(cfg, "pos_table", 48, (48 * 48, 1152), std=0.02) if args.pos_table else None
    W = vit.EncoderWeights(ep.patch, ep.blocks, ep.mergers, dev, bf16_blocks=args.bf16_blocks,
                           fp8_mergers=args.fp8_mergers, pos_table=pos_table)
    variant = args.bf16_blocks > 0 or args.fp8_mergers or args.pos_table
    if variant:
        args.no_kernels = True  # the per-kernel timing replays the all-FP8 block sequence
    px = torch.from_numpy(synth.pixels(cfg, T)).to(dev)
    g_host = np.asarray(grids, dtype=np.int32).reshape(-1, 2)
    g_dev = torch.from_numpy(g_host.copy()).to(dev)
    ws = torch.empty(vit.vit_encoder_workspace_size(T, nimg), dtype=torch.uint8, device=dev)
    out = torch.empty((4, T // 4, 4096), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    print("[bench] weights ready", file=sys.stderr, flush=True)

    def step():
        vit.vit_encoder_forward(W, px, grids, workspace=ws, out=out, grid_dev=g_dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    run = step
    if args.graph:
        # the forward allocates nothing and never synchronises: its ~250
        # launches are captured as one graph on torch's capture stream
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        print("[bench] forward captured as a HIP graph", file=sys.stderr, flush=True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        run()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    print(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f})",
          file=sys.stderr, flush=True)
    ok = bool(torch.isfinite(out.float()).all().item())

    flops = encoder_flops([h * w for h, w in grids])
    seq = [h * w for h, w in grids]
    peaks = measured_peaks(dev)
    kernels = {}
    roofline = None
    if not args.no_kernels:
        kernels = time_in_context(vit, W, px, grids, g_dev, dev, max(1, min(args.steps, 5)), peaks)
        a = kernels["attention"]
        roofline = {"bound": "mfma", "achieved": a["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(a["tflops"] / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic_from_profiles("attention"),
                    "kernel": "attention_kernel", "avg_launch_us": a["us"],
                    "algorithmic_flop_per_launch": a["flop"],
                    "peak_measured": peaks["bf16_tflops"],
                    "frac_measured": round(a["tflops"] / peaks["bf16_tflops"], 4)}
    sizes = None
    if not args.no_sizes and not variant:
        sizes = time_sizes(vit, W, dev, peaks, main=(args.workload, ms_per_step))

    line = {
        "metric": METRIC,
        "value": round(ms_per_step / nimg, 4),
        "unit": "ms/image",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"mean": round(ms_per_step, 4), "median": round(per_step_ms[len(per_step_ms) // 2], 4),
                    "min": round(per_step_ms[0], 4)},
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 GEMMs + bf16 attention, fp32 accumulate",
        "data": "synthetic (seeded; random-init weights of the tower's shapes)",
        "config": {"workload": args.workload, "description": wl["desc"], "patches": T, "images": nimg,
                   "grids": grids, "blocks": 27, "mergers": 4},
        "throughput": {"tflops_total": round(flops["total"] / (ms_per_step * 1e-3) / 1e12, 1),
                       "algorithmic_gflop_per_step": round(flops["total"] / 1e9, 1),
                       "images_per_s": round(1e3 * nimg / ms_per_step, 2)},
        "outputs_finite": ok,
        "launch": "hip_graph" if args.graph else "eager",
        "precision": {"bf16_blocks": args.bf16_blocks, "fp8_mergers": bool(args.fp8_mergers)},
        "position_table": "learned 48x48, resampled per image" if args.pos_table else None,
    }
    line["measured_peaks"] = peaks
    if sizes is not None:
        line["sizes"] = sizes
    if roofline is not None:
        line["roofline"] = roofline
        line["kernels"] = kernels
        per_step = {k: v["us"] * v["per_step"] for k, v in kernels.items()}
        line["kernel_time_share"] = {k: round(v / (ms_per_step * 1e3), 3) for k, v in per_step.items()}
        line["kernel_timing"] = ("average duration of each launch inside the running forward (the tower "
                                 "run as its per-op C-ABI calls, HIP events on the launch stream)")
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(grids, cfg)
    print(json.dumps(line), flush=True)
    return 0 if ok else 1


def _kernel_record(us, per_step, work, unit, peaks=None):
    r = {"us": round(us, 2), "per_step": per_step}
    if unit == "B":
        gbs = work / (us * 1e-6) / 1e9
        r.update(bytes=int(work), gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 3))
        if peaks:
            r["frac_hbm_measured"] = round(gbs / peaks["copy_gbs"], 3)
    else:
        tf = work / (us * 1e-6) / 1e12
        peak = PEAK_FP8_TFLOPS if unit == "F8" else PEAK_BF16_TFLOPS
        r.update(flop=int(work), tflops=round(tf, 1), frac_mfma=round(tf / peak, 4))
        if peaks:
            r["frac_mfma_measured"] = round(tf / peaks["fp8_tflops" if unit == "F8" else "bf16_tflops"], 4)
    return r


def measured_peaks(dev):
    """What this chip reaches in this run: dense MFMA loops of the two
    matrix instructions the kernels use (libvit_peak.so, two waves per SIMD
    on every CU) and a 2 x 512 MB device copy (read + write bytes)."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "vision_transformer_encoder_amd", "libvit_peak.so"))
    lib.vit_peak_mfma.restype = ctypes.c_int
    lib.vit_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.vit_peak_mfma_flops.restype = ctypes.c_double
    lib.vit_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wgs = 2 * cus
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    res = {"compute_units": cus}
    for kind, name, iters in ((0, "bf16_tflops", 20000), (1, "fp8_tflops", 10000)):
        best = 0.0
        for rep in range(4):  # the first launch warms the clocks up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if lib.vit_peak_mfma(kind, iters, wgs, out.data_ptr(), ctypes.c_void_p(stream.cuda_stream)) != 0:
                raise RuntimeError("MFMA peak probe failed to launch")
            e1.record(stream)
            torch.cuda.synchronize()
            if rep > 0:
                best = max(best, lib.vit_peak_mfma_flops(kind, iters, wgs) / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        res[name] = round(best, 1)
    src = torch.empty(256 * 1024 * 1024, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    best = 0.0
    for rep in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        if rep > 0:
            best = max(best, 2 * src.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    res["copy_gbs"] = round(best, 1)
    res["frac_of_published"] = {"bf16": round(res["bf16_tflops"] / PEAK_BF16_TFLOPS, 3),
                                "fp8": round(res["fp8_tflops"] / PEAK_FP8_TFLOPS, 3),
                                "hbm": round(res["copy_gbs"] / PEAK_HBM_GBS, 3)}
    print(f"[bench] measured peaks: {res}", file=sys.stderr, flush=True)
    del src, dst
    return res


SIZES = ("encoder_p972", "encoder_p1824", "encoder_p3888", "encoder_p6256", "encoder_varlen_6684")


def time_sizes(vit, W, dev, peaks, main=None, steps=10, warmup=3):
    """The whole forward at each image size of the pages' resolution table
    and on the packed batch: ms per step eager and replayed as one HIP
    graph, whole-forward TFLOP/s, and the attention alone (main + combine
    kernels, `steps` back-to-back launches in a graph) with its fraction of
    the published and the measured bf16 peak.  Weights are those of the
    headline workload (timing does not depend on their values)."""
    import numpy as np
    import torch

    import synth

    stream = torch.cuda.current_stream()
    out = {}
    for name in SIZES:
        grids = WORKLOADS[name]["grids"]
        seq = [h * w for h, w in grids]
        T = sum(seq)
        px = torch.from_numpy(synth.pixels(WORKLOADS[name]["cfg"], T)).to(dev)
        g_dev = torch.from_numpy(np.asarray(grids, np.int32).reshape(-1, 2)).to(dev)
        ws = torch.empty(vit.vit_encoder_workspace_size(T, len(grids)), dtype=torch.uint8, device=dev)
        o = torch.empty((4, T // 4, 4096), dtype=torch.bfloat16, device=dev)

        def step():
            vit.vit_encoder_forward(W, px, grids, workspace=ws, out=o, grid_dev=g_dev)

        def timed(run):
            for _ in range(warmup):
                run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps

        eager = timed(step)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        replay = timed(graph.replay)
        del graph
        # attention alone at this size
        H = 1152
        qkv = torch.randn((T, 3 * H), device=dev).to(torch.bfloat16)
        cu = np.concatenate([[0], np.cumsum(seq)]).astype(np.int32)
        cu_dev = torch.from_numpy(cu).to(dev)
        ao = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        aws = torch.empty(vit.vit_attention_workspace_size(), dtype=torch.uint8, device=dev)

        def attn():
            vit.vit_attention(qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], cu, cu_seqlens_dev=cu_dev, out=ao,
                              workspace=aws)

        attn()
        torch.cuda.synchronize()
        ag = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ag):
            for _ in range(steps):
                attn()
        ag.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ag.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        a_us = e0.elapsed_time(e1) * 1e3 / steps
        del ag
        fl = encoder_flops(seq)
        a_tf = sum(4 * p * p * H for p in seq) / (a_us * 1e-6) / 1e12
        ms = eager
        if main is not None and main[0] == name:
            ms = main[1]  # the headline measurement of this run
        out[name] = {"patches": T, "images": len(grids), "ms_per_step_eager": round(eager, 3),
                     "ms_per_step_graph": round(replay, 3), "ms_per_image": round(ms / len(grids), 3),
                     "tflops": round(fl["total"] / (ms * 1e-3) / 1e12, 1),
                     "attention_us": round(a_us, 1), "attention_tflops": round(a_tf, 1),
                     "attention_frac": round(a_tf / PEAK_BF16_TFLOPS, 4),
                     "attention_frac_measured": round(a_tf / peaks["bf16_tflops"], 4)}
        print(f"[bench] size {name}: {out[name]}", file=sys.stderr, flush=True)
        del px, ws, o, qkv, ao, aws
    return out


def kernel_work(T, seq):
    """Algorithmic work of one launch of each kernel of the forward and how
    many launches one forward makes: name -> (work, unit, per_step); unit
    "B" = HBM bytes, "F8" / "F16" = FLOPs of an FP8 / bf16 MFMA kernel."""
    H, B, TM = 1152, 27, T // 4
    gemm = lambda n, k: 2 * T * n * k
    return {
        "layernorm_quant": (T * (H * 2 + H + 9 * 4), "B", 2 * B),
        "fp8_gemm_qkv": (gemm(3 * H, H), "F8", B),
        "rope2d": (T * 2 * H * 2 * 2 + T * 8, "B", B),
        "attention": (sum(4 * p * p * H for p in seq), "F16", B),
        "quant_rows": (T * (H * 2 + H + 9 * 4), "B", B),
        "fp8_gemm_proj": (gemm(H, H), "F8", B),
        "fp8_gemm_fc1_gelu_quant": (gemm(4304, H), "F8", B),
        "fp8_gemm_fc2": (gemm(H, 4304), "F8", B),
        "patch_embed_bf16": (gemm(H, 1536), "F16", 1),
        "merge_layernorm": (2 * T * H * 2, "B", 4),
        "merger_fc1_bf16": (2 * TM * 4608 * 4608, "F16", 4),
        "merger_fc2_bf16": (2 * TM * 4096 * 4608, "F16", 4),
    }


def time_in_context(vit, W, px, grids, g_dev, dev, steps, peaks=None):
    """Average duration of every kernel inside the running forward: the
    tower is run as the sequence of per-op C-ABI calls vit_encoder_forward
    makes (same kernels, shapes and order, on the same stream), with HIP
    events recorded on that stream around every launch."""
    import collections

    import numpy as np
    import torch

    H = 1152
    T = px.shape[0]
    seq = [h * w for h, w in grids]
    cu = np.concatenate([[0], np.cumsum(seq)]).astype(np.int32)
    cu_dev = torch.from_numpy(cu).to(dev)
    pos = torch.from_numpy(np.concatenate([np.stack(np.meshgrid(np.arange(h), np.arange(w), indexing="ij"), -1)
                                           .reshape(-1, 2) for h, w in grids]).astype(np.int32)).to(dev)
    x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    qkv = torch.empty((T, 3 * H), dtype=torch.bfloat16, device=dev)
    o = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    aws = torch.empty(vit.vit_attention_workspace_size(), dtype=torch.uint8, device=dev)
    # every intermediate is allocated once, as the C-ABI forward does: an
    # allocation between two events could stall the host while the GPU idles
    # between them
    u8, f32 = torch.uint8, torch.float32
    ln_q = (torch.empty((T, H), dtype=u8, device=dev), torch.empty((T, H // 128), dtype=f32, device=dev))
    o_q = (torch.empty((T, H), dtype=u8, device=dev), torch.empty((T, H // 128), dtype=f32, device=dev))
    h_q = (torch.empty((T, 4352), dtype=u8, device=dev), torch.empty((T, 4352 // 128), dtype=f32, device=dev))
    y_m = torch.empty((T // 4, 4 * H), dtype=torch.bfloat16, device=dev)
    h_m = torch.empty((T // 4, 4 * H), dtype=torch.bfloat16, device=dev)
    z_m = torch.empty((T // 4, 4096), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    spans = collections.defaultdict(list)

    recording = False

    def timed(name, fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # ~0.1 ms of GPU sleep first: the host queues the start event, the op
        # and the end event while the GPU is still busy, so no host-side gap
        # of the Python per-op calls falls inside the interval
        torch.cuda._sleep(200_000)
        e0.record(stream)
        r = fn()
        e1.record(stream)
        if recording:
            spans[name].append((e0, e1))
        return r

    taps = {8: 0, 16: 1, 24: 2, 27: 3}
    # the first pass through the per-op calls is not recorded: one-time
    # costs on first use (tens of ms) would otherwise land inside whichever
    # event pair is open and inflate that kernel's average
    for step in range(steps + 1):
        recording = step > 0
        timed("patch_embed_bf16", lambda: vit.vit_bf16_gemm(px, W.patch["patch_w"], bias=W.patch["patch_b"], out=x))
        for b in range(27):
            t, q = W.blocks[b].t, W.blocks[b].q
            a_c, a_s = timed("layernorm_quant", lambda: vit.vit_layernorm_quant_fp8(x, t["ln1_g"], t["ln1_b"], out=ln_q))
            timed("fp8_gemm_qkv", lambda: vit.vit_fp8_block128_gemm(a_c, a_s, q["qkv"][0], q["qkv"][1], 3 * H, H,
                                                                    bias=t["qkv_b"], out=qkv))
            timed("rope2d", lambda: vit.vit_rope2d(qkv[:, :H], qkv[:, H:2 * H], pos))
            timed("attention", lambda: vit.vit_attention(qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], cu,
                                                         cu_seqlens_dev=cu_dev, out=o, workspace=aws))
            o_c, o_s = timed("quant_rows", lambda: vit.vit_quant_fp8_block128(o, out=o_q))
            timed("fp8_gemm_proj", lambda: vit.vit_fp8_block128_gemm(o_c, o_s, q["proj"][0], q["proj"][1], H, H,
                                                                     bias=t["proj_b"], residual=x,
                                                                     epilogue=vit.EPI_BIAS_RESIDUAL, out=x))
            a_c, a_s = timed("layernorm_quant", lambda: vit.vit_layernorm_quant_fp8(x, t["ln2_g"], t["ln2_b"], out=ln_q))
            h_c, h_s = timed("fp8_gemm_fc1_gelu_quant",
                             lambda: vit.vit_fp8_block128_gemm(a_c, a_s, q["fc1"][0], q["fc1"][1], 4304, H,
                                                               bias=t["fc1_b"], epilogue=vit.EPI_BIAS_GELU_FP8,
                                                               out=h_q))
            timed("fp8_gemm_fc2", lambda: vit.vit_fp8_block128_gemm(h_c, h_s, q["fc2"][0], q["fc2"][1], H, 4304,
                                                                    bias=t["fc2_b"], residual=x,
                                                                    epilogue=vit.EPI_BIAS_RESIDUAL, out=x))
            if b + 1 in taps:
                m = W.mergers[taps[b + 1]].t
                y = timed("merge_layernorm",
                          lambda: vit.vit_merge2x2_layernorm(x, grids, m["m_ln_g"], m["m_ln_b"], grid_dev=g_dev,
                                                             out=y_m, cu_dev=cu_dev))
                hh = timed("merger_fc1_bf16", lambda: vit.vit_bf16_gemm(y, m["m_fc1_w"], bias=m["m_fc1_b"],
                                                                        epilogue=vit.BEPI_BIAS_GELU, out=h_m))
                timed("merger_fc2_bf16", lambda: vit.vit_bf16_gemm(hh, m["m_fc2_w"], bias=m["m_fc2_b"], out=z_m))
    torch.cuda.synchronize()
    work = kernel_work(T, seq)
    res = {}
    for name, sp in spans.items():
        us = sum(e0.elapsed_time(e1) for e0, e1 in sp) * 1e3 / len(sp)
        w, unit, per_step = work[name]
        res[name] = _kernel_record(us, per_step, w, unit, peaks)
        print(f"[bench] in forward: {name}: {res[name]}", file=sys.stderr, flush=True)
    return res


def time_kernels(vit, W, T, grids, dev, reps, seq, only=None, eager=False):
    """Average launch duration of each kernel of the step, at the shapes and
    launch configuration the tower uses, measured with HIP events on the
    current stream (the stream every launch goes to)."""
    import numpy as np
    import torch

    H = 1152
    b0 = W.blocks[0]
    t = b0.t
    q = b0.q
    x = torch.randn((T, H), device=dev).to(torch.bfloat16)
    pos = torch.from_numpy(np.concatenate([np.stack(np.meshgrid(np.arange(h), np.arange(w), indexing="ij"), -1)
                                           .reshape(-1, 2) for h, w in grids]).astype(np.int32)).to(dev)
    cu = np.concatenate([[0], np.cumsum([h * w for h, w in grids])]).astype(np.int32)
    cu_dev = torch.from_numpy(cu).to(dev)
    g_dev = torch.from_numpy(np.asarray(grids, np.int32).reshape(-1, 2)).to(dev)
    qkv = torch.randn((T, 3 * H), device=dev).to(torch.bfloat16)
    a_c, a_s = vit.vit_layernorm_quant_fp8(x, t["ln1_g"], t["ln1_b"])
    h_c, h_s = vit.vit_fp8_block128_gemm(a_c, a_s, q["fc1"][0], q["fc1"][1], 4304, 1152, bias=t["fc1_b"],
                                         epilogue=vit.EPI_BIAS_GELU_FP8)
    o = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    xr = x.clone()
    m = W.mergers[0].t
    TM = T // 4
    mln = torch.randn((TM, 4608), device=dev).to(torch.bfloat16)
    mh = torch.empty((TM, 4608), dtype=torch.bfloat16, device=dev)
    mo = torch.empty((TM, 4096), dtype=torch.bfloat16, device=dev)
    px = torch.rand((T, 1536), device=dev) * 2 - 1
    xp = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ptab = torch.randn((48 * 48, H), device=dev).to(torch.bfloat16)
    pe_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    cpy_src = torch.randn((T, 4096), device=dev).to(torch.bfloat16)
    cpy_dst = torch.empty_like(cpy_src)
    att_flop = sum(4 * p * p * H for p in seq)
    gemm = lambda n, k: 2 * T * n * k
    B = 27
    cases = {
        # name: (callable, work, unit, per_step)
        "layernorm_quant": (lambda: vit.vit_layernorm_quant_fp8(x, t["ln1_g"], t["ln1_b"]),
                            T * (H * 2 + H + 9 * 4), "B", 2 * B),
        "fp8_gemm_qkv": (lambda: vit.vit_fp8_block128_gemm(a_c, a_s, q["qkv"][0], q["qkv"][1], 3 * H, H,
                                                           bias=t["qkv_b"], out=qkv), gemm(3 * H, H), "F8", B),
        "rope2d": (lambda: vit.vit_rope2d(qkv[:, :H], qkv[:, H:2 * H], pos), T * 2 * H * 2 * 2 + T * 8, "B", B),
        "attention": (lambda: vit.vit_attention(qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], cu, cu_seqlens_dev=cu_dev,
                                                out=o), att_flop, "F16", B),
        "quant_rows": (lambda: vit.vit_quant_fp8_block128(o), T * (H * 2 + H + 9 * 4), "B", B),
        "fp8_gemm_proj": (lambda: vit.vit_fp8_block128_gemm(a_c, a_s, q["proj"][0], q["proj"][1], H, H,
                                                            bias=t["proj_b"], residual=xr,
                                                            epilogue=vit.EPI_BIAS_RESIDUAL, out=xr),
                          gemm(H, H), "F8", B),
        "fp8_gemm_fc1_gelu_quant": (lambda: vit.vit_fp8_block128_gemm(a_c, a_s, q["fc1"][0], q["fc1"][1], 4304, H,
                                                                      bias=t["fc1_b"],
                                                                      epilogue=vit.EPI_BIAS_GELU_FP8),
                                    gemm(4304, H), "F8", B),
        "fp8_gemm_fc2": (lambda: vit.vit_fp8_block128_gemm(h_c, h_s, q["fc2"][0], q["fc2"][1], H, 4304,
                                                           bias=t["fc2_b"], residual=xr,
                                                           epilogue=vit.EPI_BIAS_RESIDUAL, out=xr),
                         gemm(H, 4304), "F8", B),
        "patch_embed_bf16": (lambda: vit.vit_bf16_gemm(px, W.patch["patch_w"], bias=W.patch["patch_b"], out=xp),
                             gemm(H, 1536), "F16", 1),
        "merge_layernorm": (lambda: vit.vit_merge2x2_layernorm(x, grids, m["m_ln_g"], m["m_ln_b"], grid_dev=g_dev,
                                                               cu_dev=cu_dev), 2 * T * H * 2, "B", 4),
        "merger_fc1_bf16": (lambda: vit.vit_bf16_gemm(mln, m["m_fc1_w"], bias=m["m_fc1_b"],
                                                      epilogue=vit.BEPI_BIAS_GELU, out=mh),
                            2 * TM * 4608 * 4608, "F16", 4),
        "merger_fc2_bf16": (lambda: vit.vit_bf16_gemm(mh, m["m_fc2_w"], bias=m["m_fc2_b"], out=mo),
                            2 * TM * 4096 * 4608, "F16", 4),
    }
    # input preparation of the page's image (not part of the timed forward):
    # 2172 x 724 u8 RGB read once, 6256 x 1536 f32 written
    frames_u8 = (torch.rand((1, 724, 2172, 3), device=dev) * 255).to(torch.uint8)
    pre_out = torch.empty((6256, 1536), dtype=torch.float32, device=dev)
    cases["preprocess"] = (lambda: vit.vit_preprocess_frames(frames_u8, (736, 2176), (0.5, 0.5, 0.5),
                                                             (0.5, 0.5, 0.5), out=pre_out),
                           724 * 2172 * 3 + 6256 * 1536 * 4, "B", 0)
    # the learned position table resampled to the grids (only with --pos-table
    # in the forward): the table read once, the [T, 1152] result written
    cases["pos_embed_interp"] = (lambda: vit.vit_pos_embed_interp(ptab, grids, out=pe_out, grid_dev=g_dev,
                                                                  cu_dev=cu_dev),
                                 48 * 48 * H * 2 + T * H * 2, "B", 0)
    # a plain copy of known size: the reference for the HBM byte counters
    cases["copy_calibration"] = (lambda: cpy_dst.copy_(cpy_src), 2 * cpy_src.numel() * 2, "B", 0)
    res = {}
    for name, (fn, work, unit, per_step) in cases.items():
        if only is None and per_step == 0:
            continue
        if only is not None and name != only:
            continue
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        if eager:
            stream = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            res[name] = _kernel_record(us, per_step, work, unit)
            continue
        # back-to-back launches without host gaps: capture `reps` launches in
        # a graph and time one replay on the stream it replays on
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        del graph
        r = _kernel_record(us, per_step, work, unit)
        res[name] = r
        print(f"[bench] {name}: {r}", file=sys.stderr, flush=True)
    return res


if __name__ == "__main__":
    sys.exit(main())
