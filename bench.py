#!/usr/bin/env python3
"""Throughput of the native-resolution ViT encoder on one MI355X.

One step = patchify -> 32-block tower -> PatchMerger over one batch of
synthetic images whose pixels, weights and metadata are already resident in
HBM.  Default workload: one 448x448 image (32x32 patches -> 256 merged
tokens), Qwen2-VL-2B tower (1280 wide, 16 heads, MLP 5120, QuickGELU),
merger 5120 -> 1536, bf16 operands with f32 accumulation.

Prints ONE JSON line: merged tokens/s (value, from K steps with nothing else
on the stream), patches/s, the fraction of the bf16 MFMA peak the whole step
reaches, a per-kernel-class breakdown, the roofline of the dominant kernel
(algorithmic FLOPs per launch / its average launch time from hipEvent pairs
recorded by the library on the launch stream around every launch of that
kernel during K further timed steps) and the CPU oracle (float32 mode) timed
on the host as a reported baseline.  The default invocation also measures
the 3584x3584 image (65,536 patches -> 16,384 merged tokens, merger to 3584)
in the same run and reports it under "configs", with its own roofline
(attention) and a CPU baseline extrapolated from a bounded oracle sample."""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def workload_flops(wl, grids, fold=False):
    """Algorithmic FLOPs of one step: true K (1176), block-diagonal attention
    (sum n_i^2 over images, or over windows in the windowed blocks), matrix
    products only.  "attention" is the average over the step's blocks."""
    ns = [t * gh * gw for t, gh, gw in grids]
    n, m = sum(ns), sum(ns) // 4
    d, f, pd, hid = wl.dim, wl.mlp, wl.patch_dim, wl.merged_dim
    att_full = 4 * d * sum(x * x for x in ns)
    att = att_full
    if wl.window and wl.depth:
        W = wl.window
        sq = 0
        for t, gh, gw in grids:
            rows = [min(W, gh - y) for y in range(0, gh, W)]
            cols = [min(W, gw - x) for x in range(0, gw, W)]
            sq += t * sum((r * c) ** 2 for r in rows for c in cols)
        nfull = sum(1 for b in wl.full_blocks if b < wl.depth)
        att = (nfull * att_full + (wl.depth - nfull) * 4 * d * sq) / wl.depth
    per = {
        "patch_embed": 2 * n * (wl.in_channels * wl.patch * wl.patch if fold else pd) * d,
        "qkv": 2 * n * d * 3 * d,
        "attention": att,
        "proj": 2 * n * d * d,
        "fc1": 2 * n * d * f,
        "fc2": 2 * n * f * d,
        "merge_fc1": 2 * m * hid * hid,
        "merge_fc2": 2 * m * hid * wl.out_dim,
    }
    total = per["patch_embed"] + wl.depth * (per["qkv"] + per["attention"] + per["proj"] + per["fc1"] + per["fc2"]) \
        + per["merge_fc1"] + per["merge_fc2"]
    return total, per


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "resolution_vit_vision_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch measured by rocprofv3 PMC counters (FETCH_SIZE,
    WRITE_SIZE scaled by a copy kernel), if recorded for the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    e = rec.get(f"{workload}:{kernel}")
    if not e or e.get("source_digest") != source_digest():
        return None
    return e.get("bytes_per_launch")


def _cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    return len(os.sched_getaffinity(0)), blas_threads


def cpu_baseline(wl, params, imgs):
    """The oracle as it stands, in its float32 mode (numpy, BLAS and a thread
    pool over attention items), over the whole workload on the host cores."""
    import numpy as np
    from oracle import qv_oracle as O
    cores, blas_threads = _cpu_threads()
    # whole passes over the workload until at least 10 s of CPU time (at most 4)
    passes, dt = 0, 0.0
    while passes < 4 and (passes == 0 or dt < 10.0):
        t0 = time.perf_counter()
        grids, z, out = O.encode(imgs, params, depth=wl.depth, window=wl.window, full_blocks=wl.full_blocks,
                                 dtype=np.float32)
        dt += time.perf_counter() - t0
        passes += 1
    m = out.shape[0]
    return {"value": m * passes / dt, "unit": "tokens/s", "cores": max(cores, blas_threads or 1), "kind": "oracle",
            "sample": f"whole workload ({wl.name}: {len(imgs)} image(s), {m} merged tokens, {wl.depth} blocks), "
                      f"float32 numpy, {passes} pass(es) in {dt:.1f} s",
            "seconds": dt, "passes": passes, "blas_threads": blas_threads, "affinity_cores": cores}


def cpu_baseline_extrapolated(wl, params, imgs, rows=(2048, 8192), merge_groups=2048):
    """The oracle (float32 mode) timed on a bounded sample of a workload too
    large to run whole, scaled to the whole forward and labelled so:
    patchify + patch-embed over every patch; one full-shape block evaluated at
    two counts of sampled query rows (keys and values always for every row),
    fitted as t = a + b * rows and evaluated at all rows, times the depth;
    the merger on a sample of groups scaled to all groups (it is row-linear).
    Only for unwindowed workloads (every block costs the same)."""
    import numpy as np
    from oracle import qv_oracle as O
    assert not wl.window
    cores, blas_threads = _cpu_threads()
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in wl.images]
    cu, pos, _ = O.seq_meta(grids)
    n = int(cu[-1])
    m = n // 4
    t0 = time.perf_counter()
    x = O.patchify(imgs, grids)
    z = O.patch_embed(x.astype(np.float32), params["patch_w"].astype(np.float32))
    t_embed = time.perf_counter() - t0
    del x
    angles = O.rope_angles(pos)
    bp = O.block_params(params, 0, np.float32)
    rng = np.random.default_rng(3)
    t_rows = []
    rows = tuple(min(r, n) for r in rows)
    for r in rows:
        sel = np.sort(rng.choice(n, size=r, replace=False))
        t0 = time.perf_counter()
        O.vision_block_rows(z, bp, cu, angles, sel)
        t_rows.append(time.perf_counter() - t0)
    b = (t_rows[1] - t_rows[0]) / (rows[1] - rows[0])
    a = t_rows[0] - b * rows[0]
    t_block = a + b * n
    g = min(merge_groups, m)
    t0 = time.perf_counter()
    O.patch_merge(z[:4 * g], params, dtype=np.float32)
    t_merge = (time.perf_counter() - t0) * m / g
    total = t_embed + wl.depth * t_block + t_merge
    measured = t_embed + sum(t_rows) + t_merge * g / m
    return {"value": m / total, "unit": "tokens/s", "cores": max(cores, blas_threads or 1), "kind": "oracle",
            "extrapolated": True,
            "sample": f"extrapolated from {measured:.1f} s of oracle work (float32 numpy) on {wl.name}: "
                      f"patchify + patch-embed over all {n} patches ({t_embed:.2f} s); block 0 at "
                      f"{rows[0]} and {rows[1]} sampled query rows with keys/values for all rows "
                      f"({t_rows[0]:.2f} s, {t_rows[1]:.2f} s), fitted a + b*rows = {a:.2f} s + {b * 1e3:.3f} ms/row "
                      f"and evaluated at {n} rows ({t_block:.1f} s per block) x {wl.depth} blocks; merger on "
                      f"{g} of {m} groups scaled x{m / g:.0f}",
            "seconds_estimated_forward": total, "seconds_measured": measured,
            "blas_threads": blas_threads, "affinity_cores": cores}


def copy_calibration():
    """A plain device copy of known size for scaling the HBM byte counters."""
    import torch
    n = 1 << 28  # 268M float32 = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}))


def measure(wl, steps, warmup, weights="bf16", no_fold=False, roofline_kernel=None, baseline=None, log=None):
    """Time one workload: K steps with nothing but the forward on the stream
    (value), a per-kernel-class breakdown from untimed passes, the roofline of
    the dominant matrix class from hipEvent pairs around each of its launches
    during K further steps, and the CPU baseline (None, "whole" or
    "extrapolated")."""
    import numpy as np
    import torch

    import synth
    import resolution_vit_vision_amd as qv
    from resolution_vit_vision_amd import _abi

    def say(msg):
        if log:
            print(msg, file=sys.stderr, flush=True)

    say(f"[bench] {wl.name}: drawing inputs")
    params = synth.params(wl)
    imgs = synth.pixels(wl)
    fold = not no_fold and all(f == 1 for _, _, f in wl.images)
    enc = qv.Encoder(params, imgs, depth=wl.depth, out_dim=wl.out_dim, dtype=wl.dtype, window=wl.window,
                     full_blocks=wl.full_blocks, fold=fold,
                     weights="int8" if weights == "int8" else "dtype")
    tkey = wl.name + ("+int8" if weights == "int8" else "")
    grids = enc.grids
    n = enc.n
    m = n // 4
    flops, per = workload_flops(wl, grids, fold)

    say(f"[bench] {wl.name}: {max(warmup, 1)} warm-up step(s)")
    for _ in range(max(warmup, 1)):
        enc.run()
    torch.cuda.synchronize()

    # per-kernel-class breakdown (untimed pass, one step per class)
    breakdown = {}
    for cls in _abi.KERNEL_CLASSES:
        t = qv.KernelTimer(cls)
        t.start()
        enc.run()
        ms, launches = t.stop()
        breakdown[cls] = {"ms_per_step": ms, "launches_per_step": launches}
    # the roofline line is for the slowest matrix kernel class (each class is
    # one kernel function; the LayerNorm class mixes two memory-bound kernels
    # whose single launches are 3-4x shorter than any GEMM's)
    mfma_classes = [k for k in breakdown if k in per and breakdown[k]["launches_per_step"] > 0]
    dominant = roofline_kernel or max(mfma_classes, key=lambda k: breakdown[k]["ms_per_step"])

    stream = torch.cuda.current_stream()

    def timed(k, timer=None):
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
        if timer:
            timer.start()
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(k):
            enc.run()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(k)]
        return ev[0].elapsed_time(ev[k]), time.perf_counter() - t0, per_step

    # timed region: K steps with nothing but the forward on the stream
    say(f"[bench] {wl.name}: {steps} timed step(s)")
    ms, t_wall, per_step = timed(steps)
    ms_per_step = ms / steps
    value = m * steps / (ms / 1e3)
    # roofline region: K more steps with hipEvent pairs around every launch of
    # the dominant kernel class (the pairs add a few us of stream time each,
    # which is why the throughput above is taken without them)
    timer = qv.KernelTimer(dominant)
    ms_ev, _, _ = timed(steps, timer)
    dom_ms, dom_launches = timer.stop()

    dom_avg_ms = dom_ms / max(dom_launches, 1)
    if dominant in per:
        achieved = per[dominant] / (dom_avg_ms / 1e3) / 1e12
        roofline = {"bound": "mfma", "kernel": dominant, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                    "flops_per_launch": per[dominant], "avg_launch_ms": dom_avg_ms, "launches": dom_launches,
                    "timing": "hipExtLaunchKernelGGL start/stop events around every launch of the class "
                              "(each interval also holds the launch's dispatch, ~3 us)",
                    "traffic": traffic_for(dominant, tkey)}
    else:
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": None, "avg_launch_ms": dom_avg_ms, "launches": dom_launches,
                    "traffic": traffic_for(dominant, tkey)}
    res = {
        "value": value,
        "unit": "tokens/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(np.min(per_step)),
        "dtype": wl.dtype,
        "config": {"workload": wl.name, "images": [f"{h}x{w}" for h, w, _ in wl.images][:4]
                   + (["..."] if len(wl.images) > 4 else []),
                   "n_images": len(wl.images), "patches": n, "merged_tokens": m, "depth": wl.depth,
                   "out_dim": wl.out_dim, "window": wl.window, "full_blocks": list(wl.full_blocks),
                   "patch_embed": "conv2d fold, K=592" if fold else "conv3d, K=1176",
                   "block_weights": "int8 per-row scales" if weights == "int8" else "bf16"},
        "patches_per_s": n * steps / (ms / 1e3),
        "algorithmic_tflop_per_step": flops / 1e12,
        "achieved_tflops": flops / (ms_per_step / 1e3) / 1e12,
        "frac_bf16_mfma_peak": flops / (ms_per_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "host_wall_s": t_wall,
        "ms_per_step_with_roofline_events": ms_ev / steps,
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in breakdown.items()},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    del enc
    torch.cuda.empty_cache()
    if baseline == "whole":
        say(f"[bench] {wl.name}: CPU oracle baseline (whole workload)")
        res["cpu_baseline"] = cpu_baseline(wl, params, imgs)
    elif baseline == "extrapolated":
        say(f"[bench] {wl.name}: CPU oracle baseline (sampled, extrapolated)")
        res["cpu_baseline"] = cpu_baseline_extrapolated(wl, params, imgs)
    return res


HIGH_RES = "maxres_3584"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen2vl_2b_448")
    ap.add_argument("--roofline-kernel", default=None, help="kernel class for the roofline (default: slowest)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fold", action="store_true",
                    help="keep the Conv3d patch-embed (K = 1176) for still images")
    ap.add_argument("--weights", choices=("bf16", "int8"), default="bf16",
                    help="block matrices as bf16, or int8 codes with a float32 scale per row")
    ap.add_argument("--high-res-steps", type=int, default=5,
                    help="timed steps of the 3584x3584 workload measured beside the default one (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("this encoder build runs on one GPU only: the multi-GPU path (images sharded across GPUs, "
               "K/V exchange for a single huge image) is designed but not built; run with --gpus 1")
        print(msg, file=sys.stderr)
        sys.exit(2)

    import torch  # noqa: F401

    if args.copy_calibration:
        copy_calibration()
        return

    import synth

    wl = synth.WORKLOADS[args.workload]
    small = wl.name not in (HIGH_RES, "qwen25vl_7b_3584_window", "mixed16_varlen_7b_merger", "video_448_16f")
    baseline = None if args.no_cpu_baseline else ("whole" if small else
                                                  ("extrapolated" if not wl.window else None))
    head = measure(wl, args.steps, args.warmup, args.weights, args.no_fold, args.roofline_kernel, baseline, log=True)
    result = {
        "metric": "merged vision tokens/sec",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded U(-1,1) pixels, N(0,0.02) weights)",
    }
    for k, v in head.items():
        if k not in result:
            result[k] = v
    # the high-resolution configuration, measured in the same run (default
    # invocation only): its own throughput, roofline and extrapolated baseline
    if args.workload == "qwen2vl_2b_448" and args.weights == "bf16" and args.high_res_steps > 0:
        hr = synth.WORKLOADS[HIGH_RES]
        result["configs"] = {HIGH_RES: measure(hr, args.high_res_steps, 1, "bf16", args.no_fold, None,
                                               None if args.no_cpu_baseline else "extrapolated", log=True)}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
