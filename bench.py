#!/usr/bin/env python3
"""Benchmark: pair-biased triangle attention on one MI355X.

One step = one call of the whole forward (tri_attn_fwd) on the single-GPU ceiling
workload: B=1, N=2,700 tokens, H=4, D=32, bf16 inputs, last 60 keys masked, 8 ring-step
key tiles (the 1x1 row of the Fold-CP page's Table 2 gives 2,700 tokens as one H100's
maximum).  Inputs are synthetic and seeded (workloads/), resident in HBM before timing.

Prints one JSON line.  `value` is TFLOP/s at the nominal 4*B*H*N^3*D FLOPs; `roofline`
relates the kernel's live-measured average launch time to the bf16 dense MFMA peak;
`cpu_baseline` times the fp64 oracle on a bounded sample of the same workload's rows.

`--pass` measures the other entry points on the same workload, one JSON line each:
  bwd        tri_attn_bwd (dq, dk, dv, row-summed dbias) from the forward's out and lse;
             algorithmic FLOPs 10*B*H*I*N^2*D (the S recompute, dP, dQ, dK, dV products);
             bf16 with D = 32 runs on matrix cores (bf16 MFMA peak), other cases in fp32
             vector arithmetic (fp32 vector peak)
  ending     tri_attn_fwd_ending (same FLOPs as the forward, bf16 MFMA peak)
  pair_bias  pair_bias_attn_fwd on the workload's first row (I = 1): bound by reading
             the bias -> roofline in GB/s against HBM
  ring       tri_attn_tile_state on the first key tile, tri_attn_tile_state_update on each
             middle one (the step folded into the running state), tri_attn_tile_state_final
             on the last (folded and written out): the split-tile path, against the bf16
             MFMA peak

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--no-cpu]
                    [--pass fwd|bwd|ending|pair_bias|ring]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "triangle-attention TFLOP/s (4·B·H·N³·D) and % bf16 MFMA peak, 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak (AMD published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (AMD published)
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector (AMD published)
DEFAULT_WORKLOAD = "single_gpu_n2700"
KERNEL_NAME = "bf16_mfma_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


KERNEL_SOURCES = ("kernel_bf16_mfma.hip", "launch.h")   # what the forward's kernels are built from


def kernel_source_digest() -> str:
    """SHA-256 over the sources of the forward's kernels: stored traffic counters are only
    reported while the kernels they were taken on are unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "pair_biased_triangle_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_counters(workload: str):
    """The committed rocprofv3 --pmc summary of the forward's dominant kernel on this
    workload (HBM bytes per launch, clock, MFMA busy), or None when the kernel sources
    changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return entry


def to_dev(torch, a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def cpu_baseline(w, out_gpu, torch, target_s: float):
    """Time the fp64 oracle on a bounded, deterministic sample of query rows of the same
    workload; scale to TFLOP/s with the same nominal FLOPs per row.  Also reports the
    largest |gpu - oracle| over the sample (parity spot check of the timed launch)."""
    import oracle
    cfg = w.cfg
    rng = np.random.default_rng(1234)
    total_rows = cfg.B * cfg.I * cfg.N
    flops_per_row = 4.0 * cfg.H * cfg.N * cfg.D
    probe = np.sort(rng.choice(total_rows, size=min(total_rows, 256), replace=False))
    t0 = time.perf_counter()
    oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=cfg.n_key_tiles, rows=probe)
    t_probe = time.perf_counter() - t0
    n = int(min(total_rows, max(256, len(probe) * target_s / max(t_probe, 1e-6))))
    rows = np.sort(rng.choice(total_rows, size=n, replace=False))
    t0 = time.perf_counter()
    ref, _ = oracle.tri_attn(w.q, w.k, w.v, w.bias, w.mask, n_key_tiles=cfg.n_key_tiles, rows=rows)
    secs = time.perf_counter() - t0
    got = out_gpu.view(-1, cfg.H, cfg.D)[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(got - ref)))
    return {
        "value": round(n * flops_per_row / secs / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{n} of {total_rows} query rows (b,i,j), all {cfg.H} heads and {cfg.N} keys each, "
                  f"{secs:.1f} s wall, fp64",
    }, err, n


def timed(torch, step, steps, warmup):
    """HIP events on the launch stream around `steps` calls after `warmup` untimed ones;
    returns (ms per step, wall seconds of the timed region)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0


def other_pass(args, torch, P, W, cfg) -> dict:
    """The entry points beyond the forward, timed on the same workload's inputs."""
    w = W.make_inputs(cfg)
    q, k, v, bias, mask = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    B, I, N, H, D, T = cfg.B, cfg.I, cfg.N, cfg.H, cfg.D, cfg.n_key_tiles
    fwd_flops = cfg.flops
    extra = {}
    if args.which == "bwd":
        out, lse = P.tri_attn_fwd_lse(q, k, v, bias, mask, n_key_tiles=T)
        dout = torch.randn(q.shape, dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(1))
        step = lambda: P.tri_attn_bwd(q, k, v, bias, mask, out, lse, dout)
        metric = "triangle-attention backward TFLOP/s (10·B·H·I·N²·D: S recompute, dP, dQ, dK, dV)"
        if cfg.dtype == "bf16" and D == 32:     # the matrix-core backward
            work, unit, peak, bound = 2.5 * fwd_flops, "TFLOP/s", PEAK_BF16_TFLOPS, "mfma"
            kernels = "bwd_prep_kernel + bwd_dq_lds + bwd_dkdv_lds + bwd_dbias_lds (bf16 MFMA, fp32 accumulate)"
            dtype = "bf16"
        else:
            work, unit, peak, bound = 2.5 * fwd_flops, "TFLOP/s", PEAK_FP32_TFLOPS, "alu"
            kernels = "bwd_dq_kernel + bwd_dkdv_kernel + bwd_dbias_kernel (fp32 vector)"
            dtype = "f32"
    elif args.which == "ending":
        if I != N:
            raise SystemExit("the ending orientation needs a workload with I == N")
        step = lambda: P.tri_attn_fwd_ending(q, k, v, bias, mask, n_key_tiles=T)
        work, unit, peak, bound = fwd_flops, "TFLOP/s", PEAK_BF16_TFLOPS, "mfma"
        metric = "ending-node triangle-attention TFLOP/s (4·B·H·N³·D)"
        kernels = "bias_ref_kernel + bias_image16_kernel (transposed bias) + bf16_mfma_kernel"
        dtype = cfg.dtype
    elif args.which == "pair_bias":
        shp = (B, N, H, D)
        q1, k1, v1 = (x[:, 0].contiguous().view(shp) for x in (q, k, v))
        step = lambda: P.pair_bias_attn_fwd(q1, k1, v1, bias, mask, n_key_tiles=T)
        s_in = cfg.in_bytes
        work = 3 * B * N * H * D * s_in + B * H * N * N * s_in + (4 * B * N if mask is not None else 0) + 4 * B * N * H * D
        unit, peak, bound = "GB/s", PEAK_HBM_GBS, "hbm"
        metric = "attention with pair bias GB/s (q, k, v, bias read once, out written once)"
        kernels = "pair_bias_direct_kernel (one pass over the raw bias, split keys) + state_combine_kernel"
        extra["flops_per_call"] = 4.0 * B * H * N * N * D
        dtype = cfg.dtype
    else:   # ring
        bounds = [t * (N // T) + min(t, N % T) for t in range(T + 1)]   # the forward's tiles
        acc = torch.empty((B, I, N, H, D), dtype=torch.float32, device="cuda")
        m = torch.empty((B, I, N, H), dtype=torch.float32, device="cuda")
        l = torch.empty_like(m)
        out = torch.empty_like(acc)

        def step():
            # one ring: the first step's state, every later step folded into it in place
            P.tri_attn_tile_state(q, k, v, bias, mask, key_begin=bounds[0], key_end=bounds[1], acc=acc, m=m, l=l)
            for t in range(1, T - 1):
                P.tri_attn_tile_state_update(q, k, v, bias, mask, key_begin=bounds[t], key_end=bounds[t + 1],
                                             acc=acc, m=m, l=l)
            if T > 1:
                P.tri_attn_tile_state_final(q, k, v, bias, mask, key_begin=bounds[T - 1], key_end=bounds[T],
                                            acc=acc, m=m, l=l, out=out)
            else:
                P.tri_attn_state_finalize(acc, m, l, out=out)
        work, unit, peak, bound = fwd_flops, "TFLOP/s", PEAK_BF16_TFLOPS, "mfma"
        metric = f"split-tile ring TFLOP/s ({T} ring steps folded into one state, the last one finalised, 4·B·H·I·N²·D)"
        kernels = ("per step: bias_ref_kernel + bias_image16_kernel + bf16_mfma_kernel (state mode; the middle steps "
                   "merge into the running state, the last one writes out)")
        dtype = cfg.dtype
    ms, wall = timed(torch, step, args.steps, args.warmup)
    rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
    res = {
        "metric": metric, "value": round(rate, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded counter-based normal inputs, workloads/)",
        "config": {"workload": cfg.name, "pass": args.which, "B": B, "I": I if args.which != "pair_bias" else 1,
                   "N": N, "H": H, "D": D, "n_key_tiles": T, "masked_keys": cfg.mask_last, "input_dtype": cfg.dtype},
        "wall_s_timed_region": round(wall, 4),
        "roofline": {"bound": bound, "achieved": round(rate, 3), "peak": peak, "unit": unit,
                     "frac": round(rate / peak, 4), "traffic": None, "kernels": kernels,
                     "avg_pass_ms": round(ms, 4)},
        "cpu_baseline": None,
    }
    res.update(extra)
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target wall time of the CPU baseline")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd", "ending", "pair_bias", "ring"])
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 3 plain device copies of 1 GiB (reference dispatches for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU (asked for --gpus {args.gpus}); "
              "sharding across GPUs is not implemented.", file=sys.stderr)
        return 2

    import torch

    import pair_biased_triangle_amd as P
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "dispatches": 3}))
        return 0
    P.load_library()
    cfg = W.CONFIGS[args.workload]
    if args.which != "fwd":
        print(json.dumps(other_pass(args, torch, P, W, cfg)), flush=True)
        return 0
    w = W.make_inputs(cfg)
    q, k, v, bias, mask = (to_dev(torch, x) for x in (w.q, w.k, w.v, w.bias, w.mask))
    out = torch.empty((cfg.B, cfg.I, cfg.N, cfg.H, cfg.D), dtype=torch.float32, device="cuda")
    fn = P.tri_attn_fwd if cfg.I == cfg.N else P.tri_attn_fwd_rows
    step = lambda: fn(q, k, v, bias, mask, n_key_tiles=cfg.n_key_tiles, out=out)

    stream = torch.cuda.current_stream()          # the stream the kernel is launched on
    cold_ms = None
    for u in range(args.warmup):
        if u == 0:                                 # the first call, caches not yet warm: timed on its own
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            cold_ms = c0.elapsed_time(c1)
        else:
            step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # after the timed region: the same number of calls, each between its own pair of events
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in pairs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in pairs)
    per_call = {"calls": len(per), "median_ms": round(per[len(per) // 2], 4), "min_ms": round(per[0], 4),
                "max_ms": round(per[-1], 4), "cold_first_call_ms": None if cold_ms is None else round(cold_ms, 4)}

    flops = cfg.flops
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    ctr = measured_counters(args.workload) if cfg.dtype == "bf16" else None
    traffic = int(ctr["hbm_bytes_per_launch"]) if ctr else None
    roofline = {
        "bound": "mfma",
        "achieved": round(tflops, 3),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "kernel": KERNEL_NAME if (cfg.dtype == "bf16" and cfg.D == 32) else "general_kernel",
        "avg_launch_ms": round(ms_per_step, 4),
        "algorithmic_flops_per_launch": flops,
        "algorithmic_bytes_per_launch": cfg.algorithmic_bytes,
        "hbm_gbs_algorithmic": round(cfg.algorithmic_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        # from the committed counters of the same kernel source (None once it changed): the
        # average clock under this load and the matrix-core busy share of SIMD cycles
        "clock_ghz": ctr.get("clock_ghz") if ctr else None,
        "mfma_busy_pct": ctr.get("mfma_busy_pct") if ctr else None,
        "counters_source": ctr.get("source") if ctr else None,
    }
    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded counter-based normal inputs, workloads/)",
        "config": {"workload": cfg.name, "B": cfg.B, "I": cfg.I, "N": cfg.N, "H": cfg.H, "D": cfg.D,
                   "n_key_tiles": cfg.n_key_tiles, "masked_keys": cfg.mask_last, "input_dtype": cfg.dtype,
                   "out_dtype": "fp32"},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "wall_s_timed_region": round(wall_s, 4),
        "roofline": roofline,
        "cpu_baseline": None,
        "per_call": per_call,
    }
    if not args.no_cpu:
        base, err, n = cpu_baseline(w, out, torch, args.cpu_seconds)
        result["cpu_baseline"] = base
        result["parity_sample"] = {"rows": n, "max_abs_err_vs_oracle": err, "bar": 1e-2 if cfg.dtype == "bf16" else 1e-5}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
