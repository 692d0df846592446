"""Benchmark of the PaTH attention hot path on one MI355X.

One step = one PaTH forward on the L=4096 workload (B=8, H=16, d=64, bf16,
scale 1/sqrt(d): block prepare + right-to-left scan) followed by one decode
step on the cache-8192 workload (B=64, H=16, d=64, bf16).  Inputs are seeded
synthetic tensors already resident in HBM when timing starts.

Printed: ONE JSON line.  `value` is the forward throughput in TFLOP/s under
the stated FLOP model F = sum_(b,h) (2 d L^2 + d^2 L^2 / 64) (QK^T and PV over
the causal half, plus the Householder block transport); decode bandwidth is
reported in `decode`.  Per-kernel durations come from HIP events recorded on
the stream the kernels run on (torch's current stream).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 matrix peak
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector peak
PEAK_HBM_GBS = 8000.0


def flops_path(B, H, L, d):
    return B * H * (2.0 * d * L * L + d * d * L * L / 64.0)


def decode_bytes(B, H, n, d, esize):
    return B * H * n * d * esize * 3.0  # K read + K write + V read


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--precision", default="auto", choices=["auto", "accurate"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dependent_position_encoding_fwd_amd as pa
    import synthetic

    dev = torch.device("cuda:0")
    cf = synthetic.CONFIGS[2]
    cd = synthetic.CONFIGS[5]
    print(f"[bench] generating inputs: {cf.desc}; {cd.desc}", file=sys.stderr, flush=True)
    xf = {n: (t.to(dev) if t is not None else None) for n, t in synthetic.config_inputs(2).items()}
    xd = {n: t.to(dev) for n, t in synthetic.config_inputs(5).items()}
    fargs = (xf["q"], xf["k"], xf["v"], xf["w"], xf["beta"])
    ws = pa.fwd_workspace(xf["q"], None)
    o = torch.empty_like(xf["q"])
    lse = torch.empty(xf["beta"].shape, dtype=torch.float32, device=dev)
    dws = torch.empty(max(256, pa.decode_workspace_bytes(cd.B, cd.H, cd.d, cd.cache_len)), dtype=torch.uint8,
                      device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pa.path_fwd_stage_prepare(*fargs, None, scale=cf.scale, precision=args.precision, workspace=ws)
        if ev is not None:
            ev[1].record()
        pa.path_fwd_stage_scan(*fargs, ws, None, scale=cf.scale, precision=args.precision, out=(o, lse))
        if ev is not None:
            ev[2].record()
        pa.path_decode_step(xd["q_t"], xd["k_t"], xd["v_t"], xd["w_t"], xd["beta_t"], xd["k_cache"],
                            xd["v_cache"], cd.cache_len, scale=cd.scale, workspace=dws)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    fwd_ms = prep_ms + scan_ms
    F = flops_path(cf.B, cf.H, cf.L, cf.d)
    tflops = F / (fwd_ms * 1e-3) / 1e12
    dbytes = decode_bytes(cd.B, cd.H, cd.cache_len, cd.d, 2)
    dec_gbs = dbytes / (dec_ms * 1e-3) / 1e9

    scan_tflops = F / (scan_ms * 1e-3) / 1e12
    kind = os.environ.get("PATH_BENCH_KIND", "valu_f32")
    peak = PEAK_FP32_VALU_TFLOPS if kind == "valu_f32" else PEAK_BF16_TFLOPS
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "fwd_scan_traffic.json")
    if os.path.exists(tfile):
        try:
            traffic = json.load(open(tfile)).get("bytes_per_launch")
        except Exception:
            traffic = None
    roofline = {"bound": "alu" if kind == "valu_f32" else "mfma", "achieved": round(scan_tflops, 3),
                "peak": peak, "unit": "TFLOP/s", "frac": round(scan_tflops / peak, 4), "traffic": traffic,
                "kernel": "fwd_scan", "flops_per_launch": F}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cf)

    line = {
        "metric": "PaTH fwd TFLOP/s & % bf16 MFMA peak at L=4096; decode-step HBM GB/s",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if kind == "valu_f32" else "bf16", "data": "synthetic",
        "config": {"workload": "PaTH fwd bf16 B=8 H=16 L=4096 d=64 scale=1/8 + decode bf16 B=64 H=16 d=64 "
                               "cache=8192", "global_batch": cf.B, "seq_len": cf.L, "heads": cf.H, "head_dim": cf.d,
                   "precision": args.precision, "parallelism": "single-gpu"},
        "fwd": {"ms": round(fwd_ms, 4), "prepare_ms": round(prep_ms, 4), "scan_ms": round(scan_ms, 4),
                "tflops_model": F, "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                "fa_equiv_tflops": round(cf.B * cf.H * 2.0 * cf.d * cf.L ** 2 / (fwd_ms * 1e-3) / 1e12, 3)},
        "decode": {"ms": round(dec_ms, 4), "GB_per_s": round(dec_gbs, 1), "bytes_model": dbytes,
                   "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(cf, budget_s=10.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    whole heads (all L query rows) in order until `budget_s` of wall time is spent."""
    import oracle
    import synthetic

    heads = [(b, h) for b in range(cf.B) for h in range(cf.H)]
    done = 0
    dt = 0.0
    for (b, h) in heads:
        x = synthetic.fwd_inputs(cf.B, cf.H, cf.L, cf.d, cf.dtype, cf.seed, heads=[(b, h)])
        t0 = time.perf_counter()
        oracle.path_fwd_head(x["q"][0], x["k"][0], x["v"][0], x["w"][0], x["beta"][0], None, cf.scale)
        dt += time.perf_counter() - t0
        done += 1
        if dt >= budget_s:
            break
    F = flops_path(1, done, cf.L, cf.d)
    return {"value": round(F / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads (all {cf.L} query rows each) of the L=4096 workload, "
                      f"{dt:.1f} s of oracle wall time"}


if __name__ == "__main__":
    main()
