"""Benchmark of the PaTH attention hot path on one MI355X.

One step = one PaTH forward on the L=4096 workload (B=8, H=16, d=64, bf16
storage, scale 1/8: block prepare + right-to-left scan) followed by one
decode step on the cache-8192 workload (B=64, H=16, d=64, bf16).  Inputs are
seeded synthetic tensors already resident in HBM when timing starts; there is
no cache flush between steps.  Decode steps keep mutating the same cache
(each one applies a new transition to every cached key), which leaves the
amount of work unchanged.

Printed: ONE JSON line.  `value` is the forward throughput in TFLOP/s under
the FLOP model F = sum over (b,h) of (2 d L^2 + d^2 L^2 / 64): QK^T and PV
over the causal half plus the Householder block transport of the query
state; the prepare stage is timed but earns no FLOPs.  Decode bandwidth is
reported in `decode` on 3 x B H n d x 2 bytes (keys read and written, values
read).  Per-kernel durations come from HIP events recorded on the stream the
kernels are launched on (torch's current stream, which the binding passes to
every launch); the median over the timed steps is reported.

`roofline` describes the dominant kernel, the matrix-core scan: achieved =
F / scan duration against the 2.5 PFLOP/s dense fp16/bf16 matrix peak.  Its
`traffic` (HBM bytes per launch) comes from the rocprofv3 counter summary
profiles/hbm_traffic.json and is reported only while the kernel's source
still hashes to the value recorded there; the decode kernel's traffic is
reported the same way.  After the timed steps the gated decode step
(forget-gate prefix cache beside the key cache) runs on the same cache for
the same numbers of warm-up and timed launches and is reported in
`decode_fox` on the decode bytes plus 4 bytes per cached key.

Order: one forward call, then the secondary legs (paged decode, backward,
projection, and the forward on configurations 4 and 3, each with warm-up
launches of its own), then the W warm-up steps and the K timed steps, then
the gated decode step and the CPU baseline.  The secondary legs come first so
that the headline steps start on a GPU whose clocks have settled even when W
is small: from a cold start the forward's per-step time falls by about a
quarter over its first hundred steps.  The forward legs of configurations 3
and 4 are reported in `fwd_config3` and `fwd_config4`.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--copy-ref]
                    [--no-bwd] [--no-config-legs] [--fwd-config {2,3,4}] [--fwd-only]

`--fwd-only` times the forward steps alone and prints a forward-only line (for
counter runs under rocprofv3 --pmc).

`--fwd-config` swaps the forward workload for another of the synthetic
configurations (3: B=1 H=16 L=16384 d=64; 4: B=4 H=16 L=8192 d=128 with forget
gates); the default, 2, is the headline workload above.  The roofline then
describes that configuration's scan kernel, and its traffic is reported only
for the default workload, whose counters are recorded.

Last, the backward pass (`path_attn_bwd`: gradients of q, k, v, w, beta and,
with gates, the log forget gates) runs on the forward workload with a seeded
incoming gradient dO, 2 untimed and 5 timed launches, reported in `bwd` in
TFLOP/s under F_bwd = sum over (b,h) of (5 d L^2 + 3 d^2 L^2 / 64): five
L x L x d products over the causal half (logits recomputed, dV, dO V^T, dK,
the adjoint of the queries) and three block transports (queries again, their
adjoint, the transitions' gradient).  The in-block chains earn no FLOPs.  With
bf16 storage the cross-block products run on the 16-bit matrix cores
with every fp32 operand split into bf16 hi + lo (two or three products each,
fp32 accumulation), the block prepare the same way, and the in-block part on
the fp32 matrix cores; with fp32 storage it computes in fp32 throughout.  `frac_fp32_peak` relates the rate to MI355X's
fp32 157.3 TFLOP/s.  `--no-bwd` skips it.

The paged decode step (`path_decode_step_paged`) runs on the same caches
scattered into 256-slot pages in a seeded random page order, every sequence at
length 8192, and is reported in `decode_paged` on the decode's bytes (the page
table adds 132 bytes per head), median of 50 launches after 20.  The gated
paged step (`path_decode_step_paged_fox`, the forget-gate prefix cache in the
same pages) follows in `decode_paged_fox`, on those bytes plus 4 per cached key.

The projection prologue (`path_project`: w and beta of every head from the
tokens, model width Dm = H d) runs on the forward workload's tokens and is
reported in `project`: TFLOP/s on 2 T Dm (H d + H) FLOP (T = B L tokens)
against the 2.5 PFLOP/s bf16 matrix peak, median of 50 launches after 20.

`--copy-ref` first runs a plain 1 GiB device copy, whose FETCH_SIZE and
WRITE_SIZE counters calibrate those of the other kernels in a rocprofv3
--pmc run of this script.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from dependent_position_encoding_fwd_amd.profsum import source_hash  # noqa: E402

PEAK_MFMA_F16_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
PEAK_HBM_GBS = 8000.0
PEAK_F32_TFLOPS = 157.3  # MI355X fp32, matrix and vector alike
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
COPY_REF_BYTES = 1 << 30


def flops_path(B, H, L, d):
    return B * H * (2.0 * d * L * L + d * d * L * L / 64.0)


def flops_path_bwd(B, H, L, d):
    return B * H * (5.0 * d * L * L + 3.0 * d * d * L * L / 64.0)


def decode_bytes(B, H, n, d, esize):
    return B * H * n * d * esize * 3.0  # K read + K write + V read


def load_traffic(kind: str):
    """HBM bytes per launch of one kernel ("scan" or "decode") from the
    committed counter summary, or None when there is none or the kernel's
    source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(kind, {})
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_hash(kind):
        return None
    return t.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 0.15 s of warm-up: the clocks take tens of milliseconds of load to settle
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--precision", default="auto", choices=["auto", "accurate"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-ref", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    # leave out the forward legs of configurations 3 and 4 (profiling runs, whose
    # per-kernel averages must hold the headline workload's launches only)
    ap.add_argument("--no-config-legs", action="store_true")
    # counter runs: only the forward (prepare + scan) steps; prints a forward-only line
    ap.add_argument("--fwd-only", action="store_true")
    ap.add_argument("--fwd-config", type=int, default=2, choices=[2, 3, 4])
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path (got --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import dependent_position_encoding_fwd_amd as pa
    import synthetic

    dev = torch.device("cuda:0")
    cid = args.fwd_config
    cf = synthetic.CONFIGS[cid]
    cd = synthetic.CONFIGS[5]
    print(f"[bench] generating inputs: {cf.desc}; {cd.desc}", file=sys.stderr, flush=True)
    xf = {n: (t.to(dev) if t is not None else None) for n, t in synthetic.config_inputs(cid).items()}
    gates = xf.get("log_forget")
    xd = {n: t.to(dev) for n, t in synthetic.config_inputs(5).items()}
    gd = synthetic.decode_gate_inputs(cd.B, cd.H, cd.cache_len, cd.capacity, cd.seed)
    log_f_t = gd["log_f_t"].to(dev)
    cum_cache = torch.cumsum(gd["log_f_cache"].double(), dim=-1).float().to(dev)
    fargs = (xf["q"], xf["k"], xf["v"], xf["w"], xf["beta"])
    ws = pa.fwd_workspace(xf["q"], gates)
    o = torch.empty_like(xf["q"])
    lse = torch.empty(xf["beta"].shape, dtype=torch.float32, device=dev)
    dws = torch.empty(max(256, pa.decode_workspace_bytes(cd.B, cd.H, cd.d, cd.cache_len)), dtype=torch.uint8,
                      device=dev)

    if args.copy_ref:
        src = torch.ones(COPY_REF_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy reference: {COPY_REF_BYTES} bytes read, {COPY_REF_BYTES} bytes written",
              file=sys.stderr, flush=True)
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pa.path_fwd_stage_prepare(*fargs, gates, scale=cf.scale, precision=args.precision, workspace=ws)
        if ev is not None:
            ev[1].record()
        pa.path_fwd_stage_scan(*fargs, ws, gates, scale=cf.scale, precision=args.precision, out=(o, lse))
        if ev is not None:
            ev[2].record()
        if not args.fwd_only:
            pa.path_decode_step(xd["q_t"], xd["k_t"], xd["v_t"], xd["w_t"], xd["beta_t"], xd["k_cache"],
                                xd["v_cache"], cd.cache_len, scale=cd.scale, workspace=dws)
        if ev is not None:
            ev[3].record()

    # The secondary legs (paged decode, backward, projection) run first, so the
    # headline steps below start on a GPU whose clocks have settled: with only a
    # few warm-up steps they would otherwise still be rising during the timed
    # steps.  The backward needs the forward's o and lse: one forward call first.
    # The forward legs of the other two forward configurations come last among
    # them: from a cold start the forward's per-step time falls by about a
    # quarter over its first hundred or so steps (0.1 s) while the chip's clocks
    # settle, and these legs are that much forward work.
    paged = paged_fox = bwd = proj = None
    other_fwd = {}
    if not args.fwd_only:
        pa.path_fwd_stage_prepare(*fargs, gates, scale=cf.scale, precision=args.precision, workspace=ws)
        pa.path_fwd_stage_scan(*fargs, ws, gates, scale=cf.scale, precision=args.precision, out=(o, lse))
        dbytes = decode_bytes(cd.B, cd.H, cd.cache_len, cd.d, 2)
        paged, paged_fox = paged_leg(pa, xd, gd, cd, dbytes)
        bwd = None if args.no_bwd else bwd_leg(pa, fargs, gates, cf, o, lse)
        proj = project_leg(pa, cf)
        if cid == 2 and not args.no_config_legs:
            for c in (4, 3):
                other_fwd[f"fwd_config{c}"] = fwd_leg(pa, c, args.precision)

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] {args.steps} timed steps done in {wall:.3f} s", file=sys.stderr, flush=True)
    if args.fwd_only:
        fwd_only_line(args, cf, evs, wall)
        return
    # The gated (forget-gate) decode step on the same cache, timed on its own
    # after the steps above: the same number of launches, each bracketed by events.
    fox_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.warmup + args.steps):
        if k >= args.warmup:
            fox_evs[k - args.warmup][0].record()
        pa.path_decode_step_fox(xd["q_t"], xd["k_t"], xd["v_t"], xd["w_t"], xd["beta_t"], log_f_t, xd["k_cache"],
                                xd["v_cache"], cum_cache, cd.cache_len, scale=cd.scale, workspace=dws)
        if k >= args.warmup:
            fox_evs[k - args.warmup][1].record()
    torch.cuda.synchronize()
    fox_ms = statistics.median(e[0].elapsed_time(e[1]) for e in fox_evs)
    prep_ms = statistics.median(e[0].elapsed_time(e[1]) for e in evs)
    scan_ms = statistics.median(e[1].elapsed_time(e[2]) for e in evs)
    dec_ms = statistics.median(e[2].elapsed_time(e[3]) for e in evs)
    fwd_ms = prep_ms + scan_ms
    F = flops_path(cf.B, cf.H, cf.L, cf.d)
    tflops = F / (fwd_ms * 1e-3) / 1e12
    dbytes = decode_bytes(cd.B, cd.H, cd.cache_len, cd.d, 2)
    dec_gbs = dbytes / (dec_ms * 1e-3) / 1e9
    fbytes = dbytes + 4 * cd.B * cd.H * cd.cache_len  # plus one fp32 gate prefix per cached key
    fox_gbs = fbytes / (fox_ms * 1e-3) / 1e9

    scan_tflops = F / (scan_ms * 1e-3) / 1e12
    traffic = load_traffic("scan") if cid == 2 else None
    roofline = {"bound": "mfma", "achieved": round(scan_tflops, 3), "peak": PEAK_MFMA_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(scan_tflops / PEAK_MFMA_F16_TFLOPS, 4), "traffic": traffic,
                "kernel": f"scan{cf.d}_kernel (right-to-left scan, d={cf.d})", "flops_per_launch": F,
                "launch_ms": round(scan_ms, 4), "source_sha256": source_hash("scan")}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cf)

    line = {
        "metric": "PaTH fwd TFLOP/s & % bf16 MFMA peak at L=4096; decode-step HBM GB/s",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"PaTH fwd B={cf.B} H={cf.H} L={cf.L} d={cf.d} scale={cf.scale:g}"
                               f"{' forget gates' if cf.fox else ''} (bf16 in/out) + decode B=64 H=16 d=64 "
                               "cache=8192 (bf16)", "storage": "bf16", "arith": "fp16 MFMA, fp32 accumulate",
                   "global_batch": cf.B, "seq_len": cf.L, "heads": cf.H, "head_dim": cf.d,
                   "precision": args.precision, "parallelism": "single-gpu"},
        "fwd": {"ms": round(fwd_ms, 4), "prepare_ms": round(prep_ms, 4), "scan_ms": round(scan_ms, 4),
                "flops_model": F, "frac_bf16_peak": round(tflops / PEAK_MFMA_F16_TFLOPS, 4),
                "fa_equiv_tflops": round(cf.B * cf.H * 2.0 * cf.d * cf.L ** 2 / (fwd_ms * 1e-3) / 1e12, 3)},
        "decode": {"ms": round(dec_ms, 4), "GB_per_s": round(dec_gbs, 1), "bytes_model": dbytes,
                   "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4), "traffic": load_traffic("decode"),
                   "source_sha256": source_hash("decode")},
        "decode_fox": {"ms": round(fox_ms, 4), "GB_per_s": round(fox_gbs, 1), "bytes_model": fbytes,
                       "frac_hbm_peak": round(fox_gbs / PEAK_HBM_GBS, 4),
                       "what": "gated decode step, same cache, forget-gate prefix cache (fp32)"},
        **other_fwd,
        "decode_paged": paged,
        "decode_paged_fox": paged_fox,
        "bwd": bwd,
        "project": proj,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def fwd_only_line(args, cf, evs, wall):
    """The forward's figures alone (a --fwd-only run, as used under rocprofv3 --pmc)."""
    prep_ms = statistics.median(e[0].elapsed_time(e[1]) for e in evs)
    scan_ms = statistics.median(e[1].elapsed_time(e[2]) for e in evs)
    F = flops_path(cf.B, cf.H, cf.L, cf.d)
    fwd_ms = prep_ms + scan_ms
    print(json.dumps({
        "metric": "PaTH fwd TFLOP/s (forward-only run)", "value": round(F / (fwd_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "dtype": "f16",
        "config": {"workload": f"PaTH fwd B={cf.B} H={cf.H} L={cf.L} d={cf.d} scale={cf.scale:g}"
                               f"{' forget gates' if cf.fox else ''} (bf16 in/out)", "global_batch": cf.B,
                   "seq_len": cf.L, "heads": cf.H, "head_dim": cf.d, "precision": args.precision},
        "fwd": {"ms": round(fwd_ms, 4), "prepare_ms": round(prep_ms, 4), "scan_ms": round(scan_ms, 4),
                "flops_model": F}}), flush=True)


def bwd_leg(pa, fargs, gates, cf, o, lse, warmup=2, steps=5):
    """Times path_attn_bwd on the forward workload: median of `steps` launches,
    each bracketed by HIP events on the launch stream."""
    import torch

    q = fargs[0]
    gen = torch.Generator().manual_seed(cf.seed + 4242)
    do = torch.randn(tuple(q.shape), generator=gen).to(q.dtype).to(q.device)
    nbytes = pa.bwd_workspace_bytes(cf.B, cf.H, cf.L, cf.d, pa.PATH_BF16 if q.dtype == torch.bfloat16 else pa.PATH_F32,
                                    gates is not None)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for k in range(warmup + steps):
        if k >= warmup:
            evs[k - warmup][0].record()
        pa.path_attn_bwd(*fargs, o, lse, do, gates, scale=cf.scale, workspace=ws)
        if k >= warmup:
            evs[k - warmup][1].record()
    torch.cuda.synchronize()
    ms = statistics.median(e[0].elapsed_time(e[1]) for e in evs)
    F = flops_path_bwd(cf.B, cf.H, cf.L, cf.d)
    tf = F / (ms * 1e-3) / 1e12
    print(f"[bench] backward: {ms:.3f} ms", file=sys.stderr, flush=True)
    split16 = q.dtype == torch.bfloat16
    return {"ms": round(ms, 3), "TFLOP_per_s": round(tf, 3), "flops_model": F,
            "arith": ("block prepare and cross-block products as split-bf16 MFMA (computed operands as bf16 hi + lo, "
                      "fp32 accumulate); in-block part on fp32 MFMA") if split16 else "fp32 MFMA and vector ALU",
            "frac_fp32_peak": round(tf / PEAK_F32_TFLOPS, 4),
            "what": "path_attn_bwd on the forward workload (gradients of q, k, v, w, beta"
                    f"{', log forget gates' if gates is not None else ''}), seeded dO, median of {steps}"}


def paged_leg(pa, xd, gd, cd, dbytes, page=256, warmup=20, steps=50):
    """Times path_decode_step_paged and path_decode_step_paged_fox on the decode
    workload's caches, scattered into `page`-slot pages in a seeded random order
    (lengths all cache_len); the gated step reads the prefix cache from the same
    pages.  Returns the two result records."""
    import torch

    B, H, n, d = cd.B, cd.H, cd.cache_len, cd.d
    mp = (n + 1 + page - 1) // page
    npg = B * mp
    perm = torch.randperm(npg, generator=torch.Generator().manual_seed(cd.seed)).to("cuda:0")
    table = perm.view(B, mp).to(torch.int32)

    def scatter(c):
        e = c.shape[3]
        padded = torch.zeros(B, H, mp * page, e, dtype=c.dtype, device=c.device)
        padded[:, :, : c.shape[2]] = c
        logical = padded.view(B, H, mp, page, e).permute(0, 2, 1, 3, 4).reshape(npg, H, page, e)
        pages = torch.empty_like(logical)
        pages[perm] = logical
        return pages

    kp, vp = scatter(xd["k_cache"]), scatter(xd["v_cache"])
    lens = torch.full((B,), n, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(max(256, pa.decode_workspace_bytes(B, H, d, n)), dtype=torch.uint8, device="cuda:0")
    # gated: the prefix cache in the same pages (one fp32 per key slot)
    cum = torch.cumsum(gd["log_f_cache"].double(), dim=-1).float().to("cuda:0")
    cp = scatter(cum.unsqueeze(-1)).squeeze(-1).contiguous()
    log_f_t = gd["log_f_t"].to("cuda:0")

    def timed(step):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for k in range(warmup + steps):
            if k >= warmup:
                evs[k - warmup][0].record()
            step()
            if k >= warmup:
                evs[k - warmup][1].record()
        torch.cuda.synchronize()
        return statistics.median(e[0].elapsed_time(e[1]) for e in evs)

    ms = timed(lambda: pa.path_decode_step_paged(xd["q_t"], xd["k_t"], xd["v_t"], xd["w_t"], xd["beta_t"], kp, vp,
                                                 table, lens, n, scale=cd.scale, workspace=ws))
    fms = timed(lambda: pa.path_decode_step_paged_fox(xd["q_t"], xd["k_t"], xd["v_t"], xd["w_t"], xd["beta_t"],
                                                      log_f_t, kp, vp, cp, table, lens, n, scale=cd.scale,
                                                      workspace=ws))
    gbs = dbytes / (ms * 1e-3) / 1e9
    fbytes = dbytes + 4 * B * H * n
    fgbs = fbytes / (fms * 1e-3) / 1e9
    del kp, vp, cp
    return ({"ms": round(ms, 4), "GB_per_s": round(gbs, 1), "bytes_model": dbytes,
             "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
             "what": f"paged decode step, same caches in {page}-slot pages (random page order), length {n} each"},
            {"ms": round(fms, 4), "GB_per_s": round(fgbs, 1), "bytes_model": fbytes,
             "frac_hbm_peak": round(fgbs / PEAK_HBM_GBS, 4),
             "what": f"gated paged decode step, same pages plus the forget-gate prefix cache in the same "
                     f"{page}-slot pages"})


def fwd_leg(pa, cid, precision, warmup=20, steps=20):
    """Times the forward (prepare + scan) on another synthetic configuration:
    medians of `steps` launches of each stage, bracketed by HIP events on the
    launch stream."""
    import torch

    import synthetic

    c = synthetic.CONFIGS[cid]
    print(f"[bench] forward leg: {c.desc}", file=sys.stderr, flush=True)
    x = {n: (t.to("cuda:0") if t is not None else None) for n, t in synthetic.config_inputs(cid).items()}
    g = x.get("log_forget")
    args = (x["q"], x["k"], x["v"], x["w"], x["beta"])
    ws = pa.fwd_workspace(x["q"], g)
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["beta"].shape, dtype=torch.float32, device="cuda:0")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(warmup + steps):
        if k >= warmup:
            evs[k - warmup][0].record()
        pa.path_fwd_stage_prepare(*args, g, scale=c.scale, precision=precision, workspace=ws)
        if k >= warmup:
            evs[k - warmup][1].record()
        pa.path_fwd_stage_scan(*args, ws, g, scale=c.scale, precision=precision, out=(o, lse))
        if k >= warmup:
            evs[k - warmup][2].record()
    torch.cuda.synchronize()
    prep = statistics.median(e[0].elapsed_time(e[1]) for e in evs)
    scan = statistics.median(e[1].elapsed_time(e[2]) for e in evs)
    F = flops_path(c.B, c.H, c.L, c.d)
    tf = F / ((prep + scan) * 1e-3) / 1e12
    del x, ws, o, lse
    return {"ms": round(prep + scan, 4), "prepare_ms": round(prep, 4), "scan_ms": round(scan, 4),
            "flops_model": F, "TFLOP_per_s": round(tf, 3), "frac_bf16_peak": round(tf / PEAK_MFMA_F16_TFLOPS, 4),
            "scan_frac_bf16_peak": round(F / (scan * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
            "what": f"{c.desc}, precision {precision}, median of {steps} after {warmup} warm-up launches"}


def project_leg(pa, cf, warmup=20, steps=50):
    """Times path_project on the forward workload's tokens (Dm = H d)."""
    import torch

    import synthetic

    Dm = cf.H * cf.d
    x = {n: t.to("cuda:0") for n, t in synthetic.project_inputs(cf.B, cf.L, Dm, cf.H, cf.d, cf.seed).items()}
    out = (torch.empty((cf.B, cf.H, cf.L, cf.d), dtype=torch.bfloat16, device="cuda:0"),
           torch.empty((cf.B, cf.H, cf.L), dtype=torch.float32, device="cuda:0"))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for k in range(warmup + steps):
        if k >= warmup:
            evs[k - warmup][0].record()
        pa.path_project(x["x"], x["Ww"], x["u"], x["b"], out=out)
        if k >= warmup:
            evs[k - warmup][1].record()
    torch.cuda.synchronize()
    ms = statistics.median(e[0].elapsed_time(e[1]) for e in evs)
    T = cf.B * cf.L
    F = 2.0 * T * Dm * (cf.H * cf.d + cf.H)
    tf = F / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOP_per_s": round(tf, 3), "flops_model": F, "bound": "mfma",
            "peak": PEAK_MFMA_F16_TFLOPS, "frac_bf16_peak": round(tf / PEAK_MFMA_F16_TFLOPS, 4),
            "what": f"path_project, T={T} tokens, Dm={Dm}, H={cf.H}, d={cf.d} (bf16 in, w bf16 + beta fp32 out)"}


def cpu_model():
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cf, budget_s=10.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    whole heads (all L query rows) in order until `budget_s` of wall time is spent."""
    import oracle
    import synthetic

    heads = [(b, h) for b in range(cf.B) for h in range(cf.H)]
    done = 0
    dt = 0.0
    for (b, h) in heads:
        x = synthetic.fwd_inputs(cf.B, cf.H, cf.L, cf.d, cf.dtype, cf.seed, cf.near2_frac, cf.fox, heads=[(b, h)])
        gate = x["log_forget"][0] if cf.fox else None
        t0 = time.perf_counter()
        oracle.path_fwd_head(x["q"][0], x["k"][0], x["v"][0], x["w"][0], x["beta"][0], gate, cf.scale)
        dt += time.perf_counter() - t0
        done += 1
        print(f"[bench] oracle head {done}: {dt:.1f} s", file=sys.stderr, flush=True)
        if dt >= budget_s:
            break
    F = flops_path(1, done, cf.L, cf.d)
    return {"value": round(F / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} of {len(heads)} heads (all {cf.L} query rows each) of the L={cf.L} workload, "
                      f"{dt:.1f} s of oracle wall time"}


if __name__ == "__main__":
    main()
