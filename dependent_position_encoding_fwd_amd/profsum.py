"""Summarise rocprofv3 runs of bench.py into short text files.

Three runs of `bench.py` feed it (CSV output, `-o run --output-format csv`):

* a `--kernel-trace --stats` run (kernel durations);
* a `--pmc FETCH_SIZE` run and a `--pmc WRITE_SIZE` run, both with
  `bench.py --copy-ref`, which first copies 1 GiB on the device.

FETCH_SIZE and WRITE_SIZE are in KiB per dispatch.  Each is scaled by the
factor that makes the copy kernel read and write exactly 2^30 bytes, so the
reported bytes are HBM bytes on the copy's calibration.  The copy kernel is
the last device-copy dispatch before the first forward-prepare dispatch.

    python -m dependent_position_encoding_fwd_amd.profsum \
        --stats DIR --fetch DIR --write DIR --md OUT.md --json OUT.json \
        --cmd-stats "..." --cmd-fetch "..." --cmd-write "..."

With only --stats, --md and --cmd-stats it summarises the kernel trace alone
(for example a run of `bench.py --fwd-config 4`).

With --sq DIR... (several `--pmc` runs of `bench.py --fwd-only`, each with its
own counter set) it writes the shader-counter table of the forward kernels:
clock, matrix-pipe busy share, VALU instructions per MFMA, wait shares, LDS
bank conflicts and the L1 -> L2 read latency (see sq_table for the formulas).

Each DIR holds the run's CSV files and `bench.json`, the JSON line bench.py
printed in that run.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
from collections import defaultdict

COPY_REF_BYTES = 1 << 30
_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# Sources whose text determines each measured kernel; a traffic figure is
# reported only while their hash matches the one recorded with it.
KERNEL_SOURCES = {
    "scan": ("fwd_scan64.hip", "mfma_util.h", "common.h"),
    "decode": ("decode.hip", "common.h"),
}


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()

# kernel classes, by a substring of the (mangled or demangled) name
CLASSES = (
    ("scan", "scan64_kernel"),
    ("prepare", "prepare_mfma_kernel"),
    ("cum_padded", "cum_padded_kernel"),
    ("decode_chunk", "decode_chunk_kernel"),
    ("decode_merge", "decode_merge_kernel"),
    ("copy", "copyBuffer"),
)


# the gated decode kernels (template flag true) form classes of their own
GATED = (("decode_chunk_fox", "decode_chunk_kernel"), ("decode_merge_fox", "decode_merge_kernel"))
BWD = ("bwd_pair_kernel", "bwd_transport16_kernel", "bwd_pair16_kernel", "bwd_key16_kernel", "bwd_block_kernel", "bwd_block_ut_kernel",
       "bwd_block_ut128_kernel",
       "prepare_f32_kernel", "prepare_mfma_bwd_kernel", "bwd_rowdot_kernel",
       "bwd_zero_kernel", "bwd_suffix_kernel")


# the paged decode kernels (row map PagedRows) too
PAGED = (("decode_chunk_paged", "decode_chunk_kernel"), ("decode_merge_paged", "decode_merge_kernel"))


def classify(name: str):
    for cls, key in PAGED:
        if key in name and "PagedRows" in name:
            gated = ", true," in name or ", true>" in name
            return cls + "_fox" if gated else cls
    for cls, key in GATED:
        if key in name and (", true>" in name or ", true," in name):
            return cls
    for cls, key in CLASSES:
        if key in name:
            return cls
    return None


def _one(d: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def read_counters(d: str, counter: str):
    """{dispatch_id: (kernel_name, value)} for one counter of a --pmc run."""
    vals = defaultdict(float)
    names = {}
    with open(_one(d, "*counter_collection.csv")) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            did = int(row["Dispatch_Id"])
            vals[did] += float(row["Counter_Value"])
            names[did] = row["Kernel_Name"]
    return {k: (names[k], vals[k]) for k in vals}


def per_class(counters, copy_factor):
    """Mean scaled bytes per dispatch for each kernel class, and the copy
    reference value (KiB)."""
    ids = sorted(counters)
    first_prep = min((i for i in ids if classify(counters[i][0]) == "prepare"), default=None)
    if first_prep is None:
        raise ValueError("no forward-prepare dispatch in the counter run")
    copies = [i for i in ids if classify(counters[i][0]) == "copy" and i < first_prep]
    if not copies:
        raise ValueError("no copy-reference dispatch before the first prepare dispatch (run bench.py --copy-ref)")
    ref_kib = counters[copies[-1]][1]
    factor = COPY_REF_BYTES / (ref_kib * 1024.0) if copy_factor else 1.0
    acc = defaultdict(list)
    for i in ids:
        c = classify(counters[i][0])
        if c is not None and c != "copy":
            acc[c].append(counters[i][1])
    return ref_kib, factor, {c: (statistics.mean(v), len(v)) for c, v in acc.items()}


def read_stats(d: str):
    rows = []
    with open(_one(d, "*kernel_stats.csv")) as f:
        for row in csv.DictReader(f):
            rows.append((row["Name"], int(row["Calls"]), float(row["AverageNs"]), float(row["Percentage"])))
    return rows


def read_bench(d: str):
    with open(os.path.join(d, "bench.json")) as f:
        lines = [l for l in f.read().splitlines() if l.startswith("{")]
    return json.loads(lines[-1])


def short(name: str) -> str:
    c = classify(name)
    return {"scan": "scan64_kernel (d=64 scan)", "prepare": "prepare_mfma_kernel<64>",
            "cum_padded": "cum_padded_kernel", "decode_chunk": "decode_chunk_kernel<bf16,64>",
            "decode_merge": "decode_merge_kernel<bf16,64>", "copy": "__amd_rocclr_copyBuffer",
            "decode_chunk_fox": "decode_chunk_kernel<bf16,64,gated>",
            "decode_merge_fox": "decode_merge_kernel<bf16,64,gated>",
            "decode_chunk_paged": "decode_chunk_kernel<bf16,64,paged>",
            "decode_merge_paged": "decode_merge_kernel<bf16,64,paged>",
            "decode_chunk_paged_fox": "decode_chunk_kernel<bf16,64,gated,paged>",
            "decode_merge_paged_fox": "decode_merge_kernel<bf16,64,gated,paged>"}.get(c, _short_other(name))


def _short_other(name: str) -> str:
    """A backward kernel's name without its argument list, else the first 60 characters."""
    if "project_kernel" in name:
        return "project_kernel (projection)"
    for key in BWD:
        if key in name:
            if name.startswith("_Z"):  # left mangled (bf16 arguments): the kernel's name alone
                return f"{key} (backward)"
            head = name.split("(")[0].replace("void ", "").replace("path::", "")
            return f"{head} (backward)"
    return name[:60]


def scan_algorithmic_bytes(B, H, L, d):
    """Bytes the scan must move at least once: its workspace inputs (fp16
    hi/lo keys, fp16 hi/lo block transitions, fp32 adjusted queries, fp32
    diagonal logits as a padded lower triangle of 2176 floats per block, fp16
    V^T, per-block norms, value exponents and prefix) and o, lse out."""
    Nb = (L + 63) // 64
    bh = B * H
    khl = bh * Nb * 2 * 64 * d * 2
    pmat = bh * Nb * 2 * d * d * 2
    qhat = bh * Nb * 64 * d * 4
    sdiag = bh * Nb * 2176 * 4
    small = bh * Nb * (4 + 4 + 4 + 64 * 4) + bh * 8
    v = bh * L * d * 2
    o = bh * L * d * 2
    lse = bh * L * 4
    return khl + pmat + qhat + sdiag + small + v + o + lse


def demangle(name: str) -> str:
    """Readable kernel name.  Mangled names of this library's kernels have the
    form _ZN<len><ns><len><name>I<arg>E...: the nested names and one template
    argument (Lb0/Lb1 for a bool, Li<n> for an int) are decoded; other names are
    cut at their parameter list."""
    import re
    if name.startswith("_ZN"):
        s, parts = name[3:], []
        while s and s[0].isdigit():
            m = re.match(r"(\d+)", s)
            n = int(m.group(1))
            parts.append(s[len(m.group(1)):len(m.group(1)) + n])
            s = s[len(m.group(1)) + n:]
        targ = ""
        m = re.match(r"IL(b|i)(\d+)E", s)
        if m:
            targ = "<" + ({"0": "false", "1": "true"}[m.group(2)] if m.group(1) == "b" else m.group(2)) + ">"
        if parts:
            return "::".join(parts) + targ
    return name.split("(")[0].replace("void ", "")


def trace_only(a):
    """Summary of one --kernel-trace --stats run (no counters): per-kernel
    durations and the bench line of the same run."""
    bs = read_bench(a.stats)
    rows = read_stats(a.stats)
    cfg = bs["config"]
    fwd, roof = bs["fwd"], bs["roofline"]
    lines = [f"# rocprofv3 summary: {cfg['workload']}", "",
             "Kernel trace (from the repository root on one MI355X):", "", f"    {a.cmd_stats}", "",
             "| kernel | calls | avg us | share |", "|---|---|---|---|"]
    for name, calls, avg_ns, pct in sorted(rows, key=lambda r: -r[3]):
        lines.append(f"| {demangle(name)} | {calls} | {avg_ns / 1e3:.1f} | {pct:.1f} % |")
    lines += ["", f"bench.py HIP events in the same run (median of {bs['steps']} steps): prepare {fwd['prepare_ms']} ms, "
              f"scan {fwd['scan_ms']} ms, forward {fwd['ms']} ms.",
              f"Forward: {fwd['flops_model']:.4e} FLOP per launch / {fwd['ms']} ms = {bs['value']} TFLOP/s "
              f"= {100 * fwd['frac_bf16_peak']:.1f} % of 2.5 PFLOP/s.",
              f"Scan ({roof['kernel']}): {roof['achieved']} TFLOP/s = {100 * roof['frac']:.1f} % of the MFMA peak.",
              ""]
    with open(a.md, "w") as f:
        f.write("\n".join(lines))


# MI355X: 8 XCDs of 32 CUs, 4 SIMDs per CU.  GRBM_GUI_ACTIVE is summed over
# the XCDs; the SQ_*_CYCLES counters count quad-cycles (units of 4 clocks).
N_XCD, N_SIMD = 8, 1024
MFMA_FLOP = 16 * 16 * 32 * 2  # one v_mfma_f32_16x16x32_f16


def read_sq(dirs):
    """{kernel: {counter: mean per dispatch, '_us': mean duration, '_n': dispatches}}
    over the forward kernels of several --pmc runs (each counter from the run
    that collected it)."""
    out = {}
    for d in dirs:
        per = defaultdict(dict)
        with open(_one(d, "*counter_collection.csv")) as f:
            for row in csv.DictReader(f):
                name = demangle(row["Kernel_Name"])
                if not any(k in name for k in ("scan64_kernel", "scan128_kernel", "prepare_mfma_kernel")):
                    continue
                rec = per[(name, int(row["Dispatch_Id"]))]
                rec[row["Counter_Name"]] = rec.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
                rec["_us"] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
        by = defaultdict(list)
        for (name, _), rec in per.items():
            by[name].append(rec)
        for name, recs in by.items():
            agg = out.setdefault(name, {})
            for key in recs[0]:
                vals = [r[key] for r in recs if key in r]
                if key == "_us":
                    agg.setdefault("_us_all", []).extend(vals)
                else:
                    agg[key] = statistics.mean(vals)
            agg["_n"] = max(agg.get("_n", 0), len(recs))
    for agg in out.values():
        agg["_us"] = statistics.median(agg.pop("_us_all"))
    return out


def sq_table(sq, flops=None):
    """Markdown rows of derived shader metrics per kernel.

    clock = GRBM_GUI_ACTIVE / 8 / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /
    (1024 SIMDs x GRBM_GUI_ACTIVE / 8); useful MFMA = model FLOP / 16384 per
    instruction over SQ_INSTS_MFMA (scan kernels only); VALU/MFMA =
    SQ_INSTS_VALU / SQ_INSTS_MFMA (SQ_INSTS_VALU includes the MFMAs); VALU
    active, dependency wait and any wait = SQ_ACTIVE_INST_VALU, SQ_WAIT_INST_ANY
    and SQ_WAIT_ANY over SQ_WAVE_CYCLES; LDS conflicts = SQ_LDS_BANK_CONFLICT /
    SQ_ACTIVE_INST_LDS; L2 latency = TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum."""
    def g(a, k):
        return a.get(k)

    def pct(x):
        return "-" if x is None else f"{100 * x:.1f} %"

    def ratio(a, b):
        return None if a is None or not b else a / b

    rows = ["| kernel | dispatches | median us | clock GHz | MFMA instr | MFMA busy | useful MFMA | VALU / MFMA "
            "| VALU active | dependency wait | any wait | LDS conflict / LDS active | L1->L2 latency (cycles) |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for name in sorted(sq):
        a = sq[name]
        us = a["_us"]
        grbm = g(a, "GRBM_GUI_ACTIVE")
        clock = None if grbm is None else grbm / N_XCD / (us * 1e3)
        busy = ratio(g(a, "SQ_VALU_MFMA_BUSY_CYCLES"), None if grbm is None else N_SIMD * grbm / N_XCD)
        useful = None
        if flops and "scan" in name and g(a, "SQ_INSTS_MFMA"):
            useful = flops / MFMA_FLOP / a["SQ_INSTS_MFMA"]
        vpm = ratio(g(a, "SQ_INSTS_VALU"), g(a, "SQ_INSTS_MFMA"))
        wc = g(a, "SQ_WAVE_CYCLES")
        lat = ratio(g(a, "TCP_TCC_READ_REQ_LATENCY_sum"), g(a, "TCP_TCC_READ_REQ_sum"))
        nmfma = g(a, "SQ_INSTS_MFMA")
        rows.append(
            f"| {name} | {a['_n']} | {us:.1f} | {'-' if clock is None else f'{clock:.2f}'} | "
            f"{'-' if nmfma is None else f'{nmfma:.4g}'} | {pct(busy)} | "
            f"{pct(useful)} | {'-' if vpm is None else f'{vpm:.2f}'} | {pct(ratio(g(a, 'SQ_ACTIVE_INST_VALU'), wc))} | "
            f"{pct(ratio(g(a, 'SQ_WAIT_INST_ANY'), wc))} | {pct(ratio(g(a, 'SQ_WAIT_ANY'), wc))} | "
            f"{pct(ratio(g(a, 'SQ_LDS_BANK_CONFLICT'), g(a, 'SQ_ACTIVE_INST_LDS')))} | "
            f"{'-' if lat is None else f'{lat:.0f}'} |")
    return rows


def sq_summary(a):
    bench = read_bench(a.sq[0])
    cfg = bench["config"]
    sq = read_sq(a.sq)
    lines = [f"# rocprofv3 shader counters: {cfg['workload']}", "",
             f"Precision {cfg.get('precision')}.  Counter runs (from the repository root on one MI355X), one "
             "counter set each:", ""]
    lines += [f"    {c}" for c in a.cmds]
    lines += ["", *sq_table(sq, bench["fwd"]["flops_model"]), "",
              "Formulas: " + " ".join(sq_table.__doc__.split("\n\n", 1)[1].split()), ""]
    with open(a.md, "w") as f:
        f.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--sq", nargs="+")
    ap.add_argument("--cmds", nargs="+")
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--md", required=True)
    ap.add_argument("--json")
    ap.add_argument("--cmd-stats")
    ap.add_argument("--cmd-fetch")
    ap.add_argument("--cmd-write")
    a = ap.parse_args()
    if a.sq:
        sq_summary(a)
        return
    if a.fetch is None:
        trace_only(a)
        return

    bs, bf, bw = read_bench(a.stats), read_bench(a.fetch), read_bench(a.write)
    for k in ("roofline", "decode"):
        hs = {b[k]["source_sha256"] for b in (bs, bf, bw)}
        if len(hs) != 1:
            raise ValueError(f"the three runs did not profile the same {k} kernel source")
    # the runs' sources must be the tree's: the hashes recorded below are this tree's
    for k, kind in (("roofline", "scan"), ("decode", "decode")):
        if bs[k]["source_sha256"] != source_hash(kind):
            raise ValueError(f"the {kind} kernel source changed since the profiled runs")
    fref, ffac, fetch = per_class(read_counters(a.fetch, "FETCH_SIZE"), True)
    wref, wfac, write = per_class(read_counters(a.write, "WRITE_SIZE"), True)

    def traffic(cls_list):
        fb = sum(fetch[c][0] for c in cls_list if c in fetch) * 1024.0 * ffac
        wb = sum(write[c][0] for c in cls_list if c in write) * 1024.0 * wfac
        return fb, wb

    cfg = bs["config"]
    B, H, L, d = cfg["global_batch"], cfg["heads"], cfg["seq_len"], cfg["head_dim"]
    scan_f, scan_w = traffic(["scan"])
    dec_f, dec_w = traffic(["decode_chunk", "decode_merge"])
    prep_f, prep_w = traffic(["prepare", "cum_padded"])
    alg_scan = scan_algorithmic_bytes(B, H, L, d)
    alg_dec = bs["decode"]["bytes_model"]
    out = {
        "what": "HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a 1 GiB device copy",
        "copy_ref": {"bytes_each_way": COPY_REF_BYTES, "fetch_kib": fref, "write_kib": wref,
                     "fetch_factor": ffac, "write_factor": wfac},
        "scan": {"kernel": "scan64_kernel<false>", "source_sha256": bs["roofline"]["source_sha256"],
                 "fetch_bytes_per_launch": scan_f, "write_bytes_per_launch": scan_w,
                 "bytes_per_launch": scan_f + scan_w, "algorithmic_bytes": alg_scan},
        "decode": {"kernel": "decode_chunk_kernel + decode_merge_kernel", "source_sha256":
                   bs["decode"]["source_sha256"], "fetch_bytes_per_launch": dec_f, "write_bytes_per_launch": dec_w,
                   "bytes_per_launch": dec_f + dec_w, "algorithmic_bytes": alg_dec},
        "prepare": {"kernel": "prepare_mfma_kernel (+ cum_padded_kernel with gates)", "fetch_bytes_per_launch": prep_f,
                    "write_bytes_per_launch": prep_w, "bytes_per_launch": prep_f + prep_w},
        "commands": {"fetch": a.cmd_fetch, "write": a.cmd_write},
    }
    with open(a.json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")

    stats = read_stats(a.stats)
    scan_avg = next((s[2] for s in stats if classify(s[0]) == "scan"), None)
    MiB = 1024.0 * 1024.0
    lines = [
        f"# rocprofv3 summary: PaTH forward scan + prepare (B={B} H={H} L={L} d={d}) and decode step",
        "",
        f"Workload: {cfg['workload']}; precision {cfg['precision']}.",
        "",
        "Kernel trace (from the repository root on one MI355X):",
        "",
        f"    {a.cmd_stats}",
        "",
        "| kernel | calls | avg us | share |",
        "|---|---|---|---|",
    ]
    for name, calls, avg, pct in stats[:12]:
        lines.append(f"| {short(name)} | {calls} | {avg / 1e3:.1f} | {pct:.1f} % |")
    r = bs["roofline"]
    lines += [
        "",
        f"bench.py HIP events in the same run (median of {bs['steps']} steps): prepare "
        f"{bs['fwd']['prepare_ms']:.4f} ms, scan {bs['fwd']['scan_ms']:.4f} ms, decode {bs['decode']['ms']:.4f} ms.",
        f"rocprofv3 average of the scan kernel: {scan_avg / 1e6:.4f} ms." if scan_avg else "",
        f"Scan roofline: {r['flops_per_launch']:.4e} FLOP per launch / {r['launch_ms']:.4f} ms = "
        f"{r['achieved']:.1f} TFLOP/s = {100 * r['frac']:.1f} % of 2.5 PFLOP/s.",
        f"Decode: {bs['decode']['GB_per_s']:.1f} GB/s on {alg_dec:.4e} algorithmic bytes "
        f"({100 * bs['decode']['frac_hbm_peak']:.1f} % of 8 TB/s).",
        "",
        "HBM traffic (two counter runs):",
        "",
        f"    {a.cmd_fetch}",
        f"    {a.cmd_write}",
        "",
        f"Copy reference (1 GiB read + 1 GiB written): FETCH_SIZE {fref:.0f} KiB -> factor {ffac:.4f}; "
        f"WRITE_SIZE {wref:.0f} KiB -> factor {wfac:.4f}.",
        "",
        "| kernel | fetch MiB/launch | write MiB/launch | total MiB | algorithmic MiB |",
        "|---|---|---|---|---|",
        f"| scan | {scan_f / MiB:.1f} | {scan_w / MiB:.1f} | {(scan_f + scan_w) / MiB:.1f} | {alg_scan / MiB:.1f} |",
        f"| prepare | {prep_f / MiB:.1f} | {prep_w / MiB:.1f} | {(prep_f + prep_w) / MiB:.1f} | - |",
        f"| decode (chunk + merge) | {dec_f / MiB:.1f} | {dec_w / MiB:.1f} | {(dec_f + dec_w) / MiB:.1f} | "
        f"{alg_dec / MiB:.1f} |",
        "",
        "Dispatches counted per class (fetch run): " + ", ".join(f"{c} {n}" for c, (_, n) in sorted(fetch.items())),
        "",
        f"Scan kernel source sha256: {bs['roofline']['source_sha256']}",
        f"Decode kernel source sha256: {bs['decode']['source_sha256']}",
        "",
    ]
    with open(a.md, "w") as f:
        f.write("\n".join(l for l in lines if l is not None))


if __name__ == "__main__":
    main()
