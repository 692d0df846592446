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
    ("head_reduce", "head_reduce_kernel"),
    ("decode_chunk", "decode_chunk_kernel"),
    ("decode_merge", "decode_merge_kernel"),
    ("copy", "copyBuffer"),
)


# the gated decode kernels (template flag true) form classes of their own
GATED = (("decode_chunk_fox", "decode_chunk_kernel"), ("decode_merge_fox", "decode_merge_kernel"))
BWD = ("bwd_pair_kernel", "bwd_block_kernel", "prepare_f32_kernel", "bwd_rowdot_kernel", "bwd_zero_kernel",
       "bwd_suffix_kernel")


# the paged decode kernels (row map PagedRows) too
PAGED = (("decode_chunk_paged", "decode_chunk_kernel"), ("decode_merge_paged", "decode_merge_kernel"))


def classify(name: str):
    for cls, key in PAGED:
        if key in name and "PagedRows" in name:
            return cls
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
            "head_reduce": "head_reduce_kernel", "decode_chunk": "decode_chunk_kernel<bf16,64>",
            "decode_merge": "decode_merge_kernel<bf16,64>", "copy": "__amd_rocclr_copyBuffer",
            "decode_chunk_fox": "decode_chunk_kernel<bf16,64,gated>",
            "decode_merge_fox": "decode_merge_kernel<bf16,64,gated>",
            "decode_chunk_paged": "decode_chunk_kernel<bf16,64,paged>",
            "decode_merge_paged": "decode_merge_kernel<bf16,64,paged>"}.get(c, _short_other(name))


def _short_other(name: str) -> str:
    """A backward kernel's name without its argument list, else the first 60 characters."""
    if "project_kernel" in name:
        return "project_kernel (projection)"
    for key in BWD:
        if key in name:
            head = name.split("(")[0].replace("void ", "").replace("path::", "")
            return f"{head} (backward)"
    return name[:60]


def scan_algorithmic_bytes(B, H, L, d):
    """Bytes the scan must move at least once: its workspace inputs (fp16
    hi/lo keys, fp16 hi/lo block transitions, fp32 adjusted queries, fp32
    diagonal logits, fp16 V^T, per-block norms and prefix) and o, lse out."""
    Nb = (L + 63) // 64
    bh = B * H
    khl = bh * Nb * 2 * 64 * d * 2
    pmat = bh * Nb * 2 * d * d * 2
    qhat = bh * Nb * 64 * d * 4
    sdiag = bh * Nb * 64 * 64 * 4
    small = bh * Nb * (4 + 4 + 64 * 4) + bh * 4
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--md", required=True)
    ap.add_argument("--json")
    ap.add_argument("--cmd-stats", required=True)
    ap.add_argument("--cmd-fetch")
    ap.add_argument("--cmd-write")
    a = ap.parse_args()
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
    prep_f, prep_w = traffic(["prepare", "head_reduce"])
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
        "prepare": {"kernel": "prepare_mfma_kernel + head_reduce_kernel", "fetch_bytes_per_launch": prep_f,
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
        f"| prepare + head reduce | {prep_f / MiB:.1f} | {prep_w / MiB:.1f} | {(prep_f + prep_w) / MiB:.1f} | - |",
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
