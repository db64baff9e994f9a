"""Condense rocprofv3 CSV output into the short text summaries kept beside the
benchmark (run by path, on any host; it reads CSV files only).

    python profile_counters.py stats <kernel_stats.csv> <out.txt> "<command>"
    python profile_counters.py traffic <fetch counter_collection.csv> \\
        <write counter_collection.csv> <kernel source> <out.json> "<command>" [<kernel name>]
    python profile_counters.py counters <out.txt> "<command>" \\
        <counter_collection.csv> [<counter_collection.csv> ...]
    python profile_counters.py trace <kernel_trace.csv> <out.txt> \\
        "<command>" [<kernel substring>@<grid size x> ...]

`trace` reads a kernel trace and reports, per kernel and grid size, the
median duration of its dispatches, with the timeline split into phases at
the first dispatch of each "kernel@grid" marker given (a benchmark that runs
several workloads one after the other).

`counters` averages every counter per dispatch for the decode kernels (the
launch that builds its own candidate lists apart from the plain one), the
dense decode and extend kernels and the row-gather diagnostic (whose launches come in two runs of equal length: the
decode's placement first, then each row read once) and derives the figures
quoted beside the benchmark.

`traffic` scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what the same
counters read for the benchmark's calibration copy (a 256 MiB device-to-device
copy launched three times before warm-up), then reports a kernel's (by default the sparse decode kernel's)
HBM bytes per launch together with a hash of the kernel source they were
taken on, so that a later edit of the kernel invalidates them.
"""

import csv
import hashlib
import json
import sys
from collections import defaultdict

DECODE_KERNEL = "sparse_mla_decode_kernel"
OTHER_KERNELS = ("extend_attention_kernel", "paged_gqa_decode_kernel")
COPY_BYTES = 256 << 20


def short_name(name):
    if name.startswith("(anonymous namespace)::"):
        return name[len("(anonymous namespace)::"):].split("(")[0]
    if name.startswith("void (anonymous namespace)::"):
        return name[len("void (anonymous namespace)::"):].split("(")[0]
    if name.startswith("__amd_rocclr"):
        return name
    return name.split("(")[0][:90]


def stats(src, out, command):
    rows = list(csv.DictReader(open(src)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}", "#",
             f"{'kernel':<58} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for r in rows:
        lines.append(f"{short_name(r['Name']):<58} {int(r['Calls']):>6} "
                     f"{float(r['AverageNs']) / 1e3:>9.3f} {float(r['MinNs']) / 1e3:>9.3f} "
                     f"{float(r['MaxNs']) / 1e3:>9.3f} {float(r['Percentage']):>6.2f}")
    open(out, "w").write("\n".join(lines) + "\n")


def per_kernel(path, counter):
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return vals


def calibration(vals, expect_kib):
    # the copy is a runtime blit kernel; pick the dispatches whose reading is
    # closest to the known size (the same kernel also serves small copies)
    cands = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs if v > expect_kib / 4]
    if not cands:
        raise SystemExit("no calibration copy found in the counter file")
    got = sum(cands) / len(cands)
    return expect_kib / got, got


def traffic(fetch_csv, write_csv, kernel_src, out, command, kernel=DECODE_KERNEL):
    kib = COPY_BYTES / 1024
    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    f_scale, f_copy = calibration(fetch, kib)
    w_scale, w_copy = calibration(write, kib)
    dec_f = [v for k, vs in fetch.items() if kernel in k for v in vs]
    dec_w = [v for k, vs in write.items() if kernel in k for v in vs]
    f_avg, w_avg = sum(dec_f) / len(dec_f), sum(dec_w) / len(dec_w)
    rec = {
        "command": command,
        "kernel": kernel,
        "kernel_source_sha": hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()[:16],
        "dispatches": [len(dec_f), len(dec_w)],
        "fetch_kib_raw": round(f_avg, 3),
        "write_kib_raw": round(w_avg, 3),
        "copy_fetch_kib_raw": round(f_copy, 3),
        "copy_write_kib_raw": round(w_copy, 3),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "hbm_read_bytes_per_launch": int(f_avg * f_scale * 1024),
        "hbm_write_bytes_per_launch": int(w_avg * w_scale * 1024),
    }
    rec["hbm_bytes_per_launch"] = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    others = {}
    for k in sorted(set(fetch) | set(write)):
        if k.startswith("__amd") or "at::native" in k or "void at" in k:
            continue
        fv, wv = fetch.get(k, []), write.get(k, [])
        others[k] = {"read_bytes": int(sum(fv) / max(len(fv), 1) * f_scale * 1024),
                     "write_bytes": int(sum(wv) / max(len(wv), 1) * w_scale * 1024)}
    rec["per_kernel"] = others
    json.dump(rec, open(out, "w"), indent=1)
    open(out, "a").write("\n")


def trace(src, out, command, *markers):
    """Median duration per (phase, kernel, grid) from a kernel trace."""
    rows = sorted(csv.DictReader(open(src)), key=lambda r: int(r["Start_Timestamp"]))
    starts = []
    for m in markers:
        name, grid = m.rsplit("@", 1)
        hit = [int(r["Start_Timestamp"]) for r in rows
               if name in r["Kernel_Name"] and r["Grid_Size_X"] == grid]
        if hit:
            starts.append((hit[0], m))
    starts.sort()
    groups = defaultdict(list)
    for r in rows:
        t0 = int(r["Start_Timestamp"])
        phase = 0
        for i, (ts, _) in enumerate(starts):
            if t0 >= ts:
                phase = i + 1
        k = short_name(r["Kernel_Name"])
        if k.startswith("__amd") or "at::native" in k:
            continue
        groups[(phase, k, int(r["Grid_Size_X"]))].append(
            (int(r["End_Timestamp"]) - t0) / 1e3)
    lines = ["# rocprofv3 kernel trace, median per kernel and grid size", f"# command: {command}",
             "# phases: 0 = start" + "".join(f"; {i + 1} = from the first {m}"
                                                for i, (_, m) in enumerate(starts)),
             "#", f"{'phase':>5} {'kernel':<52} {'grid_x':>8} {'calls':>6} {'median_us':>10} "
                  f"{'p10_us':>8} {'p90_us':>8}"]
    for (phase, k, g), ds in sorted(groups.items()):
        ds.sort()
        pick = lambda f: ds[min(len(ds) - 1, int(f * len(ds)))]  # noqa: E731
        lines.append(f"{phase:>5} {k:<52} {g:>8} {len(ds):>6} {pick(0.5):>10.2f} "
                     f"{pick(0.1):>8.2f} {pick(0.9):>8.2f}")
    open(out, "w").write("\n".join(lines) + "\n")


def counters(out, command, *paths):
    """Per-dispatch means of every collected counter, per kernel of interest."""
    groups = defaultdict(lambda: defaultdict(dict))  # kernel -> dispatch -> counter -> value
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = short_name(r["Kernel_Name"])
            if DECODE_KERNEL in k:  # the launch that builds its lists, or the plain one
                k = DECODE_KERNEL + (" (with normalisation)" if k.endswith("true>") else "")
            elif "row_gather" in k:  # the register or the LDS-ring variant
                k = "row_gather_kernel"
            elif not any(name in k for name in OTHER_KERNELS):
                continue
            d = groups[k][(path, int(r["Dispatch_Id"]))]
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    split = {}
    for k, disp in groups.items():
        if k == "row_gather_kernel":
            for path in paths:
                ids = sorted(i for (p, i) in disp if p == path)
                half = len(ids) // 2
                for n, sel in (("row_gather (decode placement)", ids[:half]),
                               ("row_gather (each row once)", ids[half:])):
                    split.setdefault(n, {}).update({(path, i): disp[(path, i)] for i in sel})
        else:
            split[k] = disp
    lines = ["# rocprofv3 hardware counters, mean per dispatch", f"# command: {command}", "#"]
    for k, disp in split.items():
        names = sorted({c for d in disp.values() for c in d})
        lines.append(f"{k}  ({len(disp)} dispatches across the passes)")
        for c in names:
            vals = [d[c] for d in disp.values() if c in d]
            lines.append(f"  {c:<40} {sum(vals) / len(vals):>16.1f}")
        m = {c: sum(d[c] for d in disp.values() if c in d) / max(1, sum(1 for d in disp.values() if c in d))
             for c in names}
        if "TCP_TCC_READ_REQ_sum" in m and m["TCP_TCC_READ_REQ_sum"]:
            lines.append(f"  -> mean L2 round trip seen by the L1 (cycles)  "
                         f"{m.get('TCP_TCC_READ_REQ_LATENCY_sum', 0) / m['TCP_TCC_READ_REQ_sum']:.0f}")
        if "SQ_INSTS_VALU" in m and m.get("SQ_INSTS_MFMA"):
            lines.append(f"  -> VALU instructions per MFMA                  "
                         f"{m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f}")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
            lines.append(f"  -> bf16 MFMA work (GFLOP, 512 flop per MOP)     "
                         f"{m['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.3f}")
        if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m and (m["TCC_HIT_sum"] + m["TCC_MISS_sum"]):
            lines.append(f"  -> L2 hit rate                                 "
                         f"{m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.3f}")
    open(out, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(*sys.argv[2:5])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:8])
    elif sys.argv[1] == "counters":
        counters(*sys.argv[2:])
    elif sys.argv[1] == "trace":
        trace(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
