"""Profiling helpers: HBM-traffic calibration and rocprofv3 summaries.

    python -m combine_wave_level_amd.profiling copy [--mib N] [--reps R]
        A plain device-to-device copy of N MiB (R times): the reference whose
        FETCH_SIZE / WRITE_SIZE counters calibrate the traffic counters.

    python -m combine_wave_level_amd.profiling stats --stats S.csv --title T
        --command "..." --out-md X.md [--top N]
        Writes a short markdown table of the kernel durations of a
        --kernel-trace --stats run (the N longest by total time).

    python -m combine_wave_level_amd.profiling steptraffic --fetch F.csv --write W.csv
        --copy-fetch CF.csv --copy-write CW.csv --kernels K1 K2 ... --title T
        --command "..." --out-md X.md [--out-json X.json --workload W --T T]
        Writes the calibrated HBM bytes of one pass over kernels that each
        run once per pass (the phase schedule's GEMM1, GEMM2 and combine),
        and optionally the JSON record bench.py reports as roofline.traffic
        for that schedule.

    python -m combine_wave_level_amd.profiling summarize --stats S.csv
        --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv
        --kernel NAME --workload W --T T --command "..." --out-md X.md
        --out-json X.json [--copy-mib N]
        Writes a short markdown summary (kernel durations from the
        --kernel-trace --stats run, HBM bytes per launch of NAME) and the JSON
        record bench.py reports as roofline.traffic.

The traffic record carries a digest of the sources the measured kernel is
built from (its .hip file and the device headers it includes); bench.py
reports it only while those still hash to the same digest (a changed kernel
makes the measured bytes stale).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


# Sources each measured kernel is compiled from (device code and its launch).
KERNEL_SOURCES = {
    "ffn_waved_kernel": ["ffn.hip", "ffn_parts.h", "gemm_tile.h", "moe_common.h", "wave_sched.h"],
    "phase_kernels": ["ffn.hip", "ffn_parts.h", "gemm_tile.h", "moe_common.h", "wave_sched.h"],
}


def _sources(kernel: str | None):
    if kernel in KERNEL_SOURCES:
        return [os.path.join(CSRC, n) for n in KERNEL_SOURCES[kernel]]
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))


def source_digest(kernel: str | None = None) -> str:
    """sha256 over the sources of `kernel` (all library sources when it is not
    listed in KERNEL_SOURCES), in a fixed order."""
    h = hashlib.sha256()
    for p in _sources(kernel):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(path: str, workload: str, T: int):
    """The traffic record at path if it matches the workload, T and the
    current sources; else None."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("source_digest") != source_digest(rec.get("kernel")) or rec.get("workload") != workload
            or rec.get("T") != T):
        return None
    return rec


def _copy(args) -> None:
    import torch

    n = args.mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": args.reps}))


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _kernel_counter(path, pattern, counter):
    """Mean per dispatch of `counter` over dispatches whose name matches."""
    vals = [float(r["Counter_Value"]) for r in _rows(path)
            if re.search(pattern, r["Kernel_Name"]) and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for /{pattern}/ in {path}")
    return sum(vals) / len(vals), len(vals)


def _short(name: str) -> str:
    name = name.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    name = re.sub(r"\([^()]*\)$", "", name)  # argument list
    return name.replace("moe::", "")


def _summarize(a) -> None:
    stats = _rows(a.stats)
    lines = [f"# {a.kernel}: {a.workload}, T={a.T}", "",
             "Commands (run from /tmp with TMPDIR=/tmp; REPO = repository root, OUT = the profiler output folder):", ""]
    for c in a.command:
        lines.append(f"    {c}")
    lines += ["", "Kernel durations (--kernel-trace --stats):", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    fetch_kib, nf = _kernel_counter(a.fetch, a.kernel, "FETCH_SIZE")
    write_kib, nw = _kernel_counter(a.write, a.kernel, "WRITE_SIZE")
    cf_kib, _ = _kernel_counter(a.copy_fetch, a.copy_kernel, "FETCH_SIZE")
    cw_kib, _ = _kernel_counter(a.copy_write, a.copy_kernel, "WRITE_SIZE")
    copy_bytes = a.copy_mib * (1 << 20)
    f_fetch = cf_kib * 1024.0 / copy_bytes
    f_write = cw_kib * 1024.0 / copy_bytes
    fetch_b = fetch_kib * 1024.0 / f_fetch
    write_b = write_kib * 1024.0 / f_write
    avg_ns = [float(r["AverageNs"]) for r in stats if re.search(a.kernel, r["Name"])]
    lines += ["", f"HBM traffic per launch of {a.kernel} (--pmc FETCH_SIZE, --pmc WRITE_SIZE; "
              f"{nf} and {nw} dispatches):", "",
              f"- FETCH_SIZE {fetch_kib:.0f} KiB, WRITE_SIZE {write_kib:.0f} KiB per dispatch;",
              f"- a plain {a.copy_mib} MiB copy reads FETCH_SIZE {cf_kib:.0f} KiB and WRITE_SIZE "
              f"{cw_kib:.0f} KiB: factors {f_fetch:.3f} (fetch) and {f_write:.3f} (write) per byte moved;",
              f"- calibrated: {fetch_b / 1e6:.1f} MB read + {write_b / 1e6:.1f} MB written = "
              f"{(fetch_b + write_b) / 1e6:.1f} MB per launch"]
    if avg_ns:
        lines.append(f"- at the average duration {avg_ns[0] / 1e3:.1f} us: "
                     f"{(fetch_b + write_b) / (avg_ns[0] * 1e-9) / 1e9:.0f} GB/s")
    rec = {"kernel": a.kernel, "workload": a.workload, "T": a.T, "source_digest": source_digest(a.kernel),
           "sources": [os.path.basename(p) for p in _sources(a.kernel)],
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "traffic_bytes": round(fetch_b + write_b), "fetch_factor": round(f_fetch, 4),
           "write_factor": round(f_write, 4), "avg_us": round(avg_ns[0] / 1e3, 2) if avg_ns else None}
    lines += ["", f"Source digest of the measured kernels: `{rec['source_digest'][:16]}`", ""]
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines))
    with open(a.out_json, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def _step_traffic(a) -> None:
    """HBM bytes of one pass over several kernels (each launched once per
    pass): the sum over the kernels of their mean calibrated bytes per
    dispatch."""
    cf_kib, _ = _kernel_counter(a.copy_fetch, a.copy_kernel, "FETCH_SIZE")
    cw_kib, _ = _kernel_counter(a.copy_write, a.copy_kernel, "WRITE_SIZE")
    copy_bytes = a.copy_mib * (1 << 20)
    f_fetch = cf_kib * 1024.0 / copy_bytes
    f_write = cw_kib * 1024.0 / copy_bytes
    lines = [f"# {a.title}", "",
             "Commands (run from /tmp with TMPDIR=/tmp; REPO = repository root, OUT = the profiler output folder):", ""]
    for c in a.command:
        lines.append(f"    {c}")
    lines += ["", f"Calibration: a plain {a.copy_mib} MiB copy reads FETCH_SIZE {cf_kib:.0f} KiB and WRITE_SIZE "
              f"{cw_kib:.0f} KiB: factors {f_fetch:.3f} (fetch) and {f_write:.3f} (write) per byte moved.", "",
              "| kernel | dispatches | read MB | written MB |", "|---|---|---|---|"]
    tot_r = tot_w = 0.0
    for k in a.kernels:
        fk, nf = _kernel_counter(a.fetch, k, "FETCH_SIZE")
        wk, nw = _kernel_counter(a.write, k, "WRITE_SIZE")
        rb, wb = fk * 1024.0 / f_fetch, wk * 1024.0 / f_write
        tot_r += rb
        tot_w += wb
        lines.append(f"| {k} | {nf} / {nw} | {rb / 1e6:.1f} | {wb / 1e6:.1f} |")
    lines += ["", f"One pass: {tot_r / 1e6:.1f} MB read + {tot_w / 1e6:.1f} MB written = "
              f"{(tot_r + tot_w) / 1e6:.1f} MB.", ""]
    rec = {"read_bytes": round(tot_r), "write_bytes": round(tot_w)}
    if a.out_json:
        if a.workload is None or a.T is None:
            raise SystemExit("--out-json needs --workload and --T")
        rec = {"kernel": "phase_kernels", "kernels": a.kernels, "workload": a.workload, "T": a.T,
               "source_digest": source_digest("phase_kernels"),
               "sources": [os.path.basename(p) for p in _sources("phase_kernels")],
               "fetch_bytes": round(tot_r), "write_bytes": round(tot_w), "traffic_bytes": round(tot_r + tot_w),
               "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)}
        lines += [f"Source digest of the measured kernels: `{rec['source_digest'][:16]}`", ""]
        with open(a.out_json, "w") as f:
            json.dump(rec, f, indent=1)
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(rec))


def _stats(a) -> None:
    rows = _rows(a.stats)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]) if "TotalDurationNs" in r
              else -float(r["AverageNs"]) * float(r["Calls"]))
    lines = [f"# {a.title}", "",
             "Commands (run from /tmp with TMPDIR=/tmp; REPO = repository root, OUT = the profiler output folder):", ""]
    for c in a.command:
        lines.append(f"    {c}")
    lines += ["", "Kernel durations (--kernel-trace --stats):", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows[:a.top]:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines.append("")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines))


def _counters(a) -> None:
    """Per-dispatch means of the tile counters of the given kernels (a
    --pmc CSV per pass; counters may repeat across passes, the first pass
    that has one is used)."""
    vals: dict = {}
    for path in a.pmc:
        for r in _rows(path):
            for k in a.kernels:
                if re.search(k, r["Kernel_Name"]):
                    d = vals.setdefault(k, {}).setdefault(r["Counter_Name"], {})
                    d.setdefault(path, []).append(float(r["Counter_Value"]))

    def m(k, name):
        per = vals.get(k, {}).get(name)
        if not per:
            return float("nan")
        v = next(iter(per.values()))
        return sum(v) / len(v)

    cus, simds = 256, 1024
    figs = []
    for k in a.kernels:
        act = m(k, "GRBM_GUI_ACTIVE") / 8
        req = m(k, "TCP_TCC_READ_REQ")
        hit, miss = m(k, "TCC_HIT"), m(k, "TCC_MISS")
        figs.append([
            f"{act / 1e3:.0f} K",
            f"{100 * m(k, 'SQ_VALU_MFMA_BUSY_CYCLES') / simds / act:.0f}%",
            f"{m(k, 'SQ_INSTS_VALU_MFMA_MOPS_BF16') * 512 / 1e9:.0f} G",
            f"{100 * m(k, 'SQ_LDS_IDX_ACTIVE') / cus / act:.0f}%",
            f"{100 * m(k, 'SQ_LDS_BANK_CONFLICT') / m(k, 'SQ_LDS_IDX_ACTIVE'):.1f}%",
            f"{100 * m(k, 'SQ_WAIT_ANY') / m(k, 'SQ_WAVE_CYCLES'):.0f}%",
            f"{m(k, 'VmemLatency'):.0f} cycles",
            f"{100 * m(k, 'TA_TA_BUSY') / cus / act:.0f}%",
            f"{100 * m(k, 'TD_TD_BUSY') / cus / act:.0f}%",
            f"{100 * m(k, 'TD_TC_STALL') / cus / act:.0f}%",
            f"{req / 1e6:.1f} M",
            f"{m(k, 'TCP_TCC_READ_REQ_LATENCY') / req:.0f} cycles",
            f"{100 * hit / (hit + miss):.0f}%",
        ])
    names = ["GPU-active cycles per XCD", "MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / active)",
             "bf16 MFMA FLOPs (MOPS_BF16 x 512)", "LDS busy (SQ_LDS_IDX_ACTIVE / CUs / active)",
             "LDS bank-conflict cycles / LDS active cycles",
             "wave-cycles waiting in s_waitcnt (SQ_WAIT_ANY / SQ_WAVE_CYCLES)",
             "mean vector-memory latency (VmemLatency)", "TA busy per CU", "TD busy per CU",
             "TD stalled on the L1 (TD_TC_STALL per CU)", "L1 -> L2 read requests",
             "mean L1 -> L2 read latency", "L2 hit rate (TCC_HIT / (HIT + MISS))"]
    lines = [f"# {a.title}", "",
             "Commands (run from /tmp with TMPDIR=/tmp; REPO = repository root, OUT = the profiler output folder):", ""]
    for c in a.command:
        lines.append(f"    {c}")
    lines += ["", "Per-dispatch means over the profiled dispatches.  GRBM_GUI_ACTIVE is summed over the 8 XCDs",
              "(divided by 8 below); SQ/TA/TD counters are chip totals, divided by the 1024 SIMDs or 256 CUs.", "",
              "| figure | " + " | ".join(a.kernels) + " |", "|---|" + "---|" * len(a.kernels)]
    for i, n in enumerate(names):
        lines.append(f"| {n} | " + " | ".join(f[i] for f in figs) + " |")
    lines.append("")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines))


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(prog="python -m combine_wave_level_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=3)
    t = sub.add_parser("stats")
    t.add_argument("--stats", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--command", action="append", default=[])
    t.add_argument("--out-md", required=True)
    t.add_argument("--top", type=int, default=16)
    q = sub.add_parser("counters")
    q.add_argument("--pmc", action="append", required=True)
    q.add_argument("--kernels", nargs="+", required=True)
    q.add_argument("--title", required=True)
    q.add_argument("--command", action="append", default=[])
    q.add_argument("--out-md", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--stats", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-fetch", required=True)
    s.add_argument("--copy-write", required=True)
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--copy-kernel", default="copy|Copy")
    s.add_argument("--kernel", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--T", type=int, required=True)
    s.add_argument("--command", action="append", default=[])
    s.add_argument("--out-md", required=True)
    s.add_argument("--out-json", required=True)
    st = sub.add_parser("steptraffic")
    st.add_argument("--fetch", required=True)
    st.add_argument("--write", required=True)
    st.add_argument("--copy-fetch", required=True)
    st.add_argument("--copy-write", required=True)
    st.add_argument("--copy-mib", type=int, default=1024)
    st.add_argument("--copy-kernel", default="copy|Copy")
    st.add_argument("--kernels", nargs="+", required=True)
    st.add_argument("--title", required=True)
    st.add_argument("--command", action="append", default=[])
    st.add_argument("--out-md", required=True)
    st.add_argument("--out-json", default=None)
    st.add_argument("--workload", default=None)
    st.add_argument("--T", type=int, default=None)
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        _copy(a)
    elif a.cmd == "stats":
        _stats(a)
    elif a.cmd == "steptraffic":
        _step_traffic(a)
    elif a.cmd == "counters":
        _counters(a)
    else:
        _summarize(a)


if __name__ == "__main__":
    main(sys.argv[1:])
