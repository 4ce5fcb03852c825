"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m sequence_chunked_exact_amd.profile_summary copy
        Calibration workload: a plain 1 GiB device-to-device copy, three times
        (run it under rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE).

    python -m sequence_chunked_exact_amd.profile_summary summarize \\
        --stats S.csv --fetch F.csv --write W.csv --cal-fetch CF.csv \\
        --cal-write CW.csv --kernel dkdv --workload 8b_layer --out profiles/X.md \\
        --commands "..."
        [--mfma M.csv]
        Writes a markdown summary: per-kernel average durations from the
        kernel-trace statistics, and for one kernel the FETCH_SIZE/WRITE_SIZE
        per dispatch scaled by what the same counters read for the copy of
        known size, plus the SHA-256 of the kernel source it was measured on.
        With --mfma (a run collecting SQ_VALU_MFMA_BUSY_CYCLES and
        GRBM_GUI_ACTIVE) it adds each kernel's matrix-core busy fraction:
        SQ_VALU_MFMA_BUSY_CYCLES sums over the 1024 SIMDs and
        GRBM_GUI_ACTIVE over the 8 XCDs, so busy / (GRBM / 8) / 1024 is the
        mean fraction of elapsed cycles in which a SIMD's matrix core was busy.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
COPY_BYTES = 1 << 30
N_XCD, N_SIMD = 8, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs

SHORT = {"fwd_kernel": "fwd", "bwd_kernel": "bwd", "dkdv_kernel": "dkdv", "dqs_kernel": "dq",
         "delta_kernel": "delta", "zero_kernel": "zero", "accumulate_kernel": "accumulate", "gemm_kernel": "proj",
         "residual_fwd_kernel": "residual_fwd", "residual_bwd_kernel": "residual_bwd", "wt_kernel": "proj_prep",
         "gcat_kernel": "proj_prep"}


def kernel_sources(kernel: str) -> list:
    """The source files a kernel is built from (the shared device header and its own file)."""
    own = {"proj": ["gemm_bf16.h", "projection.hip"], "head": ["gemm_bf16.h", "lm_head.hip"],
           "head_ce": ["lm_head.hip"]}.get(kernel, ["attention.hip"])
    return [os.path.join(CSRC, f) for f in ["device_common.h"] + own]


def kernel_source_sha256(kernel: str) -> str:
    h = hashlib.sha256()
    for path in kernel_sources(kernel):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(full: str) -> str:
    for key, val in sorted(SHORT.items(), key=lambda kv: -len(kv[0])):  # most specific first
        if key in full:
            return val
    return full[:40]


def per_dispatch(path: str, counter: str, name_filter=None):
    vals = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        if name_filter and short_name(r["Kernel_Name"]) != name_filter:
            continue
        vals.append(float(r["Counter_Value"]))
    return vals


def copy_main():
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x3")


def summarize_main(args):
    rows = list(csv.DictReader(open(args.stats)))
    lines = [f"# rocprofv3 summary: `{args.kernel}` kernel, `{args.workload}` workload", ""]
    lines += ["Commands (run from the repository root):", "", "```"]
    lines += [c.strip() for c in args.commands.split(";;") if c.strip()]
    lines += ["```", "", "## Kernel trace statistics", "",
              "| kernel | calls | average (us) | total (ms) | share |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f}% |")
    # a kernel built in several variants (tile shapes) has one row per variant
    mine = [r for r in rows if short_name(r["Name"]) == args.kernel]
    if mine:
        calls = sum(int(r["Calls"]) for r in mine)
        total_ns = sum(float(r["TotalDurationNs"]) for r in mine)
        lines += ["", f"`{args.kernel}` over all its variants: {calls} dispatches, mean "
                      f"{total_ns / calls / 1e3:.1f} us"]
    out = {}
    if args.fetch and args.write and args.cal_fetch and args.cal_write:
        match = args.match or args.kernel
        f = per_dispatch(args.fetch, "FETCH_SIZE", match)
        w = per_dispatch(args.write, "WRITE_SIZE", match)
        cf = max(per_dispatch(args.cal_fetch, "FETCH_SIZE"))
        cw = max(per_dispatch(args.cal_write, "WRITE_SIZE"))
        kf, kw = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
        fetch_b = statistics.mean(f) * 1024 * kf
        write_b = statistics.mean(w) * 1024 * kw
        out = {"fetch": fetch_b, "write": write_b}
        lines += ["", f"## HBM traffic of `{args.kernel}` (per dispatch, mean over {len(f)} dispatches)", "",
                  f"- copy calibration: a {COPY_BYTES} B copy reads FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE "
                  f"{cw:.0f} KiB per dispatch; scale factors {kf:.4f} (fetch) and {kw:.4f} (write)",
                  f"- FETCH_SIZE {statistics.mean(f):.0f} KiB -> {fetch_b / 1e6:.1f} MB",
                  f"- WRITE_SIZE {statistics.mean(w):.0f} KiB -> {write_b / 1e6:.1f} MB",
                  "", f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}"]
    if args.mfma:
        busy, active = {}, {}
        for r in csv.DictReader(open(args.mfma)):
            k = short_name(r["Kernel_Name"])
            tgt = busy if r["Counter_Name"] == "SQ_VALU_MFMA_BUSY_CYCLES" else \
                active if r["Counter_Name"] == "GRBM_GUI_ACTIVE" else None
            if tgt is not None:
                tgt[k] = tgt.get(k, 0.0) + float(r["Counter_Value"])
        lines += ["", "## Matrix-core busy fraction per kernel", "",
                  "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8) / 1024, summed over the run's dispatches", "",
                  "| kernel | MFMA busy |", "|---|---|"]
        for k in sorted(busy):
            if active.get(k):
                lines.append(f"| {k} | {100.0 * busy[k] / (active[k] / N_XCD) / N_SIMD:.1f}% |")
    lines += ["", f"kernel_source_sha256: {kernel_source_sha256(args.kernel)}", ""]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))
    return out


STALL_A = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
           "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "GRBM_GUI_ACTIVE")
STALL_B = ("SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_MISC", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
           "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE")


def stalls_main(args):
    """Per-kernel stall fractions from two counter passes (STALL_A, STALL_B):
    wait and issue counters over SQ_WAVE_CYCLES, matrix-core busy over the
    elapsed cycles of all SIMDs, co-issue over matrix-core busy."""
    sums = {}
    for tag, path in (("a", args.a), ("b", args.b)):
        for r in csv.DictReader(open(path)):
            k = short_name(r["Kernel_Name"])
            d = sums.setdefault(k, {})
            key = (tag, r["Counter_Name"])
            d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    lines = [f"# rocprofv3 summary: stall counters, `{args.workload}` workload", "",
             "Commands (run from the repository root):", "", "```"]
    lines += [c.strip() for c in args.commands.split(";;") if c.strip()]
    lines += ["```", "",
              "Fractions of wave cycles (SQ_WAVE_CYCLES) for the wait and issue counters; matrix cores busy as",
              "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8) / 1024; co-issue as",
              "SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES.", "",
              "| kernel | wait on dependency | wait on LDS | other waits | VALU issuing | LDS issuing | "
              "matrix cores busy | co-issue with busy matrix cores |",
              "|---|---|---|---|---|---|---|---|"]
    for k in sorted(sums):
        d = sums[k]
        wc = d.get(("a", "SQ_WAVE_CYCLES"), 0.0)
        busy = d.get(("b", "SQ_VALU_MFMA_BUSY_CYCLES"), 0.0)
        grbm = d.get(("b", "GRBM_GUI_ACTIVE"), 0.0)
        if wc <= 0 or grbm <= 0:
            continue

        def f(x):
            return f"{100.0 * x:.1f}%"
        lines.append(f"| {k} | {f(d.get(('a', 'SQ_WAIT_INST_ANY'), 0.0) / wc)} | "
                     f"{f(d.get(('a', 'SQ_WAIT_INST_LDS'), 0.0) / wc)} | {f(d.get(('a', 'SQ_WAIT_ANY'), 0.0) / wc)} | "
                     f"{f(d.get(('a', 'SQ_ACTIVE_INST_VALU'), 0.0) / wc)} | "
                     f"{f(d.get(('a', 'SQ_ACTIVE_INST_LDS'), 0.0) / wc)} | {f(busy / (grbm / N_XCD) / N_SIMD)} | "
                     f"{f(d.get(('b', 'SQ_VALU_MFMA_COEXEC_CYCLES'), 0.0) / busy) if busy else '-'} |")
    lines.append("")
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def read_traffic(path: str, kernel: str):
    """traffic_bytes_per_launch from a summary, or None if missing or stale (the
    kernel's sources have changed since the counters were taken)."""
    if not os.path.exists(path):
        return None
    vals = {}
    for ln in open(path):
        if ":" in ln and ln.split(":")[0].strip() in ("traffic_bytes_per_launch", "kernel_source_sha256"):
            k, v = ln.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_sha256(kernel) or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("copy")
    st = sub.add_parser("stalls")
    for opt in ("--a", "--b", "--workload", "--out", "--commands"):
        st.add_argument(opt, default=None)
    s = sub.add_parser("summarize")
    for opt in ("--stats", "--fetch", "--write", "--cal-fetch", "--cal-write", "--kernel", "--workload",
                "--out", "--commands", "--mfma", "--match"):
        s.add_argument(opt, default=None)
    args = ap.parse_args(argv)
    if args.cmd == "copy":
        copy_main()
    elif args.cmd == "stalls":
        stalls_main(args)
    else:
        summarize_main(args)


if __name__ == "__main__":
    sys.exit(main())
