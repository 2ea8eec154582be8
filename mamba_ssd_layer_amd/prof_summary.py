"""Summaries of rocprofv3 output for the SSD kernels (text for profiles/).

    python -m mamba_ssd_layer_amd.prof_summary kernels <trace_dir> [--first N] [--last N]
    python -m mamba_ssd_layer_amd.prof_summary traffic --fetch D --write D \
        --cal-fetch D --cal-write D --kernel chunk_output --workload long_T16k [--command C ...]
    python -m mamba_ssd_layer_amd.prof_summary busy <sq_counter_dir> --symbol S [--symbol S ...]

`kernels` prints a markdown table of the per-kernel durations (run_kernel_stats.csv)
and the gaps between consecutive SSD kernels of one forward (run_kernel_trace.csv).
`traffic` prints the JSON that bench.py reads for the roofline's `traffic` figure:
FETCH_SIZE and WRITE_SIZE of one kernel per dispatch, each scaled by what the same
counter reads for a plain device copy of known size (bench.py --calibrate-copy),
stamped with a hash of the kernel's sources so that a stale figure is not used.
`busy` prints, for any kernels named, the matrix-core busy fraction, the share of
wave time spent waiting to issue and the LDS instructions, from one SQ pass.
`counters` prints the JSON that bench.py reads for the roofline's `mfma_util` and
`dram_bytes`: from one pass of matrix-core counters (SQ_VALU_MFMA_BUSY_CYCLES,
SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE) and one of the L2's memory-side
request counters (TCC_EA0_RDREQ_DRAM_sum, TCC_EA0_WRREQ_DRAM_sum), the latter
scaled to bytes by what they read for the plain device copy.  Those requests
leave the L2 for the memory fabric: the Infinity Cache behind it may still
serve them, so they bound the HBM traffic from above, as the cold timing of
bench.py (the last-level cache flushed before each step) bounds it from the
time side.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# sources each kernel is built from (the hash covers all of them)
KERNEL_SOURCES = {
    "chunk_output": ["k25_chunk_output.hip", "ssd_stage.hpp", "ssd_device.hpp", "ssd_internal.hpp"],
    "chunk_state": ["k3_chunk_state.hip", "ssd_stage.hpp", "ssd_device.hpp", "ssd_internal.hpp"],
    "state_pass": ["k4_state_pass.hip", "ssd_device.hpp", "ssd_internal.hpp"],
}
KERNEL_SYMBOL = {
    "chunk_output": "ssd::chunk_output_kernel",
    "chunk_state": "ssd::chunk_state_kernel",
    "state_pass": "ssd::state_pass_kernel",
    "chunk_cb": "ssd::chunk_cb_kernel",
    "seq_table": "ssd::seq_table_kernel",
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def sources_hash(kernel: str) -> str | None:
    h = hashlib.sha256()
    try:
        for name in KERNEL_SOURCES[kernel]:
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError):
        return None
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    return name.replace("void ", "").split("(")[0]


def kernels_table(trace_dir: str, first: int = 0, last: int = 0) -> str:
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    ssd = [r for r in rows if "ssd::" in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in ssd)
    out = ["| kernel | calls | avg us | min us | max us | share of SSD time |", "|---|---|---|---|---|---|"]
    for r in sorted(ssd, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{100.0 * float(r['TotalDurationNs']) / total:.1f}% |")
    # gaps between consecutive SSD dispatches (end of one to start of the next)
    tr = [r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv")))
          if "ssd::" in r["Kernel_Name"]]
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    if first:
        tr = tr[:first]
    gaps = [int(b["Start_Timestamp"]) - int(a["End_Timestamp"]) for a, b in zip(tr, tr[1:])]
    gaps = [g for g in gaps if 0 <= g < 20000]  # within one forward (not across host syncs)
    if gaps:
        out.append("")
        out.append(f"Gap between consecutive SSD kernels of a forward: median {statistics.median(gaps) / 1e3:.2f} us "
                   f"over {len(gaps)} gaps" + (f" (first {first} SSD dispatches)." if first else "."))
    if last:
        # the last `last` dispatches of each kernel: bench.py's event-timed pass
        alltr = [r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv")))
                 if "ssd::" in r["Kernel_Name"]]
        alltr.sort(key=lambda r: int(r["Start_Timestamp"]))
        by = {}
        for r in alltr:
            by.setdefault(_short(r["Kernel_Name"]), []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        out.append("")
        out.append(f"Average over the last {last} dispatches of each kernel (bench.py's event-timed pass):")
        out.append("")
        out.append("| kernel | dispatches | avg us |")
        out.append("|---|---|---|")
        for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1][-last:])):
            tail = d[-last:]
            out.append(f"| {name} | {len(tail)} | {sum(tail) / len(tail) / 1e3:.1f} |")
    return "\n".join(out)


def _counter_per_dispatch(d: str, symbol: str, counter: str, reduce: str = "sum") -> float:
    """Average over the kernel's dispatches of the counter, its instances summed
    (reduce "sum") or their largest taken (reduce "max")."""
    vals = {}
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        if symbol in r["Kernel_Name"] and r["Counter_Name"] == counter:
            v = float(r["Counter_Value"])
            k = r["Dispatch_Id"]
            if reduce == "max":
                vals[k] = max(vals.get(k, 0.0), v)
            else:
                vals[k] = vals.get(k, 0.0) + v
    if not vals:
        raise SystemExit(f"no {counter} rows for {symbol} in {d}")
    return sum(vals.values()) / len(vals)


SIMDS = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
XCDS = 8  # accelerator dies; GRBM_GUI_ACTIVE comes back as the sum of their busy clocks


def counters(mfma: str, dram: str, cal_dram: str, kernel: str, workload: str, copy_mib: int,
             commands: list[str]) -> dict:
    sym = KERNEL_SYMBOL[kernel]
    busy = _counter_per_dispatch(mfma, sym, "SQ_VALU_MFMA_BUSY_CYCLES")
    mops = _counter_per_dispatch(mfma, sym, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    # one die's busy clocks: rocprofv3 reports GRBM_GUI_ACTIVE summed over the
    # dies (about 8 x 2.4 GHz x the dispatch's begin..end time)
    active = _counter_per_dispatch(mfma, sym, "GRBM_GUI_ACTIVE", "max") / XCDS
    rd = _counter_per_dispatch(dram, sym, "TCC_EA0_RDREQ_DRAM_sum")
    wr = _counter_per_dispatch(dram, sym, "TCC_EA0_WRREQ_DRAM_sum")
    crd = _counter_per_dispatch(cal_dram, COPY_KERNEL, "TCC_EA0_RDREQ_DRAM_sum")
    cwr = _counter_per_dispatch(cal_dram, COPY_KERNEL, "TCC_EA0_WRREQ_DRAM_sum")
    moved = copy_mib * float(1 << 20)
    rs, ws = moved / crd, moved / cwr
    name = next(r["Kernel_Name"] for r in csv.DictReader(open(os.path.join(mfma, "run_counter_collection.csv")))
                if sym in r["Kernel_Name"])
    return {
        "kernel": _short(name),
        "workload": workload,
        "sources": KERNEL_SOURCES[kernel],
        "sources_sha256_16": sources_hash(kernel),
        "mfma_busy_cycles_per_launch": busy,
        "gpu_active_cycles_per_launch": active,
        "mfma_util": busy / (active * SIMDS),
        "mfma_flops_bf16_per_launch": mops * 512.0,
        "dram_read_requests_per_launch": rd,
        "dram_write_requests_per_launch": wr,
        "read_bytes_per_request": rs,
        "write_bytes_per_request": ws,
        "dram_bytes_per_launch": rd * rs + wr * ws,
        "note": ("mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 dies x 1024 SIMDs); "
                 "mfma_flops_bf16_per_launch = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, the products "
                 "the kernel executes; dram bytes = "
                 "TCC_EA0_{RD,WR}REQ_DRAM_sum scaled by a plain device copy's bytes per request "
                 "(requests that leave the L2; the Infinity Cache may still serve some)"),
        "scale_reference": (f"plain device copy of {copy_mib} MiB (bench.py --calibrate-copy {copy_mib}): "
                            f"{crd:.0f} read and {cwr:.0f} write requests per launch"),
        "commands": commands,
    }


def traffic(fetch: str, write: str, cal_fetch: str, cal_write: str, kernel: str, workload: str,
            copy_mib: int, commands: list[str]) -> dict:
    sym = KERNEL_SYMBOL[kernel]
    f_kib = _counter_per_dispatch(fetch, sym, "FETCH_SIZE")
    w_kib = _counter_per_dispatch(write, sym, "WRITE_SIZE")
    moved_kib = copy_mib * 1024.0
    cf = _counter_per_dispatch(cal_fetch, COPY_KERNEL, "FETCH_SIZE")
    cw = _counter_per_dispatch(cal_write, COPY_KERNEL, "WRITE_SIZE")
    fs, ws = moved_kib / cf, moved_kib / cw
    name = next(r["Kernel_Name"] for r in csv.DictReader(open(os.path.join(fetch, "run_counter_collection.csv")))
                if sym in r["Kernel_Name"])
    return {
        "kernel": _short(name),
        "workload": workload,
        "sources": KERNEL_SOURCES[kernel],
        "sources_sha256_16": sources_hash(kernel),
        "fetch_kib_per_launch": f_kib,
        "write_kib_per_launch": w_kib,
        "fetch_scale": fs,
        "write_scale": ws,
        "bytes_per_launch": (f_kib * fs + w_kib * ws) * 1024.0,
        "scale_reference": (f"plain device copy of {copy_mib} MiB (bench.py --calibrate-copy {copy_mib}): "
                            f"FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE {cw:.1f} KiB per launch"),
        "commands": commands,
    }


def busy_table(mfma: str, symbols: list[str]) -> str:
    """Per kernel (a substring of its name), from one SQ counter pass: matrix-core
    busy fraction (as in counters()), the fraction of wave time spent waiting
    to issue an instruction (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, both in wave
    cycles), and LDS instructions per launch."""
    out = ["| kernel | MFMA util | executed MFMA GFLOP | wave time waiting to issue | LDS instructions (M) |",
           "|---|---|---|---|---|"]
    for sym in symbols:
        busy = _counter_per_dispatch(mfma, sym, "SQ_VALU_MFMA_BUSY_CYCLES")
        mops = _counter_per_dispatch(mfma, sym, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        active = _counter_per_dispatch(mfma, sym, "GRBM_GUI_ACTIVE", "max") / XCDS
        wait = _counter_per_dispatch(mfma, sym, "SQ_WAIT_INST_ANY")
        wave = _counter_per_dispatch(mfma, sym, "SQ_WAVE_CYCLES")
        lds = _counter_per_dispatch(mfma, sym, "SQ_INSTS_LDS")
        name = next(r["Kernel_Name"] for r in csv.DictReader(open(os.path.join(mfma, "run_counter_collection.csv")))
                    if sym in r["Kernel_Name"])
        out.append(f"| {_short(name)} | {busy / (active * SIMDS):.3f} | {mops * 512.0 / 1e9:.2f} | "
                   f"{wait / wave:.2f} | {lds / 1e6:.2f} |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("trace_dir")
    k.add_argument("--first", type=int, default=0, help="gaps over the first N SSD dispatches only")
    k.add_argument("--last", type=int, default=0, help="also average the last N dispatches of each kernel")
    bz = sub.add_parser("busy")
    bz.add_argument("mfma_dir")
    bz.add_argument("--symbol", action="append", required=True, help="a substring of a kernel name (repeatable)")
    t = sub.add_parser("traffic")
    for a in ("fetch", "write", "cal_fetch", "cal_write"):
        t.add_argument("--" + a.replace("_", "-"), dest=a, required=True)
    t.add_argument("--kernel", default="chunk_output", choices=sorted(KERNEL_SOURCES))
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mib", type=int, default=256)
    t.add_argument("--command", action="append", default=[])
    c = sub.add_parser("counters")
    for a_ in ("mfma", "dram", "cal_dram"):
        c.add_argument("--" + a_.replace("_", "-"), dest=a_, required=True)
    c.add_argument("--kernel", default="chunk_output", choices=sorted(KERNEL_SOURCES))
    c.add_argument("--workload", required=True)
    c.add_argument("--copy-mib", type=int, default=256)
    c.add_argument("--command", action="append", default=[])
    a = ap.parse_args(argv)
    if a.cmd == "kernels":
        print(kernels_table(a.trace_dir, a.first, a.last))
    elif a.cmd == "busy":
        print(busy_table(a.mfma_dir, a.symbol))
    elif a.cmd == "counters":
        json.dump(counters(a.mfma, a.dram, a.cal_dram, a.kernel, a.workload, a.copy_mib, a.command),
                  sys.stdout, indent=1)
        print()
    else:
        json.dump(traffic(a.fetch, a.write, a.cal_fetch, a.cal_write, a.kernel, a.workload, a.copy_mib,
                          a.command), sys.stdout, indent=1)
        print()


if __name__ == "__main__":
    main()
