"""Turn rocprofv3 output of bench.py runs into the short text summaries kept
under profiles/ (kernel-trace statistics and HBM traffic per decode launch).

Usage (after the rocprofv3 runs named in each summary's header):

    python -m decode_attention_prefix_amd.prof_summary --config 1 \
        --kt <dir with kt_kernel_stats.csv> --fetch <dir> --write <dir> [--out profiles]

Traffic: FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the decode kernel,
each scaled by what the same counter reads for bench.py's copy kernel over a
buffer of known size (--copy-probe-mb in the counter runs): the copy kernel
reads and writes exactly that many bytes, so scale = bytes / counter reading.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SRC = os.path.join(ROOT, "decode_attention_prefix_amd", "csrc", "cap_kernels.hip")


ROWS_SRC = os.path.join(ROOT, "decode_attention_prefix_amd", "csrc", "cap_rows.hip")


def kernel_hash(src: str = KERNEL_SRC) -> str:
    """Hash of a kernel source file's code (by default the attention kernels,
    decode and merge; the growth and measurement kernels live in another
    file): comments and whitespace removed, so an edit of the comments alone
    keeps counters taken on the same code."""
    with open(src) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    code = "".join(src.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def _short(name: str) -> str:
    for key in ("decode_kernel", "merge_kernel", "rows_retained_kernel", "rows_pipelined_kernel",
                "rows_reread_kernel", "read_stream_kernel", "read_kernel", "fill_kernel", "copy_stream_kernel",
                "copy_kernel", "patch_kernel", "append_kernel"):
        if key in name:
            tail = name[name.index(key):]
            return tail.split("(")[0]
    return name.split("(")[0][:60]


def kernel_stats(kt_dir: str) -> list[tuple[str, int, float, float, float]]:
    rows = []
    with open(os.path.join(kt_dir, "kt_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    return rows


def counter_means(pmc_dir: str, counter: str) -> dict[str, float]:
    vals: dict[str, list[float]] = defaultdict(list)
    with open(os.path.join(pmc_dir, "pmc_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: statistics.fmean(v) for k, v in vals.items()}


# Derived metrics as rocprofv3 defines them for this GPU (its counter list
# on the box): 256 CUs, 4 SIMDs each.  GRBM_GUI_ACTIVE arrives summed over the
# 8 XCDs (each has its own GRBM), while the formulas take its maximum over
# them; a decode launch keeps every XCD busy for the whole dispatch, so the
# per-XCD value is the sum / 8 (check: MFMA busy cycles / this value / 1024
# SIMDs matches the MFMA instruction count x 16 cycles over the kernel's
# duration).
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8


def counter_summary(pmc_dirs: list[str], target: str) -> tuple[dict, int]:
    """Mean per dispatch of every counter collected for the target kernel
    over several --pmc runs, and the number of dispatches averaged."""
    vals: dict[str, list[float]] = defaultdict(list)
    for d in pmc_dirs:
        with open(os.path.join(d, "pmc_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if _short(r["Kernel_Name"]).startswith(target):
                    vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    n = min((len(v) for v in vals.values()), default=0)
    return {k: statistics.fmean(v) for k, v in vals.items()}, n


def derived(c: dict) -> list[tuple[str, float]]:
    """The percentages rocprofv3 derives from these counters (same formulas),
    each normalised by GRBM_GUI_ACTIVE of the run that collected it."""
    out = []
    g = c.get("GRBM_GUI_ACTIVE")
    if not g:
        return out
    g /= XCD_NUM
    out.append(("GRBM_GUI_ACTIVE_per_XCD", g))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out.append(("MfmaUtil_pct", 100 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * SIMD_NUM)))
    if "SQ_ACTIVE_INST_VALU" in c:
        out.append(("VALUBusy_pct", 100 * c["SQ_ACTIVE_INST_VALU"] / CU_NUM / g))
    if "SQ_LDS_IDX_ACTIVE" in c:
        out.append(("LdsUtil_pct", 100 * c["SQ_LDS_IDX_ACTIVE"] / (g * CU_NUM)))
    if "SQ_LDS_BANK_CONFLICT" in c:
        out.append(("LDSBankConflict_pct", 100 * c["SQ_LDS_BANK_CONFLICT"] / g / CU_NUM))
    if "SQ_INST_CYCLES_SALU" in c:
        out.append(("SALUBusy_pct", 100 * c["SQ_INST_CYCLES_SALU"] / CU_NUM / g))
    if "SQ_BUSY_CYCLES" in c:
        out.append(("SQ_BUSY_CYCLES_over_GRBM_GUI_ACTIVE", c["SQ_BUSY_CYCLES"] / g))
    if "SQ_WAIT_INST_ANY" in c and "SQ_WAVE_CYCLES" in c:
        out.append(("wave_cycles_waiting_for_any_instruction_pct", 100 * c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]))
    return out


def write_counters(a, h: str, bench: str) -> None:
    c, n = counter_summary(a.pmc, a.target)
    groups = [g.replace(",", " ") for g in a.pmc_groups] if a.pmc_groups else ["?"] * len(a.pmc)
    lines = [f"rocprofv3 counters of {a.kernel}, bench.py {bench} ({a.workload})",
             "commands (one run per counter group, each with GRBM_GUI_ACTIVE):"]
    lines += [f"  cd /tmp && rocprofv3 --pmc {g} --output-format csv -d <out> -o pmc -- python3 <repo>/bench.py "
              f"{bench} --steps 3 --warmup 1" for g in groups]
    lines += [f"kernel_code_sha256_16: {h}", f"kernel: {a.kernel}", f"dispatches_averaged: {n}", "",
              "mean per dispatch (values summed over the GPU):"]
    lines += [f"  {k}: {v:.1f}" for k, v in sorted(c.items())]
    lines += ["", "derived (rocprofv3's formulas; CU_NUM 256, SIMD_NUM 1024):"]
    lines += [f"  {k}: {v:.2f}" for k, v in derived(c)]
    if a.per_unit and a.per_unit_name:
        lines += ["", f"per {a.per_unit_name} ({a.per_unit:g} of them per dispatch):"]
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM",
                  "SQ_INSTS_VALU_MFMA_MOPS_BF16"):
            if k in c:
                lines.append(f"  {k}: {c[k] / a.per_unit:.1f}")
    name = a.counters_name or f"decode_kernel_cfg{a.config}_counters.txt"
    with open(os.path.join(a.out, name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=None, help="bench.py --config (omit for --rows runs)")
    ap.add_argument("--workload", default="", help="one-line workload description")
    ap.add_argument("--kt", default=None)
    ap.add_argument("--fetch", default=None, help="omit to write the kernel-trace summary only")
    ap.add_argument("--write", default=None)
    ap.add_argument("--copy-mb", type=int, default=512)
    ap.add_argument("--alg-bytes", type=float, default=0.0,
                    help="algorithmic bytes per decode launch (unique K+V + Q [+ out])")
    ap.add_argument("--kernel", default="decode_kernel<128, false>")
    ap.add_argument("--bench-args", default="--no-cpu-baseline")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--name", default="", help="summary file name (default decode_kernel_cfg<N>_kernel_trace.txt)")
    ap.add_argument("--traffic-name", default="", help="traffic file name (default decode_kernel_cfg<N>_traffic.txt)")
    ap.add_argument("--target", default="decode_kernel", help="kernel name prefix the traffic is taken for")
    ap.add_argument("--src", choices=["attention", "rows"], default="attention",
                    help="kernel source the code hash covers")
    ap.add_argument("--pmc", nargs="*", default=[], help="rocprofv3 --pmc output dirs: write a counter summary")
    ap.add_argument("--pmc-groups", nargs="*", default=[], help="the counters of each --pmc run, comma-separated")
    ap.add_argument("--counters-name", default="", help="counter summary file name")
    ap.add_argument("--per-unit", type=float, default=0.0, help="divide instruction counts by this many units")
    ap.add_argument("--per-unit-name", default="", help="what the unit is (e.g. 'wave-step of the shared path')")
    a = ap.parse_args(argv)
    if a.pmc:
        h = kernel_hash(ROWS_SRC if a.src == "rows" else KERNEL_SRC)
        bench = (f"--config {a.config} " if a.config is not None else "") + a.bench_args
        write_counters(a, h, bench)
        return
    if a.fetch and a.write and a.alg_bytes <= 0:
        ap.error("--alg-bytes is needed with --fetch/--write")
    h = kernel_hash(ROWS_SRC if a.src == "rows" else KERNEL_SRC)
    cfg = a.config
    bench = (f"--config {cfg} " if cfg is not None else "") + a.bench_args

    kt = kernel_stats(a.kt)
    lines = [f"rocprofv3 kernel-trace summary: bench.py {bench} ({a.workload})",
             f"command: cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o kt -- "
             f"python3 <repo>/bench.py {bench}",
             f"kernel_code_sha256_16: {h}", "",
             f"{'kernel':40s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for name, calls, avg, mn, mx in kt:
        lines.append(f"{name:40s} {calls:6d} {avg:9.3f} {mn:9.3f} {mx:9.3f}")
    lines += ["", "(read_kernel and fill_kernel: the bench's cache-eviction read and buffer setup; "
              "read_stream_kernel: its plain-read probes (2 GiB, and the decode launch's own bytes); append_kernel and patch_kernel: "
              "cap_append_kv and cap_plan_refresh in its growth steps; rows_reread_kernel, copy_kernel, "
              "copy_stream_kernel and at::native kernels: the two-pass, copy and torch references of a --rows run)"]
    name = a.name or f"decode_kernel_cfg{cfg}_kernel_trace.txt"
    with open(os.path.join(a.out, name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    if not (a.fetch and a.write):
        return

    fetch = counter_means(a.fetch, "FETCH_SIZE")
    write = counter_means(a.write, "WRITE_SIZE")
    copy_kib = a.copy_mb * 1024.0
    fs = copy_kib / fetch["copy_kernel"]
    ws = copy_kib / write["copy_kernel"]
    dk = [k for k in fetch if k.startswith(a.target)][0]
    fb = fetch[dk] * fs * 1024.0
    wb = write[dk] * ws * 1024.0
    mk = [k for k in fetch if k.startswith("merge_kernel")]
    probe = f" --copy-probe-mb {a.copy_mb}" if a.target == "decode_kernel" else ""
    lines = [f"HBM traffic of one {a.kernel} launch, bench.py {bench} ({a.workload})",
             "commands (each its own run):",
             f"  cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out> -o pmc -- python3 "
             f"<repo>/bench.py {bench} --steps 3 --warmup 1{probe}",
             f"  cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out> -o pmc -- python3 "
             f"<repo>/bench.py {bench} --steps 3 --warmup 1{probe}",
             f"kernel_code_sha256_16: {h}",
             f"kernel: {a.kernel}",
             f"copy_kernel_{a.copy_mb}MiB_fetch_kib: {fetch['copy_kernel']:.1f}",
             f"copy_kernel_{a.copy_mb}MiB_write_kib: {write['copy_kernel']:.1f}",
             f"fetch_scale: {fs:.5f}",
             f"write_scale: {ws:.5f}",
             f"decode_fetch_kib_per_dispatch: {fetch[dk]:.1f}",
             f"decode_write_kib_per_dispatch: {write[dk]:.1f}"]
    if a.target != "decode_kernel":
        lines = [l.replace("decode_", "kernel_") for l in lines]
    if mk:
        lines += [f"merge_fetch_kib_per_dispatch: {fetch[mk[0]]:.1f}",
                  f"merge_write_kib_per_dispatch: {write[mk[0]]:.1f}"]
    pre = "decode" if a.target == "decode_kernel" else "kernel"
    lines += [f"{pre}_fetch_bytes: {fb:.0f}",
              f"{pre}_write_bytes: {wb:.0f}",
              f"hbm_bytes_per_launch: {fb + wb:.0f}",
              f"algorithmic_bytes_per_launch: {a.alg_bytes:.0f}",
              f"fetch_over_algorithmic: {fb / a.alg_bytes:.4f}",
              f"hbm_over_algorithmic: {(fb + wb) / a.alg_bytes:.4f}"]
    tname = a.traffic_name or f"decode_kernel_cfg{cfg}_traffic.txt"
    with open(os.path.join(a.out, tname), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
