"""Short text summaries of rocprofv3 results (rocpd SQLite databases).

  python profile_summary.py trace DB --cmd "..." [--bench JSON] --out FILE
      Per (kernel, grid): dispatch count, mean / median / min / max duration.  With
      --bench, the bench line's per-call kernel times are listed beside the trace.

  python profile_summary.py counters DB... --cmd "..." [--cmd "..."] --out FILE
      Every counter of every library kernel in the databases (mean per dispatch).

  python profile_summary.py pmc FETCH_DB WRITE_DB --cmd-fetch "..."
      --cmd-write "..." --copy-bytes N --out FILE
      Per (kernel, grid): mean FETCH_SIZE and WRITE_SIZE (KiB per dispatch).  The two
      counters are scaled to bytes by a plain device copy of N bytes that the profiled
      program ran between its first two spin-kernel dispatches (bench.py
      --copy-calibration): factor = N / (counter KiB * 1024).  For each library kernel
      a "traffic:" line gives the scaled HBM bytes per dispatch with the SHA-256 of
      the sources that kernel is built from, so a reader can tell whether the
      counters still describe the current code.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sqlite3
import statistics

_HERE = os.path.dirname(os.path.abspath(__file__))
_CSRC = os.path.join(_HERE, "quantized_matmul_amd", "csrc")

# library kernel (name prefix) -> sources it is compiled from
KERNEL_SOURCES = {
    "qmm::mmvq_": ("qmm_mmvq.hip", "qmm_internal.h"),
    "qmm::mmq_": ("qmm_mmq.hip", "qmm_mmq_common.h", "qmm_internal.h"),
    "qmm::{anonymous}::mmq_q4k_v2_": ("qmm_mmq2.hip", "qmm_mmq_common.h", "qmm_internal.h"),
    "qmm::{anonymous}::mmq_k4_q8k_v2_": ("qmm_mmq_q8k2.hip", "qmm_mmq_common.h", "qmm_internal.h"),
    "qmm::mmq_k4_q8k_": ("qmm_mmq_q8k.hip", "qmm_mmq_common.h", "qmm_internal.h"),
    "qmm::mmq_q6k_q8k_": ("qmm_mmq_q8k.hip", "qmm_mmq_common.h", "qmm_internal.h"),
    "qmm::{anonymous}::mmq_skinny_": ("qmm_skinny.hip", "qmm_mmq_common.h", "qmm_internal.h"),
    "qmm::quantize_": ("qmm_quantize.hip", "qmm_internal.h"),
    "qmm::{anonymous}::rmsnorm_": ("qmm_fused.hip", "qmm_internal.h"),
    "qmm::{anonymous}::silu_mul_": ("qmm_fused.hip", "qmm_internal.h"),
    "qmm::{anonymous}::residual_add_": ("qmm_fused.hip", "qmm_internal.h"),
}


def sources_sha256(kernel_name: str):
    """SHA-256 over the source files of a library kernel, or None for other kernels."""
    short = kernel_name.replace("void ", "")
    match = [p for p in KERNEL_SOURCES if short.startswith(p)]
    if not match:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[max(match, key=len)]:  # the most specific prefix
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    """Kernel name without the argument list: 'qmm::mmvq_q4k_kernel<1, 4, false>'."""
    name = name.replace("void ", "", 1).replace("(anonymous namespace)", "{anonymous}")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def trace_rows(db: str):
    con = sqlite3.connect(db)
    rows = list(con.execute("select name, grid_x * grid_y * grid_z, duration, start from kernels order by start"))
    con.close()
    groups = {}
    for name, grid, dur, _ in rows:
        groups.setdefault((short_name(name), grid), []).append(dur)
    out = []
    total = sum(sum(v) for v in groups.values())
    for (name, grid), d in groups.items():
        out.append({"kernel": name, "grid": grid, "calls": len(d), "mean_us": statistics.fmean(d) / 1e3,
                    "median_us": statistics.median(d) / 1e3, "min_us": min(d) / 1e3, "max_us": max(d) / 1e3,
                    "total_ms": sum(d) / 1e6, "share": sum(d) / total if total else 0.0})
    out.sort(key=lambda r: -r["total_ms"])
    return out


def cmd_trace(a):
    rows = trace_rows(a.db)
    lines = [f"# rocprofv3 kernel trace: {a.title}", "", "Command (from the repository root):", "",
             "```", a.cmd, "```", "",
             "Durations are rocprofv3 kernel-trace timestamps (end - start) per dispatch.", "",
             "| kernel | grid (threads) | calls | mean us | median us | min us | max us | total ms | share |",
             "|---|---|---|---|---|---|---|---|---|"]
    if a.kernel_filter:
        rows = [r for r in rows if a.kernel_filter in r["kernel"]]
        lines.insert(9, f"Kernels whose name contains `{a.kernel_filter}` only.")
        lines.insert(10, "")
    for r in rows:
        lines.append(f"| `{r['kernel']}` | {r['grid']} | {r['calls']} | {r['mean_us']:.2f} | {r['median_us']:.2f} "
                     f"| {r['min_us']:.2f} | {r['max_us']:.2f} | {r['total_ms']:.3f} | {100 * r['share']:.1f} % |")
    if a.bench:
        with open(a.bench) as fh:
            line = json.loads([ln for ln in fh if ln.startswith("{")][-1])
        if isinstance(line.get("detail"), dict):   # the measured-limits workload
            lines += peaks_lines(line["detail"])
            with open(a.out, "w") as fh:
                fh.write("\n".join(lines) + "\n")
            print("\n".join(lines))
            return
        lines += ["", "Bench line of the same command run without the profiler (HIP events over back-to-back "
                  "launches, per launch; under kernel tracing the launches no longer run back to back):", "",
                  "| call | kernel | event us |", "|---|---|---|"]
        for d in line.get("detail", []):
            if "fused_us" in d:  # producer-fused workload: the fused kernel and its unfused chain
                lines.append(f"| {d['call']} | fused | {d['fused_us']} |")
                lines.append(f"| {d['call']} | unfused chain (all launches) | {d['chain_us']} |")
            else:
                lines.append(f"| {d['call']} | {d['kernel']} | {d['kernel_us']} |")
        rf = line.get("roofline")
        if rf:
            lines += ["", f"Roofline kernel `{rf.get('kernel')}` ({rf.get('call')}): achieved {rf['achieved']} "
                      f"{rf['unit']} of {rf['peak']} ({100 * rf['frac']:.1f} %)."]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def peaks_lines(det):
    """The measured limits of bench.py --workload peaks (run without the profiler)."""
    out = ["", "Figures of the same command run without the profiler (HIP events; clocks from the shader and "
           "100 MHz reference counters the probes read):", "",
           "| streaming read | bytes | us | GB/s | % of 8 TB/s |", "|---|---|---|---|---|"]
    for r in det["stream_read"]:
        out.append(f"| {r['loads_per_lane']} x 16 B per lane | {r['bytes_read']} | {r['us']} | {r['GB_s']} "
                   f"| {100 * r['GB_s'] / 8000:.1f} % |")
    out += ["", "| MFMA issue rate | waves per SIMD | TOP/s (int8) or TFLOP/s (f32) | clock GHz | clocks per "
            "instruction |", "|---|---|---|---|---|"]
    for r in det["mfma"]["int8"]:
        out.append(f"| v_mfma_i32_32x32x32_i8 | {r['waves_per_simd']} | {r['T_s']} | {r['clock_GHz']} "
                   f"| {r['clocks_per_instr']} |")
    for r in det["mfma"]["f32_outer"]:
        out.append(f"| v_mfma_f32_32x32x1_2b_f32 | {r['waves_per_simd']} | {r['T_s']} | | |")
    out += ["", "| VALU instruction | clocks per wave instruction, 1 / 2 / 4 waves per SIMD |", "|---|---|"]
    for r in det["valu_instr"]:
        out.append(f"| {r['instr']} | {r['clocks_w1']} / {r['clocks_w2']} / {r['clocks_w4']} |")
    out += ["", f"LDS read: {det['lds_read']['bytes_per_cu_per_clock']} bytes per CU per clock.", "",
            "| MFMA and VALU together | VALU per MFMA | MFMA alone ms | VALU alone ms | both ms | overlap |",
            "|---|---|---|---|---|---|"]
    for r in det["overlap"]:
        out.append(f"| {r['mode']} | {r['valu_per_mfma']} | {r['mfma_ms']} | {r['valu_ms']} | {r['both_ms']} "
                   f"| {r['overlap']} |")
    out += ["", "| per-32 step (MFMAs then their epilogue, 2 waves per SIMD) | clocks per 32x32x32 block "
            "| share of int8 MFMA peak |", "|---|---|---|"]
    for r in det["burst"]:
        out.append(f"| {r['subblocks_per_burst']} sub-blocks x {r['token_blocks']} token blocks per burst "
                   f"| {r['clocks_per_block']} | {r['int8_frac_of_mfma']} |")
    pp = det["pingpong"]
    out += ["", f"Ping-pong of MFMA and epilogue phases between the two waves of a SIMD (s_barrier between "
            f"phases): {pp['pingpong']} clocks against {pp['serial']} for the same work without barriers."]
    if det.get("load_shape"):
        out += ["", "| loads only, Q4_K 12288 x 4096 (no arithmetic) | bytes | us | GB/s |", "|---|---|---|---|"]
        for r in det["load_shape"]:
            out.append(f"| {r['shape']} | {r['bytes']} | {r['us']} | {r['GB_s']} |")
    return out


def pmc_rows(db: str, counter: str):
    """[(dispatch_id, short kernel name, grid, value)] in dispatch order."""
    con = sqlite3.connect(db)
    rows = list(con.execute(
        "select dispatch_id, kernel_name, grid_size, sum(value) from counters_collection where counter_name = ? "
        "group by dispatch_id order by dispatch_id", (counter,)))
    con.close()
    return [(d, short_name(n), g, v) for d, n, g, v in rows]


def calibration(rows, copy_bytes: int):
    """Scale factor bytes / (KiB * 1024) from the copies between the first two spin kernels."""
    spins = [i for i, r in enumerate(rows) if "spin_kernel" in r[1]]
    if len(spins) < 2:
        raise SystemExit("no calibration bracket (two spin-kernel dispatches) in the profile")
    cal = [r for r in rows[spins[0] + 1: spins[1]] if "copyBuffer" in r[1]]
    if not cal:
        raise SystemExit("no copy dispatch inside the calibration bracket")
    kib = statistics.fmean(r[3] for r in cal)
    return copy_bytes / (kib * 1024.0), kib, len(cal)


def cmd_pmc(a):
    fetch = pmc_rows(a.fetch_db, "FETCH_SIZE")
    write = pmc_rows(a.write_db, "WRITE_SIZE")
    ff, fkib, fn = calibration(fetch, a.copy_bytes)
    fw, wkib, wn = calibration(write, a.copy_bytes)

    def by_kernel(rows):
        g = {}
        for _, name, grid, v in rows:
            if "spin_kernel" in name or "copyBuffer" in name:
                continue
            g.setdefault((name, grid), []).append(v)
        return {k: statistics.fmean(v) for k, v in g.items()}

    fk, wk = by_kernel(fetch), by_kernel(write)
    lines = [f"# rocprofv3 HBM counters: {a.title}", "", "Commands (from the repository root):", "",
             "```", a.cmd_fetch, a.cmd_write, "```", "",
             f"Calibration: a plain device copy of {a.copy_bytes} bytes (reads and writes that many bytes) "
             f"read FETCH_SIZE = {fkib:.1f} KiB ({fn} dispatches) and WRITE_SIZE = {wkib:.1f} KiB ({wn} "
             f"dispatches), so bytes = FETCH_SIZE x 1024 x {ff:.4f} and WRITE_SIZE x 1024 x {fw:.4f}.", "",
             "| kernel | grid (threads) | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |",
             "|---|---|---|---|---|---|"]
    traffic = []
    for key in sorted(set(fk) | set(wk), key=lambda k: -(fk.get(k, 0) + wk.get(k, 0))):
        f, w = fk.get(key, 0.0), wk.get(key, 0.0)
        rb, wb = f * 1024 * ff, w * 1024 * fw
        lines.append(f"| `{key[0]}` | {key[1]} | {f:.1f} | {w:.1f} | {rb / 1e6:.3f} | {wb / 1e6:.3f} |")
        sha = sources_sha256(key[0])
        if sha:
            traffic.append(f"traffic: kernel={key[0].replace(' ', '')} grid={key[1]} "
                           f"bytes_per_launch={int(round(rb + wb))} sources_sha256={sha}")
    lines += ["", "Scaled HBM bytes per dispatch, with the SHA-256 of the kernel's source files at the time "
              "of the run:", "", "```"] + traffic + ["```"]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counter_means(db: str):
    """{(short kernel, grid): {counter: mean per dispatch}} over all dispatches of a
    rocpd database (a counter's instances summed within each dispatch)."""
    con = sqlite3.connect(db)
    rows = list(con.execute(
        "select dispatch_id, kernel_name, grid_size, counter_name, sum(value) from counters_collection "
        "group by dispatch_id, counter_name"))
    con.close()
    acc = {}
    for _, name, grid, counter, v in rows:
        acc.setdefault((short_name(name), grid), {}).setdefault(counter, []).append(v)
    return {k: {c: statistics.fmean(v) for c, v in cs.items()} for k, cs in acc.items()}


def cmd_counters(a):
    merged = {}
    for db in a.dbs:
        for k, cs in counter_means(db).items():
            merged.setdefault(k, {}).update(cs)
    keys = [k for k in merged if any(k[0].startswith(p) for p in KERNEL_SOURCES)]
    keys.sort(key=lambda k: (k[0], -k[1]))
    counters = sorted({c for k in keys for c in merged[k]})
    lines = [f"# rocprofv3 counters: {a.title}", "", "Commands (from the repository root):", "", "```"] + a.cmd + \
            ["```", "", "Mean per dispatch (each counter's instances summed over the chip).", "",
             "| kernel | grid (threads) | " + " | ".join(counters) + " |",
             "|---|---|" + "---|" * len(counters)]
    for k in keys:
        lines.append(f"| `{k[0]}` | {k[1]} | " + " | ".join(f"{merged[k].get(c, float('nan')):.4g}" for c in counters)
                     + " |")
    if a.notes:
        lines += ["", a.notes]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


_TRAFFIC = re.compile(r"traffic: kernel=(\S+) grid=(\d+) bytes_per_launch=(\d+) sources_sha256=([0-9a-f]+)")


def read_traffic(path: str, kernel: str, grid):
    """HBM bytes per launch of `kernel` at `grid` threads (None: the kernel's only
    grid) from a pmc summary, or None when the summary is missing, lacks the kernel,
    or was taken from different sources."""
    if not os.path.exists(path):
        return None
    want = kernel.replace(" ", "")
    with open(path) as fh:
        hits = [m for m in _TRAFFIC.finditer(fh.read())
                if m.group(1) == want and (grid is None or int(m.group(2)) == grid)]
    if len(hits) != 1:
        return None   # absent, or ambiguous without a grid
    m = hits[0]
    return int(m.group(3)) if sources_sha256(kernel) == m.group(4) else None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", default="")
    t.add_argument("--bench")
    t.add_argument("--kernel-filter", default="", help="list only kernels whose name contains this")
    t.add_argument("--out", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("fetch_db")
    p.add_argument("write_db")
    p.add_argument("--cmd-fetch", required=True)
    p.add_argument("--cmd-write", required=True)
    p.add_argument("--copy-bytes", type=int, required=True)
    p.add_argument("--title", default="")
    p.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dbs", nargs="+")
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--notes", default="")
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    {"trace": cmd_trace, "pmc": cmd_pmc, "counters": cmd_counters}[a.what](a)


if __name__ == "__main__":
    main()
