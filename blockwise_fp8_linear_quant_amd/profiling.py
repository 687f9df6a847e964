"""Summaries of rocprofv3 output for the committed profile notes.

Two kinds of summary are written as short text files:

* ``stats``: the per-kernel table of a ``rocprofv3 --kernel-trace --stats
  --output-format csv`` run (calls, average and total duration, share).
* ``traffic``: HBM bytes per dispatch of the block GEMM from two
  ``rocprofv3 --pmc`` runs (``FETCH_SIZE``, then ``WRITE_SIZE``) of the same
  command.  Both counters are scaled by what they read for a plain device copy
  of known size launched in the same process (``bench.py --copy-probe-mib``),
  so the figure is in bytes rather than in the counters' own units.

The traffic summary records a digest of the GEMM kernel's source and build
flags; ``bench.py`` reports the figure only while that digest still matches,
so a changed kernel never carries counters taken from an older one.

* ``counters``: per-kernel shader counters (matrix-unit and VALU activity,
  wave wait states) from one or more ``rocprofv3 --pmc`` passes of the same
  command, normalised by the cycles ``GRBM_GUI_ACTIVE`` counts in each pass.

Usage (on the CPU, after the profiler runs):
  python -m blockwise_fp8_linear_quant_amd.profiling stats KERNEL_STATS.csv OUT.txt --command "..."
  python -m blockwise_fp8_linear_quant_amd.profiling traffic FETCH.csv WRITE.csv OUT.txt \
      --copy-bytes N --command "..."
  python -m blockwise_fp8_linear_quant_amd.profiling counters PASS1.csv [PASS2.csv ...] OUT.txt \
      --kernels block_gemm_f16_kernel quant_dual_kernel --command "..."
"""

import argparse
import csv
import hashlib
import json
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/fp8_codec.h", "build.py")
# The exact path's GEMM kernels: 256 x 128 and 128 x 128 tiles, and 128 x 128
# tiles of eight waves in two contraction groups.
GEMM_KERNELS = ("block_gemm_f16_kernel", "block_gemm_f16_kgroups_kernel")
FP8_KERNEL = "block_gemm_fp8_kernel"
COPY_KERNEL_HINTS = ("copy", "elementwise")


def is_exact_gemm(name):
    return any(k in name for k in GEMM_KERNELS)


def source_digest(files=GEMM_SOURCES):
    """sha256 over the GEMM kernel source, the codec header it includes and the build script (its flags)."""
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(_HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def short_name(name):
    """Kernel name without namespaces and the parameter list; template arguments kept."""
    name = re.sub(r"^void ", "", name)
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and i > 0 and name[i - 1] != ":":
            if not name.startswith("(anonymous", i):
                cut = i
                break
    name = name[:cut]
    return name.replace("fp8blk::(anonymous namespace)::", "")


def stats_summary(stats_csv, command, bench_json=None):
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"command: {command}", "",
             f"{'kernel':<78} {'calls':>6} {'avg_us':>9} {'total_ms':>9} {'share%':>7}"]
    for r in rows:
        lines.append(f"{short_name(r['Name'])[:78]:<78} {int(r['Calls']):>6} "
                     f"{float(r['AverageNs']) / 1e3:>9.2f} {float(r['TotalDurationNs']) / 1e6:>9.3f} "
                     f"{float(r['Percentage']):>7.2f}")
    bench = json.loads(open(bench_json).read().strip().splitlines()[-1]) if bench_json else {}
    # Each GEMM kernel family beside bench.py's own figure from the same
    # profiled process (HIP events around the timed steps on the GEMMs' stream).
    for kernels, key, rate in ((GEMM_KERNELS, "roofline", "achieved"),
                               ((FP8_KERNEL,), "fp8_matrix_core_path", "gemm_tflops")):
        sel = [r for r in rows if any(k in r["Name"] for k in kernels)]
        if not sel:
            continue
        calls = sum(int(r["Calls"]) for r in sel)
        avg_us = sum(float(r["TotalDurationNs"]) for r in sel) / calls / 1e3
        lines += ["", f"{' + '.join(kernels)} (all instantiations): {calls} calls, average {avg_us:.2f} us"]
        rec = bench.get(key)
        if rec and "avg_launch_us" in rec:
            lines += [f"bench.py in the same run: average launch {rec['avg_launch_us']:.2f} us over "
                      f"{rec['launches_per_step']} launches per step, {rec[rate]:.1f} TFLOP/s",
                      f"rocprofv3 average / bench.py average: {avg_us / rec['avg_launch_us']:.3f}"]
    return "\n".join(lines) + "\n"


def _dispatch_counters(path, counter):
    """{dispatch id: (kernel name, value)} for one counter of a counter_collection CSV."""
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, val = r["Kernel_Name"], float(r["Counter_Value"])
        if d in out:   # one row per agent/XCD instance in some versions: add them
            out[d] = (name, out[d][1] + val)
        else:
            out[d] = (name, val)
    return out


def traffic_summary(fetch_csv, write_csv, copy_bytes, command, algorithmic_bytes_per_launch=None):
    fetch = _dispatch_counters(fetch_csv, "FETCH_SIZE")
    write = _dispatch_counters(write_csv, "WRITE_SIZE")

    def copy_value(tab):
        cands = [(d, v) for d, (n, v) in tab.items()
                 if not is_exact_gemm(n) and any(h in n.lower() for h in COPY_KERNEL_HINTS)]
        if not cands:
            raise SystemExit("no copy kernel dispatch found in the counter CSV")
        return max(cands, key=lambda dv: dv[1])[1]   # the big copy of known size

    f_copy_kib, w_copy_kib = copy_value(fetch), copy_value(write)
    f_scale = copy_bytes / f_copy_kib   # bytes per counter unit
    w_scale = copy_bytes / w_copy_kib
    gf = [v for n, v in fetch.values() if is_exact_gemm(n)]
    gw = [v for n, v in write.values() if is_exact_gemm(n)]
    if not gf or not gw:
        raise SystemExit("no block GEMM dispatch in the counter CSVs")
    fetch_b = sum(gf) / len(gf) * f_scale
    write_b = sum(gw) / len(gw) * w_scale
    lines = [
        f"command: {command}",
        f"source_sha256: {source_digest()}",
        f"copy_probe_bytes: {copy_bytes}",
        f"copy_probe_fetch_kib: {f_copy_kib:.1f}",
        f"copy_probe_write_kib: {w_copy_kib:.1f}",
        f"fetch_scale_bytes_per_kib: {f_scale:.2f}",
        f"write_scale_bytes_per_kib: {w_scale:.2f}",
        f"gemm_dispatches: {len(gf)}",
        f"gemm_fetch_bytes_per_launch: {fetch_b:.0f}",
        f"gemm_write_bytes_per_launch: {write_b:.0f}",
        f"gemm_hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
    ]
    if algorithmic_bytes_per_launch:
        lines.append(f"gemm_algorithmic_bytes_per_launch: {algorithmic_bytes_per_launch:.0f}")
        lines.append(f"traffic_over_algorithmic: {(fetch_b + write_b) / algorithmic_bytes_per_launch:.3f}")
    return "\n".join(lines) + "\n"


# MI355X: 8 XCDs x 32 CUs x 4 SIMDs; a wave64 VALU instruction occupies its
# SIMD for 4 cycles; F16/BF16 dense matrix peak 2.5 PFLOP/s at 2.4 GHz.
N_XCD, N_SIMD, VALU_CYCLES, F16_PEAK_FLOP_PER_CYCLE = 8, 1024, 4, 2.5e15 / 2.4e9


def counters_summary(csvs, kernels, command):
    """Shader-counter ratios per kernel instantiation, averaged over its dispatches.

    Each pass is a separate run of the same command, so dispatches are matched
    by their id.  Cycles per dispatch come from GRBM_GUI_ACTIVE of the same
    pass (it counts on every XCD: divided by 8), and SIMD-cycles are that times
    the 1024 SIMDs.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD-cycles (it
    counts 32 cycles per 32x32x16 F16 MFMA); VALU busy = non-MFMA VALU
    instructions x 4 cycles / SIMD-cycles; wait fractions are per wave-cycle.
    """
    per = {}   # (dispatch, name) -> {counter: value, "_cyc_<pass>": cycles, "_dur": ns}
    for ip, path in enumerate(csvs):
        for r in csv.DictReader(open(path)):
            name = short_name(r["Kernel_Name"])
            if not any(k in name for k in kernels):
                continue
            key = (int(r["Dispatch_Id"]), name)
            d = per.setdefault(key, {})
            c, v = r["Counter_Name"], float(r["Counter_Value"])
            if c == "GRBM_GUI_ACTIVE":
                d[f"_cyc{ip}"] = d.get(f"_cyc{ip}", 0.0) + v / N_XCD
                d[f"_dur{ip}"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            else:
                d[c] = d.get(c, 0.0) + v
                d[f"_pass_{c}"] = ip
    groups = {}
    for (_, name), d in per.items():
        groups.setdefault(name, []).append(d)
    lines = [f"command: {command}", ""]
    for name, ds in sorted(groups.items()):
        def ratio(num, den_fn):
            vals = [d[num] / den_fn(d) for d in ds if num in d and den_fn(d)]
            return sum(vals) / len(vals) if vals else None

        def simd_cycles(c):
            def f(d):
                ip = d.get(f"_pass_{c}")
                return d.get(f"_cyc{ip}", 0.0) * N_SIMD if ip is not None else 0.0
            return f
        clk = [d[f"_cyc{i}"] / d[f"_dur{i}"] for d in ds for i in range(len(csvs)) if f"_dur{i}" in d]
        dur = [d[f"_dur{i}"] for d in ds for i in range(len(csvs)) if f"_dur{i}" in d]
        lines.append(f"kernel: {name}")
        lines.append(f"  dispatches: {len(ds)}")
        if dur:
            lines.append(f"  mean_duration_us (under the profiler): {sum(dur) / len(dur) / 1e3:.2f}")
        if clk:
            lines.append(f"  clock_ghz (GRBM_GUI_ACTIVE / 8 / duration; overstated for dispatches of a few us): "
                         f"{sum(clk) / len(clk):.2f}")
        vals = {
            "mfma_busy": ratio("SQ_VALU_MFMA_BUSY_CYCLES", simd_cycles("SQ_VALU_MFMA_BUSY_CYCLES")),
            "valu_mfma_coexec": ratio("SQ_VALU_MFMA_COEXEC_CYCLES", simd_cycles("SQ_VALU_MFMA_COEXEC_CYCLES")),
        }
        valu = [((d["SQ_INSTS_VALU"] - d.get("SQ_INSTS_MFMA", 0.0)) * VALU_CYCLES) / simd_cycles("SQ_INSTS_VALU")(d)
                for d in ds if "SQ_INSTS_VALU" in d and simd_cycles("SQ_INSTS_VALU")(d)]
        if valu:
            vals["valu_busy (non-MFMA, 4 cycles per instruction)"] = sum(valu) / len(valu)
        for k, v in vals.items():
            if v is not None:
                lines.append(f"  {k}: {v:.3f}")
        for num, den, label in (("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "valu_instructions_per_mfma (incl. MFMA)"),
                                ("SQ_INSTS_LDS", "SQ_INSTS_MFMA", "lds_instructions_per_mfma"),
                                ("SQ_WAIT_ANY", "SQ_WAVE_CYCLES", "wave_fraction_waiting_on_waitcnt_or_barrier"),
                                ("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "wave_fraction_ready_but_not_issued"),
                                ("SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES", "wave_fraction_issuing"),
                                ("SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "lds_bank_conflict_cycles_per_lds_instruction")):
            v = ratio(num, lambda d, den=den: d.get(den, 0.0))
            if v is not None:
                lines.append(f"  {label}: {v:.3f}")
        mf = [d["SQ_INSTS_MFMA"] for d in ds if "SQ_INSTS_MFMA" in d]
        if mf and clk and "f16" in name:
            flops = [d["SQ_INSTS_MFMA"] * 32768 for d in ds if "SQ_INSTS_MFMA" in d]
            lines.append(f"  mfma_flop_per_dispatch (32x32x16 F16): {sum(flops) / len(flops):.4g}")
        lines.append("")
    return "\n".join(lines)


def read_traffic(path):
    """The traffic summary as a dict, or None if missing or taken from another kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest():
        return None
    return kv


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--bench-json", help="bench.py output of the profiled command")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--algorithmic-bytes", type=float)
    c = sub.add_parser("counters")
    c.add_argument("csvs", nargs="+")
    c.add_argument("--kernels", nargs="+", required=True)
    c.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.cmd == "stats":
        text = stats_summary(a.stats_csv, a.command, a.bench_json)
    elif a.cmd == "traffic":
        text = traffic_summary(a.fetch_csv, a.write_csv, a.copy_bytes, a.command, a.algorithmic_bytes)
    else:
        *inputs, out = a.csvs
        a.out = out
        text = counters_summary(inputs, a.kernels, a.command)
    with open(a.out, "w") as f:
        f.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
