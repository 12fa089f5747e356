"""HBM traffic per kernel launch from rocprofv3 counter passes.

Two passes of the benchmark under ``rocprofv3 --pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` (``--output-format csv``), each run with
``bench.py --calibrate-copy`` so that the same process also copies a buffer
of known size.  The counters of that plain copy give a scale factor per
counter (known bytes / counted bytes), which converts every kernel's counted
kilobytes into bytes.  The summary records a digest of the kernel sources;
bench.py reports the traffic only while the digest still matches.

    python -m lm_head_vocab_amd.profiling --fetch <fetch csv> --write <write csv> \
        --copy-bytes <n> --out profiles/<name>.json \
        [--stats <rocprofv3 kernel_stats.csv> --md profiles/<name>.md]

With --stats and --md it also writes a markdown summary: the per-kernel
durations of a `rocprofv3 --kernel-trace --stats` run of the same benchmark
and the calibrated bytes per launch.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

_PKG = os.path.dirname(os.path.abspath(__file__))
# the device code (kernels and the launch structures they read); host-side
# changes, comments and formatting that leave every kernel as it was keep the
# counters valid
SOURCES = ("csrc/kernels.hip", "csrc/tile_gemm.hpp", "csrc/launch.hpp")


def _code_only(text: str) -> str:
    """The source without comments and with whitespace collapsed, so that a
    comment or formatting edit does not mark the counters stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(_PKG, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def trace_name(kernel: str) -> str:
    """Map a profiler kernel name to the library's trace name."""
    m = re.search(r"specloss::(k_\w+)(<[^(]*>)?\(", kernel)
    if not m:
        return kernel
    base, targs = m.group(1), m.group(2) or ""
    if base == "k_gemm":  # k_gemm<T, OutT, ROLE, LEAN, WNW, DUMP>
        args = [a.strip() for a in targs.strip("<>").split(",")]
        if len(args) > 2 and args[2] == "1":
            return "gemm_dW"
        return "gemm_dh_dzt" if len(args) > 5 and args[5] == "true" else "gemm_dh"
    names = {"k_stats": "stats_q", "k_stats_stage": "stats_stage", "k_dz_stage": "dz_stage",
             "k_dz": "dz", "k_div": "div", "k_combine1": "combine1", "k_combine2": "combine2", "k_stage_fix": "stage_fix",
             "k_rowdot": "rowdot", "k_transpose": "transpose", "k_validity": "validity",
             "k_reduce": "reduce", "k_seed": "seed", "k_align": "align",
             "k_stats_dual": "stats_dual", "k_div_heads": "div_heads", "k_heads_map": "heads_map",
             "k_sum_parts": "sum_partials", "k_div_raw": "div_raw", "k_dz_raw": "dz_raw",
             "k_target_gather": "target_gather"}
    name = names.get(base, base)
    if base == "k_stats":  # k_stats<T, TARGET, WNW, RAW>
        args = [a.strip() for a in targs.strip("<>").split(",")]
        return "stats_p" if len(args) > 1 and args[1] == "true" else "stats_q"
    return name


def _per_kernel(path: str, counter: str):
    vals = defaultdict(list)
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] != counter:
            continue
        vals[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return vals


def summarize(fetch_csv: str, write_csv: str, copy_bytes: int):
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    copies = [k for k in fetch if "copy" in k.lower() and "specloss" not in k]
    if not copies:
        raise RuntimeError("no copy kernel in the fetch pass")
    ck = max(copies, key=lambda k: max(fetch[k]))
    f_fetch = copy_bytes / (max(fetch[ck]) * 1024.0)
    f_write = copy_bytes / (max(write.get(ck, [0.0])) * 1024.0) if write.get(ck) else None
    # Kernels that share a trace name (e.g. one contraction built for two tile
    # shapes) are counted as one entry of the library's trace: their bytes are
    # added and divided by the dispatch count of the most frequent one.
    groups = defaultdict(list)
    for k in fetch:
        if "specloss" in k:
            groups[trace_name(k)].append(k)
    out = {}
    for name, ks in groups.items():
        launches = max(len(fetch[k]) for k in ks)
        fb = sum(sum(fetch[k]) for k in ks) / launches * 1024.0 * f_fetch
        wb = None
        if f_write and any(write.get(k) for k in ks):
            w_launches = max(len(write.get(k, [])) for k in ks)
            wb = sum(sum(write.get(k, [])) for k in ks) / w_launches * 1024.0 * f_write
        out[name] = {"fetch_bytes": fb, "write_bytes": wb,
                     "bytes_per_launch": fb + (wb or 0.0), "dispatches": launches,
                     "kernels": len(ks)}
    return {"copy_kernel": ck, "copy_bytes": copy_bytes, "factor_fetch": f_fetch,
            "factor_write": f_write, "source_digest": source_digest(), "kernels": out}


TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- "
             "python3 <repo>/bench.py --workload {w} --steps 3 --warmup 1 --no-cpu-baseline")
TRACE_STEPS = 4  # single-call steps of TRACE_CMD (warmup + timed), run before the two calls


def single_call_avg_ms(trace_csv: str, kernel: str, launches_per_step: float):
    """Average duration (ms) of `kernel`'s dispatches in the single-call steps of
    TRACE_CMD: bench.py runs those first, so they are the kernel's first
    TRACE_STEPS x launches-per-step dispatches (None if the trace has fewer)."""
    n = int(round(TRACE_STEPS * launches_per_step))
    durs = []
    for r in csv.DictReader(open(trace_csv)):
        if trace_name(r["Kernel_Name"]) == kernel:
            durs.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if n <= 0 or len(durs) < n:
        return None
    return sum(durs[:n]) / n / 1e6
PMC_CMD = ("rocprofv3 --pmc {c} --output-format csv -d <{d}> -o pmc -- python3 <repo>/bench.py "
           "--workload {w} --steps 1 --warmup 0 --no-cpu-baseline --calibrate-copy")


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES")
SIMDS_PER_SE = 32  # MI355X: 32 shader engines (4 per XCD), 8 CUs x 4 SIMDs each


def mfma_summary(pmc_csv: str) -> dict:
    """Per trace name: executed MFMA flops per launch from the MOPS counters
    (one MOP = 512 flops) and the MFMA-busy fraction of the kernel's busy
    cycles, SQ_VALU_MFMA_BUSY_CYCLES / (SIMDS_PER_SE x SQ_BUSY_CYCLES) (the
    busy cycles are summed over the shader engines, the MFMA cycles over the
    SIMDs)."""
    vals = defaultdict(lambda: defaultdict(list))
    for row in csv.DictReader(open(pmc_csv)):
        if "specloss" not in row["Kernel_Name"]:
            continue
        vals[trace_name(row["Kernel_Name"])][row["Counter_Name"]].append(float(row["Counter_Value"]))
    out = {}
    for name, c in vals.items():
        n = max(len(v) for v in c.values())
        avg = {k: sum(v) / len(v) for k, v in c.items()}
        mops = avg.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + avg.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0)
        if mops <= 0:
            continue
        busy = avg.get("SQ_BUSY_CYCLES", 0.0)
        out[name] = {"flops_per_launch": mops * 512.0, "dispatches": n,
                     "mfma_busy": avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (SIMDS_PER_SE * busy)
                     if busy else None}
    return out


def markdown(stats_csv: str, traffic: dict, workload: str, bench: dict = None,
             mfma: dict = None) -> str:
    """Markdown summary of a kernel-trace stats run and the counter passes
    (and, if given, the bench.py line of a run on the same box)."""
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# Kernel durations and HBM traffic: `{workload}` fwd+bwd", "",
           "One bench.py process runs the single call `lmhead_loss_fwd_bwd` (the headline) and the",
           "two calls `lmhead_loss_fwd` + `lmhead_loss_bwd` (beside it), so both sets of kernels",
           "appear.  Written by `python -m lm_head_vocab_amd.profiling` from the runs below.", "",
           "## Durations", "", "Command (from /tmp with TMPDIR=/tmp):", "", "```", TRACE_CMD.format(w=workload), "```",
           "", "| kernel | calls | avg ms | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"].replace("specloss::", "").replace("|", "\\|")
        if len(name) > 72:
            name = name[:69] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    out += ["", "`k_gemm<T, OutT, 1, ...>` is the dW contraction, `k_gemm<T, OutT, 0, ...>` the dh "
            "contraction (the fourth template argument selects the copy-free variant; the sixth, "
            "traced as `gemm_dh_dzt`, the dh contraction that also writes dz^T).", ""]
    if bench:
        r = bench["roofline"]
        out += [f"`python3 bench.py --workload {workload}` on the same box, just before: "
                f"{bench['value']:.0f} {bench['unit']}, {bench['ms_per_step']:.3f} ms per step; "
                f"dominant kernel `{r['kernel']}` {r['avg_launch_ms']:.4f} ms per launch (HIP events "
                f"on the library's stream), {r['achieved']:.1f} {r['unit']}, {r['frac']:.4f} of peak.",
                ""]
        trace_csv = stats_csv.replace("kernel_stats", "kernel_trace")
        per_step = bench.get("kernels", {}).get(r["kernel"], {}).get("launches_per_step")
        if os.path.exists(trace_csv) and per_step:
            avg = single_call_avg_ms(trace_csv, r["kernel"], per_step)
            if avg is not None:
                out += [f"The same kernel in the traced run's single-call steps (its first "
                        f"{int(round(TRACE_STEPS * per_step))} dispatches in `run_kernel_trace.csv`; "
                        f"the averages above also hold the two calls' launches): {avg:.4f} ms per "
                        f"launch.", ""]
    out += ["## HBM bytes per launch", "", "Commands (two passes, each its own run):", "", "```",
            PMC_CMD.format(c="FETCH_SIZE", d="fetch", w=workload),
            PMC_CMD.format(c="WRITE_SIZE", d="write", w=workload),
            "python -m lm_head_vocab_amd.profiling --fetch <fetch>/pmc_counter_collection.csv "
            "--write <write>/pmc_counter_collection.csv --copy-bytes "
            f"{traffic['copy_bytes']} --out profiles/traffic_{workload}.json --stats "
            "<out>/run_kernel_stats.csv --md <this file> --workload " + workload
            + (" --bench-json <bench.py output>" if bench else ""), "```", "",
            f"`--calibrate-copy` copies {traffic['copy_bytes'] / 2**30:g} GiB inside the same "
            f"process; the counters of that copy (`{traffic['copy_kernel']}`) give the scale "
            f"factors FETCH_SIZE x {traffic['factor_fetch']:.3f}, WRITE_SIZE x "
            f"{(traffic['factor_write'] or 0):.3f}.  Source digest of the profiled kernels: "
            f"`{traffic['source_digest']}` ({', '.join(os.path.basename(x) for x in SOURCES)}).",
            "", "| kernel | fetched GB | written GB | total GB per launch |", "|---|---:|---:|---:|"]
    for k, v in sorted(traffic["kernels"].items(), key=lambda kv: -kv[1]["bytes_per_launch"]):
        out.append(f"| {k} | {v['fetch_bytes'] / 1e9:.3f} | {(v['write_bytes'] or 0) / 1e9:.3f} | "
                   f"{v['bytes_per_launch'] / 1e9:.3f} |")
    if mfma:
        lib = {}
        if bench:
            lib = {k: v.get("tflops") for k, v in bench.get("kernels", {}).items()}
        out += ["", "## MFMA counters per launch", "", "Command (its own run):", "", "```",
                PMC_CMD.format(c=" ".join(MFMA_COUNTERS), d="mfma", w=workload).replace(
                    " --calibrate-copy", ""), "```", "",
                "Executed flops = `SQ_INSTS_VALU_MFMA_MOPS_*` x 512 (the library counts the same "
                "contractions from its schedule); MFMA busy = `SQ_VALU_MFMA_BUSY_CYCLES` / "
                f"({SIMDS_PER_SE} SIMDs per shader engine x `SQ_BUSY_CYCLES`), the fraction of "
                "the kernel's cycles in which a SIMD's matrix pipe was busy (the clock under this "
                "load is below the 2.4 GHz of the peak figure).", "",
                "| kernel | counted TFLOP per launch | MFMA busy |", "|---|---:|---:|"]
        for k, v in sorted(mfma.items(), key=lambda kv: -kv[1]["flops_per_launch"]):
            busy = "" if v["mfma_busy"] is None else f"{v['mfma_busy']:.3f}"
            out.append(f"| {k} | {v['flops_per_launch'] / 1e12:.3f} | {busy} |")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--stats", default=None, help="rocprofv3 kernel_stats.csv of the same benchmark")
    ap.add_argument("--md", default=None, help="markdown summary to write (needs --stats)")
    ap.add_argument("--workload", default="ce_bf16_8b")
    ap.add_argument("--bench-json", default=None, help="bench.py output of a run on the same box")
    ap.add_argument("--mfma", default=None, help="counter csv of the MFMA pass (MFMA_COUNTERS)")
    a = ap.parse_args()
    s = summarize(a.fetch, a.write, a.copy_bytes)
    with open(a.out, "w") as f:
        json.dump(s, f, indent=1)
    if a.md and a.stats:
        bench = None
        if a.bench_json:
            with open(a.bench_json) as f:
                bench = json.loads([l for l in f.read().splitlines() if l.strip()][-1])
        mf = mfma_summary(a.mfma) if a.mfma else None
        if mf:
            s["mfma"] = mf
            with open(a.out, "w") as f:
                json.dump(s, f, indent=1)
        with open(a.md, "w") as f:
            f.write(markdown(a.stats, s, a.workload, bench, mf))
    print(json.dumps({k: round(v["bytes_per_launch"] / 1e9, 3) for k, v in s["kernels"].items()}))


if __name__ == "__main__":
    main()
