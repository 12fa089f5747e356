"""HBM traffic per kernel launch from rocprofv3 counter passes.

Two passes of the benchmark under ``rocprofv3 --pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` (``--output-format csv``), each run with
``bench.py --calibrate-copy`` so that the same process also copies a buffer
of known size.  The counters of that plain copy give a scale factor per
counter (known bytes / counted bytes), which converts every kernel's counted
kilobytes into bytes.  The summary records a digest of the kernel sources;
bench.py reports the traffic only while the digest still matches.

    python -m lm_head_vocab_amd.profiling --fetch <fetch csv> --write <write csv> \
        --copy-bytes <n> --out profiles/<name>.json
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
# changes that leave every kernel as it was keep the counters valid
SOURCES = ("csrc/kernels.hip", "csrc/tile_gemm.hpp", "csrc/launch.hpp")


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(_PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def trace_name(kernel: str) -> str:
    """Map a profiler kernel name to the library's trace name."""
    m = re.search(r"specloss::(k_\w+)(<[^(]*>)?\(", kernel)
    if not m:
        return kernel
    base, targs = m.group(1), m.group(2) or ""
    if base == "k_gemm":  # k_gemm<T, OutT, ROLE, LEAN>
        args = [a.strip() for a in targs.strip("<>").split(",")]
        return "gemm_dW" if len(args) > 2 and args[2] == "1" else "gemm_dh"
    names = {"k_stats": "stats_q", "k_stats_stage": "stats_stage", "k_dz_stage": "dz_stage",
             "k_dz": "dz", "k_div": "div", "k_combine1": "combine1", "k_combine2": "combine2",
             "k_rowdot": "rowdot", "k_transpose": "transpose", "k_validity": "validity",
             "k_reduce": "reduce", "k_seed": "seed", "k_align": "align"}
    name = names.get(base, base)
    if "true" in targs:
        name = {"k_stats": "stats_p", "k_div": "div_stage", "k_dz_stage": "dz_div"}.get(base, name)
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
    out = {}
    for k, v in fetch.items():
        if "specloss" not in k:
            continue
        fb = sum(v) / len(v) * 1024.0 * f_fetch
        wv = write.get(k, [])
        wb = (sum(wv) / len(wv) * 1024.0 * f_write) if (wv and f_write) else None
        name = trace_name(k)
        out[name] = {"fetch_bytes": fb, "write_bytes": wb,
                     "bytes_per_launch": fb + (wb or 0.0), "dispatches": len(v)}
    return {"copy_kernel": ck, "copy_bytes": copy_bytes, "factor_fetch": f_fetch,
            "factor_write": f_write, "source_digest": source_digest(), "kernels": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    s = summarize(a.fetch, a.write, a.copy_bytes)
    with open(a.out, "w") as f:
        json.dump(s, f, indent=1)
    print(json.dumps({k: round(v["bytes_per_launch"] / 1e9, 3) for k, v in s["kernels"].items()}))


if __name__ == "__main__":
    main()
