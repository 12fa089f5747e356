"""The one-line JSON contract of bench.py.

CPU: more than one GPU is refused with a message and exit status 2 (the
check comes before anything touches a GPU).  GPU: a short run of the small
label cross-entropy workload, in this process, prints one JSON line with
the required fields, a roofline object for the dominant kernel and the
per-kernel breakdown.
"""
import contextlib
import io
import json
import subprocess
import sys

import pytest

from tests.conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.gpu
def test_bench_prints_the_contract_line(monkeypatch):
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "ce_bf16_1b", "--steps", "2",
                                      "--warmup", "1", "--no-cpu-baseline"])
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        bench.main()
    lines = [l for l in out.getvalue().splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", float),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str), ("data", str),
                     ("config", dict), ("roofline", dict)):
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "ce_bf16_1b"
    n = d["config"]["tokens"]
    assert abs(d["value"] - n / (d["ms_per_step"] * 1e-3)) <= 1e-3 * d["value"]
    roof = d["roofline"]
    assert roof["bound"] in ("mfma", "hbm", "alu") and roof["unit"] in ("TFLOP/s", "GB/s")
    assert roof["peak"] > 0 and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    assert roof["kernel"] in d["kernels"]
    assert "cpu_baseline" not in d
