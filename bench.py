#!/usr/bin/env python3
"""Benchmark of the streaming LM-head + loss step (forward + backward).

One step = the forward and backward of the mean loss over the whole batch,
inputs resident in HBM: the single call lmhead_loss_fwd_bwd (headline), and
the two calls lmhead_loss_fwd + lmhead_loss_bwd (reported beside it).  The
default workload is label cross-entropy at the Llama-3.1-8B shape
(N = 32768 tokens of one 32k sequence, H = 4096, V = 128256, bf16 inputs,
fp32 accumulation); --workload selects another synthetic workload, e.g. the
lk_hybrid divergence (lk_hybrid_bf16_8b) or the three-head ce + tv loss at
the Llama-3.1-405B shape (multihead_bf16_405b).
Prints one JSON line with tokens/s, the MFMA fractions, peak HBM, the
roofline of the dominant kernel and the fp64 CPU oracle timed on a sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ce_bf16_8b")
    ap.add_argument("--weights", default=None,
                    help="loss weights replacing the workload's, e.g. kl_div=1,ce=0.2 "
                         "(the workload's inputs are kept)")
    ap.add_argument("--chunk", type=int, default=0,
                    help="max rows per chunk (0: the library's default streaming policy)")
    ap.add_argument("--shards", type=int, default=1,
                    help="G > 1: time one vocabulary shard's calls (V/G rows of W) and the "
                         "merges, i.e. one device's step of a G-way vocabulary-parallel group")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="rows of the oracle's timed sample (0: 1536 at H = 4096, scaled by "
                         "4096 / H, at least 256: about 10-30 s on the host cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also copy a buffer of known size (for counter calibration)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="also time hipBLASLt (torch.matmul) on the step's three contraction "
                         "shapes with the same operands (label cross-entropy workloads)")
    ap.add_argument("--traffic", default=None,
                    help="counter summary giving HBM bytes per launch "
                         "(default profiles/traffic_<workload>.json)")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def copy_calibration():
    """A plain device copy of COPY_BYTES bytes (its counters scale the others)."""
    import torch
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    del x, y


def load_traffic(path, kernel):
    """Bytes per launch of `kernel` from a counter summary, None if absent or stale."""
    try:
        from lm_head_vocab_amd.profiling import source_digest
        with open(path) as f:
            t = json.load(f)
        if t.get("source_digest") != source_digest():
            return None
        return t["kernels"].get(kernel, {}).get("bytes_per_launch")
    except (OSError, ValueError, KeyError):
        return None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic
    import lm_head_vocab_amd as L
    from lm_head_vocab_amd.runner import LossRun, ShardedLossRun

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    L.load_library()
    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        copy_calibration()

    t0 = time.time()
    prob = synthetic.make_problem(args.workload)
    if args.weights:
        prob.weights = {k: float(v) for k, v in (kv.split("=") for kv in args.weights.split(","))}
        if any(k != "ce_label" for k in prob.weights) and prob.target_hidden is None:
            print("--weights: divergences need a workload with a target side", file=sys.stderr)
            sys.exit(2)
    gen_s = time.time() - t0
    N, H, V = prob.n_rows, prob.hidden_dim, prob.vocab

    if prob.dtype != "bf16":
        print("bench.py times the bf16 workloads", file=sys.stderr)
        sys.exit(2)

    def up(x):
        if x is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    def up_i(x, dt):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x).astype(dt)).to(dev)

    h = up(prob.hidden)
    W = up(prob.W)
    inputs = dict(labels=up_i(prob.labels, np.int32), mask=up_i(prob.mask, np.uint8),
                  target_hidden=up(prob.target_hidden), W_t=up(prob.W_t),
                  target_row=up_i(prob.target_row, np.int32), heads=prob.shifts)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_alloc = torch.cuda.memory_allocated()

    dh = torch.empty((N, H), dtype=torch.float32, device=dev)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    gmean = torch.ones(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    G = args.shards
    if G > 1:
        # every shard runs once so the exchange holds real records; the timed
        # step is shard 0's calls plus the merges (one device's share)
        run = ShardedLossRun(h, W, prob.weights, G, max_chunk_rows=args.chunk, **inputs)
        run.forward(stream)
        run.backward(grad_mean=gmean, dhidden=dh, dW=dW, stream=stream)
        p0, s0 = run.problems[0], run.shards[0]
        v_shard = run.bounds[1]
        chunk_rows, chunk_layout, dw_group = L.binding.lmhead_loss_chunk(
            p0, run.workspace.numel(), L.binding.CALL_BWD)
        dh_part = torch.empty((N, H), dtype=torch.float32, device=dev)
        terms = torch.empty(L.binding.NUM_KINDS, N, dtype=torch.float32, device=dev)

        def step_single():
            B = L.binding
            B.lmhead_shard_pass1(p0, s0, run.workspace, stream)
            B.lmhead_shard_merge1(p0, s0, run.saved, run.counts, stream)
            B.lmhead_shard_pass2(p0, s0, run.saved, run.workspace, stream)
            B.lmhead_shard_merge2(p0, s0, run.saved, run.counts, run.loss, terms, None,
                                  run.reduced, stream)
            B.lmhead_shard_bwd(p0, s0, None, gmean, run.counts, run.saved, run.workspace,
                               dh_part, dW[:v_shard], False, stream)
        step_two = None
    else:
        run = LossRun(h, W, prob.weights, max_chunk_rows=args.chunk, want_terms=False, **inputs)
        v_shard = V
        chunk_rows, chunk_layout, dw_group = run.chunk(L.binding.CALL_FWD_BWD)

        def step_single():
            run.forward_backward(grad_mean=gmean, dhidden=dh, dW=dW, stream=stream)

        def step_two():
            run.forward(stream)
            run.backward(grad_mean=gmean, dhidden=dh, dW=dW, stream=stream)

    def timed(step, steps, warmup):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        # room for every launch: a few per call plus at most 24 per chunk
        trace = L.binding.Trace(capacity=steps * (32 + 24 * max_chunks))
        trace.attach(run.problem)
        torch.cuda.synchronize()
        wall0 = time.time()
        for i in range(steps):
            starts[i].record(stream)
            step()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.time() - wall0
        entries = trace.read()
        if len(entries) >= trace.capacity:
            raise RuntimeError("the launch trace filled up; per-kernel times would be partial")
        kernels = summarize_trace(entries, steps)
        run.problem.trace = None
        trace.close()
        per = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
        return sum(per) / steps, per[len(per) // 2], kernels, wall

    if G == 1:
        calls = (L.binding.CALL_FWD, L.binding.CALL_BWD, L.binding.CALL_FWD_BWD)
        max_chunks = max(-(-N // run.chunk(c)[0]) for c in calls)
    else:
        max_chunks = -(-N // 256) * 2
    ms_mean, ms_med, kernels, wall = timed(step_single, args.steps, args.warmup)
    if step_two is not None:
        ms_two, ms_two_med, kernels_two, _ = timed(step_two, max(2, args.steps // 2), 1)
    peak_bytes = torch.cuda.max_memory_allocated()

    # Executed MFMA flops per step: the library's own count for every
    # contraction launch of the step (e.g. 6NHV for the single-call label
    # cross-entropy: forward, dh, dW).  Model flops: one pass over the draft
    # logits (2NHV), one over each distinct target row (2 N_t HV) and the two
    # gradient contractions (4NHV), so that recompute cannot raise the fraction.
    nhv = float(N) * H * v_shard
    n_t = 0
    if prob.target_hidden is not None:
        n_t = N if prob.target_row is None else int(prob.target_hidden.shape[0])
    model_flops = 6.0 * nhv + 2.0 * n_t * H * v_shard

    def flops_per_step(ks):
        return sum(v["work_per_launch"] * v["launches_per_step"] for v in ks.values()
                   if v["is_flops"])

    exec_flops = flops_per_step(kernels)
    tflops = exec_flops / (ms_mean * 1e-3) / 1e12
    model_tflops = model_flops / (ms_mean * 1e-3) / 1e12
    traffic_path = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")

    dom = max(kernels, key=lambda k: kernels[k]["ms_total"])
    d = kernels[dom]
    achieved = d["work_per_launch"] / (d["ms_avg"] * 1e-3) / 1e12
    kern = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": load_traffic(traffic_path, dom), "flops_per_launch": d["work_per_launch"],
            "avg_launch_ms": round(d["ms_avg"], 4), "launches_per_step": d["launches_per_step"]}

    result = {
        "metric": "fused LM-head+loss fwd+bwd tokens/s, % bf16 MFMA peak, peak HBM GiB @8B shape",
        "value": round(N / (ms_mean * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_mean, 3),
        "ms_per_step_median": round(ms_med, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded; {prob.recipe})",
        "config": {"workload": args.workload, "tokens": N, "hidden": H, "vocab": V,
                   "loss": prob.weights, "chunk_rows": chunk_rows, "bwd_layout": chunk_layout,
                   "dw_group": dw_group,
                   "call": "lmhead_loss_fwd_bwd" if G == 1 else
                   "lmhead_shard_pass1/merge1/pass2/merge2/bwd of shard 0",
                   "parallelism": "none (1 GPU)" if G == 1 else
                   f"vocab shard 0 of {G} (rows 0..{v_shard}), exchanges not timed"},
        "mfma_frac_executed": round(tflops / BF16_PEAK_TFLOPS, 4),
        "mfma_frac_model": round(model_tflops / BF16_PEAK_TFLOPS, 4),
        "executed_tflops": round(tflops, 1),
        "executed_flops_per_step_over_nhv": round(exec_flops / nhv, 3),
        "peak_hbm_gib": round(peak_bytes / 2**30, 3),
        "peak_hbm_gib_above_inputs": round((peak_bytes - base_alloc) / 2**30, 3),
        "logits_sized_limit_gib": round(N * V * 2 / 2**30, 3),
        "workspace_gib": round(run.workspace.numel() / 2**30, 3),
        "workspace_below_logits": bool(run.workspace.numel() < N * V * 2),
        "roofline": kern,
        "two_calls": None if step_two is None else {
            "value": round(N / (ms_two * 1e-3), 1), "ms_per_step": round(ms_two, 3),
            "mfma_frac_executed": round(flops_per_step(kernels_two) / (ms_two * 1e-3) / 1e12
                                        / BF16_PEAK_TFLOPS, 4),
            "mfma_frac_model": round(model_flops / (ms_two * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "kernels": {k: {"ms_per_step": round(v["ms_total"] / args.steps, 3),
                        "launches_per_step": v["launches_per_step"],
                        "tflops": round(v["work_per_launch"] / (v["ms_avg"] * 1e-3) / 1e12, 1)
                        if v["is_flops"] else None}
                    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["ms_total"])},
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(gen_s, 1),
    }
    if args.blas_reference and G == 1 and inputs["labels"] is not None:
        result["blas_reference"] = blas_reference(h, W, inputs["labels"], min(chunk_rows, N), N,
                                                  kernels)
    if not args.no_cpu_baseline:
        rows = args.cpu_sample_rows or max(256, 1536 * 4096 // prob.hidden_dim // 64 * 64)
        result["cpu_baseline"] = cpu_baseline(prob, min(rows, prob.n_rows))
    print(json.dumps(result), flush=True)
    if not result["workspace_below_logits"]:
        print(f"warning: the workspace ({result['workspace_gib']} GiB) is not below the [N, V] "
              f"bf16 logits size ({result['logits_sized_limit_gib']} GiB)", file=sys.stderr)


def blas_reference(h, W, labels, nc, N, kernels):
    """The vendor GEMM on the step's contraction shapes, same process and operands.

    One chunk of hidden rows against W (the forward logits), and that chunk's
    label cross-entropy logit gradient (softmax minus one-hot, over N tokens)
    against W (dh shape) and, transposed, against the hidden rows (dW shape).
    torch.matmul runs hipBLASLt with bf16 inputs, fp32 accumulation and bf16
    output, i.e. without the fused epilogues of the library's kernels.
    """
    import torch
    c = h[:nc]
    z = torch.matmul(c, W.t())
    p = torch.softmax(z.float(), dim=1)
    del z
    p[torch.arange(nc, device=h.device), labels[:nc].long()] -= 1.0
    dz = (p / N).to(torch.bfloat16)
    del p
    dzt = dz.t().contiguous()
    flops = 2.0 * nc * h.shape[1] * W.shape[0]

    def rate(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return round(flops / (sorted(ts)[2] * 1e-3) / 1e12, 1)

    ours = {k: round(kernels[k]["work_per_launch"] / (kernels[k]["ms_avg"] * 1e-3) / 1e12, 1)
            for k in ("stats_stage", "gemm_dh", "gemm_dh_dzt", "gemm_dW") if k in kernels}
    return {"library": "hipBLASLt via torch.matmul (bf16 in, fp32 accumulate, bf16 out)",
            "shapes": {"pass1": [nc, W.shape[0], h.shape[1]], "dh": [nc, h.shape[1], W.shape[0]],
                       "dW": [W.shape[0], h.shape[1], nc]},
            "tflops": {"pass1": rate(lambda: torch.matmul(c, W.t())),
                       "dh": rate(lambda: torch.matmul(dz, W)),
                       "dW": rate(lambda: torch.matmul(dzt, c))},
            "ours_tflops": ours}


FLOP_KERNELS = ("stats_q", "stats_p", "stats_stage", "stats_dual", "div", "div_heads", "dz",
                "gemm_dh", "gemm_dh_dzt", "gemm_dW")


def summarize_trace(entries, steps):
    """Per-kernel totals from the library's HIP-event trace of the timed steps."""
    out = {}
    for name, ms, work in entries:
        e = out.setdefault(name, {"ms_total": 0.0, "n": 0, "work": 0.0})
        e["ms_total"] += ms
        e["n"] += 1
        e["work"] += work
    for name, e in out.items():
        e["ms_avg"] = e["ms_total"] / e["n"]
        e["work_per_launch"] = e["work"] / e["n"]
        e["launches_per_step"] = e["n"] / steps
        e["is_flops"] = name in FLOP_KERNELS
    return out


def cpu_baseline(prob, rows):
    """The fp64 oracle, as it stands, on the first `rows` rows of the same workload."""
    import numpy as np
    from oracle import specloss_oracle as O
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    sel = np.arange(rows)
    t0 = time.time()
    w64 = O._weights64(O.OracleProblem.of(prob))
    widen_s = time.time() - t0
    t0 = time.time()
    seed = O.mean_seed(prob)
    O.forward(prob, rows=sel, weights64=w64)
    O.backward(prob, seed=seed, rows=sel, weights64=w64)
    dt = time.time() - t0
    return {"value": round(rows / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fwd+bwd (fp64, dense logits per 64-row block) of the first {rows} of "
                      f"{prob.n_rows} rows, full vocab and dW; {dt:.1f} s, plus {widen_s:.1f} s "
                      f"widening W to fp64 once"}


if __name__ == "__main__":
    main()
