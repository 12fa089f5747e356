"""Shared helpers of the GPU parity tests: upload a synthetic problem, run the
HIP path through the C-ABI binding, and compare against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import lm_head_vocab_amd as L
from lm_head_vocab_amd.runner import LossRun, ShardedLossRun
from oracle import specloss_oracle as O

# acceptance bars (fixed by the benchmark spec of the path)
LOSS_RTOL = 1e-3          # mean loss and per-term means, relative
# per-token losses: the same relative bar per token, with an absolute floor for
# losses that vanish exactly (tv of identical distributions is 1 - alpha with
# alpha an fp32 sum of V terms, off by up to about V * 2^-24); the floor also
# applies to the means
TOKEN_RTOL, TOKEN_ATOL = 1e-3, 1e-5
GRAD_FROB = 2e-2          # dh, dW relative Frobenius error
ARGMAX_GAP = 1e-3         # argmax labels must match where the top-2 gap is at least this


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(prob, dev="cuda"):
    def f(x):
        if x is None:
            return None
        if prob.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    def i(x, dt):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x).astype(dt)).to(dev)

    return dict(hidden=f(prob.hidden), W=f(prob.W), labels=i(prob.labels, np.int32),
                mask=i(prob.mask, np.uint8), target_hidden=f(prob.target_hidden), W_t=f(prob.W_t),
                target_row=i(prob.target_row, np.int32))


def make_run(prob, dev_inputs, **kw) -> LossRun:
    """LossRun of a synthetic problem; the transposed copies are forced unless
    flags or a workspace size are given (chunked cases then test that path)."""
    if "flags" not in kw and "workspace_bytes" not in kw:
        kw["flags"] = L.binding.FLAG_COPIES
    elif kw.get("flags") is None:
        kw["flags"] = 0
    kw.setdefault("heads", prob.shifts)  # aligned heads declare their layout
    return LossRun(dev_inputs["hidden"], dev_inputs["W"], prob.weights,
                   labels=dev_inputs["labels"], mask=dev_inputs["mask"],
                   target_hidden=dev_inputs["target_hidden"], W_t=dev_inputs["W_t"],
                   target_row=dev_inputs["target_row"], **kw)


def rel_frob(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def check_tokens(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    err = np.abs(gpu.astype(np.float64) - ref)
    bad = ~(err <= TOKEN_RTOL * np.abs(ref) + TOKEN_ATOL)  # a NaN is out of tolerance too
    worst = int(np.argmax(np.where(np.isnan(err), np.inf, err))) if err.size else 0
    assert not bad.any(), (f"{what}: {int(bad.sum())} rows out of tolerance; worst row "
                           f"{worst}: gpu {gpu[worst]} ref {ref[worst]}")


def check_flatness(gpu: np.ndarray, ref: np.ndarray, valid: np.ndarray) -> None:
    """Flatness within the per-token bar on valid rows, exactly 0 on the others."""
    check_tokens(gpu[valid], ref[valid], "flatness")
    assert np.all(gpu[~valid] == 0.0), "flatness of invalid rows must be 0"


def check_argmax(gpu_y: np.ndarray, prob, rows, valid) -> None:
    """Hard labels equal the oracle's wherever its top-2 target logits differ by >= ARGMAX_GAP."""
    Wt = O.widen(prob.W_t, prob.dtype)
    tr = rows if prob.target_row is None else np.asarray(prob.target_row)[rows]
    g = O.widen(prob.target_hidden[np.where(valid, tr, 0)], prob.dtype)
    u = g @ Wt.T
    top2 = np.sort(u, axis=1)[:, -2:]
    decisive = (top2[:, 1] - top2[:, 0] >= ARGMAX_GAP) & valid
    ref = O.argmax_lowest(u)
    assert np.array_equal(gpu_y[decisive], ref[decisive])


def ce_tie_candidates(prob, rows, valid, Wt64=None):
    """Rows whose ce label is not unique at the pages' precision.

    For each valid row of `rows` whose two largest target logits (oracle, fp64)
    differ by less than ARGMAX_GAP, the labels within ARGMAX_GAP of the maximum:
    any of them is a correct hard label there.  Returns {position in rows:
    (the oracle's label, set of candidates)}.
    """
    if "ce" not in prob.weights:
        return {}
    Wt = Wt64 if Wt64 is not None else O.widen(prob.W_t, prob.dtype)
    tr = rows if prob.target_row is None else np.asarray(prob.target_row)[rows]
    g = O.widen(prob.target_hidden[np.where(valid, tr, 0)], prob.dtype)
    u = g @ Wt.T
    out = {}
    for i in np.where(valid)[0]:
        top = np.max(u[i])
        cand = set(np.where(u[i] >= top - ARGMAX_GAP)[0].tolist())
        if len(cand) > 1:
            out[int(i)] = (int(O.argmax_lowest(u[i:i + 1])[0]), cand)
    return out


def retarget_ties(prob, rows, ref, ties, gpu_y, W64=None):
    """Oracle values with the hard label of each near-tie row set to the GPU's
    choice, after checking that the choice is one of the tied candidates.

    The expected values stay the oracle's: for a row whose ce label moves from
    y to c, the ce term becomes lse_q - z_c (the oracle's ce of that row with
    label c), the weighted loss moves by w_ce times the difference, and the
    row's logit gradient by seed * w_ce * (e_y - e_c).  Returns the adjusted
    (loss, ce term) arrays and a list of (position, y, c) for the gradients.
    """
    loss, term = ref.loss.copy(), ref.terms["ce"].copy()
    moved = []
    if not ties:
        return loss, term, moved
    W = W64 if W64 is not None else O.widen(prob.W, prob.dtype)
    w = float(prob.weights["ce"])
    for i, (y, cand) in ties.items():
        c = int(gpu_y[i])
        assert c in cand, f"row {rows[i]}: label {c} is not among the tied labels {sorted(cand)}"
        if c == y:
            continue
        z = O.widen(prob.hidden[rows[i]:rows[i] + 1], prob.dtype) @ W.T
        alt, _ = O.ce_from_logits(z, np.array([c]))
        loss[i] += w * (alt[0] - term[i])
        term[i] = alt[0]
        moved.append((i, y, c))
    return loss, term, moved


def apply_moved_labels(prob, rows, moved, seed, rdh=None, rdW=None, dW_rows=None, W64=None):
    """Shift oracle gradients for the rows whose ce label moved (see retarget_ties):
    dh_r += seed_r w_ce (W[y] - W[c]); dW[y] += seed_r w_ce h_r, dW[c] -= seed_r w_ce h_r."""
    if not moved:
        return rdh, rdW
    W = W64 if W64 is not None else O.widen(prob.W, prob.dtype)
    w = float(prob.weights["ce"])
    vpos = None if dW_rows is None else {int(v): j for j, v in enumerate(dW_rows)}
    for i, y, c in moved:
        r = rows[i]
        s = float(seed[r]) * w
        if rdh is not None:
            rdh[i] += s * (W[y] - W[c])
        if rdW is not None:
            h = O.widen(prob.hidden[r:r + 1], prob.dtype)[0]
            for v, sign in ((y, 1.0), (c, -1.0)):
                j = v if vpos is None else vpos.get(v)
                if j is not None:
                    rdW[j] += sign * s * h
    return rdh, rdW


def full_parity(prob, *, max_chunk_rows=0, check_grads=True, tag="", single_call=False,
                shards=None, workspace_bytes=None, expect_copies=None, flags=None,
                expect_kernels=None):
    """Run fwd (+bwd with the mean seed) on the GPU and compare every output with the oracle.

    single_call: use lmhead_loss_fwd_bwd instead of the two calls.
    shards: (G, bounds or None) to run the vocabulary-parallel sequence instead.
    workspace_bytes: workspace to give the calls (default: the library's size).
    expect_copies: if not None, the backward layout the trace must show: True
    or "copies" (W^T and h^T copies), "no_weight_copy" (h^T only), False or
    "no_copies" (no transpose).
    flags: backward layout flags; by default the transposed copies are forced
    (FLAG_COPIES) so chunked cases exercise that path, except when
    workspace_bytes is given (then the library chooses).
    expect_kernels: (present, absent) kernel names the trace of the calls must
    and must not show.
    """
    if flags is None:
        flags = 0 if workspace_bytes is not None else L.binding.FLAG_COPIES
    say(f"[parity] {tag} {prob.name} N={prob.n_rows} H={prob.hidden_dim} V={prob.vocab} "
        f"dtype={prob.dtype} weights={prob.weights} chunk={max_chunk_rows} single={single_call} "
        f"shards={shards}")
    dev = to_device(prob)
    if shards:
        run = ShardedLossRun(dev["hidden"], dev["W"], prob.weights, shards[0],
                             labels=dev["labels"], mask=dev["mask"],
                             target_hidden=dev["target_hidden"], W_t=dev["W_t"],
                             target_row=dev["target_row"], max_chunk_rows=max_chunk_rows,
                             bounds=shards[1], flags=flags, heads=prob.shifts)
    else:
        run = make_run(prob, dev, max_chunk_rows=max_chunk_rows, workspace_bytes=workspace_bytes,
                       flags=flags)
    trace = None
    if expect_copies is not None or expect_kernels is not None:
        trace = L.binding.Trace(capacity=4096)
        trace.attach(run.problem)
    gm = torch.ones(1, dtype=torch.float32, device="cuda")
    if single_call:
        dh_t, dW_t = run.forward_backward(grad_mean=gm)
    else:
        run.forward()
    torch.cuda.synchronize()
    ref = O.forward(prob)
    mean, term_means, n_valid = O.mean_loss(prob)
    counts = run.counts.cpu().numpy()
    assert counts[0] == ref.n_valid and counts[1] == ref.n_bad
    loss = run.loss.cpu().numpy()
    all_rows = np.arange(prob.n_rows)
    ties = ce_tie_candidates(prob, all_rows, ref.valid)
    moved = []
    if ties:
        gpu_y = run.saved_field(3, torch.int32).cpu().numpy()
        ref_loss, ref_ce, moved = retarget_ties(prob, all_rows, ref, ties, gpu_y)
        ref.loss, ref.terms["ce"] = ref_loss, ref_ce
        mean = float(np.sum(ref.loss) / max(ref.n_valid, 1))
        term_means["ce"] = float(np.sum(ref.terms["ce"]) / max(ref.n_valid, 1))
        say(f"   {len(ties)} near-tie ce rows, {len(moved)} with the other label")
    check_tokens(loss, ref.loss, "per-token loss")
    assert np.all(loss[~ref.valid] == 0.0), "masked rows must contribute exactly 0"
    red = run.reduced.cpu().numpy()
    assert abs(red[0] - mean) <= LOSS_RTOL * abs(mean) + TOKEN_ATOL, (red[0], mean)
    for k, v in term_means.items():
        got = red[1 + L.KINDS.index(k)]
        assert abs(got - v) <= LOSS_RTOL * abs(v) + TOKEN_ATOL, (k, got, v)
        check_tokens(run.term[L.KINDS.index(k)].cpu().numpy(), ref.terms[k], f"term {k}")
    lse = run.lse_q.cpu().numpy()
    assert np.allclose(lse[ref.valid], ref.lse_q[ref.valid], rtol=1e-5, atol=1e-4)
    if ref.alpha is not None and any(k in ("tv", "nla", "lk_hybrid", "jsd")
                                     for k in prob.weights):
        alpha = run.saved_field(4).cpu().numpy()
        assert np.allclose(alpha[ref.valid], ref.alpha[ref.valid], atol=1e-4)
    elif any(k in ("kl_div", "rkl") for k in prob.weights):
        # only the Kullback-Leibler divergences: no sum of min(p, q) is formed
        assert np.all(run.saved_field(4).cpu().numpy()[ref.valid] == 1.0)
    if "ce" in prob.weights:
        y = run.saved_field(3, torch.int32).cpu().numpy()
        check_argmax(y, prob, np.arange(prob.n_rows), ref.valid)
    if ref.flat is not None:
        check_flatness(run.flatness.cpu().numpy(), ref.flat, ref.valid)
    out = dict(run=run, ref=ref, loss=loss)
    if check_grads or single_call:
        if single_call:
            dh, dW = dh_t, dW_t
        else:
            dh, dW = run.backward(grad_mean=gm)
        torch.cuda.synchronize()
        rdh, rdW = O.backward(prob)
        rdh, rdW = apply_moved_labels(prob, all_rows, moved, O.mean_seed(prob), rdh, rdW)
        dh_np, dW_np = dh.cpu().numpy(), dW.cpu().numpy()
        e_dh, e_dW = rel_frob(dh_np, rdh), rel_frob(dW_np, rdW)
        say(f"   rel frob dh {e_dh:.3e} dW {e_dW:.3e}")
        assert e_dh <= GRAD_FROB and e_dW <= GRAD_FROB
        assert np.all(dh_np[~ref.valid] == 0.0), "masked rows must get a zero gradient"
        out.update(dh=dh_np, dW=dW_np, rdh=rdh, rdW=rdW)
    if trace is not None:
        out["trace"] = trace.read()
        names = {name for name, _, _ in out["trace"]}
        run.problem.trace = None
        trace.close()
        if expect_kernels is not None:
            present, absent = expect_kernels
            assert set(present) <= names and not (set(absent) & names), names
        if expect_copies is not None:
            lay = {True: "copies", False: "no_copies"}.get(expect_copies, expect_copies)
            want_wt, want_ht = {"copies": (True, True), "no_weight_copy": (False, True),
                                "no_copies": (False, False)}[lay]
            assert "gemm_dh" in names or "gemm_dh_dzt" in names, names
            assert (("transpose_W" in names) == want_wt
                    and ("transpose_h" in names) == want_ht), names
    return out
