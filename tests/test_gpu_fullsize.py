"""Parity at each workload's full size, in the launch configuration bench.py times
(the library's default workspace: its streaming chunk policy and layout).

The oracle cannot materialise every row's logits at these sizes, so:
  * the default workspace stays below the size of the [N, V] bf16 logits
    (blog, "Backward pass": the streaming loss never holds the full logits);
  * forward: per-row outputs of a seeded sample of rows (plus the first, the
    last and the rows around each chunk boundary of the calls) are compared
    with the oracle one by one; counts are compared over all rows;
  * backward with the mean seed (the benchmark's call): dh of the sampled rows
    against the oracle, and the invariant sum_v dW[v, :] = 0 over the whole
    matrix (every loss here is a function of softmax(z), whose gradient sums
    to zero over the vocabulary);
  * backward with the seed set only on the sampled rows: dh of those rows, dh
    exactly 0 elsewhere, and dW on a vocabulary subset (the sampled rows'
    labels plus seeded rows) against the oracle, which then sums exactly the
    same contributions.
"""
import numpy as np
import pytest
import torch

import synthetic
from oracle import specloss_oracle as O
import lm_head_vocab_amd as L
from lm_head_vocab_amd.memory import logits_sized_limit_bytes
from tests._gpu_helpers import (ARGMAX_GAP, GRAD_FROB, apply_moved_labels, ce_tie_candidates,
                                check_flatness, check_tokens, make_run, rel_frob,
                                retarget_ties, say, to_device)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N_SAMPLE = 96     # seeded rows per case, besides the first, last and chunk-boundary rows
N_DW_ROWS = 4096  # seeded vocabulary rows of the sampled-seed dW check


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_vocab_amd as L
    L.load_library()
    yield


def _sample_rows(n, seed, chunks):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(N_SAMPLE, n), replace=False).tolist())
    rows |= {0, n - 1}
    for c in chunks:
        for b in range(c, n, c):
            rows |= {b - 1, b}
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name,single", [("ce_bf16_1b", False), ("ce_bf16_8b", False),
                                         ("lk_hybrid_bf16_8b", False),
                                         ("multihead_bf16_405b", False),
                                         ("ce_bf16_1b", True), ("ce_bf16_8b", True),
                                         ("lk_hybrid_bf16_8b", True),
                                         ("multihead_bf16_405b", True),
                                         ("lk_hybrid_bf16_8b:kl_div", False),
                                         ("lk_hybrid_bf16_8b:rkl", True),
                                         ("lk_hybrid_bf16_8b:jsd", True)])
def test_full_size_sampled(name, single):
    """single: the same checks through the single call lmhead_loss_fwd_bwd.
    name:kind runs the workload's inputs with that loss kind alone (kl_div's
    two-call forward takes one sweep; rkl and jsd stage log q - log p)."""
    name, _, kind = name.partition(":")
    prob = synthetic.make_problem(name, weights={kind: 1.0} if kind else None)
    N, H, V = prob.n_rows, prob.hidden_dim, prob.vocab
    say(f"[fullsize] {name} N={N} H={H} V={V} weights={prob.weights} single={single}")
    dev = to_device(prob)
    run = make_run(prob, dev, flags=None)  # the default workspace, as bench.py
    limit = logits_sized_limit_bytes(N, V)
    assert run.workspace_bytes < limit, (run.workspace_bytes / 2**30, limit / 2**30)
    chunks = {run.chunk(c)[0] for c in (L.binding.CALL_FWD, L.binding.CALL_BWD,
                                        L.binding.CALL_FWD_BWD)}
    say(f"   workspace {run.workspace_bytes / 2**30:.2f} GiB (logits {limit / 2**30:.2f} GiB), "
        f"chunks {sorted(chunks)}, single-call layout {run.chunk()[1]}")
    if single:
        dh, dW = run.forward_backward(grad_mean=torch.ones(1, device="cuda"))
    else:
        run.forward()
    torch.cuda.synchronize()
    op = O.OracleProblem.of(prob)
    valid, bad = O.row_validity(op)
    counts = run.counts.cpu().numpy()
    assert counts[0] == int(valid.sum()) and counts[1] == int(bad.sum())

    rows = _sample_rows(N, prob.seed, chunks)
    w64 = O._weights64(op)
    say(f"   oracle forward on {len(rows)} rows")
    ref = O.forward(op, rows=rows, weights64=w64)
    ties = ce_tie_candidates(prob, rows, ref.valid, None if w64[1] is None else w64[1])
    moved = []
    if ties:
        gpu_y = run.saved_field(3, torch.int32).cpu().numpy()[rows]
        ref.loss, ref.terms["ce"], moved = retarget_ties(prob, rows, ref, ties, gpu_y, w64[0])
        say(f"   {len(ties)} near-tie ce rows, {len(moved)} with the other label")
    loss = run.loss.cpu().numpy()[rows]
    check_tokens(loss, ref.loss, "sampled loss")
    assert np.all(loss[~ref.valid] == 0)
    lse = run.lse_q.cpu().numpy()[rows]
    assert np.allclose(lse[ref.valid], ref.lse_q[ref.valid], rtol=1e-5, atol=1e-4)
    for k in prob.weights:
        got = run.term[L.KINDS.index(k)].cpu().numpy()[rows]
        check_tokens(got, ref.terms[k], f"term {k}")
    if ref.alpha is not None and any(k in ("tv", "nla", "lk_hybrid", "jsd") for k in prob.weights):
        alpha = run.saved_field(4).cpu().numpy()[rows]
        assert np.allclose(alpha[ref.valid], ref.alpha[ref.valid], atol=1e-4)
    if ref.flat is not None:
        check_flatness(run.flatness.cpu().numpy()[rows], ref.flat, ref.valid)
    if "ce" in prob.weights:
        y = run.saved_field(3, torch.int32).cpu().numpy()[rows]
        tr = rows if prob.target_row is None else prob.target_row[rows]
        g = O.widen(prob.target_hidden[np.where(ref.valid, tr, 0)], prob.dtype)
        u = g @ w64[1].T
        top2 = np.sort(u, axis=1)[:, -2:]
        decisive = (top2[:, 1] - top2[:, 0] >= ARGMAX_GAP) & ref.valid
        assert np.array_equal(y[decisive], O.argmax_lowest(u)[decisive])

    # backward with the mean seed, as the benchmark calls it
    say("   backward, mean seed")
    if not single:
        dh, dW = run.backward(grad_mean=torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    seed_mean = O.mean_seed(op)
    rdh, _ = O.backward(op, seed=seed_mean, rows=rows, want_dW=False, weights64=w64)
    rdh, _ = apply_moved_labels(prob, rows, moved, seed_mean, rdh, None, W64=w64[0])
    dh_s = dh[torch.from_numpy(rows).cuda()].cpu().numpy()
    e = rel_frob(dh_s, rdh)
    say(f"   mean seed: sampled dh rel frob {e:.3e}")
    assert e <= GRAD_FROB
    colsum = dW.sum(dim=0)
    ratio = float(colsum.norm() / dW.norm())
    say(f"   mean seed: |sum_v dW[v,:]| / |dW| = {ratio:.3e}")
    assert ratio < 0.05
    masked = torch.from_numpy(~valid).cuda()
    assert torch.all(dh[masked] == 0)
    del dh, dW

    # backward with the seed only on the sampled rows
    say("   backward, sampled seed")
    seed = np.zeros(N)
    seed[rows] = np.random.default_rng(7).uniform(0.5, 1.5, len(rows))
    seed = np.where(valid, seed, 0.0)
    g = torch.tensor(seed, dtype=torch.float32, device="cuda")
    dh, dW = run.forward_backward(grad_loss=g) if single else run.backward(grad_loss=g)
    torch.cuda.synchronize()
    vsel = set(np.random.default_rng(11).choice(V, min(N_DW_ROWS, V), replace=False).tolist())
    if prob.labels is not None:
        vsel |= {int(x) for x in prob.labels[rows] if 0 <= x < V}
    if "ce" in prob.weights:
        vsel |= {int(x) for x in run.saved_field(3, torch.int32).cpu().numpy()[rows] if x >= 0}
    vsel = np.array(sorted(vsel), dtype=np.int64)
    rdh, rdW = O.backward(op, seed=seed, rows=rows, dW_rows=vsel, weights64=w64)
    rdh, rdW = apply_moved_labels(prob, rows, moved, seed, rdh, rdW, dW_rows=vsel, W64=w64[0])
    e_dh = rel_frob(dh[torch.from_numpy(rows).cuda()].cpu().numpy(), rdh)
    e_dW = rel_frob(dW[torch.from_numpy(vsel).cuda()].cpu().numpy(), rdW)
    say(f"   sampled seed: dh rel frob {e_dh:.3e}, dW[{len(vsel)} rows] rel frob {e_dW:.3e}")
    assert e_dh <= GRAD_FROB and e_dW <= GRAD_FROB
    others = torch.ones(N, dtype=torch.bool, device="cuda")
    others[torch.from_numpy(rows).cuda()] = False
    assert torch.all(dh[others] == 0)
