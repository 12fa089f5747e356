"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a closed form, a library
routine (torch CPU fp64, scipy), central finite differences, an identity or
a printed value of the pages.  A plausible slip in the oracle (a dropped term,
a wrong sign, a swapped p/q, a transposed operand) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.spatial.distance as ssd
import scipy.special as ssp
import scipy.stats as sst
import torch

import synthetic
from oracle import specloss_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DIV_KINDS = ("kl_div", "rkl", "jsd", "tv", "nla", "lk_hybrid")


def _tiny(kinds, seed=0, N=3, H=5, V=7, mask=None, target=True, labels=True, scale=1.0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, H)) * scale
    W = rng.standard_normal((V, H)) * scale
    prob = O.OracleProblem(dtype="f64", vocab=V, hidden=h, W=W, weights=dict(kinds))
    if labels:
        prob.labels = rng.integers(0, V, size=N).astype(np.int32)
    if target:
        prob.target_hidden = rng.standard_normal((N, H)) * scale
        prob.W_t = rng.standard_normal((V, H)) * scale
    prob.mask = mask
    return prob


def _logprobs(rng, B, V, scale=1.0):
    z = rng.standard_normal((B, V)) * scale
    u = rng.standard_normal((B, V)) * scale
    return ssp.log_softmax(u, axis=1), ssp.log_softmax(z, axis=1), u, z


# --------------------------------------------------------------------------- P-a
def test_ce_all_equal_logits_is_log_v():
    """Closed form: with W = 0 every logit is 0, so CE = log V and dz = 1/V - e_y."""
    V, H, N = 4096, 256, 16
    rng = np.random.default_rng(1)
    prob = O.OracleProblem(dtype="f32", vocab=V, hidden=rng.standard_normal((N, H)).astype(np.float32),
                           W=np.zeros((V, H), np.float32), weights={"ce_label": 1.0},
                           labels=rng.integers(0, V, N).astype(np.int32))
    r = O.forward(prob, want_dz=True)
    assert np.allclose(r.loss, math.log(V), rtol=0, atol=1e-12)
    assert abs(math.log(4096) - 8.317766166719343) < 1e-15
    expect = np.full((N, V), 1.0 / V)
    expect[np.arange(N), prob.labels] -= 1.0
    assert np.allclose(r.dz, expect, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------- P-b
def _fd_check(prob, seed_vec, eps=1e-6, rtol=1e-6):
    """Central differences of sum_t seed_t L_t w.r.t. every h and W entry."""

    def total(p):
        return float(np.sum(seed_vec * O.forward(p).loss))

    dh, dW = O.backward(prob, seed=seed_vec)
    num_h = np.zeros_like(prob.hidden)
    for idx in np.ndindex(*prob.hidden.shape):
        hp, hm = prob.hidden.copy(), prob.hidden.copy()
        hp[idx] += eps
        hm[idx] -= eps
        a = total(O.OracleProblem(**{**prob.__dict__, "hidden": hp}))
        b = total(O.OracleProblem(**{**prob.__dict__, "hidden": hm}))
        num_h[idx] = (a - b) / (2 * eps)
    num_W = np.zeros_like(prob.W)
    for idx in np.ndindex(*prob.W.shape):
        Wp, Wm = prob.W.copy(), prob.W.copy()
        Wp[idx] += eps
        Wm[idx] -= eps
        a = total(O.OracleProblem(**{**prob.__dict__, "W": Wp}))
        b = total(O.OracleProblem(**{**prob.__dict__, "W": Wm}))
        num_W[idx] = (a - b) / (2 * eps)
    scale_h = max(1e-12, np.max(np.abs(num_h)))
    scale_W = max(1e-12, np.max(np.abs(num_W)))
    assert np.max(np.abs(dh - num_h)) / scale_h < rtol, (dh, num_h)
    assert np.max(np.abs(dW - num_W)) / scale_W < rtol, (dW, num_W)


@pytest.mark.parametrize("kind", ["ce_label", "ce", "kl_div", "rkl", "jsd", "tv", "nla"])
def test_finite_differences(kind):
    """Brute force on N=3, H=5, V=7: oracle dh, dW == central differences of its loss."""
    prob = _tiny({kind: 1.0}, seed=hash(kind) % 1000)
    rng = np.random.default_rng(7)
    seed_vec = rng.uniform(0.2, 1.0, size=prob.n_rows)
    _fd_check(prob, seed_vec)


def test_finite_differences_weighted_mix_with_mask():
    """Weighted sum of every kind except lk_hybrid, with one masked row."""
    kinds = {"ce_label": 0.3, "ce": 0.2, "kl_div": 0.5, "rkl": 0.7, "jsd": 1.1, "tv": 0.9, "nla": 0.4}
    prob = _tiny(kinds, seed=11, N=4, mask=np.array([1, 0, 1, 1], np.uint8))
    _fd_check(prob, O.mean_seed(prob))


def test_finite_differences_lk_hybrid_lambda_detached():
    """lk_hybrid's gradient equals the derivative of lam0*KL + (1-lam0)*TV, lam0 fixed."""
    prob = _tiny({"lk_hybrid": 1.0}, seed=5)
    base = O.forward(prob)
    lam0 = np.exp(-3.0 * base.alpha)
    eps = 1e-6
    seed_vec = np.array([0.3, 0.5, 0.9])

    def total(p):
        r_kl = O.forward(O.OracleProblem(**{**p.__dict__, "weights": {"kl_div": 1.0}}))
        r_tv = O.forward(O.OracleProblem(**{**p.__dict__, "weights": {"tv": 1.0}}))
        return float(np.sum(seed_vec * (lam0 * r_kl.loss + (1 - lam0) * r_tv.loss)))

    dh, dW = O.backward(prob, seed=seed_vec)
    for arr_name, grad in (("hidden", dh), ("W", dW)):
        arr = getattr(prob, arr_name)
        num = np.zeros_like(arr)
        for idx in np.ndindex(*arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            num[idx] = (total(O.OracleProblem(**{**prob.__dict__, arr_name: ap})) -
                        total(O.OracleProblem(**{**prob.__dict__, arr_name: am}))) / (2 * eps)
        assert np.max(np.abs(grad - num)) / np.max(np.abs(num)) < 1e-6
    # and the full (non-detached) derivative differs: lambda really is held fixed
    r = O.forward(prob)
    assert np.allclose(r.loss, lam0 * O.forward(O.OracleProblem(**{**prob.__dict__, "weights": {"kl_div": 1.0}})).loss
                       + (1 - lam0) * (1 - base.alpha), rtol=1e-13)


# --------------------------------------------------------------------------- P-c
def test_identical_distributions_zero_divergence():
    """p == q (W_t = W, g = h): every divergence is 0, alpha = 1, lambda = e^-3, dz = 0."""
    rng = np.random.default_rng(3)
    N, H, V = 5, 16, 50
    h = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H))
    for k in DIV_KINDS:
        prob = O.OracleProblem(dtype="f64", vocab=V, hidden=h, W=W, weights={k: 1.0},
                               target_hidden=h.copy(), W_t=W.copy())
        r = O.forward(prob, want_dz=True)
        assert np.allclose(r.alpha, 1.0, atol=1e-14)
        assert np.allclose(r.loss, 0.0, atol=1e-14), k
        assert np.allclose(r.dz, 0.0, atol=1e-15), k
    lp = np.log(np.full((1, 4), 0.25))
    lam = np.exp(-3.0 * O.overlap(lp, lp))
    assert abs(lam[0] - math.exp(-3.0)) < 1e-15


# --------------------------------------------------------------------------- P-d
def test_tv_equals_half_l1():
    """Identity: 1 - sum min(p,q) = 1/2 sum |p - q|, computed from scipy softmax."""
    rng = np.random.default_rng(4)
    logp, logq, u, z = _logprobs(rng, 20, 300, scale=2.0)
    tv, _ = O.total_variation(logp, logq)
    p, q = ssp.softmax(u, axis=1), ssp.softmax(z, axis=1)
    assert np.allclose(tv, 0.5 * np.abs(p - q).sum(axis=1), rtol=1e-13, atol=1e-15)
    nla, _ = O.neg_log_acceptance(logp, logq)
    assert np.allclose(nla, -np.log1p(-0.5 * np.abs(p - q).sum(axis=1)), rtol=1e-12)


# --------------------------------------------------------------------------- P-e
def test_jsd_bounds_and_scipy():
    """0 <= JSD <= ln 2; equals scipy's jensenshannon distance squared (natural log)."""
    rng = np.random.default_rng(5)
    logp, logq, u, z = _logprobs(rng, 16, 200, scale=3.0)
    jsd, _ = O.jensen_shannon(logp, logq)
    assert np.all(jsd >= 0) and np.all(jsd <= math.log(2))
    p, q = ssp.softmax(u, axis=1), ssp.softmax(z, axis=1)
    ref = np.array([ssd.jensenshannon(p[i], q[i]) ** 2 for i in range(16)])
    assert np.allclose(jsd, ref, rtol=1e-9, atol=1e-14)


def test_near_disjoint_supports():
    """u_0 = z_1 = +60: JSD -> ln 2, alpha -> 0, TV -> 1 (limits of the definitions)."""
    V = 64
    u = np.zeros((1, V)); u[0, 0] = 60.0
    z = np.zeros((1, V)); z[0, 1] = 60.0
    logp, logq = ssp.log_softmax(u, axis=1), ssp.log_softmax(z, axis=1)
    jsd, _ = O.jensen_shannon(logp, logq)
    tv, _ = O.total_variation(logp, logq)
    assert abs(jsd[0] - math.log(2)) < 1e-12
    assert tv[0] >= 1 - 1e-24 * V and O.overlap(logp, logq)[0] < 1e-24 * V


# --------------------------------------------------------------------------- P-f
def test_kl_rkl_gibbs_swap_and_scipy():
    """KL, rKL >= 0; KL(p||q) == scipy entropy(p, q); swapping p and q maps kl to rkl."""
    rng = np.random.default_rng(6)
    logp, logq, u, z = _logprobs(rng, 12, 100, scale=2.0)
    kl, _ = O.kl_forward(logp, logq)
    rkl, _ = O.kl_reverse(logp, logq)
    p, q = ssp.softmax(u, axis=1), ssp.softmax(z, axis=1)
    assert np.all(kl >= 0) and np.all(rkl >= 0)
    assert np.allclose(kl, [sst.entropy(p[i], q[i]) for i in range(12)], rtol=1e-11)
    assert np.allclose(rkl, [sst.entropy(q[i], p[i]) for i in range(12)], rtol=1e-11)
    kl_sw, _ = O.kl_forward(logq, logp)
    assert np.allclose(kl_sw, rkl, rtol=1e-13)


def test_worked_distributions_golden():
    """Hand-worked values on explicit three-entry distributions (tests/golden)."""
    with open(os.path.join(GOLDEN, "divergence_worked_example.json")) as f:
        g = json.load(f)
    logp = np.log(np.array([g["p"]]))
    logq = np.log(np.array([g["q"]]))
    env = {"ln": math.log, "exp": math.exp, "min": min, "abs": abs, "__builtins__": {}}
    e = {k: eval(v, env) for k, v in g["expected_expr"].items()}  # closed forms, by hand
    assert abs(O.overlap(logp, logq)[0] - e["alpha"]) < 1e-15
    assert abs(O.total_variation(logp, logq)[0][0] - e["tv"]) < 1e-15
    assert abs(O.neg_log_acceptance(logp, logq)[0][0] - e["nla"]) < 1e-14
    assert abs(O.kl_forward(logp, logq)[0][0] - e["kl_div"]) < 1e-14
    assert abs(O.kl_reverse(logp, logq)[0][0] - e["rkl"]) < 1e-14
    assert abs(O.jensen_shannon(logp, logq)[0][0] - e["jsd"]) < 1e-14
    assert abs(O.lk_hybrid(logp, logq)[0][0] - e["lk_hybrid"]) < 1e-14


# --------------------------------------------------------------------------- P-g
def test_torch_cpu_fp64_ce_and_autograd():
    """torch CPU fp64 cross_entropy(sum, ignore_index=-100) + autograd == oracle."""
    p = synthetic.make_problem("ce_fp32_small", n_rows=96, hidden_dim=64, vocab=500)
    r = O.forward(p)
    h = torch.tensor(O.widen(p.hidden, "f32"), requires_grad=True)
    W = torch.tensor(O.widen(p.W, "f32"), requires_grad=True)
    y = torch.tensor(p.labels.astype(np.int64))
    loss_sum = torch.nn.functional.cross_entropy(h @ W.T, y, reduction="sum", ignore_index=-100)
    assert abs(loss_sum.item() - r.loss.sum()) / abs(loss_sum.item()) < 1e-12
    n_valid = int((p.labels != -100).sum())
    assert r.n_valid == n_valid
    (loss_sum / n_valid).backward()
    dh, dW = O.backward(p)
    assert np.allclose(dh, h.grad.numpy(), rtol=1e-10, atol=1e-15)
    assert np.allclose(dW, W.grad.numpy(), rtol=1e-10, atol=1e-15)


def _torch_div(kind, logp_t, logq_t):
    p, q = logp_t.exp(), logq_t.exp()
    if kind == "kl_div":  # torch's kl_div(input=log q, target=log p) = sum p (log p - log q)
        return torch.nn.functional.kl_div(logq_t, logp_t, reduction="none", log_target=True).sum(1)
    if kind == "rkl":
        return torch.nn.functional.kl_div(logp_t, logq_t, reduction="none", log_target=True).sum(1)
    if kind == "jsd":
        logm = torch.log((p + q) / 2)
        return 0.5 * torch.nn.functional.kl_div(logm, logp_t, reduction="none", log_target=True).sum(1) + \
            0.5 * torch.nn.functional.kl_div(logm, logq_t, reduction="none", log_target=True).sum(1)
    if kind == "tv":
        return 0.5 * (p - q).abs().sum(1)
    if kind == "nla":
        return -torch.log1p(-0.5 * (p - q).abs().sum(1))
    raise KeyError(kind)


@pytest.mark.parametrize("kind", ["kl_div", "rkl", "jsd", "tv", "nla"])
def test_torch_autograd_divergences(kind):
    """Library route: torch kl_div / L1 forms in fp64 and autograd through log_softmax."""
    rng = np.random.default_rng(8)
    B, V = 6, 40
    u = torch.tensor(rng.standard_normal((B, V)))
    z = torch.tensor(rng.standard_normal((B, V)), requires_grad=True)
    logp_t = torch.log_softmax(u, 1)
    logq_t = torch.log_softmax(z, 1)
    ref = _torch_div(kind, logp_t, logq_t)
    ref.sum().backward()
    loss, dz = O.DIVERGENCES[kind](logp_t.numpy(), logq_t.detach().numpy())
    assert np.allclose(loss, ref.detach().numpy(), rtol=1e-11, atol=1e-15)
    assert np.allclose(dz, z.grad.numpy(), rtol=1e-9, atol=1e-14)


def test_torch_autograd_kl_through_lm_head():
    """KL(p||q) through both projections: torch fp64 autograd gives the same dh, dW."""
    prob = _tiny({"kl_div": 1.0}, seed=9, N=6, H=8, V=30)
    h = torch.tensor(prob.hidden, requires_grad=True)
    W = torch.tensor(prob.W, requires_grad=True)
    logq = torch.log_softmax(h @ W.T, 1)
    logp = torch.log_softmax(torch.tensor(prob.target_hidden) @ torch.tensor(prob.W_t).T, 1)
    L = torch.nn.functional.kl_div(logq, logp, reduction="sum", log_target=True) / prob.n_rows
    L.backward()
    dh, dW = O.backward(prob)
    assert abs(O.mean_loss(prob)[0] - L.item()) < 1e-12
    assert np.allclose(dh, h.grad.numpy(), rtol=1e-10, atol=1e-15)
    assert np.allclose(dW, W.grad.numpy(), rtol=1e-10, atol=1e-15)


def test_argmax_ties_lowest_index():
    u = np.array([[0.0, 3.0, 1.0, 3.0], [2.0, 2.0, 2.0, 2.0]])
    assert list(O.argmax_lowest(u)) == [1, 0]


# --------------------------------------------------------------------------- P-h
def test_block_size_invariance_and_uneven_mask():
    """Streaming == dense up to rounding for any chunking; normalise by valid tokens."""
    p = synthetic.make_problem("ce_bf16_1b", n_rows=200, hidden_dim=64, vocab=700)
    p.mask = np.ones(200, np.uint8)
    p.mask[:60] = 0  # every masked row sits in the first chunks
    ref = O.forward(p, block=200)
    for b in (1, 7, 64):
        r = O.forward(p, block=b)
        assert np.allclose(r.loss, ref.loss, rtol=1e-13, atol=0)
    mean, _, n = O.mean_loss(p)
    assert n == 140
    chunk = 50
    chunk_sums = [ref.loss[i:i + chunk].sum() for i in range(0, 200, chunk)]
    chunk_valid = [int(p.mask[i:i + chunk].sum()) for i in range(0, 200, chunk)]
    assert abs(sum(chunk_sums) / sum(chunk_valid) - mean) < 1e-13
    # the wrong normalisation (mean of chunk means) gives a different number
    means = [s / c for s, c in zip(chunk_sums, chunk_valid) if c]
    assert abs(np.mean(means) - mean) > 1e-4


def test_gradient_chunk_additivity():
    """dW over all rows == sum of dW over row chunks (gradient accumulation over chunks)."""
    p = synthetic.make_problem("ce_fp32_small", n_rows=40, hidden_dim=32, vocab=90)
    dh, dW = O.backward(p)
    acc = np.zeros_like(dW)
    for c0 in range(0, 40, 13):
        rows = np.arange(c0, min(40, c0 + 13))
        dh_c, dW_c = O.backward(p, rows=rows)
        assert np.allclose(dh_c, dh[rows], rtol=1e-13, atol=1e-18)
        acc += dW_c
    assert np.allclose(acc, dW, rtol=1e-12, atol=1e-18)


# --------------------------------------------------------------------------- P-i
def test_statistical_sanity():
    """Not parity: mean CE of unit-variance Gaussian logits ~ ln V + 1/2; alpha ~ 2 Phi(-d/2)."""
    p = synthetic.make_problem("ce_fp32_small")
    mean, _, _ = O.mean_loss(p)
    assert abs(mean - (math.log(4096) + 0.5)) < 0.05
    p4 = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=32, hidden_dim=1024, vocab=8192)
    r = O.forward(p4)
    delta = 0.005 * math.sqrt(1024)  # std of u - z = (W_t - W) h per logit
    assert abs(r.alpha.mean() - 2 * sst.norm.cdf(-delta / 2)) < 0.01


# --------------------------------------------------------------------------- P-k
def test_masked_rows_do_not_contribute():
    """Perturbing masked rows with finite values changes no loss, dW or unmasked dh."""
    p = synthetic.make_problem("multihead_bf16_405b", seq_len=24, hidden_dim=64, vocab=300)
    dh0, dW0 = O.backward(p)
    r0 = O.forward(p)
    masked = np.where(p.mask == 0)[0]
    assert len(masked) == 6
    p.hidden = p.hidden.copy()
    p.hidden[masked] = synthetic.f32_to_bf16_bits(np.full((6, 64), 7.5, np.float32))
    dh1, dW1 = O.backward(p)
    r1 = O.forward(p)
    assert np.array_equal(r0.loss, r1.loss)
    assert np.array_equal(dW0, dW1)
    assert np.array_equal(dh0[p.mask == 1], dh1[p.mask == 1])
    assert np.all(dh1[masked] == 0)


# --------------------------------------------------------------------------- alignment
def test_align_heads_hand_example_and_generator():
    """Targets shift per head before chunking; tails past the sequence are masked."""
    # token-major rows (t, k): t = 0 -> 1, 2; t = 1 -> 2, 3; ... t = 3 -> 4, tail
    tr, m = O.align_heads(5, (1, 2))
    assert list(tr) == [1, 2, 2, 3, 3, 4, 4, -1, -1, -1]
    assert list(m) == [1, 1, 1, 1, 1, 1, 1, 0, 0, 0]
    tr2, m2 = O.align_heads(3, (1,), batch=2, loss_mask=np.array([1, 1, 0, 1, 1, 1], np.uint8))
    assert list(tr2) == [1, -1, -1, 4, 5, -1]
    p = synthetic.make_problem("multihead_bf16_405b", seq_len=40, hidden_dim=64, vocab=128)
    tr3, m3 = O.align_heads(40, p.shifts)
    assert np.array_equal(tr3, p.target_row) and np.array_equal(m3, p.mask)


def test_validity_bad_rows():
    p = _tiny({"ce_label": 1.0}, N=5, target=False)
    p.labels = np.array([0, -100, 7, -3, 6], np.int32)
    p.mask = np.array([1, 1, 1, 0, 1], np.uint8)
    valid, bad = O.row_validity(p)
    assert list(valid) == [True, False, False, False, True]
    assert list(bad) == [False, False, True, False, False]


# --------------------------------------------------------------- flatness
def test_flatness_closed_forms():
    """Uniform p gives 1; a one-hot p gives 1/sqrt(V); two equal peaks give sqrt(2/V)."""
    V = 64
    uni = np.log(np.full((1, V), 1.0 / V))
    assert abs(O.flatness(uni)[0] - 1.0) < 1e-14
    onehot = np.full((1, V), -1e4)
    onehot[0, 3] = 0.0
    logp = ssp.log_softmax(onehot, axis=1)
    assert abs(O.flatness(logp)[0] - 1 / math.sqrt(V)) < 1e-12
    two = np.full((1, V), -1e4)
    two[0, [1, 9]] = 0.0
    assert abs(O.flatness(ssp.log_softmax(two, axis=1))[0] - math.sqrt(2 / V)) < 1e-12


def test_flatness_scipy_cosine():
    """Library route: scipy's cosine distance between p and the all-ones vector."""
    rng = np.random.default_rng(12)
    u = rng.standard_normal((5, 300)) * 2
    logp = ssp.log_softmax(u, axis=1)
    ref = [1 - ssd.cosine(np.exp(logp[i]), np.ones(300)) for i in range(5)]
    assert np.allclose(O.flatness(logp), ref, rtol=1e-12)


def test_tv_tie_rule_central_difference():
    """At exact ties the TV gradient is the central difference of the loss.

    p is q with two entries swapped, so every other entry ties bit for bit; the
    loss 1 - sum min(p, q(z)) has a kink there, and a central difference
    returns the mean of the two one-sided derivatives, i.e. the tie counted as
    1/2 (R5).  Counting ties as 0 or 1 gives a one-sided derivative instead.
    """
    rng = np.random.default_rng(13)
    V = 9
    z0 = rng.standard_normal(V)
    logq0 = ssp.log_softmax(z0)
    logp = logq0.copy()
    logp[[2, 6]] = logp[[6, 2]]
    _, dz = O.total_variation(logp[None, :], logq0[None, :])

    def tv(z):
        return 1.0 - np.minimum(np.exp(logp), np.exp(ssp.log_softmax(z))).sum()

    eps = 1e-6
    num = np.array([(tv(z0 + eps * np.eye(V)[j]) - tv(z0 - eps * np.eye(V)[j])) / (2 * eps)
                    for j in range(V)])
    assert np.count_nonzero(np.exp(logp) == np.exp(logq0)) == V - 2
    # O(eps) error: the second derivatives differ on the two sides of the kink
    assert np.allclose(dz[0], num, rtol=0, atol=1e-6), (dz[0], num)


# --------------------------------------------------------------- compositions
def _pair_problem(seed, N, H, V, weights, **kw):
    """Draft and target sides drawn independently (f64), so their argmaxes differ."""
    rng = np.random.default_rng(seed)
    return O.OracleProblem(dtype="f64", vocab=V, hidden=rng.standard_normal((N, H)),
                           W=rng.standard_normal((V, H)), weights=dict(weights),
                           target_hidden=rng.standard_normal((N, H)),
                           W_t=rng.standard_normal((V, H)), **kw)


def test_ce_label_is_argmax_of_target_logits():
    """"Available Losses", ce row: cross-entropy of the draft against argmax p.

    Library route: torch CPU fp64 cross_entropy of the draft logits h W^T against
    torch.argmax of the TARGET logits g W_t^T, and its autograd for dz, on rows
    where the draft's own argmax is a different index (so a label taken from
    the draft side fails).
    """
    prob = _pair_problem(21, N=12, H=16, V=40, weights={"ce": 1.0})
    r = O.forward(prob, want_dz=True)
    z = torch.tensor(prob.hidden) @ torch.tensor(prob.W).T
    u = torch.tensor(prob.target_hidden) @ torch.tensor(prob.W_t).T
    y = torch.argmax(u, dim=1)
    assert int((y != torch.argmax(z, dim=1)).sum()) >= prob.n_rows // 2
    assert np.array_equal(r.label, y.numpy())
    ref = torch.nn.functional.cross_entropy(z, y, reduction="none")
    assert np.allclose(r.terms["ce"], ref.numpy(), rtol=1e-12, atol=0)
    zg = z.clone().requires_grad_(True)
    torch.nn.functional.cross_entropy(zg, y, reduction="sum").backward()
    assert np.allclose(r.dz, zg.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_weighted_combination_unnormalised():
    """"Weighted Combinations": weights are used as given (not normalised) and each
    term is reported before its weight.

    {ce: 2, tv: 3}: torch CPU fp64 forms ce (cross_entropy against argmax u) and
    tv (half the L1 distance of the two softmaxes) independently; the oracle's
    per-row loss must be 2 ce + 3 tv exactly, its terms the unweighted ce and tv,
    and its dh, dW the autograd of the mean of 2 ce + 3 tv.
    """
    prob = _pair_problem(22, N=10, H=12, V=30, weights={"ce": 2.0, "tv": 3.0})
    r = O.forward(prob)
    h = torch.tensor(prob.hidden, requires_grad=True)
    W = torch.tensor(prob.W, requires_grad=True)
    z = h @ W.T
    u = torch.tensor(prob.target_hidden) @ torch.tensor(prob.W_t).T
    ce = torch.nn.functional.cross_entropy(z, torch.argmax(u, dim=1), reduction="none")
    tv = 0.5 * (torch.softmax(u, 1) - torch.softmax(z, 1)).abs().sum(1)
    assert np.allclose(r.terms["ce"], ce.detach().numpy(), rtol=1e-12, atol=0)
    assert np.allclose(r.terms["tv"], tv.detach().numpy(), rtol=1e-12, atol=0)
    assert np.allclose(r.loss, (2.0 * ce + 3.0 * tv).detach().numpy(), rtol=1e-12, atol=0)
    ((2.0 * ce + 3.0 * tv).sum() / prob.n_rows).backward()
    dh, dW = O.backward(prob)
    assert np.allclose(dh, h.grad.numpy(), rtol=1e-10, atol=1e-14)
    assert np.allclose(dW, W.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_target_rows_follow_the_head_shift():
    """Blog, "Correctness: alignment before chunking": head k at position t is paired
    with target position t + shift_k.

    Hand-built: target hidden g[t] = (t + 1) e_t and W_t = I, so the target
    logits of a row are t' + 1 at t' = its target position and 0 elsewhere.
    With shifts (1, 2) over 6 positions the valid rows' ce labels are, by hand,
    1..5 then 2..5, and lse_p = ln(e^(t'+1) + V - 1).
    """
    S, V = 6, 8
    g = np.zeros((S, V))
    for t in range(S):
        g[t, t] = t + 1.0
    target_row = np.array([1, 2, 3, 4, 5, -1, 2, 3, 4, 5, -1, -1], np.int32)
    mask = np.array([1, 1, 1, 1, 1, 0, 1, 1, 1, 1, 0, 0], np.uint8)
    rng = np.random.default_rng(23)
    prob = O.OracleProblem(dtype="f64", vocab=V, hidden=rng.standard_normal((12, V)),
                           W=rng.standard_normal((V, V)), weights={"ce": 1.0},
                           target_hidden=g, W_t=np.eye(V), target_row=target_row, mask=mask)
    r = O.forward(prob)
    valid = mask == 1
    expect = [1, 2, 3, 4, 5, 2, 3, 4, 5]
    assert list(r.label[valid]) == expect
    assert np.allclose(r.lse_p[valid], [math.log(math.exp(t + 1) + V - 1) for t in expect],
                       rtol=1e-14, atol=0)


def test_statistical_sanity_multihead_alpha():
    """Not parity: the three-head workload pairs draft h = g[t+k] with target row
    t+k, so u - z = (W_t - W) g has a per-logit std delta = 0.005 sqrt(H) and the
    mean alpha is about 2 Phi(-delta/2): 0.749 at H = 16384 (derived for large V,
    not on the pages).  A row map off by one pairs independent rows instead
    (alpha near 0.2)."""
    p = synthetic.make_problem("multihead_bf16_405b", seq_len=16, hidden_dim=16384, vocab=2048)
    r = O.forward(p)
    delta = 0.005 * math.sqrt(16384)
    expect = 2 * sst.norm.cdf(-delta / 2)
    assert abs(expect - 0.749) < 1e-3
    assert abs(r.alpha[r.valid].mean() - expect) < 0.015, r.alpha[r.valid].mean()
