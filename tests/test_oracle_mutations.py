"""The oracle's pins catch plausible slips in the oracle.

Each case plants one mistake in the oracle (on the CPU, by replacing one of
its functions for the duration of the test) and runs the pins that should
notice it; at least one of them must fail.  The mutated functions are copies
of the oracle's with the slip written in: a swapped p / q, a dropped term, a
wrong sign, a transposed reduction, an off-by-one, a missing normalisation.
"""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import specloss_oracle as O
from tests import test_oracle_pins as P

# the unmodified functions, for mutants that call through to them
_ORIG = {name: getattr(O, name) for name in ("kl_forward", "ce_from_logits", "total_variation",
                                            "align_heads", "row_validity")}


def _kl_swapped(logp, logq):
    return _ORIG["kl_forward"](logq, logp)


def _overlap_max(logp, logq):
    return np.sum(np.maximum(np.exp(logp), np.exp(logq)), axis=1)


def _ce_no_onehot(z, y):
    lse = O.logsumexp_rows(z)
    r = np.arange(z.shape[0])
    return lse - z[r, y], np.exp(z - lse[:, None])


def _ce_sign(z, y):
    loss, dz = _ORIG["ce_from_logits"](z, y)
    return -loss, dz


def _lse_columns(x):
    m = np.max(x, axis=0, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=0, keepdims=True)))[0]


def _tv_tie_one(logp, logq):
    p, q = np.exp(logp), np.exp(logq)
    alpha = np.sum(np.minimum(p, q), axis=1)
    c = np.where(q <= p, 1.0, 0.0)
    S = np.sum(q * c, axis=1, keepdims=True)
    return 1.0 - alpha, -q * (c - S)


def _tv_sign(logp, logq):
    loss, dz = _ORIG["total_variation"](logp, logq)
    return loss, -dz


def _rkl_no_mean(logp, logq):
    q = np.exp(logq)
    loss = np.sum(q * (logq - logp), axis=1)
    return loss, q * (logq - logp)


def _jsd_mixture_sum(logp, logq):
    p, q = np.exp(logp), np.exp(logq)
    logm = np.logaddexp(logp, logq)  # m = p + q, the 1/2 dropped
    loss = 0.5 * np.sum(p * (logp - logm), axis=1) + 0.5 * np.sum(q * (logq - logm), axis=1)
    g = 0.5 * (logq - logm)
    return loss, q * (g - np.sum(q * g, axis=1, keepdims=True))


def _nla_not_divided(logp, logq):
    tv_loss, tv_dz = O.total_variation(logp, logq)
    return -np.log(1.0 - tv_loss), tv_dz


def _lk_not_detached(logp, logq):
    kl, kl_dz = O.kl_forward(logp, logq)
    tv_loss, tv_dz = O.total_variation(logp, logq)
    alpha = 1.0 - tv_loss
    lam = np.exp(-3.0 * alpha)
    loss = lam * kl + (1.0 - lam) * tv_loss
    # d lam / dz = -3 lam d alpha / dz = 3 lam tv_dz: the term a detached lambda drops
    dlam = (3.0 * lam)[:, None] * tv_dz
    dz = lam[:, None] * kl_dz + (1.0 - lam)[:, None] * tv_dz + dlam * (kl - tv_loss)[:, None]
    return loss, dz


def _flatness_no_sqrt_v(logp):
    p = np.exp(logp)
    return p.sum(axis=1) / np.linalg.norm(p, axis=1)


def _argmax_highest(u):
    V = u.shape[1]
    return (V - 1 - np.argmax(u[:, ::-1], axis=1)).astype(np.int64)


def _align_off_by_one(seq_len, shifts, batch=1, loss_mask=None):
    return _ORIG["align_heads"](seq_len, [max(0, s - 1) for s in shifts], batch, loss_mask)


def _seed_unnormalised(prob):
    prob = prob if isinstance(prob, O.OracleProblem) else O.OracleProblem.of(prob)
    valid, _ = O.row_validity(prob)
    return np.where(valid, 1.0, 0.0)


def _validity_ignores_mask(prob):
    saved = prob.mask
    try:
        prob.mask = None
        return _ORIG["row_validity"](prob)
    finally:
        prob.mask = saved


def _rewrite(fn, *edits):
    """A copy of oracle function `fn` with each (old, new) source edit applied
    (the slip written into the oracle's own code), compiled in the oracle's
    namespace."""
    src = textwrap.dedent(inspect.getsource(fn))
    for old, new in edits:
        assert old in src, f"{fn.__name__} no longer contains {old!r}"
        src = src.replace(old, new)
    ns = dict(vars(O))
    exec(compile(src, f"<mutant of {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


# compositions inside the per-block forward, each slip planted in a copy of it
_block_ce_from_draft = _rewrite(O._block, ("y = argmax_lowest(u)", "y = argmax_lowest(z)"))
_block_normalised = _rewrite(
    O._block, ("loss += w * terms[k]", "loss += w / sum(act.values()) * terms[k]"),
    ("dz += w * dzs[k]", "dz += w / sum(act.values()) * dzs[k]"))
_target_rows_off_by_one = _rewrite(
    O._target_rows, ("tr = np.asarray(prob.target_row, dtype=np.int64)[idx]",
                     "tr = np.asarray(prob.target_row, dtype=np.int64)[idx] - 1"))


# (name, oracle attribute, replacement, whether DIVERGENCES holds it, pins that must notice)
MUTATIONS = [
    ("kl swaps p and q", "kl_forward", _kl_swapped, "kl_div",
     [P.test_kl_rkl_gibbs_swap_and_scipy, P.test_worked_distributions_golden]),
    ("alpha sums max instead of min", "overlap", _overlap_max, None,
     [P.test_worked_distributions_golden, P.test_identical_distributions_zero_divergence]),
    ("ce gradient drops the one-hot", "ce_from_logits", _ce_no_onehot, None,
     [P.test_ce_all_equal_logits_is_log_v, P.test_torch_cpu_fp64_ce_and_autograd]),
    ("ce loss with the wrong sign", "ce_from_logits", _ce_sign, None,
     [P.test_ce_all_equal_logits_is_log_v]),
    ("logsumexp over the token axis", "logsumexp_rows", _lse_columns, None,
     [P.test_ce_all_equal_logits_is_log_v, P.test_torch_cpu_fp64_ce_and_autograd]),
    ("tv counts ties as 1", "total_variation", _tv_tie_one, "tv",
     [P.test_tv_tie_rule_central_difference]),
    ("tv gradient with the wrong sign", "total_variation", _tv_sign, "tv",
     [lambda: P.test_torch_autograd_divergences("tv")]),
    ("rkl gradient drops the mean", "kl_reverse", _rkl_no_mean, "rkl",
     [lambda: P.test_torch_autograd_divergences("rkl")]),
    ("jsd mixture without the 1/2", "jensen_shannon", _jsd_mixture_sum, "jsd",
     [P.test_jsd_bounds_and_scipy, P.test_worked_distributions_golden]),
    ("nla gradient not divided by alpha", "neg_log_acceptance", _nla_not_divided, "nla",
     [lambda: P.test_torch_autograd_divergences("nla")]),
    ("lk_hybrid lambda not detached", "lk_hybrid", _lk_not_detached, "lk_hybrid",
     [P.test_finite_differences_lk_hybrid_lambda_detached]),
    ("flatness without sqrt(V)", "flatness", _flatness_no_sqrt_v, None,
     [P.test_flatness_closed_forms, P.test_flatness_scipy_cosine]),
    ("argmax keeps the highest tied index", "argmax_lowest", _argmax_highest, None,
     [P.test_argmax_ties_lowest_index]),
    ("head shift off by one", "align_heads", _align_off_by_one, None,
     [P.test_align_heads_hand_example_and_generator]),
    ("mean seed not divided by n_valid", "mean_seed", _seed_unnormalised, None,
     [P.test_torch_cpu_fp64_ce_and_autograd]),
    ("mask ignored", "row_validity", _validity_ignores_mask, None,
     [P.test_validity_bad_rows, P.test_masked_rows_do_not_contribute]),
    ("ce label taken from the draft logits", "_block", _block_ce_from_draft, None,
     [P.test_ce_label_is_argmax_of_target_logits, P.test_weighted_combination_unnormalised]),
    ("weights normalised by their sum", "_block", _block_normalised, None,
     [P.test_weighted_combination_unnormalised]),
    ("target row map off by one", "_target_rows", _target_rows_off_by_one, None,
     [P.test_target_rows_follow_the_head_shift, P.test_statistical_sanity_multihead_alpha]),
]


def test_pins_pass_on_the_unmodified_oracle():
    for _, _, _, _, pins in MUTATIONS:
        for pin in pins:
            pin()


@pytest.mark.parametrize("case", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_a_pin_catches_the_mutation(case, monkeypatch):
    name, attr, mutant, div_key, pins = case
    monkeypatch.setattr(O, attr, mutant)
    if div_key:
        monkeypatch.setitem(O.DIVERGENCES, div_key, mutant)
    caught = []
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError) as e:  # a pin, or numpy on a bad shape
            caught.append(type(e).__name__)
    assert caught, f"no pin noticed: {name}"
