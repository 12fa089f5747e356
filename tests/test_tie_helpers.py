"""CPU check of the GPU tests' near-tie handling of the ce label.

Where the two largest target logits are closer than the argmax bar, either
label is a correct hard label ("Available Losses", ce row: argmax p; the
lowest-index tie rule is the oracle's reading).  The helpers take the
oracle's values for the label the device chose; this test checks them
against the oracle run with that label given explicitly (ce_label has the
same formula as ce with a given label), on an exact tie.
"""
import numpy as np
import pytest

from oracle import specloss_oracle as O
from tests._gpu_helpers import apply_moved_labels, ce_tie_candidates, retarget_ties


def _tied_problem():
    rng = np.random.default_rng(31)
    N, H, V = 5, 4, 8
    a = rng.standard_normal(H)
    Wt = np.zeros((V, H))
    Wt[2] = Wt[5] = a                     # target logits tie exactly at 2 and 5
    g = rng.standard_normal((N, H))
    g *= np.sign(g @ a)[:, None]          # so that the tied pair is the maximum
    return O.OracleProblem(dtype="f64", vocab=V, hidden=rng.standard_normal((N, H)),
                           W=rng.standard_normal((V, H)), weights={"ce": 1.0},
                           target_hidden=g, W_t=Wt)


def test_other_tied_label_matches_the_oracle_with_that_label():
    prob = _tied_problem()
    rows = np.arange(prob.n_rows)
    ref = O.forward(prob)
    assert np.all(ref.label == 2)  # lowest index among the tied maxima
    ties = ce_tie_candidates(prob, rows, ref.valid)
    assert ties == {i: (2, {2, 5}) for i in range(prob.n_rows)}
    gpu_y = np.array([5, 2, 5, 5, 2])
    loss, term, moved = retarget_ties(prob, rows, ref, ties, gpu_y)
    # the oracle with those labels given explicitly
    alt = O.OracleProblem(**{**prob.__dict__, "weights": {"ce_label": 1.0},
                             "labels": gpu_y.astype(np.int32)})
    r_alt = O.forward(alt)
    assert np.allclose(loss, r_alt.loss, rtol=1e-13, atol=0)
    assert np.allclose(term, r_alt.terms["ce_label"], rtol=1e-13, atol=0)
    seed = O.mean_seed(prob)
    rdh, rdW = O.backward(prob)
    rdh, rdW = apply_moved_labels(prob, rows, moved, seed, rdh, rdW)
    adh, adW = O.backward(alt)
    assert np.allclose(rdh, adh, rtol=1e-12, atol=1e-15)
    assert np.allclose(rdW, adW, rtol=1e-12, atol=1e-15)


def test_a_label_outside_the_tie_is_rejected():
    prob = _tied_problem()
    rows = np.arange(prob.n_rows)
    ref = O.forward(prob)
    ties = ce_tie_candidates(prob, rows, ref.valid)
    with pytest.raises(AssertionError):
        retarget_ties(prob, rows, ref, ties, np.array([5, 2, 3, 5, 2]))


def test_ties_with_a_label_loss_beside_ce():
    """ce beside ce_label: the oracle's label field then holds the given labels,
    and the tie handling must still move only the ce term."""
    prob = _tied_problem()
    prob.weights = {"ce_label": 0.5, "ce": 1.0}
    prob.labels = np.array([0, 1, 7, 4, 6], np.int32)
    rows = np.arange(prob.n_rows)
    ref = O.forward(prob)
    ties = ce_tie_candidates(prob, rows, ref.valid)
    gpu_y = np.array([5, 2, 5, 2, 5])
    loss, term, moved = retarget_ties(prob, rows, ref, ties, gpu_y)
    as_label = lambda w, y: O.OracleProblem(**{**prob.__dict__, "weights": {"ce_label": w},
                                               "labels": y.astype(np.int32)})
    given, chosen = as_label(0.5, prob.labels), as_label(1.0, gpu_y)
    assert np.allclose(loss, O.forward(given).loss + O.forward(chosen).loss, rtol=1e-13, atol=0)
    assert np.allclose(term, O.forward(chosen).terms["ce_label"], rtol=1e-13, atol=0)
    rdh, rdW = O.backward(prob)
    rdh, rdW = apply_moved_labels(prob, rows, moved, O.mean_seed(prob), rdh, rdW)
    gdh, gdW = O.backward(given)
    cdh, cdW = O.backward(chosen)
    assert np.allclose(rdh, gdh + cdh, rtol=1e-12, atol=1e-15)
    assert np.allclose(rdW, gdW + cdW, rtol=1e-12, atol=1e-15)
