"""Plain float64 CPU oracle of the streaming LM-head loss.  TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import or call this module; the product path never does.  It
shares no code with the GPU path: the only common module is ``synthetic``,
which draws the inputs and holds none of the loss arithmetic.

What it computes is the dense definition of the loss, row block by row block:
the logits of every row it handles are materialised in float64 (this is the
"dense version" of the streaming cross-entropy post, section "Streaming Cross
Entropy": ``logits = lm_head(hidden)`` then ``cross_entropy(logits, targets)``),
and the divergences follow the "Available Losses" table of the vLLM
speculators "Loss Functions" page.  Inputs are the exact bf16 or fp32 bits the
GPU receives, widened without rounding.

Readings taken where the pages are silent (each is listed in the design notes):

* LM head ``W`` is ``[V, H]`` (one row per vocabulary entry), no bias, no
  temperature, no softcap; logits ``z = W h``.
* Natural logarithms; JSD mixes with weights 1/2, 1/2.
* ``kl_div`` is KL(p || q) with p the target and q the draft; ``rkl`` is KL(q || p).
* ``ce`` takes its hard label from argmax p, lowest index on ties; ``ce_label``
  is the language-model cross-entropy against given token labels.
* TV's subgradient at ``q_v == p_v`` counts the tie as 1/2.
* ``lk_hybrid`` computes alpha and lambda = exp(-3 alpha) per row; lambda is a
  constant in the backward.
* One denominator: the number of valid rows of the whole aligned token set.
* A row is valid when its mask is 1 and, if a label kind is on, its label is
  not ignore_index (-100).  An unmasked row whose label (or target row) is
  out of range counts as "bad" and is treated as masked.
* With no valid row the mean is 0 and every gradient is 0.
* Aligned heads are laid out token-major: row ``(b*S + t)*K + k`` is head k at
  position t of sequence b, paired with target position ``t + shift_k``.

Parity pins: every function here is checked against closed forms, library
routines or finite differences by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

KINDS: Tuple[str, ...] = ("ce_label", "ce", "kl_div", "rkl", "jsd", "tv", "nla", "lk_hybrid")
LABEL_KINDS = frozenset({"ce_label"})
TARGET_KINDS = frozenset({"ce", "kl_div", "rkl", "jsd", "tv", "nla", "lk_hybrid"})
IGNORE_INDEX = -100
LK_HYBRID_RATE = 3.0  # lambda = exp(-3 alpha), "Available Losses" table, lk_hybrid row


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 copy of bf16 bit patterns (uint16), float32 or float64 values."""
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
            np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":  # used by the finite-difference pins
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# row-level definitions
# ----------------------------------------------------------------------------
def logsumexp_rows(x: np.ndarray) -> np.ndarray:
    """log sum_v exp(x_v) per row, shifted by the row max (exact up to rounding)."""
    m = np.max(x, axis=1, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=1, keepdims=True)))[:, 0]


def ce_from_logits(z: np.ndarray, y: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Cross-entropy of logits against hard labels and its logit gradient.

    Streaming cross-entropy post, "Streaming Cross Entropy": the loss is a sum of
    independent per-token terms ``-log softmax(z)_y``; the gradient is
    ``softmax(z) - onehot(y)``.
    """
    lse = logsumexp_rows(z)
    r = np.arange(z.shape[0])
    loss = lse - z[r, y]
    dz = np.exp(z - lse[:, None])
    dz[r, y] -= 1.0
    return loss, dz


def kl_forward(logp: np.ndarray, logq: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """kl_div: KL(p || q) = sum_v p_v (log p_v - log q_v); d/dz = q - p.

    Speculators "Loss Functions", "Available Losses": forward KL, target to draft.
    """
    p, q = np.exp(logp), np.exp(logq)
    loss = np.sum(p * (logp - logq), axis=1)
    return loss, q - p


def kl_reverse(logp: np.ndarray, logq: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """rkl: KL(q || p) = sum_v q_v (log q_v - log p_v); d/dz = q (log q - log p - L).

    Speculators "Loss Functions", "Available Losses": reverse KL, draft to target.
    """
    q = np.exp(logq)
    loss = np.sum(q * (logq - logp), axis=1)
    dz = q * (logq - logp - loss[:, None])
    return loss, dz


def jensen_shannon(logp: np.ndarray, logq: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """jsd: 1/2 KL(p || m) + 1/2 KL(q || m), m = (p + q) / 2.

    Speculators "Loss Functions", "Available Losses": symmetric, at most log 2.
    dL/dq_v = 1/2 log(q_v / m_v), so d/dz = q (g - E_q[g]).
    """
    p, q = np.exp(logp), np.exp(logq)
    logm = np.logaddexp(logp, logq) - np.log(2.0)
    loss = 0.5 * np.sum(p * (logp - logm), axis=1) + 0.5 * np.sum(q * (logq - logm), axis=1)
    g = 0.5 * (logq - logm)
    dz = q * (g - np.sum(q * g, axis=1, keepdims=True))
    return loss, dz


def overlap(logp: np.ndarray, logq: np.ndarray) -> np.ndarray:
    """alpha = sum_v min(p_v, q_v), the speculative-decoding acceptance rate.

    Speculators "Loss Functions", "Available Losses" (the text above the table).
    """
    return np.sum(np.minimum(np.exp(logp), np.exp(logq)), axis=1)


def total_variation(logp: np.ndarray, logq: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """tv: 1 - alpha.  dL/dq_v = -c_v with c_v = 1[q_v < p_v] (1/2 on a tie).

    Speculators "Loss Functions", "Available Losses", tv row.
    d/dz = -q (c - S), S = sum_v q_v c_v.
    """
    p, q = np.exp(logp), np.exp(logq)
    alpha = np.sum(np.minimum(p, q), axis=1)
    c = np.where(q < p, 1.0, np.where(q == p, 0.5, 0.0))
    S = np.sum(q * c, axis=1, keepdims=True)
    return 1.0 - alpha, -q * (c - S)


def neg_log_acceptance(logp: np.ndarray, logq: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """nla: -log alpha; its gradient is TV's divided by alpha.

    Speculators "Loss Functions", "Available Losses", nla row.
    """
    tv_loss, tv_dz = total_variation(logp, logq)
    alpha = 1.0 - tv_loss
    return -np.log(alpha), tv_dz / alpha[:, None]


def lk_hybrid(logp: np.ndarray, logq: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """lk_hybrid: lambda KL(p || q) + (1 - lambda)(1 - alpha), lambda = exp(-3 alpha) detached.

    Speculators "Loss Functions", "Available Losses", lk_hybrid row.  Lambda is
    computed per row from that row's alpha and is a constant for the gradient.
    """
    kl, kl_dz = kl_forward(logp, logq)
    tv_loss, tv_dz = total_variation(logp, logq)
    lam = np.exp(-LK_HYBRID_RATE * (1.0 - tv_loss))
    loss = lam * kl + (1.0 - lam) * tv_loss
    dz = lam[:, None] * kl_dz + (1.0 - lam)[:, None] * tv_dz
    return loss, dz


DIVERGENCES = {
    "kl_div": kl_forward,
    "rkl": kl_reverse,
    "jsd": jensen_shannon,
    "tv": total_variation,
    "nla": neg_log_acceptance,
    "lk_hybrid": lk_hybrid,
}


def flatness(logp: np.ndarray) -> np.ndarray:
    """Cosine similarity of each row's distribution p to the uniform distribution.

    "Flatter Tokens are More Valuable for Speculative Draft Model Training"
    (summary, Approach): a token's importance score is the cosine similarity of
    the target distribution to the uniform one,
    cos(p, 1/V) = sum_v p_v / (sqrt(V) * ||p||_2).
    """
    p = np.exp(logp)
    V = p.shape[1]
    ones = np.full(V, 1.0 / V)
    return (p @ ones) / (np.linalg.norm(p, axis=1) * np.linalg.norm(ones))


def argmax_lowest(u: np.ndarray) -> np.ndarray:
    """Index of the row maximum, lowest index among equal maxima (hard label of ce)."""
    return np.argmax(u, axis=1).astype(np.int64)


# ----------------------------------------------------------------------------
# alignment (streaming cross-entropy post, "Correctness: alignment before chunking")
# ----------------------------------------------------------------------------
def align_heads(seq_len: int, shifts: Sequence[int], batch: int = 1,
                loss_mask: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Aligned target row and mask for draft heads that predict ``shift`` tokens ahead.

    Rows are token-major: row ``(b*seq_len + t)*K + k`` is head k (of K) at
    position t of sequence b.  Its target is position ``t + shift_k`` of the same
    sequence; it is valid iff that position exists and (if given) the loss mask
    of the target position is 1.  Invalid rows get target row -1.  This is done
    for the whole token set before any chunking.
    """
    K = len(shifts)
    n = K * batch * seq_len
    target_row = np.full(n, -1, dtype=np.int64)
    mask = np.zeros(n, dtype=np.uint8)
    for k, sh in enumerate(shifts):
        for b in range(batch):
            for t in range(seq_len):
                r = (b * seq_len + t) * K + k
                tt = t + sh
                if 0 <= tt < seq_len:
                    src = b * seq_len + tt
                    if loss_mask is None or loss_mask[src]:
                        target_row[r] = src
                        mask[r] = 1
    return target_row, mask


# ----------------------------------------------------------------------------
# whole-problem forward / backward
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class OracleProblem:
    """The oracle's view of a problem (same fields as ``synthetic.Problem``)."""
    dtype: str
    vocab: int
    hidden: np.ndarray
    W: np.ndarray
    weights: Dict[str, float]
    labels: Optional[np.ndarray] = None
    mask: Optional[np.ndarray] = None
    target_hidden: Optional[np.ndarray] = None
    W_t: Optional[np.ndarray] = None
    target_row: Optional[np.ndarray] = None

    @classmethod
    def of(cls, prob) -> "OracleProblem":
        return cls(dtype=prob.dtype, vocab=prob.vocab, hidden=prob.hidden, W=prob.W,
                   weights=dict(prob.weights), labels=prob.labels, mask=prob.mask,
                   target_hidden=prob.target_hidden, W_t=prob.W_t, target_row=prob.target_row)

    @property
    def n_rows(self) -> int:
        return int(self.hidden.shape[0])

    def active(self) -> Dict[str, float]:
        return {k: float(w) for k, w in self.weights.items() if float(w) != 0.0}


def row_validity(prob: OracleProblem) -> Tuple[np.ndarray, np.ndarray]:
    """(valid, bad) per row, before any chunking.

    Streaming cross-entropy post, "Correctness: alignment before chunking":
    masks are applied to the aligned token set; the valid rows form the one
    denominator of the loss.
    """
    act = prob.active()
    for k in act:
        if k not in KINDS:
            raise ValueError(f"unknown loss kind {k!r}")
    N = prob.n_rows
    valid = np.ones(N, dtype=bool) if prob.mask is None else (np.asarray(prob.mask) != 0)
    bad = np.zeros(N, dtype=bool)
    if any(k in LABEL_KINDS for k in act):
        if prob.labels is None:
            raise ValueError("a label loss needs labels")
        lab = np.asarray(prob.labels, dtype=np.int64)
        ignored = lab == IGNORE_INDEX
        out = ((lab < 0) | (lab >= prob.vocab)) & ~ignored
        valid &= ~ignored
        bad |= out & valid
        valid &= ~out
    if any(k in TARGET_KINDS for k in act):
        if prob.target_hidden is None or prob.W_t is None:
            raise ValueError("a target-vs-draft loss needs target hidden states and W_t")
        if prob.target_row is not None:
            tr = np.asarray(prob.target_row, dtype=np.int64)
            out = (tr < 0) | (tr >= prob.target_hidden.shape[0])
            bad |= out & valid
            valid &= ~out
    return valid, bad


@dataclasses.dataclass
class OracleResult:
    rows: np.ndarray                 # row indices covered
    loss: np.ndarray                 # weighted per-row loss (0 on invalid rows)
    terms: Dict[str, np.ndarray]     # unweighted per-row loss of each active kind
    lse_q: np.ndarray                # draft logsumexp
    lse_p: Optional[np.ndarray]      # target logsumexp
    label: np.ndarray                # label used by ce / ce_label (-1 where none)
    alpha: Optional[np.ndarray]      # overlap, where a target exists
    valid: np.ndarray                # per covered row
    n_valid: int                     # over the whole problem
    n_bad: int
    dz: Optional[np.ndarray] = None  # d(loss_t)/dz rows, weighted, before the seed
    flat: Optional[np.ndarray] = None  # flatness of p, where a target exists


def _target_rows(prob: OracleProblem, idx: np.ndarray, valid: np.ndarray) -> np.ndarray:
    if prob.target_row is None:
        return idx.copy()
    tr = np.asarray(prob.target_row, dtype=np.int64)[idx]
    return np.where(valid, tr, 0)  # invalid rows: any in-range row, result unused


def _block(prob: OracleProblem, idx: np.ndarray, Wd: np.ndarray, Wt: Optional[np.ndarray],
           valid_all: np.ndarray, want_dz: bool):
    act = prob.active()
    valid = valid_all[idx]
    h = widen(prob.hidden[idx], prob.dtype)
    z = h @ Wd.T                                         # logits = lm_head(hidden)
    lse_q = logsumexp_rows(z)
    logq = z - lse_q[:, None]
    B, V = z.shape
    terms: Dict[str, np.ndarray] = {}
    dzs: Dict[str, np.ndarray] = {}
    lse_p = alpha = flat = None
    label = np.full(B, -1, dtype=np.int64)
    if any(k in TARGET_KINDS for k in act):
        g = widen(prob.target_hidden[_target_rows(prob, idx, valid)], prob.dtype)
        u = g @ Wt.T
        lse_p = logsumexp_rows(u)
        logp = u - lse_p[:, None]
        alpha = overlap(logp, logq)
        flat = flatness(logp)
        if "ce" in act:
            y = argmax_lowest(u)
            label = y
            terms["ce"], dzs["ce"] = ce_from_logits(z, y)
        for k, fn in DIVERGENCES.items():
            if k in act:
                terms[k], dzs[k] = fn(logp, logq)
    if "ce_label" in act:
        y = np.asarray(prob.labels, dtype=np.int64)[idx]
        y = np.where(valid, y, 0)
        label = np.where(valid, y, -1)
        terms["ce_label"], dzs["ce_label"] = ce_from_logits(z, y)
    loss = np.zeros(B)
    dz = np.zeros((B, V)) if want_dz else None
    for k, w in act.items():
        terms[k] = np.where(valid, terms[k], 0.0)
        loss += w * terms[k]
        if want_dz:
            dz += w * dzs[k]
    if want_dz:
        dz[~valid] = 0.0
    return loss, terms, lse_q, lse_p, label, alpha, valid, dz, flat


def _weights64(prob: OracleProblem):
    Wd = widen(prob.W, prob.dtype)
    Wt = None
    if any(k in TARGET_KINDS for k in prob.active()):
        Wt = widen(prob.W_t, prob.dtype)
    return Wd, Wt


def forward(prob, rows: Optional[Iterable[int]] = None, block: int = 64,
            want_dz: bool = False, weights64=None) -> OracleResult:
    """Per-row losses of the rows ``rows`` (all rows if None), in row blocks.

    Streaming cross-entropy post, "Streaming Cross Entropy": every valid token
    contributes its own term; the block size changes nothing but rounding.
    """
    prob = prob if isinstance(prob, OracleProblem) else OracleProblem.of(prob)
    valid_all, bad_all = row_validity(prob)
    sel = np.arange(prob.n_rows) if rows is None else np.asarray(list(rows), dtype=np.int64)
    Wd, Wt = weights64 if weights64 is not None else _weights64(prob)
    parts = []
    for b0 in range(0, len(sel), block):
        parts.append(_block(prob, sel[b0:b0 + block], Wd, Wt, valid_all, want_dz))

    def cat(i):
        if not parts or parts[0][i] is None:
            return None
        return np.concatenate([p[i] for p in parts])

    act = prob.active()
    terms = {k: np.concatenate([p[1][k] for p in parts]) if parts else np.zeros(0) for k in act}
    return OracleResult(rows=sel, loss=cat(0) if parts else np.zeros(0), terms=terms,
                        lse_q=cat(2), lse_p=cat(3), label=cat(4), alpha=cat(5),
                        valid=cat(6), n_valid=int(valid_all.sum()), n_bad=int(bad_all.sum()),
                        dz=cat(7) if want_dz else None, flat=cat(8))


def mean_loss(prob) -> Tuple[float, Dict[str, float], int]:
    """(sum_t loss_t / n_valid, per-kind unweighted means, n_valid) over all rows.

    Streaming cross-entropy post, "Backward pass": normalise by the number of
    valid tokens, never by the number of chunks.
    """
    r = forward(prob)
    n = r.n_valid
    if n == 0:
        return 0.0, {k: 0.0 for k in r.terms}, 0
    return float(np.sum(r.loss) / n), {k: float(np.sum(v) / n) for k, v in r.terms.items()}, n


def mean_seed(prob) -> np.ndarray:
    """Per-row gradient seed of the mean loss: 1/n_valid on valid rows, else 0."""
    prob = prob if isinstance(prob, OracleProblem) else OracleProblem.of(prob)
    valid, _ = row_validity(prob)
    n = int(valid.sum())
    return np.where(valid, 1.0 / n, 0.0) if n else np.zeros(prob.n_rows)


def backward(prob, seed: Optional[np.ndarray] = None, rows: Optional[Iterable[int]] = None,
             block: int = 64, want_dW: bool = True, dW_rows: Optional[np.ndarray] = None,
             weights64=None):
    """(dh, dW) of sum_t seed_t * loss_t restricted to ``rows``.

    Streaming cross-entropy post, "Backward pass": per token, the logit gradient
    gives the hidden-state gradient ``dh_t = dz_t W`` and contributes
    ``dz_t^T h_t`` to the LM-head gradient.  ``seed`` defaults to the mean-loss
    seed.  With ``rows`` given, dh covers those rows and dW sums only their
    contributions (equal to the full dW when the seed is zero elsewhere).
    ``dW_rows`` restricts the returned dW to those vocabulary rows.
    """
    prob = prob if isinstance(prob, OracleProblem) else OracleProblem.of(prob)
    if seed is None:
        seed = mean_seed(prob)
    seed = np.asarray(seed, dtype=np.float64)
    valid_all, _ = row_validity(prob)
    sel = np.arange(prob.n_rows) if rows is None else np.asarray(list(rows), dtype=np.int64)
    Wd, Wt = weights64 if weights64 is not None else _weights64(prob)
    H = Wd.shape[1]
    dh = np.zeros((len(sel), H))
    vsel = np.arange(prob.vocab) if dW_rows is None else np.asarray(dW_rows, dtype=np.int64)
    dW = np.zeros((len(vsel), H)) if want_dW else None
    for b0 in range(0, len(sel), block):
        idx = sel[b0:b0 + block]
        dz = _block(prob, idx, Wd, Wt, valid_all, True)[7]
        dz = dz * seed[idx][:, None]
        dh[b0:b0 + len(idx)] = dz @ Wd
        if want_dW:
            h = widen(prob.hidden[idx], prob.dtype)
            dW += dz[:, vsel].T @ h
    return dh, dW
