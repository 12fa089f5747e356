"""Seeded synthetic workloads for the streaming LM-head loss.

Recipe (one per workload, see ``WORKLOADS``):

* Generator: numpy ``PCG64`` seeded from ``SeedSequence(1000 + index)``.  The
  root sequence is spawned into independent streams, in this fixed order:
  0 hidden, 1 LM-head weight, 2 target-weight noise, 3 labels, 4 mask
  permutation, 5 fresh rows for masked draft-head tails.  A tensor stream is
  spawned again into blocks of ``ROW_BLOCK`` rows, so large tensors are drawn
  by several threads and still come out bit-identical.
* Values are drawn in float32 and, for bf16 workloads, rounded once to bf16
  (round to nearest, ties to even).  Both the oracle and the GPU read exactly
  these bits.
* ``N(0, s)`` below means standard deviation ``s``; the one exception is the
  ``1/H`` of the small fp32 case, which is a variance (unit-variance logits).

The shapes are the model shapes of the streaming cross-entropy post (Llama
3.2 1B: H=2048, Llama 3.1 8B: H=4096 at 32k context, Llama 3.1 405B: H=16384,
all with the 128256-entry vocabulary); the synthetic values stand in for real
hidden states and trained weights.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

IGNORE_INDEX = -100
ROW_BLOCK = 2048


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _store(x: np.ndarray, bf16: bool) -> np.ndarray:
    return f32_to_bf16_bits(x) if bf16 else x


def _normal_matrix(seq: np.random.SeedSequence, rows: int, cols: int, std: float,
                   bf16: bool) -> np.ndarray:
    """rows x cols draws of N(0, std) in row blocks, each block its own child stream."""
    nblk = max(1, math.ceil(rows / ROW_BLOCK))
    children = seq.spawn(nblk)
    out = np.empty((rows, cols), dtype=np.uint16 if bf16 else np.float32)

    def work(i: int) -> None:
        r0, r1 = i * ROW_BLOCK, min(rows, (i + 1) * ROW_BLOCK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        x = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        x *= np.float32(std)
        out[r0:r1] = _store(x, bf16)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nblk)))
    return out


def _weight_pair(seq_w: np.random.SeedSequence, seq_n: np.random.SeedSequence, rows: int,
                 cols: int, std: float, noise_std: Optional[float],
                 bf16: bool) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """W ~ N(0, std) and, when ``noise_std`` is set, W_t = W + N(0, noise_std).

    W_t is formed from the float32 draws of W before rounding, then rounded once.
    """
    nblk = max(1, math.ceil(rows / ROW_BLOCK))
    cw = seq_w.spawn(nblk)
    cn = seq_n.spawn(nblk)
    dt = np.uint16 if bf16 else np.float32
    W = np.empty((rows, cols), dtype=dt)
    Wt = np.empty((rows, cols), dtype=dt) if noise_std is not None else None

    def work(i: int) -> None:
        r0, r1 = i * ROW_BLOCK, min(rows, (i + 1) * ROW_BLOCK)
        g = np.random.Generator(np.random.PCG64(cw[i]))
        x = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        x *= np.float32(std)
        W[r0:r1] = _store(x, bf16)
        if Wt is not None:
            gn = np.random.Generator(np.random.PCG64(cn[i]))
            e = gn.standard_normal((r1 - r0, cols), dtype=np.float32)
            e *= np.float32(noise_std)
            e += x
            Wt[r0:r1] = _store(e, bf16)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nblk)))
    return W, Wt


@dataclasses.dataclass
class Problem:
    """One workload's inputs.  Floating tensors are uint16 bf16 bits or float32."""
    name: str
    dtype: str                      # "bf16" or "f32"
    n_rows: int                     # N: aligned draft/student rows
    hidden_dim: int                 # H
    vocab: int                      # V
    hidden: np.ndarray              # [N, H]
    W: np.ndarray                   # [V, H]
    weights: Dict[str, float]       # loss-kind name -> weight (unnormalised)
    labels: Optional[np.ndarray] = None         # int32 [N], IGNORE_INDEX = ignored
    mask: Optional[np.ndarray] = None           # uint8 [N], 0 = masked
    target_hidden: Optional[np.ndarray] = None  # [N_t, H]
    W_t: Optional[np.ndarray] = None            # [V, H]
    target_row: Optional[np.ndarray] = None     # int32 [N]: row of target_hidden per row
    seq_len: Optional[int] = None               # multi-head layout: positions per head
    shifts: Optional[Tuple[int, ...]] = None    # multi-head layout (token-major rows,
                                                # row t * K + k): target shift per head
    seed: int = 0
    recipe: str = ""

    @property
    def n_target_rows(self) -> int:
        return 0 if self.target_hidden is None else int(self.target_hidden.shape[0])


# index -> (name, defaults).  Index i uses seed 1000 + i.
WORKLOADS = {
    "ce_fp32_small": dict(
        index=1, kind="ce", dtype="f32", n_rows=256, hidden_dim=256, vocab=4096,
        w_std=None, ignore_frac=0.10, mask_frac=0.0,
        recipe="fp32; h ~ N(0,1); W ~ N(0, var 1/H); labels U[0,V); 10% of rows -> ignore_index"),
    "ce_bf16_1b": dict(
        index=2, kind="ce", dtype="bf16", n_rows=8192, hidden_dim=2048, vocab=128256,
        w_std=0.02, ignore_frac=0.0, mask_frac=0.05,
        recipe="bf16; Llama-3.2-1B shape; h ~ N(0,1); W ~ N(0,0.02); labels U[0,V); 5% of rows mask=0"),
    "ce_bf16_8b": dict(
        index=3, kind="ce", dtype="bf16", n_rows=32768, hidden_dim=4096, vocab=128256,
        w_std=0.02, ignore_frac=0.0, mask_frac=0.0,
        recipe="bf16; Llama-3.1-8B shape, one 32k sequence; h ~ N(0,1); W ~ N(0,0.02); labels U[0,V); no mask"),
    "lk_hybrid_bf16_8b": dict(
        index=4, kind="lk_hybrid", dtype="bf16", n_rows=16384, hidden_dim=4096, vocab=128256,
        w_std=0.02, noise_std=0.005,
        recipe="bf16; draft h ~ N(0,1), target hidden = a copy of h in its own buffer; "
               "W_d ~ N(0,0.02); W_t = W_d + N(0,0.005); loss lk_hybrid"),
    "multihead_bf16_405b": dict(
        index=5, kind="multihead", dtype="bf16", seq_len=4096, shifts=(1, 2, 3),
        hidden_dim=16384, vocab=128256, w_std=0.02, noise_std=0.005,
        weights={"ce": 0.1, "tv": 0.9},
        recipe="bf16; Llama-3.1-405B shape; target hidden g ~ N(0,1) [S,H]; head k row t has "
               "h = g[t+k] and target row t+k, tail rows (t+k >= S) fresh N(0,1) and masked; "
               "W ~ N(0,0.02); W_t = W + N(0,0.005); loss 0.1*ce(argmax p) + 0.9*tv"),
}


def make_problem(name: str, *, n_rows: Optional[int] = None, hidden_dim: Optional[int] = None,
                 vocab: Optional[int] = None, seq_len: Optional[int] = None,
                 seed: Optional[int] = None, weights: Optional[Dict[str, float]] = None) -> Problem:
    """Build workload ``name``; the keyword overrides shrink it for small parity cases.

    Overrides keep the recipe (distributions, mask fractions, head layout) and
    change only the sizes or the seed.
    """
    spec = WORKLOADS[name]
    bf16 = spec["dtype"] == "bf16"
    H = int(hidden_dim or spec["hidden_dim"])
    V = int(vocab or spec["vocab"])
    s = int(seed if seed is not None else 1000 + spec["index"])
    streams = np.random.SeedSequence(s).spawn(6)
    kind = spec["kind"]

    if kind == "ce":
        N = int(n_rows or spec["n_rows"])
        w_std = spec["w_std"] if spec["w_std"] is not None else 1.0 / math.sqrt(H)
        hidden = _normal_matrix(streams[0], N, H, 1.0, bf16)
        W, _ = _weight_pair(streams[1], streams[2], V, H, w_std, None, bf16)
        labels = np.random.Generator(np.random.PCG64(streams[3])).integers(
            0, V, size=N, dtype=np.int64).astype(np.int32)
        perm = np.random.Generator(np.random.PCG64(streams[4])).permutation(N)
        mask = None
        n_ign = int(round(spec["ignore_frac"] * N))
        if n_ign:
            labels[perm[:n_ign]] = IGNORE_INDEX
        n_msk = int(round(spec["mask_frac"] * N))
        if n_msk:
            mask = np.ones(N, dtype=np.uint8)
            mask[perm[:n_msk]] = 0
        return Problem(name=name, dtype=spec["dtype"], n_rows=N, hidden_dim=H, vocab=V,
                       hidden=hidden, W=W, labels=labels, mask=mask,
                       weights=dict(weights or {"ce_label": 1.0}), seed=s, recipe=spec["recipe"])

    if kind == "lk_hybrid":
        N = int(n_rows or spec["n_rows"])
        hidden = _normal_matrix(streams[0], N, H, 1.0, bf16)
        W, Wt = _weight_pair(streams[1], streams[2], V, H, spec["w_std"], spec["noise_std"], bf16)
        return Problem(name=name, dtype=spec["dtype"], n_rows=N, hidden_dim=H, vocab=V,
                       hidden=hidden, W=W, target_hidden=hidden.copy(), W_t=Wt,
                       weights=dict(weights or {"lk_hybrid": 1.0}), seed=s, recipe=spec["recipe"])

    if kind == "multihead":
        S = int(seq_len or spec["seq_len"])
        shifts = tuple(spec["shifts"])
        K = len(shifts)
        N = K * S
        g = _normal_matrix(streams[0], S, H, 1.0, bf16)
        W, Wt = _weight_pair(streams[1], streams[2], V, H, spec["w_std"], spec["noise_std"], bf16)
        n_tail = sum(min(S, sh) for sh in shifts)
        tail = _normal_matrix(streams[5], max(n_tail, 1), H, 1.0, bf16)
        hidden = np.empty((N, H), dtype=g.dtype)
        target_row = np.full(N, -1, dtype=np.int32)
        mask = np.zeros(N, dtype=np.uint8)
        # token-major rows: row t * K + k is head k at position t (the layout
        # of specloss_align_heads); tail rows draw from the tail stream in head
        # order
        ti = 0
        for k, sh in enumerate(shifts):
            keep = max(0, S - sh)
            rows = np.arange(S) * K + k
            hidden[rows[:keep]] = g[sh:sh + keep]
            target_row[rows[:keep]] = np.arange(sh, sh + keep, dtype=np.int32)
            mask[rows[:keep]] = 1
            nt = S - keep
            hidden[rows[keep:]] = tail[ti:ti + nt]
            ti += nt
        return Problem(name=name, dtype=spec["dtype"], n_rows=N, hidden_dim=H, vocab=V,
                       hidden=hidden, W=W, mask=mask, target_hidden=g, W_t=Wt,
                       target_row=target_row, seq_len=S, shifts=shifts,
                       weights=dict(weights or spec["weights"]), seed=s, recipe=spec["recipe"])

    raise ValueError(f"unknown workload kind {kind!r}")
