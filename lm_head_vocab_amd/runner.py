"""Buffers for one loss problem and the calls that fill them.

torch allocates every device buffer (inputs stay where the caller put them);
the work itself is the C-ABI calls ``lmhead_loss_fwd`` / ``lmhead_loss_bwd``.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import torch

from . import binding as B


class LossRun:
    """One problem bound to its workspace, forward outputs and saved state."""

    def __init__(self, hidden: torch.Tensor, W: torch.Tensor, weights: Dict[str, float], *,
                 labels: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                 target_hidden: Optional[torch.Tensor] = None, W_t: Optional[torch.Tensor] = None,
                 target_row: Optional[torch.Tensor] = None, max_chunk_rows: int = 0,
                 workspace_bytes: Optional[int] = None, want_terms: bool = True,
                 flags: int = 0, heads: Optional[Sequence[int]] = None):
        dev = hidden.device
        self.inputs = dict(hidden=hidden, W=W, labels=labels, mask=mask,
                           target_hidden=target_hidden, W_t=W_t, target_row=target_row)
        self.weights = dict(weights)
        self.problem = B.make_problem(hidden, W, weights, labels=labels, mask=mask,
                                      target_hidden=target_hidden, W_t=W_t, target_row=target_row,
                                      flags=flags, heads=heads)
        N = hidden.shape[0]
        self.n_rows = N
        ws = workspace_bytes if workspace_bytes is not None else \
            B.lmhead_loss_workspace_size(self.problem, max_chunk_rows)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.loss = torch.empty(N, dtype=torch.float32, device=dev)
        self.term = torch.zeros(B.NUM_KINDS, N, dtype=torch.float32, device=dev) if want_terms else None
        self.lse_q = torch.empty(N, dtype=torch.float32, device=dev)
        self.saved = torch.empty(B.specloss_saved_bytes(N), dtype=torch.uint8, device=dev)
        self.counts = torch.zeros(2, dtype=torch.int64, device=dev)
        self.reduced = torch.empty(1 + B.NUM_KINDS, dtype=torch.float32, device=dev)

    def forward(self, stream=None) -> None:
        B.lmhead_loss_fwd(self.problem, self.workspace, self.loss, self.term, self.lse_q,
                          self.saved, self.counts, self.reduced, stream)

    def backward(self, grad_loss: Optional[torch.Tensor] = None,
                 grad_mean: Optional[torch.Tensor] = None, dhidden: Optional[torch.Tensor] = None,
                 dW: Optional[torch.Tensor] = None, accumulate_dW: bool = False,
                 want_dh: bool = True, want_dW: bool = True, stream=None):
        h, W = self.inputs["hidden"], self.inputs["W"]
        if dhidden is None and want_dh:
            dhidden = torch.empty(h.shape, dtype=torch.float32, device=h.device)
        if dW is None and want_dW:
            dW = torch.empty(W.shape, dtype=torch.float32, device=W.device)
        B.lmhead_loss_bwd(self.problem, grad_loss, grad_mean, self.counts, self.saved,
                          self.workspace, dhidden, dW, accumulate_dW, stream)
        return dhidden, dW

    def forward_backward(self, grad_loss: Optional[torch.Tensor] = None,
                         grad_mean: Optional[torch.Tensor] = None,
                         dhidden: Optional[torch.Tensor] = None, dW: Optional[torch.Tensor] = None,
                         accumulate_dW: bool = False, want_dh: bool = True, want_dW: bool = True,
                         stream=None):
        """Single call: forward outputs plus the gradients for the given seed."""
        h, W = self.inputs["hidden"], self.inputs["W"]
        if dhidden is None and want_dh:
            dhidden = torch.empty(h.shape, dtype=torch.float32, device=h.device)
        if dW is None and want_dW:
            dW = torch.empty(W.shape, dtype=torch.float32, device=W.device)
        B.lmhead_loss_fwd_bwd(self.problem, self.workspace, self.loss, self.term, self.lse_q,
                              self.saved, self.counts, self.reduced, grad_loss, grad_mean,
                              dhidden, dW, accumulate_dW, stream)
        return dhidden, dW

    @property
    def workspace_bytes(self) -> int:
        return self.workspace.numel()

    def chunk(self, call: int = B.CALL_FWD_BWD):
        """(rows per chunk, backward layout, chunks per dW contraction) the given
        call uses with this workspace."""
        return B.lmhead_loss_chunk(self.problem, self.workspace_bytes, call)

    def saved_field(self, i: int, dtype=torch.float32) -> torch.Tensor:
        """View of saved field i (SPECLOSS_SAVED_* / SavedView order) as an N-vector."""
        o = B.specloss_saved_offset(self.n_rows, i)
        return self.saved[o:o + self.n_rows * 4].view(dtype)

    @property
    def flatness(self) -> torch.Tensor:
        """Per-row flatness of the target distribution, cos(p, uniform)."""
        return self.saved_field(B.SAVED_FLATNESS)


class _LMHeadLoss(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, W, run: LossRun):
        run.forward()
        ctx.run = run
        return run.reduced[0].clone()

    @staticmethod
    def backward(ctx, g):
        run: LossRun = ctx.run
        gm = g.reshape(1).to(torch.float32).contiguous()
        want_h, want_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        dh, dW = run.backward(grad_mean=gm, want_dh=want_h, want_dW=want_w)
        h, W = run.inputs["hidden"], run.inputs["W"]
        return (None if dh is None else dh.to(h.dtype), None if dW is None else dW.to(W.dtype), None)


class _LMHeadLossTerminal(torch.autograd.Function):
    """The mean loss of a graph that ends in it: the single call forms the
    gradients of the mean with the forward, and backward scales them by the
    upstream scalar (the gradient is linear in it)."""

    @staticmethod
    def forward(ctx, hidden, W, run: LossRun):
        want_h, want_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        ctx.dtypes = (hidden.dtype, W.dtype)
        ctx.dh = ctx.dW = None
        if want_h or want_w:
            one = torch.ones(1, dtype=torch.float32, device=hidden.device)
            ctx.dh, ctx.dW = run.forward_backward(grad_mean=one, want_dh=want_h, want_dW=want_w)
        else:
            run.forward()
        return run.reduced[0].clone()

    @staticmethod
    def backward(ctx, g):
        dh, dW = ctx.dh, ctx.dW
        ctx.dh = ctx.dW = None
        g = g.to(torch.float32)
        th, tw = ctx.dtypes
        return (None if dh is None else (dh * g).to(th),
                None if dW is None else (dW * g).to(tw), None)


def lmhead_loss(hidden: torch.Tensor, W: torch.Tensor, weights: Dict[str, float], *,
                terminal: bool = False, **kw) -> torch.Tensor:
    """Mean streaming LM-head loss with autograd; gradients flow to hidden and W.

    terminal: the loss is the last node of the graph and backward will be called:
    the forward then runs the single call (lmhead_loss_fwd_bwd), which forms the
    gradients without recomputing any logits tile, and backward only scales them.
    Otherwise the forward keeps per-row state and backward recomputes the tiles
    (lmhead_loss_fwd, then lmhead_loss_bwd)."""
    run = LossRun(hidden.detach(), W.detach(), weights, **kw)
    if terminal:
        return _LMHeadLossTerminal.apply(hidden, W, run)
    return _LMHeadLoss.apply(hidden, W, run)


class ShardedLossRun(LossRun):
    """The vocabulary-parallel sequence on one device: G shards of W (and W_t).

    Shard g owns vocabulary rows [bounds[g], bounds[g+1]) (by default whole
    256-row tiles except the last shard's end); the G shard calls run one after another on the same
    stream, with one exchange buffer that every shard writes its record into.
    On G devices each shard's calls would run on its own device, the exchange
    being an all-gather of the records and the dh sum an all-reduce.
    """

    def __init__(self, hidden: torch.Tensor, W: torch.Tensor, weights: Dict[str, float],
                 n_shards: int, *, labels: Optional[torch.Tensor] = None,
                 mask: Optional[torch.Tensor] = None,
                 target_hidden: Optional[torch.Tensor] = None, W_t: Optional[torch.Tensor] = None,
                 target_row: Optional[torch.Tensor] = None, max_chunk_rows: int = 0,
                 want_terms: bool = True, bounds: Optional[list] = None, flags: int = 0,
                 heads: Optional[Sequence[int]] = None):
        dev = hidden.device
        V = W.shape[0]
        if bounds is None:
            step = -(-V // (n_shards * 256)) * 256
            bounds = [min(V, g * step) for g in range(n_shards)] + [V]
        self.bounds = [int(b) for b in bounds]
        if len(self.bounds) != n_shards + 1 or self.bounds[0] != 0 or self.bounds[-1] != V:
            raise ValueError("bounds must run from 0 to V in n_shards steps")
        if any(b1 <= b0 for b0, b1 in zip(self.bounds, self.bounds[1:])):
            raise ValueError(f"{n_shards} shards of whole 256-row tiles do not fit V={V}")
        self.inputs = dict(hidden=hidden, W=W, labels=labels, mask=mask,
                           target_hidden=target_hidden, W_t=W_t, target_row=target_row)
        self.weights = dict(weights)
        N = hidden.shape[0]
        self.n_rows = N
        self.n_shards = n_shards
        self.exchange = torch.empty(B.specloss_exchange_bytes(N, n_shards), dtype=torch.uint8,
                                    device=dev)
        self.problems, self.shards = [], []
        ws = 256
        for g in range(n_shards):
            v0, v1 = self.bounds[g], self.bounds[g + 1]
            prob = B.make_problem(hidden, W[v0:v1], weights, labels=labels, mask=mask,
                                  target_hidden=target_hidden,
                                  W_t=None if W_t is None else W_t[v0:v1], target_row=target_row,
                                  flags=flags, heads=heads)
            sh = B.Shard(vocab_offset=v0, vocab_total=V, shard=g, n_shards=n_shards,
                         exchange=self.exchange.data_ptr())
            self.problems.append(prob)
            self.shards.append(sh)
            ws = max(ws, B.lmhead_loss_workspace_size(prob, max_chunk_rows))
        self.problem = self.problems[0]
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.loss = torch.empty(N, dtype=torch.float32, device=dev)
        self.term = torch.zeros(B.NUM_KINDS, N, dtype=torch.float32, device=dev) if want_terms else None
        self.lse_q = torch.empty(N, dtype=torch.float32, device=dev)
        self.saved = torch.empty(B.specloss_saved_bytes(N), dtype=torch.uint8, device=dev)
        self.counts = torch.zeros(2, dtype=torch.int64, device=dev)
        self.reduced = torch.empty(1 + B.NUM_KINDS, dtype=torch.float32, device=dev)

    def forward(self, stream=None) -> None:
        for prob, sh in zip(self.problems, self.shards):
            B.lmhead_shard_pass1(prob, sh, self.workspace, stream)
        B.lmhead_shard_merge1(self.problems[0], self.shards[0], self.saved, self.counts, stream)
        for prob, sh in zip(self.problems, self.shards):
            B.lmhead_shard_pass2(prob, sh, self.saved, self.workspace, stream)
        B.lmhead_shard_merge2(self.problems[0], self.shards[0], self.saved, self.counts, self.loss,
                              self.term, self.lse_q,
                              self.reduced if self.term is not None else None, stream)

    def backward(self, grad_loss: Optional[torch.Tensor] = None,
                 grad_mean: Optional[torch.Tensor] = None, dhidden: Optional[torch.Tensor] = None,
                 dW: Optional[torch.Tensor] = None, accumulate_dW: bool = False,
                 want_dh: bool = True, want_dW: bool = True, stream=None):
        h, W = self.inputs["hidden"], self.inputs["W"]
        if dhidden is None and want_dh:
            dhidden = torch.empty(h.shape, dtype=torch.float32, device=h.device)
        if dW is None and want_dW:
            dW = torch.empty(W.shape, dtype=torch.float32, device=W.device)
        parts = None
        if dhidden is not None:
            parts = torch.empty((self.n_shards,) + tuple(h.shape), dtype=torch.float32,
                                device=h.device)
        for g, (prob, sh) in enumerate(zip(self.problems, self.shards)):
            v0, v1 = self.bounds[g], self.bounds[g + 1]
            B.lmhead_shard_bwd(prob, sh, grad_loss, grad_mean, self.counts, self.saved,
                               self.workspace, None if parts is None else parts[g],
                               None if dW is None else dW[v0:v1], accumulate_dW, stream)
        if parts is not None:
            B.specloss_sum_partials(parts, dhidden, stream)
        return dhidden, dW

    def forward_backward(self, *a, **kw):
        raise NotImplementedError("the vocabulary-parallel sequence is forward, then backward")
