"""Buffers for one loss problem and the calls that fill them.

torch allocates every device buffer (inputs stay where the caller put them);
the work itself is the C-ABI calls ``lmhead_loss_fwd`` / ``lmhead_loss_bwd``.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import binding as B


class LossRun:
    """One problem bound to its workspace, forward outputs and saved state."""

    def __init__(self, hidden: torch.Tensor, W: torch.Tensor, weights: Dict[str, float], *,
                 labels: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                 target_hidden: Optional[torch.Tensor] = None, W_t: Optional[torch.Tensor] = None,
                 target_row: Optional[torch.Tensor] = None, max_chunk_rows: int = 0,
                 workspace_bytes: Optional[int] = None, want_terms: bool = True):
        dev = hidden.device
        self.inputs = dict(hidden=hidden, W=W, labels=labels, mask=mask,
                           target_hidden=target_hidden, W_t=W_t, target_row=target_row)
        self.weights = dict(weights)
        self.problem = B.make_problem(hidden, W, weights, labels=labels, mask=mask,
                                      target_hidden=target_hidden, W_t=W_t, target_row=target_row)
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


def lmhead_loss(hidden: torch.Tensor, W: torch.Tensor, weights: Dict[str, float], **kw) -> torch.Tensor:
    """Mean streaming LM-head loss with autograd; gradients flow to hidden and W."""
    run = LossRun(hidden.detach(), W.detach(), weights, **kw)
    return _LMHeadLoss.apply(hidden, W, run)
