"""The allocation-free forward against the forward with a workspace (GPU).

lmhead_loss_fwd_noalloc runs the same kernels as lmhead_loss_fwd on the
library's fixed per-device scratch array instead of a caller workspace.  Two
calls in a row, the second on a smaller problem (the array keeps the first
call's contents), each compared with lmhead_loss_fwd on the same inputs:
per-row losses, terms, logsumexp, saved state and counts bit for bit (the
forward's results do not depend on the chunk), the means within the loss bar.
"""
import ctypes

import numpy as np
import pytest
import torch

import synthetic
import lm_head_vocab_amd as L
from lm_head_vocab_amd import binding as B
from lm_head_vocab_amd.runner import LossRun
from tests._gpu_helpers import LOSS_RTOL, TOKEN_ATOL, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load_library()
    yield


def _outputs(N, dev="cuda"):
    return dict(loss=torch.full((N,), float("nan"), device=dev),
                term=torch.zeros(B.NUM_KINDS, N, device=dev),
                lse=torch.full((N,), float("nan"), device=dev),
                saved=torch.full((B.specloss_saved_bytes(N),), 0xAB, dtype=torch.uint8, device=dev),
                counts=torch.full((2,), -1, dtype=torch.int64, device=dev),
                reduced=torch.full((1 + B.NUM_KINDS,), float("nan"), device=dev))


def _check_against_workspace_call(prob, with_saved):
    say(f"[noalloc] {prob.name} N={prob.n_rows} H={prob.hidden_dim} V={prob.vocab} "
        f"weights={prob.weights} saved={'given' if with_saved else 'scratch'}")
    dev = to_device(prob)
    ref = LossRun(dev["hidden"], dev["W"], prob.weights, labels=dev["labels"], mask=dev["mask"],
                  target_hidden=dev["target_hidden"], W_t=dev["W_t"],
                  target_row=dev["target_row"], heads=prob.shifts)
    ref.forward()
    out = _outputs(prob.n_rows)
    B.lmhead_loss_fwd_noalloc(ref.problem, out["loss"], out["term"], out["lse"],
                              out["saved"] if with_saved else None, out["counts"],
                              out["reduced"])
    torch.cuda.synchronize()
    assert torch.equal(out["counts"], ref.counts)
    assert torch.equal(out["loss"], ref.loss)
    assert torch.equal(out["lse"], ref.lse_q)
    for k in prob.weights:
        i = B.KINDS.index(k)
        assert torch.equal(out["term"][i], ref.term[i]), k
    got, want = out["reduced"].cpu().numpy(), ref.reduced.cpu().numpy()
    assert np.all(np.abs(got - want) <= LOSS_RTOL * np.abs(want) + TOKEN_ATOL), (got, want)
    if with_saved:
        N = prob.n_rows
        for f in range(B.SAVED_FIELDS):
            o = B.specloss_saved_offset(N, f)
            assert torch.equal(out["saved"][o:o + 4 * N], ref.saved[o:o + 4 * N]), f


def test_noalloc_forward_two_calls_second_smaller():
    big = synthetic.make_problem("multihead_bf16_405b", seq_len=700, hidden_dim=256, vocab=5000)
    _check_against_workspace_call(big, with_saved=True)
    small = synthetic.make_problem("ce_bf16_1b", n_rows=300, hidden_dim=128, vocab=900)
    _check_against_workspace_call(small, with_saved=False)


def test_noalloc_forward_rejects_a_problem_beyond_the_scratch():
    """Per-row state alone beyond the fixed array: a clear workspace error, nothing enqueued."""
    p = B.Problem()
    p.n_rows, p.hidden, p.vocab, p.in_dtype = 1 << 22, 256, 4096, B.BF16
    p.hidden_states, p.W, p.labels = 0x10000, 0x20000, 0x30000
    p.weights[B.KINDS.index("ce_label")] = 1.0
    rc = L.load_library().lmhead_loss_fwd_noalloc(ctypes.byref(p), 0x200000, None, None, None,
                                                  0x300000, None, None)
    assert rc == -3
    assert "workspace" in L.strerror(rc)
