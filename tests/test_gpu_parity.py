"""GPU parity of the HIP path against the fp64 oracle (through the C-ABI).

Small cases cover every loss kind, both dtypes, masks, ignore_index, bad
labels, ragged tails in every dimension (several 256-row vocabulary tiles,
several token tiles, chunks) and the degenerate cases.  Bars: loss and
per-term means rel <= 1e-3, dh/dW rel Frobenius <= 2e-2, masked rows exactly
0, argmax labels exact where the oracle's top-2 gap >= 1e-3, and bitwise
repeatability.
"""
import numpy as np
import pytest
import torch

import synthetic
import lm_head_vocab_amd as L
from oracle import specloss_oracle as O
from lm_head_vocab_amd.runner import ShardedLossRun
from tests._gpu_helpers import (GRAD_FROB, full_parity, make_run, rel_frob, say, to_device)

pytestmark = pytest.mark.gpu

KINDS = ("ce_label", "ce", "kl_div", "rkl", "jsd", "tv", "nla", "lk_hybrid")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_vocab_amd as L
    L.load_library()
    yield


def test_ce_fp32_small_full_size():
    """The small fp32 cross-entropy workload at its full size: every output vs the oracle."""
    p = synthetic.make_problem("ce_fp32_small")
    full_parity(p, tag="c1-full")


def test_ce_bf16_ragged():
    p = synthetic.make_problem("ce_bf16_1b", n_rows=600, hidden_dim=192, vocab=1100)
    full_parity(p, tag="ce-ragged")


def test_ce_bf16_ragged_chunked():
    """Chunks of 256 rows over 600 rows (3 chunks, ragged last)."""
    p = synthetic.make_problem("ce_bf16_1b", n_rows=600, hidden_dim=192, vocab=1100)
    full_parity(p, max_chunk_rows=256, tag="ce-chunked")


def test_lk_hybrid_ragged():
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=300, hidden_dim=128, vocab=777)
    full_parity(p, tag="lk-ragged")


def test_multihead_ce_tv():
    p = synthetic.make_problem("multihead_bf16_405b", seq_len=150, hidden_dim=256, vocab=1000)
    full_parity(p, tag="multihead")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_each_kind(kind, dtype):
    name = "lk_hybrid_bf16_8b"
    p = synthetic.make_problem(name, n_rows=280, hidden_dim=128, vocab=600, weights={kind: 1.0})
    if kind == "ce_label":
        rng = np.random.default_rng(3)
        p.labels = rng.integers(0, p.vocab, p.n_rows).astype(np.int32)
    p.mask = (np.arange(p.n_rows) % 7 != 3).astype(np.uint8)
    if dtype == "f32":
        p.dtype = "f32"
        for f in ("hidden", "W", "target_hidden", "W_t"):
            setattr(p, f, synthetic.bf16_bits_to_f32(getattr(p, f)).copy())
    full_parity(p, tag=f"kind-{kind}-{dtype}")


def test_weighted_mix_all_kinds():
    w = {"ce_label": 0.2, "ce": 0.1, "kl_div": 0.5, "rkl": 0.3, "jsd": 0.7, "tv": 0.9, "nla": 0.4,
         "lk_hybrid": 1.3}
    p = synthetic.make_problem("multihead_bf16_405b", seq_len=120, hidden_dim=128, vocab=700,
                               weights=w)
    rng = np.random.default_rng(5)
    p.labels = rng.integers(0, p.vocab, p.n_rows).astype(np.int32)
    p.labels[::11] = -100
    full_parity(p, tag="mix")


@pytest.mark.parametrize("case", ["kl", "rkl", "mix", "identical"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kl_forward_in_one_sweep(case, dtype):
    """With kl_div and rkl as the only divergences (each row with a target row
    of its own), the two-call forward takes both divergences from one pass
    over both sides (no second sweep, no separate target pass): several
    vocabulary tiles with a ragged tail, 256-row chunks with a ragged last
    one, masked rows, against the oracle; the backward then reads the KL(q||p)
    that pass saved.  Identical distributions give KL = 0."""
    weights = {"kl": {"kl_div": 1.0}, "rkl": {"rkl": 1.0}, "identical": {"kl_div": 1.0, "rkl": 1.0},
               "mix": {"kl_div": 0.5, "rkl": 0.7, "ce": 0.2, "ce_label": 0.3}}[case]
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=700, hidden_dim=192, vocab=1500,
                               weights=weights)
    rng = np.random.default_rng(17)
    p.labels = rng.integers(0, p.vocab, p.n_rows).astype(np.int32)
    p.labels[::13] = -100
    p.mask = (np.arange(p.n_rows) % 9 != 4).astype(np.uint8)
    if case == "identical":
        p.W_t = p.W.copy()
        p.target_hidden = p.hidden.copy()
    if dtype == "f32":
        p.dtype = "f32"
        for f in ("hidden", "W", "target_hidden", "W_t"):
            setattr(p, f, synthetic.bf16_bits_to_f32(getattr(p, f)).copy())
    out = full_parity(p, max_chunk_rows=256, tag=f"kl-one-sweep-{case}-{dtype}",
                      expect_kernels=(["stats_dual"], ["div", "stats_q", "stats_p"]))
    if case == "identical":
        import lm_head_vocab_amd as L
        run = out["run"]
        for k in ("kl_div", "rkl"):
            assert np.all(run.term[L.KINDS.index(k)].cpu().numpy() == 0.0)


def test_determinism_bitwise():
    p = synthetic.make_problem("multihead_bf16_405b", seq_len=100, hidden_dim=128, vocab=900)
    dev = to_device(p)
    outs = []
    for rep in range(2):
        say(f"[determinism] rep {rep}")
        run = make_run(p, dev)
        run.forward()
        dh, dW = run.backward(grad_mean=torch.ones(1, device="cuda"))
        torch.cuda.synchronize()
        fields = [run.saved_field(i, torch.int32).cpu() for i in range(10)]  # bitwise; padding excluded
        outs.append((run.loss.cpu(), run.term.cpu(), *fields, dh.cpu(), dW.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_chunk_size_invariance():
    """Forward and dh do not depend on the chunking; dW only by rounding."""
    p = synthetic.make_problem("ce_bf16_1b", n_rows=700, hidden_dim=128, vocab=900)
    dev = to_device(p)
    res = {}
    for ch in (256, 512, 0):
        say(f"[chunk] max_chunk_rows={ch}")
        run = make_run(p, dev, max_chunk_rows=ch)
        run.forward()
        dh, dW = run.backward(grad_mean=torch.ones(1, device="cuda"))
        torch.cuda.synchronize()
        res[ch] = (run.loss.cpu(), dh.cpu(), dW.cpu().numpy())
    for ch in (256, 512):
        assert torch.equal(res[ch][0], res[0][0])
        assert torch.equal(res[ch][1], res[0][1])
        assert rel_frob(res[ch][2], res[0][2]) < 1e-5


def test_masked_rows_perturbed():
    """Finite garbage in masked rows changes no loss, no dW bit and no unmasked dh bit."""
    p = synthetic.make_problem("ce_bf16_1b", n_rows=300, hidden_dim=128, vocab=800)
    outs = []
    for rep in range(2):
        if rep:
            p.hidden = p.hidden.copy()
            p.hidden[p.mask == 0] = synthetic.f32_to_bf16_bits(
                np.full((int((p.mask == 0).sum()), p.hidden_dim), 37.0, np.float32))
        dev = to_device(p)
        run = make_run(p, dev)
        run.forward()
        dh, dW = run.backward(grad_mean=torch.ones(1, device="cuda"))
        torch.cuda.synchronize()
        outs.append((run.loss.cpu(), dh.cpu(), dW.cpu()))
    m = torch.from_numpy(p.mask != 0)
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][2], outs[1][2])
    assert torch.equal(outs[0][1][m], outs[1][1][m])
    assert torch.all(outs[1][1][~m] == 0)


def test_bad_labels_counted_and_masked():
    p = synthetic.make_problem("ce_bf16_1b", n_rows=260, hidden_dim=64, vocab=500)
    p.labels = p.labels.copy()
    p.labels[[3, 50, 200]] = [500, -7, 100000]
    p.mask[[3, 200]] = 1
    p.mask[[50]] = 0  # a masked bad label is not counted
    out = full_parity(p, tag="bad-labels")
    counts = out["run"].counts.cpu().numpy()
    assert counts[1] == 2


@pytest.mark.parametrize("single", [False, True])
def test_all_rows_masked(single):
    """No valid row: mean 0 and every gradient exactly 0, by the two calls
    and by the single call (whose staged values and dz^T copy are zeros)."""
    p = synthetic.make_problem("ce_bf16_1b", n_rows=100, hidden_dim=64, vocab=300)
    p.mask = np.zeros(100, np.uint8)
    dev = to_device(p)
    run = make_run(p, dev)
    if single:
        dh, dW = run.forward_backward(grad_mean=torch.ones(1, device="cuda"))
    else:
        run.forward()
        dh, dW = run.backward(grad_mean=torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    assert run.counts.cpu().tolist() == [0, 0]
    assert float(run.reduced[0]) == 0.0
    assert torch.all(run.loss == 0) and torch.all(dh == 0) and torch.all(dW == 0)


def test_single_row_and_tiny_vocab():
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=1, hidden_dim=64, vocab=3)
    full_parity(p, tag="tiny")


def test_per_token_seed_and_accumulate():
    """grad_loss seeds per row; accumulate_dW adds onto existing contents."""
    p = synthetic.make_problem("multihead_bf16_405b", seq_len=90, hidden_dim=128, vocab=520)
    dev = to_device(p)
    run = make_run(p, dev)
    run.forward()
    rng = np.random.default_rng(9)
    seed = rng.uniform(-1, 1, p.n_rows)
    g = torch.tensor(seed, dtype=torch.float32, device="cuda")
    base = torch.full(tuple(dev["W"].shape), 0.25, dtype=torch.float32, device="cuda")
    dh, dW = run.backward(grad_loss=g, dW=base.clone(), accumulate_dW=True)
    torch.cuda.synchronize()
    valid, _ = O.row_validity(O.OracleProblem.of(p))
    rdh, rdW = O.backward(p, seed=np.where(valid, seed, 0.0))
    assert rel_frob(dh.cpu().numpy(), rdh) <= GRAD_FROB
    assert rel_frob(dW.cpu().numpy() - 0.25, rdW) <= GRAD_FROB


def test_bf16_dhidden_output():
    p = synthetic.make_problem("ce_bf16_1b", n_rows=300, hidden_dim=128, vocab=700)
    dev = to_device(p)
    run = make_run(p, dev)
    run.forward()
    dh = torch.empty(dev["hidden"].shape, dtype=torch.bfloat16, device="cuda")
    dh, _ = run.backward(grad_mean=torch.ones(1, device="cuda"), dhidden=dh, want_dW=False)
    torch.cuda.synchronize()
    rdh, _ = O.backward(p, want_dW=False)
    assert rel_frob(dh.float().cpu().numpy(), rdh) <= GRAD_FROB


def test_bf16_dhidden_single_call():
    """bf16 dhidden from the single call, whose dh contraction also writes
    dz^T (the bf16-output variant of that kernel); dW from that copy."""
    p = synthetic.make_problem("ce_bf16_1b", n_rows=600, hidden_dim=384, vocab=700)
    dev = to_device(p)
    run = make_run(p, dev, max_chunk_rows=256)
    dh = torch.empty(dev["hidden"].shape, dtype=torch.bfloat16, device="cuda")
    dh, dW = run.forward_backward(grad_mean=torch.ones(1, device="cuda"), dhidden=dh)
    torch.cuda.synchronize()
    rdh, rdW = O.backward(p)
    assert rel_frob(dh.float().cpu().numpy(), rdh) <= GRAD_FROB
    assert rel_frob(dW.cpu().numpy(), rdW) <= GRAD_FROB


def test_align_heads_kernel():
    import lm_head_vocab_amd as L
    S, B, shifts = 37, 3, (1, 2, 5)
    rng = np.random.default_rng(2)
    lm = (rng.uniform(size=S * B) > 0.2).astype(np.uint8)
    n = len(shifts) * B * S
    tr = torch.empty(n, dtype=torch.int32, device="cuda")
    mk = torch.empty(n, dtype=torch.uint8, device="cuda")
    L.specloss_align_heads(S, B, shifts, torch.from_numpy(lm).cuda(), tr, mk)
    torch.cuda.synchronize()
    rtr, rmk = O.align_heads(S, shifts, batch=B, loss_mask=lm)
    assert np.array_equal(tr.cpu().numpy(), rtr) and np.array_equal(mk.cpu().numpy(), rmk)


def test_autograd_wrapper():
    import lm_head_vocab_amd as L
    p = synthetic.make_problem("ce_bf16_1b", n_rows=200, hidden_dim=64, vocab=500)
    dev = to_device(p)
    h = dev["hidden"].clone().requires_grad_(True)
    W = dev["W"].clone().requires_grad_(True)
    loss = L.lmhead_loss(h, W, {"ce_label": 1.0}, labels=dev["labels"], mask=dev["mask"])
    loss.backward()
    mean, _, _ = O.mean_loss(p)
    rdh, rdW = O.backward(p)
    assert abs(loss.item() - mean) <= 1e-3 * abs(mean)
    assert rel_frob(h.grad.float().cpu().numpy(), rdh) <= GRAD_FROB
    assert rel_frob(W.grad.float().cpu().numpy(), rdW) <= GRAD_FROB


def test_autograd_terminal_matches_two_calls():
    """terminal=True runs the single call in the forward: the loss is bitwise the
    two-call one, the gradients agree with it and with the oracle, and an
    upstream scale other than one reaches both gradients."""
    import lm_head_vocab_amd as L
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=300, hidden_dim=128, vocab=900)
    dev = to_device(p)
    kw = dict(labels=dev["labels"], mask=dev["mask"], target_hidden=dev["target_hidden"],
              W_t=dev["W_t"], target_row=dev["target_row"])
    grads = []
    for terminal in (False, True):
        h = dev["hidden"].clone().requires_grad_(True)
        W = dev["W"].clone().requires_grad_(True)
        loss = L.lmhead_loss(h, W, p.weights, terminal=terminal, **kw)
        (2.5 * loss).backward()
        grads.append((loss.item(), h.grad.float().cpu().numpy(), W.grad.float().cpu().numpy()))
    (l0, h0, w0), (l1, h1, w1) = grads
    assert l0 == l1
    mean, _, _ = O.mean_loss(p)
    rdh, rdW = O.backward(p)
    assert abs(l1 - mean) <= 1e-3 * abs(mean)
    # the two-call backward folds the 2.5 into dz before dz is rounded to bf16 for
    # the contractions, the terminal one scales the fp32 result; both gradients are
    # then rounded to bf16 (unit roundoff 2^-8 each): 2^-7 plus the dz rounding
    assert rel_frob(h1, h0) <= 1e-2 and rel_frob(w1, w0) <= 1e-2
    assert rel_frob(h1, 2.5 * rdh) <= GRAD_FROB and rel_frob(w1, 2.5 * rdW) <= GRAD_FROB
    with torch.no_grad():   # no gradient wanted: the forward alone
        assert L.lmhead_loss(dev["hidden"], dev["W"], p.weights, terminal=True, **kw).item() == l0


# ---------------------------------------------------------------- single call
@pytest.mark.parametrize("case", ["c1_full", "ce_ragged", "ce_chunked", "argmax_ce", "mix_ce",
                                  "divergence"])
def test_single_call_forward_backward(case):
    """lmhead_loss_fwd_bwd: staged exp tiles for the cross-entropies, back-to-back otherwise."""
    if case == "c1_full":
        p, ch = synthetic.make_problem("ce_fp32_small"), 0
    elif case == "ce_ragged":
        p, ch = synthetic.make_problem("ce_bf16_1b", n_rows=600, hidden_dim=192, vocab=1100), 0
    elif case == "ce_chunked":
        p, ch = synthetic.make_problem("ce_bf16_1b", n_rows=600, hidden_dim=192, vocab=1100), 256
    elif case == "argmax_ce":
        p = synthetic.make_problem("multihead_bf16_405b", seq_len=150, hidden_dim=128, vocab=900,
                                   weights={"ce": 1.0})
        ch = 256
    elif case == "mix_ce":
        p = synthetic.make_problem("multihead_bf16_405b", seq_len=120, hidden_dim=128, vocab=700,
                                   weights={"ce": 0.3, "ce_label": 0.7})
        rng = np.random.default_rng(4)
        p.labels = rng.integers(0, p.vocab, p.n_rows).astype(np.int32)
        p.labels[::9] = -100
        ch = 0
    else:
        p, ch = synthetic.make_problem("multihead_bf16_405b", seq_len=100, hidden_dim=128,
                                      vocab=800), 256
    full_parity(p, max_chunk_rows=ch, tag=f"single-{case}", single_call=True)


@pytest.mark.parametrize("hidden,chunk,w_in_place", [(192, 256, False), (640, 256, False),
                                                     (640, 0, False), (640, 256, True)])
def test_single_call_dzt_from_dh(hidden, chunk, w_in_place):
    """With both gradients the cross-entropy single call takes dz^T from the dh
    contraction (each workgroup copies the dz slabs whose index equals its
    tile column modulo the tile columns; rows past a chunk's end go out as
    zeros); asked for dW alone, pass 1 stores dz^T itself.  The two must give
    the same dW bits.  H = 640: three tile columns over 1280 / 64 = 20 slabs
    (an uneven share); 256-row chunks of 600 rows: a ragged last chunk and
    split-K dh; w_in_place: the dh contraction reading W in place (no W^T
    copy) writes the copy too.  dh and dW also match the oracle."""
    p = synthetic.make_problem("ce_bf16_1b", n_rows=600, hidden_dim=hidden, vocab=1100)
    say(f"[dzt-from-dh] H={hidden} chunk={chunk} w_in_place={w_in_place}")
    flags = L.binding.FLAG_NO_WEIGHT_COPY if w_in_place else None
    out = full_parity(p, max_chunk_rows=chunk, tag=f"dzt-{hidden}-{chunk}", single_call=True,
                      flags=flags, expect_copies="no_weight_copy" if w_in_place else None,
                      expect_kernels=(("gemm_dh_dzt",), ("gemm_dh",)))
    run = out["run"]
    gm = torch.ones(1, dtype=torch.float32, device="cuda")
    _, dW_only = run.forward_backward(grad_mean=gm, want_dh=False)
    torch.cuda.synchronize()
    assert np.array_equal(dW_only.cpu().numpy(), out["dW"])


@pytest.mark.parametrize("case", ["far", "far_f32", "near", "zero_sum"])
def test_single_call_staged_ce_references(case):
    """The single call stages exp(z - label logit) per row.  far: logits spread
    by about 16 per unit (W ~ N(0,1), H = 256), so most rows have tiles whose
    max exceeds the label logit by more than the staging range and are
    rescaled after the forward; near: the label is the argmax by a wide
    margin (the other staged values are tiny); zero_sum: label and argmax
    weights that cancel, which takes the other staging variant."""
    if case in ("far", "far_f32"):
        p = synthetic.make_problem("ce_bf16_1b", n_rows=300, hidden_dim=256, vocab=1500)
        W = synthetic.bf16_bits_to_f32(p.W) * 50.0  # std 1
        p.W = synthetic.f32_to_bf16_bits(W)
        if case == "far_f32":
            p.dtype = "f32"
            for f in ("hidden", "W"):
                setattr(p, f, synthetic.bf16_bits_to_f32(getattr(p, f)).copy())
    elif case == "near":
        p = synthetic.make_problem("ce_bf16_1b", n_rows=300, hidden_dim=256, vocab=1500)
        h = synthetic.bf16_bits_to_f32(p.hidden).copy()
        W = synthetic.bf16_bits_to_f32(p.W)
        valid = p.labels >= 0
        # the label logit rises by 14: 1 - q_y is about 1500 e^-14 = 1e-3, the
        # label entry of dz; far larger margins put it below the fp32
        # resolution of lse (for any fp32 softmax) and the loss below its ulp
        h[valid] += 14.0 * W[p.labels[valid]] / np.linalg.norm(W[p.labels[valid]], axis=1,
                                                               keepdims=True) ** 2
        p.hidden = synthetic.f32_to_bf16_bits(h)
    else:
        p = synthetic.make_problem("multihead_bf16_405b", seq_len=120, hidden_dim=128, vocab=700,
                                   weights={"ce_label": 0.6, "ce": -0.6})
        rng = np.random.default_rng(8)
        p.labels = rng.integers(0, p.vocab, p.n_rows).astype(np.int32)
    full_parity(p, max_chunk_rows=256, tag=f"staged-{case}", single_call=True)


@pytest.mark.parametrize("kind", ["kl_div", "tv", "nla", "lk_hybrid", "rkl", "jsd"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_call_each_divergence(kind, dtype):
    """Single call per divergence kind over two chunks (the second ragged).

    Pass 2 stores q and q - p (and log q - log p for rkl and jsd) and the
    logit gradient is formed from them, with no logits recomputed.
    """
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=280, hidden_dim=128, vocab=600,
                               weights={kind: 1.0, "ce_label": 0.25})
    rng = np.random.default_rng(5)
    p.labels = rng.integers(0, p.vocab, p.n_rows).astype(np.int32)
    p.mask = (np.arange(p.n_rows) % 7 != 3).astype(np.uint8)
    if dtype == "f32":
        p.dtype = "f32"
        for f in ("hidden", "W", "target_hidden", "W_t"):
            setattr(p, f, synthetic.bf16_bits_to_f32(getattr(p, f)).copy())
    full_parity(p, max_chunk_rows=256, tag=f"single-{kind}-{dtype}", single_call=True)


def test_single_call_log_ratio_kinds_mix_and_two_calls():
    """rkl, jsd, kl_div and tv together in one single call (log q - log p formed
    from the raw logits beside q and q - p), against the oracle and against the
    two calls: the same losses bit for bit (every second sweep adds its sums in
    one order), gradients within the bar of each other."""
    w = {"rkl": 0.5, "jsd": 0.7, "kl_div": 0.2, "tv": 0.4, "ce": 0.1}
    p = synthetic.make_problem("multihead_bf16_405b", seq_len=140, hidden_dim=128, vocab=900,
                               weights=w)
    full_parity(p, max_chunk_rows=256, tag="single-logmix", single_call=True)
    dev = to_device(p)
    gm = torch.ones(1, device="cuda")
    a = make_run(p, dev, max_chunk_rows=256)
    dh1, dW1 = a.forward_backward(grad_mean=gm)
    b = make_run(p, dev, max_chunk_rows=256)
    b.forward()
    dh2, dW2 = b.backward(grad_mean=gm)
    torch.cuda.synchronize()
    assert torch.equal(a.loss, b.loss)
    assert rel_frob(dh1.cpu().numpy(), dh2.cpu().numpy()) < 1e-2
    assert rel_frob(dW1.cpu().numpy(), dW2.cpu().numpy()) < 1e-2


def test_single_call_identical_target_ties():
    """Draft and target identical: p == q exactly, every vocabulary entry is a tie.

    The indicator [q < p] is 1/2 on ties on both sides, so alpha = 1, S = 1/2
    and the tv and kl gradients vanish; only the label cross-entropy is left.
    """
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=300, hidden_dim=128, vocab=700,
                               weights={"tv": 1.0, "kl_div": 0.5, "ce_label": 1.0})
    p.W_t = p.W.copy()
    p.target_hidden = p.hidden.copy()
    rng = np.random.default_rng(6)
    p.labels = rng.integers(0, p.vocab, p.n_rows).astype(np.int32)
    out = full_parity(p, tag="single-ties", single_call=True)
    run = out["run"]
    assert np.allclose(run.saved_field(4).cpu().numpy(), 1.0, atol=1e-5)  # alpha
    assert np.allclose(run.saved_field(5).cpu().numpy(), 0.5, atol=1e-5)  # S


def _traced(run, call):
    trace = L.binding.Trace(capacity=4096)
    trace.attach(run.problem)
    out = call()
    torch.cuda.synchronize()
    names = {n for n, _, _ in trace.read()}
    run.problem.trace = None
    trace.close()
    return names, out


@pytest.mark.parametrize("case", ["mix_bf16", "mix_f32", "heads_bf16"])
def test_raw_and_recomputed_second_sweeps_agree(case):
    """The two calls either keep raw logit rows (a workspace that holds them for
    min(N, 1024) rows: the forward's second sweep reads them, the backward
    recomputes them with the pass-1 contraction and forms dz from them) or
    recompute the tiles (a smaller one, e.g. the allocation-free scratch).
    Forward: the same losses, terms and saved state bit for bit, since every
    sweep adds its sums in one order and the contractions give the same
    logits.  Backward: the same gradient formula in two kernels, so dh and dW
    agree to fp32 rounding (rel. Frobenius 1e-3) and each meets the oracle's
    bar.  Every divergence kind at once (jsd and rkl included); aligned heads
    compare the shared-target-tile sweep."""
    w = {"tv": 0.7, "ce": 0.2, "kl_div": 0.4, "rkl": 0.3, "jsd": 0.5, "nla": 0.2,
         "lk_hybrid": 0.6, "ce_label": 0.1}
    if case == "heads_bf16":
        p = _heads_problem(300, (1, 2, 3), 1, 128, 900, w, seed=29)
        raw_kernel, rec_kernel = "div_raw", "div_heads"
    else:
        p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=700, hidden_dim=128, vocab=900,
                                   weights=w)
        p.labels = np.random.default_rng(5).integers(0, p.vocab, p.n_rows).astype(np.int32)
        raw_kernel, rec_kernel = "div_raw", "div"
    if case == "mix_f32":
        p.dtype = "f32"
        for f in ("hidden", "W", "target_hidden", "W_t"):
            setattr(p, f, synthetic.bf16_bits_to_f32(getattr(p, f)).copy())
    say(f"[sweeps] {case} N={p.n_rows}")
    dev = to_device(p)
    raw = make_run(p, dev, workspace_bytes=256 << 20, flags=None)
    rec = make_run(p, dev, max_chunk_rows=256)  # raw rows for 1024 rows do not fit
    names_raw, _ = _traced(raw, raw.forward)
    names_rec, _ = _traced(rec, rec.forward)
    assert raw_kernel in names_raw and rec_kernel not in names_raw, names_raw
    assert rec_kernel in names_rec and raw_kernel not in names_rec, names_rec
    assert torch.equal(raw.counts, rec.counts)
    assert torch.equal(raw.loss, rec.loss)
    assert torch.equal(raw.term, rec.term)
    valid = torch.from_numpy(O.row_validity(O.OracleProblem.of(p))[0]).cuda()
    for f in range(L.binding.SAVED_FIELDS):
        a_f, b_f = raw.saved_field(f, torch.int32), rec.saved_field(f, torch.int32)
        assert torch.equal(a_f[valid], b_f[valid]), f"saved field {f}"

    gm = torch.ones(1, device="cuda")
    bnames_raw, (dh1, dW1) = _traced(raw, lambda: raw.backward(grad_mean=gm))
    bnames_rec, (dh2, dW2) = _traced(rec, lambda: rec.backward(grad_mean=gm))
    assert "dz_raw" in bnames_raw and "dz" not in bnames_raw, bnames_raw
    assert "dz" in bnames_rec and "dz_raw" not in bnames_rec, bnames_rec
    dh1, dW1, dh2, dW2 = (t.float().cpu().numpy() for t in (dh1, dW1, dh2, dW2))
    assert rel_frob(dh1, dh2) < 1e-3 and rel_frob(dW1, dW2) < 1e-3
    # the raw path of both calls against the oracle
    full_parity(p, workspace_bytes=256 << 20, tag=f"sweeps-raw-{case}",
                expect_kernels=([raw_kernel, "dz_raw"], [rec_kernel, "dz"]))


def test_single_call_divergence_matches_two_calls():
    """Divergence single call (second sweep over the raw logits kept by pass 1)
    against the two calls, whose forward keeps the raw logits too with this
    workspace: the same losses bit for bit, gradients within the bar of each
    other.  The recompute sweep adds the same sums in the same order, which
    test_raw_and_recomputed_second_sweeps_agree checks."""
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=700, hidden_dim=128, vocab=900)
    dev = to_device(p)
    gm = torch.ones(1, device="cuda")
    a = make_run(p, dev, max_chunk_rows=256)
    dh1, dW1 = a.forward_backward(grad_mean=gm)
    b = make_run(p, dev, max_chunk_rows=256)
    b.forward()
    dh2, dW2 = b.backward(grad_mean=gm)
    torch.cuda.synchronize()
    assert torch.equal(a.loss, b.loss)
    assert torch.equal(a.reduced, b.reduced)
    assert rel_frob(dh1.cpu().numpy(), dh2.cpu().numpy()) < 1e-2
    assert rel_frob(dW1.cpu().numpy(), dW2.cpu().numpy()) < 1e-2


def test_single_call_matches_two_calls_and_repeats():
    p = synthetic.make_problem("ce_bf16_1b", n_rows=700, hidden_dim=128, vocab=900)
    dev = to_device(p)
    gm = torch.ones(1, device="cuda")
    outs = []
    for rep in range(2):
        run = make_run(p, dev, max_chunk_rows=256)
        dh, dW = run.forward_backward(grad_mean=gm)
        torch.cuda.synchronize()
        outs.append((run.loss.cpu(), dh.cpu(), dW.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    run = make_run(p, dev, max_chunk_rows=256)
    run.forward()
    dh2, dW2 = run.backward(grad_mean=gm)
    torch.cuda.synchronize()
    assert torch.allclose(run.loss.cpu(), outs[0][0], rtol=1e-5, atol=1e-5)
    assert rel_frob(dh2.cpu().numpy(), outs[0][1].numpy()) < 1e-2
    assert rel_frob(dW2.cpu().numpy(), outs[0][2].numpy()) < 1e-2


def test_flatness_range_and_uniform_rows():
    """Flatness over target rows from uniform to sharply peaked.

    Rows whose target hidden state is zero have u = 0, so p is exactly uniform
    and the score is 1; scaling a row up sharpens p toward one-hot, whose score
    is 1/sqrt(V).  Every valid row is compared with the oracle; invalid rows
    (masked here) read exactly 0.
    """
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=520, hidden_dim=128, vocab=1300,
                               weights={"ce": 1.0, "tv": 0.5})
    th = synthetic.bf16_bits_to_f32(p.target_hidden)
    scale = np.geomspace(0.05, 40.0, p.n_rows)
    scale[::37] = 0.0
    p.target_hidden = synthetic.f32_to_bf16_bits(th * scale[:, None])
    p.mask = (np.arange(p.n_rows) % 11 != 5).astype(np.uint8)
    out = full_parity(p, tag="flatness", check_grads=False)
    flat = out["run"].flatness.cpu().numpy()
    zero = (scale == 0.0) & out["ref"].valid
    assert np.allclose(flat[zero], 1.0, rtol=1e-6), flat[zero]
    v = out["ref"].valid
    assert np.all(flat[v] >= 1.0 / np.sqrt(p.vocab) * (1 - 1e-6)) and np.all(flat[v] <= 1 + 1e-6)
    assert flat[v].min() < 0.2 and flat[v].max() > 0.99   # the sweep spans the range


def test_flatness_single_call_and_chunks():
    """The single call and chunked forwards write the same flatness bits as one unchunked forward."""
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=700, hidden_dim=128, vocab=900,
                               weights={"ce": 1.0})
    dev = to_device(p)
    a = make_run(p, dev)
    a.forward()
    b = make_run(p, dev, max_chunk_rows=256)
    b.forward_backward(grad_mean=torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    fa = a.flatness.view(torch.int32).cpu().numpy()
    fb = b.flatness.view(torch.int32).cpu().numpy()
    assert np.array_equal(fa, fb)
    ref = O.forward(p)
    from tests._gpu_helpers import check_flatness
    check_flatness(a.flatness.cpu().numpy(), ref.flat, ref.valid)



# ---------------------------------------------------------- vocabulary-parallel
@pytest.mark.parametrize("case", ["ce_label_3", "lk_ce_2_ragged", "multihead_4", "kinds_3_f32",
                                  "one_shard"])
def test_vocab_parallel_matches_oracle(case):
    """The shard sequence (pass 1 per shard, merge, pass 2 per shard, merge, local
    backward, dh partial sum) against the oracle, with shard ends inside tiles."""
    if case == "ce_label_3":
        p = synthetic.make_problem("ce_bf16_1b", n_rows=600, hidden_dim=192, vocab=1100)
        sh, ch = (3, [0, 300, 700, 1100]), 256
    elif case == "lk_ce_2_ragged":
        p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=300, hidden_dim=128, vocab=777,
                                   weights={"lk_hybrid": 1.0, "ce": 0.5})
        sh, ch = (2, [0, 333, 777]), 0
    elif case == "multihead_4":
        p = synthetic.make_problem("multihead_bf16_405b", seq_len=100, hidden_dim=128, vocab=1000)
        sh, ch = (4, None), 256
    elif case == "kinds_3_f32":
        p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=280, hidden_dim=128, vocab=900,
                                   weights={"kl_div": 0.3, "rkl": 0.2, "jsd": 0.4, "nla": 0.1,
                                            "ce_label": 0.5})
        rng = np.random.default_rng(8)
        p.labels = rng.integers(0, p.vocab, p.n_rows).astype(np.int32)
        p.labels[::13] = -100
        p.dtype = "f32"
        for f in ("hidden", "W", "target_hidden", "W_t"):
            setattr(p, f, synthetic.bf16_bits_to_f32(getattr(p, f)).copy())
        sh, ch = (3, [0, 256, 512, 900]), 0
    else:
        p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=200, hidden_dim=128, vocab=600,
                                   weights={"tv": 1.0})
        sh, ch = (1, None), 0
    full_parity(p, max_chunk_rows=ch, tag=f"vp-{case}", shards=sh)


def test_vocab_parallel_argmax_tie_across_shards():
    """Two target rows with identical weights in different shards tie on every
    token; where they hold the maximum the merged argmax is the lower index."""
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=256, hidden_dim=128, vocab=768,
                               weights={"ce": 1.0})
    Wt = synthetic.bf16_bits_to_f32(p.W_t)
    hot = synthetic.bf16_bits_to_f32(p.target_hidden).mean(axis=0)
    hot = 3.0 * hot / np.linalg.norm(hot)
    a, b = 100, 600                     # shard 0 and shard 1 of [0, 384, 768]
    Wt[a] = Wt[b] = hot
    p.W_t = synthetic.f32_to_bf16_bits(Wt)
    out = full_parity(p, tag="vp-tie", shards=(2, [0, 384, 768]), check_grads=False)
    y = out["run"].saved_field(3, torch.int32).cpu().numpy()
    g = synthetic.bf16_bits_to_f32(p.target_hidden).astype(np.float64)
    u = g @ synthetic.bf16_bits_to_f32(p.W_t).astype(np.float64).T
    top = u.argmax(axis=1)
    assert np.any(top == a)
    assert np.all(y[top == a] == a)


def test_vocab_parallel_matches_unsharded():
    """Sharded and unsharded runs agree to fp32 rounding (losses, stats) and the bar (grads)."""
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=500, hidden_dim=128, vocab=1300,
                               weights={"lk_hybrid": 1.0, "ce": 0.25})
    dev = to_device(p)
    gm = torch.ones(1, device="cuda")
    a = make_run(p, dev, max_chunk_rows=256)
    a.forward()
    dh1, dW1 = a.backward(grad_mean=gm)
    b = ShardedLossRun(dev["hidden"], dev["W"], p.weights, 3, target_hidden=dev["target_hidden"],
                       W_t=dev["W_t"], max_chunk_rows=256)
    b.forward()
    dh2, dW2 = b.backward(grad_mean=gm)
    torch.cuda.synchronize()
    assert torch.equal(a.counts, b.counts)
    assert torch.allclose(a.loss, b.loss, rtol=1e-5, atol=1e-6)
    assert torch.allclose(a.lse_q, b.lse_q, rtol=1e-6, atol=1e-5)
    assert torch.equal(a.saved_field(3, torch.int32), b.saved_field(3, torch.int32))
    assert torch.allclose(a.flatness, b.flatness, rtol=1e-5)
    assert rel_frob(dh1.cpu().numpy(), dh2.cpu().numpy()) < 1e-3
    assert rel_frob(dW1.cpu().numpy(), dW2.cpu().numpy()) < 1e-3



# ------------------------------------------------------ backward without copies
@pytest.mark.parametrize("case", ["ce_two_calls", "ce_single", "lk_single", "kinds_two_calls",
                                  "multihead_single"])
def test_backward_without_transposed_copies(case):
    """A workspace too small for the transposed copies of W, h and dz selects the
    copy-free contractions (MN-major operands through the transposing LDS
    load); same bar against the oracle, and no transpose in the trace."""
    single = case.endswith("single")
    if case.startswith("ce"):
        p = synthetic.make_problem("ce_bf16_1b", n_rows=600, hidden_dim=192, vocab=1100)
    elif case == "lk_single":
        p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=700, hidden_dim=128, vocab=900,
                                   weights={"lk_hybrid": 1.0, "ce": 0.3})
    elif case == "kinds_two_calls":
        p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=300, hidden_dim=256, vocab=777,
                                   weights={"rkl": 0.5, "jsd": 0.5, "tv": 1.0})
    else:
        p = synthetic.make_problem("multihead_bf16_405b", seq_len=150, hidden_dim=128, vocab=1000)
    import lm_head_vocab_amd as L
    dev = to_device(p)
    probe = make_run(p, dev, max_chunk_rows=256)
    # the smallest workspace that runs the backward at 256-row chunks: it
    # holds none of the transposed copies
    call = L.binding.CALL_FWD_BWD if single else L.binding.CALL_BWD
    probe.problem.flags = 0  # the layout chosen by workspace size

    def rows_at(ws):
        try:
            return L.binding.lmhead_loss_chunk(probe.problem, ws, call)[0]
        except L.binding.SpecLossError:
            return 0

    lo, hi = 1, probe.workspace_bytes
    while lo < hi:
        mid = (lo + hi) // 2
        if rows_at(mid) >= 256:
            hi = mid
        else:
            lo = mid + 1
    assert L.binding.lmhead_loss_chunk(probe.problem, lo, call) == (256, "no_copies", 1)
    if not single:
        assert L.binding.lmhead_loss_chunk(probe.problem, lo, L.binding.CALL_FWD)[0] >= 256
    del probe
    full_parity(p, max_chunk_rows=256, tag=f"lean-{case}", single_call=single,
                workspace_bytes=lo, expect_copies=False)
    # each layout forced: every copy with one chunk of all rows, and at
    # 256-row chunks the dW copies without W^T, and no copy
    full_parity(p, tag=f"copies-{case}", single_call=single, expect_copies=True,
                flags=L.binding.FLAG_COPIES)
    full_parity(p, max_chunk_rows=256, tag=f"noweightcopy-{case}", single_call=single,
                expect_copies="no_weight_copy", flags=L.binding.FLAG_NO_WEIGHT_COPY)
    full_parity(p, max_chunk_rows=256, tag=f"nocopies-{case}", single_call=single,
                expect_copies=False, flags=L.binding.FLAG_NO_COPIES)


@pytest.mark.parametrize("single", [False, True])
def test_shared_target_rows_match_per_row(single):
    """Rows that share target rows (three aligned heads) take their target
    statistics from one pass over the distinct target rows; the same problem
    with every row's target copied out (no sharing) gives the same bits."""
    p = synthetic.make_problem("multihead_bf16_405b", seq_len=200, hidden_dim=128, vocab=900,
                               weights={"ce": 0.4, "tv": 0.6})
    assert p.target_hidden.shape[0] < p.n_rows
    tr = np.where(p.target_row >= 0, p.target_row, 0)
    q = synthetic.make_problem("multihead_bf16_405b", seq_len=200, hidden_dim=128, vocab=900,
                               weights={"ce": 0.4, "tv": 0.6})
    q.target_hidden = p.target_hidden[tr].copy()
    q.target_row = None
    q.shifts = None  # no aligned-heads layout without a row map
    gm = torch.ones(1, device="cuda")
    outs = []
    for prob in (p, q):
        run = make_run(prob, to_device(prob), max_chunk_rows=256)
        if single:
            dh, dW = run.forward_backward(grad_mean=gm)
        else:
            run.forward()
            dh, dW = run.backward(grad_mean=gm)
        torch.cuda.synchronize()
        outs.append(dict(loss=run.loss.cpu(), lse_p=run.saved_field(1).cpu(),
                         y=run.saved_field(3, torch.int32).cpu(), alpha=run.saved_field(4).cpu(),
                         flat=run.flatness.cpu(), dh=dh.cpu(), dW=dW.cpu()))
    a, b = outs
    valid = torch.from_numpy(p.mask.astype(bool))
    for k in ("loss", "lse_p", "y", "alpha", "flat"):
        assert torch.equal(a[k][valid], b[k][valid]), k
    assert torch.equal(a["dh"], b["dh"]) and torch.equal(a["dW"], b["dW"])




# ------------------------------------------------------ aligned heads: shared target tiles
def _heads_problem(S, shifts, batch, H, V, weights, seed):
    """Token-major aligned heads (specloss_align_heads's layout) over `batch`
    sequences of S positions: valid rows carry the target hidden state of their
    target position, the others fresh N(0,1) rows; W ~ N(0, 0.1), W_t = W +
    N(0, 0.02) (bf16)."""
    rng = np.random.default_rng(seed)
    K = len(shifts)
    bf = synthetic.f32_to_bf16_bits
    g = rng.standard_normal((batch * S, H), dtype=np.float32)
    tr, mk = O.align_heads(S, shifts, batch=batch)
    hidden = rng.standard_normal((K * batch * S, H), dtype=np.float32)
    hidden[tr >= 0] = g[tr[tr >= 0]]
    W = 0.1 * rng.standard_normal((V, H), dtype=np.float32)
    Wt = W + 0.02 * rng.standard_normal((V, H), dtype=np.float32)
    p = synthetic.Problem(name="aligned_heads", dtype="bf16", n_rows=K * batch * S, hidden_dim=H,
                          vocab=V, hidden=bf(hidden), W=bf(W), weights=dict(weights),
                          mask=mk.astype(np.uint8), target_hidden=bf(g), W_t=bf(Wt),
                          target_row=tr.astype(np.int32), seq_len=S, shifts=tuple(shifts))
    p.labels = rng.integers(0, V, p.n_rows).astype(np.int32)
    return p


@pytest.mark.parametrize("case", ["k3_single", "k3_two_calls", "k2_batch_single",
                                  "k3_far_shifts_single", "k3_wide_shifts_single",
                                  "k3_lean_single", "k3_tv_single",
                                  "k4_single_per_row", "k3_f32_two_calls_per_row"])
def test_aligned_heads_share_target_tiles(case):
    """Declared token-major heads: each target tile is computed once for the
    heads it serves instead of once per row -- in the two-call forward's second
    sweep (k_div_heads), and in the single call's pass 1, which keeps one raw
    target row per token of a chunk's span (its target contractions then do
    about a third of the work of the per-row ones).  Against the oracle (the
    bar), and bit for bit against the same problem without the declaration:
    losses, terms, saved state, gradients.  256-row chunks split tokens between
    chunks (256 is no multiple of 3).  Four heads and fp32 inputs keep the
    per-row path (same checks)."""
    import lm_head_vocab_amd as L
    single = "single" in case
    shifts, batch = {"k3_single": ((1, 2, 3), 1), "k3_two_calls": ((1, 2, 3), 1),
                     "k2_batch_single": ((2, 0), 3), "k3_far_shifts_single": ((0, 7, 70), 2),
                     # spans overlap by more than a chunk advances: no rows are carried
                     "k3_wide_shifts_single": ((0, 1, 150), 1),
                     "k3_lean_single": ((1, 2, 3), 1), "k3_tv_single": ((1, 2, 3), 1),
                     "k4_single_per_row": ((1, 2, 3, 4), 1),
                     "k3_f32_two_calls_per_row": ((1, 2, 3), 1)}[case]
    weights = ({"tv": 0.7, "ce": 0.2, "kl_div": 0.4, "rkl": 0.3, "jsd": 0.5, "nla": 0.2,
                "lk_hybrid": 0.6, "ce_label": 0.1} if case not in ("k2_batch_single", "k3_tv_single")
               else {"lk_hybrid": 1.0, "ce": 0.3} if case == "k2_batch_single"
               else {"tv": 0.9, "ce": 0.1})  # tv + ce: the sum set taken as a constant
    S = 310 if batch == 1 else 170
    p = _heads_problem(S, shifts, batch, 128, 900, weights, seed=71)
    if "f32" in case:
        p.dtype = "f32"
        for f in ("hidden", "W", "target_hidden", "W_t"):
            setattr(p, f, synthetic.bf16_bits_to_f32(getattr(p, f)).copy())
    flags = L.binding.FLAG_NO_COPIES if case == "k3_lean_single" else None
    per_row = case.endswith("per_row")
    if single:
        shared = plain = "div_raw"
        stage, absent = "div_raw", "div"
    else:
        shared, plain = "div_heads", "div"
        stage, absent = (plain, shared) if per_row else (shared, plain)
    out = full_parity(p, max_chunk_rows=256, tag=f"heads-{case}", single_call=single, flags=flags,
                      expect_kernels=([stage], [absent]))
    run = out["run"]
    dev = to_device(p)
    ref = make_run(p, dev, max_chunk_rows=256, heads=None,
                   **({"flags": flags} if flags is not None else {}))
    trace = L.binding.Trace(capacity=4096)
    trace.attach(ref.problem)
    gm = torch.ones(1, dtype=torch.float32, device="cuda")
    if single:
        dh, dW = ref.forward_backward(grad_mean=gm)
    else:
        ref.forward()
        dh, dW = ref.backward(grad_mean=gm)
    torch.cuda.synchronize()
    recs = trace.read()
    names = {n for n, _, _ in recs}
    ref.problem.trace = None
    trace.close()
    if single:
        assert "div_raw" in names, names
        target_work = lambda rs: sum(w for n, _, w in rs if n == "stats_p")
        if not per_row:
            # spans of about N / K rows per chunk plus the shift spread; the
            # wide shifts overlap most of a span with the next one's
            bound = 0.8 if case == "k3_wide_shifts_single" else 0.7
            assert target_work(out["trace"]) < bound * target_work(recs)
    else:
        assert plain in names and shared not in names, names
    assert torch.equal(run.loss, ref.loss)
    assert torch.equal(run.term, ref.term)
    assert torch.equal(run.counts, ref.counts)
    # saved state of valid rows (masked rows pair with a different unused target row)
    valid = torch.from_numpy(p.mask.astype(bool)).cuda()
    for f in range(L.binding.SAVED_FIELDS):
        a_f, b_f = run.saved_field(f, torch.int32), ref.saved_field(f, torch.int32)
        assert torch.equal(a_f[valid], b_f[valid]), f"saved field {f}"
    assert np.array_equal(out["dh"], dh.cpu().numpy())
    assert np.array_equal(out["dW"], dW.cpu().numpy())


@pytest.mark.parametrize("single", [False, True])
def test_jsd_with_underflowing_probabilities(single):
    """Logits spread over hundreds of nats: most p_v and q_v underflow to 0 in
    fp32, where the Jensen-Shannon terms p log(p/m) and q log(q/m) must vanish
    (x log x -> 0) rather than turn into 0 * inf; every output stays finite
    and within the bar of the fp64 oracle (JSD is insensitive to a common
    error in log p and log q, so fp32's resolution of such large logits does
    not enter).  The vocabulary (777) ends inside a tile, so padded rows are
    covered too."""
    p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=300, hidden_dim=128, vocab=777,
                               weights={"jsd": 1.0})
    wide = lambda x: synthetic.bf16_bits_to_f32(x).astype(np.float32)
    p.W = synthetic.f32_to_bf16_bits(wide(p.W) * 300.0)
    p.W_t = synthetic.f32_to_bf16_bits(wide(p.W_t) * 300.0)
    ref = O.forward(p)
    z = wide(p.hidden).astype(np.float64) @ wide(p.W).astype(np.float64).T
    assert np.mean(z.max(axis=1, keepdims=True) - z > 110.0) > 0.3  # exp underflows in fp32
    out = full_parity(p, max_chunk_rows=256, tag=f"jsd-underflow-{single}", single_call=single)
    assert np.all(np.isfinite(out["loss"])) and np.all(np.isfinite(out["dh"]))
    assert np.all(np.isfinite(out["dW"]))


# ---------------------------------------------------------------- dW groups
def _dw_group_workspace(prob, call, flags, group):
    """A workspace with which `call` contracts `group` chunks per dW launch
    over a number of chunks that leaves a shorter last group, whose last
    chunk is ragged."""
    dev = to_device(prob)
    probe = make_run(prob, dev, max_chunk_rows=256, flags=flags)
    for rows in range(1024, prob.n_rows + 256, 256):
        ws = L.binding.lmhead_loss_workspace_size(probe.problem, rows)
        nc, _, g = L.binding.lmhead_loss_chunk(probe.problem, ws, call)
        chunks = -(-prob.n_rows // nc)
        if g == group and chunks > group and chunks % group and prob.n_rows % nc:
            return ws, nc
    raise AssertionError(f"no workspace gives a dW group of {group}")


@pytest.mark.parametrize("case", ["ce_single_2", "ce_two_2", "ce32_two_2", "lk_single_2",
                                  "lk_two_2", "kl_two_2", "heads_single_2", "ce_single_3",
                                  "ce_single_4", "ce32_two_3", "lk_single_4", "lk_two_4"])
def test_dw_group_matches_oracle(case):
    """G chunks per dW contraction (each writes its columns of dz^T and h^T
    copies G chunks wide): parity with the oracle, and one dW launch per
    group in the trace.  A group must save two contractions, hence seven or
    more chunks here (eleven in fp32, whose copies take more of the space)."""
    kind, calls, group = case.split("_")
    group = int(group)
    single = calls == "single"
    flags = 0
    if kind in ("ce", "ce32"):
        p = synthetic.make_problem("ce_bf16_1b", n_rows=11000 if kind == "ce32" else 7000,
                                   hidden_dim=128, vocab=700)
        if kind == "ce32":
            p.dtype = "f32"
            for f in ("hidden", "W"):
                setattr(p, f, synthetic.bf16_bits_to_f32(getattr(p, f)).copy())
    elif kind == "heads":
        p = synthetic.make_problem("multihead_bf16_405b", seq_len=2334, hidden_dim=128, vocab=700)
        flags = L.binding.FLAG_NO_WEIGHT_COPY
    else:
        w = {"lk": {"lk_hybrid": 1.0}, "kl": {"kl_div": 1.0}}[kind]
        p = synthetic.make_problem("lk_hybrid_bf16_8b", n_rows=7000, hidden_dim=128, vocab=700,
                                   weights=w)
    call = L.binding.CALL_FWD_BWD if single else L.binding.CALL_BWD
    ws, nc = _dw_group_workspace(p, call, flags, group)
    out = full_parity(p, workspace_bytes=ws, single_call=single, flags=flags,
                      tag=f"dw-group-{case}", expect_kernels=(("gemm_dW",), ()))
    n_dw = sum(1 for name, _, _ in out["trace"] if name == "gemm_dW")
    assert n_dw == -(-(-(-p.n_rows // nc)) // group), (n_dw, nc, group)
    # accumulate_dW adds every group onto the caller's dW
    run = out["run"]
    gm = torch.ones(1, dtype=torch.float32, device="cuda")
    dW = torch.from_numpy(out["dW"]).cuda()
    call = run.forward_backward if single else run.backward
    call(grad_mean=gm, dW=dW, accumulate_dW=True, want_dh=False)
    torch.cuda.synchronize()
    assert rel_frob(dW.cpu().numpy(), 2.0 * out["dW"]) <= 1e-5
