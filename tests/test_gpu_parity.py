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


def test_all_rows_masked():
    p = synthetic.make_problem("ce_bf16_1b", n_rows=100, hidden_dim=64, vocab=300)
    p.mask = np.zeros(100, np.uint8)
    dev = to_device(p)
    run = make_run(p, dev)
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


@pytest.mark.parametrize("kind", ["kl_div", "tv", "nla", "lk_hybrid", "rkl", "jsd"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_call_each_divergence(kind, dtype):
    """Single call per divergence kind over two chunks (the second ragged).

    kl_div, tv, nla and lk_hybrid take the staged path (pass 2 stores q and
    q - p, the logit gradient is formed from them); rkl and jsd run the
    forward and backward back to back.
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


def test_single_call_divergence_matches_two_calls():
    """Staged-divergence single call against the two calls: same losses bit for bit
    (the forward kernels are the same), gradients within the bar of each other."""
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
    full = probe.workspace.numel()
    Vp = -(-p.vocab // 256) * 256
    copies = p.hidden_dim * Vp * 2 + p.hidden_dim * 256 * 2 + Vp * 256 * 2
    del probe
    full_parity(p, max_chunk_rows=256, tag=f"lean-{case}", single_call=single,
                workspace_bytes=full - copies, expect_copies=False)
    # and the default workspace (chunk = all rows here) makes the copies
    full_parity(p, tag=f"copies-{case}", single_call=single, expect_copies=True, flags=0)
    # forced either way at 256-row chunks
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


