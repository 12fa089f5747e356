"""CPU tests of the C-ABI library: exports, host-side validation, memory model.

No compute call reaches the GPU here: every call below fails validation on
the host before anything is enqueued (or is a pure host query).
"""
import ctypes
import json
import os
import re
import subprocess

import pytest
import torch

import lm_head_vocab_amd as L
from lm_head_vocab_amd import binding as B
from lm_head_vocab_amd import memory as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")

E_INVAL, E_UNSUP, E_WS = -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    return L.load_library()


def test_library_exports_every_header_symbol(lib):
    with open(os.path.join(ROOT, "include", "specloss.h")) as f:
        text = f.read()
    decl = re.findall(r"^(?:int|void|size_t|const char\*|specloss_trace\*)\s+(\w+)\s*\(", text, flags=re.M)
    assert set(decl) == set(B.EXPORTS), decl
    for name in decl:
        assert hasattr(lib, name), name


def test_struct_layout_matches_header(tmp_path):
    """The ctypes mirror has the C compiler's size and offsets of specloss_problem."""
    src = tmp_path / "layout.c"
    src.write_text(
        "#include <stddef.h>\n#include <stdio.h>\n#include \"specloss.h\"\n"
        "int main(void) { printf(\"%zu %zu %zu %zu %zu\\n\", sizeof(specloss_problem), "
        "offsetof(specloss_problem, weights), offsetof(specloss_problem, trace), "
        "offsetof(specloss_problem, n_heads), offsetof(specloss_problem, head_shift)); "
        "return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
                    "-I/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got == [ctypes.sizeof(B.Problem), B.Problem.weights.offset, B.Problem.trace.offset,
                   B.Problem.n_heads.offset, B.Problem.head_shift.offset]
    assert ctypes.sizeof(B.Problem) == 160 and B.Problem.weights.offset == 96


def test_kind_names_and_errors(lib):
    assert [L.kind_name(i) for i in range(8)] == list(B.KINDS)
    assert L.kind_name(8) is None and L.kind_name(-1) is None
    assert L.strerror(0) == "success"
    assert "workspace" in L.strerror(E_WS)


def _fake(addr):
    return ctypes.c_void_p(addr)


def _problem(**kw):
    p = B.Problem()
    p.n_rows, p.hidden, p.vocab = kw.get("N", 256), kw.get("H", 256), kw.get("V", 4096)
    p.in_dtype = kw.get("dtype", B.BF16)
    p.hidden_states = kw.get("h", 0x10000)
    p.W = kw.get("W", 0x20000)
    p.labels = kw.get("labels", 0x30000)
    for k, w in kw.get("weights", {"ce_label": 1.0}).items():
        p.weights[B.KINDS.index(k)] = w
    if "target" in kw:
        p.target_hidden, p.W_t, p.n_target_rows = 0x40000, 0x50000, kw["target"]
    return p


def _ws(lib, p):
    out = ctypes.c_size_t()
    return lib.lmhead_loss_workspace_size(ctypes.byref(p), 0, ctypes.byref(out)), out.value


def _fwd(lib, p, ws=0x100000, ws_bytes=1 << 40, loss=0x200000, counts=0x300000):
    return lib.lmhead_loss_fwd(ctypes.byref(p), ws, ws_bytes, loss, None, None, None, counts,
                               None, None)


@pytest.mark.parametrize("mut,code", [
    (dict(H=100), E_UNSUP),
    (dict(H=0), E_INVAL),
    (dict(N=0), E_INVAL),
    (dict(V=-1), E_INVAL),
    (dict(dtype=7), E_UNSUP),
    (dict(weights={}), E_INVAL),
    (dict(weights={"ce_label": float("nan")}), E_INVAL),
    (dict(labels=None), E_INVAL),
    (dict(weights={"tv": 1.0}), E_INVAL),                 # target kind without target
    (dict(weights={"kl_div": 1.0}, target=10), E_INVAL),  # identity map, too few target rows
    (dict(h=0x10008), E_UNSUP),                           # misaligned hidden
    (dict(W=None), E_INVAL),
])
def test_validation(lib, mut, code):
    p = _problem(**mut)
    assert _ws(lib, p)[0] == code
    assert _fwd(lib, p) == code


def test_flags_field_and_null_problem(lib):
    p = _problem()
    for bad in (4, 5, -1):
        p.flags = bad
        assert _fwd(lib, p) == E_INVAL
    p.in_dtype = B.F32
    for flag in (B.FLAG_NO_COPIES, B.FLAG_NO_WEIGHT_COPY):
        p.flags = flag
        assert _fwd(lib, p) == E_UNSUP  # the in-place operands are bf16 only
    out = ctypes.c_size_t()
    assert lib.lmhead_loss_workspace_size(None, 0, ctypes.byref(out)) == E_INVAL
    assert lib.lmhead_loss_fwd(None, 0, 0, 0, None, None, None, 0, None, None) == E_INVAL


def test_fwd_output_checks(lib):
    p = _problem()
    assert _fwd(lib, p, loss=0) == E_INVAL
    assert _fwd(lib, p, counts=0) == E_INVAL
    assert _fwd(lib, p, counts=0x300004) == E_UNSUP
    assert _fwd(lib, p, ws=0) == E_WS
    assert _fwd(lib, p, ws_bytes=1000) == E_WS
    assert _fwd(lib, p, ws=0x100010) == E_WS  # workspace must be 256-byte aligned


def test_bwd_checks(lib):
    p = _problem()
    bwd = lib.lmhead_loss_bwd
    args = dict(gl=0x1000, gm=None, counts=0x2000, saved=0x3000, ws=0x100000, wsb=1 << 40,
                dh=0x4000, dt=B.F32, dW=0x5000)

    def call(**kw):
        a = {**args, **kw}
        return bwd(ctypes.byref(p), a["gl"], a["gm"], a["counts"], a["saved"], a["ws"], a["wsb"],
                   a["dh"], a["dt"], a["dW"], 0, None)

    assert call(gl=None) == E_INVAL
    assert call(saved=None) == E_INVAL
    assert call(counts=None) == E_INVAL
    assert call(dh=None, dW=None) == E_INVAL
    assert call(dt=5) == E_UNSUP
    assert call(wsb=100) == E_WS


def test_fwd_bwd_checks(lib):
    p = _problem()
    f = lib.lmhead_loss_fwd_bwd

    def call(gl=0x1000, gm=None, dh=0x4000, dW=0x5000, dt=B.F32, ws=0x100000, wsb=1 << 40):
        return f(ctypes.byref(p), ws, wsb, 0x200000, None, None, None, 0x300000, None, gl, gm, dh,
                 dt, dW, 0, None)

    assert call(gl=None, gm=None) == E_INVAL
    assert call(dh=None, dW=None) == E_INVAL
    assert call(dt=3) == E_UNSUP
    assert call(ws=0) == E_WS
    assert call(wsb=64) == E_WS


def test_workspace_size_grows_with_chunk_and_stays_below_logits(lib):
    p = _problem(N=32768, H=4096, V=128256)
    sizes = []
    for ch in (256, 1024, 8192):
        out = ctypes.c_size_t()
        assert lib.lmhead_loss_workspace_size(ctypes.byref(p), ch, ctypes.byref(out)) == 0
        sizes.append(out.value)
    assert sizes == sorted(sizes)
    # no buffer reaches a bf16 [N, V] tensor at the 8B shape
    assert sizes[-1] < M.logits_sized_limit_bytes(32768, 128256)


def test_saved_bytes(lib):
    assert L.specloss_saved_bytes(0) == 0
    assert L.specloss_saved_bytes(1) == 10 * 256
    assert L.specloss_saved_bytes(1000) == 10 * 4096


def test_saved_offsets(lib):
    """Fields are consecutive 256-byte aligned arrays of N 4-byte values; bad fields are rejected."""
    for n in (1, 1000, 4097):
        stride = (n * 4 + 255) // 256 * 256
        for f in range(10):
            assert B.specloss_saved_offset(n, f) == f * stride
        assert B.specloss_saved_offset(n, B.SAVED_FLATNESS) + n * 4 <= L.specloss_saved_bytes(n)
    for bad in ((0, 0), (10, -1), (10, 10)):
        with pytest.raises(B.SpecLossError):
            B.specloss_saved_offset(*bad)


def test_align_heads_validation(lib):
    arr = (ctypes.c_int32 * 2)(1, -1)
    assert lib.specloss_align_heads(10, 1, 2, arr, None, 0x1000, 0x2000, None) == E_INVAL
    arr = (ctypes.c_int32 * 1)(1)
    assert lib.specloss_align_heads(0, 1, 1, arr, None, 0x1000, 0x2000, None) == E_INVAL
    assert lib.specloss_align_heads(10, 1, 65, arr, None, 0x1000, 0x2000, None) == E_UNSUP


def test_declared_heads_validation(lib):
    """A declared aligned-heads layout: 1..4 heads, rows a multiple of the head
    count, shifts in [0, 65536], and a target row map when a target kind is on."""
    def heads_problem(K, shifts, N=300, map_=True):
        p = _problem(N=N, weights={"tv": 1.0}, target=100)
        p.target_row = 0x60000 if map_ else None
        p.n_heads = K
        for i, sh in enumerate(shifts):
            p.head_shift[i] = sh
        return p
    assert _ws(lib, heads_problem(3, (1, 2, 3)))[0] == 0
    assert _ws(lib, heads_problem(2, (0, 65536), N=302))[0] == 0
    assert _ws(lib, heads_problem(5, (1, 2, 3, 4)))[0] == E_INVAL
    assert _ws(lib, heads_problem(-1, ()))[0] == E_INVAL
    assert _ws(lib, heads_problem(3, (1, 2, 3), N=301))[0] == E_INVAL
    assert _ws(lib, heads_problem(2, (1, -2)))[0] == E_INVAL
    assert _ws(lib, heads_problem(2, (1, 65537)))[0] == E_INVAL
    assert _ws(lib, heads_problem(3, (1, 2, 3), map_=False))[0] == E_INVAL
    # the single call keeps one raw target row per token of a chunk's span
    # (about a third of the rows with three heads) instead of one per row
    plain = heads_problem(3, (1, 2, 3))
    plain.n_heads = 0
    assert _ws(lib, heads_problem(3, (1, 2, 3)))[1] < _ws(lib, plain)[1]


def test_memory_model_reproduces_page_figures():
    with open(os.path.join(GOLDEN, "page_memory_figures.json")) as f:
        g = json.load(f)["figures"]
    gib = M.GIB
    a, b, c, d = g
    assert abs(M.dense_logits_bytes(a["batch"] * a["seq"], a["vocab"], 4) / gib - a["printed_GiB"]) < a["rounding"]
    assert abs(M.hidden_bytes(b["batch"] * b["seq"], b["hidden"], 2) / gib - b["printed_GiB"]) < b["rounding"]
    assert abs(M.dense_logits_bytes(c["batch"] * c["seq"], c["vocab"], 4, with_grad=True) / gib
               - c["printed_GiB"]) < c["rounding"]
    assert abs(M.streaming_bound_bytes(d["chunk"], d["vocab"], 4) / gib - d["printed_GiB"]) < d["rounding"]
    # the literal 150_000 of the example line does not give the printed value
    assert abs(M.streaming_bound_bytes(1024, 150_000, 4) / gib - 0.97) > 0.1


def test_binding_rejects_bad_dtypes():
    with pytest.raises(ValueError):
        B.make_problem(torch.zeros(4, 64, dtype=torch.float16), torch.zeros(8, 64, dtype=torch.float16), {"ce_label": 1})
    with pytest.raises(ValueError):
        B.make_problem(torch.zeros(4, 64), torch.zeros(8, 64), {"bogus": 1})


def _shard(**kw):
    return B.Shard(vocab_offset=kw.get("off", 0), vocab_total=kw.get("VT", 8192),
                   shard=kw.get("g", 0), n_shards=kw.get("G", 2), exchange=kw.get("x", 0x50000))


def test_exchange_bytes(lib):
    assert L.binding.specloss_exchange_bytes(0, 2) == 0
    assert L.binding.specloss_exchange_bytes(10, 0) == 0
    # 14 fields of [G][round_up(N, 64)] 4-byte entries
    assert L.binding.specloss_exchange_bytes(100, 3) == 14 * 3 * 128 * 4


@pytest.mark.parametrize("bad,code", [
    (dict(g=2), E_INVAL), (dict(g=-1), E_INVAL), (dict(G=0), E_INVAL),
    (dict(off=4097), E_INVAL),            # offset + shard vocab beyond the head
    (dict(VT=0), E_INVAL), (dict(off=-1), E_INVAL),
    (dict(x=0), E_INVAL), (dict(x=0x50010), E_UNSUP),
])
def test_shard_validation(lib, bad, code):
    p = _problem(V=4096)
    sh = _shard(**bad)
    ws = ctypes.c_void_p(0x100000)
    assert lib.lmhead_shard_pass1(ctypes.byref(p), ctypes.byref(sh), ws, 1 << 30, None) == code
    assert lib.lmhead_shard_merge1(ctypes.byref(p), ctypes.byref(sh), ctypes.c_void_p(0x60000),
                                   ctypes.c_void_p(0x70000), None) == code


def test_shard_merge2_needs_terms_for_means(lib):
    p = _problem(V=4096)
    sh = _shard()
    rc = lib.lmhead_shard_merge2(ctypes.byref(p), ctypes.byref(sh), ctypes.c_void_p(0x60000),
                                 ctypes.c_void_p(0x70000), ctypes.c_void_p(0x80000), None, None,
                                 ctypes.c_void_p(0x90000), None)
    assert rc == E_INVAL


def test_sum_partials_validation(lib):
    f = lib.specloss_sum_partials
    assert f(None, 16, 2, ctypes.c_void_p(0x1000), B.F32, None) == E_INVAL
    assert f(ctypes.c_void_p(0x1000), 0, 2, ctypes.c_void_p(0x2000), B.F32, None) == E_INVAL
    assert f(ctypes.c_void_p(0x1000), 16, 0, ctypes.c_void_p(0x2000), B.F32, None) == E_INVAL
    assert f(ctypes.c_void_p(0x1000), 18, 2, ctypes.c_void_p(0x2000), B.F32, None) == E_UNSUP
    assert f(ctypes.c_void_p(0x1008), 16, 2, ctypes.c_void_p(0x2000), B.F32, None) == E_UNSUP
    assert f(ctypes.c_void_p(0x1000), 16, 2, ctypes.c_void_p(0x2000), 7, None) == E_UNSUP


def _shape(name):
    """Problem structs of the five workload shapes (host-only: fake aligned pointers)."""
    if name == "ce_fp32_small":
        return _problem(N=256, H=256, V=4096, dtype=B.F32)
    if name == "ce_bf16_1b":
        return _problem(N=8192, H=2048, V=128256)
    if name == "ce_bf16_8b":
        return _problem(N=32768, H=4096, V=128256)
    if name == "lk_hybrid_bf16_8b":
        return _problem(N=16384, H=4096, V=128256, weights={"lk_hybrid": 1.0}, target=16384)
    p = _problem(N=3 * 4096, H=16384, V=128256, weights={"ce": 0.1, "tv": 0.9}, target=4096)
    p.target_row = 0x60000
    p.n_heads = 3  # the workload declares its token-major heads
    for i, sh in enumerate((1, 2, 3)):
        p.head_shift[i] = sh
    return p


def _chunk(lib, p, ws, call, group=False):
    rows, lay, g = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
    rc = lib.lmhead_loss_chunk(ctypes.byref(p), ws, call, ctypes.byref(rows), ctypes.byref(lay),
                               ctypes.byref(g))
    return (rc, rows.value, B.LAYOUTS[lay.value]) + ((g.value,) if group else ())


@pytest.mark.parametrize("name,chunk,layout,group", [
    ("ce_bf16_1b", 1024, "copies", 4),
    ("ce_bf16_8b", 8192, "copies", 1),
    ("lk_hybrid_bf16_8b", 1280, "copies", 4),
    ("multihead_bf16_405b", 1536, "no_weight_copy", 3),
])
def test_default_chunk_streams_below_the_logits_size(lib, name, chunk, layout, group):
    """Blog, "Backward pass" / "Choosing the chunk size": the default workspace
    streams the token set in chunks well below the token count, and the whole
    workspace stays below the size of the [N, V] logits in the input dtype."""
    p = _shape(name)
    rc, ws = _ws(lib, p)
    assert rc == 0
    limit = M.logits_sized_limit_bytes(p.n_rows, p.vocab)
    assert ws < limit, (ws / 2**30, limit / 2**30)
    assert _chunk(lib, p, ws, B.CALL_FWD_BWD, group=True) == (0, chunk, layout, group)
    assert chunk <= -(-p.n_rows // 4 // 256) * 256
    rc, rows_bwd, _, group_bwd = _chunk(lib, p, ws, B.CALL_BWD, group=True)
    assert rc == 0 and 0 < rows_bwd < p.n_rows and group_bwd == group
    assert _chunk(lib, p, ws, B.CALL_FWD, group=True)[3] == 1  # no dW in the forward


def test_default_chunk_of_a_tiny_problem(lib):
    """When even 256-row chunks do not fit below the logits size (the W^T copy
    alone exceeds it), the smallest chunk with every copy is used."""
    p = _shape("ce_fp32_small")
    rc, ws = _ws(lib, p)
    assert rc == 0 and ws > M.logits_sized_limit_bytes(256, 4096, 4)
    assert _chunk(lib, p, ws, B.CALL_FWD_BWD) == (0, 256, "copies")


def test_chunk_query_validation(lib):
    p = _shape("ce_bf16_8b")
    rows, lay = ctypes.c_int64(), ctypes.c_int32()
    assert lib.lmhead_loss_chunk(ctypes.byref(p), 1 << 40, 3, ctypes.byref(rows),
                                 ctypes.byref(lay), None) == E_INVAL
    assert lib.lmhead_loss_chunk(ctypes.byref(p), 1 << 40, 0, None, ctypes.byref(lay),
                                 None) == E_INVAL
    assert _chunk(lib, p, 1000, B.CALL_BWD)[0] == E_WS
    # flags force the layout
    p.flags = B.FLAG_NO_COPIES
    rc, ws = _ws(lib, p)
    assert rc == 0 and _chunk(lib, p, ws, B.CALL_FWD_BWD)[2] == "no_copies"


@pytest.mark.parametrize("kind", ["rkl", "jsd"])
def test_fwd_bwd_rejects_a_forward_only_workspace(lib, kind):
    """A workspace that holds the forward region but not the single call's is
    rejected before anything is enqueued (no launch happens here: there is no
    GPU)."""
    p = _problem(N=4096, H=4096, V=128256, weights={kind: 1.0}, target=4096)
    ws = 32 << 20
    assert _chunk(lib, p, ws, B.CALL_FWD)[0] == 0
    assert _chunk(lib, p, ws, B.CALL_BWD)[0] == E_WS
    rc = lib.lmhead_loss_fwd_bwd(ctypes.byref(p), 0x100000, ws, 0x200000, None, None, None,
                                 0x300000, None, None, 0x1000, 0x4000, B.F32, 0x5000, 0, None)
    assert rc == E_WS


def test_size_limits(lib):
    """N, V and H below 2^30 are accepted (and the sizing arithmetic stays in
    range); at 2^30 the library answers SPECLOSS_E_UNSUPPORTED."""
    big = (1 << 30) - 64
    for kw in (dict(N=big), dict(V=big), dict(H=big)):
        rc, ws = _ws(lib, _problem(**kw))
        assert rc == 0 and 0 < ws < (1 << 62), (kw, rc, ws)
    for kw in (dict(N=1 << 30), dict(V=1 << 30), dict(H=1 << 30)):
        assert _ws(lib, _problem(**kw))[0] == E_UNSUP, kw
    # the default policy at the largest row count: at least four chunks
    p = _problem(N=big, V=128256, H=4096)
    rc, ws = _ws(lib, p)
    rows, lay = ctypes.c_int64(), ctypes.c_int32()
    assert lib.lmhead_loss_chunk(ctypes.byref(p), ws, 2, ctypes.byref(rows), ctypes.byref(lay),
                                 None) == 0
    assert 0 < rows.value <= 8192


def test_chunk_search_takes_the_largest_fitting_chunk(lib):
    """The workspace a chunk needs is not monotonic in the chunk: at H = 16384
    a 1792-row chunk gives the dh contraction 7 x 64 tiles and four split-K
    slices of fp32 partials, more than a 2048-row chunk (8 x 64 tiles, no
    split) needs.  A workspace sized for 2048 rows must give 2048 rows (without
    copies, so that no dW group is an option)."""
    p = _shape("multihead_bf16_405b")
    p.flags = B.FLAG_NO_COPIES
    sizes = {}
    for rows in (1792, 2048):
        out = ctypes.c_size_t()
        assert lib.lmhead_loss_workspace_size(ctypes.byref(p), rows, ctypes.byref(out)) == 0
        sizes[rows] = out.value
    assert sizes[1792] > sizes[2048]
    for call in (B.CALL_BWD, B.CALL_FWD_BWD):
        assert _chunk(lib, p, sizes[2048], call, group=True) == (0, 2048, "no_copies", 1)
