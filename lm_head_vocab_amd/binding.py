"""ctypes binding of libspecloss (argument marshalling only).

Every function here converts torch tensors to device pointers and calls the
C-ABI entry point of the same name; all computation runs in the HIP library.
There is no fallback: if the library is missing or a call fails, an error is
raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPECLOSS_LIBRARY may name another build of the same sources (the host-sanitized one)
LIB_PATH = os.environ.get("SPECLOSS_LIBRARY") or os.path.join(_PKG, "libspecloss.so")

KINDS = ("ce_label", "ce", "kl_div", "rkl", "jsd", "tv", "nla", "lk_hybrid")
NUM_KINDS = len(KINDS)
MAX_HEADS = 4  # SPECLOSS_MAX_HEADS
F32, BF16 = 0, 1
IGNORE_INDEX = -100
SAVED_FIELDS = 10


class SpecLossError(RuntimeError):
    """A libspecloss call returned an error code."""

    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed: {strerror(code)} ({code})")
        self.code = code


class Problem(ctypes.Structure):
    """Mirror of ``specloss_problem`` in include/specloss.h."""
    _fields_ = [
        ("n_rows", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("hidden_states", ctypes.c_void_p),
        ("W", ctypes.c_void_p),
        ("labels", ctypes.c_void_p),
        ("target_hidden", ctypes.c_void_p),
        ("n_target_rows", ctypes.c_int64),
        ("W_t", ctypes.c_void_p),
        ("target_row", ctypes.c_void_p),
        ("mask", ctypes.c_void_p),
        ("weights", ctypes.c_float * NUM_KINDS),
        ("trace", ctypes.c_void_p),
        ("n_heads", ctypes.c_int32),
        ("head_shift", ctypes.c_int32 * MAX_HEADS),
    ]


_lib: Optional[ctypes.CDLL] = None

EXPORTS = (
    "lmhead_loss_workspace_size",
    "lmhead_loss_chunk",
    "specloss_saved_bytes",
    "specloss_saved_offset",
    "lmhead_loss_fwd",
    "lmhead_loss_fwd_noalloc",
    "lmhead_loss_bwd",
    "lmhead_loss_fwd_bwd",
    "specloss_align_heads",
    "specloss_strerror",
    "specloss_kind_name",
    "specloss_trace_create",
    "specloss_trace_destroy",
    "specloss_trace_reset",
    "specloss_trace_read",
    "specloss_kernel_name",
    "specloss_exchange_bytes",
    "lmhead_shard_pass1",
    "lmhead_shard_merge1",
    "lmhead_shard_pass2",
    "lmhead_shard_merge2",
    "lmhead_shard_bwd",
    "specloss_sum_partials",
)


class Shard(ctypes.Structure):
    """specloss_shard (include/specloss.h)."""
    _fields_ = [
        ("vocab_offset", ctypes.c_int64),
        ("vocab_total", ctypes.c_int64),
        ("shard", ctypes.c_int32),
        ("n_shards", ctypes.c_int32),
        ("exchange", ctypes.c_void_p),
    ]


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libspecloss.so (built in-tree by lm_head_vocab_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m lm_head_vocab_amd.build`; "
                           "there is no fallback implementation")
    lib = ctypes.CDLL(p)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER(Problem)
    lib.lmhead_loss_workspace_size.argtypes = [P, i64, ctypes.POINTER(sz)]
    lib.lmhead_loss_workspace_size.restype = ctypes.c_int
    lib.lmhead_loss_chunk.argtypes = [P, sz, i32, ctypes.POINTER(i64), ctypes.POINTER(i32),
                                      ctypes.POINTER(i32)]
    lib.lmhead_loss_chunk.restype = ctypes.c_int
    lib.specloss_saved_bytes.argtypes = [i64]
    lib.specloss_saved_bytes.restype = sz
    lib.specloss_saved_offset.argtypes = [i64, i32, ctypes.POINTER(sz)]
    lib.specloss_saved_offset.restype = ctypes.c_int
    lib.lmhead_loss_fwd.argtypes = [P, vp, sz, vp, vp, vp, vp, vp, vp, vp]
    lib.lmhead_loss_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.lmhead_loss_fwd_noalloc.restype = ctypes.c_int
    lib.lmhead_loss_fwd.restype = ctypes.c_int
    lib.lmhead_loss_bwd.argtypes = [P, vp, vp, vp, vp, vp, sz, vp, i32, vp, ctypes.c_int, vp]
    lib.lmhead_loss_bwd.restype = ctypes.c_int
    lib.lmhead_loss_fwd_bwd.argtypes = [P, vp, sz, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                        ctypes.c_int, vp]
    lib.lmhead_loss_fwd_bwd.restype = ctypes.c_int
    lib.specloss_align_heads.argtypes = [i64, i64, i32, ctypes.POINTER(i32), vp, vp, vp, vp]
    lib.specloss_align_heads.restype = ctypes.c_int
    S = ctypes.POINTER(Shard)
    lib.specloss_exchange_bytes.argtypes = [i64, i32]
    lib.specloss_exchange_bytes.restype = sz
    lib.lmhead_shard_pass1.argtypes = [P, S, vp, sz, vp]
    lib.lmhead_shard_merge1.argtypes = [P, S, vp, vp, vp]
    lib.lmhead_shard_pass2.argtypes = [P, S, vp, vp, sz, vp]
    lib.lmhead_shard_merge2.argtypes = [P, S, vp, vp, vp, vp, vp, vp, vp]
    lib.lmhead_shard_bwd.argtypes = [P, S, vp, vp, vp, vp, vp, sz, vp, vp, ctypes.c_int, vp]
    lib.specloss_sum_partials.argtypes = [vp, i64, i32, vp, i32, vp]
    for name in ("lmhead_shard_pass1", "lmhead_shard_merge1", "lmhead_shard_pass2",
                 "lmhead_shard_merge2", "lmhead_shard_bwd", "specloss_sum_partials"):
        getattr(lib, name).restype = ctypes.c_int
    lib.specloss_strerror.argtypes = [ctypes.c_int]
    lib.specloss_strerror.restype = ctypes.c_char_p
    lib.specloss_kind_name.argtypes = [ctypes.c_int]
    lib.specloss_kind_name.restype = ctypes.c_char_p
    lib.specloss_trace_create.argtypes = [i32]
    lib.specloss_trace_create.restype = vp
    lib.specloss_trace_destroy.argtypes = [vp]
    lib.specloss_trace_destroy.restype = None
    lib.specloss_trace_reset.argtypes = [vp]
    lib.specloss_trace_reset.restype = None
    lib.specloss_trace_read.argtypes = [vp, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
    lib.specloss_trace_read.restype = ctypes.c_int
    lib.specloss_kernel_name.argtypes = [i32]
    lib.specloss_kernel_name.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().specloss_strerror(code).decode()


def kind_name(kind: int) -> Optional[str]:
    r = load_library().specloss_kind_name(kind)
    return None if r is None else r.decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libspecloss must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(code: int, what: str) -> None:
    if code != 0:
        raise SpecLossError(code, what)


def make_problem(hidden: torch.Tensor, W: torch.Tensor, weights: Dict[str, float], *,
                 labels: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                 target_hidden: Optional[torch.Tensor] = None, W_t: Optional[torch.Tensor] = None,
                 target_row: Optional[torch.Tensor] = None, flags: int = 0,
                 heads: Optional[Sequence[int]] = None) -> Problem:
    """Fill a ``specloss_problem`` from torch tensors (no copies, no checks beyond dtype).

    flags: 0 (automatic), FLAG_COPIES, FLAG_NO_WEIGHT_COPY or FLAG_NO_COPIES (backward layout).
    heads: the shifts of token-major aligned heads (specloss_align_heads's layout), or None.
    """
    if hidden.dtype not in (torch.float32, torch.bfloat16) or W.dtype != hidden.dtype:
        raise ValueError("hidden and W must both be float32 or both bfloat16")
    p = Problem()
    p.n_rows = hidden.shape[0]
    p.hidden = hidden.shape[1]
    p.vocab = W.shape[0]
    p.in_dtype = BF16 if hidden.dtype == torch.bfloat16 else F32
    p.flags = flags
    p.hidden_states = _ptr(hidden)
    p.W = _ptr(W)
    p.labels = _ptr(labels)
    p.target_hidden = _ptr(target_hidden)
    p.n_target_rows = 0 if target_hidden is None else target_hidden.shape[0]
    p.W_t = _ptr(W_t)
    p.target_row = _ptr(target_row)
    p.mask = _ptr(mask)
    for k, w in weights.items():
        if k not in KINDS:
            raise ValueError(f"unknown loss kind {k!r}; known: {KINDS}")
        p.weights[KINDS.index(k)] = float(w)
    if heads:
        if len(heads) > MAX_HEADS:
            raise ValueError(f"at most {MAX_HEADS} aligned heads can be declared")
        p.n_heads = len(heads)
        for i, sh in enumerate(heads):
            p.head_shift[i] = int(sh)
    return p


def lmhead_loss_workspace_size(problem: Problem, max_chunk_rows: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().lmhead_loss_workspace_size(ctypes.byref(problem), max_chunk_rows,
                                                     ctypes.byref(out)), "lmhead_loss_workspace_size")
    return out.value


CALL_FWD, CALL_BWD, CALL_FWD_BWD = 0, 1, 2
LAYOUTS = ("copies", "no_weight_copy", "no_copies")


def lmhead_loss_chunk(problem: Problem, ws_bytes: int, call: int = CALL_FWD_BWD):
    """(rows per chunk, backward layout name, chunks per dW contraction) the
    call uses with ws_bytes of workspace."""
    rows, lay, group = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().lmhead_loss_chunk(ctypes.byref(problem), ws_bytes, call,
                                            ctypes.byref(rows), ctypes.byref(lay),
                                            ctypes.byref(group)),
           "lmhead_loss_chunk")
    return rows.value, LAYOUTS[lay.value], group.value


def specloss_saved_bytes(n_rows: int) -> int:
    return int(load_library().specloss_saved_bytes(n_rows))


# backward layout choice (SPECLOSS_FLAG_* in include/specloss.h)
FLAG_COPIES, FLAG_NO_COPIES, FLAG_NO_WEIGHT_COPY = 1, 2, 3

# public saved fields (SPECLOSS_SAVED_* in include/specloss.h)
SAVED_LSE_Q, SAVED_LSE_P, SAVED_Y_ARG, SAVED_ALPHA, SAVED_VALID, SAVED_FLATNESS = 0, 1, 3, 4, 8, 9


def specloss_saved_offset(n_rows: int, field: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().specloss_saved_offset(n_rows, field, ctypes.byref(out)),
           "specloss_saved_offset")
    return out.value


def lmhead_loss_fwd(problem: Problem, workspace: torch.Tensor, loss: torch.Tensor,
                    term_loss: Optional[torch.Tensor], lse_q: Optional[torch.Tensor],
                    saved: Optional[torch.Tensor], counts: torch.Tensor,
                    reduced: Optional[torch.Tensor], stream=None) -> None:
    _check(load_library().lmhead_loss_fwd(
        ctypes.byref(problem), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(loss), _ptr(term_loss), _ptr(lse_q), _ptr(saved), _ptr(counts), _ptr(reduced),
        _stream(stream)), "lmhead_loss_fwd")


def lmhead_loss_fwd_noalloc(problem: Problem, loss: torch.Tensor,
                            term_loss: Optional[torch.Tensor], lse_q: Optional[torch.Tensor],
                            saved: Optional[torch.Tensor], counts: torch.Tensor,
                            reduced: Optional[torch.Tensor], stream=None) -> None:
    """The forward on the library's fixed per-device scratch (no workspace)."""
    _check(load_library().lmhead_loss_fwd_noalloc(
        ctypes.byref(problem), _ptr(loss), _ptr(term_loss), _ptr(lse_q), _ptr(saved),
        _ptr(counts), _ptr(reduced), _stream(stream)), "lmhead_loss_fwd_noalloc")


def lmhead_loss_bwd(problem: Problem, grad_loss: Optional[torch.Tensor],
                    grad_mean: Optional[torch.Tensor], counts: torch.Tensor, saved: torch.Tensor,
                    workspace: torch.Tensor, dhidden: Optional[torch.Tensor],
                    dW: Optional[torch.Tensor], accumulate_dW: bool = False, stream=None) -> None:
    dh_dtype = BF16 if (dhidden is not None and dhidden.dtype == torch.bfloat16) else F32
    _check(load_library().lmhead_loss_bwd(
        ctypes.byref(problem), _ptr(grad_loss), _ptr(grad_mean), _ptr(counts), _ptr(saved),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(dhidden), dh_dtype,
        _ptr(dW), int(bool(accumulate_dW)), _stream(stream)), "lmhead_loss_bwd")


def lmhead_loss_fwd_bwd(problem: Problem, workspace: torch.Tensor, loss: torch.Tensor,
                        term_loss: Optional[torch.Tensor], lse_q: Optional[torch.Tensor],
                        saved: Optional[torch.Tensor], counts: torch.Tensor,
                        reduced: Optional[torch.Tensor], grad_loss: Optional[torch.Tensor],
                        grad_mean: Optional[torch.Tensor], dhidden: Optional[torch.Tensor],
                        dW: Optional[torch.Tensor], accumulate_dW: bool = False, stream=None) -> None:
    dh_dtype = BF16 if (dhidden is not None and dhidden.dtype == torch.bfloat16) else F32
    _check(load_library().lmhead_loss_fwd_bwd(
        ctypes.byref(problem), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(loss), _ptr(term_loss), _ptr(lse_q), _ptr(saved), _ptr(counts), _ptr(reduced),
        _ptr(grad_loss), _ptr(grad_mean), _ptr(dhidden), dh_dtype, _ptr(dW),
        int(bool(accumulate_dW)), _stream(stream)), "lmhead_loss_fwd_bwd")


def specloss_align_heads(seq_len: int, batch: int, shifts, loss_mask: Optional[torch.Tensor],
                         target_row_out: torch.Tensor, mask_out: torch.Tensor, stream=None) -> None:
    arr = (ctypes.c_int32 * len(shifts))(*[int(s) for s in shifts])
    _check(load_library().specloss_align_heads(seq_len, batch, len(shifts), arr, _ptr(loss_mask),
                                               _ptr(target_row_out), _ptr(mask_out),
                                               _stream(stream)), "specloss_align_heads")


def specloss_exchange_bytes(n_rows: int, n_shards: int) -> int:
    return int(load_library().specloss_exchange_bytes(n_rows, n_shards))


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def lmhead_shard_pass1(problem: Problem, shard: Shard, workspace: torch.Tensor,
                       stream=None) -> None:
    _check(load_library().lmhead_shard_pass1(ctypes.byref(problem), ctypes.byref(shard),
                                             _ptr(workspace), _nbytes(workspace),
                                             _stream(stream)), "lmhead_shard_pass1")


def lmhead_shard_merge1(problem: Problem, shard: Shard, saved: torch.Tensor, counts: torch.Tensor,
                        stream=None) -> None:
    _check(load_library().lmhead_shard_merge1(ctypes.byref(problem), ctypes.byref(shard),
                                              _ptr(saved), _ptr(counts), _stream(stream)),
           "lmhead_shard_merge1")


def lmhead_shard_pass2(problem: Problem, shard: Shard, saved: torch.Tensor,
                       workspace: torch.Tensor, stream=None) -> None:
    _check(load_library().lmhead_shard_pass2(ctypes.byref(problem), ctypes.byref(shard),
                                             _ptr(saved), _ptr(workspace), _nbytes(workspace),
                                             _stream(stream)), "lmhead_shard_pass2")


def lmhead_shard_merge2(problem: Problem, shard: Shard, saved: torch.Tensor, counts: torch.Tensor,
                        loss: torch.Tensor, term_loss: Optional[torch.Tensor],
                        lse_q: Optional[torch.Tensor], reduced: Optional[torch.Tensor],
                        stream=None) -> None:
    _check(load_library().lmhead_shard_merge2(ctypes.byref(problem), ctypes.byref(shard),
                                              _ptr(saved), _ptr(counts), _ptr(loss),
                                              _ptr(term_loss), _ptr(lse_q), _ptr(reduced),
                                              _stream(stream)), "lmhead_shard_merge2")


def lmhead_shard_bwd(problem: Problem, shard: Shard, grad_loss: Optional[torch.Tensor],
                     grad_mean: Optional[torch.Tensor], counts: torch.Tensor, saved: torch.Tensor,
                     workspace: torch.Tensor, dh_partial: Optional[torch.Tensor],
                     dW: Optional[torch.Tensor], accumulate_dW: bool = False,
                     stream=None) -> None:
    for t in (dh_partial, dW):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("dh_partial and dW are fp32")
    _check(load_library().lmhead_shard_bwd(
        ctypes.byref(problem), ctypes.byref(shard), _ptr(grad_loss), _ptr(grad_mean),
        _ptr(counts), _ptr(saved), _ptr(workspace), _nbytes(workspace), _ptr(dh_partial),
        _ptr(dW), int(bool(accumulate_dW)), _stream(stream)), "lmhead_shard_bwd")


def specloss_sum_partials(parts: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """out = parts.sum(0) in order over the leading axis, by the library's kernel."""
    if parts.dtype != torch.float32 or not parts.is_contiguous() or not out.is_contiguous():
        raise TypeError("parts: contiguous fp32 [n_parts, ...]; out: contiguous")
    n = out.numel()
    if parts.numel() != n * parts.shape[0]:
        raise ValueError("parts must hold n_parts copies of out's shape")
    dt = BF16 if out.dtype == torch.bfloat16 else F32
    _check(load_library().specloss_sum_partials(_ptr(parts), n, parts.shape[0], _ptr(out), dt,
                                                _stream(stream)), "specloss_sum_partials")


class Trace:
    """Per-launch HIP-event timing of library calls (specloss_trace_*)."""

    def __init__(self, capacity: int = 4096):
        self._lib = load_library()
        self.handle = self._lib.specloss_trace_create(capacity)
        if not self.handle:
            raise RuntimeError("specloss_trace_create failed")
        self.capacity = capacity

    def attach(self, problem: Problem) -> None:
        problem.trace = self.handle

    def reset(self) -> None:
        self._lib.specloss_trace_reset(self.handle)

    def read(self):
        """List of (kernel name, ms, work) for every recorded launch, in launch order."""
        n = self.capacity
        ids = (ctypes.c_int32 * n)()
        ms = (ctypes.c_float * n)()
        work = (ctypes.c_double * n)()
        cnt = ctypes.c_int32(0)
        _check(self._lib.specloss_trace_read(self.handle, n, ids, ms, work, ctypes.byref(cnt)),
               "specloss_trace_read")
        m = min(cnt.value, n)
        return [(self._lib.specloss_kernel_name(ids[i]).decode(), ms[i], work[i]) for i in range(m)]

    def close(self) -> None:
        if self.handle:
            self._lib.specloss_trace_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
