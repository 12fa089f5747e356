"""Memory model of the LM-loss path (host arithmetic only).

Streaming cross-entropy post, "The logits bottleneck in long-context
draft-head training": a dense logits tensor takes tokens x vocab x dtype
bytes (twice that with its gradient); "Backward pass": streaming bounds the
loss path's peak by chunk x vocab x dtype x 2.
"""
from __future__ import annotations

GIB = float(1 << 30)


def dense_logits_bytes(tokens: int, vocab: int, dtype_bytes: int = 4, with_grad: bool = False) -> int:
    """Bytes of a materialised [tokens, vocab] logits tensor (x2 with its gradient)."""
    return tokens * vocab * dtype_bytes * (2 if with_grad else 1)


def hidden_bytes(tokens: int, hidden: int, dtype_bytes: int = 2) -> int:
    return tokens * hidden * dtype_bytes


def streaming_bound_bytes(chunk: int, vocab: int, dtype_bytes: int = 4) -> int:
    """The post's bound on the loss path's peak: chunk x vocab x dtype x 2."""
    return chunk * vocab * dtype_bytes * 2


def logits_sized_limit_bytes(tokens: int, vocab: int, dtype_bytes: int = 2) -> int:
    """Size of the [tokens, vocab] logits in the input dtype (bf16 by default): the
    default workspace of the HIP path stays below it."""
    return tokens * vocab * dtype_bytes
