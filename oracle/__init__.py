"""fp64 CPU oracle of the streaming LM-head loss.  TEST INFRASTRUCTURE ONLY.

Imported only by the test suite, the package smoke check and the benchmark's
CPU-baseline leg.  The product path never imports it and has no CPU fallback.
"""
from . import specloss_oracle  # noqa: F401
from .specloss_oracle import (  # noqa: F401
    KINDS, OracleProblem, OracleResult, align_heads, backward, forward, mean_loss, mean_seed,
    row_validity, widen,
)
