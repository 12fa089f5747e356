"""libspecloss: streaming LM-head + loss (forward and backward) on MI355X.

The work runs in the HIP library ``libspecloss.so`` (built with
``python -m lm_head_vocab_amd.build``); this package only marshals torch
tensors into its C-ABI.  There is no CPU or eager fallback.
"""
from .binding import (  # noqa: F401
    IGNORE_INDEX, KINDS, SpecLossError, kind_name, lmhead_loss_bwd, lmhead_loss_fwd,
    lmhead_loss_fwd_bwd,
    lmhead_loss_workspace_size, load_library, make_problem, specloss_align_heads,
    specloss_saved_bytes, strerror,
)
from .runner import LossRun, lmhead_loss  # noqa: F401
