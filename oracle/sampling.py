"""Oracle: greedy sampling of a step's logits.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page "The roofline flips: why optimising small models is a different
performance game", section "The point of the title: why it flips in SLMs",
counts the argmax over the logits and the copy of the chosen token back as
per-step work beside the kernels; the NanoFlow review, section "Runtime
details that keep the pipeline fed", forms the next iteration's batch before
the current one finishes.  Neither page defines ties or invalid values; the
reading used here: the token is the lowest index whose logit equals the
row's maximum over its non-NaN entries, and a row with no non-NaN entry
gives token 0.
"""
from __future__ import annotations

import numpy as np


def greedy_token(row) -> int:
    """Greedy choice for one row of logits (float values)."""
    best_i = -1
    best_v = None
    for i, v in enumerate(np.asarray(row, dtype=np.float64).tolist()):
        if v != v:  # NaN
            continue
        if best_v is None or v > best_v:
            best_v, best_i = v, i
    return 0 if best_i < 0 else best_i


def greedy_tokens(logits) -> np.ndarray:
    """Greedy choice for every row of [n_rows, vocab] logits."""
    logits = np.asarray(logits)
    return np.array([greedy_token(r) for r in logits], dtype=np.int32)
