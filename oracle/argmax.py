"""Per-node argmax over the target vocabulary logits.

Test infrastructure only (see the package docstring).

The target "verifies" each proposed token (Aurora section 2; Runtime Draft
Model Training, "Overview"); under greedy verification the target's token at
a node is the argmax of its logits.  Reading for ties: the lowest index wins.
The decision is taken in the logits' own precision (float32 compares are
exact), with -0.0 == +0.0 as IEEE comparison says.  Inputs must be finite.
"""
from __future__ import annotations

import numpy as np


def vocab_argmax(logits) -> np.ndarray:
    """logits: float32[rows][V] -> int32[rows], the first index of the row max."""
    x = np.asarray(logits, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] < 1:
        raise ValueError("logits must be [rows][V] with V >= 1")
    if not np.isfinite(x).all():
        raise ValueError("logits must be finite")
    out = np.empty(x.shape[0], dtype=np.int32)
    for r in range(x.shape[0]):
        row = x[r]
        best = row.max()
        out[r] = np.flatnonzero(row == best)[0]
    return out
