"""The commit step after verification: keep the accepted path, label outcomes.

Test infrastructure only (see the package docstring).

What it computes, and the reading of the pages it follows:

  * The verify step ends with the accepted draft tokens of each request (the
    accepted path) and, for every proposed token, whether the target accepted
    or rejected it; those outcomes are what the serving engine streams to the
    training buffer (Aurora, everytik.com and chernovdev.ru mirrors, section
    2 "serve-to-train flywheel", description of the inference server and the
    table mapping accepted tokens to positive and rejected proposals to
    negative feedback).
  * Reading: the cache keeps the prefix, the root (tree node 0, the last
    committed token, at row P) and the accepted nodes in path order, so the
    accepted node at depth k moves to row P + k, k = 1..L.  The new prefix
    length is P + 1 + L; the rows after it are free for the next tree.  The
    bonus token (the target's token after the last accepted one) has no K/V
    yet and is not stored.
  * Labels: 2 for the root, 1 for an accepted draft node (on the path), 0 for
    a rejected one.

Everything reads the caches as they were before the step (a plain gather),
with no in-place ordering concerns.
"""
from __future__ import annotations

import numpy as np

LABEL_REJECTED, LABEL_ACCEPTED, LABEL_ROOT = 0, 1, 2


def _check_path(path_row, L, N) -> None:
    if not 0 <= L <= N - 1:
        raise ValueError(f"accept_len {L} is not in [0, {N - 1}]")
    if path_row[0] != 0:
        raise ValueError("the accepted path must start at the root (node 0)")
    for k in range(1, L + 1):
        if not (path_row[k - 1] < path_row[k] < N):
            raise ValueError(f"path node {path_row[k]} at depth {k} is out of order or range")


def commit_accepted(k_cache, v_cache, prefix_lens, accept_len, path_nodes, N):
    """Returns (k_new, v_new, new_prefix_lens int32[B], labels int8[B][N]).

    k_cache, v_cache: arrays [B][Hkv][S_max][...] of any element type (copied,
    not modified); prefix_lens, accept_len int[B]; path_nodes int[B][>= L+1].
    """
    k_new = np.array(k_cache, copy=True)
    v_new = np.array(v_cache, copy=True)
    B = len(prefix_lens)
    new_prefix = np.zeros(B, dtype=np.int32)
    labels = np.zeros((B, N), dtype=np.int8)
    for b in range(B):
        P, L = int(prefix_lens[b]), int(accept_len[b])
        path = [int(x) for x in path_nodes[b]]
        _check_path(path, L, N)
        for k in range(1, L + 1):
            src = P + path[k]
            k_new[b, :, P + k] = k_cache[b, :, src]
            v_new[b, :, P + k] = v_cache[b, :, src]
        new_prefix[b] = P + 1 + L
        labels[b, 0] = LABEL_ROOT
        for k in range(1, L + 1):
            labels[b, path[k]] = LABEL_ACCEPTED
    return k_new, v_new, new_prefix, labels
