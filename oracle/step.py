"""One whole verify step on the CPU: mask, attention, argmax, accept walk.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .argmax import vocab_argmax
from .attention import tree_attention
from .tree import accept_walk, build_masks


def verify_step(parents, draft_tokens, prefix_lens, q, k_cache, v_cache, logits, sm_scale, *,
                q_fmt, kv_fmt, k_scale=None, v_scale=None, V=None):
    """Returns a dict with mask, depth, out, lse, argmax, accept_len,
    path_nodes and out_tokens (numpy arrays; attention in float64)."""
    mask, depth = build_masks(parents)
    out, lse = tree_attention(q, k_cache, v_cache, prefix_lens, parents, sm_scale,
                              q_fmt=q_fmt, kv_fmt=kv_fmt, k_scale=k_scale, v_scale=v_scale)
    t = vocab_argmax(logits)
    if V is None:
        V = np.asarray(logits).shape[1]
    accept_len, path_nodes, out_tokens = accept_walk(parents, draft_tokens, t, V=V)
    return dict(mask=mask, depth=depth, out=out, lse=lse, argmax=t, accept_len=accept_len,
                path_nodes=path_nodes, out_tokens=out_tokens)
