"""Paged K/V caches: the token-major page layout of a serving engine's cache.

Test infrastructure only (see the package docstring).

The verify pass runs inside a serving engine (SGLang or vLLM: Aurora, section 2,
the inference server) whose caches are paged.  Reading: the pool holds
num_pages pages of page_size tokens, each token a [Hkv][D] row block
(token-major); request b's logical token t lives in page
block_table[b][t // page_size], slot t % page_size.  Attention over a paged
cache is attention over the gathered contiguous cache, which is what this
module builds.
"""
from __future__ import annotations

import numpy as np


def gather_pages(pages, block_table, page_size: int, S_max: int):
    """pages [num_pages][page_size][Hkv][...] -> contiguous [B][Hkv][S_max][...]
    (token t of request b from page block_table[b][t // page_size])."""
    pages = np.asarray(pages)
    B = len(block_table)
    Hkv = pages.shape[2]
    out = np.empty((B, Hkv, S_max) + pages.shape[3:], dtype=pages.dtype)
    for b in range(B):
        for t in range(S_max):
            page = int(block_table[b][t // page_size])
            out[b, :, t] = pages[page, t % page_size]
    return out
