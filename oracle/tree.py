"""Tree structure: ancestor sets, 64-bit ancestor masks and the accept walk.

Test infrastructure only (see the package docstring).

Conventions (readings of the pages, which describe the tree only as "the
causal structure of the speculative tree", Aurora section 2, closing
paragraph):

  * a draft tree with N nodes is a parent array p[0..N-1] with p[0] = -1 (the
    root, i.e. the last committed token) and 0 <= p[i] < i for i >= 1;
  * anc*(i) = {i, p[i], p[p[i]], ..., 0}: a node sees itself and its
    ancestors (ancestor-or-self);
  * depth(i) = |anc*(i)| - 1, counted in edges from the root.
"""
from __future__ import annotations

import numpy as np

MAX_NODES = 64


def _check_parents(p) -> None:
    n = len(p)
    if not 1 <= n <= MAX_NODES:
        raise ValueError(f"tree has {n} nodes; 1..{MAX_NODES} supported")
    if p[0] != -1:
        raise ValueError("parents[0] must be -1 (the root)")
    for i in range(1, n):
        if not 0 <= p[i] < i:
            raise ValueError(f"parents[{i}] = {p[i]} is not in [0, {i})")


def ancestors(p, i: int) -> list[int]:
    """anc*(i) listed from i up to the root, by walking parent pointers."""
    out = [i]
    while p[out[-1]] != -1:
        out.append(int(p[out[-1]]))
    return out


def children_of(p) -> list[list[int]]:
    kids: list[list[int]] = [[] for _ in range(len(p))]
    for i in range(1, len(p)):
        kids[int(p[i])].append(i)
    return kids


def build_masks(parents) -> tuple[np.ndarray, np.ndarray]:
    """Ancestor-or-self bitmasks and depths for a batch of trees.

    parents: int[B][N].  Returns (mask uint64[B][N], depth int32[B][N]) where
    bit j of mask[b][i] is set iff j is in anc*(i) of request b.
    Raises ValueError on an invalid parent array.
    """
    parents = np.asarray(parents)
    B, N = parents.shape
    mask = np.zeros((B, N), dtype=np.uint64)
    depth = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        p = [int(x) for x in parents[b]]
        _check_parents(p)
        for i in range(N):
            a = ancestors(p, i)
            bits = 0
            for j in a:
                bits |= 1 << j
            mask[b, i] = np.uint64(bits)
            depth[b, i] = len(a) - 1
    return mask, depth


def accept_walk(parents, draft_tokens, target_argmax, V: int | None = None):
    """Accept walk for a batch of trees.

    Reading of the step (the pages give only its result, acceptance length =
    draft tokens accepted per verification step, Runtime Draft Model
    Training, "Evaluation"; Aurora section 2 maps maximal return to maximal
    acceptance length):

      t[i] = the target's argmax at node i;
      node i >= 1 *matches* iff draft_tokens[i] == t[p[i]] (the target, having
      read the path up to p[i], would have produced exactly i's draft token);
      walk(u) returns the best (depth, end node) reachable from u through
      matched children: deeper wins, equal depth goes to the lower end index;
      (L, e) = walk(0); the accepted path is anc*(e) from the root down.

    Returns (accept_len int32[B], path_nodes int32[B][N], out_tokens
    int32[B][N]); path_nodes[k] is the path's node at depth k and
    out_tokens[k] = t[path_nodes[k]] for k = 0..L (the L accepted draft tokens
    followed by the target's bonus token), both padded with -1.
    """
    parents = np.asarray(parents)
    draft_tokens = np.asarray(draft_tokens)
    target_argmax = np.asarray(target_argmax).reshape(parents.shape)
    B, N = parents.shape
    accept_len = np.zeros(B, dtype=np.int32)
    path_nodes = np.full((B, N), -1, dtype=np.int32)
    out_tokens = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        p = [int(x) for x in parents[b]]
        _check_parents(p)
        d = [int(x) for x in draft_tokens[b]]
        t = [int(x) for x in target_argmax[b]]
        if V is not None:
            for x in d + t:
                if not 0 <= x < V:
                    raise ValueError(f"token {x} outside [0, {V})")
        kids = children_of(p)

        def matches(c: int) -> bool:
            return d[c] == t[p[c]]

        def walk(u: int, depth_u: int) -> tuple[int, int]:
            best = (depth_u, u)
            for c in kids[u]:          # increasing index order
                if matches(c):
                    r = walk(c, depth_u + 1)
                    if r[0] > best[0] or (r[0] == best[0] and r[1] < best[1]):
                        best = r
            return best

        L, e = walk(0, 0)
        path = ancestors(p, e)[::-1]   # root first, increasing depth
        assert len(path) == L + 1
        accept_len[b] = L
        for k, node in enumerate(path):
            path_nodes[b, k] = node
            out_tokens[b, k] = t[node]
    return accept_len, path_nodes, out_tokens
