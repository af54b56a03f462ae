"""Pins for the CPU oracle: checks against closed forms, brute force and
independent library routines.  Each check takes the oracle routine under test
as an argument, so ``test_oracle_mutations.py`` can run the same checks on a
deliberately broken copy of the oracle and confirm that they fail.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers

def all_parent_arrays(n: int):
    """Every valid parent array with n nodes (p[0] = -1, 0 <= p[i] < i)."""
    for tail in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1, *tail]


def closure_masks(p) -> list[int]:
    """Ancestor-or-self sets by transitive closure of the child->parent
    relation (Warshall), an algorithm independent of parent-pointer walks."""
    n = len(p)
    R = [[i == j for j in range(n)] for i in range(n)]
    for i in range(1, n):
        R[i][p[i]] = True
    for k in range(n):
        for i in range(n):
            if R[i][k]:
                for j in range(n):
                    if R[k][j]:
                        R[i][j] = True
    return [sum(1 << j for j in range(n) if R[i][j]) for i in range(n)]


def brute_force_walk(p, d, t):
    """Enumerate every root-to-node path, keep the fully matched ones and take
    the deepest, ties to the lower end index."""
    n = len(p)
    best = None
    for e in range(n):
        path = [e]
        while path[-1] != 0:
            path.append(p[path[-1]])
        path = path[::-1]
        if all(d[path[k]] == t[path[k - 1]] for k in range(1, len(path))):
            key = (len(path) - 1, -e)
            if best is None or key > best[0]:
                best = (key, path)
    L = best[0][0]
    path = best[1]
    return L, path, [t[x] for x in path]


def read_golden(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def ints(s: str) -> list[int]:
    return [int(x, 0) for x in s.split()]


# ------------------------------------------------------------------- mask

def check_mask_golden(build_masks):
    for name, par, masks, depths in read_golden("mask_hand_examples.txt"):
        m, dep = build_masks(np.array([ints(par)], dtype=np.int32))
        assert [int(x) for x in m[0]] == ints(masks), name
        assert [int(x) for x in dep[0]] == ints(depths), name


def check_mask_closed_forms(build_masks):
    for n in (1, 2, 6, 33, 63, 64):
        chain = np.arange(-1, n - 1, dtype=np.int32)[None]
        m, dep = build_masks(chain)
        assert [int(x) for x in m[0]] == [(1 << (i + 1)) - 1 for i in range(n)]
        assert list(dep[0]) == list(range(n))
        star = np.array([[-1] + [0] * (n - 1)], dtype=np.int32)
        m, dep = build_masks(star)
        assert [int(x) for x in m[0]] == [1] + [1 | (1 << i) for i in range(1, n)]
        assert list(dep[0]) == [0] + [1] * (n - 1)


def check_mask_brute_force(build_masks, max_n: int = 7):
    for n in range(1, max_n + 1):
        arrs = list(all_parent_arrays(n))
        m, dep = build_masks(np.array(arrs, dtype=np.int32))
        for b, p in enumerate(arrs):
            want = closure_masks(p)
            assert [int(x) for x in m[b]] == want, p
            assert [int(x) for x in dep[b]] == [bin(w).count("1") - 1 for w in want], p


# ------------------------------------------------------------------- walk

def check_walk_golden(accept_walk):
    for name, par, d, t, L, path, toks in read_golden("walk_hand_examples.txt"):
        p = ints(par)
        n = len(p)
        al, pn, ot = accept_walk(np.array([p]), np.array([ints(d)]), np.array([ints(t)]))
        Lw = int(L)
        assert int(al[0]) == Lw, name
        assert list(pn[0]) == ints(path) + [-1] * (n - Lw - 1), name
        assert list(ot[0]) == ints(toks) + [-1] * (n - Lw - 1), name


def check_walk_brute_force(accept_walk, max_n: int = 6, draws: int = 4, seed: int = 0):
    rng = np.random.default_rng(seed)
    for n in range(1, max_n + 1):
        arrs = list(all_parent_arrays(n))
        for _ in range(draws):
            Vs = int(rng.integers(1, 4))
            d = rng.integers(0, Vs, size=(len(arrs), n))
            t = rng.integers(0, Vs, size=(len(arrs), n))
            al, pn, ot = accept_walk(np.array(arrs), d, t)
            for b, p in enumerate(arrs):
                L, path, toks = brute_force_walk(p, list(d[b]), list(t[b]))
                assert int(al[b]) == L, (p, d[b], t[b])
                assert list(pn[b][:L + 1]) == path and all(x == -1 for x in pn[b][L + 1:])
                assert list(ot[b][:L + 1]) == toks and all(x == -1 for x in ot[b][L + 1:])


def check_walk_chain_closed_forms(accept_walk):
    n = 6
    p = np.arange(-1, n - 1)[None]
    t = np.array([[11, 12, 13, 14, 15, 16]])
    all_match = np.array([[0, 11, 12, 13, 14, 15]])
    al, pn, ot = accept_walk(p, all_match, t)
    assert int(al[0]) == n - 1
    assert list(ot[0]) == [11, 12, 13, 14, 15, 16]      # accepted drafts, then the bonus
    for k in range(1, n):
        d = all_match.copy()
        d[0, k] = 999
        al, pn, ot = accept_walk(p, d, t)
        assert int(al[0]) == k - 1
        assert list(pn[0][:k]) == list(range(k))
    al, pn, ot = accept_walk(np.array([[-1]]), np.array([[5]]), np.array([[7]]))
    assert int(al[0]) == 0 and list(pn[0]) == [0] and list(ot[0]) == [7]


def check_walk_depth_bound_and_greedy(accept_walk, build_masks, seed: int = 1):
    """L never exceeds the tree's depth; when sibling draft tokens are
    distinct the longest path is the greedy one (follow the one matching
    child at every level)."""
    rng = np.random.default_rng(seed)
    for _ in range(300):
        n = int(rng.integers(1, 20))
        p = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        t = list(rng.integers(0, 5, size=n))
        kids = [[] for _ in range(n)]
        for i in range(1, n):
            kids[p[i]].append(i)
        d = [int(rng.integers(0, 1000))] + [0] * (n - 1)
        for u in range(n):                   # distinct draft tokens among siblings
            for c, tok in zip(kids[u], rng.permutation(8)):
                d[c] = int(tok)
        al, pn, ot = accept_walk(np.array([p]), np.array([d]), np.array([t]))
        _, dep = build_masks(np.array([p]))
        assert int(al[0]) <= int(dep[0].max())
        u, L = 0, 0
        while True:
            nxt = [c for c in kids[u] if d[c] == t[u]]
            assert len(nxt) <= 1
            if not nxt:
                break
            u, L = nxt[0], L + 1
        assert int(al[0]) == L


# --------------------------------------------------------------- argmax

def check_argmax_constructed(vocab_argmax):
    rows = np.zeros((7, 16), dtype=np.float32)
    rows[0] = 1.0                                   # all equal -> 0
    rows[1] = -3.0
    rows[1, [3, 7]] = 2.5                           # duplicated maxima -> 3
    rows[2] = np.linspace(-1, 1, 16)
    rows[2, 9] = 100.0                              # planted spike
    rows[3] = -1.0
    rows[3, 5] = -0.0
    rows[3, 2] = 0.0                                # +0 and -0 compare equal -> 2
    rows[4] = -np.float32(3.4e38)                   # extreme finite values
    rows[4, 15] = np.float32(3.4e38)
    rows[5] = np.arange(16, dtype=np.float32)[::-1]  # strictly decreasing -> 0
    rows[6] = -2.0
    rows[6, 1] = -0.0
    rows[6, 4] = 0.0                                # -0 first, +0 later: still the first -> 1
    got = vocab_argmax(rows)
    assert list(got) == [0, 3, 9, 2, 15, 0, 1]


def check_argmax_brute_force(vocab_argmax, seed: int = 2):
    rng = np.random.default_rng(seed)
    x = rng.integers(-3, 4, size=(200, 37)).astype(np.float32)  # many ties
    x[rng.random(x.shape) < 0.1] = -0.0
    got = vocab_argmax(x)
    for r in range(x.shape[0]):
        best = 0
        for v in range(1, x.shape[1]):
            if x[r, v] > x[r, best]:
                best = v
        assert int(got[r]) == best


# ------------------------------------------------------------- attention

def sdpa_f64(q, k, v, mask, scale):
    """torch's scaled_dot_product_attention on CPU in float64 (math path),
    q: [H][M][D], k/v: [H][L][D], mask bool [M][L]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()


def rand_case(rng, B, N, Hq, Hkv, D, P, S_extra=3, tree="random"):
    if tree == "chain":
        parents = np.tile(np.arange(-1, N - 1), (B, 1)).astype(np.int32)
    elif tree == "star":
        parents = np.tile(np.array([-1] + [0] * (N - 1)), (B, 1)).astype(np.int32)
    else:
        parents = np.stack([[-1] + [int(rng.integers(0, i)) for i in range(1, N)]
                            for _ in range(B)]).astype(np.int32)
    prefix = np.asarray(P, dtype=np.int32).reshape(-1)
    if prefix.size == 1:
        prefix = np.full(B, int(prefix[0]), dtype=np.int32)
    S = int(prefix.max()) + N + S_extra
    q = rng.standard_normal((B, N, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    return parents, prefix, q, k, v


def check_attention_chain_is_causal(tree_attention, seed: int = 3):
    """A chain-shaped tree equals bottom-right-aligned causal attention over
    prefix + chain."""
    rng = np.random.default_rng(seed)
    for (B, N, Hq, Hkv, D, P) in [(2, 6, 4, 2, 8, 5), (1, 5, 2, 1, 16, 0), (2, 8, 6, 3, 4, [3, 11])]:
        parents, prefix, q, k, v = rand_case(rng, B, N, Hq, Hkv, D, P, tree="chain")
        sc = 0.3
        out, lse = tree_attention(q, k, v, prefix, parents, sc, q_fmt="f32", kv_fmt="f32")
        g = Hq // Hkv
        for b in range(B):
            Pb = int(prefix[b])
            L = Pb + N
            causal = np.tril(np.ones((N, L), dtype=bool), k=Pb)
            kk = np.repeat(k[b, :, :L].astype(np.float64), g, axis=0)
            vv = np.repeat(v[b, :, :L].astype(np.float64), g, axis=0)
            qq = q[b].astype(np.float64).transpose(1, 0, 2)      # [Hq][N][D]
            ref = sdpa_f64(qq, kk, vv, causal, sc).transpose(1, 0, 2)
            np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)
            s = sc * np.einsum("hnd,hld->hnl", qq, kk)
            s = np.where(causal[None], s, -np.inf)
            ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy().transpose(1, 0)
            np.testing.assert_allclose(lse[b], ref_lse, rtol=1e-12, atol=1e-12)


def check_attention_one_node_is_decode(tree_attention, seed: int = 4):
    """A one-node tree equals plain decode attention over P+1 keys."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D = 3, 4, 2, 8
    parents, prefix, q, k, v = rand_case(rng, B, 1, Hq, Hkv, D, [0, 7, 20])
    out, _ = tree_attention(q, k, v, prefix, parents, 0.25, q_fmt="f32", kv_fmt="f32")
    for b in range(B):
        L = int(prefix[b]) + 1
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            ref = sdpa_f64(q[b, :, h][None].astype(np.float64), k[b, kvh, :L][None].astype(np.float64),
                           v[b, kvh, :L][None].astype(np.float64), np.ones((1, L), dtype=bool), 0.25)
            np.testing.assert_allclose(out[b, 0, h], ref[0, 0], rtol=1e-12, atol=1e-12)


def check_attention_node_locality(tree_attention, seed: int = 5):
    """Each node's output equals causal attention over the prefix plus its own
    root-to-node chain (K/V rows gathered from the cache)."""
    rng = np.random.default_rng(seed)
    for (B, N, Hq, Hkv, D, P) in [(2, 9, 4, 2, 8, [6, 0]), (1, 16, 2, 2, 4, 13), (1, 7, 3, 1, 5, 2)]:
        parents, prefix, q, k, v = rand_case(rng, B, N, Hq, Hkv, D, P)
        out, _ = tree_attention(q, k, v, prefix, parents, 0.5, q_fmt="f32", kv_fmt="f32")
        g = Hq // Hkv
        for b in range(B):
            Pb = int(prefix[b])
            for i in range(N):
                chain = [i]
                while parents[b][chain[-1]] != -1:
                    chain.append(int(parents[b][chain[-1]]))
                rows = list(range(Pb)) + [Pb + j for j in sorted(chain)]
                for h in range(Hq):
                    kk = k[b, h // g, rows].astype(np.float64)[None]
                    vv = v[b, h // g, rows].astype(np.float64)[None]
                    qq = q[b, i, h].astype(np.float64)[None, None]
                    ref = sdpa_f64(qq, kk, vv, np.ones((1, len(rows)), dtype=bool), 0.5)
                    np.testing.assert_allclose(out[b, i, h], ref[0, 0], rtol=1e-12, atol=1e-12)


def check_attention_gqa_is_mha(tree_attention, seed: int = 6):
    """GQA equals MHA after repeating each KV head over its query group."""
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv, D = 2, 7, 6, 2, 8
    parents, prefix, q, k, v = rand_case(rng, B, N, Hq, Hkv, D, [4, 9])
    out, lse = tree_attention(q, k, v, prefix, parents, 0.3, q_fmt="f32", kv_fmt="f32")
    g = Hq // Hkv
    out2, lse2 = tree_attention(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), prefix, parents,
                                0.3, q_fmt="f32", kv_fmt="f32")
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def check_attention_closed_form(tree_attention):
    """P = 0, N = 2 (root and one child), D = 1, sm_scale = 1: the root sees
    only its own key; the child sees both."""
    q = np.array([[[[0.5]], [[1.0]]]], dtype=np.float32)           # [1][2][1][1]
    k = np.array([[[[2.0], [-1.0]]]], dtype=np.float32)             # [1][1][2][1]
    v = np.array([[[[3.0], [7.0]]]], dtype=np.float32)
    out, lse = tree_attention(q, k, v, np.array([0]), np.array([[-1, 0]]), 1.0, q_fmt="f32", kv_fmt="f32")
    assert out[0, 0, 0, 0] == 3.0
    assert lse[0, 0, 0] == 1.0                                      # 0.5 * 2
    e0, e1 = math.exp(2.0), math.exp(-1.0)
    assert abs(out[0, 1, 0, 0] - (3.0 * e0 + 7.0 * e1) / (e0 + e1)) < 1e-14
    assert abs(lse[0, 1, 0] - math.log(e0 + e1)) < 1e-14
    # two siblings under the root: each sees the root and itself only
    q3 = np.ones((1, 3, 1, 1), dtype=np.float32)
    k3 = np.array([[[[0.0], [1.0], [2.0]]]], dtype=np.float32)
    v3 = np.array([[[[1.0], [10.0], [100.0]]]], dtype=np.float32)
    out3, _ = tree_attention(q3, k3, v3, np.array([0]), np.array([[-1, 0, 0]]), 1.0, q_fmt="f32", kv_fmt="f32")
    e = math.exp
    assert abs(out3[0, 1, 0, 0] - (1.0 + 10.0 * e(1)) / (1 + e(1))) < 1e-12
    assert abs(out3[0, 2, 0, 0] - (1.0 + 100.0 * e(2)) / (1 + e(2))) < 1e-12


def check_attention_ignores_rows_past_tree(tree_attention, seed: int = 7):
    """Cache rows at or beyond P_b + N belong to nobody: filling them with NaN
    changes nothing."""
    rng = np.random.default_rng(seed)
    parents, prefix, q, k, v = rand_case(rng, 2, 5, 2, 1, 4, [3, 8], S_extra=4)
    out, _ = tree_attention(q, k, v, prefix, parents, 0.7, q_fmt="f32", kv_fmt="f32")
    k2, v2 = k.copy(), v.copy()
    for b in range(2):
        k2[b, :, int(prefix[b]) + 5:] = np.nan
        v2[b, :, int(prefix[b]) + 5:] = np.nan
    out2, _ = tree_attention(q, k2, v2, prefix, parents, 0.7, q_fmt="f32", kv_fmt="f32")
    np.testing.assert_array_equal(out, out2)


def _pin_formats(q, k, v, fmt, rng):
    """The rand_case arrays in the storage format fmt, as the oracle takes them,
    and their exact float64 values decoded by torch's own conversions."""
    if fmt == "f32":
        return q, k, v, None, None, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    tq = torch.from_numpy(q).to(torch.bfloat16)
    qb = tq.view(torch.int16).numpy().view(np.uint16)
    if fmt == "bf16":
        tk, tv = torch.from_numpy(k).to(torch.bfloat16), torch.from_numpy(v).to(torch.bfloat16)
        return (qb, tk.view(torch.int16).numpy().view(np.uint16), tv.view(torch.int16).numpy().view(np.uint16),
                None, None, tq.double().numpy(), tk.double().numpy(), tv.double().numpy())
    # e4m3 caches with one float32 scale per KV head
    ks = (np.abs(k).max(axis=(0, 2, 3)) / 448.0).astype(np.float32)
    vs = (np.abs(v).max(axis=(0, 2, 3)) / 448.0).astype(np.float32)
    tk = (torch.from_numpy(k) / torch.from_numpy(ks)[None, :, None, None]).to(torch.float8_e4m3fn)
    tv = (torch.from_numpy(v) / torch.from_numpy(vs)[None, :, None, None]).to(torch.float8_e4m3fn)
    kf = tk.double().numpy() * ks.astype(np.float64)[None, :, None, None]
    vf = tv.double().numpy() * vs.astype(np.float64)[None, :, None, None]
    return (qb, tk.view(torch.uint8).numpy(), tv.view(torch.uint8).numpy(), ks, vs, tq.double().numpy(), kf, vf)


def check_attention_bh(tree_attention_bh, tree_attention, seed: int = 18):
    """The one-(request, head) oracle call: bit for bit the batched call's
    slice for every pair, and float64 SDPA over the request's kv head (head h
    reads kv head h // g) with a dense mask from a parent chase written here;
    fp32, bf16 and e4m3 caches, ragged prefixes, GQA groups of 1 to 6."""
    rng = np.random.default_rng(seed)
    for (B, N, Hq, Hkv, D, P, fmt) in [(3, 7, 6, 2, 8, [5, 0, 12], "f32"), (2, 5, 8, 2, 16, [9, 3], "bf16"),
                                       (2, 6, 4, 4, 8, [2, 7], "e4m3"), (1, 4, 6, 1, 4, 3, "f32"),
                                       (2, 9, 6, 3, 8, [11, 1], "e4m3")]:
        parents, prefix, q, k, v = rand_case(rng, B, N, Hq, Hkv, D, P)
        qo, ko, vo, ks, vs, qf, kf, vf = _pin_formats(q, k, v, fmt, rng)
        qfmt = "f32" if fmt == "f32" else "bf16"
        sc = 0.4
        out, lse = tree_attention(qo, ko, vo, prefix, parents, sc, q_fmt=qfmt, kv_fmt=fmt, k_scale=ks, v_scale=vs)
        g = Hq // Hkv
        for b in range(B):
            Pb = int(prefix[b])
            L = Pb + N
            mask = np.zeros((N, L), dtype=bool)
            mask[:, :Pb] = True
            for i in range(N):
                j = i
                while j != -1:
                    mask[i, Pb + j] = True
                    j = int(parents[b][j])
            for h in range(Hq):
                ob, lb = tree_attention_bh(qo, ko, vo, prefix, parents, sc, b, h, q_fmt=qfmt, kv_fmt=fmt,
                                           k_scale=ks, v_scale=vs)
                np.testing.assert_array_equal(ob, out[b, :, h])
                np.testing.assert_array_equal(lb, lse[b, :, h])
                ref = sdpa_f64(qf[b, :, h][None], kf[b, h // g, :L][None], vf[b, h // g, :L][None], mask, sc)[0]
                np.testing.assert_allclose(ob, ref, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------ commit

def _row_tagged_cache(B, Hkv, S, width=3):
    """K/V whose every element says which (request, head, row) it came from."""
    b, h, r, c = np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(S), np.arange(width), indexing="ij")
    k = (b * 1_000_000 + h * 10_000 + r * 10 + c).astype(np.int64)
    return k, -k


def check_commit_golden(commit_accepted):
    for name, par, P, L, path, stored, labels in read_golden("commit_hand_examples.txt"):
        par, P, L, path, stored, labels = ints(par), int(P), int(L), ints(path), ints(stored), ints(labels)
        N = len(par)
        k, v = _row_tagged_cache(1, 2, P + N + 2)
        pn = np.full((1, N), -1, dtype=np.int32)
        pn[0, :L + 1] = path
        k2, v2, newp, lab = commit_accepted(k, v, np.array([P]), np.array([L]), pn, N)
        assert int(newp[0]) == P + 1 + L, name
        assert list(lab[0]) == labels, (name, list(lab[0]))
        for j, node in enumerate(stored):
            assert np.array_equal(k2[0, :, P + j], k[0, :, P + node]), (name, j)
            assert np.array_equal(v2[0, :, P + j], v[0, :, P + node]), (name, j)
        rest = [r for r in range(k.shape[2]) if not P + 1 <= r <= P + L]
        assert np.array_equal(k2[0, :, rest], k[0, :, rest]) and np.array_equal(v2[0, :, rest], v[0, :, rest]), name


def check_commit_against_parent_chase(commit_accepted, accept_walk, seed: int = 8):
    """Random trees and tokens: the committed rows P+1..P+L hold, in order, the
    nodes met walking parent links up from the accepted path's end node (found
    here independently of the walk's own path output), labels mark exactly
    those nodes, every other row and request is untouched."""
    rng = np.random.default_rng(seed)
    for trial in range(60):
        B, N, Hkv = 3, int(rng.integers(1, 12)), 2
        parents = np.zeros((B, N), dtype=np.int32)
        for b in range(B):
            parents[b, 0] = -1
            for i in range(1, N):
                parents[b, i] = rng.integers(0, i)
        d = rng.integers(0, 3, size=(B, N)).astype(np.int32)
        t = rng.integers(0, 3, size=(B, N)).astype(np.int32)
        L, path, _ = accept_walk(parents, d, t, V=3)
        prefix = rng.integers(0, 6, size=B)
        S = int(prefix.max()) + N + 1
        k, v = _row_tagged_cache(B, Hkv, S)
        k2, v2, newp, lab = commit_accepted(k, v, prefix, L, path, N)
        for b in range(B):
            P, Lb = int(prefix[b]), int(L[b])
            chain, n = [], int(path[b][Lb])
            while n != -1:
                chain.append(n)
                n = int(parents[b, n])
            chain.reverse()
            assert len(chain) == Lb + 1 and chain[0] == 0
            for j, node in enumerate(chain):
                assert np.array_equal(k2[b, :, P + j], k[b, :, P + node])
                assert np.array_equal(v2[b, :, P + j], v[b, :, P + node])
            others = [r for r in range(S) if not P + 1 <= r <= P + Lb]
            assert np.array_equal(k2[b, :, others], k[b, :, others])
            assert int(newp[b]) == P + 1 + Lb
            want = [0] * N
            want[0] = 2
            for node in chain[1:]:
                want[node] = 1
            assert list(lab[b]) == want


# ------------------------------------------------------------------- paged

def check_gather_pages_round_trip(gather_pages, seed: int = 9):
    """Scatter a tagged contiguous cache into shuffled pages (written here
    token by token), gather it back: identical, including a request whose
    pages are shared with nobody and a partially filled last page."""
    rng = np.random.default_rng(seed)
    for B, Hkv, S_max, ps in [(3, 2, 40, 8), (2, 1, 64, 16), (1, 3, 7, 4)]:
        maxp = -(-S_max // ps)
        contig = _row_tagged_cache(B, Hkv, S_max)[0]
        num_pages = B * maxp + 3
        perm = rng.permutation(num_pages)[: B * maxp].reshape(B, maxp)
        pages = np.full((num_pages, ps, Hkv, contig.shape[-1]), -7, dtype=contig.dtype)
        for b in range(B):
            for t in range(S_max):
                pages[perm[b, t // ps], t % ps] = contig[b, :, t]
        back = gather_pages(pages, perm, ps, S_max)
        assert np.array_equal(back, contig)


def check_gather_pages_identity(gather_pages):
    """Pages laid out request after request in order: the gather is a reshape."""
    B, Hkv, ps, maxp = 2, 2, 4, 3
    pages = np.arange(B * maxp * ps * Hkv * 5).reshape(B * maxp, ps, Hkv, 5)
    table = np.arange(B * maxp).reshape(B, maxp)
    want = pages.reshape(B, maxp * ps, Hkv, 5).transpose(0, 2, 1, 3)
    assert np.array_equal(gather_pages(pages, table, ps, maxp * ps), want)


# ---------------------------------------------------------------- backward

def _backward_case(rng, B, N, Hq, Hkv, D, P, tree="random"):
    parents, prefix, q, k, v = rand_case(rng, B, N, Hq, Hkv, D, P, tree=tree)
    d_out = rng.standard_normal(q.shape).astype(np.float32)
    return parents, prefix, q, k, v, d_out


def _dense_mask_by_walk(parents_b, P):
    """bool[N][P+N] by parent-pointer chase, written here so the pin does not
    lean on the oracle's own mask."""
    N = len(parents_b)
    A = np.zeros((N, P + N), dtype=bool)
    A[:, :P] = True
    for i in range(N):
        j = i
        while j != -1:
            A[i, P + j] = True
            j = int(parents_b[j])
    return A


def _torch_loss(q, k, v, d_out, parents, prefix, scale, Hq, Hkv):
    """sum <dO, out> through torch's float64 SDPA (math path), GQA by
    repeat_interleave; q, k, v are float64 leaf tensors."""
    g = Hq // Hkv
    B, N = q.shape[0], q.shape[1]
    total = torch.zeros((), dtype=torch.float64)
    for b in range(B):
        Pb = int(prefix[b])
        L = Pb + N
        A = torch.from_numpy(_dense_mask_by_walk(parents[b], Pb))
        kk = k[b, :, :L].repeat_interleave(g, dim=0)                  # [Hq][L][D]
        vv = v[b, :, :L].repeat_interleave(g, dim=0)
        qq = q[b].transpose(0, 1)                                      # [Hq][N][D]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=A, scale=scale)
        total = total + (o.transpose(0, 1) * torch.from_numpy(d_out[b].astype(np.float64))).sum()
    return total


def check_backward_autograd(tree_attention_backward, seed: int = 10):
    """Gradients equal torch autograd through float64 SDPA with the dense tree
    mask, for random trees, ragged prefixes and GQA."""
    rng = np.random.default_rng(seed)
    for (B, N, Hq, Hkv, D, P) in [(2, 7, 4, 2, 8, [5, 0]), (1, 9, 6, 3, 4, 11), (2, 5, 2, 2, 16, [2, 9])]:
        parents, prefix, q, k, v, d_out = _backward_case(rng, B, N, Hq, Hkv, D, P)
        sc = 0.4
        dq, dk, dv = tree_attention_backward(q, k, v, prefix, parents, d_out, sc, q_fmt="f32", kv_fmt="f32")
        tq, tk, tv = (torch.from_numpy(x.astype(np.float64)).requires_grad_(True) for x in (q, k, v))
        _torch_loss(tq, tk, tv, d_out, parents, prefix, sc, Hq, Hkv).backward()
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def check_backward_finite_differences(tree_attention_backward, seed: int = 11):
    """Central differences of sum <dO, out> (out from torch's float64 SDPA)
    at a sample of q, K and V entries agree with the gradients."""
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv, D = 1, 6, 4, 2, 4
    parents, prefix, q, k, v, d_out = _backward_case(rng, B, N, Hq, Hkv, D, [3])
    sc, h = 0.6, 1e-6
    dq, dk, dv = tree_attention_backward(q, k, v, prefix, parents, d_out, sc, q_fmt="f32", kv_fmt="f32")
    base = [torch.from_numpy(x.astype(np.float64)) for x in (q, k, v)]

    def loss(which, idx, delta):
        xs = [t.clone() for t in base]
        xs[which][idx] += delta
        return float(_torch_loss(*xs, d_out, parents, prefix, sc, Hq, Hkv))

    L = int(prefix[0]) + N
    picks = [(0, (0, i, hh, d)) for i in range(N) for hh in (0, 3) for d in (0, 2)]
    picks += [(w, (0, kvh, c, d)) for w in (1, 2) for kvh in (0, 1) for c in range(L) for d in (1, 3)]
    picks += [(1, (0, 0, L, 0)), (2, (0, 1, L + 1, 2))]                 # rows past the tree
    grads = (dq, dk, dv)
    for which, idx in picks:
        fd = (loss(which, idx, h) - loss(which, idx, -h)) / (2 * h)
        assert abs(grads[which][idx] - fd) <= 1e-7 + 1e-6 * abs(fd), (which, idx, grads[which][idx], fd)


def check_backward_invariants(tree_attention_backward, seed: int = 12):
    """Sum over keys of dK is zero (each row's softmax gradient sums to zero);
    sum over keys of dV is the sum of dO over the rows sharing the kv head
    (each row's weights sum to one); rows past the tree get nothing."""
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv, D = 3, 8, 6, 2, 5
    parents, prefix, q, k, v, d_out = _backward_case(rng, B, N, Hq, Hkv, D, [0, 4, 13])
    dq, dk, dv = tree_attention_backward(q, k, v, prefix, parents, d_out, 0.8, q_fmt="f32", kv_fmt="f32")
    g = Hq // Hkv
    for b in range(B):
        L = int(prefix[b]) + N
        for kvh in range(Hkv):
            np.testing.assert_allclose(dk[b, kvh, :L].sum(axis=0), 0.0, atol=1e-12)
            want = d_out[b, :, kvh * g:(kvh + 1) * g].astype(np.float64).sum(axis=(0, 1))
            np.testing.assert_allclose(dv[b, kvh, :L].sum(axis=0), want, rtol=1e-12, atol=1e-12)
            assert not dk[b, kvh, L:].any() and not dv[b, kvh, L:].any()


def check_backward_subtree_locality(tree_attention_backward, seed: int = 13):
    """With dO non-zero for one node i only, the tree rows that receive K/V
    gradient are exactly i's ancestors-or-self (the prefix rows all do)."""
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv, D, P = 1, 10, 2, 1, 4, 3
    parents, prefix, q, k, v, d_out = _backward_case(rng, B, N, Hq, Hkv, D, [P])
    for i in range(N):
        d1 = np.zeros_like(d_out)
        d1[0, i] = d_out[0, i]
        _, dk, dv = tree_attention_backward(q, k, v, prefix, parents, d1, 0.5, q_fmt="f32", kv_fmt="f32")
        chain, j = set(), i
        while j != -1:
            chain.add(j)
            j = int(parents[0][j])
        for jj in range(N):
            hit = bool(np.abs(dv[0, 0, P + jj]).sum() > 0)
            assert hit == (jj in chain), (i, jj)
            if jj not in chain:
                assert not dk[0, 0, P + jj].any()
        assert np.abs(dv[0, 0, :P]).sum(axis=1).min() > 0


def check_backward_closed_form(tree_attention_backward):
    """P = 0, root and one child, D = 1, sm_scale = 1.  The root sees only its
    own key: dq_root = 0 and its dO goes to v_0 whole.  The child has weights
    w0, w1 = softmax(q1 k0, q1 k1): d out1/d q1 = w0 w1 (k1 - k0)(v1 - v0),
    d out1/d k1 = -d out1/d k0 = q1 w0 w1 (v1 - v0), d out1/d v_c = w_c."""
    q0, q1, k0, k1, v0, v1, a, c = 0.5, 1.5, 2.0, -1.0, 3.0, 7.0, 0.25, -2.0
    q = np.array([[[[q0]], [[q1]]]], dtype=np.float32)
    k = np.array([[[[k0], [k1]]]], dtype=np.float32)
    v = np.array([[[[v0], [v1]]]], dtype=np.float32)
    dO = np.array([[[[a]], [[c]]]], dtype=np.float32)
    dq, dk, dv = tree_attention_backward(q, k, v, np.array([0]), np.array([[-1, 0]]), dO, 1.0,
                                         q_fmt="f32", kv_fmt="f32")
    e0, e1 = math.exp(q1 * k0), math.exp(q1 * k1)
    w0, w1 = e0 / (e0 + e1), e1 / (e0 + e1)
    assert dq[0, 0, 0, 0] == 0.0
    assert abs(dq[0, 1, 0, 0] - c * w0 * w1 * (k1 - k0) * (v1 - v0)) < 1e-14
    assert abs(dk[0, 0, 1, 0] - c * q1 * w0 * w1 * (v1 - v0)) < 1e-14
    assert abs(dk[0, 0, 0, 0] + c * q1 * w0 * w1 * (v1 - v0)) < 1e-14
    assert abs(dv[0, 0, 0, 0] - (a + c * w0)) < 1e-14
    assert abs(dv[0, 0, 1, 0] - c * w1) < 1e-14


# -------------------------------------------------------------------- fp8

def check_e4m3_encode_against_torch(encode_e4m3, seed: int = 15):
    """Round-to-nearest-even e4m3 encoding equals torch's float8_e4m3fn
    conversion: random magnitudes over the whole range (subnormals included),
    every finite code's own value, and the midpoints between neighbours."""
    rng = np.random.default_rng(seed)
    from oracle import e4m3_decode_table
    tab = e4m3_decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(tab[c])])
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-0.02, 0.02, 2000),
                        tab[finite], rng.standard_normal(2000) * 30])
    pos = np.sort(np.unique(tab[finite][tab[finite] >= 0]))
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, mids, -mids]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = encode_e4m3(x)
    # -0.0 and +0.0 both decode to zero; compare values for zeros, codes otherwise
    same = (got == ref) | ((tab[got] == 0) & (tab[ref] == 0))
    assert same.all(), (x[~same][:5], got[~same][:5], ref[~same][:5])


def check_e4m3_ties_go_to_even(encode_e4m3):
    """Midpoints between consecutive codes round to the code with an even
    mantissa: 1.0625 (between 1.0 = 0x38 and 1.125 = 0x39) -> 0x38, 1.1875
    (between 0x39 and 1.25 = 0x3A) -> 0x3A."""
    assert encode_e4m3(np.array([1.0625]))[0] == 0x38
    assert encode_e4m3(np.array([1.1875]))[0] == 0x3A
    assert encode_e4m3(np.array([-1.1875]))[0] == 0xBA


def check_row_quantization(quantize_rows_e4m3, dequantize_rows_e4m3, seed: int = 16):
    """Each row's largest magnitude becomes exactly +-448; a row of zeros keeps
    scale 1 and zero codes; every element is within half an e4m3 step
    (relative 2^-4) of its value, or within the subnormal step."""
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((7, 5, 128)) * rng.uniform(0.01, 30, (7, 5, 1))).astype(np.float32)
    q[3, 2] = 0.0
    codes, scale = quantize_rows_e4m3(q)
    assert codes.shape == q.shape and scale.shape == q.shape[:-1]
    assert scale[3, 2] == 1.0 and not codes[3, 2].any()
    from oracle import e4m3_decode_table
    tab = e4m3_decode_table()
    for idx in np.ndindex(q.shape[:-1]):
        if not q[idx].any():
            continue
        j = int(np.argmax(np.abs(q[idx])))
        assert abs(tab[codes[idx][j]]) == 448.0
    qh = dequantize_rows_e4m3(codes, scale)
    amax = np.abs(q).max(axis=-1, keepdims=True)
    step = np.maximum(np.abs(q) * 2.0 ** -4, amax / 448 * 2.0 ** -10)
    assert (np.abs(qh - q) <= step * (1 + 1e-6)).all()


def check_e2m1_table(e2m1_decode_table):
    """The 16 OCP E2M1 values, listed by hand: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6},
    sign in the top bit of the nibble."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    tab = e2m1_decode_table()
    assert list(tab[:8]) == want
    assert list(-tab[8:]) == want


def check_e2m1_packing(decode_e2m1_packed, seed: int = 17):
    """Element 2j sits in the low nibble of byte j: decoding codes packed by a
    packer written here gives the codes' values in order, times the scale."""
    rng = np.random.default_rng(seed)
    vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])
    codes = rng.integers(0, 16, size=(3, 5, 128))
    packed = np.zeros((3, 5, 64), dtype=np.uint8)
    for j in range(64):
        packed[..., j] = codes[..., 2 * j] + 16 * codes[..., 2 * j + 1]
    got = decode_e2m1_packed(packed, 0.375)
    np.testing.assert_array_equal(got, vals[codes] * 0.375)
