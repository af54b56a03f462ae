"""GPU parity of the commit step (spec_commit_accepted, and over a paged
cache spec_commit_accepted_paged) against the oracle.

The caches are compared byte for byte: the step only moves rows.  The accepted
paths come from the GPU's own mask / argmax / walk (those are checked against
the oracle elsewhere); the oracle commits the same paths on the same bytes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_attention_verify_parent_amd as st
from tests.gpu_util import log, paginate, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

CASES = {
    "tree16_ragged_bf16": W[2].replace(B=6, prefix_lo=100, prefix_hi=700, V=12, p_match=0.9, seed=51),
    "tree16_fp8kv": W[4].replace(B=4, prefix_lo=300, prefix_hi=300, V=12, p_match=0.9, seed=52),
    "chain6_f32": W[0].replace(B=3, V=8, p_match=0.8, seed=53),
    "chain6_bf16_d128": W[1].replace(B=4, prefix_lo=40, prefix_hi=40, V=6, p_match=0.9, seed=54),
    "tree64_deep_bf16": W[2].replace(B=3, N=64, max_depth=30, max_children=2, Hq=8, Hkv=2, prefix_lo=0,
                                     prefix_hi=90, V=4, p_match=0.95, seed=55),
}


def _bytes(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _walk_on_gpu(d, w):
    anc, _, _ = st.tree_mask_build(d["parents"])
    t = st.vocab_argmax(d["logits"])
    L, path, _, err = st.accept_walk(d["parents"], anc, d["draft_tokens"], t.view(w.B, w.N), w.V)
    return L, path, err


@pytest.mark.parametrize("name", list(CASES))
def test_commit_matches_oracle(name):
    w = CASES[name]
    log(f"[commit] {name} B={w.B} N={w.N} Hkv={w.Hkv} D={w.D} kv={w.kv_dtype}")
    x = synth.make_inputs(w)
    d = to_device(x)
    L, path, err = _walk_on_gpu(d, w)
    kb, vb = _bytes(d["k_cache"]), _bytes(d["v_cache"])
    newp, lab, err = st.commit_accepted(d["k_cache"], d["v_cache"], d["prefix_lens"], L, path, err=err)
    torch.cuda.synchronize()
    assert int(err[0]) == 0
    Lc, pc = L.cpu().numpy(), path.cpu().numpy()
    log(f"  accept_len {list(Lc)}")
    if w.tree == "random":     # the case must exercise real moves, not only paths already in place
        assert any(pc[b][k] != k for b in range(w.B) for k in range(1, int(Lc[b]) + 1)), list(Lc)
    ko, vo, po, lo = oracle.commit_accepted(kb, vb, x["prefix_lens"], Lc, pc, w.N)
    assert np.array_equal(_bytes(d["k_cache"]), ko)
    assert np.array_equal(_bytes(d["v_cache"]), vo)
    assert np.array_equal(newp.cpu().numpy(), po)
    assert np.array_equal(lab.cpu().numpy(), lo)


def test_commit_moves_rows_across_each_other():
    """Paths that move a row onto another accepted node's source row, built by
    hand: tree [-1 0 0 1 1 2], path 0-2-5 (row P+2 is written by depth 2 and read
    by depth 1) next to a root-only request and a fully accepted chain."""
    B, N, Hkv, D, S = 3, 6, 2, 64, 20
    g = torch.Generator().manual_seed(5)
    k = torch.randn(B, Hkv, S, D, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, Hkv, S, D, generator=g).to(torch.bfloat16).cuda()
    prefix = torch.tensor([3, 7, 0], dtype=torch.int32).cuda()
    L = torch.tensor([2, 0, 5], dtype=torch.int32).cuda()
    path = torch.tensor([[0, 2, 5, -1, -1, -1], [0, -1, -1, -1, -1, -1], [0, 1, 2, 3, 4, 5]],
                        dtype=torch.int32).cuda()
    kb, vb = _bytes(k), _bytes(v)
    newp, lab, err = st.commit_accepted(k, v, prefix, L, path)
    torch.cuda.synchronize()
    assert int(err[0]) == 0
    ko, vo, po, lo = oracle.commit_accepted(kb, vb, prefix.cpu().numpy(), L.cpu().numpy(), path.cpu().numpy(), N)
    assert np.array_equal(_bytes(k), ko) and np.array_equal(_bytes(v), vo)
    assert list(newp.cpu().numpy()) == [6, 8, 6]
    assert lab.cpu().numpy().tolist() == [[2, 0, 1, 0, 0, 1], [2, 0, 0, 0, 0, 0], [2, 1, 1, 1, 1, 1]]


def test_commit_flags_bad_input_and_leaves_cache_alone():
    B, N, Hkv, D, S = 3, 5, 1, 64, 16
    k = torch.randn(B, Hkv, S, D).to(torch.bfloat16).cuda()
    v = torch.randn(B, Hkv, S, D).to(torch.bfloat16).cuda()
    good = torch.tensor([[0, 2, -1, -1, -1]] * B, dtype=torch.int32).cuda()
    for what, prefix, L, path, bit in [
        ("accept_len past the tree", [2, 2, 2], [1, 5, 1], good, st.DERR_PATH),
        ("path not from the root", [2, 2, 2], [1, 1, 1],
         torch.tensor([[0, 2, -1, -1, -1], [1, 2, -1, -1, -1], [0, 2, -1, -1, -1]], dtype=torch.int32).cuda(),
         st.DERR_PATH),
        ("path not increasing", [2, 2, 2], [2, 2, 2],
         torch.tensor([[0, 2, 3, -1, -1], [0, 3, 3, -1, -1], [0, 1, 4, -1, -1]], dtype=torch.int32).cuda(),
         st.DERR_PATH),
        ("prefix past the cache", [2, 12, 2], [1, 1, 1], good, st.DERR_PREFIX),
    ]:
        kk, vv = k.clone(), v.clone()
        pre = torch.tensor(prefix, dtype=torch.int32).cuda()
        Lt = torch.tensor(L, dtype=torch.int32).cuda()
        newp, lab, err = st.commit_accepted(kk, vv, pre, Lt, path)
        torch.cuda.synchronize()
        assert int(err[0]) & bit, what
        # request 1 is the bad one: its rows are untouched; the others are committed
        assert torch.equal(kk[1], k[1]) and torch.equal(vv[1], v[1]), what
        ko, vo, po, lo = oracle.commit_accepted(_bytes(k)[[0, 2]], _bytes(v)[[0, 2]], np.array(prefix)[[0, 2]],
                                                np.array(L)[[0, 2]], path.cpu().numpy()[[0, 2]], N)
        assert np.array_equal(_bytes(kk)[[0, 2]], ko) and np.array_equal(_bytes(vv)[[0, 2]], vo), what


# ---- the same step over a paged cache (spec_commit_accepted_paged): the
# oracle gathers the pool back to the contiguous layout (its own gather) and
# commits there; the pool's pages that no request uses stay as they were.
PAGED = {
    "tree16_ragged_bf16_p16": (CASES["tree16_ragged_bf16"], 16),
    "tree16_fp8kv_p32": (CASES["tree16_fp8kv"], 32),
    "chain6_f32_p8": (CASES["chain6_f32"], 8),
    "tree64_deep_bf16_p1": (CASES["tree64_deep_bf16"], 1),
}


def _paged_case(w, ps, seed=3, corrupt=None):
    x = synth.make_inputs(w)
    d = to_device(x)
    L, path, err = _walk_on_gpu(d, w)
    kp, table = paginate(x["k_cache"], ps, np.random.default_rng(seed))
    vp, _ = paginate(x["v_cache"], ps, np.random.default_rng(seed))
    if corrupt is not None:
        table = table.copy()
        corrupt(table, kp.shape[0])
    kp, vp = kp.cuda(), vp.cuda()
    kb, vb = _bytes(kp), _bytes(vp)
    newp, lab, err = st.commit_accepted(kp, vp, d["prefix_lens"], L, path, block_table=torch.from_numpy(table).cuda(),
                                        err=err)
    torch.cuda.synchronize()
    return x, table, kb, vb, kp, vp, L.cpu().numpy(), path.cpu().numpy(), newp.cpu().numpy(), lab.cpu().numpy(), err


@pytest.mark.parametrize("name", list(PAGED))
def test_paged_commit_matches_oracle(name):
    w, ps = PAGED[name]
    log(f"[commit paged] {name} B={w.B} N={w.N} Hkv={w.Hkv} D={w.D} kv={w.kv_dtype} page={ps}")
    x, table, kb, vb, kp, vp, Lc, pc, newp, lab, err = _paged_case(w, ps)
    assert int(err[0]) == 0
    S_pad = table.shape[1] * ps
    ko, vo, po, lo = oracle.commit_accepted(oracle.gather_pages(kb, table, ps, S_pad),
                                            oracle.gather_pages(vb, table, ps, S_pad), x["prefix_lens"], Lc, pc, w.N)
    assert np.array_equal(oracle.gather_pages(_bytes(kp), table, ps, S_pad), ko)
    assert np.array_equal(oracle.gather_pages(_bytes(vp), table, ps, S_pad), vo)
    assert np.array_equal(newp, po) and np.array_equal(lab, lo)
    unused = np.setdiff1d(np.arange(kb.shape[0]), table.reshape(-1))
    assert len(unused) > 0
    assert np.array_equal(_bytes(kp)[unused], kb[unused]) and np.array_equal(_bytes(vp)[unused], vb[unused])


def test_paged_commit_flags_a_page_outside_the_pool():
    w = CASES["tree16_ragged_bf16"]
    ps = 16
    pre = synth.make_inputs(w)["prefix_lens"]

    def corrupt(table, num_pages):
        table[1, int(pre[1]) // ps] = num_pages + 3          # the page of request 1's root row
    x, table, kb, vb, kp, vp, Lc, pc, newp, lab, err = _paged_case(w, ps, corrupt=corrupt)
    assert int(err[0]) == st.DERR_PAGE
    # request 1 is left alone; the others are committed as the oracle does
    keep = [b for b in range(w.B) if b != 1]
    S_pad = table.shape[1] * ps
    tk = table[keep]
    ko, vo, po, lo = oracle.commit_accepted(oracle.gather_pages(kb, tk, ps, S_pad), oracle.gather_pages(vb, tk, ps, S_pad),
                                            x["prefix_lens"][keep], Lc[keep], pc[keep], w.N)
    assert np.array_equal(oracle.gather_pages(_bytes(kp), tk, ps, S_pad), ko)
    assert np.array_equal(oracle.gather_pages(_bytes(vp), tk, ps, S_pad), vo)
    assert np.array_equal(newp[keep], po) and np.array_equal(lab[keep], lo)
    # every page request 1 maps (inside the pool) is unchanged
    own = np.array([p for p in table[1] if 0 <= p < kb.shape[0]])
    assert np.array_equal(_bytes(kp)[own], kb[own]) and np.array_equal(_bytes(vp)[own], vb[own])
