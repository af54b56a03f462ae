"""The verify step over a paged cache (spec_verify_step_paged: masks, the
paged attention, argmax and accept walk in one launch) on the GPU.

It equals the four separate calls with the paged attention
(spec_tree_attn_verify_paged, whose own parity with the oracle is tested over
the oracle's gather of the pages) bit for bit, its integer outputs equal the
oracle's, it leaves the prep part of its workspace zeroed, and a page id outside the pool is
flagged while the argmax and the walk stay exact.  The attention output is
also held to the oracle's (the pages hold the contiguous cache's values).
"""
import numpy as np
import pytest
import torch

import synth
import tree_attention_verify_parent_amd as st
from tests.gpu_util import check_attention, check_integers, log, oracle_step, paginate, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

# (workload, page size): the prologue scan at the full chain6_b8 size (2054
# tokens over 129 pages), tail scanners (V = 5003 ragged, N = 60 with V =
# 4099), fp8 pages, one-token pages with D = 64, one 4096-token page per
# request.
CASES = {
    "chain6_b8_bf16_p16": (W[1], 16),
    "tree16_ragged_V5003_p64": (W[2].replace(B=4, prefix_lo=100, prefix_hi=1500, V=5003, seed=41), 64),
    "tree60_V4099_p128": (W[3].replace(B=2, prefix_lo=777, prefix_hi=777, V=4099, seed=42), 128),
    "tree60_fp8kv_ragged_p32": (W[3].replace(B=2, kv_dtype="e4m3", prefix_lo=150, prefix_hi=900, V=2000, seed=46), 32),
    "tree16_fp8kv_p32": (W[4].replace(B=4, prefix_lo=333, prefix_hi=333, V=6000, seed=43), 32),
    "tree16_d64_p1": (W[2].replace(B=3, D=64, Hq=8, Hkv=2, prefix_lo=40, prefix_hi=300, V=1000, seed=44), 1),
    # the largest page: every request's tokens in one page of 4096
    "chain6_p4096": (W[1].replace(B=3, prefix_lo=100, prefix_hi=2500, V=3000, seed=45), 4096),
}

KEYS = ("mask", "depth", "argmax", "accept_len", "path_nodes", "out_tokens", "err")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    st.lib()


def _paged_inputs(w, ps, seed=7):
    x = synth.make_inputs(w)
    d = to_device(x)
    kp, table = paginate(x["k_cache"], ps, np.random.default_rng(seed))
    vp, _ = paginate(x["v_cache"], ps, np.random.default_rng(seed))
    return x, d, kp.cuda(), vp.cuda(), table


def _run(d, x, kp, vp, table, fused=True, workspace=None):
    r = st.verify_step(d["parents"], d["draft_tokens"], d["prefix_lens"], d["q"], kp, vp, d["logits"],
                       x["sm_scale"], k_scale=d["k_scale"], v_scale=d["v_scale"], block_table=table,
                       fused=fused, workspace=workspace)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in r.items()}


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def _same(a, b):
    for k in KEYS:
        assert np.array_equal(a[k].numpy(), b[k].numpy()), k
    assert np.array_equal(_bits(a["out"]), _bits(b["out"]))
    assert np.array_equal(a["lse"].numpy(), b["lse"].numpy())


@pytest.mark.parametrize("name", list(CASES))
def test_paged_step_equals_the_four_calls(name):
    w, ps = CASES[name]
    log(f"[step paged] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} V={w.V} page={ps} kv={w.kv_dtype}")
    x, d, kp, vp, table = _paged_inputs(w, ps)
    t = torch.from_numpy(table).cuda()
    a = _run(d, x, kp, vp, t, fused=True)
    b = _run(d, x, kp, vp, t, fused=False)
    _same(a, b)
    assert int(a["err"][0]) == 0
    r = oracle_step(x)
    got = {k: (v.numpy().view(np.uint64) if k == "mask" else v.numpy()) for k, v in a.items() if k in KEYS}
    check_integers(got, r, name)
    check_attention(a["out"].float().numpy(), r["out"], w.kv_dtype, name)


def test_paged_step_reuses_its_zeroed_workspace():
    w, ps = CASES["tree16_ragged_V5003_p64"]
    log(f"[step paged] workspace reuse B={w.B} page={ps}")
    x, d, kp, vp, table = _paged_inputs(w, ps, seed=9)
    t = torch.from_numpy(table).cuda()
    ws = torch.zeros(st.verify_step_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, table.shape[1] * ps),
                     dtype=torch.uint8, device="cuda")
    prep = (w.B * w.N * 12 + w.B * 4 + 255) // 256 * 256      # keys and counters; the attention's part follows
    a = _run(d, x, kp, vp, t, workspace=ws)
    assert int(ws[:prep].count_nonzero()) == 0
    b = _run(d, x, kp, vp, t, workspace=ws)
    assert int(ws[:prep].count_nonzero()) == 0
    _same(a, b)


def test_paged_step_flags_a_page_outside_the_pool():
    w = W[2].replace(B=3, prefix_lo=200, prefix_hi=200, V=3001, seed=45)
    log(f"[step paged] bad page id B={w.B} V={w.V}")
    x, d, kp, vp, table = _paged_inputs(w, 16, seed=3)
    table = table.copy()
    table[1, 3] = kp.shape[0] + 4                    # in request 1's used range, outside the pool
    t = torch.from_numpy(table).cuda()
    a = _run(d, x, kp, vp, t, fused=True)
    b = _run(d, x, kp, vp, t, fused=False)
    _same(a, b)                                      # both read page 0 in its place
    assert int(a["err"][0]) == st.DERR_PAGE
    r = oracle_step(x)
    got = {k: (v.numpy().view(np.uint64) if k == "mask" else v.numpy()) for k, v in a.items() if k in KEYS}
    check_integers(got, r, "bad page")
