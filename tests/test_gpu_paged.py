"""GPU parity of the paged-cache attention (spec_tree_attn_verify_paged).

Synthetic contiguous caches are scattered into shuffled token-major pages; the
oracle gathers them back (its own gather, pinned on the CPU) and runs the same
attention; the GPU reads the pages through the block table.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_attention_verify_parent_amd as st
from tests.gpu_util import check_attention, log, oracle_views, paginate, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

CASES = {
    "tree16_ragged_bf16_p16": (W[2].replace(B=5, prefix_lo=100, prefix_hi=1500, V=10, seed=61), 16),
    "tree16_ragged_bf16_p64": (W[2].replace(B=5, prefix_lo=100, prefix_hi=1500, V=10, seed=62), 64),
    "chain6_bf16_p32": (W[1].replace(B=4, prefix_lo=700, prefix_hi=700, V=10, seed=63), 32),
    "tree16_fp8kv_p16": (W[4].replace(B=3, prefix_lo=500, prefix_hi=500, V=10, seed=64), 16),
    "tree60_bf16_p128": (W[3].replace(B=1, prefix_lo=900, prefix_hi=900, V=10, seed=65), 128),
    # 960 packed rows over e4m3 pages and ragged prefixes (the 8-wave plan's paged path)
    "tree60_fp8kv_ragged_p16": (W[3].replace(B=2, kv_dtype="e4m3", prefix_lo=200, prefix_hi=1100, V=10, seed=67), 16),
    "tree16_d64_p1": (W[2].replace(B=3, D=64, Hq=8, Hkv=2, prefix_lo=40, prefix_hi=300, V=10, seed=66), 1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_paged_attention_matches_oracle(name):
    w, ps = CASES[name]
    log(f"[paged] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} page={ps} kv={w.kv_dtype}")
    x = synth.make_inputs(w, with_logits=False)
    rng = np.random.default_rng(7)
    kp, table = paginate(x["k_cache"], ps, rng)
    vp, _ = paginate(x["v_cache"], ps, np.random.default_rng(7))
    d = to_device(x)
    anc, _, _ = st.tree_mask_build(d["parents"])
    out, lse, err = st.tree_attn_verify_paged(d["q"], kp.cuda(), vp.cuda(), d["prefix_lens"], anc,
                                              torch.from_numpy(table).cuda(), x["sm_scale"],
                                              k_scale=d["k_scale"], v_scale=d["v_scale"])
    torch.cuda.synchronize()
    assert int(err[0]) == 0
    # the oracle's own gather of the pages, then the contiguous oracle
    S_pad = table.shape[1] * ps
    ko = oracle.gather_pages(kp.view(torch.uint8).numpy(), table, ps, S_pad)
    vo = oracle.gather_pages(vp.view(torch.uint8).numpy(), table, ps, S_pad)
    xg = dict(x)
    xg["k_cache"] = torch.from_numpy(ko).view(x["k_cache"].dtype)
    xg["v_cache"] = torch.from_numpy(vo).view(x["v_cache"].dtype)
    qo, kg, vg = oracle_views(xg)
    ro, rl = oracle.tree_attention(qo, kg, vg, x["prefix_lens"], x["parents"], x["sm_scale"],
                                   q_fmt=w.q_dtype, kv_fmt=w.kv_dtype, k_scale=x["k_scale"], v_scale=x["v_scale"])
    check_attention(out.float().cpu().numpy(), ro, w.kv_dtype, name)


def test_paged_flags_bad_page_ids():
    w = W[2].replace(B=3, prefix_lo=200, prefix_hi=200, V=10, seed=67)
    x = synth.make_inputs(w, with_logits=False)
    kp, table = paginate(x["k_cache"], 16, np.random.default_rng(3))
    vp, _ = paginate(x["v_cache"], 16, np.random.default_rng(3))
    table = table.copy()
    table[1, 3] = kp.shape[0] + 4                    # outside the pool, in the used range of request 1
    d = to_device(x)
    anc, _, _ = st.tree_mask_build(d["parents"])
    out, lse, err = st.tree_attn_verify_paged(d["q"], kp.cuda(), vp.cuda(), d["prefix_lens"], anc,
                                              torch.from_numpy(table).cuda(), x["sm_scale"])
    torch.cuda.synchronize()
    assert int(err[0]) & st.DERR_PAGE
    # requests that use only valid pages are still correct
    qo, ko, vo = oracle_views(x)
    for b in (0, 2):
        for h in (0, w.Hq - 1):
            ro, _ = oracle.tree_attention_bh(qo, ko, vo, x["prefix_lens"], x["parents"], x["sm_scale"], b, h,
                                             q_fmt="bf16", kv_fmt="bf16")
            check_attention(out[b, :, h].float().cpu().numpy(), ro, "bf16", f"b{b} h{h}")
