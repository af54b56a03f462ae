"""GPU parity of the attention's backward pass (spec_tree_attn_backward)
against the oracle's float64 gradients on the same seeded inputs.

The GPU backward takes the GPU forward pass's own output and log-sum-exp
(as a training step would); the oracle differentiates the exact attention of
the same q, K, V and upstream gradient.

Tolerance.  Like the forward pass, the kernel rounds the probabilities p (and
here also ds) to bf16 before the products that sum over rows or keys, so an
element's error is about 2^-9 times the largest term of its sum, not of the
(possibly cancelling) sum itself.  The forward pass's bound is (2e-2, 1e-2)
on outputs of unit-scale inputs; gradients have no unit scale (a request's
scale like 1 / its key count), so the absolute term is taken against the
largest gradient magnitude of the request:
    |gpu - oracle| <= 2e-2 * max_b|oracle| + 1e-2 * |oracle|   elementwise,
plus a relative L2 error of at most 1e-2 over the whole tensor and,
separately, over the tree rows of dK and dV (a handful of rows per request,
the only ones the mask shapes, which an L2 over all rows would drown out).
The fp32 path is held to 1e-4 in both terms.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_attention_verify_parent_amd as st
from tests.gpu_util import bits16, check_grad, check_tree_rows, log, per_request

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
SENTINEL = 123.0

# (workload, what it exercises): packed rows M = g*N pad to 32, 64 or 128;
# D = 64 and 128; one tile (dq written directly) and many (run partials
# merged); ragged prefixes, empty prefixes, trees whose nodes span tiles.
CASES = {
    "chain6_g4_d128_p2048": W[1].replace(B=2, seed=31),
    "tree16_g8_d128_ragged": W[2].replace(B=3, prefix_lo=100, prefix_hi=1500, seed=32),
    "tree8_g8_d128": W[2].replace(B=2, N=8, max_depth=3, prefix_lo=61, prefix_hi=900, seed=33),
    "chain6_g4_d64_ragged": W[1].replace(B=3, D=64, prefix_lo=300, prefix_hi=700, seed=34),
    "tree16_g8_d64": W[2].replace(B=2, D=64, prefix_lo=0, prefix_hi=400, seed=35),
    "tree8_g8_d64": W[2].replace(B=2, N=8, D=64, max_depth=4, prefix_lo=1000, prefix_hi=1000, seed=36),
    "one_tile_direct": W[1].replace(B=3, prefix_lo=5, prefix_hi=50, seed=37),
    "tree64_g2_deep": W[2].replace(B=2, N=64, Hq=4, Hkv=2, max_depth=30, max_children=2, prefix_lo=0,
                                   prefix_hi=200, seed=38),
    # more than 128 packed rows: the separate dq pass (128-row tiles of the rows) and dK / dV pass
    # (runs of 128-key tiles, the rows streamed 64 at a time).  The 60-node tree of 16 query heads per
    # KV head (960 rows: 8 dq tiles, 15 row steps) over short ragged prefixes (runs of one key tile);
    # the same tree over 16 requests (runs of two key tiles); 160 rows (a partial dq tile and row
    # step); D = 64 over 320 rows with empty prefixes
    "tree60_g16_d128_rowtiles": W[3].replace(B=2, prefix_lo=150, prefix_hi=400, seed=40),
    "tree60_g16_d128_key_runs": W[3].replace(B=16, prefix_lo=200, prefix_hi=600, seed=43),
    # three (request, kv head) sequences: the workgroup grid pads them to a multiple of 8
    "tree20_g16_hkv1_three_seqs": W[2].replace(B=3, N=20, Hq=16, Hkv=1, max_depth=5, max_children=3, prefix_lo=30,
                                               prefix_hi=500, seed=44),
    "tree20_g8_d128_two_tiles": W[2].replace(B=2, N=20, max_depth=5, max_children=3, prefix_lo=64,
                                             prefix_hi=700, seed=41),
    "tree40_g8_d64_three_tiles": W[2].replace(B=2, N=40, D=64, max_depth=6, max_children=4, prefix_lo=0,
                                              prefix_hi=300, seed=42),
    "chain6_f32": W[0],
    # the fp32 path with a branching tree, D = 128, ragged prefixes over several key chunks per wave
    "tree16_f32_d128_ragged": W[0].replace(B=3, N=16, Hq=8, Hkv=2, D=128, tree="random", max_depth=5, max_children=3,
                                           prefix_lo=0, prefix_hi=700, seed=36),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    st.lib()


def _views(x):
    w = x["workload"]
    if w.q_dtype == "f32":
        return x["q"].numpy(), x["k_cache"].numpy(), x["v_cache"].numpy(), x["d_out"].numpy()
    return bits16(x["q"]), bits16(x["k_cache"]), bits16(x["v_cache"]), bits16(x["d_out"])


def run_gpu(x, workspace=None):
    w = x["workload"]
    dev = "cuda"
    q, k, v = x["q"].to(dev), x["k_cache"].to(dev), x["v_cache"].to(dev)
    do = x["d_out"].to(dev)
    parents = torch.from_numpy(x["parents"]).to(dev)
    prefix = torch.from_numpy(x["prefix_lens"]).to(dev)
    anc, _, err = st.tree_mask_build(parents)
    out, lse, err = st.tree_attn_verify(q, k, v, prefix, anc, x["sm_scale"], err=err)
    dk = torch.full_like(k, SENTINEL)
    dv = torch.full_like(v, SENTINEL)
    dq, dk, dv, err = st.tree_attn_backward(q, k, v, prefix, anc, out, lse, do, x["sm_scale"], dk=dk, dv=dv,
                                            workspace=workspace, err=err)
    torch.cuda.synchronize()
    return dq.float().cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy(), int(err[0])


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    w = CASES[name]
    log(f"[backward] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} P=[{w.prefix_lo},{w.prefix_hi}] "
        f"dtype={w.q_dtype} seed={w.seed}")
    x = synth.make_backward_inputs(w)
    dq, dk, dv, err = run_gpu(x)
    assert err == 0
    qo, ko, vo, doo = _views(x)
    rq, rk, rv = oracle.tree_attention_backward(qo, ko, vo, x["prefix_lens"], x["parents"], doo, x["sm_scale"],
                                                q_fmt=w.q_dtype, kv_fmt=w.kv_dtype)
    S = w.S_max
    live = np.zeros((w.B, 1, S, 1), dtype=bool)
    for b in range(w.B):
        live[b, 0, :int(x["prefix_lens"][b]) + w.N] = True
    live = np.broadcast_to(live, dk.shape)
    # rows past each request's tree are not written
    assert (dk[~live] == SENTINEL).all() and (dv[~live] == SENTINEL).all()
    got = per_request(dq, dk, dv, x["prefix_lens"], w.N)
    want = per_request(rq, rk, rv, x["prefix_lens"], w.N)
    for gname, gg, ww in zip(("dq", "dk", "dv"), got, want):
        check_grad(gg, ww, gname, w.q_dtype)
    check_tree_rows(dk, dv, rk, rv, x["prefix_lens"], w.N)


def test_backward_is_deterministic_and_reuses_its_workspace():
    """Two calls on one workspace: the run partials are summed in run order and
    the counters are left at zero, so the second call repeats the first bit
    for bit."""
    w = CASES["chain6_g4_d128_p2048"]
    x = synth.make_backward_inputs(w)
    ws = torch.zeros(st.attn_backward_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.S_max), dtype=torch.uint8,
                     device="cuda")
    assert ws.numel() > 0
    a = run_gpu(x, ws)
    b = run_gpu(x, ws)
    for g1, g2 in zip(a[:3], b[:3]):
        assert np.array_equal(g1, g2)
    assert int(ws.view(torch.int32)[-w.B * w.Hkv:].abs().sum()) == 0


@pytest.mark.parametrize("name", ["tree8_g8_d128", "tree20_g8_d128_two_tiles"])
def test_backward_flags_a_bad_prefix_and_keeps_the_others(name):
    w = CASES[name].replace(B=3, seed=39)
    log(f"[backward bad prefix] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} seed={w.seed}")
    x = synth.make_backward_inputs(w)
    bad = x["prefix_lens"].copy()
    bad[1] = w.S_max - w.N + 1                                  # its tree would run past the cache
    dev = "cuda"
    q, k, v, do = (x[n].to(dev) for n in ("q", "k_cache", "v_cache", "d_out"))
    parents = torch.from_numpy(x["parents"]).to(dev)
    anc, _, _ = st.tree_mask_build(parents)
    good_prefix = torch.from_numpy(x["prefix_lens"]).to(dev)
    out, lse, _ = st.tree_attn_verify(q, k, v, good_prefix, anc, x["sm_scale"])
    dq, dk, dv, err = st.tree_attn_backward(q, k, v, torch.from_numpy(bad).to(dev), anc, out, lse, do,
                                            x["sm_scale"])
    torch.cuda.synchronize()
    assert int(err[0]) & st.DERR_PREFIX
    qo, ko, vo, doo = _views(x)
    keep = [0, 2]
    rq, rk, rv = oracle.tree_attention_backward(qo[keep], ko[keep], vo[keep], x["prefix_lens"][keep],
                                                x["parents"][keep], doo[keep], x["sm_scale"], q_fmt="bf16",
                                                kv_fmt="bf16")
    got = per_request(dq.float().cpu().numpy()[keep], dk.float().cpu().numpy()[keep],
                      dv.float().cpu().numpy()[keep], x["prefix_lens"][keep], w.N)
    want = per_request(rq, rk, rv, x["prefix_lens"][keep], w.N)
    for gname, gg, ww in zip(("dq", "dk", "dv"), got, want):
        check_grad(gg, ww, gname + " (good requests)", "bf16")


def test_backward_row_tiles_are_deterministic():
    """More than 128 packed rows, two calls on one workspace: every gradient
    element is summed by one workgroup in a fixed order (no partial sums, no
    atomics), so the second call repeats the first bit for bit."""
    w = CASES["tree60_g16_d128_rowtiles"]
    x = synth.make_backward_inputs(w)
    ws = torch.zeros(st.attn_backward_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.S_max), dtype=torch.uint8,
                     device="cuda")
    a = run_gpu(x, ws)
    b = run_gpu(x, ws)
    assert a[3] == 0 and b[3] == 0
    for g1, g2 in zip(a[:3], b[:3]):
        assert np.array_equal(g1, g2)
