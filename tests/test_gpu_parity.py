"""GPU parity: the HIP library against the CPU oracle on the same seeded
inputs.  Integer outputs (masks, depths, argmax, accept lengths, paths,
tokens) must match bit for bit; attention must satisfy
|gpu - oracle| <= atol + rtol*|oracle| elementwise with (atol, rtol) =
(2e-2, 1e-2) for bf16 KV and (6e-2, 1e-2) for fp8 KV, and a relative L2 error
of at most 1e-2.  The fp32 path is held to (1e-4, 1e-4).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_attention_verify_parent_amd as st
from tests.gpu_util import (bits16, check_attention, check_integers, gpu_step, log, oracle_step,
                            oracle_views, to_device)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

# Reduced versions of the five workloads: same structure (tree shape, GQA
# ratio, head dim, dtypes), sizes the oracle finishes in seconds, ragged
# prefixes that are not multiples of the 64-token tile.
SMALL = {
    "chain6_f32": W[0],
    "chain6_b8_bf16_p2048": W[1],
    "tree16_ragged_bf16": W[2].replace(B=4, prefix_lo=100, prefix_hi=1500, V=5003, seed=12),
    "tree60_bf16": W[3].replace(B=2, prefix_lo=777, prefix_hi=777, V=4099, seed=13),
    "tree16_fp8kv": W[4].replace(B=4, prefix_lo=333, prefix_hi=333, V=6000, seed=14),
    # 960 packed rows (the 8-wave, 256-row plan): ragged prefixes, and an e4m3 cache
    "tree60_ragged_bf16": W[3].replace(B=3, prefix_lo=90, prefix_hi=1900, V=3001, seed=15),
    "tree60_fp8kv": W[3].replace(B=2, kv_dtype="e4m3", prefix_lo=600, prefix_hi=600, V=3001, seed=16),
}


def lse_ok(got, want):
    np.testing.assert_allclose(got, want, rtol=1e-4, atol=1e-3)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    st.lib()


@pytest.mark.parametrize("name", list(SMALL))
def test_verify_step_parity(name):
    w = SMALL[name]
    log(f"[parity] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} P=[{w.prefix_lo},{w.prefix_hi}] "
        f"kv={w.kv_dtype} seed={w.seed}")
    x = synth.make_inputs(w)
    g = gpu_step(x)
    r = oracle_step(x)
    assert int(g["err"][0]) == 0
    check_integers(g, r, name)
    check_attention(g["out"], r["out"], w.kv_dtype, name)
    lse_ok(g["lse"], r["lse"])
    log(f"  accept_len={g['accept_len'].tolist()}")


# ----------------------------------------------------------------- masks

def test_mask_parity_random_trees():
    rng = np.random.default_rng(20)
    for N in (1, 2, 7, 16, 33, 60, 63, 64):
        par = np.stack([[-1] + [int(rng.integers(0, i)) for i in range(1, N)] for _ in range(37)]).astype(np.int32)
        par[0] = np.arange(-1, N - 1)                           # a chain
        par[1] = [-1] + [0] * (N - 1)                           # a star
        anc, dep, err = st.tree_mask_build(torch.from_numpy(par).cuda())
        torch.cuda.synchronize()
        m, d = oracle.build_masks(par)
        assert int(err[0]) == 0
        assert np.array_equal(anc.cpu().numpy().view(np.uint64), m), N
        assert np.array_equal(dep.cpu().numpy(), d), N


def test_mask_flags_bad_parents():
    good = [-1, 0, 0, 1]
    for bit, bad in [(st.DERR_ROOT, [0, 0, 0, 1]), (st.DERR_PARENT, [-1, 0, 2, 1]),
                     (st.DERR_PARENT, [-1, -1, 0, 1]), (st.DERR_PARENT, [-1, 0, 0, 7])]:
        par = torch.tensor([good, bad, good], dtype=torch.int32).cuda()
        anc, dep, err = st.tree_mask_build(par)
        torch.cuda.synchronize()
        assert int(err[0]) & bit, bad
        m, _ = oracle.build_masks(np.array([good]))
        got = anc.cpu().numpy().view(np.uint64)
        assert np.array_equal(got[0], m[0]) and np.array_equal(got[2], m[0])   # neighbours unaffected


# ----------------------------------------------------------------- argmax

def _argmax_case(x: torch.Tensor):
    got = st.vocab_argmax(x.cuda())
    torch.cuda.synchronize()
    want = oracle.vocab_argmax(x.numpy() if x.is_contiguous() else x.contiguous().numpy())
    assert np.array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("rows,V", [(5, 1), (3, 7), (48, 32000), (7, 1000), (300, 4099), (260, 151936)])
def test_argmax_parity_random(rows, V):
    g = torch.Generator().manual_seed(rows * 1000 + V)
    _argmax_case(torch.randn(rows, V, generator=g))


def test_argmax_ties_and_signed_zeros():
    V = 70001
    x = torch.full((12, V), -5.0)
    x[0] = 1.0                                                  # all equal -> 0
    x[1, [5, 40000, 70000]] = 3.0                               # ties across threads/waves -> 5
    x[2, [69999, 1024, 4096]] = 2.0                             # -> 1024
    x[3] = -0.0
    x[3, 9] = 0.0                                               # -0 everywhere, +0 at 9 -> 0
    x[4, 70000] = 9.0                                           # last element
    x[5, 3] = -0.0
    x[5, 2] = 0.0                                               # -> 2
    x[5, 1] = -6.0
    x[6] = torch.arange(V, dtype=torch.float32) % 17            # periodic maxima -> 16
    x[7, 4] = 0.0
    x[7, 1] = -0.0                                              # -0 first, +0 later -> 1
    x[8] = -3.4e38
    x[9, [64, 65]] = 1.0                                        # neighbours within one float4
    x[10, [1023 * 4 + 3, 1024 * 4]] = 1.0                       # straddling an unroll step
    x[11, [V - 1, V - 2]] = 1.0
    _argmax_case(x)
    _argmax_case(x[:200].repeat(2, 1)[:260])                    # many-rows path


def test_argmax_strided_and_misaligned_rows():
    g = torch.Generator().manual_seed(3)
    base = torch.randn(9, 5003, generator=g)
    _argmax_case(base[:, :5001])                                # row stride 5003 != V
    big = torch.randn(6, 4099, generator=g).cuda()
    sub = big[:, 1:]                                            # 4-byte offset: scalar path
    got = st.vocab_argmax(sub)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.vocab_argmax(sub.cpu().contiguous().numpy()))


# ----------------------------------------------------------------- accept walk

def test_walk_parity_random_small_vocab():
    rng = np.random.default_rng(21)
    for N in (1, 2, 6, 16, 40, 64):
        B = 257
        par = np.stack([[-1] + [int(rng.integers(0, i)) for i in range(1, N)] for _ in range(B)]).astype(np.int32)
        V = 3
        d = rng.integers(0, V, size=(B, N)).astype(np.int32)
        t = rng.integers(0, V, size=(B, N)).astype(np.int32)
        dp = torch.from_numpy(par).cuda()
        anc, _, _ = st.tree_mask_build(dp)
        L, path, toks, err = st.accept_walk(dp, anc, torch.from_numpy(d).cuda(), torch.from_numpy(t).cuda(), V)
        torch.cuda.synchronize()
        wl, wp, wt = oracle.accept_walk(par, d, t, V=V)
        assert int(err[0]) == 0
        assert np.array_equal(L.cpu().numpy(), wl), N
        assert np.array_equal(path.cpu().numpy(), wp), N
        assert np.array_equal(toks.cpu().numpy(), wt), N


def test_walk_all_match_and_zero_match_chains():
    N, V = 64, 1000
    par = np.arange(-1, N - 1, dtype=np.int32)[None].repeat(2, 0)
    t = np.arange(N, dtype=np.int32)[None].repeat(2, 0) + 100
    d = np.zeros((2, N), dtype=np.int32)
    d[0, 1:] = t[0, :-1]                        # every node matches -> L = 63
    d[1, 1:] = 7                                # nothing matches -> L = 0
    dp = torch.from_numpy(par).cuda()
    anc, _, _ = st.tree_mask_build(dp)
    L, path, toks, err = st.accept_walk(dp, anc, torch.from_numpy(d).cuda(), torch.from_numpy(t).cuda(), V)
    torch.cuda.synchronize()
    wl, wp, wt = oracle.accept_walk(par, d, t, V=V)
    assert list(L.cpu().numpy()) == [63, 0] == list(wl)
    assert np.array_equal(path.cpu().numpy(), wp) and np.array_equal(toks.cpu().numpy(), wt)


def test_walk_flags_bad_tokens():
    par = torch.tensor([[-1, 0, 1]], dtype=torch.int32).cuda()
    anc, _, _ = st.tree_mask_build(par)
    for d, t in [([0, 5, 1], [1, 2, 3]), ([0, 1, 1], [1, -2, 3])]:
        _, _, _, err = st.accept_walk(par, anc, torch.tensor([d], dtype=torch.int32).cuda(),
                                      torch.tensor([t], dtype=torch.int32).cuda(), 5)
        torch.cuda.synchronize()
        assert int(err[0]) & st.DERR_TOKEN


# ----------------------------------------------------------------- attention edge cases

def _attn_case(w, what, **kw):
    x = synth.make_inputs(w, with_logits=False)
    for k, v in kw.items():
        x[k] = v
    d = to_device(x)
    anc, _, _ = st.tree_mask_build(d["parents"])
    out, lse, err = st.tree_attn_verify(d["q"], d["k_cache"], d["v_cache"], d["prefix_lens"], anc,
                                        x["sm_scale"], k_scale=d["k_scale"], v_scale=d["v_scale"])
    torch.cuda.synchronize()
    assert int(err[0]) == 0
    qo, ko, vo = oracle_views(x)
    ro, rl = oracle.tree_attention(qo, ko, vo, x["prefix_lens"], x["parents"], x["sm_scale"],
                                   q_fmt=w.q_dtype, kv_fmt=w.kv_dtype, k_scale=x["k_scale"],
                                   v_scale=x["v_scale"])
    check_attention(out.float().cpu().numpy(), ro, w.kv_dtype, what)
    lse_ok(lse.cpu().numpy(), rl)
    return out


EDGE = {
    "one_node_p0": W[1].replace(B=3, N=1, prefix_lo=0, prefix_hi=0, V=10),
    "one_node_p65": W[1].replace(B=2, N=1, prefix_lo=65, prefix_hi=65, V=10),
    "chain64_p1": W[1].replace(B=2, N=64, Hq=8, Hkv=8, prefix_lo=1, prefix_hi=1, V=10),
    "tree64_ragged": W[2].replace(B=3, N=64, max_depth=20, max_children=4, Hq=16, Hkv=2,
                                  prefix_lo=0, prefix_hi=200, V=10, seed=31),
    "tree16_d64": W[2].replace(B=2, D=64, prefix_lo=63, prefix_hi=129, V=10, seed=32),
    "fp8_d64_g4": W[4].replace(B=2, D=64, Hq=8, Hkv=2, prefix_lo=500, prefix_hi=500, V=10, seed=33),
    "gqa1_m16": W[1].replace(B=2, N=16, Hq=2, Hkv=2, prefix_lo=70, prefix_hi=70, V=10, seed=34,
                             tree="random", max_depth=5, max_children=3),
    "m48_four_waves_rb1": W[1].replace(B=2, N=12, Hq=16, Hkv=4, prefix_lo=190, prefix_hi=190, V=10, seed=35),
    "m960_tiles": W[3].replace(B=1, prefix_lo=130, prefix_hi=130, V=10, seed=36),
    # 256 packed rows with D = 64 (128-row tiles: the 8-wave plan is for D = 128), bf16 and e4m3 caches
    "m256_d64": W[2].replace(B=2, N=32, D=64, prefix_lo=200, prefix_hi=700, V=10, seed=38),
    "m256_d64_fp8": W[2].replace(B=2, N=32, D=64, kv_dtype="e4m3", prefix_lo=300, prefix_hi=300, V=10, seed=39),
    "f32_d128": W[0].replace(B=2, D=128, Hq=6, Hkv=3, N=9, prefix_lo=31, prefix_hi=300, tree="random",
                             max_depth=4, max_children=3, V=10, seed=37),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_attention_edge_cases(name):
    w = EDGE[name]
    log(f"[edge] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} P=[{w.prefix_lo},{w.prefix_hi}] kv={w.kv_dtype}")
    _attn_case(w, name)


RAMPS = {
    # 960 packed rows (the 8-wave plan), one piece per sequence
    "m960_rising": (W[3].replace(B=1, prefix_lo=900, prefix_hi=900, V=10, seed=81), "rising"),
    # 128 rows over ragged prefixes (balanced pieces, split merges)
    "m128_rising_ragged": (W[2].replace(B=3, prefix_lo=300, prefix_hi=2500, V=10, seed=82), "rising"),
    "m128_sawtooth": (W[2].replace(B=2, prefix_lo=1500, prefix_hi=1500, V=10, seed=83), "sawtooth"),
    # 24 rows, fixed splits and their merge
    "m24_sawtooth": (W[1].replace(B=2, prefix_lo=2000, prefix_hi=2000, V=10, seed=84), "sawtooth"),
}


@pytest.mark.parametrize("name", list(RAMPS))
def test_attention_moving_row_max(name):
    """Scores whose row maxima keep rising along the sequence (K rows scaled up
    to 16x with the token position) or jump up every 256 tokens (a sawtooth of
    scales 1..12): the running reference max of the online softmax then moves
    on many tiles, by more and by less than its lag, inside pieces and across
    the split merge."""
    w, shape = RAMPS[name]
    x = synth.make_inputs(w, with_logits=False)
    k = x["k_cache"].float()
    t = torch.arange(k.shape[2], dtype=torch.float32)
    f = 1.0 + 15.0 * t / k.shape[2] if shape == "rising" else 1.0 + (t // 256) % 12
    k = (k * f[None, None, :, None]).to(x["k_cache"].dtype)
    log(f"[moving max] {name}: K scaled {shape}, up to {float(f.max()):.0f}x")
    _attn_case(w, name, k_cache=k)


def test_attention_many_splits_short_requests():
    """Cache capacity far above the used length: many splits per request in the
    grid, most of them empty; requests of 1, 2 and several splits side by side."""
    w = W[1].replace(B=4, prefix_lo=3000, prefix_hi=3000, V=10)
    x = synth.make_inputs(w, with_logits=False)
    x["prefix_lens"] = np.array([0, 250, 700, 2990], dtype=np.int32)
    _attn_case(w, "many_splits", prefix_lens=x["prefix_lens"])


# Requests that fill their caches run the fixed splits: a sequence's
# ceil(S_max / 64) tiles dealt out in order, the same count to each split and
# one more to each of the last (tiles mod splits).  Lengths chosen for 4
# splits with two longer ones (1100 tokens), 13 (3333), 2 (520), 64 (16390)
# and one whole-sequence piece (259), in bf16 and on the e4m3 decode path.
FIXED = {
    "S1100_4x_r2": W[1].replace(B=2, Hq=8, Hkv=2, prefix_lo=1094, prefix_hi=1094, V=10, seed=51),
    "S3333_13x_r1": W[1].replace(B=2, Hq=8, Hkv=2, prefix_lo=3327, prefix_hi=3327, V=10, seed=52),
    "S520_2x_r1": W[1].replace(B=2, Hq=8, Hkv=2, prefix_lo=514, prefix_hi=514, V=10, seed=53),
    "S16390_64x_r1": W[1].replace(B=2, Hq=8, Hkv=2, prefix_lo=16384, prefix_hi=16384, V=10, seed=54),
    "S259_whole": W[1].replace(B=2, Hq=8, Hkv=2, prefix_lo=253, prefix_hi=253, V=10, seed=55),
    "fp8_S1100": W[4].replace(B=2, Hq=16, Hkv=2, N=6, tree="chain", prefix_lo=1094, prefix_hi=1094, V=10, seed=56),
}


@pytest.mark.parametrize("name", list(FIXED))
def test_attention_fixed_split_remainders(name):
    w = FIXED[name]
    log(f"[fixed] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} P={w.prefix_lo} kv={w.kv_dtype}")
    _attn_case(w, name)


def test_attention_balanced_many_requests():
    """More than 64 requests with ragged lengths: the per-request length table
    spans several 64-entry blocks (two-level search), units cross many short
    sequences (several whole sequences and partial pieces per unit)."""
    w = W[2].replace(B=150, N=5, Hq=8, Hkv=2, D=64, prefix_lo=0, prefix_hi=700, V=10, seed=41,
                     max_depth=3, max_children=2)
    log(f"[balanced] B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} P=[{w.prefix_lo},{w.prefix_hi}]")
    _attn_case(w, "balanced_many_requests")


def test_attention_ragged_with_one_bad_prefix():
    """A ragged batch where one request's prefix length is out of range: it is
    flagged and skipped, the others are balanced and correct."""
    w = W[2].replace(B=6, prefix_lo=100, prefix_hi=2500, V=10, seed=42)
    x = synth.make_inputs(w, with_logits=False)
    d = to_device(x)
    pre = x["prefix_lens"].copy()
    pre[3] = w.S_max                                 # P + N > S_max
    d["prefix_lens"] = torch.from_numpy(pre).cuda()
    anc, _, _ = st.tree_mask_build(d["parents"])
    out, lse, err = st.tree_attn_verify(d["q"], d["k_cache"], d["v_cache"], d["prefix_lens"], anc,
                                        x["sm_scale"])
    torch.cuda.synchronize()
    assert int(err[0]) & st.DERR_PREFIX
    qo, ko, vo = oracle_views(x)
    keep = [b for b in range(w.B) if b != 3]
    ro, rl = oracle.tree_attention(qo[keep], ko[keep], vo[keep], x["prefix_lens"][keep], x["parents"][keep],
                                   x["sm_scale"], q_fmt=w.q_dtype, kv_fmt=w.kv_dtype)
    check_attention(out.float().cpu().numpy()[keep], ro, w.kv_dtype, "ragged_bad_prefix")


def test_attention_is_deterministic():
    w = SMALL["tree16_ragged_bf16"]
    x = synth.make_inputs(w, with_logits=False)
    d = to_device(x)
    anc, _, _ = st.tree_mask_build(d["parents"])
    outs = []
    for _ in range(3):
        o, l, _ = st.tree_attn_verify(d["q"], d["k_cache"], d["v_cache"], d["prefix_lens"], anc, x["sm_scale"])
        outs.append((bits16(o), l.cpu().numpy().copy()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])


def test_attention_flags_bad_prefix_and_spares_others():
    w = W[1].replace(B=3, prefix_lo=100, prefix_hi=100, V=10)
    x = synth.make_inputs(w, with_logits=False)
    d = to_device(x)
    anc, _, _ = st.tree_mask_build(d["parents"])
    for bad in (-1, 101):                                       # 101 + 6 > S_max = 106
        pl = torch.tensor([100, bad, 100], dtype=torch.int32).cuda()
        out, lse, err = st.tree_attn_verify(d["q"], d["k_cache"], d["v_cache"], pl, anc, x["sm_scale"])
        torch.cuda.synchronize()
        assert int(err[0]) & st.DERR_PREFIX
        qo, ko, vo = oracle_views(x)
        for b in (0, 2):
            for h in (0, w.Hq - 1):
                ro, _ = oracle.tree_attention_bh(qo, ko, vo, x["prefix_lens"], x["parents"], x["sm_scale"],
                                                 b, h, q_fmt="bf16", kv_fmt="bf16")
                check_attention(out[b, :, h].float().cpu().numpy(), ro, "bf16", f"prefix{bad} b{b} h{h}")


def test_attention_workspace_too_small_is_rejected():
    w = SMALL["chain6_b8_bf16_p2048"]
    x = synth.make_inputs(w.replace(B=2), with_logits=False)
    d = to_device(x)
    anc, _, _ = st.tree_mask_build(d["parents"])
    need = st.attn_workspace_bytes(2, w.N, w.Hq, w.Hkv, w.D, w.S_max)
    assert need > 0
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(st.SpecError, match="WORKSPACE"):
        st.tree_attn_verify(d["q"], d["k_cache"], d["v_cache"], d["prefix_lens"], anc, x["sm_scale"],
                            workspace=ws)


def test_attention_workspace_is_reusable_across_calls():
    """One zero-filled workspace, several calls with different split counts
    per request: the split counters reset themselves after every call."""
    w = W[1].replace(B=3, prefix_lo=2500, prefix_hi=2500, V=10, seed=41)
    x = synth.make_inputs(w, with_logits=False)
    d = to_device(x)
    anc, _, _ = st.tree_mask_build(d["parents"])
    need = st.attn_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.S_max)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    qo, ko, vo = oracle_views(x)
    for pl in ([2500, 2500, 2500], [10, 1999, 700], [2500, 64, 1300], [2500, 2500, 2500]):
        pre = np.array(pl, dtype=np.int32)
        out, lse, err = st.tree_attn_verify(d["q"], d["k_cache"], d["v_cache"], torch.from_numpy(pre).cuda(),
                                            anc, x["sm_scale"], workspace=ws)
        torch.cuda.synchronize()
        assert int(err[0]) == 0
        ro, rl = oracle.tree_attention(qo, ko, vo, pre, x["parents"], x["sm_scale"], q_fmt="bf16", kv_fmt="bf16")
        check_attention(out.float().cpu().numpy(), ro, "bf16", f"reuse {pl}")
        lse_ok(lse.cpu().numpy(), rl)
