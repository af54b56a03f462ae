"""The fused verify step (spec_verify_step: masks, attention, argmax and
accept walk in one launch, the split kernel's for bf16 and e4m3 caches or the
fp32 kernel's) on the GPU.

Every other GPU parity test of the whole step (test_gpu_parity,
test_gpu_fullsize) already runs through the fused entry point against the
oracle.  Here: it equals the four separate calls bit for bit (the attention
kernel is the same, and integer outputs are exact), its argmax keeps the
lowest index when equal maxima sit in different chunks (each chunk is a
different workgroup folding into one 64-bit key), rows that are strided or
not 16-byte aligned, the workspace it leaves zeroed, and the device error
flags.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_attention_verify_parent_amd as st
from tests.gpu_util import check_attention, check_integers, log, oracle_step, paginate, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

# (workload, what it exercises): the prologue scan (bf16 and the fp8 cache's
# half-size chunks, V a multiple of 4, few rows) or tail scanners (V = 5003
# ending on a scalar tail, 151936 in 19 chunks per row, 4099 in one, N = 60);
# the fp32 kernel's launch.
CASES = {
    "chain6_b8_bf16_p2048": W[1],
    "tree16_ragged_V5003": W[2].replace(B=4, prefix_lo=100, prefix_hi=1500, V=5003, seed=21),
    "tree16_V151936": W[2].replace(B=3, prefix_lo=64, prefix_hi=300, seed=22),
    "tree60_V4099": W[3].replace(B=2, prefix_lo=777, prefix_hi=777, V=4099, seed=23),
    "tree16_fp8kv": W[4].replace(B=4, prefix_lo=333, prefix_hi=333, V=6000, seed=24),
    # 960 packed rows (the 8-wave plan) over an e4m3 cache and ragged prefixes
    "tree60_fp8kv_ragged": W[3].replace(B=2, kv_dtype="e4m3", prefix_lo=200, prefix_hi=1000, V=3001, seed=26),
    "chain6_f32_V1000": W[0],
    # the fp32 kernel with ~32 key chunks per row, about 8 per wave
    "tree16_f32_d128_p2000": W[0].replace(B=2, N=16, tree="random", max_depth=5, max_children=3, Hq=8, Hkv=2, D=128,
                                          prefix_lo=1500, prefix_hi=2000, V=5000, seed=25),
}

KEYS = ("mask", "depth", "argmax", "accept_len", "path_nodes", "out_tokens", "err")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    st.lib()


def _run(d, x, logits=None, fused=True, workspace=None):
    r = st.verify_step(d["parents"], d["draft_tokens"], d["prefix_lens"], d["q"], d["k_cache"], d["v_cache"],
                       d["logits"] if logits is None else logits, x["sm_scale"], k_scale=d["k_scale"],
                       v_scale=d["v_scale"], fused=fused, workspace=workspace)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in r.items()}


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_fused_step_equals_the_four_calls(name):
    w = CASES[name]
    log(f"[step] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} V={w.V} kv={w.kv_dtype} seed={w.seed}")
    x = synth.make_inputs(w)
    d = to_device(x)
    a = _run(d, x, fused=True)
    b = _run(d, x, fused=False)
    for k in KEYS:
        assert np.array_equal(a[k].numpy(), b[k].numpy()), k
    assert np.array_equal(_bits(a["out"]), _bits(b["out"]))
    assert np.array_equal(a["lse"].numpy(), b["lse"].numpy())
    assert int(a["err"][0]) == 0
    # and the integer outputs against the oracle's
    r = oracle_step(x)
    got = {k: (v.numpy().view(np.uint64) if k == "mask" else v.numpy()) for k, v in a.items() if k in KEYS}
    check_integers(got, r, name)


def _small_step(V, seed=5, base=None):
    w = (W[0] if base is None else base).replace(B=2, V=V, seed=seed)
    x = synth.make_inputs(w)
    return w, x, to_device(x)


# Where the argmax runs: the fp32 kernel's prep blocks; bf16 with V a
# multiple of 4 and few rows: the attention workgroups' prologue (one chunk
# each, the mask waves walking); bf16 otherwise: scanning workgroups in the
# attention's tail.
TIE_PATHS = {"f32_kernel": (W[0], 70001), "bf16_prologue": (W[1], 70000), "bf16_tail": (W[1], 70001)}


@pytest.mark.parametrize("path", list(TIE_PATHS))
def test_ties_across_chunks_go_to_the_lowest_index(path):
    # 12 rows of V ~ 70000 logits: 9 to 18 chunks per row; equal maxima placed
    # in different chunks, signed zeros, an all-equal row, the last elements
    base, V = TIE_PATHS[path]
    w, x, d = _small_step(V, base=base)
    rows = w.B * w.N
    lg = torch.full((rows, w.V), -5.0)
    lg[0] = 1.0                                                 # all equal -> 0
    lg[1, [V - 1, 40000, 8192 * 3 + 5]] = 3.0                   # -> 24581
    lg[2, [V - 2, 8191, 8192]] = 2.0                            # neighbouring chunks -> 8191
    lg[3] = -0.0
    lg[3, 60000] = 0.0                                          # -0 == +0 everywhere -> 0
    lg[4, V - 1] = 9.0                                          # the last element
    lg[5, [V - 3, V - 1]] = 4.0                                 # the tail against a float4 -> V - 3
    lg[6, [30000]] = -0.0
    lg[6, [10000]] = 0.0
    lg[6] = torch.where(lg[6] == -5.0, torch.tensor(-1.0), lg[6])   # zeros in two chunks -> 10000
    lg[7] = -3.4e38
    lg[8, 16383] = 1e-30
    lg[8, 16384] = 1e-30                                        # a chunk boundary -> 16383
    lg[9] = torch.arange(w.V, dtype=torch.float32) % 1000       # maxima in every chunk -> 999
    lg[10, 50000] = 7.0
    lg[11, 12345] = -4.0
    got = _run(d, x, logits=lg.cuda())
    want = oracle.vocab_argmax(lg.numpy())
    assert want.tolist()[:10] == [0, 24581, 8191, 0, V - 1, V - 3, 10000, 0, 16383, 999]
    assert np.array_equal(got["argmax"].numpy(), want)
    ref = _run(d, x, logits=lg.cuda(), fused=False)
    for k in KEYS:
        assert np.array_equal(got[k].numpy(), ref[k].numpy()), k


@pytest.mark.parametrize("base", ["f32_kernel", "bf16_one_launch"])
def test_strided_and_misaligned_logits(base):
    w, x, d = _small_step(5003, seed=6, base=W[0] if base == "f32_kernel" else W[1])
    rows = w.B * w.N
    g = torch.Generator().manual_seed(7)
    base_lg = torch.randn(rows, 5005, generator=g).cuda()
    for lg in (base_lg[:, :5003], base_lg[:, 1:5004], base_lg[:, 2:]):   # stride 5005; 4- and 8-byte offsets
        got = _run(d, x, logits=lg)
        ref = _run(d, x, logits=lg, fused=False)
        for k in KEYS:
            assert np.array_equal(got[k].numpy(), ref[k].numpy()), k
        assert np.array_equal(got["argmax"].numpy(), oracle.vocab_argmax(lg.cpu().contiguous().numpy()))


def test_workspace_is_left_zeroed_and_reused():
    w = CASES["tree16_ragged_V5003"]
    x = synth.make_inputs(w)
    d = to_device(x)
    nbytes = st.verify_step_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.S_max)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    a = _run(d, x, workspace=ws)
    prep = (w.B * w.N * 12 + w.B * 4 + 255) // 256 * 256
    assert int(ws[:prep].count_nonzero()) == 0
    b = _run(d, x, workspace=ws)
    for k in KEYS:
        assert np.array_equal(a[k].numpy(), b[k].numpy()), k
    assert np.array_equal(_bits(a["out"]), _bits(b["out"]))
    # a different batch on the same workspace
    x2 = synth.make_inputs(w.replace(seed=99))
    d2 = to_device(x2)
    c = _run(d2, x2, workspace=ws)
    r = oracle_step(x2)
    got = {k: (v.numpy().view(np.uint64) if k == "mask" else v.numpy()) for k, v in c.items() if k in KEYS}
    check_integers(got, r, "second batch")


def test_flags_bad_parents_and_tokens():
    w = CASES["tree16_ragged_V5003"]
    x = synth.make_inputs(w)
    d = to_device(x)
    par = d["parents"].clone()
    par[1, 5] = 7                                               # not an earlier node
    r = st.verify_step(par, d["draft_tokens"], d["prefix_lens"], d["q"], d["k_cache"], d["v_cache"], d["logits"],
                       x["sm_scale"])
    torch.cuda.synchronize()
    assert int(r["err"][0]) & st.DERR_PARENT
    want = oracle_step(x)
    for b in (0, 2, 3):                                         # the other requests are untouched
        assert r["accept_len"][b].item() == want["accept_len"][b]
        assert np.array_equal(r["path_nodes"][b].cpu().numpy(), want["path_nodes"][b])
    tok = d["draft_tokens"].clone()
    tok[2, 3] = w.V
    r = st.verify_step(d["parents"], tok, d["prefix_lens"], d["q"], d["k_cache"], d["v_cache"], d["logits"],
                       x["sm_scale"])
    torch.cuda.synchronize()
    assert int(r["err"][0]) == st.DERR_TOKEN


def test_too_small_workspace_is_rejected_before_any_launch():
    w = CASES["chain6_f32_V1000"]
    x = synth.make_inputs(w)
    d = to_device(x)
    nbytes = st.verify_step_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.S_max)
    ws = torch.zeros(nbytes - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(st.SpecError):
        _run(d, x, workspace=ws)


# Edge cases through the fused entry point, each against the four calls and the
# oracle: a single-node tree (nothing to accept), a one-token vocabulary, one
# request, a full 64-node tree with an fp8 cache, a prefix of zero.
EDGE = {
    "one_node": W[1].replace(B=3, N=1, prefix_lo=100, prefix_hi=300, V=4096, seed=41),
    "vocab_1": W[1].replace(B=2, V=1, seed=42),
    "one_request": W[2].replace(B=1, prefix_lo=2000, prefix_hi=2000, V=8192, seed=43),
    "tree64_fp8": W[4].replace(B=2, N=64, Hq=8, Hkv=4, max_depth=12, max_children=4, prefix_lo=130,
                               prefix_hi=700, V=1024, seed=44),
    "prefix_0": W[2].replace(B=2, prefix_lo=0, prefix_hi=0, V=2000, seed=45),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_fused_step_edge_cases(name):
    w = EDGE[name]
    log(f"[step edge] {name} B={w.B} N={w.N} V={w.V} kv={w.kv_dtype} seed={w.seed}")
    x = synth.make_inputs(w)
    d = to_device(x)
    a = _run(d, x, fused=True)
    b = _run(d, x, fused=False)
    for k in KEYS:
        assert np.array_equal(a[k].numpy(), b[k].numpy()), k
    assert np.array_equal(_bits(a["out"]), _bits(b["out"]))
    assert int(a["err"][0]) == 0
    r = oracle_step(x)
    got = {k: (v.numpy().view(np.uint64) if k == "mask" else v.numpy()) for k, v in a.items() if k in KEYS}
    check_integers(got, r, name)


def test_fused_step_flags_a_bad_prefix_and_keeps_the_others():
    w = CASES["chain6_b8_bf16_p2048"].replace(B=4, prefix_lo=500, prefix_hi=1500, seed=46)
    x = synth.make_inputs(w)
    d = to_device(x)
    bad = d["prefix_lens"].clone()
    bad[2] = w.S_max - w.N + 1                                  # its tree would run past the cache
    r = st.verify_step(d["parents"], d["draft_tokens"], bad, d["q"], d["k_cache"], d["v_cache"], d["logits"],
                       x["sm_scale"])
    torch.cuda.synchronize()
    assert int(r["err"][0]) == st.DERR_PREFIX
    want = oracle_step(x)
    # masks, argmax and walk do not depend on the prefix lengths: every request's are exact
    assert np.array_equal(r["argmax"].cpu().numpy(), want["argmax"])
    assert np.array_equal(r["accept_len"].cpu().numpy(), want["accept_len"])
    assert np.array_equal(r["mask"].cpu().numpy().view(np.uint64), want["mask"])


# (workload, page size or 0 for a contiguous cache): the split kernel's step
# on an e4m3 cache, the fp32 kernel's, and the paged step
GRAPH_CASES = {
    "fp8kv": (CASES["tree16_fp8kv"], 0),
    "f32": (W[0].replace(B=2, V=3000), 0),
    "bf16_paged_p16": (W[2].replace(B=3, prefix_lo=200, prefix_hi=900, V=3001), 16),
}


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_fused_step_replays_in_a_graph(name):
    """Steps captured in a HIP graph on one workspace: every replay, with eager
    work and synchronisation in between, repeats the eager results bit for bit
    (the workspace's keys and counters are left zeroed by each step, and the
    step records no memset)."""
    w, ps = GRAPH_CASES[name]
    log(f"[step graph] {name} B={w.B} N={w.N} kv={w.kv_dtype} page={ps}")
    cases = [synth.make_inputs(w.replace(seed=s)) for s in (51, 52)]
    devs = [to_device(x) for x in cases]
    S = w.S_max
    if ps:
        for j, x in enumerate(cases):
            kp, table = paginate(x["k_cache"], ps, np.random.default_rng(j))
            vp, _ = paginate(x["v_cache"], ps, np.random.default_rng(j))
            devs[j]["k_cache"], devs[j]["v_cache"] = kp.cuda(), vp.cuda()
            devs[j]["table"] = torch.from_numpy(table).cuda()
            S = table.shape[1] * ps
    ws = torch.zeros(st.verify_step_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, S), dtype=torch.uint8,
                     device="cuda")
    outs = [st.step_outputs(w.B, w.N, d["q"]) for d in devs]

    def step(j):
        d = devs[j]
        st.verify_step(d["parents"], d["draft_tokens"], d["prefix_lens"], d["q"], d["k_cache"], d["v_cache"],
                       d["logits"], cases[j]["sm_scale"], k_scale=d["k_scale"], v_scale=d["v_scale"], workspace=ws,
                       outs=outs[j], block_table=d.get("table"))

    for j in range(2):
        step(j)
    torch.cuda.synchronize()
    eager = [{k: v.clone() for k, v in o.items()} for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)                                                 # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in (0, 1, 0):
            step(j)
    for rep in range(3):
        for o in outs:
            for k in o:
                o[k].fill_(-7 if o[k].dtype != torch.int8 else 0)
        g.replay()
        torch.cuda.synchronize()
        for j in range(2):
            for k in KEYS[:-1]:
                assert torch.equal(outs[j][k], eager[j][k]), (rep, j, k)
            assert torch.equal(outs[j]["out"].view(torch.int16), eager[j]["out"].view(torch.int16)), (rep, j)
        assert int(ws[:(w.B * w.N * 12 + w.B * 4 + 255) // 256 * 256].count_nonzero()) == 0
        torch.cuda.synchronize()


# The largest batch the attention takes (1024 requests): the per-request
# length table full, 256 mask workgroups in the step; ragged (balanced shares)
# and uniform (fixed splits, one piece per sequence) prefixes.
MAX_BATCH = {
    "b1024_ragged": W[2].replace(B=1024, N=4, Hq=4, Hkv=1, D=64, prefix_lo=0, prefix_hi=120, V=50, seed=61,
                                 max_depth=3, max_children=2),
    "b1024_uniform": W[1].replace(B=1024, N=4, Hq=4, Hkv=1, D=64, prefix_lo=60, prefix_hi=60, V=50, seed=62),
}


@pytest.mark.parametrize("name", list(MAX_BATCH))
def test_step_at_the_largest_batch(name):
    w = MAX_BATCH[name]
    log(f"[step max batch] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} P=[{w.prefix_lo},{w.prefix_hi}]")
    x = synth.make_inputs(w)
    d = to_device(x)
    a = _run(d, x, fused=True)
    b = _run(d, x, fused=False)
    for k in KEYS:
        assert np.array_equal(a[k].numpy(), b[k].numpy()), k
    assert np.array_equal(_bits(a["out"]), _bits(b["out"]))
    assert int(a["err"][0]) == 0
    r = oracle_step(x)
    got = {k: (v.numpy().view(np.uint64) if k == "mask" else v.numpy()) for k, v in a.items() if k in KEYS}
    check_integers(got, r, name)
    check_attention(a["out"].float().numpy(), r["out"], w.kv_dtype, name)
