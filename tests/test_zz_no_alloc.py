"""spec_verify_step_static (the verify step on the library's static
scratch, for callers that cannot allocate) against spec_verify_step with a
caller workspace, through the C ABI: two calls in a row, the second with a
smaller input, each compared with the workspace entry point's outputs on the
same inputs -- bit for bit, since both run the same kernels.  Then a graph
of the static call, replayed with eager work between replays."""
import numpy as np
import pytest
import torch

import synth
import tree_attention_verify_parent_amd as st
from tests.gpu_util import log, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CASES = [
    W[2].replace(B=6, prefix_lo=300, prefix_hi=2100, V=20000, seed=91),      # ragged 16-node trees
    W[1].replace(B=2, prefix_lo=500, prefix_hi=500, V=3000, seed=92),        # smaller: a chain
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    st.lib()


def _run(fn, w, d, x):
    o = st.step_outputs(w.B, w.N, d["q"])
    fn(o)
    torch.cuda.synchronize()
    return {k: v.clone() for k, v in o.items()}


def _static(w, d, x):
    return lambda o: st.verify_step_static(d["parents"], d["draft_tokens"], d["prefix_lens"], d["q"], d["k_cache"],
                                           d["v_cache"], d["logits"], x["sm_scale"], k_scale=d["k_scale"],
                                           v_scale=d["v_scale"], outs=o)


def _with_workspace(w, d, x):
    ws = torch.zeros(st.verify_step_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.S_max), dtype=torch.uint8,
                     device=d["q"].device)
    return lambda o: st.verify_step(d["parents"], d["draft_tokens"], d["prefix_lens"], d["q"], d["k_cache"],
                                    d["v_cache"], d["logits"], x["sm_scale"], k_scale=d["k_scale"],
                                    v_scale=d["v_scale"], workspace=ws, outs=o)


def _same(a, b, what):
    for k in a:
        assert torch.equal(a[k], b[k]), f"{what}: {k} differs"


def test_static_scratch_matches_workspace_entry_point():
    for w in CASES:
        log(f"[static] {w.name} B={w.B} N={w.N} P=[{w.prefix_lo},{w.prefix_hi}] V={w.V} seed={w.seed}")
        x = synth.make_inputs(w)
        d = to_device(x)
        want = _run(_with_workspace(w, d, x), w, d, x)
        assert int(want["err"][0]) == 0
        got = _run(_static(w, d, x), w, d, x)
        _same(got, want, w.name)
        log(f"  equal; accept_len={got['accept_len'].tolist()}")


def test_static_scratch_in_a_graph():
    w = CASES[1]
    x = synth.make_inputs(w)
    d = to_device(x)
    want = _run(_with_workspace(w, d, x), w, d, x)
    o = st.step_outputs(w.B, w.N, d["q"])
    call = _static(w, d, x)
    call(o)                                     # eager first: set-up outside the capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(o)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in o:
            if k != "err":
                o[k].fill_(-7 if o[k].dtype != torch.bfloat16 else 0.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in o.items()}
        _same(got, want, f"replay {rep}")
        # eager work between replays, on the same scratch
        _run(_static(w, d, x), w, d, x)
    log("  three replays equal")
