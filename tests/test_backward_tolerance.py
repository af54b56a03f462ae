"""The backward pass's parity bound is not vacuous (CPU only): gradients of a
slightly wrong problem -- one node hung under another parent, one query row's
upstream gradient dropped, ds without its softmax scale -- computed by the
oracle itself, fail the same checks the GPU gradients must pass."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bits16, check_grad, check_tree_rows, per_request

W = synth.WORKLOADS
CASES = [W[2].replace(B=2, N=8, D=64, max_depth=4, prefix_lo=300, prefix_hi=300, seed=36),
         W[2].replace(B=2, prefix_lo=100, prefix_hi=400, seed=40)]


def _fails(got, ref, prefix, N):
    fails = []
    for gname, a, b in zip(("dq", "dk", "dv"), per_request(*got, prefix, N), per_request(*ref, prefix, N)):
        try:
            check_grad(a, b, gname, "bf16")
        except AssertionError:
            fails.append(gname)
    try:
        check_tree_rows(got[1], got[2], ref[1], ref[2], prefix, N)
    except AssertionError:
        fails.append("tree rows")
    return fails


@pytest.mark.parametrize("w", CASES, ids=["tree8_d64", "tree16_d128"])
def test_bound_rejects_planted_mistakes(w):
    x = synth.make_backward_inputs(w)
    qo, ko, vo, doo = bits16(x["q"]), bits16(x["k_cache"]), bits16(x["v_cache"]), bits16(x["d_out"])
    pre, par, sc = x["prefix_lens"], x["parents"], x["sm_scale"]

    def grads(parents=par, d_out=doo):
        return oracle.tree_attention_backward(qo, ko, vo, pre, parents, d_out, sc, q_fmt="bf16", kv_fmt="bf16")

    ref = grads()
    assert _fails(ref, ref, pre, w.N) == []
    moved = par.copy()
    j = w.N - 1
    moved[0, j] = (moved[0, j] + 1) % j
    assert set(_fails(grads(parents=moved), ref, pre, w.N)) == {"dq", "dk", "dv", "tree rows"}   # a mask error
    dropped = doo.copy()
    dropped[1, 3, 5] = 0
    assert {"dq", "dk", "dv"} <= set(_fails(grads(d_out=dropped), ref, pre, w.N))
    unscaled = (ref[0] / sc, ref[1] / sc, ref[2])
    assert set(_fails(unscaled, ref, pre, w.N)) == {"dq", "dk", "tree rows"}
