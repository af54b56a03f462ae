"""GPU parity at the five workloads' full sizes, in the launch configuration
the bench times.  Masks, argmax, accept lengths, paths and tokens are compared
in full; attention is compared on every head and node of whole requests (the
first and last request, and for ragged prefixes also the shortest and the
longest), which the oracle computes one request at a time, plus a few single
(request, head) pairs from the oracle's one-pair call.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check_attention, check_integers, gpu_step, log, oracle_views

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("idx", range(5))
def test_full_size_workload(idx):
    w = synth.WORKLOADS[idx]
    log(f"[full] {w.name}: generating inputs (seed {w.seed})")
    x = synth.make_inputs(w)
    log(f"[full] {w.name}: GPU step")
    g = gpu_step(x)
    assert int(g["err"][0]) == 0
    log(f"[full] {w.name}: oracle integers")
    mask, depth = oracle.build_masks(x["parents"])
    t = oracle.vocab_argmax(x["logits"].numpy())
    L, path, toks = oracle.accept_walk(x["parents"], x["draft_tokens"], t, V=w.V)
    check_integers(g, dict(mask=mask, depth=depth, argmax=t, accept_len=L, path_nodes=path,
                           out_tokens=toks), w.name)
    log(f"  accept_len mean={L.mean():.2f} max={L.max()} (tree depth {depth.max()}); "
        f"argmax==planted {np.mean(t == x['planted'].reshape(-1)):.3f}")
    qo, ko, vo = oracle_views(x)
    reqs = {0, w.B - 1, int(np.argmin(x["prefix_lens"])), int(np.argmax(x["prefix_lens"]))}
    for b in sorted(reqs):
        sl = slice(b, b + 1)
        ro, rl = oracle.tree_attention(qo[sl], ko[sl], vo[sl], x["prefix_lens"][sl], x["parents"][sl],
                                       x["sm_scale"], q_fmt=w.q_dtype, kv_fmt=w.kv_dtype, k_scale=x["k_scale"],
                                       v_scale=x["v_scale"])
        check_attention(g["out"][b], ro[0], w.kv_dtype, f"{w.name} request {b} (all {w.Hq} heads) "
                                                         f"P={x['prefix_lens'][b]}")
        np.testing.assert_allclose(g["lse"][b], rl[0], rtol=1e-4, atol=1e-3)
    rng = np.random.default_rng(100 + idx)
    for _ in range(3):
        b, h = int(rng.integers(0, w.B)), int(rng.integers(0, w.Hq))
        ro, rl = oracle.tree_attention_bh(qo, ko, vo, x["prefix_lens"], x["parents"], x["sm_scale"], b, h,
                                          q_fmt=w.q_dtype, kv_fmt=w.kv_dtype, k_scale=x["k_scale"],
                                          v_scale=x["v_scale"])
        check_attention(g["out"][b, :, h], ro, w.kv_dtype, f"{w.name} b{b} h{h} P={x['prefix_lens'][b]}")
        np.testing.assert_allclose(g["lse"][b, :, h], rl, rtol=1e-4, atol=1e-3)
