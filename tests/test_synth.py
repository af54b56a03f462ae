"""Checks of the seeded input generator (CPU only)."""
import numpy as np
import pytest
import torch

import synth


def small(w, **kw):
    base = dict(B=min(w.B, 4), prefix_lo=min(w.prefix_lo, 300), prefix_hi=min(w.prefix_hi, 700),
                V=min(w.V, 2000))
    base.update(kw)
    return w.replace(**base)


@pytest.mark.parametrize("idx", range(5))
def test_shapes_and_dtypes(idx):
    w = small(synth.WORKLOADS[idx])
    x = synth.make_inputs(w)
    B, N, S = w.B, w.N, w.S_max
    assert x["parents"].shape == (B, N) and x["parents"].dtype == np.int32
    assert x["draft_tokens"].shape == (B, N)
    assert x["q"].shape == (B, N, w.Hq, w.D)
    assert x["k_cache"].shape == (B, w.Hkv, S, w.D) == x["v_cache"].shape
    assert x["logits"].shape == (B * N, w.V) and x["logits"].dtype == torch.float32
    want = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}
    assert x["q"].dtype == want[w.q_dtype]
    assert x["k_cache"].dtype == want[w.kv_dtype]
    assert (x["prefix_lens"] >= w.prefix_lo).all() and (x["prefix_lens"] <= w.prefix_hi).all()
    assert ((x["draft_tokens"] >= 0) & (x["draft_tokens"] < w.V)).all()
    if w.kv_dtype == "e4m3":
        assert x["k_scale"].shape == (w.Hkv,) and (x["k_scale"] > 0).all()
        codes = x["k_cache"].view(torch.uint8)
        assert not ((codes & 0x7F) == 0x7F).any()          # no NaN codes


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_tree_limits_and_bfs_order(idx):
    w = small(synth.WORKLOADS[idx], B=40)
    p = synth.make_inputs(w, with_logits=False)["parents"]
    for row in p:
        assert row[0] == -1
        assert all(0 <= row[i] < i for i in range(1, len(row)))
        assert all(row[i] <= row[i + 1] for i in range(1, len(row) - 1))   # BFS: parents non-decreasing
        depth = [0] * len(row)
        for i in range(1, len(row)):
            depth[i] = depth[row[i]] + 1
        assert max(depth) <= w.max_depth
        assert np.bincount(row[1:], minlength=len(row)).max() <= w.max_children


def test_chain_workloads_are_chains():
    for idx in (0, 1):
        p = synth.make_inputs(small(synth.WORKLOADS[idx]), with_logits=False)["parents"]
        assert (p == np.arange(-1, p.shape[1] - 1)).all()


def test_seeded_and_deterministic():
    w = small(synth.WORKLOADS[2])
    a, b = synth.make_inputs(w), synth.make_inputs(w)
    for k in ("parents", "draft_tokens", "prefix_lens", "planted"):
        assert np.array_equal(a[k], b[k])
    assert torch.equal(a["k_cache"], b["k_cache"]) and torch.equal(a["logits"], b["logits"])
    c = synth.make_inputs(w, seed=123)
    assert not torch.equal(a["k_cache"], c["k_cache"])
    d = synth.make_inputs(w, with_logits=False)                  # skipping logits changes nothing else
    assert np.array_equal(a["draft_tokens"], d["draft_tokens"]) and torch.equal(a["q"], d["q"])


def test_planted_tokens_and_draft_match_rate():
    w = small(synth.WORKLOADS[1], B=64, V=500)
    x = synth.make_inputs(w)
    lg = x["logits"].numpy()
    planted = x["planted"].reshape(-1)
    assert (lg[np.arange(lg.shape[0]), planted] > 2.0).mean() > 0.95
    par = x["parents"]
    copies = x["draft_tokens"][:, 1:] == np.take_along_axis(x["planted"], par[:, 1:], axis=1)
    assert abs(copies.mean() - w.p_match) < 0.06


def test_config0_values_are_scaled():
    x = synth.make_inputs(synth.WORKLOADS[0])
    assert 0.09 < float(x["k_cache"].std()) < 0.16
