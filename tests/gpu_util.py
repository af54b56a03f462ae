"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its C-ABI binding, hand the same bytes to the oracle, compare.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import tree_attention_verify_parent_amd as st

# Attention tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle| elementwise,
# plus a relative L2 guard so that a vanishing output cannot pass on atol alone.
TOL = {"bf16": (2e-2, 1e-2), "e4m3": (6e-2, 1e-2), "f32": (1e-4, 1e-4)}
REL_L2 = 1e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_views(x: dict):
    """The exact bytes the GPU reads, in the form the oracle takes."""
    w = x["workload"]
    q = x["q"]
    if w.q_dtype == "f32":
        qo = q.numpy()
    else:
        qo = bits16(q)
    if w.kv_dtype == "f32":
        ko, vo = x["k_cache"].numpy(), x["v_cache"].numpy()
    elif w.kv_dtype == "bf16":
        ko, vo = bits16(x["k_cache"]), bits16(x["v_cache"])
    else:
        ko = x["k_cache"].view(torch.uint8).numpy()
        vo = x["v_cache"].view(torch.uint8).numpy()
    return qo, ko, vo


def to_device(x: dict, dev="cuda") -> dict:
    d = {}
    for k in ("parents", "draft_tokens", "prefix_lens"):
        d[k] = torch.from_numpy(np.ascontiguousarray(x[k])).to(dev)
    for k in ("q", "k_cache", "v_cache", "logits"):
        if x.get(k) is not None:
            d[k] = x[k].to(dev)
    for k in ("k_scale", "v_scale"):
        d[k] = None if x.get(k) is None else torch.from_numpy(x[k]).to(dev)
    return d


def gpu_step(x: dict, dev="cuda") -> dict:
    d = to_device(x, dev)
    r = st.verify_step(d["parents"], d["draft_tokens"], d["prefix_lens"], d["q"], d["k_cache"],
                       d["v_cache"], d["logits"], x["sm_scale"], k_scale=d["k_scale"],
                       v_scale=d["v_scale"])
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in r.items()}
    out["mask"] = out["mask"].numpy().view(np.uint64)
    out["out"] = out["out"].float().numpy()
    for k in ("depth", "argmax", "accept_len", "path_nodes", "out_tokens", "err"):
        out[k] = out[k].numpy()
    out["lse"] = out["lse"].numpy()
    return out


def oracle_step(x: dict) -> dict:
    w = x["workload"]
    qo, ko, vo = oracle_views(x)
    return oracle.verify_step(x["parents"], x["draft_tokens"], x["prefix_lens"], qo, ko, vo,
                              x["logits"].numpy(), x["sm_scale"], q_fmt=w.q_dtype, kv_fmt=w.kv_dtype,
                              k_scale=x["k_scale"], v_scale=x["v_scale"])


def check_attention(got, want, kv_fmt: str, what: str = "") -> dict:
    atol, rtol = TOL[kv_fmt]
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    worst = float((err / bound).max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    stats = dict(max_abs=float(err.max()) if err.size else 0.0, rel_l2=rel, worst_ratio=worst)
    log(f"  {what} attention: max_abs={stats['max_abs']:.3e} rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert worst <= 1.0, f"{what}: {stats}"
    assert rel <= REL_L2, f"{what}: {stats}"
    return stats


def check_integers(got: dict, want: dict, what: str = "") -> None:
    assert np.array_equal(got["mask"], want["mask"]), f"{what}: mask"
    assert np.array_equal(got["depth"], want["depth"]), f"{what}: depth"
    assert np.array_equal(got["argmax"], want["argmax"]), f"{what}: argmax"
    assert np.array_equal(got["accept_len"], want["accept_len"]), f"{what}: accept_len"
    assert np.array_equal(got["path_nodes"], want["path_nodes"]), f"{what}: path_nodes"
    assert np.array_equal(got["out_tokens"], want["out_tokens"]), f"{what}: out_tokens"


# Backward-pass gradients: |gpu - oracle| <= a * max_b|oracle| + r * |oracle|
# elementwise per request b, relative L2 <= 1e-2 over the tensor and over the
# tree rows of dK / dV (the reasoning is in tests/test_gpu_backward.py).
GRAD_TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}


def check_grad(got, want, what, fmt):
    """got / want: lists with one array per request (that request's rows)."""
    a, r = GRAD_TOL[fmt]
    worst, num, den, max_abs = 0.0, 0.0, 0.0, 0.0
    for gb, wb in zip(got, want):
        gb = np.asarray(gb, dtype=np.float64)
        wb = np.asarray(wb, dtype=np.float64)
        assert np.isfinite(gb).all(), f"{what}: non-finite"
        scale = float(np.abs(wb).max())
        err = np.abs(gb - wb)
        worst = max(worst, float((err / (a * scale + r * np.abs(wb))).max()))
        max_abs = max(max_abs, float(err.max()))
        num += float(np.sum((gb - wb) ** 2))
        den += float(np.sum(wb ** 2))
    rel = (num / max(den, 1e-300)) ** 0.5
    log(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert worst <= 1.0 and rel <= 1e-2, (what, worst, rel)


def per_request(dq, dk, dv, prefix, N):
    """Each request's dq, and its dk / dv rows below P_b + N."""
    L = [int(p) + N for p in prefix]
    return ([dq[b] for b in range(len(L))], [dk[b][:, :L[b]] for b in range(len(L))],
            [dv[b][:, :L[b]] for b in range(len(L))])


def check_tree_rows(dk, dv, rk, rv, prefix, N):
    for gname, G, R in (("dk", dk, rk), ("dv", dv, rv)):
        g = np.concatenate([G[b][:, int(p):int(p) + N].ravel() for b, p in enumerate(prefix)]).astype(np.float64)
        r = np.concatenate([R[b][:, int(p):int(p) + N].ravel() for b, p in enumerate(prefix)])
        rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
        log(f"  {gname} tree rows: rel_l2={rel:.3e}")
        assert rel <= 1e-2, (gname, rel)


def paginate(cache: torch.Tensor, page_size: int, rng):
    """[B][Hkv][S][D] -> (pages [num_pages][page_size][Hkv][D], table int32[B][max_pages]) with the
    pages of all requests shuffled through one pool (plus unused pages)."""
    B, Hkv, S, D = cache.shape
    maxp = -(-S // page_size)
    num_pages = B * maxp + 5
    perm = rng.permutation(num_pages)[: B * maxp].reshape(B, maxp).astype(np.int32)
    padded = torch.zeros(B, Hkv, maxp * page_size, D, dtype=cache.dtype)
    padded[:, :, :S] = cache
    pages = torch.zeros(num_pages, page_size, Hkv, D, dtype=cache.dtype)
    blocks = padded.view(B, Hkv, maxp, page_size, D).permute(0, 2, 3, 1, 4)     # [B][maxp][ps][Hkv][D]
    pages[torch.from_numpy(perm.reshape(-1)).long()] = blocks.reshape(B * maxp, page_size, Hkv, D)
    return pages, perm
