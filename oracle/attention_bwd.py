"""Backward pass of the tree-masked attention, in float64.

Test infrastructure only (see the package docstring).

What is computed, and the reading of the pages it follows:

  * Aurora trains the draft model on each verification's accepted and
    rejected branches at once: the custom tree mask lets every branch go
    through one batched forward and backward pass (Aurora, everytik.com and
    chernovdev.ru mirrors, section 2, closing paragraph on tree attention).
  * Reading: the backward pass of the same attention as ``attention.py``,
    under the same mask.  Given the upstream gradient dO of every output
    row, it returns the gradients of  sum_{b,i,h} <dO[b,i,h], out[b,i,h]>
    with respect to q and to the K and V cache rows that the forward pass
    reads (prefix rows and tree rows of each request).  Rows at or past
    P_b + N take no part in the forward pass; their gradient is zero.

For one request, one query head h (kv head kvh = h // g) and the N x L
visibility A of the forward pass (L = P + N keys), with w the softmax
weights of the forward pass:

    dV[c]   += sum_i w[i][c] * dO[i]                      (out = w V)
    dw[i][c] = <dO[i], V[c]>
    ds[i][c] = w[i][c] * (dw[i][c] - sum_c' w[i][c'] dw[i][c'])
                                                         (softmax Jacobian)
    dq[i]    = sm_scale * sum_c ds[i][c] K[c]            (s = sm_scale q K^T)
    dK[c]   += sm_scale * sum_i ds[i][c] q[i]

dK and dV sum over the g query heads that share kv head kvh.  Masked
entries have w = 0, so they contribute nothing.
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64, _request, dense_tree_mask


def _softmax_weights(Q, Kf, A, sm_scale):
    """w [N][L] of the forward pass, masked entries exactly 0."""
    s = float(sm_scale) * (Q @ Kf.T)
    s = np.where(A, s, -np.inf)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def _attend_backward(Q, Kf, Vf, A, dO, sm_scale):
    """One head: Q, dO [N][D]; Kf, Vf [L][D]; A bool[N][L].
    Returns (dQ [N][D], dK [L][D], dV [L][D]) in float64."""
    w = _softmax_weights(Q, Kf, A, sm_scale)
    dV = w.T @ dO
    dw = dO @ Vf.T
    ds = w * (dw - (w * dw).sum(axis=1, keepdims=True))
    dQ = float(sm_scale) * (ds @ Kf)
    dK = float(sm_scale) * (ds.T @ Q)
    return dQ, dK, dV


def tree_attention_backward(q, k_cache, v_cache, prefix_lens, parents, d_out, sm_scale, *, q_fmt, kv_fmt):
    """Gradients (dq float64[B][N][Hq][D], dk, dv float64[B][Hkv][S_max][D]).

    q, d_out: [B][N][Hq][D] in q_fmt ("f32" values or "bf16" uint16 bit
    patterns); k_cache, v_cache: [B][Hkv][S_max][D] in kv_fmt ("f32" or
    "bf16"); parents int[B][N]; prefix_lens int[B].
    """
    B, N, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    dq = np.zeros((B, N, Hq, D), dtype=np.float64)
    dk = np.zeros((B, Hkv, S_max, D), dtype=np.float64)
    dv = np.zeros((B, Hkv, S_max, D), dtype=np.float64)
    for b in range(B):
        P, L, g = _request(q, k_cache, prefix_lens, b)
        A = dense_tree_mask(parents[b], P)
        for kvh in range(Hkv):
            Kf = _as_f64(np.asarray(k_cache[b, kvh, :L]), kv_fmt)
            Vf = _as_f64(np.asarray(v_cache[b, kvh, :L]), kv_fmt)
            for h in range(kvh * g, (kvh + 1) * g):
                Q = _as_f64(np.asarray(q[b, :, h, :]), q_fmt)
                dO = _as_f64(np.asarray(d_out[b, :, h, :]), q_fmt)
                dQh, dKh, dVh = _attend_backward(Q, Kf, Vf, A, dO, sm_scale)
                dq[b, :, h, :] = dQh
                dk[b, kvh, :L] += dKh
                dv[b, kvh, :L] += dVh
    return dq, dk, dv
