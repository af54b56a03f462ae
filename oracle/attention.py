"""Tree-masked attention over a KV-cache prefix, in float64.

Test infrastructure only (see the package docstring).

What is computed (Aurora section 2, closing paragraph: a custom attention
mask that respects the speculative tree's causal structure; the target
verifies the whole proposal in one parallel pass, Runtime Draft Model
Training, "Overview"):

  For request b with prefix length P, tree node i and query head h
  (kv head = h // g, g = Hq / Hkv, contiguous GQA groups -- a reading, the
  pages are silent on head grouping):
    keys c = 0 .. P+N-1 of the cache, where row c < P is a prefix token and
    row P+j is tree node j (a reading: the tree's K/V rows are appended to the
    request's cache right after its prefix);
    A[i][c] = (c < P) or (c - P in anc*(i));
    s_c = sm_scale * <q[b,i,h,:], K[b,kvh,c,:]>            for A[i][c];
    w_c = exp(s_c - max s) / sum_c' exp(s_c' - max s);
    out[b,i,h,:] = sum_c w_c * V[b,kvh,c,:];
    lse[b,i,h]  = max s + log(sum_c exp(s_c - max s)).

Inputs are upcast exactly to float64: float32 as is, bf16 from its bit
pattern (the upper 16 bits of a float32), OCP e4m3fn and e2m1 (two codes a
byte, element 2j in the low nibble of byte j) from their definitions times
the per-KV-head float32 scale.
"""
from __future__ import annotations

import numpy as np

from .tree import _check_parents, ancestors


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 OCP FP8 E4M3 ("e4m3fn") codes, float64.

    Layout: sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
    field 0 encodes subnormals m/8 * 2^-6; 0x7F and 0xFF are NaN; there are
    no infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            tab[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


_E4M3 = e4m3_decode_table()


def e2m1_decode_table() -> np.ndarray:
    """Value of each of the 16 OCP FP4 E2M1 codes, float64.

    Layout: sign bit, 2 exponent bits (bias 1), 1 mantissa bit.  Exponent
    field 0 encodes the subnormal m * 0.5; there are no infinities or NaNs,
    so the largest magnitude is 1.5 * 2^2 = 6.
    """
    tab = np.empty(16, dtype=np.float64)
    for code in range(16):
        s = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        tab[code] = s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return tab


_E2M1 = e2m1_decode_table()


def decode_e2m1_packed(packed, scale: float) -> np.ndarray:
    """Packed e2m1 rows [..., D/2] (element 2j in the low nibble of byte j)
    -> float64 [..., D], times the fp32 scale."""
    b = np.asarray(packed, dtype=np.uint8)
    lo, hi = _E2M1[b & 0xF], _E2M1[b >> 4]
    out = np.stack([lo, hi], axis=-1).reshape(*b.shape[:-1], 2 * b.shape[-1])
    return out * float(scale)


def decode_e4m3(codes, scale: float) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)] * float(scale)


def _as_f64(x, fmt: str) -> np.ndarray:
    if fmt == "f64":                 # values already exact in float64 (e.g. a dequantized e4m3 q)
        return np.asarray(x, dtype=np.float64)
    if fmt == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(x)
    raise ValueError(fmt)


def dense_tree_mask(parents_b, P: int) -> np.ndarray:
    """A[i][c] for one request: bool[N][P+N]."""
    p = [int(x) for x in parents_b]
    _check_parents(p)
    N = len(p)
    A = np.zeros((N, P + N), dtype=bool)
    A[:, :P] = True
    for i in range(N):
        for j in ancestors(p, i):
            A[i, P + j] = True
    return A


def _kv_rows(cache, b: int, kvh: int, L: int, fmt: str, scale) -> np.ndarray:
    rows = np.asarray(cache[b, kvh, :L])
    if fmt == "e4m3":
        return decode_e4m3(rows, scale[kvh])
    if fmt == "e2m1":
        return decode_e2m1_packed(rows, scale[kvh])
    return _as_f64(rows, fmt)


def _attend(Q, Kf, Vf, A, sm_scale):
    """Q [N][D], Kf/Vf [L][D] float64, A bool[N][L] -> (out [N][D], lse [N])."""
    s = float(sm_scale) * (Q @ Kf.T)                         # [N][L]
    s = np.where(A, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)                                        # masked -> exp(-inf) = 0
    den = e.sum(axis=1, keepdims=True)
    w = e / den
    out = w @ Vf
    lse = (m + np.log(den))[:, 0]
    return out, lse


def _request(q, k_cache, prefix_lens, b):
    B, N, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    P = int(prefix_lens[b])
    if P < 0 or P + N > S_max:
        raise ValueError(f"prefix {P} + {N} nodes does not fit {S_max} cache rows")
    return P, P + N, Hq // Hkv


def tree_attention_bh(q, k_cache, v_cache, prefix_lens, parents, sm_scale, b, h, *,
                      q_fmt, kv_fmt, k_scale=None, v_scale=None):
    """Outputs of all N nodes of request b for query head h.

    q: [B][N][Hq][D] (float32 values, or uint16 bf16 bit patterns);
    k_cache/v_cache: [B][Hkv][S_max][D] (float32, uint16 bf16 bits or uint8
    e4m3 codes).  Returns (out float64[N][D], lse float64[N]).
    """
    P, L, g = _request(q, k_cache, prefix_lens, b)
    kvh = h // g
    A = dense_tree_mask(parents[b], P)
    Kf = _kv_rows(k_cache, b, kvh, L, kv_fmt, k_scale)
    Vf = _kv_rows(v_cache, b, kvh, L, kv_fmt, v_scale)
    Q = _as_f64(np.asarray(q[b, :, h, :]), q_fmt)            # [N][D]
    return _attend(Q, Kf, Vf, A, sm_scale)


def tree_attention(q, k_cache, v_cache, prefix_lens, parents, sm_scale, *,
                   q_fmt, kv_fmt, k_scale=None, v_scale=None):
    """All outputs: (out float64[B][N][Hq][D], lse float64[B][N][Hq]).

    Same arithmetic as tree_attention_bh for every (b, h); the exact upcast
    of a kv head's rows is done once and shared by the heads of its group.
    """
    B, N, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    out = np.empty((B, N, Hq, D), dtype=np.float64)
    lse = np.empty((B, N, Hq), dtype=np.float64)
    for b in range(B):
        P, L, g = _request(q, k_cache, prefix_lens, b)
        A = dense_tree_mask(parents[b], P)
        for kvh in range(Hkv):
            Kf = _kv_rows(k_cache, b, kvh, L, kv_fmt, k_scale)
            Vf = _kv_rows(v_cache, b, kvh, L, kv_fmt, v_scale)
            for h in range(kvh * g, (kvh + 1) * g):
                Q = _as_f64(np.asarray(q[b, :, h, :]), q_fmt)
                out[b, :, h, :], lse[b, :, h] = _attend(Q, Kf, Vf, A, sm_scale)
    return out, lse
