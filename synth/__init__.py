"""Seeded synthetic inputs for the speculative-tree verify step.

This module is shared by the tests, the bench and the smoke check. It draws
inputs and nothing else: it builds no ancestor mask, computes no attention,
takes no argmax and walks no tree. Both the CPU oracle and the GPU library
receive exactly the arrays produced here.

Workload recipe (the pages' serving runs use a lookahead of 5 -- Aurora,
"end-to-end throughput at different batch sizes" tables -- and batches of up
to 32; the pages' datasets are not used, these synthetic draws stand in):

  * one seed per workload, split by ``numpy.random.SeedSequence(seed).spawn``
    into eight PCG64 streams, one per component, in this order: prefix
    lengths, parent arrays, planted target tokens, logits, draft tokens, Q,
    K, V (so any component can be drawn without the others);
  * logits are N(0,1) float32; each node's planted target token gets +5;
  * a child's draft token copies its parent's planted token with
    probability ``p_match``, else it is uniform over the vocabulary; the
    root's draft token (the last committed token) is uniform;
  * Q/K/V are N(0,1) (times ``qkv_scale``) rounded to the storage dtype
    (bf16 round-to-nearest-even); for the fp8 KV workload K and V are
    quantised per KV head to OCP e4m3fn with scale = amax/448;
  * trees: chains ``[-1, 0, 1, ...]``, or random parent arrays where each
    new node picks a parent uniformly among earlier nodes whose depth is
    below ``max_depth`` and whose child count is below ``max_children``,
    then relabelled in breadth-first order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    prefix_lo: int
    prefix_hi: int
    V: int
    q_dtype: str           # "f32" | "bf16"
    kv_dtype: str          # "f32" | "bf16" | "e4m3" | "e2m1" (packed, two codes a byte)
    p_match: float
    tree: str = "chain"    # "chain" | "random"
    max_depth: int = 0
    max_children: int = 0
    qkv_scale: float = 1.0
    seed: int = 0

    @property
    def S_max(self) -> int:
        return self.prefix_hi + self.N

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, by what they are.  Sizes follow the verify-step
# shapes described in the design notes (lookahead-5 chains, branching trees,
# a long-context 60-node tree, an fp8 KV cache).
WORKLOADS = [
    Workload("chain6_b1_h4x1_d64_p128_f32", B=1, N=6, Hq=4, Hkv=1, D=64,
             prefix_lo=128, prefix_hi=128, V=1000, q_dtype="f32", kv_dtype="f32",
             p_match=0.7, qkv_scale=1.0 / 8.0, seed=0),
    Workload("chain6_b8_h32x8_d128_p2048_bf16", B=8, N=6, Hq=32, Hkv=8, D=128,
             prefix_lo=2048, prefix_hi=2048, V=32000, q_dtype="bf16", kv_dtype="bf16",
             p_match=0.7, seed=1),
    Workload("tree16_b32_h64x8_d128_p512-8192_bf16", B=32, N=16, Hq=64, Hkv=8, D=128,
             prefix_lo=512, prefix_hi=8192, V=151936, q_dtype="bf16", kv_dtype="bf16",
             p_match=0.6, tree="random", max_depth=5, max_children=3, seed=2),
    Workload("tree60_b16_h64x4_d128_p32768_bf16", B=16, N=60, Hq=64, Hkv=4, D=128,
             prefix_lo=32768, prefix_hi=32768, V=151936, q_dtype="bf16", kv_dtype="bf16",
             p_match=0.5, tree="random", max_depth=6, max_children=10, seed=3),
    Workload("tree16_b64_h64x8_d128_p4096_fp8kv", B=64, N=16, Hq=64, Hkv=8, D=128,
             prefix_lo=4096, prefix_hi=4096, V=151936, q_dtype="bf16", kv_dtype="e4m3",
             p_match=0.7, tree="random", max_depth=5, max_children=3, seed=4),
]

E4M3_MAX = 448.0


def random_tree(rng: np.random.Generator, n: int, max_depth: int, max_children: int) -> np.ndarray:
    """A random parent array with n nodes, depth <= max_depth and at most
    max_children children per node, relabelled breadth-first.

    Depth and child counts are tracked only to honour the generator's limits.
    """
    par = [-1]
    dep = [0]
    kids = [0]
    order_children: list[list[int]] = [[]]
    for i in range(1, n):
        cand = [j for j in range(i) if dep[j] < max_depth and kids[j] < max_children]
        if not cand:
            raise ValueError("tree limits leave no room for another node")
        j = cand[int(rng.integers(0, len(cand)))]
        par.append(j)
        dep.append(dep[j] + 1)
        kids.append(0)
        kids[j] += 1
        order_children.append([])
        order_children[j].append(i)
    # breadth-first relabel: children keep the order in which they were drawn
    new_of = {0: 0}
    queue = [0]
    out_par = [-1]
    head = 0
    while head < len(queue):
        u = queue[head]
        head += 1
        for c in order_children[u]:
            new_of[c] = len(queue)
            queue.append(c)
            out_par.append(new_of[u])
    return np.asarray(out_par, dtype=np.int32)


def make_parents(rng: np.random.Generator, w: Workload) -> np.ndarray:
    if w.tree == "chain":
        one = np.arange(-1, w.N - 1, dtype=np.int32)
        return np.tile(one, (w.B, 1))
    return np.stack([random_tree(rng, w.N, w.max_depth, w.max_children) for _ in range(w.B)])


def _to_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(dtype)


def quantize_e4m3_per_head(x: np.ndarray) -> tuple[torch.Tensor, np.ndarray]:
    """x: [B][Hkv][S][D] float32 -> (e4m3fn tensor, scale float32[Hkv]).

    scale[h] = amax(|x[:, h]|) / 448; the codes are x/scale clamped to the
    e4m3fn range and rounded to nearest even by torch's cast.
    """
    amax = np.abs(x).max(axis=(0, 2, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t / torch.from_numpy(scale).view(1, -1, 1, 1)
    t = t.clamp_(-E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn), scale


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def quantize_e2m1_per_head(x: np.ndarray) -> tuple[torch.Tensor, np.ndarray]:
    """x: [B][Hkv][S][D] float32 -> (packed uint8 [B][Hkv][S][D/2], scale
    float32[Hkv]): scale[h] = amax(|x[:, h]|) / 6, each x/scale rounded to the
    nearest e2m1 value (ties to the even code), element 2j in the low nibble
    of byte j."""
    amax = np.abs(x).max(axis=(0, 2, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(6.0), np.float32(1.0)).astype(np.float32)
    y = (x / scale[None, :, None, None]).astype(np.float64)
    a = np.minimum(np.abs(y), 6.0)
    # nearest magnitude index; a tie goes to the even index (the even code)
    d = np.abs(a[..., None] - E2M1_VALUES)
    best = d.min(axis=-1, keepdims=True)
    cand = (d == best)
    even_pref = cand & ((np.arange(8) % 2) == 0)
    idx = np.where(even_pref.any(axis=-1), even_pref.argmax(axis=-1), cand.argmax(axis=-1))
    code = (idx | np.where((y < 0) & (idx > 0), 8, 0)).astype(np.uint8)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return torch.from_numpy(np.ascontiguousarray(packed)), scale


def make_inputs(w: Workload, seed: Optional[int] = None, with_logits: bool = True) -> dict:
    """Draw one batch of verify-step inputs for workload ``w``.

    Returns CPU tensors / arrays:
      parents int32[B][N], draft_tokens int32[B][N], planted int32[B][N],
      prefix_lens int32[B], q [B][N][Hq][D], k_cache/v_cache [B][Hkv][S_max][D],
      k_scale/v_scale float32[Hkv] (fp8 and fp4 only, else None),
      logits float32[B*N][V] (unless with_logits=False), sm_scale.
    Tree node j of request b lives in cache row prefix_lens[b] + j.
    """
    seed = w.seed if seed is None else seed
    streams = [np.random.Generator(np.random.PCG64(s))
               for s in np.random.SeedSequence(seed).spawn(8)]
    r_prefix, r_tree, r_plant, r_logit, r_draft, r_q, r_k, r_v = streams
    B, N, V = w.B, w.N, w.V
    if w.prefix_lo == w.prefix_hi:
        prefix = np.full(B, w.prefix_lo, dtype=np.int32)
    else:
        prefix = r_prefix.integers(w.prefix_lo, w.prefix_hi, size=B, endpoint=True).astype(np.int32)
    parents = make_parents(r_tree, w)
    planted = r_plant.integers(0, V, size=(B, N)).astype(np.int32)
    logits = None
    if with_logits:
        lg = r_logit.standard_normal((B * N, V), dtype=np.float32)
        lg[np.arange(B * N), planted.reshape(-1)] += np.float32(5.0)
        logits = torch.from_numpy(lg)
    u = r_draft.random((B, N))
    uni = r_draft.integers(0, V, size=(B, N)).astype(np.int32)
    par_tok = np.take_along_axis(planted, np.maximum(parents, 0), axis=1)
    draft = np.where(u < w.p_match, par_tok, uni).astype(np.int32)
    draft[:, 0] = uni[:, 0]
    S = w.S_max
    q = r_q.standard_normal((B, N, w.Hq, w.D), dtype=np.float32)
    if w.qkv_scale != 1.0:
        q *= np.float32(w.qkv_scale)
    k = r_k.standard_normal((B, w.Hkv, S, w.D), dtype=np.float32)
    if w.qkv_scale != 1.0:
        k *= np.float32(w.qkv_scale)
    kt, ks = _kv_storage(k, w)
    del k
    v = r_v.standard_normal((B, w.Hkv, S, w.D), dtype=np.float32)
    if w.qkv_scale != 1.0:
        v *= np.float32(w.qkv_scale)
    vt, vs = _kv_storage(v, w)
    del v
    return dict(
        workload=w,
        parents=parents,
        draft_tokens=draft,
        planted=planted,
        prefix_lens=prefix,
        q=_to_storage(q, w.q_dtype),
        k_cache=kt,
        v_cache=vt,
        k_scale=ks,
        v_scale=vs,
        logits=logits,
        sm_scale=1.0 / math.sqrt(w.D),
    )


def make_backward_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """The verify-step inputs of ``w`` (without logits) plus an upstream
    gradient d_out [B][N][Hq][D] ~ N(0, 1) in q's dtype, drawn from a stream
    of its own, for the attention's backward pass.  fp8 caches are not
    differentiated: ``w`` must use f32 or bf16 K/V."""
    if w.kv_dtype not in ("f32", "bf16"):
        raise ValueError("the backward pass takes f32 or bf16 caches")
    x = make_inputs(w, seed, with_logits=False)
    seed = w.seed if seed is None else seed
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xB0]).generate_state(2)))
    g = r.standard_normal((w.B, w.N, w.Hq, w.D), dtype=np.float32)
    x["d_out"] = _to_storage(g, w.q_dtype)
    return x


def _kv_storage(x: np.ndarray, w: Workload):
    if w.kv_dtype == "e4m3":
        return quantize_e4m3_per_head(x)
    if w.kv_dtype == "e2m1":
        return quantize_e2m1_per_head(x)
    return _to_storage(x, w.kv_dtype), None


def workload_by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)
