#!/usr/bin/env python3
"""Verify-step throughput on one MI355X.

One step = the whole verify hot path for one batch of synthetic inputs that
are already resident in HBM: ancestor-mask build, tree-masked split-KV
attention, per-node vocabulary argmax, accept walk -- by default one
spec_verify_step call (one launch: the attention kernel's grid also holds
the mask, argmax and walk workgroups); --unfused times the four separate
calls instead.

The headline workload is the long-context EAGLE-style tree: 16 requests,
60-node trees, 64 query heads over 4 KV heads, head dim 128, 32768-token
prefixes, bf16, vocabulary 151936.  Every other workload gets an entry of its
own in ``per_workload`` (same measurements, its own step count).

Timing: W untimed warm-up steps, then exactly K steps timed with torch.cuda
synchronisation on both sides.  Steps run as replays of HIP graphs, each
holding up to --steps-per-graph consecutive steps (fewer when a step is
long, and a shorter graph for a remainder, so any K and W work).  Each step
reads one of R input replicas, with R chosen so that the replicas together
exceed the GPU's last-level (MALL) cache, so every step streams its K/V and
logits from HBM.  HIP events around every graph replay give the p10 / p50 /
p90 of the per-step time.

The dominant kernel (the tree attention) is also timed on its own with HIP
events on the stream that runs it: a graph of back-to-back attention calls
over the replicas, elapsed time / number of calls.  Its algorithmic bytes
(each K/V byte of every request's prefix + tree once per KV head, Q, outputs,
masks) or flops (dense packed tiles) over that time give roofline.achieved.

The CPU oracle is timed first, before the GPU is touched, on a process pool
over requests (one request per worker, one BLAS thread each).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
BF16_RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)       # flop per byte
METRIC = "tree-verify steps/sec and achieved HBM GB/s (% of peak) on 1 MI355X"
HEADLINE = "tree60_b16_h64x4_d128_p32768_bf16"
GRAPH_TARGET_S = 500e-6          # a graph holds about this much GPU work (at most --steps-per-graph steps)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE, help="headline workload: name or index 0-4")
    ap.add_argument("--workloads", default="all",
                    help="workloads of the per_workload block: 'all', 'none' or a comma list of names / indices")
    ap.add_argument("--per-workload-seconds", type=float, default=0.25,
                    help="timed GPU time per non-headline workload (its step count follows from it)")
    ap.add_argument("--no-graph", action="store_true", help="launch each step's calls eagerly")
    ap.add_argument("--unfused", action="store_true",
                    help="time the four separate calls (mask, attention, argmax, walk) instead of spec_verify_step")
    ap.add_argument("--steps-per-graph", type=int, default=25,
                    help="at most this many verify steps captured in one HIP graph")
    ap.add_argument("--replica-bytes", type=float, default=1.0e9,
                    help="total bytes of input replicas to rotate through (defeats the MALL)")
    ap.add_argument("--attn-calls", type=int, default=200, help="at most this many calls per attention timing graph")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=20.0)
    ap.add_argument("--cpu-workers", type=int, default=0, help="oracle worker processes (0: min(16, host CPUs))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the commit, paged, backward and fp8 timings")
    ap.add_argument("--page-size", type=int, default=16,
                    help="page size of the paged-cache timings (doubled until a request fits the block table; "
                         "0: skip)")
    ap.add_argument("--copy-calibration", type=float, default=0,
                    help="only run a plain float32 elementwise copy that reads and writes this many "
                         "bytes (5 launches) and exit: the reference point that scales the HBM byte "
                         "counters of a rocprofv3 --pmc pass")
    return ap.parse_args(argv)


def graph_blocks(start: int, count: int, per_graph: int) -> list:
    """Steps start .. start+count-1 as (first step, length) blocks of at most
    per_graph steps: whole blocks, then one shorter block for the remainder."""
    per_graph = max(1, int(per_graph))
    out, i, end = [], int(start), int(start) + int(count)
    while i < end:
        n = min(per_graph, end - i)
        out.append((i, n))
        i += n
    return out


def steps_per_graph(step_s: float, cap: int) -> int:
    """Steps per graph: about GRAPH_TARGET_S of work, 1 .. cap."""
    return int(max(1, min(cap, round(GRAPH_TARGET_S / max(step_s, 1e-9)))))


def percentiles(samples):
    s = sorted(samples)
    if not s:
        return None

    def q(p):
        x = p * (len(s) - 1)
        lo = int(math.floor(x))
        hi = min(lo + 1, len(s) - 1)
        return s[lo] + (s[hi] - s[lo]) * (x - lo)
    return dict(p10=q(0.1), p50=q(0.5), p90=q(0.9))


def copy_calibration(nbytes):
    import torch
    n = int(nbytes) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}), flush=True)


def measured_copy_gbs(nbytes=1 << 30, reps=10):
    """HBM bandwidth of a plain device-to-device copy (bytes read + written per second)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return round(gbs, 1)


def workload(name):
    import synth
    if str(name).isdigit():
        return synth.WORKLOADS[int(name)]
    return synth.workload_by_name(name)


def algorithmic_bytes(w, prefix_lens):
    """Bytes each step must move, by kernel (each input read once, each output
    written once), and the attention's flops on dense packed tiles."""
    kv_elem = {"f32": 4, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    q_elem = {"f32": 4, "bf16": 2}[w.q_dtype]
    B, N = w.B, w.N
    tokens = int(sum(int(p) + N for p in prefix_lens))
    kv = tokens * w.Hkv * w.D * 2 * kv_elem
    q = B * N * w.Hq * w.D * q_elem
    attn = kv + 2 * q + 8 * B * N + 4 * B + 4 * B * N * w.Hq + (8 * w.Hkv if w.kv_dtype == "e4m3" else 0)
    argmax = B * N * w.V * 4 + 4 * B * N
    mask = 16 * B * N
    walk = 28 * B * N + 4 * B
    flops = 4 * w.D * w.Hq * N * tokens
    return dict(attention=attn, kv=kv, argmax=argmax, mask=mask, walk=walk,
                step=attn + argmax + mask + walk, attn_flops=flops, tokens=tokens)


def attention_bound(w):
    """The roof that bounds the attention: the bf16 matrix cores when its
    intensity (flop per K/V byte = g*N for bf16) is past the ridge, else HBM."""
    return "mfma" if (w.kv_dtype == "bf16" and w.group * w.N > BF16_RIDGE) else "hbm"


def kernel_source_sha():
    from tree_attention_verify_parent_amd.rocprof_summary import source_sha
    return source_sha(ROOT)


def measured_traffic(wname):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wname}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, one request per worker process

_CPU = {}


def _limit_blas():
    try:
        from threadpoolctl import threadpool_limits
        _CPU["limits"] = threadpool_limits(1)
    except Exception:
        pass


def _oracle_request(b):
    """One request of the oracle's verify step (forked worker; inputs from _CPU)."""
    import oracle
    d = _CPU
    w = d["w"]
    sl = slice(b, b + 1)
    t0 = time.perf_counter()
    oracle.verify_step(d["parents"][sl], d["draft"][sl], d["prefix"][sl], d["q"][sl], d["k"][sl], d["v"][sl],
                       d["logits"][b * w.N:(b + 1) * w.N], d["sm_scale"], q_fmt=w.q_dtype, kv_fmt=w.kv_dtype,
                       k_scale=d["k_scale"], v_scale=d["v_scale"], V=w.V)
    return time.perf_counter() - t0


def cpu_baseline(x, seconds, workers):
    """Oracle steps/s on a bounded sample: rounds of one request per worker
    (requests are independent in every part of the step) until the budget is
    spent or the batch is done, full steps repeated while time remains."""
    import multiprocessing as mp
    from tests.gpu_util import oracle_views
    w = x["workload"]
    qo, ko, vo = oracle_views(x)
    _CPU.update(w=w, parents=x["parents"], draft=x["draft_tokens"], prefix=x["prefix_lens"], q=qo, k=ko, v=vo,
                logits=x["logits"].numpy(), sm_scale=x["sm_scale"], k_scale=x["k_scale"], v_scale=x["v_scale"])
    host = os.cpu_count() or 1
    workers = int(workers) if workers else min(16, host)
    workers = max(1, min(workers, w.B))
    ctx = mp.get_context("fork")
    done_req, t_spent, steps_done = 0, 0.0, 0
    with ctx.Pool(workers, initializer=_limit_blas) as pool:
        t0 = time.perf_counter()
        while True:
            b0 = done_req % w.B
            batch = list(range(b0, min(w.B, b0 + workers)))
            pool.map(_oracle_request, batch, chunksize=1)
            done_req += len(batch)
            t_spent = time.perf_counter() - t0
            if done_req % w.B == 0:
                steps_done += 1
            if t_spent >= seconds:
                break
    _CPU.clear()
    value = (done_req / w.B) / t_spent
    return dict(value=round(value, 4), unit="steps/s", cores=workers, kind="oracle", host_cpus=host,
                sample=f"{done_req} requests of {w.name} ({done_req / w.B:.3g} steps of {w.B} requests), "
                       f"one request per worker process, {workers} processes x 1 BLAS thread, {t_spent:.1f} s")


# ---------------------------------------------------------------------------
# GPU measurement of one workload

class Timer:
    """HIP events on the current stream; elapsed milliseconds."""

    def __init__(self):
        import torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop_ms(self):
        import torch
        self.b.record()
        torch.cuda.synchronize()
        return self.a.elapsed_time(self.b)


def time_graph_calls(fn, R, calls, reps=5):
    """Average µs per call of `calls` back-to-back calls fn(replica) captured in
    one graph, replayed `reps` times after one untimed replay."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in range(calls):
            fn(c % R)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t = Timer()
    t.start()
    for _ in range(reps):
        g.replay()
    us = t.stop_ms() * 1e3 / (reps * calls)
    del g
    return us


def measure(w, x, args, steps, warmup, extras):
    """Steps/s of the whole verify step on workload w, and the attention's roofline."""
    import torch

    import synth
    import tree_attention_verify_parent_amd as st

    dev = torch.device("cuda:0")
    B, N = w.B, w.N
    bytes_ = algorithmic_bytes(w, x["prefix_lens"])

    # ---- inputs in HBM, replicated so the rotation exceeds the MALL
    per_replica = (x["q"].numel() * x["q"].element_size() + 2 * x["k_cache"].numel() * x["k_cache"].element_size()
                   + x["logits"].numel() * 4)
    free = torch.cuda.mem_get_info()[0]
    R = int(max(1, min(64, math.ceil(args.replica_bytes / per_replica), (0.4 * free) // per_replica)))
    parents = torch.from_numpy(x["parents"]).to(dev)
    draft = torch.from_numpy(x["draft_tokens"]).to(dev)
    prefix = torch.from_numpy(x["prefix_lens"]).to(dev)
    ks = None if x["k_scale"] is None else torch.from_numpy(x["k_scale"]).to(dev)
    vs = None if x["v_scale"] is None else torch.from_numpy(x["v_scale"]).to(dev)
    q0, k0, v0, l0 = (x["q"].to(dev), x["k_cache"].to(dev), x["v_cache"].to(dev), x["logits"].to(dev))
    qs, kcs, vcs, lgs = [q0], [k0], [v0], [l0]
    for _ in range(1, R):
        qs.append(q0.clone())
        kcs.append(k0.clone())
        vcs.append(v0.clone())
        lgs.append(l0.clone())

    outs = st.step_outputs(B, N, q0)
    anc, acc_len, path, err = outs["mask"], outs["accept_len"], outs["path_nodes"], outs["err"]
    ws = torch.zeros(max(st.attn_workspace_bytes(B, N, w.Hq, w.Hkv, w.D, w.S_max), 16), dtype=torch.uint8,
                     device=dev)                                        # zeroed once, reused
    step_ws = torch.zeros(max(st.verify_step_workspace_bytes(B, N, w.Hq, w.Hkv, w.D, w.S_max), 16),
                          dtype=torch.uint8, device=dev)
    out, lse = outs["out"], outs["lse"]

    def attention(r):
        st.tree_attn_verify(qs[r], kcs[r], vcs[r], prefix, anc, x["sm_scale"], k_scale=ks, v_scale=vs,
                            out=out, lse=lse, workspace=ws, err=err)

    def step(r):
        st.verify_step(parents, draft, prefix, qs[r], kcs[r], vcs[r], lgs[r], x["sm_scale"], k_scale=ks,
                       v_scale=vs, workspace=ws if args.unfused else step_ws, fused=not args.unfused, outs=outs)

    # eager warm-up over every replica (loads kernels), then the error word
    for r in range(R):
        step(r)
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise SystemExit(f"{w.name}: device error word 0x{int(err.item()):x}")
    # rough step time (eager, so at least the launch cost): sizes the graphs
    t0 = time.perf_counter()
    for r in range(2 * R):
        step(r % R)
    torch.cuda.synchronize()
    est = (time.perf_counter() - t0) / (2 * R)
    if steps is None:                                    # per-workload entry: steps from the time budget
        steps = int(max(20, min(20000, round(args.per_workload_seconds / est))))
        warmup = int(max(5, steps // 10))
    S = steps_per_graph(est, args.steps_per_graph)

    # graphs for every (first replica, length) block of the warm-up and the timed steps
    warm_blocks = graph_blocks(0, warmup, S)
    timed_blocks = graph_blocks(warmup, steps, S)
    graphs = {}
    if not args.no_graph:
        for i0, n in warm_blocks + timed_blocks:
            key = (i0 % R, n)
            if key in graphs:
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(n):
                    step((i0 + j) % R)
            graphs[key] = g
        torch.cuda.synchronize()

    def run_block(i0, n):
        if graphs:
            graphs[(i0 % R, n)].replay()
        else:
            for j in range(n):
                step((i0 + j) % R)

    for i0, n in warm_blocks:
        run_block(i0, n)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(timed_blocks) + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for k, (i0, n) in enumerate(timed_blocks):
        run_block(i0, n)
        evs[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step_us = [evs[k].elapsed_time(evs[k + 1]) * 1e3 / n for k, (_, n) in enumerate(timed_blocks)]
    pct = percentiles(per_step_us)
    ev_ms = evs[0].elapsed_time(evs[-1]) / steps
    if int(err.item()) != 0:
        raise SystemExit(f"{w.name}: device error word 0x{int(err.item()):x} after the timed steps")
    accept_mean = float(acc_len.float().mean().item())
    graphs.clear()

    # ---- dominant kernel: back-to-back attention calls, HIP events on the
    # stream that runs them
    calls = int(max(R, min(args.attn_calls, math.ceil(0.1 / max(est, 1e-6)))))
    attn_us = time_graph_calls(attention, R, calls)
    bound = attention_bound(w)
    if bound == "hbm":
        achieved = bytes_["attention"] / (attn_us * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4))
    else:
        achieved = bytes_["attn_flops"] / (attn_us * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4))
    roof["traffic"] = measured_traffic(w.name)
    roof["kernel"] = ("tree_attn_f32_kernel" if w.kv_dtype == "f32" else
                      "tree_attn_split_kernel (split-KV tree attention, split merge fused)")
    roof["launch_us"] = round(attn_us, 3)
    roof["bytes_per_launch"] = bytes_["attention"]
    roof["flops_per_launch"] = bytes_["attn_flops"]
    roof["hbm_gbs"] = round(bytes_["attention"] / (attn_us * 1e-6) / 1e9, 1)
    roof["hbm_frac"] = round(roof["hbm_gbs"] / PEAK_HBM_GBS, 4)
    roof["mfma_tflops"] = round(bytes_["attn_flops"] / (attn_us * 1e-6) / 1e12, 1)
    roof["calls_timed"] = calls

    res = dict(
        workload=w.name, steps=steps, warmup=warmup, steps_per_s=round(steps / wall, 2),
        ms_per_step=round(wall * 1e3 / steps, 5), ms_per_step_events=round(ev_ms, 5),
        step_us_p10=round(pct["p10"], 3), step_us_p50=round(pct["p50"], 3), step_us_p90=round(pct["p90"], 3),
        tree_tokens_per_s=round(steps / wall * B * N, 1),
        step_hbm_gbs=round(bytes_["step"] / (wall / steps) / 1e9, 1),
        step_bytes=bytes_["step"], accept_len_mean=round(accept_mean, 3),
        steps_per_graph=S if not args.no_graph else None, graphs=len(timed_blocks), replicas=R,
        step="unfused (4 calls)" if args.unfused else "spec_verify_step (1 launch)",
        attention=roof, wall_s=wall)

    if not extras:
        return res
    reps = 5

    # ---- the commit step after verification (keep the accepted path's K/V,
    # label outcomes): back-to-back calls on the accepted paths of the last
    # step, in place on the cache replicas (the rows it moves do not change its cost)
    newp = torch.empty(B, dtype=torch.int32, device=dev)
    labels = torch.empty((B, N), dtype=torch.int8, device=dev)
    commit_us = time_graph_calls(
        lambda r: st.commit_accepted(kcs[r], vcs[r], prefix, acc_len, path, new_prefix_lens=newp, labels=labels,
                                     err=err), R, calls, reps)
    kv_elem = {"f32": 4, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    moved = int(acc_len.sum().item()) * w.Hkv * w.D * kv_elem * 2 * 2      # K and V rows, read + write
    res["commit_step"] = dict(launch_us=round(commit_us, 3), bytes_per_launch=moved + B * N + 12 * B,
                              accept_len_sum=int(acc_len.sum().item()))

    # ---- the same attention over a paged cache: every replica's K/V scattered
    # into a shuffled pool of token-major pages, read through a block table
    ps = args.page_size
    while ps and -(-w.S_max // ps) > 2048:          # a block table holds at most 2048 pages per request
        ps *= 2
    if ps and w.kv_dtype != "f32":
        maxp = -(-w.S_max // ps)
        num_pages = B * maxp
        gen = torch.Generator().manual_seed(11)
        perm = torch.randperm(num_pages, generator=gen).view(B, maxp).to(torch.int32)
        table = perm.to(dev)
        flat = perm.view(-1).long().to(dev)

        def paginate(c):
            pad = torch.zeros(B, w.Hkv, maxp * ps, w.D, dtype=c.dtype, device=dev)
            pad[:, :, : w.S_max] = c
            blocks = pad.view(B, w.Hkv, maxp, ps, w.D).permute(0, 2, 3, 1, 4).reshape(B * maxp, ps, w.Hkv, w.D)
            pages = torch.empty_like(blocks)
            pages[flat] = blocks
            return pages

        kps = [paginate(kcs[r]) for r in range(R)]
        vps = [paginate(vcs[r]) for r in range(R)]
        ws_p = torch.zeros(max(st.attn_workspace_bytes(B, N, w.Hq, w.Hkv, w.D, maxp * ps), 16),
                           dtype=torch.uint8, device=dev)
        paged_us = time_graph_calls(
            lambda r: st.tree_attn_verify_paged(qs[r], kps[r], vps[r], prefix, anc, table, x["sm_scale"], k_scale=ks,
                                                v_scale=vs, out=out, lse=lse, workspace=ws_p, err=err),
            R, calls, reps)
        pbytes = bytes_["attention"] + B * maxp * 4
        paged = dict(page_size=ps, launch_us=round(paged_us, 3), achieved_gbs=round(pbytes / paged_us / 1e3, 1),
                     frac=round(pbytes / paged_us / 1e3 / PEAK_HBM_GBS, 4))
        ws_sp = torch.zeros(st.verify_step_workspace_bytes(B, N, w.Hq, w.Hkv, w.D, maxp * ps), dtype=torch.uint8,
                            device=dev)
        paged["step_us"] = round(time_graph_calls(
            lambda r: st.verify_step(parents, draft, prefix, qs[r], kps[r], vps[r], lgs[r], x["sm_scale"],
                                     k_scale=ks, v_scale=vs, block_table=table, workspace=ws_sp, outs=outs),
            R, calls, reps), 3)
        if int(err.item()) != 0:
            raise SystemExit(f"{w.name} paged step: device error word 0x{int(err.item()):x}")
        newp_p = torch.empty(B, dtype=torch.int32, device=dev)
        labels_p = torch.empty((B, N), dtype=torch.int8, device=dev)
        paged["commit_us"] = round(time_graph_calls(
            lambda r: st.commit_accepted(kps[r], vps[r], prefix, acc_len, path, block_table=table,
                                         new_prefix_lens=newp_p, labels=labels_p, err=err), R, calls, reps), 3)
        if int(err.item()) != 0:
            raise SystemExit(f"{w.name} paged commit: device error word 0x{int(err.item()):x}")
        res["paged_attention"] = paged
        del kps, vps

    # ---- e4m3 caches: the same attention in fp8 arithmetic (both products on
    # the fp8 matrix cores, q and p quantized in the kernel), and over an e2m1 cache
    if w.kv_dtype == "e4m3" and w.D == 128:
        f8_us = time_graph_calls(
            lambda r: st.tree_attn_verify_f8(qs[r], kcs[r], vcs[r], prefix, anc, x["sm_scale"], ks, vs, out=out,
                                             lse=lse, workspace=ws, err=err), R, calls, reps)
        f8 = dict(kernel="tree_attn_split_kernel (fp8 arithmetic)", launch_us=round(f8_us, 3),
                  achieved_gbs=round(bytes_["attention"] / f8_us / 1e3, 1),
                  hbm_frac=round(bytes_["attention"] / f8_us / 1e3 / PEAK_HBM_GBS, 4),
                  achieved_tflops=round(bytes_["attn_flops"] / f8_us / 1e6, 1),
                  fp8_mfma_frac=round(bytes_["attn_flops"] / f8_us / 1e6 / PEAK_FP8_TFLOPS, 4))
        x4 = synth.make_inputs(w.replace(kv_dtype="e2m1"), with_logits=False)
        k4, v4 = x4["k_cache"].to(dev), x4["v_cache"].to(dev)
        ks4, vs4 = torch.from_numpy(x4["k_scale"]).to(dev), torch.from_numpy(x4["v_scale"]).to(dev)
        R4 = int(max(1, min(64, math.ceil(args.replica_bytes / (2 * k4.numel())))))
        k4s = [k4] + [k4.clone() for _ in range(R4 - 1)]
        v4s = [v4] + [v4.clone() for _ in range(R4 - 1)]
        f4_us = time_graph_calls(
            lambda c: st.tree_attn_verify_f4(qs[c % R], k4s[c % R4], v4s[c % R4], prefix, anc, x["sm_scale"], ks4,
                                             vs4, out=out, lse=lse, workspace=ws, err=err), R * R4, calls, reps)
        b4 = bytes_["attention"] - bytes_["kv"] // 2             # K/V at half a byte per element
        f8["fp4_cache"] = dict(launch_us=round(f4_us, 3), achieved_gbs=round(b4 / f4_us / 1e3, 1),
                               hbm_frac=round(b4 / f4_us / 1e3 / PEAK_HBM_GBS, 4),
                               achieved_tflops=round(bytes_["attn_flops"] / f4_us / 1e6, 1))
        res["f8_attention"] = f8
        del k4s, v4s

    # ---- bf16 caches: the scores on the fp8 matrix cores (q per row and each
    # K tile rounded to e4m3 in the kernel, p and V in bf16); outside the
    # parity contract, like the fp8 arithmetic above
    if w.kv_dtype == "bf16" and w.D == 128:
        kq = torch.ones(w.Hkv, dtype=torch.float32, device=dev)
        s8_us = time_graph_calls(
            lambda r: st.tree_attn_verify_f8_scores(qs[r], kcs[r], vcs[r], prefix, anc, x["sm_scale"], kq, out=out,
                                                    lse=lse, workspace=ws, err=err), R, calls, reps)
        res["f8_scores"] = dict(kernel="tree_attn_split_kernel (fp8 scores over a bf16 cache)",
                                launch_us=round(s8_us, 3), achieved_tflops=round(bytes_["attn_flops"] / s8_us / 1e6, 1),
                                achieved_gbs=round(bytes_["attention"] / s8_us / 1e3, 1),
                                vs_bf16=round(attn_us / s8_us, 3))

    # ---- the attention's backward pass (training on the verified tree):
    # back-to-back calls over the replicas, each writing its own dK / dV.
    # Shapes the backward pass refuses (its status says so) are skipped.
    if w.kv_dtype in ("f32", "bf16"):
        gd = torch.Generator().manual_seed(12)
        d_out = torch.randn(q0.shape, generator=gd).to(q0.dtype).to(dev)
        attention(0)
        out_b, lse_b = out.clone(), lse.clone()
        dq_b = torch.empty_like(q0)
        dks = [torch.empty_like(k0) for _ in range(R)]
        dvs = [torch.empty_like(v0) for _ in range(R)]
        ws_b = torch.zeros(max(st.attn_backward_workspace_bytes(B, N, w.Hq, w.Hkv, w.D, w.S_max), 16),
                           dtype=torch.uint8, device=dev)

        def backward(r):
            st.tree_attn_backward(qs[r], kcs[r], vcs[r], prefix, anc, out_b, lse_b, d_out, x["sm_scale"], dq=dq_b,
                                  dk=dks[r], dv=dvs[r], workspace=ws_b, err=err)
        try:
            backward(0)
        except st.SpecError as e:
            res["backward"] = dict(skipped=str(e))
        else:
            torch.cuda.synchronize()
            bcalls = int(max(R, min(calls, math.ceil(0.1 / max(3 * attn_us * 1e-6, 1e-6)))))
            bwd_us = time_graph_calls(backward, R, bcalls, reps)
            q_bytes = q0.numel() * q0.element_size()
            # K, V read and dK, dV written once; q, out, dO read and dq written once
            bbytes = 2 * bytes_["kv"] + 4 * q_bytes + 4 * B * N * w.Hq + 8 * B * N + 4 * B
            # five products (S, dP, dV, dK, dq) against the forward pass's two
            bflops = bytes_["attn_flops"] * 5 // 2
            # more than 128 packed rows: row statistics, then the dq and dK / dV passes
            kname = ("bwd_rowstat_kernel + tree_attn_bwd_dq_kernel + tree_attn_bwd_dkdv_kernel"
                     if w.group * N > 128 else "tree_attn_bwd_kernel")
            res["backward"] = dict(kernel=kname, launch_us=round(bwd_us, 3),
                                   bytes_per_launch=bbytes, achieved_gbs=round(bbytes / bwd_us / 1e3, 1),
                                   frac=round(bbytes / bwd_us / 1e3 / PEAK_HBM_GBS, 4),
                                   mfma_tflops=round(bflops / bwd_us / 1e6, 1))
        del dks, dvs
    return res


def selected_workloads(spec, headline):
    import synth
    if spec == "none":
        return []
    if spec == "all":
        return list(synth.WORKLOADS)
    return [workload(s.strip()) for s in spec.split(",") if s.strip()]


def main(argv=None):
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the verify step is measured per GPU, and the library has no "
              "multi-GPU path (requests would shard across GPUs with no exchange).",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import synth
    t_start = time.perf_counter()
    head = workload(args.workload)
    print(f"[bench] generating {head.name}", file=sys.stderr, flush=True)
    xh = synth.make_inputs(head)

    # the oracle first, before anything touches the GPU (its pool forks)
    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] cpu_baseline on {head.name}", file=sys.stderr, flush=True)
        cpu = cpu_baseline(xh, args.cpu_baseline_seconds, args.cpu_workers)

    import torch
    import tree_attention_verify_parent_amd as st
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    st.lib()

    copy_gbs = measured_copy_gbs()
    print(f"[bench] {head.name}: {args.steps} timed steps after {args.warmup}", file=sys.stderr, flush=True)
    hres = measure(head, xh, args, args.steps, args.warmup, extras=not args.no_extras)
    del xh
    torch.cuda.empty_cache()

    per = {}
    for w in selected_workloads(args.workloads, head):
        if w.name == head.name:
            r = dict(hres)
        else:
            print(f"[bench] {w.name}", file=sys.stderr, flush=True)
            x = synth.make_inputs(w)
            r = measure(w, x, args, None, None, extras=not args.no_extras)
            del x
            torch.cuda.empty_cache()
        a = r["attention"]
        if a["bound"] == "hbm":
            a["frac_of_copy"] = round(a["hbm_gbs"] / copy_gbs, 4)
        r.pop("wall_s", None)
        per[w.name] = r

    roof = {k: hres["attention"][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                              "launch_us", "bytes_per_launch", "flops_per_launch", "hbm_gbs",
                                              "hbm_frac")}
    line = {
        "metric": METRIC,
        "value": hres["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": hres["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if head.kv_dtype == "f32" else ("bf16" if head.kv_dtype == "bf16" else "bf16+e4m3kv"),
        "data": "synthetic",
        "config": {"workload": head.name, "batch": head.B, "tree_nodes": head.N, "q_heads": head.Hq,
                   "kv_heads": head.Hkv, "head_dim": head.D, "prefix": [head.prefix_lo, head.prefix_hi],
                   "vocab": head.V, "step": hres["step"], "graph": not args.no_graph,
                   "steps_per_graph": hres["steps_per_graph"], "replicas": hres["replicas"]},
        "tree_tokens_per_s": hres["tree_tokens_per_s"],
        "step_us_p10": hres["step_us_p10"], "step_us_p50": hres["step_us_p50"], "step_us_p90": hres["step_us_p90"],
        "ms_per_step_events": hres["ms_per_step_events"],
        "step_hbm_gbs": hres["step_hbm_gbs"],
        "step_hbm_frac": round(hres["step_hbm_gbs"] / PEAK_HBM_GBS, 4),
        "accept_len_mean": hres["accept_len_mean"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "copy_gbs": copy_gbs,
        "per_workload": per,
        "bench_wall_s": round(time.perf_counter() - t_start, 1),
    }
    for k in ("commit_step", "paged_attention", "backward", "f8_attention", "f8_scores"):
        if k in hres:
            line[k] = hres[k]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
