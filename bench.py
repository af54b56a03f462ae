#!/usr/bin/env python3
"""Verify-step throughput on one MI355X.

One step = the whole verify hot path for one batch of synthetic inputs that
are already resident in HBM: ancestor-mask build, tree-masked split-KV
attention, per-node vocabulary argmax, accept walk -- by default one
spec_verify_step call (one launch: the attention kernel's grid also holds
the mask, argmax and walk workgroups); --unfused times the four separate
calls instead.  The default workload is
the batch-8 lookahead-5 chain in bf16 (32 query heads over 8 KV heads,
head dim 128, 2048-token prefixes, 32000-token vocabulary).

Timing: W untimed warm-up steps, then K steps timed with torch.cuda
synchronisation on both sides.  Each step replays a HIP graph holding the
step's library calls for one of R input replicas; R is chosen so that the replicas
together exceed the GPU's last-level (MALL) cache, so every step streams its
K/V and logits from HBM.

The dominant kernel (the tree attention) is also timed on its own with HIP
events on the stream that runs it: a graph of back-to-back attention calls
over the replicas, elapsed time / number of calls.  Its algorithmic bytes
(each K/V byte of every request's prefix+tree once per KV head, Q, outputs,
masks) over that time give roofline.achieved.

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
METRIC = "tree-verify steps/sec and achieved HBM GB/s (% of peak) on 1 MI355X"
DEFAULT_WORKLOAD = "chain6_b8_h32x8_d128_p2048_bf16"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, help="workload name or index 0-4")
    ap.add_argument("--no-graph", action="store_true", help="launch each step's calls eagerly")
    ap.add_argument("--unfused", action="store_true",
                    help="time the four separate calls (mask, attention, argmax, walk) instead of spec_verify_step")
    ap.add_argument("--two-streams", action="store_true",
                    help="run argmax and accept walk on a second stream, concurrent with mask build "
                         "and attention (default: one stream)")
    ap.add_argument("--steps-per-graph", type=int, default=25,
                    help="verify steps captured in one HIP graph (amortises the graph launch)")
    ap.add_argument("--order", default="mask,attn,argmax,walk",
                    help="order of the four calls within a step on one stream")
    ap.add_argument("--replica-bytes", type=float, default=1.0e9,
                    help="total bytes of input replicas to rotate through (defeats the MALL)")
    ap.add_argument("--attn-calls", type=int, default=200, help="calls in the attention timing graph")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-commit", action="store_true", help="skip timing the commit step")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the attention's backward pass")
    ap.add_argument("--page-size", type=int, default=16,
                    help="also time the attention, the whole step (spec_verify_step_paged) and the commit "
                         "over a paged copy of the cache with this page size (0: skip)")
    ap.add_argument("--copy-calibration", type=float, default=0,
                    help="only run a plain float32 elementwise copy that reads and writes this many "
                         "bytes (5 launches) and exit: the reference point that scales the HBM byte "
                         "counters of a rocprofv3 --pmc pass")
    return ap.parse_args()


def copy_calibration(nbytes):
    import torch
    n = int(nbytes) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}), flush=True)


def workload(name):
    import synth
    if name.isdigit():
        return synth.WORKLOADS[int(name)]
    return synth.workload_by_name(name)


def algorithmic_bytes(w, prefix_lens):
    """Bytes each step must move, by kernel (each input read once, each output
    written once)."""
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


def cpu_baseline(x, seconds):
    """The CPU oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    from tests.gpu_util import oracle_views
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = 1
    w = x["workload"]
    qo, ko, vo = oracle_views(x)
    logits = x["logits"].numpy()
    B, N = w.B, w.N

    def run(nreq):
        sl = slice(0, nreq)
        oracle.verify_step(x["parents"][sl], x["draft_tokens"][sl], x["prefix_lens"][sl], qo[sl], ko[sl],
                           vo[sl], logits[: nreq * N], x["sm_scale"], q_fmt=w.q_dtype, kv_fmt=w.kv_dtype,
                           k_scale=x["k_scale"], v_scale=x["v_scale"], V=w.V)

    t0 = time.perf_counter()
    run(1)
    one = time.perf_counter() - t0
    if one * B <= seconds:
        reps, done, t0 = 0, 0.0, time.perf_counter()
        while done < seconds:
            run(B)
            reps += 1
            done = time.perf_counter() - t0
        return dict(value=reps / done, unit="steps/s", cores=int(cores), kind="oracle",
                    sample=f"{reps} full steps ({B} requests each), {done:.1f} s")
    nreq = max(1, min(B, int(seconds / max(one, 1e-9))))
    t0 = time.perf_counter()
    run(nreq)
    dt = time.perf_counter() - t0
    return dict(value=(nreq / B) / dt, unit="steps/s", cores=int(cores), kind="oracle",
                sample=f"{nreq} of {B} requests of one step ({dt:.1f} s), scaled to a full step")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the verify step is measured per GPU, and the library has no "
              "multi-GPU path (requests would shard across GPUs with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    import synth
    import tree_attention_verify_parent_amd as st

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    st.lib()
    dev = torch.device("cuda:0")
    w = workload(args.workload)
    x = synth.make_inputs(w)
    B, N = w.B, w.N
    bytes_ = algorithmic_bytes(w, x["prefix_lens"])

    # ---- inputs in HBM, replicated so the rotation exceeds the MALL
    per_replica = (x["q"].numel() * x["q"].element_size() + 2 * x["k_cache"].numel() * x["k_cache"].element_size()
                   + x["logits"].numel() * 4)
    free = torch.cuda.mem_get_info()[0]
    R = int(max(1, min(64, math.ceil(args.replica_bytes / per_replica), (0.5 * free) // per_replica)))
    parents = torch.from_numpy(x["parents"]).to(dev)
    draft = torch.from_numpy(x["draft_tokens"]).to(dev)
    prefix = torch.from_numpy(x["prefix_lens"]).to(dev)
    ks = None if x["k_scale"] is None else torch.from_numpy(x["k_scale"]).to(dev)
    vs = None if x["v_scale"] is None else torch.from_numpy(x["v_scale"]).to(dev)
    qs, kcs, vcs, lgs = [], [], [], []
    q0, k0, v0, l0 = (x["q"].to(dev), x["k_cache"].to(dev), x["v_cache"].to(dev), x["logits"].to(dev))
    for r in range(R):
        qs.append(q0 if r == 0 else q0.clone())
        kcs.append(k0 if r == 0 else k0.clone())
        vcs.append(v0 if r == 0 else v0.clone())
        lgs.append(l0 if r == 0 else l0.clone())

    anc = torch.empty((B, N), dtype=torch.int64, device=dev)
    depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    out = torch.empty_like(q0)
    lse = torch.empty((B, N, w.Hq), dtype=torch.float32, device=dev)
    amax = torch.empty(B * N, dtype=torch.int32, device=dev)
    acc_len = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    toks = torch.empty((B, N), dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws_bytes = st.attn_workspace_bytes(B, N, w.Hq, w.Hkv, w.D, w.S_max)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)   # zeroed once, reused
    step_ws = torch.zeros(st.verify_step_workspace_bytes(B, N, w.Hq, w.Hkv, w.D, w.S_max), dtype=torch.uint8,
                          device=dev)
    outs = dict(mask=anc, depth=depth, out=out, lse=lse, argmax=amax, accept_len=acc_len, path_nodes=path,
                out_tokens=toks, err=err)
    side = torch.cuda.Stream(device=dev) if args.two_streams else None
    ev_mask = torch.cuda.Event()

    def attention(r):
        st.tree_attn_verify(qs[r], kcs[r], vcs[r], prefix, anc, x["sm_scale"], k_scale=ks, v_scale=vs,
                            out=out, lse=lse, workspace=ws, err=err)

    order = args.order.split(",")
    assert sorted(order) == ["argmax", "attn", "mask", "walk"] and order.index("mask") < order.index("attn") \
        and order.index("mask") < order.index("walk") and order.index("argmax") < order.index("walk"), order

    def step(r):
        if not args.unfused:
            st.verify_step(parents, draft, prefix, qs[r], kcs[r], vcs[r], lgs[r], x["sm_scale"], k_scale=ks,
                           v_scale=vs, workspace=step_ws, outs=outs)
            return
        if side is None:
            for name in order:
                if name == "mask":
                    st.tree_mask_build(parents, anc_mask=anc, depth=depth, err=err)
                elif name == "attn":
                    attention(r)
                elif name == "argmax":
                    st.vocab_argmax(lgs[r], out=amax)
                else:
                    st.accept_walk(parents, anc, draft, amax.view(B, N), w.V, accept_len=acc_len,
                                   path_nodes=path, out_tokens=toks, err=err)
            return
        # two streams: mask -> attention on the main stream; argmax -> accept
        # walk (after the mask) on the side stream; joined at the end
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        st.tree_mask_build(parents, anc_mask=anc, depth=depth, err=err)
        ev_mask.record(main)
        with torch.cuda.stream(side):
            st.vocab_argmax(lgs[r], out=amax)
            side.wait_event(ev_mask)
            st.accept_walk(parents, anc, draft, amax.view(B, N), w.V, accept_len=acc_len, path_nodes=path,
                           out_tokens=toks, err=err)
        attention(r)
        main.wait_stream(side)

    # eager warm-up (loads kernels), then correctness sanity of the result
    for r in range(R):
        step(r)
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise SystemExit(f"device error word 0x{int(err.item()):x}")

    # each graph holds steps_per_graph consecutive steps (replicas rotate
    # inside it); a step is never split across graphs
    S = max(1, args.steps_per_graph)
    graphs = None
    if not args.no_graph:
        graphs = []
        for gi in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(S):
                    step((gi * S + j) % R)
            graphs.append(g)
        torch.cuda.synchronize()

    def run_steps(k, start=0):
        if graphs is not None:
            assert k % S == 0, "steps and warmup must be multiples of --steps-per-graph"
            for i in range(start // S, (start + k) // S):
                graphs[i % R].replay()
        else:
            for i in range(start, start + k):
                step(i % R)

    run_steps(args.warmup)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    run_steps(args.steps, args.warmup)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    steps_per_s = args.steps / wall

    # ---- dominant kernel: back-to-back attention calls, HIP events on the
    # stream that runs them
    calls = max(args.attn_calls, R)
    ag = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ag):
        for c in range(calls):
            attention(c % R)
    torch.cuda.synchronize()
    ag.replay()
    torch.cuda.synchronize()
    reps = 5
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(reps):
        ag.replay()
    a1.record()
    torch.cuda.synchronize()
    attn_us = a0.elapsed_time(a1) * 1e3 / (reps * calls)

    hbm_bound = not (w.kv_dtype == "bf16" and w.group * w.N > 312)
    if hbm_bound:
        achieved = bytes_["attention"] / (attn_us * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4))
    else:
        achieved = bytes_["attn_flops"] / (attn_us * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4))
    roof["traffic"] = measured_traffic(w.name)
    roof["kernel"] = "tree_attn_split_kernel (split-KV tree attention, split merge fused)"
    roof["launch_us"] = round(attn_us, 3)
    roof["bytes_per_launch"] = bytes_["attention"]

    # ---- the commit step after verification (keep the accepted path's K/V,
    # label outcomes): a graph of back-to-back calls on the accepted paths of
    # the warm-up step, in place on the cache replicas (the rows it moves do
    # not change its cost)
    commit = None
    if not args.no_commit:
        newp = torch.empty(B, dtype=torch.int32, device=dev)
        labels = torch.empty((B, N), dtype=torch.int8, device=dev)
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            for c in range(calls):
                st.commit_accepted(kcs[c % R], vcs[c % R], prefix, acc_len, path, new_prefix_lens=newp,
                                   labels=labels, err=err)
        torch.cuda.synchronize()
        cg.replay()
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(reps):
            cg.replay()
        c1.record()
        torch.cuda.synchronize()
        commit_us = c0.elapsed_time(c1) * 1e3 / (reps * calls)
        kv_elem = {"f32": 4, "bf16": 2, "e4m3": 1}[w.kv_dtype]
        moved = int(acc_len.sum().item()) * w.Hkv * w.D * kv_elem * 2 * 2      # K and V rows, read + write
        commit = dict(launch_us=round(commit_us, 3), bytes_per_launch=moved + B * N + 12 * B,
                      accept_len_sum=int(acc_len.sum().item()))

    # ---- the same attention over a paged cache: every replica's K/V scattered
    # into a shuffled pool of token-major pages, read through a block table
    paged = None
    ps = args.page_size
    # no fp32 paged path; a block table holds at most 2048 pages per request
    if ps and w.kv_dtype != "f32" and -(-w.S_max // ps) <= 2048:
        maxp = -(-w.S_max // ps)
        num_pages = B * maxp
        g = torch.Generator().manual_seed(11)
        perm = torch.randperm(num_pages, generator=g).view(B, maxp).to(torch.int32)
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
        pg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pg):
            for c in range(calls):
                st.tree_attn_verify_paged(qs[c % R], kps[c % R], vps[c % R], prefix, anc, table, x["sm_scale"],
                                          k_scale=ks, v_scale=vs, out=out, lse=lse, workspace=ws_p, err=err)
        torch.cuda.synchronize()
        pg.replay()
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        for _ in range(reps):
            pg.replay()
        p1.record()
        torch.cuda.synchronize()
        paged_us = p0.elapsed_time(p1) * 1e3 / (reps * calls)
        pbytes = bytes_["attention"] + B * maxp * 4
        paged = dict(page_size=ps, launch_us=round(paged_us, 3), achieved_gbs=round(pbytes / paged_us / 1e3, 1),
                     frac=round(pbytes / paged_us / 1e3 / PEAK_HBM_GBS, 4))
        # the whole step over the pages (spec_verify_step_paged, one launch)
        ws_sp = torch.zeros(st.verify_step_workspace_bytes(B, N, w.Hq, w.Hkv, w.D, maxp * ps), dtype=torch.uint8,
                            device=dev)
        sg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sg):
            for c in range(calls):
                st.verify_step(parents, draft, prefix, qs[c % R], kps[c % R], vps[c % R], lgs[c % R], x["sm_scale"],
                               k_scale=ks, v_scale=vs, block_table=table, workspace=ws_sp, outs=outs)
        torch.cuda.synchronize()
        sg.replay()
        torch.cuda.synchronize()
        if int(err.item()) != 0:
            raise SystemExit(f"paged step: device error word 0x{int(err.item()):x}")
        p0.record()
        for _ in range(reps):
            sg.replay()
        p1.record()
        torch.cuda.synchronize()
        paged["step_us"] = round(p0.elapsed_time(p1) * 1e3 / (reps * calls), 3)
        # the commit over the pages (spec_commit_accepted_paged), on the accepted
        # paths of the last step, in place (the rows it moves do not change its cost)
        newp_p = torch.empty(B, dtype=torch.int32, device=dev)
        labels_p = torch.empty((B, N), dtype=torch.int8, device=dev)
        cg_p = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg_p):
            for c in range(calls):
                st.commit_accepted(kps[c % R], vps[c % R], prefix, acc_len, path, block_table=table,
                                   new_prefix_lens=newp_p, labels=labels_p, err=err)
        torch.cuda.synchronize()
        cg_p.replay()
        torch.cuda.synchronize()
        if int(err.item()) != 0:
            raise SystemExit(f"paged commit: device error word 0x{int(err.item()):x}")
        p0.record()
        for _ in range(reps):
            cg_p.replay()
        p1.record()
        torch.cuda.synchronize()
        paged["commit_us"] = round(p0.elapsed_time(p1) * 1e3 / (reps * calls), 3)
        del kps, vps, sg, cg_p

    # ---- e4m3 caches: the same attention in fp8 arithmetic (both products on
    # the fp8 matrix cores, q and p quantized in the kernel)
    f8 = None
    if w.kv_dtype == "e4m3" and w.D == 128:
        fg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(fg):
            for c in range(calls):
                st.tree_attn_verify_f8(qs[c % R], kcs[c % R], vcs[c % R], prefix, anc, x["sm_scale"], ks, vs,
                                       out=out, lse=lse, workspace=ws, err=err)
        torch.cuda.synchronize()
        fg.replay()
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(reps):
            fg.replay()
        f1.record()
        torch.cuda.synchronize()
        f8_us = f0.elapsed_time(f1) * 1e3 / (reps * calls)
        f8 = dict(kernel="tree_attn_split_kernel (fp8 arithmetic)", launch_us=round(f8_us, 3),
                  achieved_gbs=round(bytes_["attention"] / f8_us / 1e3, 1),
                  hbm_frac=round(bytes_["attention"] / f8_us / 1e3 / PEAK_HBM_GBS, 4),
                  achieved_tflops=round(bytes_["attn_flops"] / f8_us / 1e6, 1),
                  fp8_mfma_frac=round(bytes_["attn_flops"] / f8_us / 1e6 / PEAK_FP8_TFLOPS, 4))
        # the same shapes over an e2m1 (FP4) cache: half the K/V bytes
        x4 = synth.make_inputs(w.replace(kv_dtype="e2m1"), with_logits=False)
        k4, v4 = x4["k_cache"].to(dev), x4["v_cache"].to(dev)
        ks4, vs4 = torch.from_numpy(x4["k_scale"]).to(dev), torch.from_numpy(x4["v_scale"]).to(dev)
        R4 = int(max(1, min(64, math.ceil(args.replica_bytes / (2 * k4.numel())))))
        k4s = [k4] + [k4.clone() for _ in range(R4 - 1)]
        v4s = [v4] + [v4.clone() for _ in range(R4 - 1)]
        g4 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g4):
            for c in range(calls):
                st.tree_attn_verify_f4(qs[c % R], k4s[c % R4], v4s[c % R4], prefix, anc, x["sm_scale"], ks4, vs4,
                                       out=out, lse=lse, workspace=ws, err=err)
        torch.cuda.synchronize()
        g4.replay()
        torch.cuda.synchronize()
        f0.record()
        for _ in range(reps):
            g4.replay()
        f1.record()
        torch.cuda.synchronize()
        f4_us = f0.elapsed_time(f1) * 1e3 / (reps * calls)
        b4 = bytes_["attention"] - bytes_["kv"] // 2             # K/V at half a byte per element
        f8["fp4_cache"] = dict(launch_us=round(f4_us, 3), achieved_gbs=round(b4 / f4_us / 1e3, 1),
                               hbm_frac=round(b4 / f4_us / 1e3 / PEAK_HBM_GBS, 4),
                               achieved_tflops=round(bytes_["attn_flops"] / f4_us / 1e6, 1))
        del k4s, v4s

    # ---- the attention's backward pass (training on the verified tree):
    # back-to-back calls over the replicas, each writing its own dK / dV
    backward = None
    if not args.no_backward and w.kv_dtype in ("f32", "bf16") and w.group * N <= 128:
        gd = torch.Generator().manual_seed(12)
        d_out = torch.randn(q0.shape, generator=gd).to(q0.dtype).to(dev)
        out_b = out.clone()
        lse_b = lse.clone()
        dq_b = torch.empty_like(q0)
        dks = [torch.empty_like(k0) for _ in range(R)]
        dvs = [torch.empty_like(v0) for _ in range(R)]
        ws_b = torch.zeros(max(st.attn_backward_workspace_bytes(B, N, w.Hq, w.Hkv, w.D, w.S_max), 16),
                           dtype=torch.uint8, device=dev)
        bg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(bg):
            for c in range(calls):
                st.tree_attn_backward(qs[c % R], kcs[c % R], vcs[c % R], prefix, anc, out_b, lse_b, d_out,
                                      x["sm_scale"], dq=dq_b, dk=dks[c % R], dv=dvs[c % R], workspace=ws_b,
                                      err=err)
        torch.cuda.synchronize()
        bg.replay()
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(reps):
            bg.replay()
        b1.record()
        torch.cuda.synchronize()
        bwd_us = b0.elapsed_time(b1) * 1e3 / (reps * calls)
        q_bytes = q0.numel() * q0.element_size()
        # K, V read and dK, dV written once; q, out, dO read and dq written once
        bbytes = 2 * bytes_["kv"] + 4 * q_bytes + 4 * B * N * w.Hq + 8 * B * N + 4 * B
        backward = dict(kernel="tree_attn_bwd_kernel", launch_us=round(bwd_us, 3), bytes_per_launch=bbytes,
                        achieved_gbs=round(bbytes / bwd_us / 1e3, 1),
                        frac=round(bbytes / bwd_us / 1e3 / PEAK_HBM_GBS, 4))
        del dks, dvs

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, args.cpu_baseline_seconds)

    line = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.kv_dtype == "f32" else ("bf16" if w.kv_dtype == "bf16" else "bf16+e4m3kv"),
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "tree_nodes": N, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "prefix": [w.prefix_lo, w.prefix_hi], "vocab": w.V,
                   "graph": graphs is not None, "steps_per_graph": S if graphs is not None else None,
                   "step": "unfused (4 calls)" if args.unfused else "spec_verify_step (1 launch)",
                   "two_streams": side is not None and args.unfused,
                   "order": args.order if args.unfused else None, "replicas": R},
        "tree_tokens_per_s": round(steps_per_s * B * N, 1),
        "step_hbm_gbs": round(bytes_["step"] / (ms_per_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(bytes_["step"] / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "ms_per_step_events": round(ev_ms, 5),
        "accept_len_mean": round(float(acc_len.float().mean().item()), 3),
        "roofline": roof,
        "cpu_baseline": cpu,
        "commit_step": commit,
        "paged_attention": paged,
        "backward": backward,
        "f8_attention": f8,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
