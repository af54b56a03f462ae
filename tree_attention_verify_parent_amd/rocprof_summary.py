"""Summarise rocprofv3 result databases into short text tables.

    python -m tree_attention_verify_parent_amd.rocprof_summary stats DIR [--cmd "..."] [--by-grid] [--by-segment N]
        per-kernel call count and average / min / max duration (kernel trace);
        --by-grid keeps launches of one kernel with different grids apart
        (the verify step's one-launch attention has a larger grid than the
        attention alone); --by-segment N also keeps apart runs of consecutive
        launches of one (kernel, grid) that other kernels interrupt, numbered
        #1, #2, ... in launch order, and lists runs of at least N launches
        (two workloads can launch the same kernel with the same grid)
    python -m tree_attention_verify_parent_amd.rocprof_summary pmc DIR [--cmd "..."]
        per-kernel average of every collected counter (one --pmc pass)
    python -m tree_attention_verify_parent_amd.rocprof_summary traffic \\
            FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR --kernel NAME --copy-bytes BYTES --out JSON
        HBM bytes per launch of NAME from a FETCH_SIZE pass and a WRITE_SIZE pass,
        each scaled by what the same counter reads for a plain elementwise copy
        that reads and writes BYTES bytes (bench.py --copy-calibration BYTES,
        profiled with the same counter).

DIR is a rocprofv3 output directory (-d); every *_results.db below it is read.
"""
from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import re
import sqlite3
import sys

SHORT = ("tree_attn_split_kernel", "tree_attn_f32_kernel", "vocab_argmax_kernel", "accept_walk_kernel",
         "tree_mask_build_kernel", "commit_accepted_kernel", "tree_attn_bwd_kernel", "tree_attn_bwd_f32_kernel",
         "tree_attn_bwd_dq_kernel", "tree_attn_bwd_dkdv_kernel", "bwd_rowstat_kernel")


def _mangled_args(tail: str) -> str:
    """Template arguments of an Itanium-mangled name made of integer and bool
    literals only (``ILi128ELb0EE`` -> ``<128,false>``); '' otherwise."""
    m = re.match(r"I((?:L[a-z]-?\d+E)+)E", tail)
    if not m:
        return ""
    vals = []
    for kind, v in re.findall(r"L([a-z])(-?\d+)E", m.group(1)):
        vals.append(("true" if v != "0" else "false") if kind == "b" else v)
    return "<" + ",".join(vals) + ">"


def short_name(name: str) -> str:
    """Kernel name without namespace and argument list, template arguments kept
    (demangled names from the trace, or mangled ones from the counter runs)."""
    for k in sorted(SHORT, key=len, reverse=True):
        if k in name:
            tpl = name.split(k, 1)[1]
            if tpl.startswith("<"):
                return k + tpl[:tpl.find("(")]
            return k + _mangled_args(tpl)
    if "elementwise" in name.lower():
        return "elementwise:" + name[:56]
    return name[:70]


def dbs(d):
    out = sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True))
    if not out:
        raise SystemExit(f"no *_results.db under {d}")
    return out


def kernel_stats(d, by_grid=False, by_segment=0):
    launches = []
    for db in dbs(d):
        c = sqlite3.connect(db)
        for name, start, end, gx, wx in c.execute("select name, start, end, grid_x, workgroup_x from kernels"):
            key = short_name(name)
            if by_grid or by_segment:
                key += f" [{gx // max(wx, 1)} wg]"
            launches.append((start, end, key))
    launches.sort()
    agg = collections.defaultdict(list)
    if not by_segment:
        for start, end, key in launches:
            agg[key].append((end - start) / 1e3)
        return agg
    runs = collections.Counter()
    prev = None
    for start, end, key in launches:
        if key != prev:
            runs[key] += 1
            prev = key
        agg[f"#{runs[key]} {key}"].append((end - start) / 1e3)
    return {k: v for k, v in agg.items() if len(v) >= by_segment}


def pmc(d):
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for db in dbs(d):
        c = sqlite3.connect(db)
        cols = [r[1] for r in c.execute("pragma table_info(counters_collection)")]
        ci = {n: i for i, n in enumerate(cols)}
        kname = "kernel_name" if "kernel_name" in ci else "name"
        for r in c.execute("select * from counters_collection"):
            agg[short_name(r[ci[kname]])][r[ci["counter_name"]]].append(float(r[ci["value"]]))
    return agg


ATTENTION_SOURCES = ("common.h", "gfx950.h", "tree_attn.hip", "host_api.h", "step_ops.h", "argmax_ops.h",
                     "tree_ops.h")


def source_sha(root):
    """Digest of the attention kernel's sources: counter runs stay valid while
    these are unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(root, "tree_attention_verify_parent_amd", "csrc")
    for f in ATTENTION_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["stats", "pmc", "traffic"])
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--kernel", default="tree_attn_split_kernel")
    ap.add_argument("--copy-bytes", type=float, default=0)
    ap.add_argument("--out", default="")
    ap.add_argument("--by-grid", action="store_true")
    ap.add_argument("--by-segment", type=int, default=0)
    a = ap.parse_args(argv)
    if a.cmd:
        print(f"command: {a.cmd}")
    if a.mode == "stats":
        agg = kernel_stats(a.dirs[0], a.by_grid, a.by_segment)
        tot = sum(sum(v) for v in agg.values())
        w = 72 if a.by_segment else 58
        print(f"{'kernel':{w}s} {'calls':>7s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}")
        # segments in launch order (of their first launch), kernels by total time
        items = list(agg.items()) if a.by_segment else sorted(agg.items(), key=lambda kv: -sum(kv[1]))
        for k, v in items:
            print(f"{k[:w]:{w}s} {len(v):7d} {sum(v)/len(v):9.3f} {min(v):9.3f} {max(v):9.3f} {100*sum(v)/tot:6.1f}")
    elif a.mode == "pmc":
        agg = pmc(a.dirs[0])
        for k, ctrs in sorted(agg.items()):
            n = max(len(v) for v in ctrs.values())
            vals = ", ".join(f"{c}={sum(v)/len(v):.4g}" for c, v in sorted(ctrs.items()))
            print(f"{k} ({n} dispatches): {vals}")
    else:
        if len(a.dirs) != 4:
            raise SystemExit("traffic needs FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR")
        fetch, write, cfetch, cwrite = (pmc(d) for d in a.dirs)

        def avg(agg, kern, ctr):
            # the exact name (template arguments included), else the one kernel it prefixes
            hits = [k for k, ctrs in agg.items() if ctr in ctrs and (k == kern or k.startswith(kern + "<"))]
            if kern in hits:
                hits = [kern]
            if len(hits) != 1:
                raise SystemExit(f"{ctr} for {kern}: {'none' if not hits else 'ambiguous: ' + ', '.join(hits)}")
            v = agg[hits[0]][ctr]
            return sum(v) / len(v)

        def copy_avg(agg, ctr):
            best = None
            for k, ctrs in agg.items():
                if k.startswith("elementwise:") and ctr in ctrs:
                    v = sum(ctrs[ctr]) / len(ctrs[ctr])
                    best = v if best is None else max(best, v)
            if best is None:
                raise SystemExit(f"no copy kernel with {ctr}")
            return best

        kf, kw = avg(fetch, a.kernel, "FETCH_SIZE"), avg(write, a.kernel, "WRITE_SIZE")
        cf, cw = copy_avg(cfetch, "FETCH_SIZE"), copy_avg(cwrite, "WRITE_SIZE")
        # the copy reads and writes copy_bytes each: bytes per counter unit
        f_scale, w_scale = a.copy_bytes / cf, a.copy_bytes / cw
        res = dict(kernel=a.kernel, fetch_counter=kf, write_counter=kw, copy_fetch_counter=cf,
                   copy_write_counter=cw, copy_bytes=a.copy_bytes, fetch_scale=f_scale, write_scale=w_scale,
                   fetch_bytes=kf * f_scale, write_bytes=kw * w_scale,
                   bytes_per_launch=kf * f_scale + kw * w_scale,
                   kernel_source_sha=source_sha(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))),
                   command=a.cmd)
        print(json.dumps(res, indent=1))
        if a.out:
            with open(a.out, "w") as f:
                json.dump(res, f, indent=1)


if __name__ == "__main__":
    sys.exit(main())
