"""Build libspectree.so in-tree with hipcc for gfx950.

    python -m tree_attention_verify_parent_amd.build [--debug-save-temps]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB = os.path.join(PKG_DIR, "libspectree.so")
SOURCES = ["tree_walk.hip", "argmax.hip", "tree_attn.hip", "commit.hip", "tree_attn_bwd.hip",
           "tree_attn_bwd_wide.hip", "step.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU ops are disabled for all device code: hipcc would otherwise
# form v_pk_{add,mul,fma}_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc_command(out: str = LIB, extra=()) -> list[str]:
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
            "-Wall", "-Wno-unused-function", *DEVICE_FLAGS,
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *extra,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libspectree.so")
    # drop the host pass's notice about the GPU-only target feature
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and noise not in ln]
    if msgs and verbose:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    extra = []
    if "--debug-save-temps" in sys.argv:
        extra.append("--save-temps")
    print(build(verbose=True, extra=extra))
