"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every library source with the sanitizers on the host side only (the
GPU code objects are compiled as usual; no GPU is needed, since nothing is
launched) together with tests/sanitize/host_checks.cpp, then runs the driver:
it sweeps the size functions over normal and extreme shapes and sends every
entry point null, misaligned, mis-typed and mis-sized arguments, checking the
status each must return.  Any memory error or undefined behaviour aborts the
run.  CPU only; about a minute and a half, most of it compiling."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_attention_verify_parent_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["tree_walk.hip", "argmax.hip", "tree_attn.hip", "commit.hip", "tree_attn_bwd.hip",
           "tree_attn_bwd_wide.hip", "step.hip"]
# sanitizers on the host pass only: each -fsanitize flag right after -Xarch_host
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SANITIZE,
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    def compile_one(src_out):
        src, out, extra = src_out
        r = subprocess.run([HIPCC, *FLAGS, *extra, "-c", src, "-o", out], capture_output=True, text=True,
                           timeout=900)
        return src, r.returncode, r.stderr[-2000:]

    jobs = [(os.path.join(CSRC, s), str(tmp_path / (s + ".o")), []) for s in SOURCES]
    jobs.append((os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), str(tmp_path / "host_checks.o"),
                 ["-x", "hip"]))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 8)) as ex:
        for src, rc, err in ex.map(compile_one, jobs):
            assert rc == 0, f"{src}: {err}"
    exe = str(tmp_path / "host_checks")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SANITIZE[:4], *[j[1] for j in jobs], "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "host checks OK" in r.stdout, r.stdout + r.stderr
    shutil.rmtree(tmp_path, ignore_errors=True)
