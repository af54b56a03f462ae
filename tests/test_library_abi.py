"""The C-ABI library loads and exports every symbol that include/spectree.h
declares; host-side argument checks reject bad calls before any launch.
CPU only: no call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import tree_attention_verify_parent_amd as st

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "spectree.h")

(SPEC_OK, SPEC_ERR_NULL, SPEC_ERR_SHAPE, SPEC_ERR_DTYPE, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP, SPEC_ERR_ALIGN,
 SPEC_ERR_SCRATCH) = range(8)
FAKE = ctypes.c_void_p(0x1000)        # never dereferenced: every call below fails host checks first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(st.library_path):
        pytest.skip("libspectree.so not built")
    return st.lib()


def test_header_declares_the_four_steps():
    names = declared_functions()
    for n in ("spec_tree_mask_build", "spec_tree_attn_verify", "spec_vocab_argmax", "spec_accept_walk",
              "spec_tree_attn_workspace_bytes", "spec_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n
    assert sorted(st.EXPORTS) == sorted(declared_functions())


def test_status_strings(L):
    for s in range(8):
        assert L.spec_status_string(s).decode().startswith("SPEC_")
    assert b"unknown" in L.spec_status_string(99)


def test_workspace_bytes_is_pure_and_rejects_bad_shapes(L):
    f = L.spec_tree_attn_workspace_bytes
    assert f(8, 6, 32, 8, 128, 2054) == f(8, 6, 32, 8, 128, 2054) > 0
    # two partial slots of M_pad x (D + 2) floats per unit, one counter per (request, kv head, M-tile):
    # 256 units of one 32-row tile for M = 24; 512 units of one 128-row tile for M = 128
    assert f(8, 6, 32, 8, 128, 2054) == 2 * 256 * 32 * (128 * 4 + 8) + 8 * 8 * 4
    assert f(64, 16, 64, 8, 128, 4112) == 2 * 512 * 128 * (128 * 4 + 8) + 64 * 8 * 4
    # M = 960 (an even number of 128-row tiles): one 8-wave workgroup a CU over 256-row tiles, so 4 M-tiles,
    # 64 units of one split each, slots for 2 per unit
    assert f(16, 60, 64, 4, 128, 32828) == 2 * 64 * 1024 * (128 * 4 + 8) + 64 * 4 * 4
    # M = 376 (three 128-row tiles, which 256-row tiles would pad to 512): the 4-wave plan, 512 // 3 units
    # of 3 splits (a sequence of 33 tiles), two slots per unit
    assert f(8, 47, 64, 8, 128, 2054) == 2 * (512 // 3) * 384 * (128 * 4 + 8) + 64 * 3 * 4
    # M = 256 with D = 64: 128-row tiles (two M-tiles, so two counters per sequence), 512 slots / 2 = 256 units
    assert f(2, 32, 64, 8, 64, 1000) == 2 * 256 * 256 * (64 * 4 + 8) + 16 * 2 * 4
    assert f(1024, 6, 32, 8, 128, 2 ** 21 - 1) > 0
    for bad in [(0, 6, 32, 8, 128, 2054), (8, 0, 32, 8, 128, 2054), (8, 65, 32, 8, 128, 2054),
                (8, 6, 30, 8, 128, 2054), (8, 6, 32, 8, 96, 2054), (8, 6, 32, 8, 128, 5),
                (1025, 6, 32, 8, 128, 2054), (1024, 6, 32, 8, 128, 2 ** 21),
                (1, 6, 1024, 1024, 128, 2 ** 21)]:
        assert f(*bad) == 0, bad


def test_mask_build_host_checks(L):
    assert L.spec_tree_mask_build(None, 1, 6, FAKE, None, None, None) == SPEC_ERR_NULL
    assert L.spec_tree_mask_build(FAKE, 1, 6, None, None, None, None) == SPEC_ERR_NULL
    assert L.spec_tree_mask_build(FAKE, 0, 6, FAKE, None, None, None) == SPEC_ERR_SHAPE
    assert L.spec_tree_mask_build(FAKE, 1, 0, FAKE, None, None, None) == SPEC_ERR_SHAPE
    assert L.spec_tree_mask_build(FAKE, 1, 65, FAKE, None, None, None) == SPEC_ERR_SHAPE


def test_accept_walk_host_checks(L):
    args = [FAKE] * 4
    outs = [FAKE] * 3
    assert L.spec_accept_walk(None, *args[1:], 1, 6, 10, *outs, None, None) == SPEC_ERR_NULL
    assert L.spec_accept_walk(*args, 1, 6, 10, None, FAKE, FAKE, None, None) == SPEC_ERR_NULL
    assert L.spec_accept_walk(*args, 1, 65, 10, *outs, None, None) == SPEC_ERR_SHAPE
    assert L.spec_accept_walk(*args, 1, 6, 0, *outs, None, None) == SPEC_ERR_SHAPE


def test_argmax_host_checks(L):
    assert L.spec_vocab_argmax(None, 4, 10, 10, FAKE, None) == SPEC_ERR_NULL
    assert L.spec_vocab_argmax(FAKE, 0, 10, 10, FAKE, None) == SPEC_ERR_SHAPE
    assert L.spec_vocab_argmax(FAKE, 4, 10, 9, FAKE, None) == SPEC_ERR_SHAPE
    assert L.spec_vocab_argmax(FAKE, 4, 0, 10, FAKE, None) == SPEC_ERR_SHAPE


def _attn(L, q=FAKE, qd=1, k=FAKE, v=FAKE, kvd=1, ks=None, vs=None, shape=(8, 6, 32, 8, 128, 2054),
          out=FAKE, ws=None, wsb=0, scale=0.088):
    return L.spec_tree_attn_verify(q, qd, k, v, kvd, ks, vs, FAKE, FAKE, *shape, scale, out, None, ws,
                                   wsb, None, None)


def test_attention_host_checks(L):
    assert _attn(L, q=None) == SPEC_ERR_NULL
    assert _attn(L, out=None) == SPEC_ERR_NULL
    assert _attn(L, qd=0, kvd=1) == SPEC_ERR_DTYPE                  # f32 q with bf16 kv
    assert _attn(L, qd=2, kvd=2) == SPEC_ERR_DTYPE                  # fp8 q
    assert _attn(L, qd=1, kvd=2) == SPEC_ERR_NULL                   # fp8 kv needs scales
    assert _attn(L, shape=(8, 6, 30, 8, 128, 2054)) == SPEC_ERR_SHAPE    # Hq % Hkv
    assert _attn(L, shape=(8, 6, 32, 8, 96, 2054)) == SPEC_ERR_SHAPE     # D
    assert _attn(L, shape=(8, 65, 32, 8, 128, 2054)) == SPEC_ERR_SHAPE   # N
    assert _attn(L, shape=(1025, 6, 32, 8, 128, 2054)) == SPEC_ERR_SHAPE  # B beyond the length table
    assert _attn(L, scale=0.0) == SPEC_ERR_SHAPE                    # the softmax scale must be positive
    assert _attn(L, scale=float("nan")) == SPEC_ERR_SHAPE
    assert _attn(L, shape=(1024, 6, 32, 8, 128, 2 ** 21)) == SPEC_ERR_SHAPE  # B * S_max reaches 2^31
    assert _attn(L, shape=(8, 6, 32, 8, 128, 5)) == SPEC_ERR_SHAPE       # S_max < N
    assert _attn(L, q=ctypes.c_void_p(0x1004)) == SPEC_ERR_ALIGN
    assert _attn(L) == SPEC_ERR_WORKSPACE                            # split path needs scratch
    need = L.spec_tree_attn_workspace_bytes(8, 6, 32, 8, 128, 2054)
    assert _attn(L, ws=FAKE, wsb=need - 1) == SPEC_ERR_WORKSPACE


def test_f8_scores_host_checks(L):
    def f(q=FAKE, shape=(8, 6, 32, 8, 128, 2054), scale=0.088, ws=None, wsb=0):
        return L.spec_tree_attn_verify_f8_scores(q, FAKE, FAKE, None, FAKE, FAKE, *shape, scale, FAKE, None, ws, wsb,
                                                 None, None)
    assert f(q=None) == SPEC_ERR_NULL
    assert f(shape=(8, 6, 32, 8, 64, 2054)) == SPEC_ERR_SHAPE      # D = 128 only
    assert f(shape=(8, 65, 32, 8, 128, 2054)) == SPEC_ERR_SHAPE
    assert f(scale=-1.0) == SPEC_ERR_SHAPE
    assert f(q=ctypes.c_void_p(0x1004)) == SPEC_ERR_ALIGN
    assert f() == SPEC_ERR_WORKSPACE
    need = L.spec_tree_attn_workspace_bytes(8, 6, 32, 8, 128, 2054)
    assert f(ws=FAKE, wsb=need - 1) == SPEC_ERR_WORKSPACE


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(st.SpecError):
        st.tree_mask_build(torch.zeros((1, 6), dtype=torch.int32))


def test_commit_host_checks(L):
    def commit(k=FAKE, v=FAKE, dt=1, shape=(4, 6, 8, 128, 2054), newp=FAKE):
        return L.spec_commit_accepted(k, v, dt, FAKE, FAKE, FAKE, *shape, newp, None, None, None)
    assert commit(k=None) == SPEC_ERR_NULL
    assert commit(newp=None) == SPEC_ERR_NULL
    assert commit(dt=7) == SPEC_ERR_DTYPE
    assert commit(shape=(4, 65, 8, 128, 2054)) == SPEC_ERR_SHAPE
    assert commit(shape=(4, 6, 8, 96, 2054)) == SPEC_ERR_SHAPE
    assert commit(shape=(0, 6, 8, 128, 2054)) == SPEC_ERR_SHAPE
    assert commit(shape=(4, 6, 8, 128, 5)) == SPEC_ERR_SHAPE


def test_paged_attention_host_checks(L):
    def paged(table=FAKE, qd=1, kvd=1, max_pages=40, page_size=16, num_pages=100, shape=(4, 6, 32, 8, 128),
              scale=0.088):
        return L.spec_tree_attn_verify_paged(FAKE, qd, FAKE, FAKE, kvd, None, None, FAKE, FAKE, table, max_pages,
                                             page_size, num_pages, *shape, scale, FAKE, None, None, 0, None, None)
    assert paged(table=None) == SPEC_ERR_NULL
    assert paged(qd=0, kvd=0) == SPEC_ERR_DTYPE                     # no fp32 paged path
    assert paged(kvd=2) == SPEC_ERR_NULL                            # fp8 pages need scales
    assert paged(page_size=24) == SPEC_ERR_SHAPE                    # not a power of two
    assert paged(max_pages=2049) == SPEC_ERR_SHAPE
    assert paged(num_pages=0) == SPEC_ERR_SHAPE
    assert paged(shape=(4, 65, 32, 8, 128)) == SPEC_ERR_SHAPE
    assert paged(scale=-1.0) == SPEC_ERR_SHAPE
    assert paged() == SPEC_ERR_WORKSPACE                            # every check passed but the workspace


def test_backward_workspace_bytes(L):
    f = L.spec_tree_attn_backward_workspace_bytes
    # M = 24 rows padded to 32; 64 (request, kv head) sequences of 33 tiles of 64 keys, 4 runs each to
    # give the 256 CUs a workgroup each (runs of 9 tiles): one fp32 partial of 32 x 128 per run, one
    # counter per sequence
    assert f(8, 6, 32, 8, 128, 2054) == 64 * 4 * 32 * 128 * 4 + 64 * 4
    assert f(1, 6, 4, 1, 64, 134) == 3 * 32 * 64 * 4 + 4             # 3 tiles: runs of one tile
    # no run longer than 24 tiles: 512 sequences of 129 tiles -> 6 runs of 22
    assert f(64, 16, 64, 8, 128, 8208) == 512 * 6 * 128 * 128 * 4 + 512 * 4
    assert f(64, 16, 64, 8, 128, 64) == 0                            # one tile: dq is written directly
    # more than 128 packed rows (8 x 17 = 136): the separate dq and dK / dV passes keep no partial sums;
    # the workspace holds D and lse * log2(e) of each (request, node, head) row, 256-byte aligned each
    assert f(8, 17, 64, 8, 128, 2054) == 2 * ((8 * 17 * 64 * 4 + 255) & ~255)
    # 16 x 60 = 960 rows: the same two arrays, whatever the cache length
    assert f(4, 60, 64, 4, 128, 64) == f(4, 60, 64, 4, 128, 32828) == 2 * 4 * 60 * 64 * 4
    for bad in [(8, 6, 32, 8, 96, 2054), (8, 65, 64, 8, 128, 2054), (8, 6, 30, 8, 128, 2054),
                (0, 6, 32, 8, 128, 2054), (8, 6, 32, 8, 128, 5)]:
        assert f(*bad) == 0, bad


def test_backward_host_checks(L):
    def bwd(q=FAKE, dt=1, lse=FAKE, dq=FAKE, shape=(8, 6, 32, 8, 128, 2054), scale=0.088, ws=None, wsb=0):
        return L.spec_tree_attn_backward(q, FAKE, FAKE, dt, FAKE, FAKE, FAKE, lse, FAKE, *shape, scale, dq,
                                         FAKE, FAKE, ws, wsb, None, None)
    assert bwd(q=None) == SPEC_ERR_NULL
    assert bwd(lse=None) == SPEC_ERR_NULL                         # the forward pass's lse is required
    assert bwd(dq=None) == SPEC_ERR_NULL
    assert bwd(dt=2) == SPEC_ERR_DTYPE                            # no fp8 gradients
    assert bwd(shape=(8, 65, 64, 8, 128, 2054)) == SPEC_ERR_SHAPE  # more than 64 nodes
    assert bwd(shape=(8, 6, 32, 8, 96, 2054)) == SPEC_ERR_SHAPE
    assert bwd(scale=0.0) == SPEC_ERR_SHAPE
    assert bwd(q=ctypes.c_void_p(0x1004)) == SPEC_ERR_ALIGN
    assert bwd() == SPEC_ERR_WORKSPACE
    need = L.spec_tree_attn_backward_workspace_bytes(8, 6, 32, 8, 128, 2054)
    assert bwd(ws=FAKE, wsb=need - 1) == SPEC_ERR_WORKSPACE


def test_verify_step_workspace_bytes(L):
    f = L.spec_verify_step_workspace_bytes
    # a 64-bit argmax key and a counter per node, a counter per request (8*6*12 + 8*4 = 608 bytes,
    # rounded up to 768), then the attention's workspace
    assert f(8, 6, 32, 8, 128, 2054) == 768 + L.spec_tree_attn_workspace_bytes(8, 6, 32, 8, 128, 2054)
    assert f(64, 64, 64, 8, 128, 4160) == 64 * 64 * 12 + 256 + L.spec_tree_attn_workspace_bytes(64, 64, 64, 8, 128,
                                                                                                4160)
    for bad in [(0, 6, 32, 8, 128, 2054), (8, 0, 32, 8, 128, 2054), (8, 65, 32, 8, 128, 2054),
                (8, 6, 32, 8, 96, 2054), (8, 6, 30, 8, 128, 2054), (8, 6, 32, 8, 128, 5)]:
        assert f(*bad) == 0, bad


def test_verify_step_host_checks(L):
    need = L.spec_verify_step_workspace_bytes(8, 6, 32, 8, 128, 2054)

    def step(parents=FAKE, logits=FAKE, out=FAKE, V=32000, stride=32000, qd=1, kvd=1,
             shape=(8, 6, 32, 8, 128, 2054), scale=0.088, ws=FAKE, wsb=need, q=FAKE):
        return L.spec_verify_step(parents, FAKE, FAKE, q, qd, FAKE, FAKE, kvd, None, None, logits, V, stride,
                                  *shape, scale, FAKE, None, out, None, FAKE, FAKE, FAKE, FAKE, ws, wsb, None,
                                  None)
    assert step(parents=None) == SPEC_ERR_NULL
    assert step(logits=None) == SPEC_ERR_NULL
    assert step(out=None) == SPEC_ERR_NULL                        # the attention's checks come first too
    assert step(V=0, stride=0) == SPEC_ERR_SHAPE
    assert step(stride=31999) == SPEC_ERR_SHAPE
    assert step(V=2 ** 31, stride=2 ** 31) == SPEC_ERR_SHAPE
    assert step(shape=(8, 65, 32, 8, 128, 2054)) == SPEC_ERR_SHAPE
    assert step(shape=(8, 6, 32, 8, 96, 2054)) == SPEC_ERR_SHAPE
    assert step(qd=0) == SPEC_ERR_DTYPE
    assert step(kvd=2) == SPEC_ERR_NULL                           # fp8 cache without scales
    assert step(scale=0.0) == SPEC_ERR_SHAPE
    assert step(q=ctypes.c_void_p(0x1004)) == SPEC_ERR_ALIGN
    assert step(ws=None) == SPEC_ERR_WORKSPACE
    assert step(wsb=need - 1) == SPEC_ERR_WORKSPACE               # the attention's part is one byte short
    assert step(wsb=100) == SPEC_ERR_WORKSPACE                    # not even the argmax keys fit
    assert step(ws=ctypes.c_void_p(0x1008)) == SPEC_ERR_ALIGN


def test_verify_step_static_host_checks(L):
    """Refusals come before the scratch's set-up (which needs a GPU): bad
    arguments as spec_verify_step's, sizes past the static scratch as
    SPEC_ERR_SCRATCH."""
    def step(parents=FAKE, logits=FAKE, out=FAKE, V=32000, stride=32000, qd=1, kvd=1,
             shape=(8, 6, 32, 8, 128, 2054), scale=0.088, q=FAKE):
        return L.spec_verify_step_static(parents, FAKE, FAKE, q, qd, FAKE, FAKE, kvd, None, None, logits, V, stride,
                                         *shape, scale, FAKE, None, out, None, FAKE, FAKE, FAKE, FAKE, None, None)
    assert step(parents=None) == SPEC_ERR_NULL
    assert step(logits=None) == SPEC_ERR_NULL
    assert step(out=None) == SPEC_ERR_NULL
    assert step(stride=31999) == SPEC_ERR_SHAPE
    assert step(shape=(8, 65, 32, 8, 128, 2054)) == SPEC_ERR_SHAPE
    assert step(qd=0) == SPEC_ERR_DTYPE
    assert step(kvd=2) == SPEC_ERR_NULL
    assert step(scale=0.0) == SPEC_ERR_SHAPE
    assert step(q=ctypes.c_void_p(0x1004)) == SPEC_ERR_ALIGN
    limit = 72 << 20
    big = (64, 60, 64, 4, 128, 32828)                       # a workspace of about 260 MB
    assert L.spec_verify_step_workspace_bytes(*big) > limit
    assert step(shape=big, V=1000, stride=1000) == SPEC_ERR_SCRATCH
    ok = (16, 60, 64, 4, 128, 32828)
    assert 0 < L.spec_verify_step_workspace_bytes(*ok) <= limit
    with open(HEADER) as f:
        assert "#define SPEC_STATIC_SCRATCH_BYTES (72u << 20)" in f.read()


def test_verify_step_paged_host_checks(L):
    # 8 requests of 6 nodes over 16-token pages, 129 pages each (S_max 2064)
    need = L.spec_verify_step_workspace_bytes(8, 6, 32, 8, 128, 129 * 16)
    assert need > 0

    def step(parents=FAKE, table=FAKE, out=FAKE, V=32000, stride=32000, qd=1, kvd=1, pages=(129, 16, 1100),
             shape=(8, 6, 32, 8, 128), scale=0.088, ws=FAKE, wsb=need, q=FAKE):
        return L.spec_verify_step_paged(parents, FAKE, FAKE, q, qd, FAKE, FAKE, kvd, None, None, table, *pages,
                                        FAKE, V, stride, *shape, scale, FAKE, None, out, None, FAKE, FAKE, FAKE,
                                        FAKE, ws, wsb, None, None)
    assert step(parents=None) == SPEC_ERR_NULL
    assert step(table=None) == SPEC_ERR_NULL
    assert step(out=None) == SPEC_ERR_NULL
    assert step(stride=31999) == SPEC_ERR_SHAPE
    assert step(shape=(8, 65, 32, 8, 128)) == SPEC_ERR_SHAPE
    assert step(shape=(8, 6, 32, 8, 96)) == SPEC_ERR_SHAPE
    assert step(qd=0, kvd=0) == SPEC_ERR_DTYPE                    # no fp32 pages
    assert step(kvd=2) == SPEC_ERR_NULL                           # fp8 pages without scales
    assert step(pages=(129, 24, 1100)) == SPEC_ERR_SHAPE          # page size not a power of two
    assert step(pages=(129, 8192, 1100)) == SPEC_ERR_SHAPE
    assert step(pages=(2049, 16, 1100)) == SPEC_ERR_SHAPE         # table wider than 2048 pages
    assert step(pages=(129, 16, 0)) == SPEC_ERR_SHAPE
    assert step(scale=float("inf")) == SPEC_ERR_SHAPE
    assert step(q=ctypes.c_void_p(0x1004)) == SPEC_ERR_ALIGN
    assert step(ws=None) == SPEC_ERR_WORKSPACE
    assert step(wsb=need - 1) == SPEC_ERR_WORKSPACE
    assert step(ws=ctypes.c_void_p(0x1008)) == SPEC_ERR_ALIGN


def test_commit_paged_host_checks(L):
    def commit(table=FAKE, kvd=1, pages=(16, 16, 40), shape=(4, 6, 2, 128), k=FAKE, newp=FAKE):
        return L.spec_commit_accepted_paged(k, FAKE, kvd, table, *pages, FAKE, FAKE, FAKE, *shape, newp, None,
                                            None, None)
    assert commit(table=None) == SPEC_ERR_NULL
    assert commit(k=None) == SPEC_ERR_NULL
    assert commit(newp=None) == SPEC_ERR_NULL
    assert commit(kvd=7) == SPEC_ERR_DTYPE
    assert commit(pages=(16, 12, 40)) == SPEC_ERR_SHAPE           # page size not a power of two
    assert commit(pages=(16, 8192, 40)) == SPEC_ERR_SHAPE
    assert commit(pages=(2049, 16, 40)) == SPEC_ERR_SHAPE         # table wider than 2048 pages
    assert commit(pages=(16, 16, 0)) == SPEC_ERR_SHAPE
    assert commit(pages=(1, 4, 40)) == SPEC_ERR_SHAPE             # 4 rows cannot hold a 6-node tree
    assert commit(shape=(4, 6, 2, 96)) == SPEC_ERR_SHAPE
    assert commit(shape=(4, 65, 2, 128)) == SPEC_ERR_SHAPE
    assert commit(k=ctypes.c_void_p(0x1008)) == SPEC_ERR_ALIGN


def test_binding_constants_match_the_header():
    """The binding's dtype codes, device error bits and node limit are the
    header's (read from include/spectree.h, not from the library)."""
    with open(HEADER) as f:
        text = f.read()
    defines = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (SPEC_\w+)\s+(\d+)u?\b", text)}
    enums = {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(SPEC_(?:F32|BF16|FP8_E4M3|FP4_E2M1))\s*=\s*(\d+)", text)}
    assert defines["SPEC_MAX_NODES"] == st.MAX_NODES
    for name in ("ROOT", "PARENT", "PREFIX", "TOKEN", "PATH", "PAGE"):
        assert defines["SPEC_DERR_" + name] == getattr(st, "DERR_" + name), name
    assert (enums["SPEC_F32"], enums["SPEC_BF16"], enums["SPEC_FP8_E4M3"]) == (st.SPEC_F32, st.SPEC_BF16,
                                                                               st.SPEC_FP8_E4M3)
    statuses = {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(SPEC_(?:OK|ERR_\w+))\s*=\s*(\d+)", text)}
    assert statuses == {"SPEC_OK": SPEC_OK, "SPEC_ERR_NULL": SPEC_ERR_NULL, "SPEC_ERR_SHAPE": SPEC_ERR_SHAPE,
                        "SPEC_ERR_DTYPE": SPEC_ERR_DTYPE, "SPEC_ERR_WORKSPACE": SPEC_ERR_WORKSPACE,
                        "SPEC_ERR_HIP": SPEC_ERR_HIP, "SPEC_ERR_ALIGN": SPEC_ERR_ALIGN,
                        "SPEC_ERR_SCRATCH": SPEC_ERR_SCRATCH}
