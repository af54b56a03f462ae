"""spectree: speculative-decoding tree verify step on AMD MI355X (gfx950).

A thin ctypes binding over ``libspectree.so`` (``include/spectree.h``).  The
functions here only marshal arguments: every step runs in the library's HIP
kernels, on the caller's current torch stream.  Torch is used for device
memory and streams only.  There is no CPU fallback: if the library or a GPU
is missing, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "SpecError", "lib", "tree_mask_build", "attn_workspace_bytes", "tree_attn_verify", "tree_attn_verify_paged",
    "vocab_argmax", "accept_walk", "commit_accepted", "verify_step", "attn_backward_workspace_bytes",
    "tree_attn_backward", "tree_attn_verify_f8", "tree_attn_verify_f4", "tree_attn_verify_f8_scores", "verify_step_static", "DERR_ROOT",
    "DERR_PARENT",
    "DERR_PREFIX", "DERR_TOKEN", "DERR_PATH", "DERR_PAGE", "library_path", "verify_step_workspace_bytes", "step_outputs",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libspectree.so")

SPEC_F32, SPEC_BF16, SPEC_FP8_E4M3 = 0, 1, 2
DERR_ROOT, DERR_PARENT, DERR_PREFIX, DERR_TOKEN, DERR_PATH, DERR_PAGE = 1, 2, 4, 8, 16, 32
MAX_NODES = 64

_DTYPE = {torch.float32: SPEC_F32, torch.bfloat16: SPEC_BF16, torch.float8_e4m3fn: SPEC_FP8_E4M3}

EXPORTS = ["spec_tree_mask_build", "spec_tree_attn_workspace_bytes", "spec_tree_attn_verify",
           "spec_tree_attn_verify_paged", "spec_tree_attn_verify_f8", "spec_tree_attn_verify_f4",
           "spec_tree_attn_verify_f8_scores",
           "spec_vocab_argmax", "spec_accept_walk", "spec_commit_accepted", "spec_commit_accepted_paged",
           "spec_tree_attn_backward_workspace_bytes", "spec_tree_attn_backward", "spec_verify_step_workspace_bytes",
           "spec_verify_step", "spec_verify_step_paged", "spec_verify_step_static", "spec_status_string"]


class SpecError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load libspectree.so (built in-tree by ``build.py``) or raise."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise SpecError(f"{library_path} is missing: build it with "
                        "`python -m tree_attention_verify_parent_amd.build`")
    L = ctypes.CDLL(library_path)
    c_i, c_p, c_i64, c_sz, c_f = ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    L.spec_tree_mask_build.argtypes = [c_p, c_i, c_i, c_p, c_p, c_p, c_p]
    L.spec_tree_mask_build.restype = c_i
    L.spec_tree_attn_workspace_bytes.argtypes = [c_i] * 6
    L.spec_tree_attn_workspace_bytes.restype = c_sz
    L.spec_tree_attn_verify.argtypes = [c_p, c_i, c_p, c_p, c_i, c_p, c_p, c_p, c_p,
                                        c_i, c_i, c_i, c_i, c_i, c_i, c_f, c_p, c_p, c_p, c_sz,
                                        c_p, c_p]
    L.spec_tree_attn_verify.restype = c_i
    L.spec_tree_attn_verify_paged.argtypes = [c_p, c_i, c_p, c_p, c_i, c_p, c_p, c_p, c_p, c_p, c_i, c_i, c_i,
                                              c_i, c_i, c_i, c_i, c_i, c_f, c_p, c_p, c_p, c_sz, c_p, c_p]
    L.spec_tree_attn_verify_paged.restype = c_i
    L.spec_tree_attn_verify_f8.argtypes = [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_i, c_i, c_i, c_i, c_i, c_i, c_f,
                                           c_p, c_p, c_p, c_sz, c_p, c_p]
    L.spec_tree_attn_verify_f8.restype = c_i
    L.spec_tree_attn_verify_f4.argtypes = L.spec_tree_attn_verify_f8.argtypes
    L.spec_tree_attn_verify_f4.restype = c_i
    L.spec_tree_attn_verify_f8_scores.argtypes = [c_p, c_p, c_p, c_p, c_p, c_p, c_i, c_i, c_i, c_i, c_i, c_i, c_f,
                                                  c_p, c_p, c_p, c_sz, c_p, c_p]
    L.spec_tree_attn_verify_f8_scores.restype = c_i
    L.spec_vocab_argmax.argtypes = [c_p, c_i64, c_i64, c_i64, c_p, c_p]
    L.spec_vocab_argmax.restype = c_i
    L.spec_accept_walk.argtypes = [c_p, c_p, c_p, c_p, c_i, c_i, c_i, c_p, c_p, c_p, c_p, c_p]
    L.spec_accept_walk.restype = c_i
    L.spec_commit_accepted.argtypes = [c_p, c_p, c_i, c_p, c_p, c_p, c_i, c_i, c_i, c_i, c_i, c_p, c_p, c_p, c_p]
    L.spec_commit_accepted.restype = c_i
    L.spec_commit_accepted_paged.argtypes = [c_p, c_p, c_i, c_p, c_i, c_i, c_i, c_p, c_p, c_p, c_i, c_i, c_i, c_i,
                                             c_p, c_p, c_p, c_p]
    L.spec_commit_accepted_paged.restype = c_i
    L.spec_tree_attn_backward_workspace_bytes.argtypes = [c_i] * 6
    L.spec_tree_attn_backward_workspace_bytes.restype = c_sz
    L.spec_tree_attn_backward.argtypes = [c_p, c_p, c_p, c_i, c_p, c_p, c_p, c_p, c_p, c_i, c_i, c_i, c_i, c_i, c_i,
                                          c_f, c_p, c_p, c_p, c_p, c_sz, c_p, c_p]
    L.spec_tree_attn_backward.restype = c_i
    L.spec_verify_step_workspace_bytes.argtypes = [c_i] * 6
    L.spec_verify_step_workspace_bytes.restype = c_sz
    L.spec_verify_step.argtypes = [c_p, c_p, c_p, c_p, c_i, c_p, c_p, c_i, c_p, c_p, c_p, c_i64, c_i64,
                                   c_i, c_i, c_i, c_i, c_i, c_i, c_f, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                   c_p, c_sz, c_p, c_p]
    L.spec_verify_step.restype = c_i
    L.spec_verify_step_paged.argtypes = [c_p, c_p, c_p, c_p, c_i, c_p, c_p, c_i, c_p, c_p, c_p, c_i, c_i, c_i,
                                         c_p, c_i64, c_i64, c_i, c_i, c_i, c_i, c_i, c_f, c_p, c_p, c_p, c_p, c_p,
                                         c_p, c_p, c_p, c_p, c_sz, c_p, c_p]
    L.spec_verify_step_paged.restype = c_i
    L.spec_verify_step_static.argtypes = L.spec_verify_step.argtypes[:-4] + [c_p, c_p]
    L.spec_verify_step_static.restype = c_i
    L.spec_status_string.argtypes = [c_i]
    L.spec_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise SpecError(lib().spec_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise SpecError("spectree takes device tensors only")
    if not t.is_contiguous():
        raise SpecError("spectree takes contiguous tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _err_word(err: Optional[torch.Tensor], device) -> torch.Tensor:
    if err is not None:
        return err
    return torch.zeros(1, dtype=torch.int32, device=device)


def tree_mask_build(parents: torch.Tensor, *, anc_mask=None, depth=None, err=None, stream=None):
    """parents int32[B][N] -> (anc_mask int64[B][N] (uint64 bit patterns),
    depth int32[B][N], err int32[1])."""
    B, N = parents.shape
    dev = parents.device
    anc_mask = torch.empty((B, N), dtype=torch.int64, device=dev) if anc_mask is None else anc_mask
    depth = torch.empty((B, N), dtype=torch.int32, device=dev) if depth is None else depth
    err = _err_word(err, dev)
    _check(lib().spec_tree_mask_build(_ptr(parents), B, N, _ptr(anc_mask), _ptr(depth), _ptr(err),
                                      _stream(stream)))
    return anc_mask, depth, err


def attn_workspace_bytes(B, N, Hq, Hkv, D, S_max) -> int:
    return int(lib().spec_tree_attn_workspace_bytes(B, N, Hq, Hkv, D, S_max))


def tree_attn_verify(q, k_cache, v_cache, prefix_lens, anc_mask, sm_scale, *, k_scale=None,
                     v_scale=None, out=None, lse=None, want_lse=True, workspace=None, err=None,
                     stream=None):
    """Tree-masked attention.  q [B][N][Hq][D] (f32 or bf16); caches
    [B][Hkv][S_max][D] (f32, bf16 or float8_e4m3fn); returns (out, lse, err)."""
    B, N, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    if q.dtype not in _DTYPE or k_cache.dtype not in _DTYPE or v_cache.dtype != k_cache.dtype:
        raise SpecError(f"unsupported dtypes q={q.dtype} kv={k_cache.dtype}/{v_cache.dtype}")
    if tuple(k_cache.shape) != (B, Hkv, S_max, D) or tuple(v_cache.shape) != (B, Hkv, S_max, D):
        raise SpecError("k_cache / v_cache must be [B][Hkv][S_max][D] matching q")
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    ws_need = attn_workspace_bytes(B, N, Hq, Hkv, D, S_max)
    if workspace is None and ws_need:
        # zero-filled once; every call leaves it ready for the next (counters back at zero)
        workspace = torch.zeros(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    err = _err_word(err, dev)
    _check(lib().spec_tree_attn_verify(
        _ptr(q), _DTYPE[q.dtype], _ptr(k_cache), _ptr(v_cache), _DTYPE[k_cache.dtype],
        _ptr(k_scale), _ptr(v_scale), _ptr(prefix_lens), _ptr(anc_mask),
        B, N, Hq, Hkv, D, S_max, float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _ptr(err), _stream(stream)))
    return out, lse, err


def tree_attn_verify_paged(q, k_pages, v_pages, prefix_lens, anc_mask, block_table, sm_scale, *,
                           k_scale=None, v_scale=None, out=None, lse=None, want_lse=True, workspace=None,
                           err=None, stream=None):
    """Tree-masked attention over a paged cache: q [B][N][Hq][D] bf16; pages
    [num_pages][page_size][Hkv][D] (bf16 or float8_e4m3fn); block_table
    int32[B][max_pages]; returns (out, lse, err)."""
    B, N, Hq, D = q.shape
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    max_pages = block_table.shape[1]
    dev = q.device
    if q.dtype not in _DTYPE or k_pages.dtype not in _DTYPE or v_pages.dtype != k_pages.dtype:
        raise SpecError(f"unsupported dtypes q={q.dtype} kv={k_pages.dtype}/{v_pages.dtype}")
    if tuple(k_pages.shape) != (num_pages, page_size, Hkv, D) or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise SpecError("k_pages / v_pages must be [num_pages][page_size][Hkv][D] matching q")
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    ws_need = attn_workspace_bytes(B, N, Hq, Hkv, D, max_pages * page_size)
    if workspace is None and ws_need:
        workspace = torch.zeros(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    err = _err_word(err, dev)
    _check(lib().spec_tree_attn_verify_paged(
        _ptr(q), _DTYPE[q.dtype], _ptr(k_pages), _ptr(v_pages), _DTYPE[k_pages.dtype], _ptr(k_scale),
        _ptr(v_scale), _ptr(prefix_lens), _ptr(anc_mask), _ptr(block_table), max_pages, page_size, num_pages,
        B, N, Hq, Hkv, D, float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _ptr(err),
        _stream(stream)))
    return out, lse, err


def tree_attn_verify_f8(q, k_cache, v_cache, prefix_lens, anc_mask, sm_scale, k_scale, v_scale, *, out=None,
                        lse=None, want_lse=True, workspace=None, err=None, stream=None):
    """Tree-masked attention in fp8 arithmetic over an e4m3 cache: q [B][N][Hq][128]
    bf16; caches [B][Hkv][S_max][128] float8_e4m3fn with float32 k_scale /
    v_scale [Hkv].  Returns (out bf16, lse, err)."""
    B, N, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.float8_e4m3fn or v_cache.dtype != k_cache.dtype:
        raise SpecError(f"fp8 arithmetic takes bf16 q and float8_e4m3fn caches, not {q.dtype} / {k_cache.dtype}")
    if tuple(k_cache.shape) != (B, Hkv, S_max, D) or tuple(v_cache.shape) != (B, Hkv, S_max, D):
        raise SpecError("k_cache / v_cache must be [B][Hkv][S_max][D] matching q")
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    ws_need = attn_workspace_bytes(B, N, Hq, Hkv, D, S_max)
    if workspace is None and ws_need:
        workspace = torch.zeros(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    err = _err_word(err, dev)
    _check(lib().spec_tree_attn_verify_f8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(prefix_lens), _ptr(anc_mask),
        B, N, Hq, Hkv, D, S_max, float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _ptr(err),
        _stream(stream)))
    return out, lse, err


def tree_attn_verify_f8_scores(q, k_cache, v_cache, prefix_lens, anc_mask, sm_scale, k_scale=None, *, out=None,
                               lse=None, want_lse=True, workspace=None, err=None, stream=None):
    """Tree-masked attention over bf16 caches with the scores on the fp8 matrix
    cores: q [B][N][Hq][128] and caches [B][Hkv][S_max][128] bf16; k_scale
    (optional float32 [Hkv]) sets the power of two K is divided by before
    rounding to e4m3.  Returns (out bf16, lse, err)."""
    B, N, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise SpecError(f"fp8 scores take bf16 q and bf16 caches, not {q.dtype} / {k_cache.dtype}")
    if tuple(k_cache.shape) != (B, Hkv, S_max, D) or tuple(v_cache.shape) != (B, Hkv, S_max, D):
        raise SpecError("k_cache / v_cache must be [B][Hkv][S_max][D] matching q")
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    ws_need = attn_workspace_bytes(B, N, Hq, Hkv, D, S_max)
    if workspace is None and ws_need:
        workspace = torch.zeros(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    err = _err_word(err, dev)
    _check(lib().spec_tree_attn_verify_f8_scores(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(prefix_lens), _ptr(anc_mask),
        B, N, Hq, Hkv, D, S_max, float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _ptr(err),
        _stream(stream)))
    return out, lse, err


def tree_attn_verify_f4(q, k_cache, v_cache, prefix_lens, anc_mask, sm_scale, k_scale, v_scale, *, out=None,
                        lse=None, want_lse=True, workspace=None, err=None, stream=None):
    """Tree-masked attention in fp8 arithmetic over an e2m1 (fp4) cache: q
    [B][N][Hq][128] bf16; caches [B][Hkv][S_max][64] uint8, two e2m1 codes a
    byte (element 2j in the low nibble); float32 k_scale / v_scale [Hkv].
    Returns (out bf16, lse, err)."""
    B, N, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise SpecError(f"fp4 caches are packed uint8 with bf16 q, not {q.dtype} / {k_cache.dtype}")
    if tuple(k_cache.shape) != (B, Hkv, S_max, D // 2) or tuple(v_cache.shape) != (B, Hkv, S_max, D // 2):
        raise SpecError("k_cache / v_cache must be [B][Hkv][S_max][D/2] packed e2m1 matching q")
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    ws_need = attn_workspace_bytes(B, N, Hq, Hkv, D, S_max)
    if workspace is None and ws_need:
        workspace = torch.zeros(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    err = _err_word(err, dev)
    _check(lib().spec_tree_attn_verify_f4(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(prefix_lens), _ptr(anc_mask),
        B, N, Hq, Hkv, D, S_max, float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _ptr(err),
        _stream(stream)))
    return out, lse, err


def vocab_argmax(logits: torch.Tensor, *, out=None, stream=None) -> torch.Tensor:
    """logits float32[rows][V] (row stride may exceed V) -> int32[rows]."""
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1:
        raise SpecError("logits must be a float32 [rows][V] tensor with unit column stride")
    rows, V = logits.shape
    out = torch.empty(rows, dtype=torch.int32, device=logits.device) if out is None else out
    _check(lib().spec_vocab_argmax(ctypes.c_void_p(logits.data_ptr()), rows, V, logits.stride(0),
                                   _ptr(out), _stream(stream)))
    return out


def accept_walk(parents, anc_mask, draft_tokens, target_argmax, V, *, accept_len=None,
                path_nodes=None, out_tokens=None, err=None, stream=None):
    """Returns (accept_len int32[B], path_nodes int32[B][N], out_tokens int32[B][N], err)."""
    B, N = parents.shape
    dev = parents.device
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    path_nodes = torch.empty((B, N), dtype=torch.int32, device=dev) if path_nodes is None else path_nodes
    out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev) if out_tokens is None else out_tokens
    err = _err_word(err, dev)
    _check(lib().spec_accept_walk(_ptr(parents), _ptr(anc_mask), _ptr(draft_tokens), _ptr(target_argmax),
                                  B, N, int(V), _ptr(accept_len), _ptr(path_nodes), _ptr(out_tokens),
                                  _ptr(err), _stream(stream)))
    return accept_len, path_nodes, out_tokens, err


def commit_accepted(k_cache, v_cache, prefix_lens, accept_len, path_nodes, *, block_table=None,
                    new_prefix_lens=None, labels=None, want_labels=True, err=None, stream=None):
    """In place: request b's accepted path node at depth k moves to cache row
    prefix_lens[b] + k.  Returns (new_prefix_lens int32[B], labels int8[B][N]
    or None, err).  With ``block_table`` (int32 [B][max_pages]) the caches are
    pools of pages [num_pages][page_size][Hkv][D] (spec_commit_accepted_paged)."""
    B, N = path_nodes.shape
    if k_cache.dtype not in _DTYPE or v_cache.dtype != k_cache.dtype or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise SpecError("k_cache / v_cache must be matching 4-d tensors of a supported dtype")
    dev = k_cache.device
    new_prefix_lens = torch.empty(B, dtype=torch.int32, device=dev) if new_prefix_lens is None else new_prefix_lens
    if labels is None and want_labels:
        labels = torch.empty((B, N), dtype=torch.int8, device=dev)
    err = _err_word(err, dev)
    if block_table is not None:
        num_pages, page_size, Hkv, D = k_cache.shape
        _check(lib().spec_commit_accepted_paged(
            _ptr(k_cache), _ptr(v_cache), _DTYPE[k_cache.dtype], _ptr(block_table), block_table.shape[1],
            page_size, num_pages, _ptr(prefix_lens), _ptr(accept_len), _ptr(path_nodes), B, N, Hkv, D,
            _ptr(new_prefix_lens), _ptr(labels), _ptr(err), _stream(stream)))
        return new_prefix_lens, labels, err
    if k_cache.shape[0] != B:
        raise SpecError("k_cache / v_cache must be [B][Hkv][S_max][D]")
    _, Hkv, S_max, D = k_cache.shape
    _check(lib().spec_commit_accepted(_ptr(k_cache), _ptr(v_cache), _DTYPE[k_cache.dtype], _ptr(prefix_lens),
                                      _ptr(accept_len), _ptr(path_nodes), B, N, Hkv, D, S_max,
                                      _ptr(new_prefix_lens), _ptr(labels), _ptr(err), _stream(stream)))
    return new_prefix_lens, labels, err


def attn_backward_workspace_bytes(B, N, Hq, Hkv, D, S_max) -> int:
    return int(lib().spec_tree_attn_backward_workspace_bytes(B, N, Hq, Hkv, D, S_max))


def tree_attn_backward(q, k_cache, v_cache, prefix_lens, anc_mask, out, lse, d_out, sm_scale, *, dq=None,
                       dk=None, dv=None, workspace=None, err=None, stream=None):
    """Backward pass of tree_attn_verify: q, out, d_out [B][N][Hq][D] and
    caches [B][Hkv][S_max][D], all float32 or all bf16; lse float32[B][N][Hq]
    from the forward pass.  Returns (dq, dk, dv, err).  Rows of dk / dv at or
    past prefix_lens[b] + N are not written (zero when allocated here)."""
    B, N, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    dts = {q.dtype, k_cache.dtype, v_cache.dtype, out.dtype, d_out.dtype}
    if len(dts) != 1 or q.dtype not in (torch.float32, torch.bfloat16):
        raise SpecError(f"q, caches, out and d_out must share one dtype, float32 or bfloat16: {dts}")
    if tuple(k_cache.shape) != (B, Hkv, S_max, D) or tuple(v_cache.shape) != (B, Hkv, S_max, D):
        raise SpecError("k_cache / v_cache must be [B][Hkv][S_max][D] matching q")
    if tuple(out.shape) != tuple(q.shape) or tuple(d_out.shape) != tuple(q.shape):
        raise SpecError("out and d_out must have q's shape")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.zeros_like(k_cache) if dk is None else dk
    dv = torch.zeros_like(v_cache) if dv is None else dv
    ws_need = attn_backward_workspace_bytes(B, N, Hq, Hkv, D, S_max)
    if workspace is None and ws_need:
        workspace = torch.zeros(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    err = _err_word(err, dev)
    _check(lib().spec_tree_attn_backward(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _DTYPE[q.dtype], _ptr(prefix_lens), _ptr(anc_mask), _ptr(out),
        _ptr(lse), _ptr(d_out), B, N, Hq, Hkv, D, S_max, float(sm_scale), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), ws_bytes, _ptr(err), _stream(stream)))
    return dq, dk, dv, err


def verify_step_workspace_bytes(B, N, Hq, Hkv, D, S_max) -> int:
    return int(lib().spec_verify_step_workspace_bytes(B, N, Hq, Hkv, D, S_max))


def step_outputs(B, N, q):
    """Preallocated outputs for verify_step(..., outs=...)."""
    dev = q.device
    return dict(mask=torch.empty((B, N), dtype=torch.int64, device=dev),
                depth=torch.empty((B, N), dtype=torch.int32, device=dev),
                out=torch.empty_like(q),
                lse=torch.empty((B, N, q.shape[2]), dtype=torch.float32, device=dev),
                argmax=torch.empty(B * N, dtype=torch.int32, device=dev),
                accept_len=torch.empty(B, dtype=torch.int32, device=dev),
                path_nodes=torch.empty((B, N), dtype=torch.int32, device=dev),
                out_tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
                err=torch.zeros(1, dtype=torch.int32, device=dev))


def verify_step(parents, draft_tokens, prefix_lens, q, k_cache, v_cache, logits, sm_scale, *,
                k_scale=None, v_scale=None, block_table=None, workspace=None, fused=True, outs=None, debug=False,
                stream=None):
    """One verify step on the GPU: masks, attention, argmax, accept walk.

    ``fused`` (default): spec_verify_step, one launch, with
    ``workspace`` (zero-filled before its
    first use, left ready for reuse; allocated here when None).  ``fused=False``: the
    four separate calls (``workspace`` is then the attention's).  Both enqueue on one stream and give the same
    results; nothing synchronises unless ``debug`` is set, in which case the
    device error word is read and a non-zero value raises.  ``outs``
    (from step_outputs; its error word is OR'ed into, not cleared) receives
    the results instead of fresh tensors.  With ``block_table`` (int32
    [B][max_pages]) the caches are pools of pages [num_pages][page_size][Hkv][D]
    (spec_verify_step_paged; unfused: spec_tree_attn_verify_paged).
    """
    dev = q.device
    B, N = parents.shape
    Hq, D = q.shape[2], q.shape[3]
    paged = block_table is not None
    if paged:
        num_pages, page_size, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
        max_pages = block_table.shape[1]
        S_max = max_pages * page_size
    else:
        Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    o = step_outputs(B, N, q) if outs is None else outs
    anc, depth, out, lse, t = o["mask"], o["depth"], o["out"], o["lse"], o["argmax"]
    L, path, toks, err = o["accept_len"], o["path_nodes"], o["out_tokens"], o["err"]
    if not fused:
        tree_mask_build(parents, anc_mask=anc, depth=depth, err=err, stream=stream)
        if paged:
            tree_attn_verify_paged(q, k_cache, v_cache, prefix_lens, anc, block_table, sm_scale, k_scale=k_scale,
                                   v_scale=v_scale, out=out, lse=lse, workspace=workspace, err=err, stream=stream)
        else:
            tree_attn_verify(q, k_cache, v_cache, prefix_lens, anc, sm_scale, k_scale=k_scale, v_scale=v_scale,
                             out=out, lse=lse, workspace=workspace, err=err, stream=stream)
        vocab_argmax(logits, out=t, stream=stream)
        accept_walk(parents, anc, draft_tokens, t.view(B, N), logits.shape[1], accept_len=L, path_nodes=path,
                    out_tokens=toks, err=err, stream=stream)
    else:
        if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[0] != B * N:
            raise SpecError("logits must be a float32 [B*N][V] tensor with unit column stride")
        if q.dtype not in _DTYPE or k_cache.dtype not in _DTYPE or v_cache.dtype != k_cache.dtype:
            raise SpecError(f"unsupported dtypes q={q.dtype} k={k_cache.dtype} v={v_cache.dtype}")
        V = logits.shape[1]
        if workspace is None:
            workspace = torch.zeros(max(verify_step_workspace_bytes(B, N, Hq, Hkv, D, S_max), 16),
                                    dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
        if paged:
            if tuple(k_cache.shape) != (num_pages, page_size, Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
                raise SpecError("k / v pages must be [num_pages][page_size][Hkv][D] matching q")
            _check(lib().spec_verify_step_paged(
                _ptr(parents), _ptr(draft_tokens), _ptr(prefix_lens), _ptr(q), _DTYPE[q.dtype], _ptr(k_cache),
                _ptr(v_cache), _DTYPE[k_cache.dtype], _ptr(k_scale), _ptr(v_scale), _ptr(block_table), max_pages,
                page_size, num_pages, ctypes.c_void_p(logits.data_ptr()), V, logits.stride(0), B, N, Hq, Hkv, D,
                float(sm_scale), _ptr(anc), _ptr(depth), _ptr(out), _ptr(lse), _ptr(t), _ptr(L), _ptr(path),
                _ptr(toks), _ptr(workspace), ws_bytes, _ptr(err), _stream(stream)))
        else:
            _check(lib().spec_verify_step(
                _ptr(parents), _ptr(draft_tokens), _ptr(prefix_lens), _ptr(q), _DTYPE[q.dtype], _ptr(k_cache),
                _ptr(v_cache), _DTYPE[k_cache.dtype], _ptr(k_scale), _ptr(v_scale),
                ctypes.c_void_p(logits.data_ptr()), V, logits.stride(0), B, N, Hq, Hkv, D, S_max, float(sm_scale),
                _ptr(anc), _ptr(depth), _ptr(out), _ptr(lse), _ptr(t), _ptr(L), _ptr(path), _ptr(toks),
                _ptr(workspace), ws_bytes, _ptr(err), _stream(stream)))
    res = dict(mask=anc, depth=depth, out=out, lse=lse, argmax=t, accept_len=L, path_nodes=path,
               out_tokens=toks, err=err)
    if debug:
        e = int(err.item())
        if e:
            raise SpecError(f"device data error bits 0x{e:x}")
    return res


def verify_step_static(parents, draft_tokens, prefix_lens, q, k_cache, v_cache, logits, sm_scale, *, outs,
                       k_scale=None, v_scale=None, stream=None):
    """spec_verify_step_static: the one-launch verify step on the library's
    static scratch.  Allocates nothing, here or in the library: ``outs``
    (from step_outputs, made beforehand) receives every result and its error
    word is OR'ed into.  Calls that overlap in time on one GPU race."""
    if outs is None:
        raise SpecError("verify_step_static takes preallocated outputs (step_outputs)")
    B, N = parents.shape
    Hq, D = q.shape[2], q.shape[3]
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[0] != B * N:
        raise SpecError("logits must be a float32 [B*N][V] tensor with unit column stride")
    if q.dtype not in _DTYPE or k_cache.dtype not in _DTYPE or v_cache.dtype != k_cache.dtype:
        raise SpecError(f"unsupported dtypes q={q.dtype} k={k_cache.dtype} v={v_cache.dtype}")
    o = outs
    _check(lib().spec_verify_step_static(
        _ptr(parents), _ptr(draft_tokens), _ptr(prefix_lens), _ptr(q), _DTYPE[q.dtype], _ptr(k_cache),
        _ptr(v_cache), _DTYPE[k_cache.dtype], _ptr(k_scale), _ptr(v_scale), ctypes.c_void_p(logits.data_ptr()),
        logits.shape[1], logits.stride(0), B, N, Hq, Hkv, D, S_max, float(sm_scale), _ptr(o["mask"]),
        _ptr(o["depth"]), _ptr(o["out"]), _ptr(o["lse"]), _ptr(o["argmax"]), _ptr(o["accept_len"]),
        _ptr(o["path_nodes"]), _ptr(o["out_tokens"]), _ptr(o["err"]), _stream(stream)))
    return o
