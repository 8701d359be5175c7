"""Thin ctypes binding of libsa.so (argument marshalling only).

Every function takes torch tensors for device memory, checks dtypes, shapes
and devices, allocates outputs the caller did not pass, and calls the C entry
point of the same name on the current HIP stream. All computation happens in
the library's kernels; if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsa.so")

H, G, D, DI = 64, 4, 192, 256
MAX_TOPK = 512
MAX_SPLITS = 64

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(5)
EXPORTED = ["sa_status_string", "sa_indexer_topk_workspace_size", "sa_indexer_topk", "sa_indexer_topk_fp8",
            "sa_resolve_num_splits", "sa_sparse_decode", "sa_sparse_decode_fp8kv", "sa_swa_decode",
            "sa_swa_decode_fp8kv", "sa_merge", "sa_indexer_topk_grouped_workspace_size",
            "sa_indexer_topk_grouped", "sa_sparse_decode_grouped", "sa_indexer_topk_noalloc"]
FORMAT_BF16, FORMAT_FP8_E4M3 = 0, 1
# num_splits requests (besides a count n > 0): each token's partition count
# follows its own attended length only (batch invariant), or the call's size so
# that the grid fills the GPU
SPLITS_BY_LENGTH, SPLITS_FILL_GPU = 0, -1


class SAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class PagedDesc(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("batch", ctypes.c_int),
                ("max_pages_per_seq", ctypes.c_int), ("num_pages", ctypes.c_int)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsa.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                           " or `python sparse_block_indexed_amd/build.py`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.sa_status_string.restype = ctypes.c_char_p
    lib.sa_status_string.argtypes = [i32]
    lib.sa_indexer_topk_workspace_size.restype = sz
    lib.sa_indexer_topk_workspace_size.argtypes = [i32, i32, i32]
    lib.sa_resolve_num_splits.restype = i32
    lib.sa_resolve_num_splits.argtypes = [i32, i32, i32]
    for fn in (lib.sa_indexer_topk, lib.sa_indexer_topk_fp8):
        fn.restype = i32
        fn.argtypes = [vp, vp, PagedDesc, vp, vp, i32, i32, vp, vp, sz, vp]
    lib.sa_sparse_decode.restype = i32
    lib.sa_sparse_decode.argtypes = [vp, vp, vp, PagedDesc, vp, vp, vp, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp]
    lib.sa_swa_decode.restype = i32
    lib.sa_swa_decode.argtypes = [vp, vp, vp, PagedDesc, vp, vp, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp]
    lib.sa_sparse_decode_fp8kv.restype = i32
    lib.sa_sparse_decode_fp8kv.argtypes = [vp, vp, vp, f32, f32, PagedDesc, vp, vp, vp, i32, i32, f32, i32, vp, vp,
                                           vp, vp, vp, vp]
    lib.sa_swa_decode_fp8kv.restype = i32
    lib.sa_swa_decode_fp8kv.argtypes = [vp, vp, vp, f32, f32, PagedDesc, vp, vp, i32, i32, f32, i32, vp, vp, vp, vp,
                                        vp, vp]
    lib.sa_indexer_topk_grouped_workspace_size.restype = sz
    lib.sa_indexer_topk_grouped_workspace_size.argtypes = [i32, i32, i32]
    lib.sa_indexer_topk_grouped.restype = i32
    lib.sa_indexer_topk_grouped.argtypes = [vp, vp, i32, PagedDesc, vp, vp, i32, i32, vp, vp, sz, vp]
    lib.sa_sparse_decode_grouped.restype = i32
    lib.sa_sparse_decode_grouped.argtypes = [vp, vp, vp, i32, f32, f32, PagedDesc, vp, vp, vp, i32, i32, f32, i32,
                                             vp, vp, vp, vp, vp, vp]
    lib.sa_indexer_topk_noalloc.restype = i32
    lib.sa_indexer_topk_noalloc.argtypes = [vp, vp, PagedDesc, vp, vp, i32, i32, vp, vp]
    lib.sa_merge.restype = i32
    lib.sa_merge.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != SA_OK:
        raise SAError(fn, status, load_library().sa_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device, shape=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _desc(page_table: torch.Tensor, seq_lens: torch.Tensor, num_pages: int) -> PagedDesc:
    dev = page_table.device
    _need(page_table, "page_table", torch.int32, dev)
    _need(seq_lens, "seq_lens", torch.int32, dev, (page_table.shape[0],))
    return PagedDesc(page_table.data_ptr(), seq_lens.data_ptr(), page_table.shape[0], page_table.shape[1],
                     int(num_pages))


def indexer_workspace_size(n_tok: int, max_pages_per_seq: int, topk: int = MAX_TOPK, per_group: bool = False) -> int:
    lib = load_library()
    fn = lib.sa_indexer_topk_grouped_workspace_size if per_group else lib.sa_indexer_topk_workspace_size
    return int(fn(n_tok, max_pages_per_seq, topk))


def resolve_num_splits(n_tok: int, max_blocks_per_token: int, num_splits: int = 0) -> int:
    return int(load_library().sa_resolve_num_splits(n_tok, max_blocks_per_token, num_splits))


def indexer_topk(q_idx, k_idx_cache, page_table, seq_lens, q_seq, q_pos, topk: int = MAX_TOPK,
                 sel_idx=None, workspace=None, stream=None):
    """Top-k historical blocks per query token (ascending, -1 padded): int32 [n_tok][topk].

    k_idx_cache is bf16, or one-byte OCP E4M3 keys (torch.float8_e4m3fn, or
    their codes as torch.uint8), which go to sa_indexer_topk_fp8. A q_idx of
    shape [n_tok][4][256] (one query per KV group) selects per group through
    sa_indexer_topk_grouped and returns int32 [n_tok][4][topk]."""
    lib = load_library()
    dev = q_idx.device
    n_tok = q_idx.shape[0]
    per_group = q_idx.dim() == 3
    _need(q_idx, "q_idx", torch.bfloat16, dev, (n_tok, G, DI) if per_group else (n_tok, DI))
    fp8 = k_idx_cache.dtype in (torch.uint8, torch.float8_e4m3fn)
    if fp8:
        k_idx_cache = k_idx_cache.view(torch.uint8)
    _need(k_idx_cache, "k_idx_cache", torch.uint8 if fp8 else torch.bfloat16, dev)
    if k_idx_cache.dim() != 3 or tuple(k_idx_cache.shape[1:]) != (8, DI):
        raise ValueError("k_idx_cache: expected [num_pages][8][256]")
    _need(q_seq, "q_seq", torch.int32, dev, (n_tok,))
    _need(q_pos, "q_pos", torch.int32, dev, (n_tok,))
    pd = _desc(page_table, seq_lens, k_idx_cache.shape[0])
    sel_shape = (n_tok, G, topk) if per_group else (n_tok, topk)
    if sel_idx is None:
        sel_idx = torch.empty(sel_shape, dtype=torch.int32, device=dev)
    _need(sel_idx, "sel_idx", torch.int32, dev, sel_shape)
    need = indexer_workspace_size(n_tok, pd.max_pages_per_seq, topk, per_group)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    tail = (pd, _ptr(q_seq), _ptr(q_pos), n_tok, topk, _ptr(sel_idx), _ptr(workspace), workspace.numel(),
            _stream(stream))
    if per_group:
        name = "sa_indexer_topk_grouped"
        st = lib.sa_indexer_topk_grouped(_ptr(q_idx), _ptr(k_idx_cache), FORMAT_FP8_E4M3 if fp8 else FORMAT_BF16,
                                         *tail)
    else:
        name = "sa_indexer_topk_fp8" if fp8 else "sa_indexer_topk"
        st = getattr(lib, name)(_ptr(q_idx), _ptr(k_idx_cache), *tail)
    _check(name, st)
    return sel_idx


NOALLOC_SCRATCH_BYTES = 64 << 20   # SA_NOALLOC_SCRATCH_BYTES


def indexer_topk_noalloc(q_idx, k_idx_cache, page_table, seq_lens, q_seq, q_pos, topk: int = MAX_TOPK,
                         sel_idx=None, stream=None):
    """sa_indexer_topk_noalloc: the bf16-key selection with the library's own
    per-GPU scratch array as workspace (no workspace argument). Pass sel_idx to
    allocate nothing at all; calls that overlap on one GPU race."""
    lib = load_library()
    dev = q_idx.device
    n_tok = q_idx.shape[0]
    _need(q_idx, "q_idx", torch.bfloat16, dev, (n_tok, DI))
    _need(k_idx_cache, "k_idx_cache", torch.bfloat16, dev)
    if k_idx_cache.dim() != 3 or tuple(k_idx_cache.shape[1:]) != (8, DI):
        raise ValueError("k_idx_cache: expected [num_pages][8][256]")
    _need(q_seq, "q_seq", torch.int32, dev, (n_tok,))
    _need(q_pos, "q_pos", torch.int32, dev, (n_tok,))
    pd = _desc(page_table, seq_lens, k_idx_cache.shape[0])
    if sel_idx is None:
        sel_idx = torch.empty((n_tok, topk), dtype=torch.int32, device=dev)
    _need(sel_idx, "sel_idx", torch.int32, dev, (n_tok, topk))
    st = lib.sa_indexer_topk_noalloc(_ptr(q_idx), _ptr(k_idx_cache), pd, _ptr(q_seq), _ptr(q_pos), n_tok, topk,
                                     _ptr(sel_idx), _stream(stream))
    _check("sa_indexer_topk_noalloc", st)
    return sel_idx


def _decode_buffers(n_tok, S, dev, out, out_lse, part_o, part_lse, want_out=True):
    if out is None and want_out:
        out = torch.empty((n_tok, H, D), dtype=torch.bfloat16, device=dev)
    if out_lse is None:
        out_lse = torch.empty((n_tok, H), dtype=torch.float32, device=dev)
    if S > 1:
        if part_o is None:
            part_o = torch.empty((n_tok, S, H, D), dtype=torch.float32, device=dev)
        if part_lse is None:
            part_lse = torch.empty((n_tok, S, H), dtype=torch.float32, device=dev)
        _need(part_o, "part_o", torch.float32, dev, (n_tok, S, H, D))
        _need(part_lse, "part_lse", torch.float32, dev, (n_tok, S, H))
    if out is not None:
        _need(out, "out", torch.bfloat16, dev, (n_tok, H, D))
    _need(out_lse, "out_lse", torch.float32, dev, (n_tok, H))
    return out, out_lse, part_o, part_lse


def merge_counters(n_tok: int, device) -> torch.Tensor:
    """A zeroed counter buffer for split decode calls that merge in the same
    launch (allocate once; every call leaves it zero)."""
    return torch.zeros((max(n_tok, 1), G), dtype=torch.int32, device=device)


def _counters(c, n_tok, dev):
    if c is None:
        return None
    _need(c, "merge_counters", torch.int32, dev)
    if c.dim() != 2 or c.shape[1] != G or c.shape[0] < n_tok:
        raise ValueError(f"merge_counters: expected [>= {n_tok}][{G}] int32")
    return _ptr(c)


def _is_fp8(t) -> bool:
    return t.dtype in (torch.uint8, torch.float8_e4m3fn)


def _check_attn_inputs(q, k_cache, v_cache, q_seq, q_pos, k_scale, v_scale):
    """Checks shapes and dtypes; returns (dev, n_tok, fp8, k_cache, v_cache).

    Caches are both bf16, or both one-byte E4M3 (float8_e4m3fn or uint8 codes,
    returned as uint8 views), which need k_scale and v_scale."""
    dev = q.device
    n_tok = q.shape[0]
    _need(q, "q", torch.bfloat16, dev, (n_tok, H, D))
    fp8 = _is_fp8(k_cache)
    if fp8 != _is_fp8(v_cache):
        raise ValueError("k_cache and v_cache must both be bf16 or both one-byte")
    if fp8:
        if k_scale is None or v_scale is None:
            raise ValueError("one-byte caches need k_scale and v_scale")
        k_cache, v_cache = k_cache.view(torch.uint8), v_cache.view(torch.uint8)
    elif k_scale is not None or v_scale is not None:
        raise ValueError("k_scale / v_scale apply to one-byte caches only")
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(c, name, torch.uint8 if fp8 else torch.bfloat16, dev)
        if c.dim() != 4 or tuple(c.shape[1:]) != (G, 8, 8 * D):
            raise ValueError(f"{name}: expected [num_pages][4][8][1536]")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache differ in shape")
    _need(q_seq, "q_seq", torch.int32, dev, (n_tok,))
    _need(q_pos, "q_pos", torch.int32, dev, (n_tok,))
    return dev, n_tok, fp8, k_cache, v_cache


def sparse_decode(q, k_cache, v_cache, page_table, seq_lens, q_seq, q_pos, sel_idx, softmax_scale: float,
                  num_splits: int = 0, out=None, out_lse=None, part_o=None, part_lse=None,
                  partials_only: bool = False, stream=None, k_scale: Optional[float] = None,
                  v_scale: Optional[float] = None, merge_counters=None):
    """Attention over selected + current blocks. Returns (out, out_lse) or, with
    partials_only, (part_o, part_lse) of the resolved number of splits. One-byte
    caches (with k_scale, v_scale) go to sa_sparse_decode_fp8kv. A sel_idx of
    shape [n_tok][4][topk] (one set per KV group) goes to sa_sparse_decode_grouped.
    merge_counters (int32 [>= n_tok][4], zero before first use, left zero) makes
    a split call merge in the same launch; without them the merge is a second
    launch."""
    lib = load_library()
    dev, n_tok, fp8, k_cache, v_cache = _check_attn_inputs(q, k_cache, v_cache, q_seq, q_pos, k_scale, v_scale)
    per_group = sel_idx.dim() == 3
    topk = sel_idx.shape[-1]
    _need(sel_idx, "sel_idx", torch.int32, dev, (n_tok, G, topk) if per_group else (n_tok, topk))
    pd = _desc(page_table, seq_lens, k_cache.shape[0])
    S = resolve_num_splits(n_tok, topk + 1, num_splits)
    out, out_lse, part_o, part_lse = _decode_buffers(n_tok, S, dev, out, out_lse, part_o, part_lse,
                                                     want_out=not partials_only)
    tail = (pd, _ptr(q_seq), _ptr(q_pos), _ptr(sel_idx), n_tok, topk, float(softmax_scale), int(num_splits),
            _ptr(part_o), _ptr(part_lse), _counters(merge_counters, n_tok, dev),
            None if partials_only else _ptr(out), _ptr(out_lse), _stream(stream))
    if per_group:
        name = "sa_sparse_decode_grouped"
        st = lib.sa_sparse_decode_grouped(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                          FORMAT_FP8_E4M3 if fp8 else FORMAT_BF16,
                                          float(k_scale) if fp8 else 1.0, float(v_scale) if fp8 else 1.0, *tail)
    elif fp8:
        name = "sa_sparse_decode_fp8kv"
        st = lib.sa_sparse_decode_fp8kv(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale), float(v_scale), *tail)
    else:
        name = "sa_sparse_decode"
        st = lib.sa_sparse_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), *tail)
    _check(name, st)
    return (part_o, part_lse) if partials_only else (out, out_lse)


def swa_decode(q, k_cache, v_cache, page_table, seq_lens, q_seq, q_pos, window: int, softmax_scale: float,
               num_splits: int = 0, out=None, out_lse=None, part_o=None, part_lse=None,
               partials_only: bool = False, stream=None, k_scale: Optional[float] = None,
               v_scale: Optional[float] = None, merge_counters=None):
    """Sliding-window attention over positions max(0, p - window + 1) .. p.
    One-byte caches (with k_scale, v_scale) go to sa_swa_decode_fp8kv."""
    lib = load_library()
    dev, n_tok, fp8, k_cache, v_cache = _check_attn_inputs(q, k_cache, v_cache, q_seq, q_pos, k_scale, v_scale)
    pd = _desc(page_table, seq_lens, k_cache.shape[0])
    S = resolve_num_splits(n_tok, window // 8 + 2, num_splits)
    out, out_lse, part_o, part_lse = _decode_buffers(n_tok, S, dev, out, out_lse, part_o, part_lse,
                                                     want_out=not partials_only)
    tail = (pd, _ptr(q_seq), _ptr(q_pos), n_tok, int(window), float(softmax_scale), int(num_splits), _ptr(part_o),
            _ptr(part_lse), _counters(merge_counters, n_tok, dev), None if partials_only else _ptr(out),
            _ptr(out_lse), _stream(stream))
    if fp8:
        name = "sa_swa_decode_fp8kv"
        st = lib.sa_swa_decode_fp8kv(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale), float(v_scale), *tail)
    else:
        name = "sa_swa_decode"
        st = lib.sa_swa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), *tail)
    _check(name, st)
    return (part_o, part_lse) if partials_only else (out, out_lse)


def merge(part_o, part_lse, out=None, out_lse=None, stream=None):
    """Merge [n_tok][S][heads][dim] partial outputs into bf16 [n_tok][heads][dim] and lse."""
    lib = load_library()
    dev = part_o.device
    n_tok, S, nh, dh = part_o.shape
    _need(part_o, "part_o", torch.float32, dev)
    _need(part_lse, "part_lse", torch.float32, dev, (n_tok, S, nh))
    if out is None:
        out = torch.empty((n_tok, nh, dh), dtype=torch.bfloat16, device=dev)
    if out_lse is None:
        out_lse = torch.empty((n_tok, nh), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, dev, (n_tok, nh, dh))
    _need(out_lse, "out_lse", torch.float32, dev, (n_tok, nh))
    st = lib.sa_merge(_ptr(part_o), _ptr(part_lse), n_tok, S, nh, dh, _ptr(out), _ptr(out_lse), _stream(stream))
    _check("sa_merge", st)
    return out, out_lse


def sparse_layer(q, q_idx, k_cache, v_cache, k_idx_cache, page_table, seq_lens, q_seq, q_pos,
                 softmax_scale: float, topk: int = MAX_TOPK, num_splits: int = 0, workspace=None, stream=None,
                 k_scale: Optional[float] = None, v_scale: Optional[float] = None, merge_counters=None):
    """The sparse layer's whole decode step: indexer top-k, then attention (+ merge)."""
    sel = indexer_topk(q_idx, k_idx_cache, page_table, seq_lens, q_seq, q_pos, topk, workspace=workspace,
                       stream=stream)
    out, lse = sparse_decode(q, k_cache, v_cache, page_table, seq_lens, q_seq, q_pos, sel, softmax_scale,
                             num_splits=num_splits, stream=stream, k_scale=k_scale, v_scale=v_scale,
                             merge_counters=merge_counters)
    return sel, out, lse
