"""The C ABI on the host: the library loads, exports every function the header
declares, and rejects bad arguments with the documented status before touching
the device (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")


@pytest.fixture(scope="module")
def lib():
    from sparse_block_indexed_amd import ops
    if not os.path.exists(ops.LIB_PATH):
        from sparse_block_indexed_amd import build
        build.build()
    return ops.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ["sa_indexer_topk", "sa_indexer_topk_fp8", "sa_sparse_decode", "sa_sparse_decode_fp8kv",
              "sa_swa_decode", "sa_swa_decode_fp8kv", "sa_merge", "sa_indexer_topk_workspace_size",
              "sa_status_string", "sa_resolve_num_splits", "sa_indexer_topk_grouped",
              "sa_indexer_topk_grouped_workspace_size", "sa_sparse_decode_grouped"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    from sparse_block_indexed_amd import ops
    assert lib.sa_status_string(ops.SA_OK) == b"SA_OK"
    assert lib.sa_status_string(ops.SA_ERR_WORKSPACE) == b"SA_ERR_WORKSPACE"
    assert lib.sa_status_string(99) == b"SA_ERR_UNKNOWN"


def test_workspace_size(lib):
    assert lib.sa_indexer_topk_workspace_size(0, 16, 512) == 0
    a = lib.sa_indexer_topk_workspace_size(1, 128, 512)
    b = lib.sa_indexer_topk_workspace_size(2, 128, 512)
    c = lib.sa_indexer_topk_workspace_size(2, 256, 512)
    assert 0 < a < b < c
    assert a % 256 == 0
    # per token: scores (4 B per historical block)
    assert a >= 128 * 8 * 4
    # histories over 16,384 blocks also hold, per token, one (count, edge) pair
    # per chunk of at least 64 blocks and candidate lists (8 B per entry) for
    # every chunk length the host may pick: up to 512 entries per chunk, at most the chunk
    blocks = 16384 * 8
    lists = max(-(-blocks // c) * min(c, 512) for c in (64, 128, 256, 512, 1024, 2048))
    assert lists == blocks
    assert lib.sa_indexer_topk_workspace_size(1, 16384, 512) >= blocks * 4 + (blocks // 64) * 8 + lists * 8
    # the 128K verify batch fits the no-alloc entry point's scratch array
    assert lib.sa_indexer_topk_workspace_size(256, 2048, 512) <= 64 << 20


def test_resolve_num_splits(lib):
    r = lib.sa_resolve_num_splits
    fill, by_len = -1, 0
    # fill the GPU: follows the call's size
    assert r(256, 513, fill) == 1       # 128K verify batch: the grid already fills the GPU
    assert r(1, 513, fill) == 32        # one token: 129 chunks over 32 partitions (1 chunk per wave)
    assert r(64, 66, fill) == 1         # sliding window, batch 64: one workgroup per (token, group)
    assert r(4, 513, fill) == 16
    assert r(16, 513, fill) == 4        # the grid reaches 256 workgroups first
    assert r(1, 66, fill) == 4          # one-token window: 17 chunks
    assert r(1, 1, fill) == 1           # nothing to split
    # by length: one partition per 128 blocks of the longest list, whatever the call's size
    for n in (1, 4, 64, 256, 100000):
        assert r(n, 513, by_len) == 5
        assert r(n, 66, by_len) == 1
        assert r(n, 514, by_len) == 5
        assert r(n, 4096 // 8 + 2, by_len) == 5
    assert r(1, 128, by_len) == 1 and r(1, 129, by_len) == 2
    assert r(3, 513, 7) == 7            # explicit value kept
    assert r(3, 513, 1000) == 64        # clamped
    assert r(3, 513, -5) == 1           # not a request: one partition


def _desc(ops, batch=1, max_pages=16, num_pages=16, pt=0x1000, sl=0x2000):
    return ops.PagedDesc(pt, sl, batch, max_pages, num_pages)


P = 0x10000          # an aligned fake device address; never dereferenced by these calls


def test_indexer_topk_validation(lib):
    from sparse_block_indexed_amd import ops
    d = _desc(ops)
    ws = lib.sa_indexer_topk_workspace_size(4, 16, 512)
    f = lib.sa_indexer_topk
    assert f(None, None, d, None, None, 0, 512, None, None, 0, None) == ops.SA_OK           # n_tok = 0: no-op
    assert f(P, P, d, P, P, -1, 512, P, P, ws, None) == ops.SA_ERR_INVALID_ARG
    assert f(None, P, d, P, P, 4, 512, P, P, ws, None) == ops.SA_ERR_INVALID_ARG
    assert f(P, P, d, P, None, 4, 512, P, P, ws, None) == ops.SA_ERR_INVALID_ARG
    assert f(P, P, d, P, P, 4, 512, P, None, ws, None) == ops.SA_ERR_INVALID_ARG
    assert f(P + 8, P, d, P, P, 4, 512, P, P, ws, None) == ops.SA_ERR_INVALID_ARG         # misaligned
    assert f(P, P, d, P, P, 4, 512, P, P + 16, ws, None) == ops.SA_ERR_INVALID_ARG        # workspace alignment
    assert f(P, P, d, P, P, 4, 0, P, P, ws, None) == ops.SA_ERR_UNSUPPORTED
    assert f(P, P, d, P, P, 4, 513, P, P, ws, None) == ops.SA_ERR_UNSUPPORTED
    assert f(P, P, d, P, P, 4, 512, P, P, ws - 1, None) == ops.SA_ERR_WORKSPACE
    assert f(P, P, _desc(ops, batch=0), P, P, 4, 512, P, P, ws, None) == ops.SA_ERR_INVALID_ARG
    assert f(P, P, _desc(ops, pt=0), P, P, 4, 512, P, P, ws, None) == ops.SA_ERR_INVALID_ARG
    assert f(P, P, _desc(ops, num_pages=1 << 26), P, P, 4, 512, P, P, ws, None) == ops.SA_ERR_UNSUPPORTED
    f8 = lib.sa_indexer_topk_fp8
    assert f8(None, None, d, None, None, 0, 512, None, None, 0, None) == ops.SA_OK
    assert f8(P, None, d, P, P, 4, 512, P, P, ws, None) == ops.SA_ERR_INVALID_ARG
    assert f8(P, P, d, P, P, 4, 600, P, P, ws, None) == ops.SA_ERR_UNSUPPORTED
    assert f8(P, P, d, P, P, 4, 512, P, P, ws - 1, None) == ops.SA_ERR_WORKSPACE


def test_sparse_decode_validation(lib):
    from sparse_block_indexed_amd import ops
    d = _desc(ops)
    f = lib.sa_sparse_decode
    ok = dict(q=P, k=P, v=P, qs=P, qp=P, sel=P, n=4, topk=512, sc=0.07, S=1, po=None, pl=None, ctr=None, out=P,
              ol=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], d, a["qs"], a["qp"], a["sel"], a["n"], a["topk"], ctypes.c_float(a["sc"]),
                 a["S"], a["po"], a["pl"], a["ctr"], a["out"], a["ol"], None)

    assert call(n=0, q=None, k=None, v=None, sel=None, out=None) == ops.SA_OK
    assert call(n=-1) == ops.SA_ERR_INVALID_ARG
    assert call(q=None) == ops.SA_ERR_INVALID_ARG
    assert call(sel=None) == ops.SA_ERR_INVALID_ARG
    assert call(topk=0) == ops.SA_ERR_UNSUPPORTED
    assert call(topk=600) == ops.SA_ERR_UNSUPPORTED
    assert call(sc=float("nan")) == ops.SA_ERR_INVALID_ARG
    assert call(S=-2) == ops.SA_ERR_INVALID_ARG                        # below SA_SPLITS_FILL_GPU
    assert call(S=-1, po=None, pl=None) == ops.SA_ERR_INVALID_ARG     # fill the GPU: 16 partitions need partials
    assert call(S=65) == ops.SA_ERR_UNSUPPORTED
    assert call(out=None) == ops.SA_ERR_INVALID_ARG                    # S == 1 needs out
    assert call(S=4, po=None, pl=P) == ops.SA_ERR_INVALID_ARG         # S > 1 needs partials
    assert call(k=P + 4) == ops.SA_ERR_INVALID_ARG                     # misaligned cache
    assert call(S=4, po=P, pl=P, ctr=P + 2) == ops.SA_ERR_INVALID_ARG  # misaligned merge counters


def test_fp8kv_decode_validation(lib):
    """The one-byte K/V entry points check what the bf16 ones check, plus the scales."""
    from sparse_block_indexed_amd import ops
    d = _desc(ops)
    f = lib.sa_sparse_decode_fp8kv
    ok = dict(q=P, k=P, v=P, ks=0.03, vs=0.06, qs=P, qp=P, sel=P, n=4, topk=512, sc=0.07, S=1, out=P)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], ctypes.c_float(a["ks"]), ctypes.c_float(a["vs"]), d, a["qs"], a["qp"],
                 a["sel"], a["n"], a["topk"], ctypes.c_float(a["sc"]), a["S"], None, None, None, a["out"], None,
                 None)

    assert call(n=0, q=None, k=None, v=None, sel=None, out=None) == ops.SA_OK
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert call(ks=bad) == ops.SA_ERR_INVALID_ARG
        assert call(vs=bad) == ops.SA_ERR_INVALID_ARG
    assert call(ks=1e30, sc=1e30) == ops.SA_ERR_INVALID_ARG          # logit scale overflows fp32
    assert call(sel=None) == ops.SA_ERR_INVALID_ARG
    assert call(topk=513) == ops.SA_ERR_UNSUPPORTED
    assert call(v=P + 8) == ops.SA_ERR_INVALID_ARG
    w = lib.sa_swa_decode_fp8kv
    assert w(P, P, P, ctypes.c_float(1.0), ctypes.c_float(1.0), d, P, P, 0, 512, ctypes.c_float(0.1), 0,
             None, None, None, None, None, None) == ops.SA_OK
    assert w(P, P, P, ctypes.c_float(1.0), ctypes.c_float(0.0), d, P, P, 2, 512, ctypes.c_float(0.1), 1,
             None, None, None, P, None, None) == ops.SA_ERR_INVALID_ARG
    assert w(P, P, P, ctypes.c_float(1.0), ctypes.c_float(1.0), d, P, P, 2, 0, ctypes.c_float(0.1), 1,
             None, None, None, P, None, None) == ops.SA_ERR_UNSUPPORTED


def test_binding_checks_fp8_cache_arguments():
    """The Python binding refuses mixed cache dtypes and missing scales before any call."""
    import torch
    from sparse_block_indexed_amd import ops
    q = torch.zeros(1, 64, 192, dtype=torch.bfloat16)
    k8 = torch.zeros(1, 4, 8, 1536, dtype=torch.uint8)
    kb = torch.zeros(1, 4, 8, 1536, dtype=torch.bfloat16)
    i = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="both"):
        ops._check_attn_inputs(q, k8, kb, i, i, 1.0, 1.0)
    with pytest.raises(ValueError, match="need k_scale"):
        ops._check_attn_inputs(q, k8, k8, i, i, None, 1.0)
    with pytest.raises(ValueError, match="one-byte caches only"):
        ops._check_attn_inputs(q, kb, kb, i, i, 1.0, None)
    dev, n, fp8, k, v = ops._check_attn_inputs(q, k8.view(torch.float8_e4m3fn), k8, i, i, 0.5, 0.25)
    assert fp8 and n == 1 and k.dtype == torch.uint8 and v.dtype == torch.uint8


def test_grouped_entry_points_validation(lib):
    """Per-KV-group selection: the workspace covers 4 query rows per token; bad
    formats, sizes and buffers are refused before any launch."""
    from sparse_block_indexed_amd import ops
    d = _desc(ops)
    assert lib.sa_indexer_topk_grouped_workspace_size(3, 16, 512) == lib.sa_indexer_topk_workspace_size(12, 16, 512)
    assert lib.sa_indexer_topk_grouped_workspace_size(0, 16, 512) == 0
    assert lib.sa_indexer_topk_grouped_workspace_size(1 << 29, 16, 512) == 0
    ws = lib.sa_indexer_topk_grouped_workspace_size(4, 16, 512)
    f = lib.sa_indexer_topk_grouped
    assert f(None, None, 0, d, None, None, 0, 512, None, None, 0, None) == ops.SA_OK
    assert f(P, P, 2, d, P, P, 4, 512, P, P, ws, None) == ops.SA_ERR_UNSUPPORTED           # key format
    assert f(P, P, -1, d, P, P, 4, 512, P, P, ws, None) == ops.SA_ERR_UNSUPPORTED
    assert f(P, P, 0, d, P, P, 4, 512, P, P, ws - 1, None) == ops.SA_ERR_WORKSPACE
    assert f(P, P, 1, d, P, P, 4, 512, P, P, lib.sa_indexer_topk_workspace_size(4, 16, 512), None) \
        == ops.SA_ERR_WORKSPACE                                                            # per-token size is short
    assert f(P, P, 0, d, P, P, 4, 0, P, P, ws, None) == ops.SA_ERR_UNSUPPORTED
    assert f(P, P, 0, d, P, P, 1 << 29, 512, P, P, ws, None) == ops.SA_ERR_UNSUPPORTED
    assert f(P, None, 0, d, P, P, 4, 512, P, P, ws, None) == ops.SA_ERR_INVALID_ARG
    g = lib.sa_sparse_decode_grouped
    one = ctypes.c_float(1.0)

    def call(fmt=0, ks=one, vs=one, sel=P, n=4, topk=512, out=P):
        return g(P, P, P, fmt, ks, vs, d, P, P, sel, n, topk, ctypes.c_float(0.07), 1, None, None, None, out, None,
                 None)

    assert g(None, None, None, 0, one, one, d, None, None, None, 0, 512, ctypes.c_float(0.07), 0, None, None,
             None, None, None, None) == ops.SA_OK
    assert call(fmt=3) == ops.SA_ERR_UNSUPPORTED
    assert call(sel=None) == ops.SA_ERR_INVALID_ARG
    assert call(topk=513) == ops.SA_ERR_UNSUPPORTED
    assert call(fmt=1, vs=ctypes.c_float(0.0)) == ops.SA_ERR_INVALID_ARG                  # fp8 checks its scales
    assert call(n=1 << 29) == ops.SA_ERR_UNSUPPORTED
    assert call(out=None) == ops.SA_ERR_INVALID_ARG


def test_grid_limits_are_refused(lib):
    """Calls whose grids would reach 2^32 threads are refused before any launch."""
    from sparse_block_indexed_amd import ops
    d = _desc(ops)
    huge_ws = ctypes.c_size_t(1 << 62)
    assert lib.sa_indexer_topk(P, P, d, P, P, 1 << 23, 512, P, P, huge_ws, None) == ops.SA_ERR_UNSUPPORTED
    long_d = _desc(ops, max_pages=1 << 20, num_pages=1 << 20)                  # 8M-block histories
    assert lib.sa_indexer_topk(P, P, long_d, P, P, 1 << 16, 512, P, P, huge_ws, None) == ops.SA_ERR_UNSUPPORTED
    f = lib.sa_sparse_decode
    assert f(P, P, P, d, P, P, P, 1 << 22, 512, ctypes.c_float(0.1), 1, None, None, None, P, None, None) \
        == ops.SA_ERR_UNSUPPORTED                                               # 2^22 tokens x 4 groups x 256
    assert f(P, P, P, d, P, P, P, 1 << 18, 512, ctypes.c_float(0.1), 2, P, P, None, P, None, None) \
        == ops.SA_ERR_UNSUPPORTED                                               # the merge: 2^18 x 64 heads x 256
    assert lib.sa_merge(P, P, 1 << 18, 2, 64, 192, P, None, None) == ops.SA_ERR_UNSUPPORTED


def test_swa_and_merge_validation(lib):
    from sparse_block_indexed_amd import ops
    d = _desc(ops)
    f = lib.sa_swa_decode
    assert f(P, P, P, d, P, P, 0, 512, ctypes.c_float(0.1), 0, None, None, None, None, None, None) == ops.SA_OK
    assert f(P, P, P, d, P, P, 2, 0, ctypes.c_float(0.1), 1, None, None, None, P, None, None) == ops.SA_ERR_UNSUPPORTED
    assert f(P, P, P, d, P, P, 2, 5000, ctypes.c_float(0.1), 1, None, None, None, P, None, None) \
        == ops.SA_ERR_UNSUPPORTED
    m = lib.sa_merge
    assert m(None, None, 0, 1, 64, 192, None, None, None) == ops.SA_OK
    assert m(P, P, 2, 0, 64, 192, P, None, None) == ops.SA_ERR_INVALID_ARG
    assert m(P, P, 2, 65, 64, 192, P, None, None) == ops.SA_ERR_UNSUPPORTED
    assert m(P, P, 2, 4, 64, 190, P, None, None) == ops.SA_ERR_UNSUPPORTED
    assert m(None, P, 2, 4, 64, 192, P, None, None) == ops.SA_ERR_INVALID_ARG


def test_product_path_refuses_to_run_without_the_library(tmp_path):
    from sparse_block_indexed_amd import ops
    saved = ops._lib
    ops._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            ops.load_library(str(tmp_path / "libsa.so"))
    finally:
        ops._lib = saved


def test_product_path_does_not_import_the_oracle():
    import subprocess
    import sys
    code = ("import sys; import sparse_block_indexed_amd.ops, sparse_block_indexed_amd.bytes_model, "
            "sparse_block_indexed_amd.inputs; print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "False"
