"""sa_indexer_topk_noalloc (the indexer with the library's per-GPU scratch
array as workspace) through the C ABI against sa_indexer_topk with a caller
workspace: equal selections, bit for bit, on two calls in a row (the second one
smaller, so it runs on scratch holding the first call's contents), and the
oracle agrees on sampled tokens. A request larger than the array is refused."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_block_indexed_amd import inputs as I

from gpu_helpers import OracleView, device_tables

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(lib, ops, wl):
    pt, sl, qs, qp = device_tables(wl)
    n = wl.n_tok
    pd = ops.PagedDesc(pt.data_ptr(), sl.data_ptr(), pt.shape[0], pt.shape[1], wl.k_idx_cache.shape[0])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws_bytes = lib.sa_indexer_topk_workspace_size(n, pt.shape[1], 512)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ref = torch.full((n, 512), -7, dtype=torch.int32, device="cuda")
    got = torch.full((n, 512), -7, dtype=torch.int32, device="cuda")
    args = (ctypes.c_void_p(wl.q_idx.data_ptr()), ctypes.c_void_p(wl.k_idx_cache.data_ptr()), pd,
            ctypes.c_void_p(qs.data_ptr()), ctypes.c_void_p(qp.data_ptr()), n, 512)
    assert lib.sa_indexer_topk(*args, ctypes.c_void_p(ref.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws_bytes,
                               stream) == ops.SA_OK
    assert lib.sa_indexer_topk_noalloc(*args, ctypes.c_void_p(got.data_ptr()), stream) == ops.SA_OK
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_indexer_equals_workspace_indexer_on_two_calls():
    from sparse_block_indexed_amd import ops
    lib = ops.load_library()
    big = I.named_workload("mtp_verify_128k_b64", device="cuda")
    small = I.make_workload(I.WorkloadSpec("noalloc_small", batch=3, seq_lens=[9000, 300, 40000], q_per_seq=2),
                            seed=81, device="cuda")
    for wl in (big, small):
        print(f"no-alloc indexer: {wl.spec.name}, {wl.n_tok} tokens", flush=True)
        ref, got = _both(lib, ops, wl)
        assert torch.equal(got, ref), wl.spec.name
        ov = OracleView(wl)
        got_h = got.cpu().numpy()
        for t in sorted({0, wl.n_tok - 1, wl.n_tok // 2}):
            assert got_h[t].tolist() == ov.selection(t).tolist(), (wl.spec.name, t)
    # the binding's wrapper runs the same entry point
    pt, sl, qs, qp = device_tables(small)
    sel = ops.indexer_topk_noalloc(small.q_idx, small.k_idx_cache, pt, sl, qs, qp, 512)
    torch.cuda.synchronize()
    assert torch.equal(sel, got)


def test_noalloc_indexer_refuses_sizes_beyond_the_scratch_array():
    from sparse_block_indexed_amd import ops
    lib = ops.load_library()
    wl = I.make_workload(I.WorkloadSpec("noalloc_big", batch=1, seq_lens=[131072], q_per_seq=1), seed=82,
                         device="cuda")
    # 1,100 query rows of 131,072-token histories need more workspace than the array holds
    n = 1100
    q_idx = wl.q_idx.expand(n, -1).contiguous()
    qs = torch.zeros(n, dtype=torch.int32, device="cuda")
    qp = torch.full((n,), 131071, dtype=torch.int32, device="cuda")
    pt, sl, _, _ = device_tables(wl)
    assert lib.sa_indexer_topk_workspace_size(n, pt.shape[1], 512) > ops.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ops.SAError) as e:
        ops.indexer_topk_noalloc(q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512)
    assert e.value.status == ops.SA_ERR_WORKSPACE
