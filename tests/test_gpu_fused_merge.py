"""Split decode calls that merge in the same launch (merge_counters given): the
last partition of each (token, KV group) to finish merges the partials in
partition order with the merge kernel's arithmetic, so the results must equal
the two-launch path (partials, then sa_merge) bit for bit, and the counters
must be back at zero after every call. Covered: the sparse and window layers,
one-byte KV, per-group selection, three split counts, two calls in a row, graph
replays, and the 1M and 8K workloads in the benchmark's configuration."""
import numpy as np
import pytest
import torch

from sparse_block_indexed_amd import inputs as I

from gpu_helpers import (SCALE, SPLITS_FILL_GPU, OracleView, assert_close_outputs, bf16_to_np, device_tables)

pytestmark = pytest.mark.gpu

SMALL = I.WorkloadSpec("small_mixed", batch=12, seq_lens=[1, 7, 8, 9, 63, 64, 65, 300, 1000, 4103, 4111, 9000],
                       q_per_seq=3, spare_pages=5)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_block_indexed_amd import ops
    ops.load_library()


def _say(msg):
    print(msg, flush=True)


def _both(fn, n_tok, **kw):
    """fn(merge_counters=...) twice with counters (fresh output buffers) and once without."""
    from sparse_block_indexed_amd import ops
    ctr = ops.merge_counters(n_tok, "cuda")
    a = fn(merge_counters=ctr, **kw)
    b = fn(merge_counters=ctr, **kw)
    ref = fn(merge_counters=None, **kw)
    torch.cuda.synchronize()
    assert (ctr == 0).all(), "counters not back at zero"
    return a, b, ref


@pytest.mark.parametrize("S", [2, 5, 32])
@pytest.mark.parametrize("layer", ["sparse", "window", "sparse_fp8kv", "window_fp8kv", "sparse_grouped"])
def test_fused_merge_equals_merge_launch(S, layer):
    _say(f"fused merge {layer} S={S}")
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(SMALL, seed=91, device="cuda")
    pt, sl, qs, qp = device_tables(wl)
    kv = {}
    kc, vc = wl.k_cache, wl.v_cache
    if "fp8" in layer:
        kc, vc = I.quantize_kv_fp8(wl.k_cache, wl.v_cache, 1 / 32, 1 / 16)
        kv = dict(k_scale=1 / 32, v_scale=1 / 16)
    if layer.startswith("sparse"):
        qidx = I.grouped_index_queries(wl.n_tok, seed=92, device="cuda") if "grouped" in layer else wl.q_idx
        sel = ops.indexer_topk(qidx, wl.k_idx_cache, pt, sl, qs, qp, 512)

        def fn(merge_counters):
            return ops.sparse_decode(wl.q, kc, vc, pt, sl, qs, qp, sel, SCALE, num_splits=S,
                                     merge_counters=merge_counters, **kv)
    else:
        def fn(merge_counters):
            return ops.swa_decode(wl.q, kc, vc, pt, sl, qs, qp, 512, SCALE, num_splits=S,
                                  merge_counters=merge_counters, **kv)
    a, b, ref = _both(fn, wl.n_tok)
    for got in (a, b):
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    if layer == "sparse":   # and against the oracle
        ov = OracleView(wl)
        sel_h = sel.cpu().numpy()
        refs = [ov.sparse(t, sel_h[t]) for t in range(wl.n_tok)]
        assert_close_outputs(bf16_to_np(a[0]), a[1].cpu().numpy(), np.stack([r[0] for r in refs]),
                             np.stack([r[1] for r in refs]), f"fused S={S}")


@pytest.mark.parametrize("name", ["decode_8k_b1", "decode_1m_b4", "swa_decode_32k_b64"])
def test_fused_merge_on_the_workloads(name):
    """The benchmark's configuration (partitions filling the GPU) with the merge
    in the same launch: equal to the two-launch path, and to the oracle."""
    _say(f"fused merge {name}")
    from sparse_block_indexed_amd import ops
    wl = I.named_workload(name, device="cuda")
    pt, sl, qs, qp = device_tables(wl)
    if name.startswith("swa"):
        def fn(merge_counters):
            return ops.swa_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, 512, SCALE, num_splits=SPLITS_FILL_GPU,
                                  merge_counters=merge_counters)
        sel = None
    else:
        sel = ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512)

        def fn(merge_counters):
            return ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel, SCALE,
                                     num_splits=SPLITS_FILL_GPU, merge_counters=merge_counters)
    a, b, ref = _both(fn, wl.n_tok)
    assert torch.equal(a[0], ref[0]) and torch.equal(a[1], ref[1]) and torch.equal(b[0], ref[0])
    ov = OracleView(wl)
    toks = list(range(wl.n_tok)) if wl.n_tok <= 8 else list(range(0, wl.n_tok, 9))
    if sel is None:
        refs = [ov.swa(t) for t in toks]
    else:
        sel_h = sel.cpu().numpy()
        refs = [ov.sparse(t, sel_h[t]) for t in toks]
    assert_close_outputs(bf16_to_np(a[0][toks]), a[1][toks].cpu().numpy(), np.stack([r[0] for r in refs]),
                         np.stack([r[1] for r in refs]), name)


def test_fused_merge_graph_replays():
    """A captured step whose split calls merge in the same launch: each replay
    (eager work in between) equals the eager result, and the counters stay zero."""
    _say("fused merge under graph capture")
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(SMALL, seed=93, device="cuda")
    pt, sl, qs, qp = device_tables(wl)
    n = wl.n_tok
    S = 4
    ctr = ops.merge_counters(n, "cuda")
    sel = torch.empty((n, 512), dtype=torch.int32, device="cuda")
    ws = torch.zeros(ops.indexer_workspace_size(n, wl.max_pages_per_seq, 512), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    po, pl = torch.empty((n, S, 64, 192), **f32), torch.empty((n, S, 64), **f32)
    out = torch.empty((n, 64, 192), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((n, 64), **f32)
    wout, wlse = torch.empty_like(out), torch.empty_like(lse)

    def step():
        ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512, sel_idx=sel, workspace=ws)
        ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel, SCALE, num_splits=S, out=out,
                          out_lse=lse, part_o=po, part_lse=pl, merge_counters=ctr)
        ops.swa_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, 512, SCALE, num_splits=S, out=wout,
                       out_lse=wlse, part_o=po, part_lse=pl, merge_counters=ctr)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (sel, out, lse, wout, wlse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for t in (out, lse, wout, wlse):
            t.fill_(float("nan"))
        ops.swa_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, 64, SCALE)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((sel, out, lse, wout, wlse), ref):
            assert torch.equal(got, want), f"replay {r}"
        assert (ctr == 0).all()
