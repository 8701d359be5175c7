"""The library's calls under HIP graph capture: a captured step replayed several
times, with eager work and synchronisations between the replays, must give
bitwise the results of the same calls run eagerly (every kernel is
deterministic and the inputs do not change). The library enqueues kernels
only: no allocation, no memset, no synchronisation inside a call.
"""
import math

import numpy as np
import pytest
import torch

from sparse_block_indexed_amd import inputs as I

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(192.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_block_indexed_amd import ops
    ops.load_library()


def _say(msg):
    print(msg, flush=True)


class _Step:
    """Preallocated buffers and the calls of one step (sparse layer + window layer)."""

    def __init__(self, wl, num_splits, fp8_kv=False):
        from sparse_block_indexed_amd import ops
        self.ops = ops
        self.wl = wl
        dev = wl.q.device
        self.tabs = wl.device_ints(dev)
        n = wl.n_tok
        if fp8_kv:
            kc, vc = I.quantize_kv_fp8(wl.k_cache, wl.v_cache, 1 / 32, 1 / 16)
            self.kv = (kc, vc, dict(k_scale=1 / 32, v_scale=1 / 16))
        else:
            self.kv = (wl.k_cache, wl.v_cache, {})
        self.S = ops.resolve_num_splits(n, 513, num_splits)
        self.Sw = ops.resolve_num_splits(n, 512 // 8 + 2, num_splits)
        self.num_splits = num_splits
        self.sel = torch.empty((n, 512), dtype=torch.int32, device=dev)
        self.ws = torch.empty(ops.indexer_workspace_size(n, wl.max_pages_per_seq, 512), dtype=torch.uint8,
                              device=dev)
        mk = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
        self.out = torch.empty((n, 64, 192), dtype=torch.bfloat16, device=dev)
        self.lse = mk(n, 64)
        self.po = mk(n, self.S, 64, 192) if self.S > 1 else None
        self.pl = mk(n, self.S, 64) if self.S > 1 else None
        self.wout = torch.empty_like(self.out)
        self.wlse = mk(n, 64)
        self.wpo = mk(n, self.Sw, 64, 192) if self.Sw > 1 else None
        self.wpl = mk(n, self.Sw, 64) if self.Sw > 1 else None

    def run(self):
        ops, wl = self.ops, self.wl
        pt, sl, qs, qp = self.tabs
        kc, vc, kw = self.kv
        ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512, sel_idx=self.sel, workspace=self.ws)
        ops.sparse_decode(wl.q, kc, vc, pt, sl, qs, qp, self.sel, SCALE, num_splits=self.num_splits, out=self.out,
                          out_lse=self.lse, part_o=self.po, part_lse=self.pl, **kw)
        ops.swa_decode(wl.q, kc, vc, pt, sl, qs, qp, 512, SCALE, num_splits=self.num_splits, out=self.wout,
                       out_lse=self.wlse, part_o=self.wpo, part_lse=self.wpl, **kw)

    def outputs(self):
        return [self.sel, self.out, self.lse, self.wout, self.wlse]

    def poison(self):
        self.sel.fill_(-7)
        for t in (self.out, self.lse, self.wout, self.wlse):
            t.fill_(float("nan"))


def _graph_vs_eager(wl, num_splits, fp8_kv=False, replays=3):
    step = _Step(wl, num_splits, fp8_kv)
    step.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in step.outputs()]
    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    torch.cuda.synchronize()
    other = _Step(wl, num_splits, fp8_kv)
    for r in range(replays):
        step.poison()
        other.run()                       # eager work of the program between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(["sel", "out", "lse", "swa out", "swa lse"], step.outputs(), ref):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager result"
    for got, want in zip(other.outputs(), ref):
        assert torch.equal(got, want)


SMALL = I.WorkloadSpec("small_mixed", batch=12,
                       seq_lens=[1, 7, 8, 9, 63, 64, 65, 300, 1000, 4103, 4111, 9000],
                       q_per_seq=3, spare_pages=5)


@pytest.mark.parametrize("num_splits,fp8_kv", [(1, False), (3, False), (0, True), (0, False), (-1, False)])
def test_small_step_graph_replays_match_eager(num_splits, fp8_kv):
    _say(f"graph small S={num_splits} fp8_kv={fp8_kv}")
    wl = I.make_workload(SMALL, seed=71, device="cuda")
    _graph_vs_eager(wl, num_splits, fp8_kv)


def test_long_history_step_graph_replays_match_eager():
    """Histories past the finalize limit (candidate lists in the score pass + the select launch) under capture."""
    _say("graph long history")
    wl = I.make_workload(I.WorkloadSpec("long", batch=2, seq_lens=[200000, 30000], q_per_seq=2), seed=72,
                         device="cuda")
    _graph_vs_eager(wl, 0)


@pytest.mark.parametrize("q_per_seq", [20, 70])
def test_mfma_scorer_steps_graph_replays_match_eager(q_per_seq):
    """20 query tokens per sequence take the 16-row MFMA scorer and 70 the score
    GEMM (and cacheable K/V loads); both under capture."""
    _say(f"graph mfma scorers q_per_seq={q_per_seq}")
    wl = I.make_workload(I.WorkloadSpec("mfma_graph", batch=2, seq_lens=[5000, 9000], q_per_seq=q_per_seq),
                         seed=74, device="cuda")
    _graph_vs_eager(wl, 0)


def test_mtp_verify_step_graph_replays_match_eager():
    """The 128K MTP verify workload as the benchmark replays it."""
    _say("graph mtp_verify_128k_b64")
    wl = I.named_workload("mtp_verify_128k_b64", device="cuda")
    _graph_vs_eager(wl, -1, replays=2)


def test_calls_on_two_streams_at_once_match_eager():
    """The library keeps no global state: two steps with their own buffers and
    workspaces, enqueued on two streams (default priority) so that they can run
    at the same time, give bitwise the results of running them one by one."""
    _say("two streams")
    wa = I.make_workload(SMALL, seed=75, device="cuda")
    wb = I.make_workload(I.WorkloadSpec("long", batch=2, seq_lens=[200000, 30000], q_per_seq=2), seed=76,
                         device="cuda")
    sa, sb = _Step(wa, 3), _Step(wb, 0)
    sa.run()
    sb.run()
    torch.cuda.synchronize()
    ref_a = [t.clone() for t in sa.outputs()]
    ref_b = [t.clone() for t in sb.outputs()]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for r in range(3):
        sa.poison()
        sb.poison()
        torch.cuda.synchronize()
        for st, step in zip(streams, (sa, sb)):
            with torch.cuda.stream(st):
                step.run()
        torch.cuda.synchronize()
        for got, want in zip(sa.outputs() + sb.outputs(), ref_a + ref_b):
            assert torch.equal(got, want), f"round {r}"


def test_hybrid_layer_group_graph():
    """Three window layers and one sparse layer, each with its own Q and caches
    over the same sequences, captured as one graph: every replay equals each
    layer's own eager call bit for bit, and two layers agree with the oracle."""
    _say("graph hybrid layer group")
    from gpu_helpers import OracleView, assert_close_outputs, bf16_to_np
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(SMALL, seed=73, device="cuda")
    layers = [I.layer_inputs(wl, seed=500 + i) for i in range(3)] + [wl]
    pt, sl, qs, qp = wl.device_ints("cuda")
    n = wl.n_tok
    S = 2
    outs = [torch.empty((n, 64, 192), dtype=torch.bfloat16, device="cuda") for _ in layers]
    lses = [torch.empty((n, 64), dtype=torch.float32, device="cuda") for _ in layers]
    po = torch.empty((n, S, 64, 192), dtype=torch.float32, device="cuda")
    pl = torch.empty((n, S, 64), dtype=torch.float32, device="cuda")
    sel = torch.empty((n, 512), dtype=torch.int32, device="cuda")
    ws = torch.empty(ops.indexer_workspace_size(n, wl.max_pages_per_seq, 512), dtype=torch.uint8, device="cuda")

    def group():
        for i in range(3):
            L = layers[i]
            ops.swa_decode(L.q, L.k_cache, L.v_cache, pt, sl, qs, qp, 512, SCALE, num_splits=S, out=outs[i],
                           out_lse=lses[i], part_o=po, part_lse=pl)
        ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512, sel_idx=sel, workspace=ws)
        ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel, SCALE, num_splits=S, out=outs[3],
                          out_lse=lses[3], part_o=po, part_lse=pl)

    # each layer on its own, eagerly, into fresh buffers
    ref = []
    for i in range(3):
        L = layers[i]
        ref.append(ops.swa_decode(L.q, L.k_cache, L.v_cache, pt, sl, qs, qp, 512, SCALE, num_splits=S))
    ref_sel = ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512)
    ref.append(ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, ref_sel, SCALE, num_splits=S))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        group()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        group()
    for r in range(3):
        for t in outs + lses:
            t.fill_(float("nan"))
        ops.swa_decode(layers[1].q, layers[1].k_cache, layers[1].v_cache, pt, sl, qs, qp, 64, SCALE)   # eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, ref_sel)
        for i in range(4):
            assert torch.equal(outs[i], ref[i][0]) and torch.equal(lses[i], ref[i][1]), f"replay {r} layer {i}"
    # the layers really differ, and layer 1 (window) and layer 3 (sparse) match the oracle
    assert not torch.equal(outs[0], outs[1])
    ov1, ov3 = OracleView(layers[1]), OracleView(wl)
    toks = range(0, n, 5)
    r1 = [ov1.swa(t) for t in toks]
    assert_close_outputs(bf16_to_np(outs[1][list(toks)]), lses[1][list(toks)].cpu().numpy(),
                         np.stack([x[0] for x in r1]), np.stack([x[1] for x in r1]), "group window layer")
    sel_h = sel.cpu().numpy()
    r3 = [ov3.sparse(t, sel_h[t]) for t in toks]
    for t in toks:
        assert sel_h[t].tolist() == ov3.selection(t).tolist()
    assert_close_outputs(bf16_to_np(outs[3][list(toks)]), lses[3][list(toks)].cpu().numpy(),
                         np.stack([x[0] for x in r3]), np.stack([x[1] for x in r3]), "group sparse layer")
