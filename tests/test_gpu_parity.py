"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded, device-resident inputs.

Selections must match bit for bit (index inputs are small integers, so scores
are exact). Outputs must be within max-abs 2e-2 and relative RMS 5e-3 of the
oracle, lse within 1e-3.
"""
import math

import numpy as np
import pytest
import torch

from oracle import sa_oracle as O
from sparse_block_indexed_amd import inputs as I

from gpu_helpers import (SCALE, SPLITS_FILL_GPU, OracleView, assert_close_outputs, bf16_to_np, device_tables,
                         run_sparse_layer, run_swa)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_block_indexed_amd import ops
    ops.load_library()


def _say(msg):
    print(msg, flush=True)


def _check_all(wl, sel, out, lse, tokens, topk=512, what=""):
    ov = OracleView(wl)
    sel_h = sel.cpu().numpy()
    outs, refs, lses, rlses = [], [], [], []
    for t in tokens:
        ref_sel = ov.selection(t, topk)
        assert sel_h[t].tolist() == ref_sel.tolist(), f"{what}: token {t} selection differs"
        ro, rl = ov.sparse(t, ref_sel)
        outs.append(bf16_to_np(out[t]))
        lses.append(lse[t].cpu().numpy())
        refs.append(ro)
        rlses.append(rl)
    return assert_close_outputs(np.stack(outs), np.stack(lses), np.stack(refs), np.stack(rlses), what)


# a mixed small batch: contexts around every block/page/top-k boundary, 3 verify tokens each
SMALL = I.WorkloadSpec("small_mixed", batch=12,
                       seq_lens=[1, 7, 8, 9, 63, 64, 65, 300, 1000, 4103, 4111, 9000],
                       q_per_seq=3, spare_pages=5)


@pytest.mark.parametrize("num_splits", [0, -1, 1, 3])
def test_small_mixed_sparse(num_splits):
    _say(f"small_mixed sparse S={num_splits}")
    wl = I.make_workload(SMALL, seed=11, device="cuda")
    sel, out, lse = run_sparse_layer(wl, num_splits=num_splits)
    _check_all(wl, sel, out, lse, range(wl.n_tok), what=f"small S={num_splits}")


@pytest.mark.parametrize("window,num_splits", [(512, 0), (512, -1), (512, 1), (64, 2), (1, 1), (4096, 0), (4096, -1)])
def test_small_mixed_swa(window, num_splits):
    _say(f"small_mixed swa W={window} S={num_splits}")
    wl = I.make_workload(SMALL, seed=12, device="cuda")
    out, lse = run_swa(wl, window=window, num_splits=num_splits)
    ov = OracleView(wl)
    refs = [ov.swa(t, window) for t in range(wl.n_tok)]
    assert_close_outputs(bf16_to_np(out), lse.cpu().numpy(), np.stack([r[0] for r in refs]),
                         np.stack([r[1] for r in refs]), f"swa W={window}")


@pytest.mark.parametrize("seed", range(4))
def test_random_window_calls(seed):
    """Seeded random window calls: 1-6 sequences of random lengths, 1-4 query
    tokens each, a window in 1 .. 4096 and any split setting; every token
    against the oracle."""
    from gpu_helpers import run_swa
    rng = np.random.default_rng(2000 + seed)
    batch = int(rng.integers(1, 7))
    lens = [int(rng.integers(1, 40000)) for _ in range(batch)]
    q = int(rng.integers(1, 5))
    window = int(rng.choice([1, int(rng.integers(2, 600)), 512, int(rng.integers(600, 4097))]))
    num_splits = int(rng.choice([0, -1, 1, 2, 5]))
    what = f"random window {seed}: lens {lens}, q {q}, window {window}, splits {num_splits}"
    _say(what)
    wl = I.make_workload(I.WorkloadSpec(f"rwin{seed}", batch=batch, seq_lens=lens, q_per_seq=q), seed=400 + seed,
                         device="cuda")
    out, lse = run_swa(wl, window=window, num_splits=num_splits)
    ov = OracleView(wl)
    refs = [ov.swa(t, window) for t in range(wl.n_tok)]
    assert_close_outputs(bf16_to_np(out), lse.cpu().numpy(), np.stack([r[0] for r in refs]),
                         np.stack([r[1] for r in refs]), what)


@pytest.mark.parametrize("topk", [1, 7, 100, 511])
def test_small_topk_values(topk):
    _say(f"topk={topk}")
    wl = I.make_workload(SMALL, seed=13, device="cuda")
    sel, out, lse = run_sparse_layer(wl, topk=topk)
    _check_all(wl, sel, out, lse, range(wl.n_tok), topk=topk, what=f"topk={topk}")


@pytest.mark.parametrize("topk", [1, 7, 100, 511])
def test_small_topk_values_on_long_histories(topk):
    """The candidate-list path (histories past 16,384 blocks, whose per-chunk
    budgets follow k) with small k, next to a short row of the same call."""
    _say(f"long histories, topk={topk}")
    spec = I.WorkloadSpec("long_topk", batch=3, seq_lens=[140000, 131080, 3000], q_per_seq=2)
    wl = I.make_workload(spec, seed=17, device="cuda")
    sel, out, lse = run_sparse_layer(wl, topk=topk)
    _check_all(wl, sel, out, lse, range(wl.n_tok), topk=topk, what=f"long topk={topk}")


@pytest.mark.parametrize("seed", range(8))
def test_random_calls(seed):
    """Seeded random calls: 1-5 sequences of random lengths (half of them with
    one history past 16,384 blocks, so that the candidate-list path runs), 1-4
    query tokens per sequence, k in {1, 16, 100, 512}, index values in [-4, 4],
    {0, 1} or [-1, 1] (ties), and any split setting; every token's selection and
    output against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    batch = int(rng.integers(1, 6))
    lens = [int(rng.integers(1, 20000)) for _ in range(batch)]
    if rng.random() < 0.5:
        lens[int(rng.integers(0, batch))] = int(rng.integers(131080, 180000))
    q = int(rng.integers(1, 5))
    topk = int(rng.choice([1, 16, 100, 512]))
    lo, hi = [(-4, 4), (0, 1), (-1, 1)][int(rng.integers(0, 3))]
    num_splits = int(rng.choice([0, -1, 1, 3]))
    what = f"random {seed}: lens {lens}, q {q}, k {topk}, idx [{lo}, {hi}], splits {num_splits}"
    _say(what)
    spec = I.WorkloadSpec(f"random{seed}", batch=batch, seq_lens=lens, q_per_seq=q, idx_lo=lo, idx_hi=hi)
    wl = I.make_workload(spec, seed=300 + seed, device="cuda")
    sel, out, lse = run_sparse_layer(wl, topk=topk, num_splits=num_splits)
    _check_all(wl, sel, out, lse, range(wl.n_tok), topk=topk, what=what)


# The five workloads run at full size in the launch configuration the benchmark
# times (partition count following the call's size).

def test_decode_8k_b1():
    _say("decode_8k_b1")
    wl = I.named_workload("decode_8k_b1", device="cuda")
    sel, out, lse = run_sparse_layer(wl, num_splits=SPLITS_FILL_GPU)
    _check_all(wl, sel, out, lse, range(wl.n_tok), what="decode_8k")


def test_mtp_verify_128k_b64():
    """The headline workload: every token's selection and every token's output."""
    _say("mtp_verify_128k_b64")
    wl = I.named_workload("mtp_verify_128k_b64", device="cuda")
    sel, out, lse = run_sparse_layer(wl, num_splits=SPLITS_FILL_GPU)
    _check_all(wl, sel, out, lse, range(wl.n_tok), what="mtp_verify_128k")


def test_swa_decode_32k_b64():
    _say("swa_decode_32k_b64")
    wl = I.named_workload("swa_decode_32k_b64", device="cuda")
    out, lse = run_swa(wl, num_splits=SPLITS_FILL_GPU)
    ov = OracleView(wl)
    refs = [ov.swa(t) for t in range(wl.n_tok)]
    assert_close_outputs(bf16_to_np(out), lse.cpu().numpy(), np.stack([r[0] for r in refs]),
                         np.stack([r[1] for r in refs]), "swa_32k")


def test_decode_1m_b4():
    _say("decode_1m_b4")
    wl = I.named_workload("decode_1m_b4", device="cuda")
    sel, out, lse = run_sparse_layer(wl, num_splits=SPLITS_FILL_GPU)
    _check_all(wl, sel, out, lse, range(wl.n_tok), what="decode_1m")


def test_prefill_chunk_16k_at_112k():
    """Every one of the 16,384 tokens' selections against the oracle (they share
    one sequence's keys, so the oracle's scores come from one fp64 product per
    batch of rows), and the outputs of 66 tokens spread over the chunk: the
    first and last token and one token of every 256 (a fourth of the score
    GEMM's 64-token tiles, in every position of the tile)."""
    _say("prefill_chunk_16k_at_112k")
    wl = I.named_workload("prefill_chunk_16k_at_112k", device="cuda")
    sel, out, lse = run_sparse_layer(wl, num_splits=SPLITS_FILL_GPU)
    ov = OracleView(wl)
    sel_h = sel.cpu().numpy()
    assert len(set(int(b) for b in wl.q_seq)) == 1
    cbs = np.asarray(wl.q_pos) // 8
    keys = ov.keys(int(wl.q_seq[0]), int(cbs.max()))
    qi = O.bf16_to_f64(I.bf16_bits(wl.q_idx))
    for t0 in range(0, wl.n_tok, 1024):
        scores = O.indexer_scores(qi[t0:t0 + 1024].T, keys)      # [blocks][rows]
        for j in range(scores.shape[1]):
            t = t0 + j
            ref = O.select_top_blocks(scores[:cbs[t], j], 512)
            assert sel_h[t].tolist() == ref.tolist(), f"prefill token {t} selection differs"
    sample = sorted({0, wl.n_tok - 1} | {256 * i + (37 * i) % 256 for i in range(wl.n_tok // 256)})
    assert len(sample) >= 64
    _check_all(wl, sel, out, lse, sample, what="prefill_chunk")


def test_verify_token_alone_equals_it_in_the_batch():
    """With num_splits = 0 a token's partition count follows its own list only:
    a verify token of the 128K workload run alone (one-token call) is bitwise
    what it is as one of 4 verify tokens in the batch-64 call, and so is the
    window layer. The selection is exact either way."""
    _say("batch invariance, headline token alone")
    from sparse_block_indexed_amd import ops
    wl = I.named_workload("mtp_verify_128k_b64", device="cuda")
    pt, sl, qs, qp = device_tables(wl)
    sel = ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512)
    out, lse = ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel, SCALE, num_splits=0)
    wout, wlse = ops.swa_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, 512, SCALE, num_splits=0)
    for t in (0, 1, 2, 3, 129, 255):
        one = slice(t, t + 1)
        sel1 = ops.indexer_topk(wl.q_idx[one], wl.k_idx_cache, pt, sl, qs[one], qp[one], 512)
        o1, l1 = ops.sparse_decode(wl.q[one], wl.k_cache, wl.v_cache, pt, sl, qs[one], qp[one], sel1, SCALE,
                                   num_splits=0)
        w1, wl1 = ops.swa_decode(wl.q[one], wl.k_cache, wl.v_cache, pt, sl, qs[one], qp[one], 512, SCALE,
                                 num_splits=0)
        torch.cuda.synchronize()
        assert torch.equal(sel1[0], sel[t]), t
        assert torch.equal(o1[0], out[t]) and torch.equal(l1[0], lse[t]), t
        assert torch.equal(w1[0], wout[t]) and torch.equal(wl1[0], wlse[t]), t
    assert ops.resolve_num_splits(1, 513, 0) == ops.resolve_num_splits(256, 513, 0)
    _check_all(wl, sel, out, lse, [0, 129, 255], what="split by length")


def test_split_by_length_gives_short_lists_fewer_partitions():
    """num_splits = 0 with histories of every length class in one call: the
    extent is the longest list's count, shorter lists use their own count and
    leave the rest of their partitions empty; the merged results match the
    oracle and equal each token run alone."""
    _say("split by length, mixed lengths")
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(SMALL, seed=15, device="cuda")
    pt, sl, qs, qp = device_tables(wl)
    sel = ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512)
    S = ops.resolve_num_splits(wl.n_tok, 513, 0)
    assert S > 1
    po = torch.full((wl.n_tok, S, 64, 192), float("nan"), device="cuda")
    pl = torch.empty((wl.n_tok, S, 64), device="cuda")
    out, lse = ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel, SCALE, num_splits=0,
                                 part_o=po, part_lse=pl)
    torch.cuda.synchronize()
    _check_all(wl, sel, out, lse, range(wl.n_tok), what="split by length")
    for t in range(0, wl.n_tok, 5):
        one = slice(t, t + 1)
        o1, l1 = ops.sparse_decode(wl.q[one], wl.k_cache, wl.v_cache, pt, sl, qs[one], qp[one], sel[one], SCALE,
                                   num_splits=0)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out[t]) and torch.equal(l1[0], lse[t]), t


def test_all_scores_tied_takes_lowest_blocks():
    """Index query of zeros: every score is 0, so the first 512 blocks win. In
    the first call (histories up to 5000 blocks: finalize) the threshold bin
    holds every score, more than the finalize's LDS tie buffer: the ordered
    select over all scores. In the second (a 17,500-block history: candidate
    lists) every chunk lists all of its keys, more than the select pass holds
    in LDS: the ordered select over all scores as well."""
    _say("all tied")
    for name, lens in (("tied", [40001, 5000]), ("tied_long", [140000, 5000])):
        wl = I.make_workload(I.WorkloadSpec(name, batch=2, seq_lens=lens, q_per_seq=2), seed=21, device="cuda")
        wl.q_idx.zero_()
        sel, out, lse = run_sparse_layer(wl)
        sel_h = sel.cpu().numpy()
        for t in range(wl.n_tok):
            cb = int(wl.q_pos[t]) // 8
            assert sel_h[t].tolist() == list(range(min(512, cb))) + [-1] * (512 - min(512, cb)), f"{name} {t}"
        _check_all(wl, sel, out, lse, range(wl.n_tok), what=name)


def test_overflowing_candidate_list_is_reread():
    """One chunk whose list would exceed the 512-entry cap: 30 one-token
    sequences of 140,000 tokens (17,504-block tables) make the host score in
    chunks of 1,024 blocks (30 x 18 chunks >= 512 workgroups), and the first
    1,024 blocks of sequence 0 all carry the key 4*sign(q), the highest score
    any key in [-4, 4] can reach. That chunk lists nothing (its edge is
    "none"), the select pass re-reads it, and sequence 0 must select blocks
    0 .. 511; every selection and output against the oracle."""
    _say("overflowing candidate list")
    spec = I.WorkloadSpec("overflow", batch=30, seq_lens=[140000] * 30, q_per_seq=1)
    wl = I.make_workload(spec, seed=23, device="cuda")
    t0 = int(np.flatnonzero(np.asarray(wl.q_seq) == 0)[0])
    pages = torch.from_numpy(np.asarray(wl.page_table[0][:128], dtype=np.int64)).to(wl.k_idx_cache.device)
    top = (4 * torch.sign(wl.q_idx[t0].float())).to(wl.k_idx_cache.dtype)
    wl.k_idx_cache[pages] = top.view(1, 1, -1).expand(128, 8, -1)
    sel, out, lse = run_sparse_layer(wl)
    sel_h = sel.cpu().numpy()
    assert sel_h[t0].tolist() == list(range(512))
    # the list header of (row t0, chunk 0) in the workspace: count 0, edge "none"
    # (headers follow the 256-byte aligned fp32 scores [n_tok][17,504], 18 per row)
    from sparse_block_indexed_amd import ops
    pt, sl, qs, qp = device_tables(wl)
    ws = torch.zeros(ops.indexer_workspace_size(wl.n_tok, wl.max_pages_per_seq, 512), dtype=torch.uint8,
                     device="cuda")
    sel2 = ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(sel2, sel)
    mhb = wl.max_pages_per_seq * 8
    meta_off = (wl.n_tok * mhb * 4 + 255) // 256 * 256
    nck = (mhb + 1023) // 1024
    head = ws[meta_off + 8 * (t0 * nck):meta_off + 8 * (t0 * nck + 2)].cpu().view(torch.int32).numpy().view(np.uint32)
    assert head[0] == 0 and head[1] == 0xFFFFFFFF, head
    assert head[3] != 0xFFFFFFFF and 0 < head[2] <= 512, head   # chunk 1 listed normally
    ov = OracleView(wl)
    for t in range(wl.n_tok):
        assert sel_h[t].tolist() == ov.selection(t).tolist(), f"token {t}"
    _check_all(wl, sel, out, lse, range(wl.n_tok), what="overflow")


def test_heavy_ties():
    """Index inputs in {0, 1}: many blocks share the threshold score. One call
    of finalize rows, one with a 17,500-block row (candidate lists holding
    long runs of tied keys, then the select pass)."""
    _say("heavy ties")
    for name, lens in (("ties01", [20000, 33000, 70000]), ("ties01_long", [140000, 33000])):
        spec = I.WorkloadSpec(name, batch=len(lens), seq_lens=lens, q_per_seq=2, idx_lo=0, idx_hi=1)
        wl = I.make_workload(spec, seed=22, device="cuda")
        sel, out, lse = run_sparse_layer(wl)
        ov = OracleView(wl)
        sel_h = sel.cpu().numpy()
        for t in range(wl.n_tok):
            assert sel_h[t].tolist() == ov.selection(t).tolist(), f"{name} token {t}"


def test_invalid_tokens_attend_nothing():
    _say("invalid tokens")
    spec = I.WorkloadSpec("inv", batch=2, seq_lens=[3000, 2000], q_per_seq=2)
    wl = I.make_workload(spec, seed=23, device="cuda")
    wl.q_seq[0] = -1           # sequence id out of range
    wl.q_seq[1] = 2            # = batch
    wl.q_pos[2] = 2000         # = seq_len of sequence 1
    sel, out, lse = run_sparse_layer(wl)
    for t in range(3):
        assert (sel[t] == -1).all()
        assert (out[t] == 0).all()
        assert torch.isneginf(lse[t]).all()
    _check_all(wl, sel, out, lse, [3], what="valid neighbour")


def test_invalid_positions_on_the_long_select_paths():
    """Tokens whose position is at or past their sequence's length but inside
    the page table, so that their rows are located and scored: one on the
    finalize (history above topk), one on the long-history select (candidate
    lists in the score pass, then the select pass; history above 16K blocks). Both select
    nothing and attend nothing, in the sparse and the window layer; every other
    token matches the oracle."""
    _say("invalid positions, long select paths")
    from gpu_helpers import run_swa
    spec = I.WorkloadSpec("inv_long", batch=2, seq_lens=[140000, 6000], q_per_seq=3)
    wl = I.make_workload(spec, seed=25, device="cuda")
    assert wl.max_pages_per_seq * 64 > 139000
    t1 = [t for t in range(wl.n_tok) if int(wl.q_seq[t]) == 1]
    bad = t1[:2]
    wl.q_pos[bad[0]] = 9000        # 1,125 historical blocks: finalize
    wl.q_pos[bad[1]] = 139000      # 17,375 historical blocks: long-history select
    sel, out, lse = run_sparse_layer(wl)
    wout, wlse = run_swa(wl)
    for t in bad:
        assert (sel[t] == -1).all(), f"token {t} selected blocks"
        assert (out[t] == 0).all() and torch.isneginf(lse[t]).all()
        assert (wout[t] == 0).all() and torch.isneginf(wlse[t]).all()
    _check_all(wl, sel, out, lse, [t for t in range(wl.n_tok) if t not in bad], what="valid tokens")


def test_poison_unread_blocks_and_future_positions():
    """NaN in every K/V block that is neither selected nor current, and in the
    current block past the query position: outputs bit-identical."""
    _say("poison")
    spec = I.WorkloadSpec("poison", batch=2, seq_lens=[6001, 9003], q_per_seq=1)
    wl = I.make_workload(spec, seed=24, device="cuda")
    pt, sl, qs, qp = device_tables(wl)
    sel, out, lse = run_sparse_layer(wl, tabs=(pt, sl, qs, qp))
    sel_h = sel.cpu().numpy()
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device="cuda")
    for t in range(wl.n_tok):
        b, p = int(wl.q_seq[t]), int(wl.q_pos[t])
        keep = set(int(x) for x in sel_h[t] if x >= 0) | {p // 8}
        row = wl.page_table[b]
        for blk in range((int(wl.seq_lens[b]) + 7) // 8):
            if blk in keep:
                continue
            page = int(row[blk // 8])
            wl.k_cache[page, :, blk % 8] = nan
            wl.v_cache[page, :, blk % 8] = nan
        # future positions inside the current block: positions p+1 .. 8*cb+7
        cbk = p // 8
        page = int(row[cbk // 8])
        for pos in range(p + 1, 8 * cbk + 8):
            for g in range(4):
                I.pack_k_rows(wl.k_cache, row, [pos], g, torch.full((1, 192), float("nan")))
                I.pack_v_rows(wl.v_cache, row, [pos], g, torch.full((1, 192), float("nan")))
    from sparse_block_indexed_amd import ops
    out2, lse2 = ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("q_per_seq,fp8_keys", [(2, False), (20, False), (70, False), (70, True)])
def test_unreadable_pages_rank_last_and_are_skipped(q_per_seq, fp8_keys):
    """Page-table entries outside [0, num_pages) (-1, and past the cache) on some
    historical pages: their blocks score -inf, so they rank last (lower block
    index first among them) and are chosen only when fewer readable blocks
    exist; the attention skips their tokens. Covers the per-token scorer (2
    tokens per sequence), the 16-row MFMA scorer (20) and the score GEMM (70)."""
    _say(f"unreadable pages q_per_seq={q_per_seq} fp8={fp8_keys}")
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(I.WorkloadSpec("bad_pages", batch=2, seq_lens=[3000, 9000], q_per_seq=q_per_seq),
                         seed=61, device="cuda")
    kidx = I.fp8_e4m3_codes(wl.k_idx_cache) if fp8_keys else wl.k_idx_cache
    ov = OracleView(wl, kidx_fp8=kidx if fp8_keys else None)   # reads keys through the intact table
    bad = {0: [3, 10], 1: [0, 40, 100]}                         # logical pages, none holds a current block
    pt_bad = wl.page_table.copy()
    for b, pages in bad.items():
        for i, lp in enumerate(pages):
            pt_bad[b, lp] = -1 if i % 2 == 0 else wl.num_pages + 7
    _, sl, qs, qp = device_tables(wl)
    pt = torch.as_tensor(pt_bad, dtype=torch.int32, device="cuda")
    sel = ops.indexer_topk(wl.q_idx, kidx, pt, sl, qs, qp, 512)
    out, lse = ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel, SCALE)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    outs, refs, lses, rlses = [], [], [], []
    for t in range(wl.n_tok):
        b, p = int(wl.q_seq[t]), int(wl.q_pos[t])
        cb = p // 8
        assert all(lp != p // 64 for lp in bad[b])
        q = O.bf16_to_f64(I.bf16_bits(wl.q_idx[t]))
        scores = O.indexer_scores(q, ov.keys(b, cb))
        for lp in bad[b]:
            scores[8 * lp:min(8 * lp + 8, cb)] = -np.inf
        ref_sel = O.select_top_blocks(scores, 512)
        assert sel_h[t].tolist() == ref_sel.tolist(), f"token {t} selection differs"
        if t % 9 == 0:
            pos = O.sparse_token_positions(ref_sel, p)
            pos = pos[~np.isin(pos // 64, bad[b])]
            ro, rl = ov.attention(t, pos)
            outs.append(bf16_to_np(out[t]))
            lses.append(lse[t].cpu().numpy())
            refs.append(ro)
            rlses.append(rl)
    assert_close_outputs(np.stack(outs), np.stack(lses), np.stack(refs), np.stack(rlses), "unreadable pages")


@pytest.mark.parametrize("num_splits", [1, 3])
def test_unreadable_pages_in_the_window_are_skipped(num_splits):
    """Window layer: page-table entries outside [0, num_pages) (-1, and past the
    cache) on pages inside the window (never the query's own page): the
    tokens of those pages are skipped, the rest of the window attended."""
    _say(f"unreadable window pages S={num_splits}")
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(I.WorkloadSpec("bad_win", batch=2, seq_lens=[3000, 9000], q_per_seq=2), seed=62,
                         device="cuda")
    window = 2048
    ov = OracleView(wl)   # reads K/V through the intact table
    bad = {}
    pt_bad = wl.page_table.copy()
    for b in range(wl.batch):
        last = (int(wl.seq_lens[b]) - 2) // 64   # the page of the sequence's first query token
        bad[b] = [last - 2, last - 5]
        pt_bad[b, last - 2] = -1
        pt_bad[b, last - 5] = wl.num_pages + 3
    _, sl, qs, qp = device_tables(wl)
    pt = torch.as_tensor(pt_bad, dtype=torch.int32, device="cuda")
    out, lse = ops.swa_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, window, SCALE, num_splits=num_splits)
    torch.cuda.synchronize()
    outs, refs, lses, rlses = [], [], [], []
    for t in range(wl.n_tok):
        b, p = int(wl.q_seq[t]), int(wl.q_pos[t])
        assert all(lp != p // 64 for lp in bad[b])
        pos = O.window_positions(p, window)
        pos = pos[~np.isin(pos // 64, bad[b])]
        ro, rl = ov.attention(t, pos)
        outs.append(bf16_to_np(out[t]))
        lses.append(lse[t].cpu().numpy())
        refs.append(ro)
        rlses.append(rl)
    assert_close_outputs(np.stack(outs), np.stack(lses), np.stack(refs), np.stack(rlses), "unreadable window pages")


def test_deterministic_and_batch_invariant():
    _say("determinism")
    wl = I.named_workload("decode_8k_b1", device="cuda", seed=31)
    wl_big = I.make_workload(I.WorkloadSpec("bi", batch=5, seq_lens=[8192, 3000, 20000, 8192, 500], q_per_seq=1),
                             seed=32, device="cuda")
    # place config-0's sequence as sequence 3 of the bigger batch
    b3 = wl_big.page_table[3]
    wl_big.k_cache[torch.as_tensor(b3[:128].astype(np.int64), device="cuda")] = wl.k_cache[:128]
    wl_big.v_cache[torch.as_tensor(b3[:128].astype(np.int64), device="cuda")] = wl.v_cache[:128]
    wl_big.k_idx_cache[torch.as_tensor(b3[:128].astype(np.int64), device="cuda")] = wl.k_idx_cache[:128]
    wl_big.q[3] = wl.q[0]
    wl_big.q_idx[3] = wl.q_idx[0]
    for S in (1, 8):
        s1, o1, l1 = run_sparse_layer(wl, num_splits=S)
        s2, o2, l2 = run_sparse_layer(wl, num_splits=S)
        assert torch.equal(s1, s2) and torch.equal(o1, o2) and torch.equal(l1, l2)
        s3, o3, l3 = run_sparse_layer(wl_big, num_splits=S)
        assert torch.equal(s1[0], s3[3]) and torch.equal(o1[0], o3[3]) and torch.equal(l1[0], l3[3])


def test_sparse_layer_call_equals_its_two_steps():
    """ops.sparse_layer (indexer top-k, then attention) gives bitwise what the
    two binding calls give."""
    _say("sparse_layer convenience call")
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(SMALL, seed=14, device="cuda")
    pt, sl, qs, qp = device_tables(wl)
    sel, out, lse = ops.sparse_layer(wl.q, wl.q_idx, wl.k_cache, wl.v_cache, wl.k_idx_cache, pt, sl, qs, qp, SCALE,
                                     num_splits=3)
    sel2, out2, lse2 = run_sparse_layer(wl, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2) and torch.equal(out, out2) and torch.equal(lse, lse2)


def test_split_count_changes_only_rounding():
    _say("splits")
    wl = I.named_workload("decode_8k_b1", device="cuda", seed=33)
    ref = None
    for S in (1, 2, 5, 32, 64):
        sel, out, lse = run_sparse_layer(wl, num_splits=S)
        if ref is None:
            ref = (out, lse)
            continue
        assert_close_outputs(bf16_to_np(out), lse.cpu().numpy(), bf16_to_np(ref[0]), ref[1].cpu().numpy(), f"S={S}")


def test_page_permutation_invariance():
    _say("page permutation")
    spec = I.WorkloadSpec("perm", batch=2, seq_lens=[7000, 12345], q_per_seq=2)
    wl = I.make_workload(spec, seed=34, device="cuda")
    sel1, out1, lse1 = run_sparse_layer(wl, num_splits=2)
    perm = np.random.default_rng(5).permutation(wl.num_pages)
    inv = torch.as_tensor(np.argsort(perm).astype(np.int64), device="cuda")
    # new physical page perm[i] holds old page i
    wl.k_cache = wl.k_cache[inv].contiguous()
    wl.v_cache = wl.v_cache[inv].contiguous()
    wl.k_idx_cache = wl.k_idx_cache[inv].contiguous()
    wl.page_table = np.where(wl.page_table >= 0, perm[np.maximum(wl.page_table, 0)], -1).astype(np.int32)
    sel2, out2, lse2 = run_sparse_layer(wl, num_splits=2)
    assert torch.equal(sel1, sel2) and torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_closed_forms_constant_v_and_zero_q():
    _say("closed forms")
    spec = I.WorkloadSpec("cf", batch=2, seq_lens=[5000, 777], q_per_seq=2)
    wl = I.make_workload(spec, seed=35, device="cuda")
    const = torch.randn(4, 192, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    # constant V per group: every (page, group, block) unit holds the group's row for all 8 tokens
    v = const.to("cuda")[:, :, None].expand(4, 192, 8).reshape(4, 1536)
    wl.v_cache[:] = v[None, :, None, :]
    sel, out, lse = run_sparse_layer(wl)
    for t in range(wl.n_tok):
        for h in range(64):
            assert torch.equal(out[t, h].float(), const[h // 16].float().cuda()), (t, h)
    # Q = 0: uniform weights -> lse = ln(number of attended tokens)
    wl.q.zero_()
    sel, out, lse = run_sparse_layer(wl)
    for t in range(wl.n_tok):
        n = len(O.sparse_token_positions(sel[t].cpu().numpy(), int(wl.q_pos[t])))
        assert torch.allclose(lse[t], torch.full_like(lse[t], math.log(n)), atol=1e-4)


def _merge_against_oracle(po, pl, out, lse, tokens, what):
    refs = [O.merge(po[t].double().numpy(), pl[t].double().numpy()) for t in tokens]
    assert_close_outputs(bf16_to_np(out[list(tokens)]), lse[list(tokens)].cpu().numpy(),
                         np.stack([r[0] for r in refs]), np.stack([r[1] for r in refs]), what)
    for t, (ro, rl) in zip(tokens, refs):
        gl = lse[t].cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), (what, t)
        fin = np.isfinite(rl)
        assert np.abs(gl[fin] - rl[fin]).max(initial=0.0) <= 1e-4, (what, t)


def test_merge_entry_point():
    _say("merge")
    from sparse_block_indexed_amd import ops
    g = torch.Generator().manual_seed(7)
    n_tok, S = 5, 6
    po = torch.randn(n_tok, S, 64, 192, generator=g)
    pl = torch.randn(n_tok, S, 64, generator=g) * 3
    pl[0, 2:] = -float("inf")
    pl[1, :] = -float("inf")
    out, lse = ops.merge(po.cuda(), pl.cuda())
    torch.cuda.synchronize()
    assert (out[1] == 0).all() and torch.isneginf(lse[1]).all()
    _merge_against_oracle(po, pl, out, lse, [0, 2, 3, 4], "merge")


def test_merge_ignores_nan_in_empty_partitions():
    """A partition with lse = -inf carries no weight whatever its slot holds:
    NaN and inf there leave the output bitwise equal to the same merge with
    finite values there."""
    _say("merge, NaN in empty partitions")
    from sparse_block_indexed_amd import ops
    g = torch.Generator().manual_seed(8)
    n_tok, S = 4, 9
    po = torch.randn(n_tok, S, 64, 192, generator=g)
    pl = torch.randn(n_tok, S, 64, generator=g) * 3
    pl[:, 1::3] = -float("inf")
    pl[2, :, 5:] = -float("inf")
    out_ref, lse_ref = ops.merge(po.cuda(), pl.cuda())
    po_bad = po.clone()
    empty = torch.isneginf(pl)[..., None].expand_as(po)
    po_bad[empty] = float("nan")
    po_bad[0, 1, :3] = float("inf")
    out, lse = ops.merge(po_bad.cuda(), pl.cuda())
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
    _merge_against_oracle(po_bad, pl, out, lse, range(n_tok), "merge with NaN in empty partitions")


@pytest.mark.parametrize("heads,dim,S", [(16, 128, 2), (3, 4, 64), (2, 1024, 5), (1024, 8, 1), (64, 192, 33)])
def test_merge_entry_point_shapes(heads, dim, S):
    """sa_merge is generic in heads (<= 1024), head dim (multiple of 4, <= 1024)
    and partitions (<= 64)."""
    _say(f"merge {heads}x{dim} S={S}")
    from sparse_block_indexed_amd import ops
    g = torch.Generator().manual_seed(heads * 7 + dim + S)
    n_tok = 3
    po = torch.randn(n_tok, S, heads, dim, generator=g)
    pl = torch.randn(n_tok, S, heads, generator=g) * 4
    if S > 1:
        pl[0, ::2] = -float("inf")                 # some empty partitions
    out, lse = ops.merge(po.cuda(), pl.cuda())
    torch.cuda.synchronize()
    _merge_against_oracle(po, pl, out, lse, range(n_tok), f"merge {heads}x{dim} S={S}")


def test_zero_tokens_is_a_no_op():
    from sparse_block_indexed_amd import ops
    spec = I.WorkloadSpec("z", batch=1, seq_lens=[100], q_per_seq=1)
    wl = I.make_workload(spec, seed=36, device="cuda")
    pt, sl, _, _ = device_tables(wl)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    sel = ops.indexer_topk(wl.q_idx[:0], wl.k_idx_cache, pt, sl, e, e, 512)
    out, lse = ops.sparse_decode(wl.q[:0], wl.k_cache, wl.v_cache, pt, sl, e, e, sel, SCALE)
    torch.cuda.synchronize()
    assert sel.shape == (0, 512) and out.shape == (0, 64, 192)


def test_prefill_gemm_path_mixed_tiles():
    """Enough tokens per sequence for the MFMA score GEMM; the second 64-token
    tile holds tokens of both sequences and one invalid token."""
    _say("gemm mixed tiles")
    spec = I.WorkloadSpec("gemm_mixed", batch=2, seq_lens=[5000, 20000], q_per_seq=70)
    wl = I.make_workload(spec, seed=41, device="cuda")
    wl.q_pos[100] = int(wl.seq_lens[1])      # out of range: attends nothing
    sel, out, lse = run_sparse_layer(wl)
    assert (sel[100] == -1).all() and (out[100] == 0).all()
    _check_all(wl, sel, out, lse, [t for t in range(wl.n_tok) if t != 100], what="gemm mixed")


def test_prefill_gemm_path_several_tiles_per_workgroup_and_passes():
    """The score GEMM with 16K-block histories and 5 token tiles: each workgroup
    scores 4 block tiles (both register sets of its pipeline, twice), and the
    third token tile holds rows of both sequences (a second pass, which some
    workgroups' tile ranges skip: the shorter history ends first)."""
    _say("gemm several tiles per workgroup")
    spec = I.WorkloadSpec("gemm_multi", batch=2, seq_lens=[131072, 70000], q_per_seq=160)
    wl = I.make_workload(spec, seed=43, device="cuda")
    sel, out, lse = run_sparse_layer(wl)
    ov = OracleView(wl)
    sel_h = sel.cpu().numpy()
    for t in range(wl.n_tok):
        assert sel_h[t].tolist() == ov.selection(t).tolist(), f"token {t} selection differs"
    _check_all(wl, sel, out, lse, [0, 127, 159, 160, 200, 319], what="gemm several tiles")


# ---------------------------------------------------------------------------
# One-byte (OCP FP8 E4M3) index keys
# ---------------------------------------------------------------------------

def _check_selection(wl, sel, tokens, topk=512, kidx_fp8=None, what=""):
    ov = OracleView(wl, kidx_fp8=kidx_fp8)
    sel_h = sel.cpu().numpy()
    for t in tokens:
        assert sel_h[t].tolist() == ov.selection(t, topk).tolist(), f"{what}: token {t}"


@pytest.mark.parametrize("name", ["mtp_verify_128k_b64", "decode_1m_b4"])
def test_fp8_index_keys_match_bf16_and_oracle(name):
    """Integer keys are exact in E4M3: the one-byte path must select exactly what
    the bf16 path and the oracle (decoding the codes itself) select."""
    _say(f"fp8 keys {name}")
    from sparse_block_indexed_amd import ops
    wl = I.named_workload(name, device="cuda")
    pt, sl, qs, qp = device_tables(wl)
    codes = I.fp8_e4m3_codes(wl.k_idx_cache)
    sel8 = ops.indexer_topk(wl.q_idx, codes, pt, sl, qs, qp, 512)
    sel16 = ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512)
    torch.cuda.synchronize()
    assert torch.equal(sel8, sel16)
    sample = range(wl.n_tok) if wl.n_tok <= 8 else range(0, wl.n_tok, 16)
    _check_selection(wl, sel8, sample, kidx_fp8=codes, what=f"fp8 keys {name}")


def test_fp8_index_keys_general_codes():
    """Random E4M3 codes across eight binades (values 1/8 .. 30, both signs) with
    integer queries: scores stay exact in fp32, so the selection checks the
    hardware's decoding of every such code against the oracle's. Covers the
    per-token scorer (short and long histories) and the prefill GEMM."""
    _say("fp8 general codes")
    from sparse_block_indexed_amd import ops
    for spec in (I.WorkloadSpec("f8a", batch=3, seq_lens=[3000, 20000, 140000], q_per_seq=2),
                 I.WorkloadSpec("f8g", batch=2, seq_lens=[5000, 9000], q_per_seq=70)):
        wl = I.make_workload(spec, seed=52, device="cuda")
        g = torch.Generator(device="cuda").manual_seed(6)
        shape = wl.k_idx_cache.shape
        e = torch.randint(4, 12, shape, generator=g, device="cuda", dtype=torch.int32)
        m = torch.randint(0, 8, shape, generator=g, device="cuda", dtype=torch.int32)
        sg = torch.randint(0, 2, shape, generator=g, device="cuda", dtype=torch.int32)
        codes = ((sg << 7) | (e << 3) | m).to(torch.uint8)
        pt, sl, qs, qp = device_tables(wl)
        sel = ops.indexer_topk(wl.q_idx, codes, pt, sl, qs, qp, 512)
        torch.cuda.synchronize()
        toks = range(wl.n_tok) if wl.n_tok <= 8 else range(0, wl.n_tok, 7)
        _check_selection(wl, sel, toks, kidx_fp8=codes, what=spec.name)


@pytest.mark.parametrize("fp8_keys", [False, True])
def test_sixteen_row_mfma_scorer_mixed_sequences(fp8_keys):
    """16 .. 63 query rows per sequence take the 16-row MFMA scorer. With 20
    verify tokens per sequence its 16-row groups straddle sequences, and short
    histories (5 and 64 tokens) leave rows with nothing to score."""
    _say(f"mfma16 mixed fp8={fp8_keys}")
    from sparse_block_indexed_amd import ops
    spec = I.WorkloadSpec("m16", batch=5, seq_lens=[5, 64, 1000, 4111, 16000], q_per_seq=20, spare_pages=3)
    wl = I.make_workload(spec, seed=41, device="cuda")
    assert wl.n_tok >= 16 * wl.batch           # the 16-row path
    pt, sl, qs, qp = device_tables(wl)
    kidx = I.fp8_e4m3_codes(wl.k_idx_cache) if fp8_keys else wl.k_idx_cache
    sel = ops.indexer_topk(wl.q_idx, kidx, pt, sl, qs, qp, 512)
    out, lse = ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel, SCALE)
    torch.cuda.synchronize()
    ov = OracleView(wl, kidx_fp8=kidx if fp8_keys else None)
    sel_h = sel.cpu().numpy()
    for t in range(wl.n_tok):
        assert sel_h[t].tolist() == ov.selection(t).tolist(), f"token {t}"
    toks = list(range(0, wl.n_tok, 7))
    refs = [ov.sparse(t, sel_h[t]) for t in toks]
    assert_close_outputs(bf16_to_np(out[toks]), lse[toks].cpu().numpy(), np.stack([r[0] for r in refs]),
                         np.stack([r[1] for r in refs]), "mfma16")
    # equal to the per-token scorer's selection (the same call split into 4-token calls)
    for t0 in range(0, wl.n_tok, 4):
        t1 = min(wl.n_tok, t0 + 4)
        part = ops.indexer_topk(wl.q_idx[t0:t1].contiguous(), kidx, pt, sl, qs[t0:t1].contiguous(),
                                qp[t0:t1].contiguous(), 512)
        assert torch.equal(part, sel[t0:t1])


def test_finalize_step_count_boundaries():
    """The finalize runs the instantiation sized to the row's history: 2, 4,
    8, 16 or 32 scores per thread of 512, so rows of 1,024 / 2,048 / 4,096 /
    8,192 blocks are the largest the first four hold. One row on either side of
    every boundary, all in one call, checked against the oracle."""
    _say("finalize step boundaries")
    hist = [1024, 1025, 2048, 2049, 4096, 4097, 8192, 8193]
    wl = I.make_workload(I.WorkloadSpec("steps", batch=len(hist), seq_lens=[8 * h + 1 for h in hist], q_per_seq=1),
                         seed=52, device="cuda")
    assert sorted(int(p) // 8 for p in wl.q_pos) == hist
    sel, out, lse = run_sparse_layer(wl)
    _check_all(wl, sel, out, lse, range(wl.n_tok), what="finalize step boundaries")


@pytest.mark.parametrize("q_per_seq", [3, 4])
@pytest.mark.parametrize("fp8_keys", [False, True])
def test_long_histories_with_three_and_four_tokens_per_sequence(q_per_seq, fp8_keys):
    """Histories past the finalize limit scored in runs of 3 or 4 tokens of one
    sequence (the score pass then keeps each row's chunk and its histogram in
    LDS and lists its candidates), then the select launch; every selection
    against the oracle."""
    _say(f"long histories, {q_per_seq} tokens per sequence, fp8={fp8_keys}")
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(I.WorkloadSpec("long_runs", batch=2, seq_lens=[140000, 20000], q_per_seq=q_per_seq),
                         seed=44, device="cuda")
    pt, sl, qs, qp = device_tables(wl)
    kidx = I.fp8_e4m3_codes(wl.k_idx_cache) if fp8_keys else wl.k_idx_cache
    sel = ops.indexer_topk(wl.q_idx, kidx, pt, sl, qs, qp, 512)
    torch.cuda.synchronize()
    _check_selection(wl, sel, range(wl.n_tok), kidx_fp8=kidx if fp8_keys else None,
                     what=f"long runs of {q_per_seq}")


def test_history_limits_of_the_select_paths():
    """Around the select paths' size limits, every selection checked against
    the oracle: a call whose longest history is exactly 16,384 blocks (scores
    held and selected by finalize alone), the same sequences plus one 8 tokens
    longer (every row then takes the per-chunk candidate lists and the select
    pass), and a context just past 2^17 blocks (513 chunks of 256 blocks)."""
    from sparse_block_indexed_amd import ops
    cases = [("finalize limit", [131072, 70000], 2),
             ("candidate lists", [131072, 131080, 70000], 2),
             ("past 2^17 blocks", [1048576 + 64], 1)]
    for name, lens, q in cases:
        _say(f"limits: {name}")
        wl = I.make_workload(I.WorkloadSpec(name, batch=len(lens), seq_lens=lens, q_per_seq=q), seed=51,
                             device="cuda")
        sel, out, lse = run_sparse_layer(wl)
        _check_all(wl, sel, out, lse, range(wl.n_tok), what=name)
        del wl, sel, out, lse
        torch.cuda.empty_cache()
