"""GPU parity of per-KV-group selection (sa_indexer_topk_grouped +
sa_sparse_decode_grouped) against the fp64 oracle: every (token, group)
selection bit for bit, outputs within max-abs 2e-2 / rel-RMS 5e-3, lse 1e-3."""
import numpy as np
import pytest
import torch

from sparse_block_indexed_amd import inputs as I

from gpu_helpers import SCALE, OracleView, assert_close_outputs, bf16_to_np, device_tables

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_block_indexed_amd import ops
    ops.load_library()


def _say(msg):
    print(msg, flush=True)


def _run(wl, qg, num_splits=0, kidx=None, kv=None, topk=512):
    from sparse_block_indexed_amd import ops
    pt, sl, qs, qp = device_tables(wl)
    sel = ops.indexer_topk(qg, wl.k_idx_cache if kidx is None else kidx, pt, sl, qs, qp, topk)
    kc, vc, kw = (wl.k_cache, wl.v_cache, {}) if kv is None else (kv[0], kv[1], dict(k_scale=kv[2], v_scale=kv[3]))
    out, lse = ops.sparse_decode(wl.q, kc, vc, pt, sl, qs, qp, sel, SCALE, num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    return sel, out, lse


def _check(wl, qg, sel, out, lse, sel_tokens, attn_tokens, kidx_fp8=None, kv=None, what="", topk=512):
    assert sel.shape == (wl.n_tok, 4, topk)
    ov = OracleView(wl, kidx_fp8=kidx_fp8, kv_fp8=kv)
    sel_h = sel.cpu().numpy()
    refs = {}
    for t in sel_tokens:
        ref = ov.selection_grouped(t, qg, topk)
        for g in range(4):
            assert sel_h[t, g].tolist() == ref[g].tolist(), f"{what}: token {t} group {g} selection differs"
        refs[t] = ref
    outs, ros, lses, rls = [], [], [], []
    for t in attn_tokens:
        ro, rl = ov.sparse_grouped(t, refs[t] if t in refs else ov.selection_grouped(t, qg, topk))
        outs.append(bf16_to_np(out[t]))
        lses.append(lse[t].cpu().numpy())
        ros.append(ro)
        rls.append(rl)
    return assert_close_outputs(np.stack(outs), np.stack(lses), np.stack(ros), np.stack(rls), what)


SMALL = I.WorkloadSpec("small_mixed", batch=12,
                       seq_lens=[1, 7, 8, 9, 63, 64, 65, 300, 1000, 4103, 4111, 9000],
                       q_per_seq=3, spare_pages=5)


@pytest.mark.parametrize("num_splits", [0, -1, 1, 3])
def test_grouped_small_mixed(num_splits):
    _say(f"grouped small S={num_splits}")
    wl = I.make_workload(SMALL, seed=91, device="cuda")
    qg = I.grouped_index_queries(wl.n_tok, seed=5, device="cuda")
    sel, out, lse = _run(wl, qg, num_splits)
    toks = range(wl.n_tok)
    _check(wl, qg, sel, out, lse, toks, toks, what=f"grouped S={num_splits}")
    # the long histories must really differ between groups
    s = sel.cpu().numpy()
    assert any(len({tuple(s[t, g]) for g in range(4)}) > 1 for t in range(wl.n_tok))


def test_grouped_with_equal_queries_equals_shared_path():
    """All four group queries equal to the token's shared query: selections per
    group equal the shared selection, outputs and lse bitwise equal."""
    _say("grouped == shared")
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(SMALL, seed=92, device="cuda")
    qg = wl.q_idx[:, None, :].expand(wl.n_tok, 4, 256).contiguous()
    pt, sl, qs, qp = device_tables(wl)
    for S in (1, 3):
        sel_g = ops.indexer_topk(qg, wl.k_idx_cache, pt, sl, qs, qp, 512)
        sel_s = ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512)
        og, lg = ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel_g, SCALE, num_splits=S)
        os_, ls = ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel_s, SCALE, num_splits=S)
        torch.cuda.synchronize()
        for g in range(4):
            assert torch.equal(sel_g[:, g], sel_s)
        assert torch.equal(og, os_) and torch.equal(lg, ls)


def test_grouped_mtp_verify_128k_b64():
    """The 128K verify workload with per-group queries: selections of 64 tokens
    (all 4 groups), attention of 16."""
    _say("grouped mtp_verify_128k_b64")
    wl = I.named_workload("mtp_verify_128k_b64", device="cuda")
    qg = I.grouped_index_queries(wl.n_tok, seed=9, device="cuda")
    sel, out, lse = _run(wl, qg)
    rng = np.random.default_rng(1)
    sel_tok = sorted(rng.choice(wl.n_tok, size=64, replace=False).tolist())
    _check(wl, qg, sel, out, lse, sel_tok, sel_tok[::4], what="grouped 128K")


def test_grouped_fp8_keys_and_fp8_kv():
    _say("grouped fp8 keys + fp8 kv")
    wl = I.make_workload(SMALL, seed=93, device="cuda")
    qg = I.grouped_index_queries(wl.n_tok, seed=6, device="cuda")
    codes = I.fp8_e4m3_codes(wl.k_idx_cache)
    kc, vc = I.quantize_kv_fp8(wl.k_cache, wl.v_cache, 1 / 32, 1 / 16)
    kv = (kc, vc, 1 / 32, 1 / 16)
    sel, out, lse = _run(wl, qg, 0, kidx=codes, kv=kv)
    toks = range(wl.n_tok)
    _check(wl, qg, sel, out, lse, toks, toks, kidx_fp8=codes, kv=kv, what="grouped fp8")


def test_grouped_prefill_gemm_and_long_histories():
    """Many tokens per sequence (the MFMA score GEMM) and histories past the
    finalize limit (candidate lists + the select launch), per group."""
    _say("grouped gemm + long")
    for spec, stride in ((I.WorkloadSpec("gg", batch=2, seq_lens=[5000, 9000], q_per_seq=70), 9),
                         (I.WorkloadSpec("gl", batch=2, seq_lens=[200000, 30000], q_per_seq=2), 1)):
        wl = I.make_workload(spec, seed=94, device="cuda")
        qg = I.grouped_index_queries(wl.n_tok, seed=7, device="cuda")
        sel, out, lse = _run(wl, qg)
        toks = list(range(0, wl.n_tok, stride))
        _check(wl, qg, sel, out, lse, toks, toks[:6], what=spec.name)


def test_grouped_mtp_verify_fp8_keys_takes_the_16_row_scorer():
    """Per-group queries of the 128K workload (16 rows per sequence) with
    one-byte keys: the 16-row MFMA scorer; selections of 32 tokens."""
    _say("grouped mtp_verify_128k_b64, fp8 keys")
    wl = I.named_workload("mtp_verify_128k_b64", device="cuda")
    qg = I.grouped_index_queries(wl.n_tok, seed=10, device="cuda")
    codes = I.fp8_e4m3_codes(wl.k_idx_cache)
    sel, out, lse = _run(wl, qg, kidx=codes)
    rng = np.random.default_rng(2)
    toks = sorted(rng.choice(wl.n_tok, size=32, replace=False).tolist())
    _check(wl, qg, sel, out, lse, toks, toks[:4], kidx_fp8=codes, what="grouped 128K fp8 keys")


@pytest.mark.parametrize("seed", range(4))
def test_random_grouped_calls(seed):
    """Seeded random per-group calls: 1-4 sequences of random lengths (half of
    them with one history past 16,384 blocks), 1-4 query tokens each (1-3 use
    the per-token scorer's runs, 4 the 16-row MFMA scorer when every sequence
    has 4), random per-group index queries and any split setting; every (token,
    group) selection and every output against the oracle; k in {1, 100, 512}."""
    rng = np.random.default_rng(3000 + seed)
    batch = int(rng.integers(1, 5))
    lens = [int(rng.integers(1, 20000)) for _ in range(batch)]
    if rng.random() < 0.5:
        lens[int(rng.integers(0, batch))] = int(rng.integers(131080, 160000))
    q = int(rng.integers(1, 5))
    num_splits = int(rng.choice([0, -1, 1, 3]))
    topk = int(rng.choice([1, 100, 512]))
    what = f"random grouped {seed}: lens {lens}, q {q}, k {topk}, splits {num_splits}"
    _say(what)
    wl = I.make_workload(I.WorkloadSpec(f"rgrp{seed}", batch=batch, seq_lens=lens, q_per_seq=q), seed=500 + seed,
                         device="cuda")
    qg = I.grouped_index_queries(wl.n_tok, seed=600 + seed, device="cuda")
    sel, out, lse = _run(wl, qg, num_splits=num_splits, topk=topk)
    _check(wl, qg, sel, out, lse, range(wl.n_tok), range(wl.n_tok), what=what, topk=topk)
