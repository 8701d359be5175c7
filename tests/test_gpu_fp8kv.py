"""GPU parity of the one-byte (OCP FP8 E4M3) K/V entry points against the fp64
oracle, which decodes the same codes itself.

The codes are the lossy part; once they are fixed both sides attend the same
values, so the bar is the bf16 path's: max-abs 2e-2, relative RMS 5e-3, lse
within 1e-3. With power-of-two scales the one-byte path must also reproduce the
bf16 path bit for bit on the dequantised caches (scaling by a power of two
commutes with every rounding step).
"""
import numpy as np
import pytest
import torch

from sparse_block_indexed_amd import inputs as I

from gpu_helpers import (SCALE, SPLITS_FILL_GPU, OracleView, assert_close_outputs, bf16_to_np, device_tables,
                         run_sparse_layer, run_swa)

pytestmark = pytest.mark.gpu

KS, VS = 1.0 / 32, 1.0 / 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_block_indexed_amd import ops
    ops.load_library()


def _say(msg):
    print(msg, flush=True)


def _quantize(wl, ks=KS, vs=VS):
    kc, vc = I.quantize_kv_fp8(wl.k_cache, wl.v_cache, ks, vs)
    for c in (kc, vc):
        assert not ((c & 0x7F) == 0x7F).any(), "quantisation produced a NaN code"
    return kc, vc, ks, vs


def _dequantize_to_bf16(kv):
    """bf16 caches (bf16 layouts) holding exactly code * scale."""
    kc, vc, ks, vs = kv
    P = kc.shape[0]
    k = kc.view(torch.float8_e4m3fn).float() * ks
    k = k.view(P, 4, 8, 3, 8, 8, 8).permute(0, 1, 2, 3, 5, 4, 6).reshape(P, 4, 8, 1536)
    v = vc.view(torch.float8_e4m3fn).float() * vs
    return k.to(torch.bfloat16).contiguous(), v.to(torch.bfloat16).contiguous()


def _check_sparse(wl, kv, sel, out, lse, tokens, topk=512, what=""):
    ov = OracleView(wl, kv_fp8=kv)
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


SMALL = I.WorkloadSpec("small_mixed", batch=12,
                       seq_lens=[1, 7, 8, 9, 63, 64, 65, 300, 1000, 4103, 4111, 9000],
                       q_per_seq=3, spare_pages=5)


@pytest.mark.parametrize("num_splits", [0, -1, 1, 3])
def test_fp8kv_small_mixed_sparse(num_splits):
    _say(f"fp8kv small_mixed sparse S={num_splits}")
    wl = I.make_workload(SMALL, seed=61, device="cuda")
    kv = _quantize(wl)
    sel, out, lse = run_sparse_layer(wl, num_splits=num_splits, kv_fp8=kv)
    _check_sparse(wl, kv, sel, out, lse, range(wl.n_tok), what=f"fp8kv small S={num_splits}")


@pytest.mark.parametrize("window,num_splits", [(512, 0), (64, 2), (1, 1), (4096, 0)])
def test_fp8kv_small_mixed_swa(window, num_splits):
    _say(f"fp8kv small_mixed swa W={window} S={num_splits}")
    wl = I.make_workload(SMALL, seed=62, device="cuda")
    kv = _quantize(wl)
    out, lse = run_swa(wl, window=window, num_splits=num_splits, kv_fp8=kv)
    ov = OracleView(wl, kv_fp8=kv)
    refs = [ov.swa(t, window) for t in range(wl.n_tok)]
    assert_close_outputs(bf16_to_np(out), lse.cpu().numpy(), np.stack([r[0] for r in refs]),
                         np.stack([r[1] for r in refs]), f"fp8kv swa W={window}")


def test_fp8kv_mtp_verify_128k_b64():
    """The headline workload at full size in the benchmark's launch
    configuration: every token's selection and output."""
    _say("fp8kv mtp_verify_128k_b64")
    wl = I.named_workload("mtp_verify_128k_b64", device="cuda")
    kv = _quantize(wl)
    sel, out, lse = run_sparse_layer(wl, kv_fp8=kv, num_splits=SPLITS_FILL_GPU)
    _check_sparse(wl, kv, sel, out, lse, range(wl.n_tok), what="fp8kv mtp_verify_128k")


def test_fp8kv_swa_decode_32k_b64():
    _say("fp8kv swa_decode_32k_b64")
    wl = I.named_workload("swa_decode_32k_b64", device="cuda")
    kv = _quantize(wl)
    out, lse = run_swa(wl, kv_fp8=kv, num_splits=SPLITS_FILL_GPU)
    ov = OracleView(wl, kv_fp8=kv)
    refs = [ov.swa(t) for t in range(wl.n_tok)]
    assert_close_outputs(bf16_to_np(out), lse.cpu().numpy(), np.stack([r[0] for r in refs]),
                         np.stack([r[1] for r in refs]), "fp8kv swa_32k")


def test_cacheable_loads_window_and_one_byte_kv():
    """Calls with more than 64 query tokens per sequence (a prefill-like call)
    read K/V with ordinary, cacheable loads instead of non-temporal ones: the
    one-byte sparse layer and the window layer in both cache forms on that
    path, against the oracle on sampled tokens (the window with 2 partitions
    too)."""
    _say("cacheable loads: fp8 sparse, window bf16 and fp8")
    wl = I.make_workload(I.WorkloadSpec("cacheable", batch=2, seq_lens=[5000, 9000], q_per_seq=70),
                         seed=95, device="cuda")
    assert wl.n_tok > 64 * wl.batch
    kv = _quantize(wl)
    toks = list(range(0, wl.n_tok, 13)) + [wl.n_tok - 1]
    sel, out, lse = run_sparse_layer(wl, kv_fp8=kv)
    _check_sparse(wl, kv, sel, out, lse, toks, what="cacheable fp8kv sparse")
    for form, kvf in (("bf16", None), ("fp8", kv)):
        ov = OracleView(wl, kv_fp8=kvf)
        refs = [ov.swa(t) for t in toks]
        for S in (0, 2):
            out, lse = run_swa(wl, num_splits=S, kv_fp8=kvf)
            assert_close_outputs(bf16_to_np(out[toks]), lse[toks].cpu().numpy(), np.stack([r[0] for r in refs]),
                                 np.stack([r[1] for r in refs]), f"cacheable swa {form} S={S}")


def test_fp8kv_general_codes():
    """Every finite E4M3 code (subnormals, both signs, up to +-448) in K and V:
    checks the hardware's decoding of each code against the oracle's."""
    _say("fp8kv general codes")
    wl = I.make_workload(I.WorkloadSpec("f8kv", batch=3, seq_lens=[700, 5000, 12000], q_per_seq=2),
                         seed=63, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(7)
    shape = (wl.k_cache.shape[0], 4, 8, 1536)
    kc = torch.randint(0, 256, shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    kc[(kc & 0x7F) == 0x7F] ^= 0x01                 # NaN codes -> +-448
    vc[(vc & 0x7F) == 0x7F] ^= 0x01
    kv = (kc, vc, 1.0 / 256, 1.0 / 64)
    for S in (0, 2):
        sel, out, lse = run_sparse_layer(wl, num_splits=S, kv_fp8=kv)
        _check_sparse(wl, kv, sel, out, lse, range(wl.n_tok), what=f"general codes S={S}")
        out_w, lse_w = run_swa(wl, num_splits=S, kv_fp8=kv)
        ov = OracleView(wl, kv_fp8=kv)
        refs = [ov.swa(t) for t in range(wl.n_tok)]
        assert_close_outputs(bf16_to_np(out_w), lse_w.cpu().numpy(), np.stack([r[0] for r in refs]),
                             np.stack([r[1] for r in refs]), f"general codes swa S={S}")


@pytest.mark.parametrize("num_splits", [1, 4])
def test_fp8kv_equals_bf16_path_on_dequantised_caches(num_splits):
    """Power-of-two scales: the one-byte path and the bf16 path over caches
    holding exactly code * scale give bitwise identical outputs and lse."""
    _say(f"fp8kv vs bf16 S={num_splits}")
    from sparse_block_indexed_amd import ops
    wl = I.make_workload(SMALL, seed=64, device="cuda")
    kv = _quantize(wl)
    kb, vb = _dequantize_to_bf16(kv)
    pt, sl, qs, qp = device_tables(wl)
    sel = ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, 512)
    o8, l8 = ops.sparse_decode(wl.q, kv[0], kv[1], pt, sl, qs, qp, sel, SCALE, num_splits=num_splits,
                               k_scale=kv[2], v_scale=kv[3])
    o16, l16 = ops.sparse_decode(wl.q, kb, vb, pt, sl, qs, qp, sel, SCALE, num_splits=num_splits)
    w8, wl8 = ops.swa_decode(wl.q, kv[0], kv[1], pt, sl, qs, qp, 512, SCALE, num_splits=num_splits,
                             k_scale=kv[2], v_scale=kv[3])
    w16, wl16 = ops.swa_decode(wl.q, kb, vb, pt, sl, qs, qp, 512, SCALE, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(o8, o16) and torch.equal(l8, l16)
    assert torch.equal(w8, w16) and torch.equal(wl8, wl16)


def test_fp8kv_poison_unread_blocks_and_future_positions():
    """The NaN code in every block that is neither selected nor current, and in
    the current block past the query position: outputs bit-identical."""
    _say("fp8kv poison")
    from sparse_block_indexed_amd import ops
    spec = I.WorkloadSpec("poison", batch=2, seq_lens=[6001, 9003], q_per_seq=1)
    wl = I.make_workload(spec, seed=65, device="cuda")
    kv = _quantize(wl)
    kc, vc = kv[0], kv[1]
    pt, sl, qs, qp = device_tables(wl)
    sel, out, lse = run_sparse_layer(wl, tabs=(pt, sl, qs, qp), kv_fp8=kv)
    sel_h = sel.cpu().numpy()
    nan_row = torch.full((1, 192), 0x7F, dtype=torch.uint8)
    for t in range(wl.n_tok):
        b, p = int(wl.q_seq[t]), int(wl.q_pos[t])
        keep = set(int(x) for x in sel_h[t] if x >= 0) | {p // 8}
        row = wl.page_table[b]
        for blk in range((int(wl.seq_lens[b]) + 7) // 8):
            if blk in keep:
                continue
            page = int(row[blk // 8])
            kc[page, :, blk % 8] = 0x7F
            vc[page, :, blk % 8] = 0x7F
        cbk = p // 8
        for pos in range(p + 1, 8 * cbk + 8):
            for g in range(4):
                I.pack_k_rows_fp8(kc, row, [pos], g, nan_row)
                I.pack_v_rows_fp8(vc, row, [pos], g, nan_row)
    out2, lse2 = ops.sparse_decode(wl.q, kc, vc, pt, sl, qs, qp, sel, SCALE, k_scale=kv[2], v_scale=kv[3])
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(lse, lse2)


def test_fp8kv_constant_v_closed_form():
    """Every V code equal to c: each output is exactly bf16(decode(c) * v_scale)
    whatever K holds, and lse matches the oracle."""
    _say("fp8kv constant V")
    wl = I.make_workload(SMALL, seed=66, device="cuda")
    kv = _quantize(wl)
    vc = torch.full_like(kv[1], 0x3B)                # 1.375
    kv = (kv[0], vc, kv[2], 0.5)
    sel, out, lse = run_sparse_layer(wl, kv_fp8=kv)
    want = torch.full_like(out, 1.375 * 0.5)
    valid = torch.isfinite(lse).all(dim=1)
    assert valid.all()
    assert torch.equal(out, want)
    ov = OracleView(wl, kv_fp8=kv)
    for t in range(wl.n_tok):
        ro, rl = ov.sparse(t, sel[t].cpu().numpy())
        assert np.abs(lse[t].cpu().numpy() - rl).max() <= 1e-3


@pytest.mark.parametrize("seed", range(4))
def test_fp8kv_random_calls(seed):
    """Seeded random one-byte K/V calls: 1-5 sequences of random lengths (half
    of them with one history past 16,384 blocks), 1-4 query tokens each, k in
    {1, 100, 512}, any split setting, then the window layer over the same caches
    with a random window; every token against the oracle's own decoding."""
    rng = np.random.default_rng(4000 + seed)
    batch = int(rng.integers(1, 6))
    lens = [int(rng.integers(1, 20000)) for _ in range(batch)]
    if rng.random() < 0.5:
        lens[int(rng.integers(0, batch))] = int(rng.integers(131080, 160000))
    q = int(rng.integers(1, 5))
    topk = int(rng.choice([1, 100, 512]))
    num_splits = int(rng.choice([0, -1, 1, 3]))
    window = int(rng.choice([1, 512, int(rng.integers(2, 4097))]))
    what = f"fp8kv random {seed}: lens {lens}, q {q}, k {topk}, splits {num_splits}, window {window}"
    _say(what)
    wl = I.make_workload(I.WorkloadSpec(f"f8r{seed}", batch=batch, seq_lens=lens, q_per_seq=q), seed=700 + seed,
                         device="cuda")
    kv = _quantize(wl)
    sel, out, lse = run_sparse_layer(wl, topk=topk, num_splits=num_splits, kv_fp8=kv)
    _check_sparse(wl, kv, sel, out, lse, range(wl.n_tok), topk=topk, what=what)
    wout, wlse = run_swa(wl, window=window, num_splits=num_splits, kv_fp8=kv)
    ov = OracleView(wl, kv_fp8=kv)
    refs = [ov.swa(t, window) for t in range(wl.n_tok)]
    assert_close_outputs(bf16_to_np(wout), wlse.cpu().numpy(), np.stack([r[0] for r in refs]),
                         np.stack([r[1] for r in refs]), what + " (window)")
