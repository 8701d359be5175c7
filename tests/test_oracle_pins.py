"""Pins of the fp64 oracle against things other than itself.

Each test ties one oracle function to a hand-worked value, a closed form, a
brute-force enumeration or an independent library routine (torch's
scaled_dot_product_attention in float64), so that a dropped term, a wrong
sign, index or head->group map, or a transposed operand fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sa_oracle as O
from sparse_block_indexed_amd import inputs as I

GOLD = os.path.join(os.path.dirname(__file__), "golden")
SCALE = 1.0 / math.sqrt(192.0)


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# bf16 decoding: closed forms of the IEEE encoding
# ---------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0000, 0x8000, 0x7F80, 0x0001, 0x4380], dtype=np.uint16)
    vals = O.bf16_to_f64(bits)
    assert vals[0] == 1.0
    assert vals[1] == -2.0
    assert vals[2] == 3.140625              # 1.5703125 * 2
    assert vals[3] == 0.0 and not np.signbit(vals[3])
    assert vals[4] == 0.0 and np.signbit(vals[4])
    assert np.isinf(vals[5]) and vals[5] > 0
    assert vals[6] == 2.0 ** -133           # smallest bf16 subnormal
    assert vals[7] == 256.0


# ---------------------------------------------------------------------------
# Cache layout: the oracle's accessors against the packer and hand offsets
# ---------------------------------------------------------------------------

def test_layout_hand_offsets():
    # K element (page 3, group 2, position 13 in page, dim 37): block 1, token 5,
    # dim chunk 4, dim-in-chunk 5.  V element: block 1, dim 37, token 5.
    num_pages = 5
    k = np.zeros(num_pages * 4 * 8 * 1536, dtype=np.uint16)
    v = np.zeros_like(k)
    unit = ((3 * 4 + 2) * 8 + 1) * 1536
    k[unit + 4 * 64 + 5 * 8 + 5] = 0x3F80    # 1.0
    v[unit + 37 * 8 + 5] = 0xC000            # -2.0
    page_row = np.array([7, 3, 0, 0], dtype=np.int64)   # logical page 1 -> physical 3
    kr = O.k_rows(k, page_row, [64 + 13], 2)
    vr = O.v_rows(v, page_row, [64 + 13], 2)
    assert kr[0, 37] == 1.0 and np.count_nonzero(kr) == 1
    assert vr[0, 37] == -2.0 and np.count_nonzero(vr) == 1


def test_layout_round_trip_with_packer():
    torch.manual_seed(0)
    num_pages = 4
    k = torch.zeros(num_pages, 4, 8, 1536, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    kidx = torch.zeros(num_pages, 8, 256, dtype=torch.bfloat16)
    page_row = np.array([2, 0, 3, 1])
    positions = [0, 5, 63, 64, 100, 200, 255]
    for g in range(4):
        rows_k = torch.randn(len(positions), 192).to(torch.bfloat16)
        rows_v = torch.randn(len(positions), 192).to(torch.bfloat16)
        I.pack_k_rows(k, page_row, positions, g, rows_k)
        I.pack_v_rows(v, page_row, positions, g, rows_v)
        np.testing.assert_array_equal(O.k_rows(I.bf16_bits(k), page_row, positions, g), rows_k.double().numpy())
        np.testing.assert_array_equal(O.v_rows(I.bf16_bits(v), page_row, positions, g), rows_v.double().numpy())
    keys = torch.randint(-4, 5, (32, 256)).to(torch.bfloat16)
    for b in range(32):
        I.pack_index_key(kidx, page_row, b, keys[b])
    np.testing.assert_array_equal(O.index_keys(I.bf16_bits(kidx), page_row, 32), keys.double().numpy())


# ---------------------------------------------------------------------------
# Selection: hand-worked case, brute force, invariants
# ---------------------------------------------------------------------------

def test_topk_hand_worked_tie():
    g = _gold("topk_tiny_tie.json")
    s = O.indexer_scores(np.array(g["q_idx"], float), np.array(g["keys"], float))
    np.testing.assert_array_equal(s, g["worked_scores"])
    for case in g["cases"]:
        got = O.select_top_blocks(s, case["k"])
        assert got.tolist() == case["expected"], case


def _brute_force_select(scores, k):
    """Repeatedly take the best remaining block (largest score, then lowest id)."""
    remaining = list(range(len(scores)))
    chosen = []
    for _ in range(min(k, len(scores))):
        best = remaining[0]
        for b in remaining[1:]:
            if scores[b] > scores[best]:
                best = b
        chosen.append(best)
        remaining.remove(best)
    return sorted(chosen) + [-1] * (k - len(chosen))


@pytest.mark.parametrize("seed", range(25))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    k = int(rng.integers(1, 70))
    lo = int(rng.integers(-4, 0))
    q = rng.integers(lo, 5, size=6).astype(float)
    keys = rng.integers(lo, 5, size=(n, 6)).astype(float)
    s = O.indexer_scores(q, keys)
    np.testing.assert_array_equal(s, [sum(q[d] * keys[b, d] for d in range(6)) for b in range(n)])
    got = O.select_top_blocks(s, k).tolist()
    assert got == _brute_force_select(list(s), k)


@pytest.mark.parametrize("seed", range(5))
def test_topk_invariants_realistic(seed):
    rng = np.random.default_rng(100 + seed)
    cb = int(rng.integers(513, 3000))
    q = rng.integers(-4, 5, size=256).astype(float)
    keys = rng.integers(-4, 5, size=(cb, 256)).astype(float)
    s = O.indexer_scores(q, keys)
    sel = O.select_top_blocks(s, 512)
    assert len(sel) == 512 and (sel >= 0).all()
    assert (np.diff(sel) > 0).all()                  # ascending, unique
    assert sel.max() < cb
    worst = s[sel].min()
    rest = np.setdiff1d(np.arange(cb), sel)
    assert (s[rest] <= worst).all()
    # every unchosen block tied with the weakest chosen one has a larger index
    tied_out = rest[s[rest] == worst]
    tied_in = sel[s[sel] == worst]
    if len(tied_out):
        assert tied_out.min() > tied_in.max()


def test_topk_negative_zero_ties_with_zero():
    s = O.indexer_scores(np.array([1.0, -1.0]), np.array([[0.0, 0.0], [-1.0, -1.0], [1.0, 1.0]]))
    assert not np.signbit(s).any()
    assert O.select_top_blocks(s, 2).tolist() == [0, 1]


def test_topk_degenerate_counts():
    assert O.indexer_topk_token(np.ones(4), np.zeros((0, 4)), 3).tolist() == [-1, -1, -1]
    assert O.select_top_blocks(np.array([5.0]), 4).tolist() == [0, -1, -1, -1]
    assert O.select_top_blocks(np.zeros(10), 3).tolist() == [0, 1, 2]   # all tied


# ---------------------------------------------------------------------------
# Attention: hand-worked, closed forms, and torch SDPA (float64) as the
# textbook routine when the selection covers every earlier block
# ---------------------------------------------------------------------------

def test_attention_two_token_hand_worked():
    g = _gold("attention_two_token.json")
    q = np.zeros((64, 3))
    q[:, 0] = math.log(3.0)
    k = [np.array([[0.0, 0.0, 0.0], [1.0, 0.0, 0.0]])] * 4
    v = [np.array([g["v0"], g["v1"]])] * 4
    out, lse = O.attend(q, k, v, 1.0)
    np.testing.assert_allclose(out, np.tile(g["expected_o"], (64, 1)), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, g["expected_lse"], rtol=0, atol=1e-15)
    po, pl = O.merge(np.stack([np.tile(g["v0"], (64, 1)), np.tile(g["v1"], (64, 1))]),
                     np.stack([np.zeros(64), np.full(64, math.log(3.0))]))
    np.testing.assert_allclose(po, out, atol=1e-15)
    np.testing.assert_allclose(pl, lse, atol=1e-15)


def test_attention_closed_forms():
    rng = np.random.default_rng(3)
    n = 37
    q = rng.standard_normal((64, 192))
    k = [rng.standard_normal((n, 192)) for _ in range(4)]
    # constant V -> output equals the constant
    const = [np.tile(rng.standard_normal(192), (n, 1)) for _ in range(4)]
    out, _ = O.attend(q, k, const, SCALE)
    for h in range(64):
        np.testing.assert_allclose(out[h], const[h // 16][0], atol=1e-12)
    # Q = 0 -> uniform weights: mean of V, lse = ln n
    v = [rng.standard_normal((n, 192)) for _ in range(4)]
    out, lse = O.attend(np.zeros((64, 192)), k, v, SCALE)
    for h in range(64):
        np.testing.assert_allclose(out[h], v[h // 16].mean(axis=0), atol=1e-12)
    np.testing.assert_allclose(lse, math.log(n), atol=1e-12)
    # one token -> O = V[0], lse = its logit
    out, lse = O.attend(q, [x[:1] for x in k], [x[:1] for x in v], SCALE)
    for h in range(64):
        np.testing.assert_allclose(out[h], v[h // 16][0], atol=1e-12)
        np.testing.assert_allclose(lse[h], SCALE * q[h] @ k[h // 16][0], atol=1e-12)


def _dense_seq(seq_len, seed, num_pages_extra=2):
    """A one-sequence paged cache built from dense per-token rows."""
    rng = np.random.default_rng(seed)
    n_pages = (seq_len + 63) // 64
    num_pages = n_pages + num_pages_extra
    page_row = rng.permutation(num_pages)[:n_pages]
    gen = torch.Generator().manual_seed(seed)
    dense_k = torch.randn(4, seq_len, 192, generator=gen).to(torch.bfloat16)
    dense_v = torch.randn(4, seq_len, 192, generator=gen).to(torch.bfloat16)
    q = torch.randn(64, 192, generator=gen).to(torch.bfloat16)
    k_cache = torch.zeros(num_pages, 4, 8, 1536, dtype=torch.bfloat16)
    v_cache = torch.zeros_like(k_cache)
    pos = list(range(seq_len))
    for g in range(4):
        I.pack_k_rows(k_cache, page_row, pos, g, dense_k[g])
        I.pack_v_rows(v_cache, page_row, pos, g, dense_v[g])
    return page_row, dense_k, dense_v, q, k_cache, v_cache


def _sdpa(q, dense_k, dense_v, mask_positions):
    """torch SDPA in float64 over the given positions; GQA maps head h to group h // 16."""
    qq = q.double()[None, :, None, :]                       # [1, 64, 1, 192]
    kk = dense_k.double()[None, :, mask_positions, :]       # [1, 4, n, 192]
    vv = dense_v.double()[None, :, mask_positions, :]
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=SCALE, enable_gqa=True)
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("seq_len", [1, 7, 8, 9, 300, 1000, 4103])
def test_sparse_equals_dense_causal_when_all_blocks_fit(seq_len):
    page_row, dk, dv, q, kc, vc = _dense_seq(seq_len, seed=seq_len)
    p = seq_len - 1
    cb = p // 8
    kidx = torch.randint(-4, 5, (kc.shape[0], 8, 256), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    q_idx = torch.randint(-4, 5, (256,), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    sel, out, lse = O.sparse_layer_token(I.bf16_bits(q), I.bf16_bits(q_idx), I.bf16_bits(kc),
                                         I.bf16_bits(vc), I.bf16_bits(kidx), page_row, p, 512, SCALE)
    assert sel[:cb].tolist() == list(range(cb)) and (sel[cb:] == -1).all()
    ref = _sdpa(q, dk, dv, list(range(p + 1)))
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("seed", range(4))
def test_sparse_matches_masked_dense_with_small_k(seed):
    seq_len = 64 * 3 + 11 + seed * 5
    page_row, dk, dv, q, kc, vc = _dense_seq(seq_len, seed=50 + seed)
    p = seq_len - 1 - seed
    cb = p // 8
    k = 5
    gen = torch.Generator().manual_seed(seed)
    kidx = torch.randint(-4, 5, (kc.shape[0], 8, 256), generator=gen).to(torch.bfloat16)
    q_idx = torch.randint(-4, 5, (256,), generator=gen).to(torch.bfloat16)
    sel, out, _ = O.sparse_layer_token(I.bf16_bits(q), I.bf16_bits(q_idx), I.bf16_bits(kc),
                                       I.bf16_bits(vc), I.bf16_bits(kidx), page_row, p, k, SCALE)
    # brute-force selection from the keys read straight from the tensor
    s = [float(sum(float(q_idx[d]) * float(kidx[page_row[b // 8], b % 8, d]) for d in range(256)))
         for b in range(cb)]
    assert sel.tolist() == _brute_force_select(s, k)
    attended = [8 * b + i for b in sel if b >= 0 for i in range(8)] + list(range(8 * cb, p + 1))
    assert max(attended) == p and len(set(attended)) == len(attended)
    np.testing.assert_allclose(out, _sdpa(q, dk, dv, sorted(attended)), atol=1e-12, rtol=0)


@pytest.mark.parametrize("seq_len,window", [(1, 512), (300, 512), (512, 512), (513, 512), (1000, 512), (777, 64)])
def test_swa_matches_dense_window(seq_len, window):
    page_row, dk, dv, q, kc, vc = _dense_seq(seq_len, seed=7 + seq_len)
    p = seq_len - 1
    out, _ = O.swa_token(I.bf16_bits(q), I.bf16_bits(kc), I.bf16_bits(vc), page_row, p, window, SCALE)
    lo = max(0, p - window + 1)
    assert len(O.window_positions(p, window)) == min(window, p + 1)
    np.testing.assert_allclose(out, _sdpa(q, dk, dv, list(range(lo, p + 1))), atol=1e-12, rtol=0)


def test_unselected_blocks_are_never_read():
    seq_len = 64 * 4
    page_row, dk, dv, q, kc, vc = _dense_seq(seq_len, seed=9)
    p = seq_len - 1
    sel = np.array([2, 5, 11, -1], dtype=np.int64)
    base_out, base_lse = O.sparse_attention_token(I.bf16_bits(q), I.bf16_bits(kc), I.bf16_bits(vc),
                                                  page_row, sel, p, SCALE)
    kb, vb = I.bf16_bits(kc).copy(), I.bf16_bits(vc).copy()
    # NaN into every block that is neither selected nor current
    attended = {2, 5, 11, p // 8}
    for blk in range(seq_len // 8):
        if blk in attended:
            continue
        page = page_row[blk // 8]
        for g in range(4):
            off = ((page * 4 + g) * 8 + blk % 8) * 1536
            kb.reshape(-1)[off:off + 1536] = 0x7FC0
            vb.reshape(-1)[off:off + 1536] = 0x7FC0
    out, lse = O.sparse_attention_token(I.bf16_bits(q), kb, vb, page_row, sel, p, SCALE)
    np.testing.assert_array_equal(out, base_out)
    np.testing.assert_array_equal(lse, base_lse)


# ---------------------------------------------------------------------------
# Merge: identity, split invariance, empty partitions
# ---------------------------------------------------------------------------

def test_merge_single_partition_identity():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((1, 64, 192))
    l = rng.standard_normal((1, 64))
    mo, ml = O.merge(o, l)
    np.testing.assert_allclose(mo, o[0], atol=1e-15)
    np.testing.assert_allclose(ml, l[0], atol=1e-15)


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_merge_of_split_equals_unsplit(splits):
    rng = np.random.default_rng(splits)
    n = 50
    q = rng.standard_normal((64, 192)) * 3
    k = [rng.standard_normal((n, 192)) for _ in range(4)]
    v = [rng.standard_normal((n, 192)) for _ in range(4)]
    full_o, full_l = O.attend(q, k, v, SCALE)
    cuts = np.sort(rng.choice(np.arange(1, n), size=splits - 1, replace=False))
    parts = np.split(np.arange(n), cuts)
    po, pl = [], []
    for idx in parts:
        a, b = O.attend(q, [x[idx] for x in k], [x[idx] for x in v], SCALE)
        po.append(a)
        pl.append(b)
    # an empty partition: lse -inf, output ignored
    po.append(np.full((64, 192), 123.0))
    pl.append(np.full(64, -np.inf))
    mo, ml = O.merge(np.stack(po), np.stack(pl))
    np.testing.assert_allclose(mo, full_o, atol=1e-12)
    np.testing.assert_allclose(ml, full_l, atol=1e-12)


def test_merge_all_empty():
    mo, ml = O.merge(np.zeros((2, 64, 192)), np.full((2, 64), -np.inf))
    assert (mo == 0).all() and np.isneginf(ml).all()


def test_merge_ignores_whatever_an_empty_partition_holds():
    """An empty partition carries no weight (SGLang blog, "Kernels from
    StepFun": only attended partitions enter the merge): NaN or inf in its
    slot changes nothing, bit for bit, against the merge without it."""
    rng = np.random.default_rng(3)
    po = rng.standard_normal((3, 64, 192))
    pl = rng.standard_normal((3, 64)) * 2
    ref_o, ref_l = O.merge(po, pl)
    for junk in (np.nan, np.inf, -np.inf):
        po2 = np.concatenate([po[:1], np.full((1, 64, 192), junk), po[1:]])
        pl2 = np.concatenate([pl[:1], np.full((1, 64), -np.inf), pl[1:]])
        mo, ml = O.merge(po2, pl2)
        np.testing.assert_array_equal(mo, ref_o)
        np.testing.assert_array_equal(ml, ref_l)


# ---------------------------------------------------------------------------
# One-byte index keys: OCP FP8 E4M3 decoding
# ---------------------------------------------------------------------------

def test_fp8_e4m3_hand_values():
    codes = np.array([0x00, 0x80, 0x38, 0xB8, 0x40, 0x44, 0x48, 0x7E, 0xFE, 0x01, 0x08, 0x07, 0x7F, 0xFF],
                     dtype=np.uint8)
    v = O.fp8_e4m3_to_f64(codes)
    assert v[0] == 0.0 and not np.signbit(v[0])
    assert v[1] == 0.0 and np.signbit(v[1])
    assert v[2] == 1.0 and v[3] == -1.0
    assert v[4] == 2.0 and v[5] == 3.0 and v[6] == 4.0
    assert v[7] == 448.0 and v[8] == -448.0          # largest finite
    assert v[9] == 2.0 ** -9                          # smallest subnormal
    assert v[10] == 2.0 ** -6                         # smallest normal
    assert v[11] == 7 * 2.0 ** -9                     # largest subnormal
    assert np.isnan(v[12]) and np.isnan(v[13])


def test_fp8_e4m3_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.fp8_e4m3_to_f64(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert ((ref == got) | both_nan).all()
    assert (np.signbit(ref) == np.signbit(got))[~both_nan].all()


def test_fp8_keys_give_the_bf16_selection_for_small_integers():
    rng = np.random.default_rng(8)
    ints = rng.integers(-4, 5, size=(3, 8, 256))
    bf = torch.from_numpy(ints).to(torch.bfloat16)
    f8 = torch.from_numpy(ints).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    page_row = np.array([2, 0, 1])
    k_bf = O.index_keys(I.bf16_bits(bf), page_row, 20)
    k_f8 = O.index_keys(f8, page_row, 20, fp8=True)
    np.testing.assert_array_equal(k_bf, k_f8)
    np.testing.assert_array_equal(k_f8[9], ints[0, 1])      # block 9 = logical page 1 -> physical 0, block 1


# ---------------------------------------------------------------------------
# One-byte K/V caches
# ---------------------------------------------------------------------------

def test_fp8_kv_layout_hand_offsets_and_packer():
    num_pages = 3
    k = torch.zeros(num_pages, 4, 8, 1536, dtype=torch.uint8)
    v = torch.zeros_like(k)
    page_row = np.array([2, 0, 1])
    # hand offsets: K (page 1, group 3, position 70 -> logical page 1 = physical 0, block 0, token 6, dim 100)
    kf = k.view(-1).numpy()
    kf[((0 * 4 + 3) * 8 + 0) * 1536 + 1 * 512 + 6 * 64 + 36] = 0x38    # 1.0 (dim-block 1, dim 64 + 36)
    vf = v.view(-1).numpy()
    vf[((0 * 4 + 3) * 8 + 0) * 1536 + 100 * 8 + 6] = 0xC0              # -2.0
    kr = O.k_rows_fp8(kf, page_row, [70], 3, 0.5)
    vr = O.v_rows_fp8(vf, page_row, [70], 3, 0.25)
    assert kr[0, 100] == 0.5 and np.count_nonzero(kr) == 1
    assert vr[0, 100] == -0.5 and np.count_nonzero(vr) == 1
    # packer round trip
    gen = torch.Generator().manual_seed(3)
    positions = [0, 7, 64, 100, 191]
    for g in range(4):
        rk = torch.randint(0, 0x7E, (len(positions), 192), generator=gen).to(torch.uint8)
        rv = torch.randint(0x80, 0xFE, (len(positions), 192), generator=gen).to(torch.uint8)
        I.pack_k_rows_fp8(k, page_row, positions, g, rk)
        I.pack_v_rows_fp8(v, page_row, positions, g, rv)
        np.testing.assert_array_equal(O.k_rows_fp8(k.numpy(), page_row, positions, g, 2.0),
                                      O.fp8_e4m3_to_f64(rk.numpy()) * 2.0)
        np.testing.assert_array_equal(O.v_rows_fp8(v.numpy(), page_row, positions, g, 3.0),
                                      O.fp8_e4m3_to_f64(rv.numpy()) * 3.0)


def test_quantize_kv_fp8_matches_the_rows():
    """The one-byte caches hold the E4M3 codes of K/V divided by the scale, in
    the one-byte layouts (checked through both accessors)."""
    page_row, dk, dv, q, kc, vc = _dense_seq(200, seed=12)
    kq, vq = I.quantize_kv_fp8(kc, vc, 1 / 32, 1 / 16)
    pos = list(range(200))
    for g in range(4):
        want_k = (dk[g].float() * 32).to(torch.float8_e4m3fn).double().numpy() / 32
        want_v = (dv[g].float() * 16).to(torch.float8_e4m3fn).double().numpy() / 16
        np.testing.assert_array_equal(O.k_rows_fp8(kq.numpy(), page_row, pos, g, 1 / 32), want_k)
        np.testing.assert_array_equal(O.v_rows_fp8(vq.numpy(), page_row, pos, g, 1 / 16), want_v)


@pytest.mark.parametrize("seq_len", [9, 700, 4103])
def test_fp8_kv_attention_equals_sdpa_on_decoded_rows(seq_len):
    page_row, dk, dv, q, kc, vc = _dense_seq(seq_len, seed=30 + seq_len)
    ks, vs = 1 / 32, 1 / 16
    kq, vq = I.quantize_kv_fp8(kc, vc, ks, vs)
    p = seq_len - 1
    sel = np.arange(min(512, p // 8))
    sel = np.concatenate([sel, -np.ones(512 - len(sel), dtype=np.int64)])
    out, _ = O.sparse_attention_token(I.bf16_bits(q), kq.numpy(), vq.numpy(), page_row, sel, p, SCALE,
                                      fp8_scales=(ks, vs))
    dk8 = (dk.float() / ks).to(torch.float8_e4m3fn).double() * ks
    dv8 = (dv.float() / vs).to(torch.float8_e4m3fn).double() * vs
    ref = _sdpa(q, dk8, dv8, list(range(p + 1)))
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# Per-KV-group selection
# ---------------------------------------------------------------------------

def _grouped_inputs(seq_len, seed):
    page_row, dk, dv, q, kc, vc = _dense_seq(seq_len, seed=seed)
    g = torch.Generator().manual_seed(seed + 100)
    kidx = torch.randint(-4, 5, (kc.shape[0], 8, 256), generator=g).to(torch.bfloat16)
    qg = torch.randint(-4, 5, (4, 256), generator=g).to(torch.bfloat16)
    return page_row, dk, dv, q, kc, vc, kidx, qg


def test_grouped_selection_with_equal_queries_is_the_shared_selection():
    page_row, dk, dv, q, kc, vc, kidx, qg = _grouped_inputs(5000, seed=81)
    qg[:] = qg[0]
    p = 4999
    args = (I.bf16_bits(kc), I.bf16_bits(vc), I.bf16_bits(kidx), page_row, p, 512, SCALE)
    sels, out_g, lse_g = O.sparse_layer_token_grouped(I.bf16_bits(q), I.bf16_bits(qg), *args)
    sel, out, lse = O.sparse_layer_token(I.bf16_bits(q), I.bf16_bits(qg[0]), *args)
    for g in range(4):
        assert sels[g].tolist() == sel.tolist()
    np.testing.assert_array_equal(out_g, out)
    np.testing.assert_array_equal(lse_g, lse)


@pytest.mark.parametrize("seq_len", [9, 700, 5000])
def test_grouped_heads_of_each_group_match_the_shared_layer_with_that_query(seq_len):
    """Group g's 16 heads see exactly what the shared layer gives them when the
    whole token uses group g's index query."""
    page_row, dk, dv, q, kc, vc, kidx, qg = _grouped_inputs(seq_len, seed=82 + seq_len)
    p = seq_len - 1
    args = (I.bf16_bits(kc), I.bf16_bits(vc), I.bf16_bits(kidx), page_row, p, 512, SCALE)
    sels, out_g, lse_g = O.sparse_layer_token_grouped(I.bf16_bits(q), I.bf16_bits(qg), *args)
    distinct = set()
    for g in range(4):
        sel, out, lse = O.sparse_layer_token(I.bf16_bits(q), I.bf16_bits(qg[g]), *args)
        assert sels[g].tolist() == sel.tolist()
        h = slice(16 * g, 16 * g + 16)
        np.testing.assert_array_equal(out_g[h], out[h])
        np.testing.assert_array_equal(lse_g[h], lse[h])
        distinct.add(tuple(sel.tolist()))
    if p // 8 > 512:
        assert len(distinct) > 1          # the groups really chose differently


def test_grouped_layer_against_brute_force_and_sdpa():
    """Per group: top-k by brute-force integer scores (Python loops, ties to the
    lower block), then torch SDPA over that group's tokens for its 16 heads."""
    seq_len, k = 64 * 4 + 13, 6
    page_row, dk, dv, q, kc, vc, kidx, qg = _grouped_inputs(seq_len, seed=90)
    p = seq_len - 1
    cb = p // 8
    sels, out_g, lse_g = O.sparse_layer_token_grouped(I.bf16_bits(q), I.bf16_bits(qg), I.bf16_bits(kc),
                                                      I.bf16_bits(vc), I.bf16_bits(kidx), page_row, p, k, SCALE)
    kid = kidx.to(torch.int64)
    for g in range(4):
        qi = [int(x) for x in qg[g].to(torch.int64)]
        scores = []
        for blk in range(cb):
            row = kid[int(page_row[blk // 8]), blk % 8]
            scores.append(sum(qi[d] * int(row[d]) for d in range(256)))
        order = sorted(range(cb), key=lambda b: (-scores[b], b))[:k]
        assert sels[g].tolist() == sorted(order)
        positions = [8 * b + i for b in sorted(order) for i in range(8)] + list(range(8 * cb, p + 1))
        ref = _sdpa(q, dk, dv, positions)
        h = slice(16 * g, 16 * g + 16)
        np.testing.assert_allclose(out_g[h], ref[h], atol=1e-12, rtol=0)
