"""Planted mistakes in the oracle must fail its pins.

Each case below patches one plausible mistake into the oracle module (a
wrong head -> group map, a reversed tie-break, a dropped query position, an
unnormalised merge, a K layout read as V, an off-by-one window, a base-2 lse,
a dropped or sign-flipped score term, a wrong E4M3 bias, ...) and runs the pin
tests of test_oracle_pins.py against it: at least one pin has to fail. The
patch lives only inside the test (pytest's monkeypatch), on the CPU.
"""
import math

import numpy as np
import pytest

import test_oracle_pins as P
from oracle import sa_oracle as O

ORIG = {name: getattr(O, name) for name in (
    "attend", "select_top_blocks", "indexer_scores", "sparse_token_positions", "window_positions", "merge",
    "v_rows", "fp8_e4m3_to_f64", "bf16_to_f64", "index_keys", "sparse_attention_token_grouped")}

# The pins, fastest first; a case stops at the first pin that fails.
PINS = [
    (P.test_bf16_decode_known_patterns, {}),
    (P.test_topk_hand_worked_tie, {}),
    (P.test_topk_degenerate_counts, {}),
    (P.test_topk_negative_zero_ties_with_zero, {}),
    (P.test_layout_hand_offsets, {}),
    (P.test_attention_two_token_hand_worked, {}),
    (P.test_attention_closed_forms, {}),
    (P.test_merge_single_partition_identity, {}),
    (P.test_merge_all_empty, {}),
    (P.test_merge_ignores_whatever_an_empty_partition_holds, {}),
    (P.test_merge_of_split_equals_unsplit, {"splits": 3}),
    (P.test_fp8_e4m3_hand_values, {}),
    (P.test_topk_brute_force, {"seed": 0}),
    (P.test_topk_brute_force, {"seed": 1}),
    (P.test_topk_invariants_realistic, {"seed": 0}),
    (P.test_layout_round_trip_with_packer, {}),
    (P.test_sparse_equals_dense_causal_when_all_blocks_fit, {"seq_len": 300}),
    (P.test_sparse_matches_masked_dense_with_small_k, {"seed": 0}),
    (P.test_swa_matches_dense_window, {"seq_len": 777, "window": 64}),
    (P.test_swa_matches_dense_window, {"seq_len": 1000, "window": 512}),
    (P.test_grouped_heads_of_each_group_match_the_shared_layer_with_that_query, {"seq_len": 700}),
    (P.test_grouped_layer_against_brute_force_and_sdpa, {}),
]


def _first_failing_pin():
    for fn, kwargs in PINS:
        try:
            fn(**kwargs)
        except Exception:   # an assertion, or an index error from a wrong layout
            return fn.__name__
    return None


# --- the planted mistakes -----------------------------------------------------

def _select_ties_to_higher_index(scores, k):
    n = len(scores)
    order = np.lexsort((-np.arange(n), -np.asarray(scores, dtype=np.float64)))
    out = np.full(k, -1, dtype=np.int64)
    chosen = np.sort(order[:min(k, n)])
    out[:len(chosen)] = chosen
    return out


def _positions_without_query(sel, p):
    return ORIG["sparse_token_positions"](sel, p)[:-1]


def _positions_without_current_block(sel, p):
    pos = ORIG["sparse_token_positions"](sel, p)
    return pos[pos < 8 * (p // 8)]


def _window_one_too_many(p, window):
    return np.arange(max(0, p - window), p + 1, dtype=np.int64)


def _merge_unnormalised(part_o, part_lse):
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    M = part_lse.max(axis=0)
    out = np.zeros(part_o.shape[1:])
    lse = np.full(part_lse.shape[1], -np.inf)
    for h in range(part_lse.shape[1]):
        if not np.isfinite(M[h]):
            continue
        w = np.exp(part_lse[:, h] - M[h])
        out[h] = (w[:, None] * part_o[:, h, :]).sum(axis=0)   # no division by the weight sum
        lse[h] = M[h] + np.log(w.sum())
    return out, lse


def _merge_without_empty_rule(part_o, part_lse):
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    M = part_lse.max(axis=0)
    with np.errstate(invalid="ignore"):   # -inf - -inf: the NaN the pins must catch
        w = np.exp(part_lse - M[None, :])
        return (w[:, :, None] * part_o).sum(axis=0) / w.sum(axis=0)[:, None], M + np.log(w.sum(axis=0))


def _merge_zero_weight_product(part_o, part_lse):
    # empty partitions weighted by a product with 0 instead of being left out
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    out = np.zeros(part_o.shape[1:])
    lse = np.full(part_lse.shape[1], -np.inf)
    for h in range(part_lse.shape[1]):
        live = np.isfinite(part_lse[:, h])
        if not live.any():
            continue
        M = part_lse[live, h].max()
        w = np.exp(part_lse[:, h] - M)
        with np.errstate(invalid="ignore"):
            out[h] = (w[:, None] * part_o[:, h, :]).sum(axis=0) / w.sum()
        lse[h] = M + np.log(w.sum())
    return out, lse


def _attend_base2_lse(q, ks, vs, scale):
    o, lse = ORIG["attend"](q, ks, vs, scale)
    return o, lse / math.log(2.0)


def _attend_unscaled(q, ks, vs, scale):
    return ORIG["attend"](q, ks, vs, 1.0)


def _scores_last_dim_dropped(q, keys):
    return ORIG["indexer_scores"](np.asarray(q)[:-1], np.asarray(keys)[:, :-1])


def _scores_negated(q, keys):
    return -ORIG["indexer_scores"](q, keys) + 0.0


def _e4m3_bias_8(bits):
    return ORIG["fp8_e4m3_to_f64"](bits) / 2.0


def _bf16_shift_15(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


def _index_keys_page_and_slot_swapped(kidx_bits, page_row, n_blocks, fp8=False):
    arr = np.asarray(kidx_bits).reshape(-1, 8, O.DI)
    decode = O.fp8_e4m3_to_f64 if fp8 else O.bf16_to_f64
    out = np.empty((n_blocks, arr.shape[2]))
    for beta in range(n_blocks):
        out[beta] = decode(arr[int(page_row[beta % 8]), beta // 8])
    return out


def _grouped_all_take_group_0(q_heads_bits, k_cache_bits, v_cache_bits, page_row, sels, p, scale, fp8_scales=None):
    sels = np.stack([np.asarray(sels[0])] * 4)
    return ORIG["sparse_attention_token_grouped"](q_heads_bits, k_cache_bits, v_cache_bits, page_row, sels, p,
                                                  scale, fp8_scales)


MUTATIONS = {
    "head h reads group h // 32": ("HEADS_PER_GROUP", 32),
    "ties go to the higher block id": ("select_top_blocks", _select_ties_to_higher_index),
    "the query's own position is dropped": ("sparse_token_positions", _positions_without_query),
    "the current block is dropped": ("sparse_token_positions", _positions_without_current_block),
    "the window holds one token too many": ("window_positions", _window_one_too_many),
    "the merge is not normalised": ("merge", _merge_unnormalised),
    "the merge gives empty partitions weight": ("merge", _merge_without_empty_rule),
    "the merge multiplies empty partitions by zero": ("merge", _merge_zero_weight_product),
    "K is read through the V layout": ("k_rows", ORIG["v_rows"]),
    "lse is in base 2": ("attend", _attend_base2_lse),
    "the softmax scale is ignored": ("attend", _attend_unscaled),
    "the last index dim is dropped": ("indexer_scores", _scores_last_dim_dropped),
    "the score sign is flipped": ("indexer_scores", _scores_negated),
    "E4M3 decoded with bias 8": ("fp8_e4m3_to_f64", _e4m3_bias_8),
    "bf16 bits shifted by 15": ("bf16_to_f64", _bf16_shift_15),
    "index-key page and slot swapped": ("index_keys", _index_keys_page_and_slot_swapped),
    "every group attends group 0's selection": ("sparse_attention_token_grouped", _grouped_all_take_group_0),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_oracle_mistake_fails_a_pin(name, monkeypatch):
    attr, value = MUTATIONS[name]
    monkeypatch.setattr(O, attr, value)
    assert _first_failing_pin() is not None, f"planted mistake '{name}' passed every pin"


def test_unpatched_oracle_passes_the_pins():
    assert _first_failing_pin() is None
