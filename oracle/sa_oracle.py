"""Plain fp64 CPU oracle of the block-indexed sparse attention step.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with
the HIP library or its Python binding, and it imports neither.

What is computed follows the pages as follows (every step cites its source):

* "Step 5 Preview: Day-0 Inference and RL Support with SGLang and Miles"
  (SGLang blog), section "Hybrid Attention": three of four layers read the
  latest 512 tokens; the fourth scores summaries of 8-token blocks, keeps up to
  512 earlier blocks and reads their tokens plus the current block.  Section
  "Kernels from StepFun": decode attention runs over the selected blocks only,
  split into partitions whose partial results are merged; the indexer scores
  each query against the compressed history in the paged cache.
* Step 5 Preview open-weights blog, table in "What the config says": 64 query
  heads, 4 KV groups, head dim 192; one 256-dim key per 8-token block; top 512
  blocks.  Section "What sparse attention does and doesn't save": the sparse
  layer picks historical blocks plus the current one.

Readings where the pages are silent (each is listed in the design notes):

* Index score = plain dot product of the token's 256-dim index query with the
  block key; no scale, no activation (any positive scale leaves the ranking
  unchanged).
* Index keys may also be stored in one byte (OCP FP8 E4M3), the open-weights
  blog's "one or two bytes" per key value ("What sparse attention does and
  doesn't save"); the score is the same dot product of the decoded values.
* K/V of the sparse layers may be stored in one byte (the open-weights blog,
  "Fitting it on a node": FP8 KV for the full-attention layers, lossy): value =
  E4M3 code * per-cache scale; attention is the same exact softmax over the
  decoded values.
* One selection per query token, shared by all four KV groups (the default);
  or, the other reading of "each KV group picks" in the open-weights blog's
  "What sparse attention does and doesn't save", one index query and one top-k
  set per (token, KV group) over the same one-per-block keys.
* Historical blocks of a token at position p are blocks 0 .. floor(p/8)-1; the
  current block floor(p/8) is always attended, its tokens up to p only.
* "Up to 512": if fewer historical blocks exist, all are kept.
* Ties at the selection threshold go to the lower block index.
* Selected block ids are reported ascending, padded with -1.
* Head h reads KV group h // 16.  Logits are scale * <q, k> with a given scale,
  no softcap, no sinks.
* The sliding window of a token at position p is positions max(0, p-511) .. p.
* lse is the natural-log log-sum-exp of the scaled logits.

Everything is float64.  bf16 inputs are converted exactly from their bits.
All parts of this module have at least one pin in the CPU test suite.
"""
from __future__ import annotations

import numpy as np

H, G, D, DI = 64, 4, 192, 256
BS, PS = 8, 64
BPP = PS // BS
HEADS_PER_GROUP = H // G


# ---------------------------------------------------------------------------
# bf16 bits -> float64 (exact)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64; exact, since bf16 is the top half of fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp8_e4m3_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) to float64, from the format's definition:
    sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds
    subnormals m * 2^-9; the all-ones exponent with all-ones mantissa is NaN
    (the format has no infinities)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * val
    return np.where((e == 15) & (m == 7), np.nan, val)


# ---------------------------------------------------------------------------
# Cache accessors.  The layouts are this library's storage format:
#   K: [page][group][block-in-page][24 dim chunks][8 tokens][8 dims]
#   V: [page][group][block-in-page][192 dims][8 tokens]
#   index keys: [page][block-in-page][256]
# ---------------------------------------------------------------------------

def _unit_offset(page: int, g: int, blk_in_page: int) -> int:
    return ((page * G + g) * BPP + blk_in_page) * (BS * D)


def k_rows(k_cache_bits: np.ndarray, page_row: np.ndarray, positions, g: int) -> np.ndarray:
    """K rows (float64 [n][192]) of the given token positions of one sequence, group g."""
    flat = np.asarray(k_cache_bits).reshape(-1)
    out = np.empty((len(positions), D), dtype=np.float64)
    d = np.arange(D)
    for i, pos in enumerate(positions):
        page = int(page_row[pos // PS])
        r = pos % PS
        base = _unit_offset(page, g, r // BS)
        t = r % BS
        out[i] = bf16_to_f64(flat[base + (d // 8) * 64 + t * 8 + (d % 8)])
    return out


def v_rows(v_cache_bits: np.ndarray, page_row: np.ndarray, positions, g: int) -> np.ndarray:
    """V rows (float64 [n][192]) of the given token positions of one sequence, group g."""
    flat = np.asarray(v_cache_bits).reshape(-1)
    out = np.empty((len(positions), D), dtype=np.float64)
    d = np.arange(D)
    for i, pos in enumerate(positions):
        page = int(page_row[pos // PS])
        r = pos % PS
        base = _unit_offset(page, g, r // BS)
        out[i] = bf16_to_f64(flat[base + d * 8 + (r % BS)])
    return out


# One-byte (OCP FP8 E4M3) K/V caches: the value is code * scale, with a scale
# per cache (per layer).  Layouts:
#   K: [page][group][block-in-page][3 dim-blocks][8 tokens][64 dims]
#      (token k, dim d at (d // 64) * 512 + k * 64 + d % 64 inside its block)
#   V: [page][group][block-in-page][192 dims][8 tokens]
FP8_UNIT = BS * D
_K8_DIM_OFFSET = (np.arange(D) // 64) * (BS * 64) + np.arange(D) % 64


def k_rows_fp8(k_codes: np.ndarray, page_row: np.ndarray, positions, g: int, k_scale: float) -> np.ndarray:
    """K rows (float64 [n][192]) of the given token positions, group g, from E4M3 codes."""
    flat = np.asarray(k_codes).reshape(-1)
    out = np.empty((len(positions), D), dtype=np.float64)
    for i, pos in enumerate(positions):
        page = int(page_row[pos // PS])
        r = pos % PS
        base = ((page * G + g) * BPP + r // BS) * FP8_UNIT + (r % BS) * 64
        out[i] = fp8_e4m3_to_f64(flat[base + _K8_DIM_OFFSET]) * k_scale
    return out


def v_rows_fp8(v_codes: np.ndarray, page_row: np.ndarray, positions, g: int, v_scale: float) -> np.ndarray:
    """V rows (float64 [n][192]) of the given token positions, group g, from E4M3 codes."""
    flat = np.asarray(v_codes).reshape(-1)
    out = np.empty((len(positions), D), dtype=np.float64)
    d = np.arange(D)
    for i, pos in enumerate(positions):
        page = int(page_row[pos // PS])
        r = pos % PS
        base = ((page * G + g) * BPP + r // BS) * FP8_UNIT
        out[i] = fp8_e4m3_to_f64(flat[base + d * BS + (r % BS)]) * v_scale
    return out


def index_keys(kidx_bits: np.ndarray, page_row: np.ndarray, n_blocks: int, fp8: bool = False) -> np.ndarray:
    """Index keys (float64 [n_blocks][256]) of blocks 0 .. n_blocks-1 of one sequence.

    The cache holds bf16 bit patterns (uint16), or with fp8=True one-byte OCP
    E4M3 codes (uint8), as [page][8 blocks][256]."""
    arr = np.asarray(kidx_bits).reshape(-1, BPP, DI)
    decode = fp8_e4m3_to_f64 if fp8 else bf16_to_f64
    out = np.empty((n_blocks, arr.shape[2]), dtype=np.float64)
    for beta in range(n_blocks):
        out[beta] = decode(arr[int(page_row[beta // BPP]), beta % BPP])
    return out


# ---------------------------------------------------------------------------
# Indexer score and top-k block selection
# (SGLang blog, "Hybrid Attention" and "Kernels from StepFun"; open-weights
#  blog, config table and "What sparse attention does and doesn't save")
# ---------------------------------------------------------------------------

def current_block(p: int) -> int:
    """Index of the 8-token block that holds position p."""
    return p // BS


def indexer_scores(q_idx: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """s[b] = sum_d q_idx[d] * keys[b, d] for every historical block b (plain dot product)."""
    s = np.asarray(keys, dtype=np.float64) @ np.asarray(q_idx, dtype=np.float64)
    return s + 0.0  # -0.0 becomes +0.0, so the two zeros rank as equal


def select_top_blocks(scores: np.ndarray, k: int) -> np.ndarray:
    """Up to k blocks with the largest scores; ties go to the lower block index.

    Returns the chosen block ids in ascending order, padded with -1 to length k.
    """
    n = len(scores)
    order = np.lexsort((np.arange(n), -np.asarray(scores, dtype=np.float64)))
    chosen = np.sort(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(chosen)] = chosen
    return out


def indexer_topk_token(q_idx: np.ndarray, keys_hist: np.ndarray, k: int) -> np.ndarray:
    """Selection of one query token from the keys of its historical blocks."""
    if len(keys_hist) == 0:
        return np.full(k, -1, dtype=np.int64)
    return select_top_blocks(indexer_scores(q_idx, keys_hist), k)


# ---------------------------------------------------------------------------
# Attention over a token set (exact softmax, GQA head->group map h // 16)
# ---------------------------------------------------------------------------

def attend(q_heads: np.ndarray, k_by_group, v_by_group, scale: float):
    """Softmax attention of 64 heads over one token set.

    q_heads: [64][192]; k_by_group[g], v_by_group[g]: [n][192] rows of the
    attended tokens for KV group g (same token order in K and V).
    Returns O [64][192] and the natural-log lse [64].
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    O = np.zeros((q_heads.shape[0], q_heads.shape[1]), dtype=np.float64)
    lse = np.zeros(q_heads.shape[0], dtype=np.float64)
    for h in range(q_heads.shape[0]):
        g = h // HEADS_PER_GROUP
        z = scale * (k_by_group[g] @ q_heads[h])
        m = z.max()
        e = np.exp(z - m)
        ssum = e.sum()
        O[h] = (e / ssum) @ v_by_group[g]
        lse[h] = m + np.log(ssum)
    return O, lse


def sparse_token_positions(sel: np.ndarray, p: int) -> np.ndarray:
    """Tokens a sparse-layer query at position p attends: the selected blocks' tokens
    and the current block's tokens up to p."""
    cb = current_block(p)
    blocks = [int(b) for b in sel if b >= 0]
    pos = [BS * b + i for b in blocks for i in range(BS)]
    pos += list(range(BS * cb, p + 1))
    return np.asarray(pos, dtype=np.int64)


def window_positions(p: int, window: int) -> np.ndarray:
    """Tokens a sliding-window query at position p attends: max(0, p-window+1) .. p."""
    return np.arange(max(0, p - window + 1), p + 1, dtype=np.int64)


def attend_positions(q_heads, k_cache_bits, v_cache_bits, page_row, positions, scale, fp8_scales=None):
    """Attention of one token over the given positions of its sequence. With
    fp8_scales = (k_scale, v_scale) the caches hold E4M3 codes (one-byte layouts)."""
    if fp8_scales is None:
        ks = [k_rows(k_cache_bits, page_row, positions, g) for g in range(G)]
        vs = [v_rows(v_cache_bits, page_row, positions, g) for g in range(G)]
    else:
        ks = [k_rows_fp8(k_cache_bits, page_row, positions, g, fp8_scales[0]) for g in range(G)]
        vs = [v_rows_fp8(v_cache_bits, page_row, positions, g, fp8_scales[1]) for g in range(G)]
    return attend(q_heads, ks, vs, scale)


# ---------------------------------------------------------------------------
# Split-K merge (SGLang blog, "Kernels from StepFun": partitions + merge)
# ---------------------------------------------------------------------------

def merge(part_o: np.ndarray, part_lse: np.ndarray):
    """Combine per-partition (O, lse) into the result over the union of partitions.

    part_o: [S][heads][dim] normalised partial outputs; part_lse: [S][heads].
    Partitions with lse = -inf (nothing attended) carry no weight: they are left
    out of the sum, so whatever their part_o holds does not matter.
    """
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    out = np.zeros(part_o.shape[1:], dtype=np.float64)
    lse = np.full(part_lse.shape[1], -np.inf)
    for h in range(part_lse.shape[1]):
        live = np.isfinite(part_lse[:, h])
        if not live.any():
            continue
        M = part_lse[live, h].max()
        w = np.exp(part_lse[live, h] - M)
        out[h] = (w[:, None] * part_o[live, h, :]).sum(axis=0) / w.sum()
        lse[h] = M + np.log(w.sum())
    return out, lse


# ---------------------------------------------------------------------------
# Whole-token drivers over a paged workload (host copies of the caches)
# ---------------------------------------------------------------------------

def attend_positions_by_group(q_heads, k_cache_bits, v_cache_bits, page_row, positions_by_group, scale,
                              fp8_scales=None):
    """Attention of one token where KV group g attends its own token positions
    positions_by_group[g] (the heads of group g see only those)."""
    ks, vs = [], []
    for g in range(G):
        pos = positions_by_group[g]
        if fp8_scales is None:
            ks.append(k_rows(k_cache_bits, page_row, pos, g))
            vs.append(v_rows(v_cache_bits, page_row, pos, g))
        else:
            ks.append(k_rows_fp8(k_cache_bits, page_row, pos, g, fp8_scales[0]))
            vs.append(v_rows_fp8(v_cache_bits, page_row, pos, g, fp8_scales[1]))
    return attend(q_heads, ks, vs, scale)


# Per-KV-group selection (open-weights blog, "What sparse attention does and
# doesn't save": each KV group picks its own up-to-512 historical blocks plus
# the current one). The index key stays one per block; each group brings its
# own index query, scores the same keys and keeps its own top-k.

def sparse_layer_token_grouped(q_heads_bits, q_idx_bits_by_group, k_cache_bits, v_cache_bits, kidx_bits,
                               page_row, p: int, k: int, scale: float, fp8_scales=None, kidx_fp8=False):
    """Per-group indexer -> top-k -> attention, for one query token.
    q_idx_bits_by_group: [4][256] bf16 bits. Returns (sel [4][k], O [64][192], lse [64])."""
    cb = current_block(p)
    keys = index_keys(kidx_bits, page_row, cb, fp8=kidx_fp8)
    sels = np.stack([indexer_topk_token(bf16_to_f64(q_idx_bits_by_group[g]), keys, k) for g in range(G)])
    O, lse = sparse_attention_token_grouped(q_heads_bits, k_cache_bits, v_cache_bits, page_row, sels, p, scale,
                                            fp8_scales)
    return sels, O, lse


def sparse_attention_token_grouped(q_heads_bits, k_cache_bits, v_cache_bits, page_row, sels, p, scale,
                                   fp8_scales=None):
    """Attention of one query token given each group's selected blocks (sels [4][k])."""
    pos = [sparse_token_positions(np.asarray(sels[g]), p) for g in range(G)]
    return attend_positions_by_group(bf16_to_f64(q_heads_bits), k_cache_bits, v_cache_bits, page_row, pos,
                                     scale, fp8_scales)


def sparse_layer_token(q_heads_bits, q_idx_bits, k_cache_bits, v_cache_bits, kidx_bits,
                       page_row, p: int, k: int, scale: float):
    """Indexer -> top-k -> attention over selected + current block, for one query token."""
    cb = current_block(p)
    keys = index_keys(kidx_bits, page_row, cb)
    sel = indexer_topk_token(bf16_to_f64(q_idx_bits), keys, k)
    pos = sparse_token_positions(sel, p)
    O, lse = attend_positions(bf16_to_f64(q_heads_bits), k_cache_bits, v_cache_bits,
                              page_row, pos, scale)
    return sel, O, lse


def sparse_attention_token(q_heads_bits, k_cache_bits, v_cache_bits, page_row, sel, p, scale, fp8_scales=None):
    """Attention of one query token given its selected blocks."""
    pos = sparse_token_positions(np.asarray(sel), p)
    return attend_positions(bf16_to_f64(q_heads_bits), k_cache_bits, v_cache_bits,
                            page_row, pos, scale, fp8_scales)


def swa_token(q_heads_bits, k_cache_bits, v_cache_bits, page_row, p: int, window: int,
              scale: float, fp8_scales=None):
    """Sliding-window attention of one query token."""
    pos = window_positions(p, window)
    return attend_positions(bf16_to_f64(q_heads_bits), k_cache_bits, v_cache_bits,
                            page_row, pos, scale, fp8_scales)
