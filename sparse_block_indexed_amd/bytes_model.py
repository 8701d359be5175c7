"""Byte and flop arithmetic of the sparse layer (no attention arithmetic here).

Two uses:
* the KV and read-volume arithmetic of the Step 5 Preview open-weights blog
  (sections "Why GQA, and what it costs" and "What sparse attention does and
  doesn't save"), reproduced so that tests can pin it to the printed figures;
* the algorithmic bytes and flops one launch of each kernel must move, which
  the benchmark divides by measured time.
"""
from __future__ import annotations

import numpy as np

G, D, DI, H = 4, 192, 256, 64
BS, PS = 8, 64
BF16 = 2
UNIT_BYTES = BS * D * BF16          # one (page, group, block) unit of K or V: 3072 B


def kv_bytes_per_token_per_layer(groups: int = G, head_dim: int = D, elem_bytes: int = BF16) -> int:
    """K and V of every KV group for one token in one full-attention layer."""
    return 2 * groups * head_dim * elem_bytes


def kv_bytes_per_token(sparse_layers: int = 23) -> int:
    return sparse_layers * kv_bytes_per_token_per_layer()


def session_kv_bytes(tokens: int, sparse_layers: int = 23) -> int:
    return tokens * kv_bytes_per_token(sparse_layers)


def swa_read_bytes_per_step(swa_layers: int = 69, window: int = 512) -> int:
    """Window reads of all sliding-window layers for one decode token."""
    return swa_layers * window * kv_bytes_per_token_per_layer()


def selected_read_bytes_per_step(sparse_layers: int = 23, topk: int = 512) -> int:
    """Selected blocks plus the current block, all sparse layers, one decode token."""
    return sparse_layers * (topk + 1) * BS * kv_bytes_per_token_per_layer()


def indexer_read_bytes_per_step(context: int, sparse_layers: int = 23, key_bytes: int = BF16) -> int:
    """Index keys scanned per decode token: one DI-wide key per 8-token block."""
    return sparse_layers * (context // BS) * DI * key_bytes


# ---------------------------------------------------------------------------
# Per-launch algorithmic traffic of this library's kernels
# ---------------------------------------------------------------------------

def indexer_topk_bytes(q_seq: np.ndarray, q_pos: np.ndarray, topk: int, key_bytes: int = BF16,
                       queries_per_token: int = 1) -> int:
    """Each sequence's index keys once (up to its longest history; key_bytes per
    value), the index queries, and the selection written."""
    q_seq = np.asarray(q_seq)
    q_pos = np.asarray(q_pos)
    total = 0
    for b in np.unique(q_seq):
        total += int((q_pos[q_seq == b] // BS).max()) * DI * key_bytes
    total += len(q_seq) * queries_per_token * DI * BF16          # index queries
    total += len(q_seq) * queries_per_token * topk * 4           # sel_idx (int32)
    return total


def unique_kv_units(q_seq, q_pos, blocks_of_token) -> int:
    """Number of distinct (sequence, block) pairs the attention must read."""
    seen = set()
    for t in range(len(q_seq)):
        b = int(q_seq[t])
        for blk in blocks_of_token(t):
            seen.add((b, int(blk)))
    return len(seen)


def sparse_attention_bytes(q_seq, q_pos, sel_idx: np.ndarray, num_heads: int = H,
                           write_lse: bool = True, kv_bytes: int = BF16) -> int:
    """Distinct K and V units of the selected + current blocks (all 4 groups), Q read,
    O written (bf16), selection read, lse written. kv_bytes = 1 for one-byte caches."""
    sel_idx = np.asarray(sel_idx)
    n_tok = len(q_seq)

    def blocks(t):
        s = sel_idx[t]
        return list(s[s >= 0]) + [int(q_pos[t]) // BS]

    units = unique_kv_units(q_seq, q_pos, blocks)
    total = units * G * 2 * BS * D * kv_bytes
    total += n_tok * num_heads * D * BF16 * 2       # Q in, O out
    total += sel_idx.size * 4
    if write_lse:
        total += n_tok * num_heads * 4
    return total


def sparse_attention_bytes_grouped(q_seq, q_pos, sel_idx: np.ndarray, num_heads: int = H,
                                   write_lse: bool = True, kv_bytes: int = BF16) -> int:
    """Per-KV-group selection (sel_idx [n_tok][4][k]): distinct (sequence, group,
    block) K and V units, Q read, O written, the selections read, lse written."""
    sel_idx = np.asarray(sel_idx)
    n_tok = len(q_seq)
    units = 0
    for g in range(G):
        def blocks(t, g=g):
            s = sel_idx[t, g]
            return list(s[s >= 0]) + [int(q_pos[t]) // BS]
        units += unique_kv_units(q_seq, q_pos, blocks)
    total = units * 2 * BS * D * kv_bytes
    total += n_tok * num_heads * D * BF16 * 2
    total += sel_idx.size * 4
    if write_lse:
        total += n_tok * num_heads * 4
    return total


def swa_attention_bytes(q_seq, q_pos, window: int, num_heads: int = H, write_lse: bool = True,
                        kv_bytes: int = BF16) -> int:
    """Distinct K and V blocks touched by the windows, Q read, O written."""
    def blocks(t):
        p = int(q_pos[t])
        lo = max(0, p - window + 1)
        return range(lo // BS, p // BS + 1)

    units = unique_kv_units(q_seq, q_pos, blocks)
    n_tok = len(q_seq)
    total = units * G * 2 * BS * D * kv_bytes + n_tok * num_heads * D * BF16 * 2
    if write_lse:
        total += n_tok * num_heads * 4
    return total


def sparse_attention_flops(q_pos, sel_idx: np.ndarray, num_heads: int = H) -> int:
    """QK^T and PV flops over the attended tokens (2 flop per multiply-add)."""
    sel_idx = np.asarray(sel_idx)
    total = 0
    for t in range(len(q_pos)):
        p = int(q_pos[t])
        n_attended = int((sel_idx[t] >= 0).sum()) * BS + (p - (p // BS) * BS + 1)
        total += num_heads * n_attended * D * 2 * 2
    return total


def indexer_flops(q_pos) -> int:
    return int(sum((int(p) // BS) * DI * 2 for p in q_pos))


def swa_attention_flops(q_pos, window: int, num_heads: int = H) -> int:
    """QK^T and PV flops over each token's window."""
    return int(sum(num_heads * (int(p) - max(0, int(p) - window + 1) + 1) * D * 2 * 2 for p in q_pos))
