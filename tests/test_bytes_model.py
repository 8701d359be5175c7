"""The byte arithmetic printed in the Step 5 Preview open-weights blog
(sections "Why GQA, and what it costs" and "What sparse attention does and
doesn't save"), reproduced by the bytes model to the precision printed there."""
import numpy as np

from sparse_block_indexed_amd import bytes_model as B


def test_kv_bytes_per_token_per_layer():
    assert B.kv_bytes_per_token_per_layer() == 3072            # printed: 3,072 bytes


def test_session_sizes():
    assert round(B.kv_bytes_per_token() / 1000, 1) == 70.7      # about 70.7 KB per token
    assert round(B.session_kv_bytes(131072) / 1e9, 1) == 9.3    # 128K session about 9.3 GB
    assert round(B.session_kv_bytes(1048576) / 1e9) == 74       # 1M session about 74 GB


def test_decode_step_reads_at_1m():
    assert round(B.swa_read_bytes_per_step() / 1e6) == 109      # sliding window about 109 MB
    assert round(B.selected_read_bytes_per_step() / 1e6, -1) == 290   # selected about 290 MB
    one = B.indexer_read_bytes_per_step(1048576, key_bytes=1) / 1e9
    two = B.indexer_read_bytes_per_step(1048576, key_bytes=2) / 1e9
    assert round(one, 1) == 0.8 and round(two, 1) == 1.5        # 0.8 to 1.5 GB
    assert B.indexer_read_bytes_per_step(1048576) > B.selected_read_bytes_per_step()


def test_launch_bytes_count_distinct_blocks():
    q_seq = np.array([0, 0])
    q_pos = np.array([100, 101])        # same current block 12
    sel = np.array([[0, 3, -1], [3, 5, -1]])
    # distinct blocks {0, 3, 5, 12}: 4 units x 4 groups x (K + V) x 3072 B
    expect = 4 * 4 * 2 * 3072 + 2 * 64 * 192 * 2 * 2 + sel.size * 4 + 2 * 64 * 4
    assert B.sparse_attention_bytes(q_seq, q_pos, sel) == expect


def test_grouped_launch_bytes_count_distinct_blocks_per_group():
    q_seq = np.array([0, 0])
    q_pos = np.array([100, 101])        # current block 12 for both
    sel = np.full((2, 4, 3), -1)
    sel[0, 0, :2] = [0, 3]
    sel[1, 0, :2] = [3, 5]               # group 0: {0, 3, 5, 12} -> 4 units
    sel[0, 1, :1] = [7]                  # group 1: {7, 12} -> 2 units
    # groups 2, 3: current block only -> 1 unit each
    units = 4 + 2 + 1 + 1
    expect = units * 2 * 3072 + 2 * 64 * 192 * 2 * 2 + sel.size * 4 + 2 * 64 * 4
    assert B.sparse_attention_bytes_grouped(q_seq, q_pos, sel) == expect
    # one-byte caches halve the unit
    assert B.sparse_attention_bytes_grouped(q_seq, q_pos, sel, kv_bytes=1) == expect - units * 2 * 1536
    # all groups choosing alike: the shared form's count
    same = np.repeat(np.array([[0, 3, -1], [3, 5, -1]])[:, None, :], 4, axis=1)
    assert B.sparse_attention_bytes_grouped(q_seq, q_pos, same) == \
        B.sparse_attention_bytes(q_seq, q_pos, same[:, 0]) + 2 * 3 * 3 * 4
