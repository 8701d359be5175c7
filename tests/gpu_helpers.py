"""Helpers for the GPU parity tests: run the library through its binding and
compute the oracle's answer for the same device-resident inputs, reading back
only the pages each token needs."""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import sa_oracle as O
from sparse_block_indexed_amd import inputs as I

SCALE = 1.0 / math.sqrt(192.0)
SPLITS_BY_LENGTH = 0       # a token's partition count follows its own list length (batch invariant)
SPLITS_FILL_GPU = -1       # the count follows the call's size (the benchmark's launch configuration)
MAX_ABS = 2e-2
REL_RMS = 5e-3
LSE_ABS = 1e-3


def device_tables(wl, device="cuda"):
    return wl.device_ints(device)


def _kv_args(wl, kv_fp8):
    """(k_cache, v_cache, scale kwargs) of the bf16 caches, or of kv_fp8 =
    (k_codes, v_codes, k_scale, v_scale)."""
    if kv_fp8 is None:
        return wl.k_cache, wl.v_cache, {}
    kc, vc, ks, vs = kv_fp8
    return kc, vc, dict(k_scale=ks, v_scale=vs)


def run_sparse_layer(wl, topk=512, num_splits=0, scale=SCALE, tabs=None, kidx=None, kv_fp8=None):
    from sparse_block_indexed_amd import ops
    pt, sl, qs, qp = tabs if tabs is not None else device_tables(wl)
    sel = ops.indexer_topk(wl.q_idx, wl.k_idx_cache if kidx is None else kidx, pt, sl, qs, qp, topk)
    kc, vc, kw = _kv_args(wl, kv_fp8)
    out, lse = ops.sparse_decode(wl.q, kc, vc, pt, sl, qs, qp, sel, scale, num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    return sel, out, lse


def run_swa(wl, window=512, num_splits=0, scale=SCALE, tabs=None, kv_fp8=None):
    from sparse_block_indexed_amd import ops
    pt, sl, qs, qp = tabs if tabs is not None else device_tables(wl)
    kc, vc, kw = _kv_args(wl, kv_fp8)
    out, lse = ops.swa_decode(wl.q, kc, vc, pt, sl, qs, qp, window, scale, num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    return out, lse


class OracleView:
    """Host-side oracle over a device workload; caches each sequence's index keys.
    With kidx_fp8 (uint8 E4M3 codes) the index keys are read from it instead;
    with kv_fp8 = (k_codes, v_codes, k_scale, v_scale) the attention reads the
    one-byte caches."""

    def __init__(self, wl, kidx_fp8=None, kv_fp8=None):
        self.wl = wl
        self.kidx_fp8 = kidx_fp8
        self.kv_fp8 = kv_fp8
        self._keys = {}

    def keys(self, b, cb):
        have = self._keys.get(b)
        if have is None or have.shape[0] < cb:
            npg = (cb + 7) // 8
            pages = torch.as_tensor(self.wl.page_table[b, :npg].astype(np.int64), device=self.wl.k_idx_cache.device)
            if self.kidx_fp8 is None:
                kidx = I.bf16_bits(self.wl.k_idx_cache.index_select(0, pages))
                have = O.index_keys(kidx, np.arange(npg), npg * 8)
            else:
                kidx = self.kidx_fp8.index_select(0, pages).cpu().numpy()
                have = O.index_keys(kidx, np.arange(npg), npg * 8, fp8=True)
            self._keys[b] = have
        return have[:cb]

    def selection(self, t, topk=512):
        b, p = int(self.wl.q_seq[t]), int(self.wl.q_pos[t])
        cb = p // 8
        q = O.bf16_to_f64(I.bf16_bits(self.wl.q_idx[t]))
        return O.indexer_topk_token(q, self.keys(b, cb), topk)

    def attention(self, t, positions, scale=SCALE):
        wl = self.wl
        b = int(wl.q_seq[t])
        row = wl.page_table[b]
        logical = np.unique(np.asarray(positions) // 64)
        phys = row[logical].astype(np.int64)
        dev = wl.k_cache.device
        idx = torch.as_tensor(phys, device=dev)
        compact = np.full(row.shape[0], -1, dtype=np.int64)
        compact[logical] = np.arange(len(logical))
        q = O.bf16_to_f64(I.bf16_bits(wl.q[t]))
        if self.kv_fp8 is not None:
            k8, v8, ks, vs = self.kv_fp8
            kc = k8.index_select(0, idx).cpu().numpy()
            vc = v8.index_select(0, idx).cpu().numpy()
            return O.attend_positions(q, kc, vc, compact, positions, scale, fp8_scales=(ks, vs))
        kc = I.bf16_bits(wl.k_cache.index_select(0, idx))
        vc = I.bf16_bits(wl.v_cache.index_select(0, idx))
        return O.attend_positions(q, kc, vc, compact, positions, scale)

    def selection_grouped(self, t, q_idx_groups, topk=512):
        """Per-group selections [4][topk] of token t for index queries [n_tok][4][256]."""
        b, p = int(self.wl.q_seq[t]), int(self.wl.q_pos[t])
        keys = self.keys(b, p // 8)
        qg = q_idx_groups[t]
        return np.stack([O.indexer_topk_token(O.bf16_to_f64(I.bf16_bits(qg[g])), keys, topk) for g in range(4)])

    def sparse_grouped(self, t, sels, scale=SCALE):
        wl = self.wl
        b, p = int(wl.q_seq[t]), int(wl.q_pos[t])
        row = wl.page_table[b]
        positions = [O.sparse_token_positions(np.asarray(sels[g]), p) for g in range(4)]
        logical = np.unique(np.concatenate(positions) // 64)
        idx = torch.as_tensor(row[logical].astype(np.int64), device=wl.k_cache.device)
        compact = np.full(row.shape[0], -1, dtype=np.int64)
        compact[logical] = np.arange(len(logical))
        q = O.bf16_to_f64(I.bf16_bits(wl.q[t]))
        if self.kv_fp8 is not None:
            k8, v8, ks, vs = self.kv_fp8
            kc, vc = k8.index_select(0, idx).cpu().numpy(), v8.index_select(0, idx).cpu().numpy()
            return O.attend_positions_by_group(q, kc, vc, compact, positions, scale, fp8_scales=(ks, vs))
        kc = I.bf16_bits(wl.k_cache.index_select(0, idx))
        vc = I.bf16_bits(wl.v_cache.index_select(0, idx))
        return O.attend_positions_by_group(q, kc, vc, compact, positions, scale)

    def sparse(self, t, sel, scale=SCALE):
        return self.attention(t, O.sparse_token_positions(np.asarray(sel), int(self.wl.q_pos[t])), scale)

    def swa(self, t, window=512, scale=SCALE):
        return self.attention(t, O.window_positions(int(self.wl.q_pos[t]), window), scale)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return O.bf16_to_f64(I.bf16_bits(t))


def assert_close_outputs(got_out, got_lse, ref_out, ref_lse, what=""):
    """The output tolerance: max-abs 2e-2 and relative RMS 5e-3 over the compared
    set against the fp64 oracle; lse within 1e-3."""
    got_out = np.asarray(got_out, dtype=np.float64)
    ref_out = np.asarray(ref_out, dtype=np.float64)
    assert np.isfinite(got_out).all(), f"{what}: non-finite output"
    err = np.abs(got_out - ref_out)
    rel = np.sqrt((err ** 2).sum()) / max(np.sqrt((ref_out ** 2).sum()), 1e-300)
    assert err.max() <= MAX_ABS, f"{what}: max abs {err.max():.3e}"
    assert rel <= REL_RMS, f"{what}: rel rms {rel:.3e}"
    if got_lse is not None:
        gl = np.asarray(got_lse, dtype=np.float64)
        rl = np.asarray(ref_lse, dtype=np.float64)
        same = gl == rl                      # equal infinities (heads that attended nothing) count as equal
        with np.errstate(invalid="ignore"):
            dl = np.where(same, 0.0, np.abs(gl - rl))
        assert not np.isnan(dl).any() and dl.max() <= LSE_ABS, f"{what}: lse max abs {dl.max():.3e}"
    return err.max(), rel
