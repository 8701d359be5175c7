"""Seeded synthetic inputs and the paged-cache storage format.

This module is shared by the oracle tests, the GPU tests and the benchmark.
It holds no arithmetic of the attention method: it draws random values,
builds page tables and packs per-token rows into the documented cache layout.

Shapes follow the model description in "Step 5 Preview: Day-0 Inference and
RL Support with SGLang and Miles" (section "Hybrid Attention": 8-token blocks,
top-512 blocks, 512-token window; serving flags: page size 64, bf16 KV) and the
config table of the Step 5 Preview open-weights blog (section "What the config
says": 64 query heads, 4 KV groups, head dim 192, one 256-dim index key per
8-token block).

Cache layouts (all bf16, all contiguous; the pages fix none of them):

* ``k_cache`` ``[num_pages][4 groups][8 blocks][24 chunks][8 tokens][8 dims]``
  -- inside one 8-token block of one group, dims are cut into 24 chunks of 8;
  the 8 tokens of one chunk are adjacent (16 bytes each).
* ``v_cache`` ``[num_pages][4 groups][8 blocks][192 dims][8 tokens]``
  -- inside one block the 8 values of one dim are adjacent.
* ``k_idx_cache`` ``[num_pages][8 blocks][256]`` -- one index key per block.

Every (page, group, block) unit of K or V is 3072 contiguous bytes, so the
unit that block selection picks is also the unit of every HBM read.

One-byte (OCP FP8 E4M3) forms, 1536-byte units with the same addressing:

* K ``[num_pages][4][8 blocks][3 dim-blocks][8 tokens][64 dims]`` -- dim d of a
  token sits in dim-block d // 64 at d % 64, so the 4 tokens x 64 dims that one
  load step of the attention kernel reads are 256 contiguous bytes.
* V ``[num_pages][4][8 blocks][192 dims][8 tokens]``, as in bf16.
* index keys ``[num_pages][8 blocks][256]``.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

# shape constants of the sparse layer
H = 64          # query heads
G = 4           # KV groups
R = H // G      # query heads per group
D = 192         # head dim of K and V
DI = 256        # indexer dim
BS = 8          # tokens per index block
PS = 64         # tokens per cache page
BPP = PS // BS  # blocks per page
TOPK = 512
WINDOW = 512
BLOCK_ELEMS = BS * D  # bf16 elements in one (page, group, block) unit


@dataclasses.dataclass
class WorkloadSpec:
    name: str
    batch: int
    seq_lens: Optional[List[int]] = None      # explicit lengths, or
    seq_len_range: Optional[tuple] = None     # inclusive uniform range
    q_per_seq: int = 1                        # query tokens at the end of each sequence
    identity_pages: bool = False              # contiguous (unpermuted) page table
    idx_lo: int = -4                          # index inputs: integers in [idx_lo, idx_hi]
    idx_hi: int = 4
    kv_dist: str = "normal"                   # "normal" N(0,1) bf16
    q_positions: Optional[List[int]] = None   # explicit positions for 1-seq prefill chunks
    spare_pages: int = 0


# The five workloads, by name, with their default seeds: decode at 8K, MTP
# verify at 96K-128K (the headline), sliding-window decode at 16K-32K, decode
# at 1M, and a 16K prefill chunk.
WORKLOADS = {
    "decode_8k_b1": (WorkloadSpec("decode_8k_b1", batch=1, seq_lens=[8192], q_per_seq=1, identity_pages=True), 0),
    "mtp_verify_128k_b64": (WorkloadSpec("mtp_verify_128k_b64", batch=64, seq_len_range=(98304, 131072),
                                         q_per_seq=4), 1),
    "swa_decode_32k_b64": (WorkloadSpec("swa_decode_32k_b64", batch=64, seq_len_range=(16384, 32768),
                                        q_per_seq=1), 2),
    "decode_1m_b4": (WorkloadSpec("decode_1m_b4", batch=4, seq_lens=[1048576] * 4, q_per_seq=1), 3),
    "prefill_chunk_16k_at_112k": (WorkloadSpec("prefill_chunk_16k_at_112k", batch=1, seq_lens=[131072],
                                               q_per_seq=16384), 4),
}


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    seed: int
    batch: int
    n_tok: int
    num_pages: int
    max_pages_per_seq: int
    seq_lens: np.ndarray      # int32 [batch]
    page_table: np.ndarray    # int32 [batch][max_pages_per_seq], -1 where unused
    q_seq: np.ndarray         # int32 [n_tok]
    q_pos: np.ndarray         # int32 [n_tok]
    q: torch.Tensor           # bf16 [n_tok][64][192]
    q_idx: torch.Tensor       # bf16 [n_tok][256]
    k_cache: torch.Tensor     # bf16 [num_pages][4][8][1536]
    v_cache: torch.Tensor     # bf16 [num_pages][4][8][1536]
    k_idx_cache: torch.Tensor # bf16 [num_pages][8][256]

    def device_ints(self, device):
        """page_table, seq_lens, q_seq, q_pos as int32 tensors on ``device``."""
        mk = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        return mk(self.page_table), mk(self.seq_lens), mk(self.q_seq), mk(self.q_pos)


def _draw_seq_lens(spec: WorkloadSpec, rng: np.random.Generator) -> np.ndarray:
    if spec.seq_lens is not None:
        out = np.asarray(spec.seq_lens, dtype=np.int64)
        assert len(out) == spec.batch
        return out
    lo, hi = spec.seq_len_range
    return rng.integers(lo, hi + 1, size=spec.batch, dtype=np.int64)


def _randn_bf16(shape, gen: torch.Generator, device, chunk_rows: int = 4096) -> torch.Tensor:
    """N(0,1) rounded to bf16, drawn in row chunks so big pools need no fp32 copy."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device,
                                  dtype=torch.float32).to(torch.bfloat16)
    return out


def _randint_bf16(shape, lo: int, hi: int, gen: torch.Generator, device,
                  chunk_rows: int = 8192) -> torch.Tensor:
    """Integers uniform in [lo, hi] stored exactly as bf16."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randint(lo, hi + 1, (r1 - r0, flat.shape[1]), generator=gen,
                                    device=device, dtype=torch.int32).to(torch.bfloat16)
    return out


def make_workload(spec: WorkloadSpec, seed: int, device="cpu") -> Workload:
    """Build a seeded workload. Host-side tables come from numpy, tensors from torch."""
    rng = np.random.default_rng(seed)
    seq_lens = _draw_seq_lens(spec, rng)
    pages_per_seq = (seq_lens + PS - 1) // PS
    max_pages = int(pages_per_seq.max())
    num_pages = int(pages_per_seq.sum()) + spec.spare_pages
    perm = np.arange(num_pages) if spec.identity_pages else rng.permutation(num_pages)
    page_table = np.full((spec.batch, max_pages), -1, dtype=np.int32)
    cur = 0
    for b in range(spec.batch):
        n = int(pages_per_seq[b])
        page_table[b, :n] = perm[cur:cur + n]
        cur += n
    q_seq, q_pos = [], []
    for b in range(spec.batch):
        L = int(seq_lens[b])
        nq = min(spec.q_per_seq, L)
        for j in range(nq):
            q_seq.append(b)
            q_pos.append(L - nq + j)
    q_seq = np.asarray(q_seq, dtype=np.int32)
    q_pos = np.asarray(q_pos, dtype=np.int32)
    n_tok = len(q_seq)

    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    q = _randn_bf16((n_tok, H, D), gen, dev)
    q_idx = _randint_bf16((n_tok, DI), spec.idx_lo, spec.idx_hi, gen, dev)
    k_cache = _randn_bf16((num_pages, G, BPP, BLOCK_ELEMS), gen, dev, chunk_rows=1024)
    v_cache = _randn_bf16((num_pages, G, BPP, BLOCK_ELEMS), gen, dev, chunk_rows=1024)
    k_idx_cache = _randint_bf16((num_pages, BPP, DI), spec.idx_lo, spec.idx_hi, gen, dev)
    return Workload(spec=spec, seed=seed, batch=spec.batch, n_tok=n_tok, num_pages=num_pages,
                    max_pages_per_seq=max_pages, seq_lens=seq_lens.astype(np.int32),
                    page_table=page_table, q_seq=q_seq, q_pos=q_pos, q=q, q_idx=q_idx,
                    k_cache=k_cache, v_cache=v_cache, k_idx_cache=k_idx_cache)


def layer_inputs(wl: Workload, seed: int) -> Workload:
    """Another layer over the same sequences: the page table, lengths and query
    positions of ``wl``, with its own seeded Q, K/V caches, index queries and
    index keys (each layer of a model has its own caches)."""
    dev = wl.q.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    spec = wl.spec
    return dataclasses.replace(
        wl, seed=seed,
        q=_randn_bf16(tuple(wl.q.shape), gen, dev),
        q_idx=_randint_bf16(tuple(wl.q_idx.shape), spec.idx_lo, spec.idx_hi, gen, dev),
        k_cache=_randn_bf16(tuple(wl.k_cache.shape), gen, dev, chunk_rows=1024),
        v_cache=_randn_bf16(tuple(wl.v_cache.shape), gen, dev, chunk_rows=1024),
        k_idx_cache=_randint_bf16(tuple(wl.k_idx_cache.shape), spec.idx_lo, spec.idx_hi, gen, dev))


def grouped_index_queries(n_tok: int, seed: int, device="cpu", lo: int = -4, hi: int = 4) -> torch.Tensor:
    """One index query per (token, KV group): integers in [lo, hi] as bf16, [n_tok][4][256]."""
    gen = torch.Generator(device=torch.device(device))
    gen.manual_seed(seed)
    return _randint_bf16((n_tok, G, DI), lo, hi, gen, torch.device(device))


def named_workload(name: str, device="cpu", seed: Optional[int] = None) -> Workload:
    """One of the five named workloads (WORKLOADS), with its default seed unless one is given."""
    spec, default_seed = WORKLOADS[name]
    return make_workload(spec, default_seed if seed is None else seed, device)


# ---------------------------------------------------------------------------
# Storage format: write per-token rows into the cache layouts above.
# ---------------------------------------------------------------------------

def pack_k_rows(k_cache: torch.Tensor, page_table_row: np.ndarray, positions, g: int,
                rows: torch.Tensor) -> None:
    """Store K rows ``rows[i]`` (192 values) of token ``positions[i]``, group ``g``."""
    flat = k_cache.view(-1)
    for i, pos in enumerate(positions):
        page = int(page_table_row[pos // PS])
        r = pos % PS
        base = ((page * G + g) * BPP + r // BS) * BLOCK_ELEMS
        t = r % BS
        d = torch.arange(D)
        idx = base + (d // 8) * 64 + t * 8 + d % 8
        flat[idx.to(flat.device)] = rows[i].to(flat.dtype).to(flat.device)


def pack_v_rows(v_cache: torch.Tensor, page_table_row: np.ndarray, positions, g: int,
                rows: torch.Tensor) -> None:
    """Store V rows ``rows[i]`` (192 values) of token ``positions[i]``, group ``g``."""
    flat = v_cache.view(-1)
    for i, pos in enumerate(positions):
        page = int(page_table_row[pos // PS])
        r = pos % PS
        base = ((page * G + g) * BPP + r // BS) * BLOCK_ELEMS
        t = r % BS
        idx = base + torch.arange(D) * 8 + t
        flat[idx.to(flat.device)] = rows[i].to(flat.dtype).to(flat.device)


def pack_index_key(k_idx_cache: torch.Tensor, page_table_row: np.ndarray, block: int,
                   key: torch.Tensor) -> None:
    """Store the 256-dim index key of 8-token block ``block``."""
    page = int(page_table_row[block // BPP])
    k_idx_cache[page, block % BPP, :] = key.to(k_idx_cache.dtype)


def fp8_e4m3_codes(t: torch.Tensor) -> torch.Tensor:
    """One-byte OCP E4M3 codes (uint8) of a tensor's values, rounded by torch
    (exact for the small integers of the index inputs)."""
    return t.to(torch.float8_e4m3fn).view(torch.uint8)


FP8_UNIT = BS * D   # bytes in one (page, group, block) unit of a one-byte K or V cache


def quantize_kv_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: float, v_scale: float,
                    chunk_pages: int = 2048):
    """One-byte (OCP E4M3) copies of bf16 K/V caches: code = round(x / scale).

    K goes from the bf16 layout [page][group][block][24 chunks][8 tokens][8 dims]
    to the one-byte layout [page][group][block][3 dim-blocks][8 tokens][64 dims];
    V keeps its [192 dims][8 tokens] order. Returns uint8 tensors
    [num_pages][4][8][1536]."""
    P = k_cache.shape[0]
    kq = torch.empty((P, G, BPP, FP8_UNIT), dtype=torch.uint8, device=k_cache.device)
    vq = torch.empty_like(kq)
    for p0 in range(0, P, chunk_pages):
        p1 = min(P, p0 + chunk_pages)
        # chunk c = 8 * j + c' of the bf16 form -> dim-block j, dims 8c' .. 8c'+7 of it
        k = k_cache[p0:p1].view(p1 - p0, G, BPP, 3, 8, BS, 8).permute(0, 1, 2, 3, 5, 4, 6)
        k = k.reshape(p1 - p0, G, BPP, FP8_UNIT).float() / k_scale
        kq[p0:p1] = k.to(torch.float8_e4m3fn).view(torch.uint8)
        v = v_cache[p0:p1].float() / v_scale
        vq[p0:p1] = v.to(torch.float8_e4m3fn).view(torch.uint8)
    return kq, vq


def pack_k_rows_fp8(k_codes: torch.Tensor, page_row: np.ndarray, positions, g: int, rows: torch.Tensor) -> None:
    """Store one-byte K rows (uint8 codes, 192 each) in the one-byte K layout."""
    flat = k_codes.view(-1)
    d = torch.arange(D)
    dim_off = (d // 64) * (BS * 64) + d % 64
    for i, pos in enumerate(positions):
        page = int(page_row[pos // PS])
        r = pos % PS
        base = ((page * G + g) * BPP + r // BS) * FP8_UNIT + (r % BS) * 64
        flat[(base + dim_off).to(flat.device)] = rows[i].to(flat.device)


def pack_v_rows_fp8(v_codes: torch.Tensor, page_row: np.ndarray, positions, g: int, rows: torch.Tensor) -> None:
    """Store one-byte V rows (uint8 codes, 192 each) in the one-byte V layout."""
    flat = v_codes.view(-1)
    for i, pos in enumerate(positions):
        page = int(page_row[pos // PS])
        r = pos % PS
        base = ((page * G + g) * BPP + r // BS) * FP8_UNIT
        idx = base + torch.arange(D) * BS + (r % BS)
        flat[idx.to(flat.device)] = rows[i].to(flat.device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a tensor as a numpy uint16 array (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
