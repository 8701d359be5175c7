// Indexer score + top-k block select for gfx950.
//
// What is computed: SGLang blog "Step 5 Preview: Day-0 Inference and RL Support
// with SGLang and Miles", section "Hybrid Attention" (score summaries of 8-token
// blocks, keep up to 512 historical blocks) and section "Kernels from StepFun"
// (the indexer scores each query against compressed history in the paged
// cache); Step 5 Preview open-weights blog, config table (one 256-dim key per
// 8-token block, top 512 blocks) and "What sparse attention does and doesn't
// save" (the scan over every block key is the read that grows with context).
//
// Pipeline (launches on the caller's stream; a query row is a token, or a
// (token, KV group) with per-group selection):
//  1. score     stream every historical index key of a sequence once per pass
//               and write fp32 scores. Three scorers, by query rows per
//               sequence: up to 4 rows share a pass of the per-token scorer
//               (v_dot2 bf16 -> fp32, eight lanes per key, DPP reduction);
//               16 .. 63 rows take the 16-row MFMA scorer; 64 and more (a
//               prefill chunk) the MFMA GEMM. One-byte E4M3 keys are widened
//               to bf16 on the way in. For histories over kFuseLimit blocks
//               the per-token scorer also lists, for each (row, chunk of
//               blocks), its local candidates: every score at or above the
//               21-bit key prefix that holds the chunk's T-th largest score,
//               in block order, with that prefix's lower edge.
//  2. select    (histories over kFuseLimit) per row: the exact k-th largest key tau_U of
//               the union of the row's candidate lists; a chunk whose edge lies
//               above tau_U may hold unlisted keys >= tau_U and is re-read from
//               its stored scores; the top k of everything >= tau_U (ties at
//               the k-th key taken in block order) are written ascending.
//     finalize  (histories up to kFuseLimit) per row: histogram of the top 11 key bits from
//               register-held scores, everything above the threshold bin is
//               chosen; within the threshold bin the needed keys are taken by
//               rank (larger key, then lower block id) or, for large bins, by
//               two more radix levels, the ids tied at the exact threshold
//               being taken in block order; one scan over the bitmaps places
//               every chosen id, written ascending.
//  Rows that do not fit the LDS structures take an ordered select over all of
//  their stored scores instead.

#include <algorithm>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxGroup = 4;
constexpr int kMaxChunkBlocks = 4096;   // the host never picks a larger score chunk
constexpr int kPagePasses = (kMaxChunkBlocks / kBlocksPerPage + 1 + kThreads - 1) / kThreads;   // page-id reads per thread

__device__ __forceinline__ u32x4 load16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
// index keys are read once per call
__device__ __forceinline__ u32x4 load16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0 maps like +0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Historical block count of query row t as located from its sequence and
// position alone (0 when either is out of range): every read it leads to stays
// inside its table. token_valid() adds the sequence-length check, which decides
// validity only, so kernels issue their reads first and consume it later.
__device__ __forceinline__ int located_blocks(const IndexerArgs& a, int t, int* seq_out, int* pos_out) {
  const int b = a.q_seq[t >> a.q_shift];
  const int p = a.q_pos[t >> a.q_shift];
  *seq_out = b;
  *pos_out = p;
  // no short circuit: both reads are issued together
  return ((b >= 0) & (b < a.batch) & (p >= 0) & (p < a.max_pages * kPageTokens)) ? p >> 3 : 0;
}

// The length of sequence b, read without a branch (b clamped; batch >= 1), so
// that the read is issued at once and waited for only where it is used.
__device__ __forceinline__ int seq_len_of(const IndexerArgs& a, int b) {
  return a.seq_lens[min(max(b, 0), a.batch - 1)];
}

__device__ __forceinline__ bool token_valid(const IndexerArgs& a, int b, int p, int len) {
  return (b >= 0) & (b < a.batch) & (p >= 0) & (p < a.max_pages * kPageTokens) & (p < len);
}

// Historical block count of query row t (0 for an invalid token).
__device__ __forceinline__ int hist_blocks(const IndexerArgs& a, int t, int* seq_out) {
  int p;
  const int n = located_blocks(a, t, seq_out, &p);
  return token_valid(a, *seq_out, p, seq_len_of(a, *seq_out)) ? n : 0;
}

// ---------------------------------------------------------------------------
// wave- and block-wide helpers (NT threads = NT / 64 waves)
// ---------------------------------------------------------------------------

// Inclusive prefix sum over the 64 lanes of a wave, with DPP moves: shifts by
// 1, 2, 4 and 8 lanes inside each row of 16, then lane 15 of each row added to
// the next row and lane 31 to the upper half.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15 (rows 1, 3)
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31 (rows 2, 3)
  return x;
}

// Exclusive suffix sum over the NT threads of the block: the sum of v over
// threads with a larger index. s_tmp holds NT / 64 words.
template <int NT>
__device__ uint32_t block_suffix_exclusive(uint32_t v, uint32_t* s_tmp) {
  const int wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  const uint32_t wave_tot = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
  if ((threadIdx.x & 63) == 63) s_tmp[wave] = x;
  __syncthreads();
  uint32_t above = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) above += w > wave ? s_tmp[w] : 0u;
  __syncthreads();
  return above + wave_tot - x;
}

// Exclusive prefix sum over the NT threads; *total receives the block total.
template <int NT>
__device__ uint32_t block_prefix_exclusive(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if ((threadIdx.x & 63) == 63) s_tmp[wave] = x;
  __syncthreads();
  uint32_t below = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t y = s_tmp[w];
    below += w < wave ? y : 0u;
    tot += y;
  }
  __syncthreads();
  *total = tot;
  return below + x - v;
}

// Among bins h[0..nbins) (a higher bin holds larger keys), find the bin that
// holds the k-th largest element: above < k <= above + h[bin], where above is
// the count in higher bins. Needs sum(h) >= k >= 1, nbins a multiple of 2 NT
// and h 16-byte aligned. Result is broadcast through s_res[0] (bin) and
// s_res[1] (above).
template <int NT>
__device__ void select_bin(const uint32_t* h, int nbins, uint32_t k, uint32_t* s_tmp, uint32_t* s_res) {
  if (threadIdx.x == 0) {   // defined result even for inconsistent input
    s_res[0] = 0u;
    s_res[1] = 0u;
  }
  const int per = nbins / NT;
  const int b0 = threadIdx.x * per;
  uint32_t part = 0;
  if (per % 4 == 0) {   // 16-byte reads: consecutive lanes read consecutive bytes
    for (int i = 0; i < per; i += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(h + b0 + i);
      part += q.x + q.y + q.z + q.w;
    }
  } else {
    for (int i = 0; i < per; i += 2) {
      const uint2 q = *reinterpret_cast<const uint2*>(h + b0 + i);
      part += q.x + q.y;
    }
  }
  uint32_t cum = block_suffix_exclusive<NT>(part, s_tmp);
  if (cum < k && cum + part >= k) {
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t c = h[b0 + i];
      if (cum + c >= k) {
        s_res[0] = (uint32_t)(b0 + i);
        s_res[1] = cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// 2. score
// ---------------------------------------------------------------------------
// Sum over the 8 lanes of an aligned lane octet, with DPP moves (no LDS):
// swap neighbours, swap pairs, then add the mirrored half-row. Every lane of
// the octet ends with the same bits.
__device__ __forceinline__ float octet_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  return v;
}

// Score one step: 8 blocks per wave, 8 lanes per block key (lane q8 holds the
// 16-byte chunks q8 + 8i, i = 0..3, of the key, so each load instruction reads
// whole 128-byte lines).
// Key bytes per block and 16-byte loads per lane (8 lanes per key).
template <bool kFp8> struct KeyFmt {
  static constexpr int kBytes = kFp8 ? kKeyBytes / 2 : kKeyBytes;
  static constexpr int kLoads = kBytes / 128;
};

// Two OCP E4M3 bytes (selected half of a 32-bit word) to a bf16 pair; exact.
template <bool kHiHalf>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHiHalf));
}

// Score one step for NQ query tokens. Lane q8 of a block's octet holds the
// 16-byte chunks q8 + 8i of the key: for bf16 keys 8 dims each (i < 4), for fp8
// keys 16 dims each (i < 2), converted to bf16 pairs before the v_dot2.
template <int NQ, bool kCand, bool kFp8>
__device__ __forceinline__ void score_step(const IndexerArgs& a, const int* hslot, const int* ncb,
                                           const u32x4* s_q, const u32x4 (&kv)[KeyFmt<kFp8>::kLoads], int beta,
                                           bool in, bool ok, int q8, uint32_t (*s_hist)[kHistBins],
                                           float (&sc)[NQ]) {
  // The run's queries are read from LDS; the compiler keeps them in registers
  // across the steps (4 rows: about 60 more VGPRs, still two waves per SIMD;
  // 3% faster than re-reading them at every step).
  const int qoff = q8;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    float s = 0.f;
    if constexpr (!kFp8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 q = s_q[j * (kKeyBytes / 16) + qoff + 8 * i];   // broadcast read
#pragma unroll
        for (int w = 0; w < 4; ++w) s = dot2(kv[i][w], q[w], s);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // key dims (q8 + 8i) * 16 .. +16 <-> query u32x4 2 * (q8 + 8i) and the next
        const u32x4 q0 = s_q[j * (kKeyBytes / 16) + 2 * (qoff + 8 * i)];
        const u32x4 q1 = s_q[j * (kKeyBytes / 16) + 2 * (qoff + 8 * i) + 1];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t qa = w < 2 ? q0[2 * w] : q1[2 * (w - 2)];
          const uint32_t qb = w < 2 ? q0[2 * w + 1] : q1[2 * (w - 2) + 1];
          s = dot2(fp8x2_to_bf16x2<false>(kv[i][w]), qa, s);
          s = dot2(fp8x2_to_bf16x2<true>(kv[i][w]), qb, s);
        }
      }
    }
    s = octet_sum(s);
    sc[j] = ok ? s : -INFINITY;   // an unreadable page ranks last
    // candidate lists: the chunk's histogram of the top 11 key bits (lane j of
    // the octet adds row j's score)
    if constexpr (kCand) {
      if (in && q8 == j && beta < ncb[j]) atomicAdd(&s_hist[hslot[j]][score_key(sc[j]) >> 21], 1u);
    }
  }
}

// One pass over blocks [lo, hi) of one sequence for NQ of its query tokens.
// Each wave owns a contiguous range of blocks, walked in steps of 8 blocks
// (one 8-lane octet per block) and groups of 4 steps. Four steps (16 KB per
// wave) are in flight: after a step is scored its buffer is refilled with the
// same step of the next group. Refills are unconditional (a step past the end
// reads the cache's first key and stores nothing), so each wait leaves the
// other buffers' loads in flight. After a group, lane (octet b, q8 < 4) holds
// the scores of block 8*q8 + b of the group, so one store per token writes 32
// consecutive scores (a whole 128-byte line).
template <int NQ, bool kCand, bool kFp8>
__device__ void score_run(const IndexerArgs& a, const int* tok, const int* hslot, const int* ncb, int lo, int hi,
                          const int32_t* s_pages, const u32x4* s_q, uint32_t (*s_hist)[kHistBins],
                          float (*s_sc)[kCandChunkMax]) {
  constexpr int KB = KeyFmt<kFp8>::kBytes;
  constexpr int KL = KeyFmt<kFp8>::kLoads;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q8 = lane & 7;
  const int sub = lane >> 3;
  const int page0 = lo >> 3;
  const int per_wave = ((hi - lo + 127) / 128) * 32;   // whole groups of 32 blocks
  const int wlo = lo + wave * per_wave;
  const int whi = min(hi, wlo + per_wave);
  if (wlo >= whi) return;
  const int ngroups = (whi - wlo + 31) / 32;
  auto locate = [&](int beta, bool& in, bool& ok) -> const uint8_t* {
    in = beta < whi;
    const int page = in ? s_pages[(beta >> 3) - page0] : -1;
    ok = in && page >= 0 && page < a.num_pages;
    const size_t off = ok ? ((size_t)page * kBlocksPerPage + (beta & 7)) * KB : 0;
    return a.k_idx_cache + off + q8 * 16;
  };
  u32x4 k0[KL], k1[KL], k2[KL], k3[KL];
  bool in0, ok0, in1, ok1, in2, ok2, in3, ok3;
  auto fill = [&](u32x4 (&kv)[KL], int beta, bool& in, bool& ok) {
    const uint8_t* p = locate(beta, in, ok);
#pragma unroll
    for (int i = 0; i < KL; ++i) kv[i] = load16_stream(p + i * 128);
  };
  int base = wlo;   // first block of the current group
  fill(k0, base + sub, in0, ok0);
  fill(k1, base + 8 + sub, in1, ok1);
  fill(k2, base + 16 + sub, in2, ok2);
  fill(k3, base + 24 + sub, in3, ok3);
  for (int g = 0; g < ngroups; ++g, base += 32) {
    float keep[NQ], sc[NQ];
    score_step<NQ, kCand, kFp8>(a, hslot, ncb, s_q, k0, base + sub, in0, ok0, q8, s_hist, sc);
#pragma unroll
    for (int j = 0; j < NQ; ++j) keep[j] = sc[j];
    fill(k0, base + 32 + sub, in0, ok0);
    score_step<NQ, kCand, kFp8>(a, hslot, ncb, s_q, k1, base + 8 + sub, in1, ok1, q8, s_hist, sc);
#pragma unroll
    for (int j = 0; j < NQ; ++j) keep[j] = q8 == 1 ? sc[j] : keep[j];
    fill(k1, base + 40 + sub, in1, ok1);
    score_step<NQ, kCand, kFp8>(a, hslot, ncb, s_q, k2, base + 16 + sub, in2, ok2, q8, s_hist, sc);
#pragma unroll
    for (int j = 0; j < NQ; ++j) keep[j] = q8 == 2 ? sc[j] : keep[j];
    fill(k2, base + 48 + sub, in2, ok2);
    score_step<NQ, kCand, kFp8>(a, hslot, ncb, s_q, k3, base + 24 + sub, in3, ok3, q8, s_hist, sc);
#pragma unroll
    for (int j = 0; j < NQ; ++j) keep[j] = q8 == 3 ? sc[j] : keep[j];
    fill(k3, base + 56 + sub, in3, ok3);
    const int beta = base + 8 * q8 + sub;   // the block whose scores this lane keeps (q8 < 4)
    if (q8 < 4 && beta < whi) {
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        if (beta < ncb[j]) {
          a.scores[(size_t)tok[j] * a.max_hist_blocks + beta] = keep[j];
          if constexpr (kCand) s_sc[hslot[j]][beta - lo] = keep[j];
        }
      }
    }
  }
}

// Local candidate budget of one chunk of a row: twice the chunk's expected
// share of the row's top k, plus 4 (at least 8, at most the chunk).
__device__ __forceinline__ int local_budget(int topk, int chunk_blocks, int row_blocks) {
  const int share = (2 * topk * chunk_blocks + row_blocks - 1) / max(row_blocks, 1);
  return min(chunk_blocks, max(8, share + 4));
}

// Lists the local candidates of one (row, chunk): every key at or above the
// edge E = the lower end of the 21-bit key prefix (two radix levels of 11 and
// 10 bits) that holds the chunk's T-th largest key (E = 0 when n <= T: all n),
// as (key, block id) in ascending block order, and the pair (count, E): every
// key of the chunk >= E is in the list, which holds about T keys plus those
// tied with the T-th at 21 bits. A list longer than the capacity is not
// written; its edge is then 0xFFFFFFFF (no key of the chunk is known to be
// listed), so the select pass re-reads the chunk. hist (the chunk's level-1
// histogram) is overwritten.
__device__ void emit_chunk_candidates(const IndexerArgs& a, int row, int chunk, int nck_all, int lo, int n, int T,
                                      uint32_t* hist, const float* sc, uint32_t* s_tmp, uint32_t* s_res) {
  constexpr int kPer = kCandChunkMax / kThreads;
  // thread i owns entries kPer*i .. kPer*i + kPer - 1 (consecutive blocks)
  const int e0 = (int)threadIdx.x * kPer;
  uint32_t keys[kPer];
#pragma unroll
  for (int i = 0; i < kPer; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(sc + e0 + i);   // past n: read, never listed
    keys[i] = score_key(v.x);
    keys[i + 1] = score_key(v.y);
    keys[i + 2] = score_key(v.z);
    keys[i + 3] = score_key(v.w);
  }
  uint32_t edge = 0;
  if (n > T) {
    select_bin<kThreads>(hist, kHistBins, (uint32_t)T, s_tmp, s_res);
    const uint32_t b = s_res[0], above = s_res[1];
    // second level: bits 20..10 of the keys in bin b
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (e0 + i < n && (keys[i] >> 21) == b) atomicAdd(&hist[(keys[i] >> 10) & (kHistBins - 1)], 1u);
    __syncthreads();
    select_bin<kThreads>(hist, kHistBins, (uint32_t)T - above, s_tmp, s_res);
    edge = b << 21 | s_res[0] << 10;
  }
  uint32_t take = 0, cnt = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool tk = e0 + i < n && keys[i] >= edge;
    take |= tk ? 1u << i : 0u;
    cnt += tk ? 1u : 0u;
  }
  uint32_t total;
  const uint32_t off = block_prefix_exclusive<kThreads>(cnt, s_tmp, &total);
  const bool overflow = total > (uint32_t)a.cand_cap;
  if (!overflow) {
    uint2* dst = a.cand + (size_t)row * a.cand_row_stride + (size_t)chunk * a.cand_cap + off;
    uint32_t pos = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if ((take >> i) & 1u) dst[pos++] = make_uint2(keys[i], (uint32_t)(lo + e0 + i));
  }
  if (threadIdx.x == 0)
    a.cand_meta[(size_t)row * nck_all + chunk] = overflow ? make_uint2(0u, 0xFFFFFFFFu) : make_uint2(total, edge);
  __syncthreads();   // the scratch words of the scan and of select_bin are reused by the next row
}

// Runs of up to GS query tokens of one sequence share a pass over its keys; GS
// is the host's group size, so a one-token decode does not pay for four query
// register sets. With kCand (histories over kFuseLimit blocks) the
// workgroup's chunk of every row is kept in LDS (scores and their histogram)
// and listed as local candidates at the end; shorter rows are selected by
// finalize from their stored scores.
static_assert(kMaxGroup == 4 && kMaxGroup * (kKeyBytes / 16) <= kThreads, "one index-query load per thread");
static_assert(kCandChunkMax % (4 * kThreads) == 0, "whole float4 reads of a chunk row");

template <int GS, bool kCand, bool kFp8>
__global__ __launch_bounds__(kThreads) void score_kernel(IndexerArgs a) {
  __shared__ __align__(16) uint32_t s_hist[kCand ? GS : 1][kCand ? kHistBins : 4];
  __shared__ __align__(16) float s_sc[kCand ? GS : 1][kCand ? kCandChunkMax : 4];
  __shared__ int32_t s_pages[kPagePasses * kThreads];   // page ids of the current run's blocks (padded)
  __shared__ u32x4 s_q[kThreads];   // index queries of the current run (padded)
  __shared__ uint32_t s_tmp[kThreads / 64];
  __shared__ uint32_t s_res[2];
  const int nchunk = (a.max_hist_blocks + a.chunk_blocks - 1) / a.chunk_blocks;
  const int chunk = blockIdx.x % nchunk;
  const int grp = blockIdx.x / nchunk;
  const int t0 = grp * GS;
  const int ng = min(GS, a.n_tok - t0);
  // Rows are located without the sequence-length check: a row past its
  // sequence's length is scored all the same (its lists are never used), and
  // no read waits for that check.
  int seq[kMaxGroup], ncb[kMaxGroup];
  for (int j = 0; j < kMaxGroup; ++j) {
    ncb[j] = 0;
    seq[j] = -1;
    int pj;
    if (j < ng) ncb[j] = min(located_blocks(a, t0 + j, &seq[j], &pj), a.max_hist_blocks);
  }
  const int lo = chunk * a.chunk_blocks;
  bool any = false;
  for (int j = 0; j < ng; ++j) any |= ncb[j] > lo;
  if (!any) return;

  if constexpr (kCand)
    for (int i = threadIdx.x; i < ng * kHistBins; i += kThreads) (&s_hist[0][0])[i] = 0u;

  // (without kCand the row arrays are stand-ins that are never touched)
  uint32_t (*hist_rows)[kHistBins] = reinterpret_cast<uint32_t (*)[kHistBins]>(&s_hist[0][0]);
  float (*sc_rows)[kCandChunkMax] = reinterpret_cast<float (*)[kCandChunkMax]>(&s_sc[0][0]);
  uint32_t done = 0;
  for (int j0 = 0; j0 < ng; ++j0) {
    if ((done >> j0) & 1u) continue;
    int tok[kMaxGroup] = {t0, t0, t0, t0}, hslot[kMaxGroup], cbs[kMaxGroup];
    int nq = 0, hi = lo;
    for (int j = j0; j < ng; ++j) {
      if (((done >> j) & 1u) == 0 && seq[j] == seq[j0]) {
        done |= 1u << j;
        if (ncb[j] > lo) {
          tok[nq] = t0 + j;
          hslot[nq] = j;
          cbs[nq] = ncb[j];
          hi = max(hi, min(ncb[j], lo + a.chunk_blocks));
          ++nq;
        }
      }
    }
    if (nq == 0) continue;
    // Physical pages of blocks [lo, hi) of this sequence and the run's index
    // queries, read in one pass before the barrier (reads clamped into their
    // tables, LDS writes unconditional: no read waits behind another).
    const int32_t* prow = a.page_table + (size_t)seq[j0] * a.max_pages + (lo >> 3);
    const int np = ((hi - 1) >> 3) - (lo >> 3) + 1;
    const int qi = min((int)threadIdx.x / (kKeyBytes / 16), nq - 1);
    const int tq = qi == 0 ? tok[0] : qi == 1 ? tok[1] : qi == 2 ? tok[2] : tok[3];
    const u32x4 qv = load16(a.q_idx + (size_t)tq * kKeyBytes + (threadIdx.x % (kKeyBytes / 16)) * 16);
    int pg[kPagePasses];
#pragma unroll
    for (int r = 0; r < kPagePasses; ++r) pg[r] = prow[min((int)threadIdx.x + r * kThreads, np - 1)];
    __syncthreads();   // the previous run is done with s_pages and s_q (and the histograms are clear)
    s_q[threadIdx.x] = qv;
#pragma unroll
    for (int r = 0; r < kPagePasses; ++r) s_pages[threadIdx.x + r * kThreads] = pg[r];
    __syncthreads();
    if (nq == 1) score_run<1, kCand, kFp8>(a, tok, hslot, cbs, lo, hi, s_pages, s_q, hist_rows, sc_rows);
    if constexpr (GS >= 2) { if (nq == 2) score_run<2, kCand, kFp8>(a, tok, hslot, cbs, lo, hi, s_pages, s_q, hist_rows, sc_rows); }
    if constexpr (GS >= 3) { if (nq == 3) score_run<3, kCand, kFp8>(a, tok, hslot, cbs, lo, hi, s_pages, s_q, hist_rows, sc_rows); }
    if constexpr (GS >= 4) { if (nq == 4) score_run<4, kCand, kFp8>(a, tok, hslot, cbs, lo, hi, s_pages, s_q, hist_rows, sc_rows); }
  }
  if constexpr (!kCand) return;
  __syncthreads();
  // each row's local candidates of this chunk
  for (int j = 0; j < ng; ++j) {
    if (ncb[j] <= lo) continue;   // (uniform) this chunk holds nothing of row j
    const int n = min(ncb[j], lo + a.chunk_blocks) - lo;
    emit_chunk_candidates(a, t0 + j, chunk, nchunk, lo, n, local_budget(a.topk, a.chunk_blocks, ncb[j]), s_hist[j],
                          s_sc[j], s_tmp, s_res);
  }
}

// ---------------------------------------------------------------------------
// 2b. score as an MFMA GEMM (calls with long runs of query tokens of one
//     sequence, e.g. a prefill chunk, and histories of at most kFuseLimit)
// ---------------------------------------------------------------------------
// A workgroup owns 64 consecutive query tokens and a range of block tiles of
// their sequence's history. Wave w computes tokens 16w..16w+15 against each
// 32-block key tile with v_mfma_f32_16x16x32_bf16 (A = index queries, held in
// registers; B = keys, staged through LDS rows padded to 528 bytes so that the
// 16-byte fragment reads of 16 lanes hit 64 distinct banks). The page ids of
// the workgroup's block range are read into LDS once per pass, so a tile's key
// loads depend on no other global read; they are issued two tiles ahead (two
// register sets), and one barrier per tile orders the LDS buffers. Each wave
// passes its 16 x 32 scores through LDS and stores them as 16 bytes per lane (8
// whole 128-byte row pieces per store). Rows of another sequence than the one
// being processed are handled in further passes.
constexpr int kGemmTokens = 64;
constexpr int kGemmBlocks = 32;
constexpr int kKeyStride = kKeyBytes + 16;
constexpr int kGemmMaxTiles = kFuseLimit / kGemmBlocks;           // tiles of the longest history
constexpr int kGemmPages = kGemmMaxTiles * kGemmBlocks / kBlocksPerPage;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

template <bool kFp8>
__global__ __launch_bounds__(kThreads) void score_gemm_kernel(IndexerArgs a, int tiles_per_wg) {
  constexpr int KB = KeyFmt<kFp8>::kBytes;
  __shared__ uint8_t s_keys[2][kGemmBlocks * kKeyStride];
  __shared__ int s_pages[kGemmPages];   // pass's pages, from its first tile on; -1 = unreadable
  __shared__ float4 s_c[kThreads / 64][16][kGemmBlocks / 4 + 1];   // per wave: its 16 rows of a tile's scores
  __shared__ int s_tok_cb[kGemmTokens];
  __shared__ int s_tok_seq[kGemmTokens];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * kGemmTokens;
  const int tile0 = blockIdx.y * tiles_per_wg;
  if (tid < kGemmTokens) {
    int b = -1;
    int cbt = 0;
    if (t0 + tid < a.n_tok) cbt = min(hist_blocks(a, t0 + tid, &b), a.max_hist_blocks);
    s_tok_cb[tid] = cbt;
    s_tok_seq[tid] = cbt > 0 ? b : -1;
  }
  __syncthreads();
  // A fragments: token row 16*wave + lq, dims 32*i + 8*lg .. +8
  const int my_row = wave * 16 + lq;
  const int t_a = min(t0 + my_row, a.n_tok - 1);
  u32x4 qa[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qa[i] = load16(a.q_idx + (size_t)t_a * kKeyBytes + (32 * i + 8 * lg) * 2);

  uint64_t done = 0;   // rows already processed (identical in every thread)
  for (;;) {
    int seq = -1, hi = 0;
    for (int r = 0; r < kGemmTokens; ++r) {
      if ((done >> r) & 1ull) continue;
      if (s_tok_seq[r] < 0) {
        done |= 1ull << r;
        continue;
      }
      if (seq < 0) seq = s_tok_seq[r];
      if (s_tok_seq[r] == seq) hi = max(hi, s_tok_cb[r]);
    }
    if (seq < 0) break;
    uint64_t active = 0;
    for (int r = 0; r < kGemmTokens; ++r)
      if (((done >> r) & 1ull) == 0 && s_tok_seq[r] == seq) active |= 1ull << r;
    done |= active;
    const int ntiles = (hi + kGemmBlocks - 1) / kGemmBlocks;
    const int tl0 = tile0, tl1 = min(ntiles, tile0 + tiles_per_wg);
    if (tl0 >= tl1) continue;
    // page ids of blocks tl0*32 .. min(hi, tl1*32) - 1 (every page index < max_pages: hi <= p/8)
    const int pg0 = tl0 * (kGemmBlocks / kBlocksPerPage);
    const int npg = min((tl1 - tl0) * (kGemmBlocks / kBlocksPerPage), (hi + kBlocksPerPage - 1) / kBlocksPerPage - pg0);
    {
      const int32_t* prow = a.page_table + (size_t)seq * a.max_pages + pg0;
      for (int i = tid; i < npg; i += kThreads) {
        const int pg = prow[i];
        s_pages[i] = (pg >= 0 && pg < a.num_pages) ? pg : -1;
      }
    }
    __syncthreads();
    // key tile staging: thread tid moves 16-byte pieces tid + 256*j of the
    // tile's keys (bf16: 8 dims per piece; fp8: 16 dims, widened to bf16 in LDS)
    constexpr int kPieces = kGemmBlocks * (KB / 16) / kThreads;
    constexpr int kPerKey = KB / 16;
    u32x4 ra[kPieces], rb[kPieces];
    auto fetch = [&](int tile, u32x4 (&kreg)[kPieces]) {
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        const int piece = tid + kThreads * j;
        const int blk = piece / kPerKey, part = piece % kPerKey;
        const int beta = tile * kGemmBlocks + blk;
        const int page = beta < hi ? s_pages[(beta >> 3) - pg0] : -1;
        const size_t off = page >= 0 ? ((size_t)page * kBlocksPerPage + (beta & 7)) * KB + part * 16 : 0;
        kreg[j] = load16_stream(a.k_idx_cache + off);
      }
    };
    auto stash = [&](int buf, const u32x4 (&kreg)[kPieces]) {
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        const int piece = tid + kThreads * j;
        const int blk = piece / kPerKey, part = piece % kPerKey;
        if constexpr (!kFp8) {
          *reinterpret_cast<u32x4*>(&s_keys[buf][blk * kKeyStride + part * 16]) = kreg[j];
        } else {
          u32x4 lo, hi2;
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            lo[2 * w] = fp8x2_to_bf16x2<false>(kreg[j][w]);
            lo[2 * w + 1] = fp8x2_to_bf16x2<true>(kreg[j][w]);
            hi2[2 * w] = fp8x2_to_bf16x2<false>(kreg[j][w + 2]);
            hi2[2 * w + 1] = fp8x2_to_bf16x2<true>(kreg[j][w + 2]);
          }
          *reinterpret_cast<u32x4*>(&s_keys[buf][blk * kKeyStride + part * 32]) = lo;
          *reinterpret_cast<u32x4*>(&s_keys[buf][blk * kKeyStride + part * 32 + 16]) = hi2;
        }
      }
    };
    // One tile: its keys are in s_keys[buf]; `spare` held them (free now) and
    // takes tile + 2; `next` holds tile + 1, stashed into the other buffer at
    // the end. That buffer was last read before the previous tile's barrier.
    auto step = [&](int tile, int buf, u32x4 (&spare)[kPieces], const u32x4 (&next)[kPieces]) {
      if (tile + 2 < tl1) fetch(tile + 2, spare);
      constexpr int kSub = kGemmBlocks / 16;
      f32x4 c[kSub];
#pragma unroll
      for (int n = 0; n < kSub; ++n) {
        c[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4 kb = *reinterpret_cast<const u32x4*>(
              &s_keys[buf][(16 * n + lq) * kKeyStride + (32 * i + 8 * lg) * 2]);
          c[n] = mfma_bf16(qa[i], kb, c[n]);
        }
      }
      // c[n][r]: token row 16*wave + 4*lg + r, block tile*kGemmBlocks + 16*n + lq. The wave's 16 x 32
      // scores go through LDS so that each store writes 16 bytes per lane, 8 whole rows of the tile
#pragma unroll
      for (int n = 0; n < kSub; ++n) {
        const int beta = tile * kGemmBlocks + 16 * n + lq;
        const bool readable = beta < hi && s_pages[(min(beta, hi - 1) >> 3) - pg0] >= 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          reinterpret_cast<float*>(&s_c[wave][4 * lg + r][0])[16 * n + lq] = readable ? c[n][r] : -INFINITY;
      }
      {
        const int ch = lane & 7;
        const int beta0 = tile * kGemmBlocks + 4 * ch;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rr = (lane >> 3) + 8 * h;
          const int row = wave * 16 + rr;
          const float4 v = s_c[wave][rr][ch];
          // a store that starts inside the row's history may run up to 3 blocks past it: those scores
          // are never read, and rows are a multiple of 8 blocks long, so it stays inside the row
          if (((active >> row) & 1ull) && beta0 < s_tok_cb[row])
            *reinterpret_cast<float4*>(&a.scores[(size_t)(t0 + row) * a.max_hist_blocks + beta0]) = v;
        }
      }
      if (tile + 1 < tl1) stash(buf ^ 1, next);
      __syncthreads();
    };
    fetch(tl0, ra);
    if (tl0 + 1 < tl1) fetch(tl0 + 1, rb);
    stash(0, ra);
    __syncthreads();
    for (int tile = tl0; tile < tl1; tile += 2) {
      step(tile, 0, ra, rb);
      if (tile + 1 < tl1) step(tile + 1, 1, rb, ra);
    }
  }
}

// ---------------------------------------------------------------------------
// 2c. score with MFMA for 16 query rows of one sequence (e.g. 4 verify tokens
//     x 4 KV groups with per-group selection), histories of at most kFuseLimit
// ---------------------------------------------------------------------------
// A workgroup owns 16 consecutive query rows and a chunk of block ids. Each
// wave walks a contiguous part of the chunk in tiles of 16 blocks:
// v_mfma_f32_16x16x32_bf16 with A = the 16 index queries (registers, loaded
// once) and B = the 16 keys of the tile, loaded straight from the cache into
// registers (lane (lq, lg): block lq of the tile). k-step i of lane group lg
// covers dims 64*(i/2) + 16*lg + 8*(i%2) .. +8, so a lane's two k-steps of a
// 64-dim slice are 16 contiguous dims (32 B of bf16, 16 B of fp8), so one load
// instruction reads half of each key's 128-byte lines and the next one the
// other half: the key loads are cacheable (non-temporal loads fetched every
// line twice from L2: 160 -> 151 us for the 128K batch's per-group indexer).
// The next tile's keys are loaded while the current one is multiplied. Rows of another
// sequence than the one being processed are handled in further passes.
constexpr int kMfmaRows = 16;
constexpr int kMfmaTile = 16;

template <bool kFp8>
__global__ __launch_bounds__(kThreads) void score_mfma_kernel(IndexerArgs a) {
  constexpr int KB = KeyFmt<kFp8>::kBytes;
  constexpr int KL = kFp8 ? 4 : 8;   // 16-byte loads per lane per tile
  __shared__ int32_t s_pages[kMaxChunkBlocks / kBlocksPerPage + 1];
  __shared__ int s_row_cb[kMfmaRows];
  __shared__ int s_row_seq[kMfmaRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 15, lg = lane >> 4;
  const int nchunk = (a.max_hist_blocks + a.chunk_blocks - 1) / a.chunk_blocks;
  const int chunk = blockIdx.x % nchunk;
  const int r0 = (blockIdx.x / nchunk) * kMfmaRows;
  if (tid < kMfmaRows) {   // rows located as in score_kernel (no sequence-length check)
    int b = -1, p, cbt = 0;
    if (r0 + tid < a.n_tok) cbt = min(located_blocks(a, r0 + tid, &b, &p), a.max_hist_blocks);
    s_row_cb[tid] = cbt;
    s_row_seq[tid] = cbt > 0 ? b : -1;
  }
  // A: query row r0 + lq (clamped to the last row; rows past the end store nothing)
  u32x4 qa[8];
  {
    const uint8_t* qrow = a.q_idx + (size_t)min(r0 + lq, a.n_tok - 1) * kKeyBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) qa[i] = load16(qrow + (64 * (i >> 1) + 16 * lg + 8 * (i & 1)) * 2);
  }
  __syncthreads();
  const int lo = chunk * a.chunk_blocks;
  uint32_t done = 0;
  for (;;) {
    int seq = -1, hi = lo;
    for (int r = 0; r < kMfmaRows; ++r) {
      if ((done >> r) & 1u) continue;
      if (s_row_seq[r] < 0 || s_row_cb[r] <= lo) {
        done |= 1u << r;
        continue;
      }
      if (seq < 0) seq = s_row_seq[r];
      if (s_row_seq[r] == seq) hi = max(hi, min(s_row_cb[r], lo + a.chunk_blocks));
    }
    if (seq < 0) break;
    uint32_t active = 0;
    for (int r = 0; r < kMfmaRows; ++r)
      if (((done >> r) & 1u) == 0 && s_row_seq[r] == seq) active |= 1u << r;
    done |= active;
    const int32_t* prow = a.page_table + (size_t)seq * a.max_pages;
    const int page0 = lo >> 3;
    const int np = ((hi - 1) >> 3) - page0 + 1;
    __syncthreads();   // the previous pass is done with s_pages
    for (int i = tid; i < np; i += kThreads) s_pages[i] = prow[page0 + i];
    __syncthreads();
    const int per_wave = ((hi - lo + 4 * kMfmaTile - 1) / (4 * kMfmaTile)) * kMfmaTile;
    const int wlo = lo + wave * per_wave;
    const int whi = min(hi, wlo + per_wave);
    if (wlo < whi) {
      u32x4 k0[KL], k1[KL];   // two tile buffers (static indices: the loop is unrolled by two)
      bool ok0 = false, ok1 = false;
      auto fetch = [&](u32x4 (&kb)[KL], bool& okb, int base) {
        const int beta = base + lq;
        const int page = beta < whi ? s_pages[(beta >> 3) - page0] : -1;
        const bool ok = page >= 0 && page < a.num_pages;
        okb = ok;
        const uint8_t* p = a.k_idx_cache + (ok ? ((size_t)page * kBlocksPerPage + (beta & 7)) * KB : 0);
#pragma unroll
        for (int j = 0; j < KL; ++j) {
          // bf16: slice j/2 (64 dims = 128 B), half j%2 of the lane's 32 B; fp8: slice j, the lane's 16 B
          const int off = kFp8 ? 64 * j + 16 * lg : 128 * (j >> 1) + 32 * lg + 16 * (j & 1);
          kb[j] = load16(p + off);   // cacheable: the other half of each 128-byte line comes from L1
        }
      };
      const int ntiles = (whi - wlo + kMfmaTile - 1) / kMfmaTile;
      // rows this lane stores (D: rows 4*lg + r, block lq of the tile)
      int cb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * lg + r;
        cb[r] = ((active >> row) & 1u) ? s_row_cb[row] : 0;
      }
      // one tile: prefetch tile n + 1 into `nxt`, multiply `cur`, store the scores
      auto tile = [&](int n, u32x4 (&cur)[KL], bool okc, u32x4 (&nxt)[KL], bool& okn) {
        const int base = wlo + n * kMfmaTile;
        if (n + 1 < ntiles) fetch(nxt, okn, base + kMfmaTile);
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          u32x4 b;
          if constexpr (kFp8) {
            const u32x4 w = cur[i >> 1];
            const int h = (i & 1) * 2;
            b = u32x4{fp8x2_to_bf16x2<false>(w[h]), fp8x2_to_bf16x2<true>(w[h]), fp8x2_to_bf16x2<false>(w[h + 1]),
                      fp8x2_to_bf16x2<true>(w[h + 1])};
          } else {
            b = cur[i];
          }
          c = mfma_bf16(qa[i], b, c);
        }
        const int beta = base + lq;
        if (beta < whi) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (beta < cb[r])
              a.scores[(size_t)(r0 + 4 * lg + r) * a.max_hist_blocks + beta] = okc ? c[r] : -INFINITY;
        }
      };
      fetch(k0, ok0, wlo);
      for (int n = 0; n < ntiles; n += 2) {
        tile(n, k0, ok0, k1, ok1);
        if (n + 1 < ntiles) tile(n + 1, k1, ok1, k0, ok0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. finalize (MFMA scorers) and the ordered select shared by both selects
// ---------------------------------------------------------------------------
constexpr int kFinalThreads = 512;

constexpr int kTieCap = 2048;   // threshold-bin entries resolved in LDS
constexpr int kRankMax = 256;   // threshold bins up to this size are resolved by ranking

__device__ __forceinline__ uint64_t tz_entry(uint32_t key, uint32_t beta) { return (uint64_t)key << 32 | (uint32_t)~beta; }
__device__ __forceinline__ uint32_t tz_key(uint64_t e) { return (uint32_t)(e >> 32); }
__device__ __forceinline__ uint32_t tz_block(uint64_t e) { return ~(uint32_t)e; }

// Writes the ids of the bits set in sel_bm, together with the first need_eq
// ids (in block order) of the bits set in eq_bm, in ascending order to out
// (at most k; -1 past the last). Thread i owns the contiguous id range
// [i*perb, (i+1)*perb), perb = ceil(nbits / threads): it reads the (at most
// kEmitWords) words its range touches all at once, one scan of its packed
// (chosen, tied) counts gives its offsets (one barrier), and it places its ids
// -- taking the leading tied ids of its range -- in LDS (s_ids, k entries),
// which is then written out in one coalesced pass.
constexpr int kEmitWords = kFuseLimit / 32 / kFinalThreads + 1;

__device__ __forceinline__ void emit_selection(const uint32_t* sel_bm, const uint32_t* eq_bm, uint32_t need_eq, int nbits, int k,
                               int32_t* out, uint32_t* s_tmp, int32_t* s_ids) {
  constexpr int kW = kFinalThreads / 64;
  const int wave = threadIdx.x >> 6;
  const bool use_eq = need_eq > 0u;   // block-uniform
  const int nw = (nbits + 31) >> 5;
  const int perb = (nbits + kFinalThreads - 1) / kFinalThreads;
  const int bb0 = min(nbits, (int)threadIdx.x * perb), bb1 = min(nbits, bb0 + perb);
  const int wlo = bb0 >> 5;
  const int nwt = bb1 > bb0 ? ((bb1 - 1) >> 5) - wlo + 1 : 0;   // words this range touches
  uint32_t sw[kEmitWords], ew[kEmitWords];
  uint32_t cs = 0, ce = 0;
#pragma unroll
  for (int i = 0; i < kEmitWords; ++i) {
    const int w = wlo + i;
    const int lo = min(max(bb0 - 32 * w, 0), 31), hi = min(max(bb1 - 32 * w, 0), 32);
    const uint32_t mask = i < nwt ? (hi >= 32 ? 0xffffffffu : (1u << hi) - 1u) & ~((1u << lo) - 1u) : 0u;
    const int wr = min(w, nw - 1);   // clamped read: every read is issued, none waits on another
    sw[i] = sel_bm[wr] & mask;
    ew[i] = use_eq ? eq_bm[wr] & mask : 0u;
    cs += (uint32_t)__popc(sw[i]);
    ce += (uint32_t)__popc(ew[i]);
  }
  // packed scan: chosen ids <= k and tied ids <= the tie capacity, both below 2^16
  const uint32_t packed = cs | ce << 16;
  const uint32_t incl = wave_incl_scan(packed);
  if ((threadIdx.x & 63) == 63) s_tmp[wave] = incl;
  __syncthreads();
  uint32_t below = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    const uint32_t y = s_tmp[i];
    below += i < wave ? y : 0u;
    tot += y;
  }
  const uint32_t ex = below + incl - packed;
  uint32_t sbefore = ex & 0xffffu, ebefore = ex >> 16;   // chosen / tied ids in lower ranges
#pragma unroll
  for (int i = 0; i < kEmitWords; ++i) {
    uint32_t take = 0;
    if (ebefore < need_eq && ew[i] != 0u) {
      const uint32_t r = need_eq - ebefore;
      if ((uint32_t)__popc(ew[i]) <= r) {
        take = ew[i];
      } else {
        uint32_t rest = ew[i];
        for (uint32_t j = 0; j < r; ++j) {
          const uint32_t low = rest & (0u - rest);
          take |= low;
          rest ^= low;
        }
      }
    }
    uint32_t fin = sw[i] | take;
    uint32_t pos = sbefore + min(need_eq, ebefore);
    while (fin != 0u) {
      const int bit = __ffs(fin) - 1;
      fin &= fin - 1u;
      if (pos < (uint32_t)k) s_ids[pos] = (wlo + i) * 32 + bit;
      ++pos;
    }
    sbefore += (uint32_t)__popc(sw[i]);
    ebefore += (uint32_t)__popc(ew[i]);
  }
  __syncthreads();
  const int n_out = (int)min((uint32_t)k, (tot & 0xffffu) + min(need_eq, tot >> 16));
  for (int i = threadIdx.x; i < k; i += kFinalThreads) out[i] = i < n_out ? s_ids[i] : -1;   // -1 only if inconsistent
}

static_assert(kTieCap * 2 >= SA_MAX_TOPK, "the tie buffer stages the output ids");
static_assert(SA_MAX_TOPK < (1 << 16) && kTieCap < (1 << 16), "emit_selection packs two counts in 32 bits");

struct alignas(16) FinalizeLds {
  uint64_t tz[kTieCap];     // threshold-bin entries: key << 32 | ~block id (a larger entry ranks first)
  uint32_t h[kHistBins];
  uint32_t tmp[2 * (kFinalThreads / 64)];   // block scans; emit_selection uses both halves
  uint32_t res[2];
  uint32_t n_tz;
};

// Exact k-th largest (k >= 1, at most m) of the keys key_at(0 .. m-1): three
// radix levels of 11, 11 and 10 bits, histograms in h[kHistBins]; *count_gt
// receives how many keys are strictly larger. NT threads, all of them call it.
template <int NT, typename KeyAt>
__device__ uint32_t radix_kth(KeyAt key_at, int m, uint32_t k, uint32_t* h, uint32_t* tmp, uint32_t* res,
                              uint32_t* count_gt) {
  __syncthreads();
  uint32_t prefix = 0, above = 0;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int lvl = 0; lvl < 3; ++lvl) {
    const int sh = shifts[lvl];
    const int nb = 1 << widths[lvl];
    const int hs = sh + widths[lvl];
    for (int i = threadIdx.x; i < kHistBins; i += NT) h[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < m; i += NT) {
      const uint32_t key = key_at(i);
      if (lvl == 0 || (key >> hs) == (prefix >> hs)) atomicAdd(&h[(key >> sh) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    select_bin<NT>(h, nb, k - above, tmp, res);
    prefix |= res[0] << sh;
    above += res[1];
    __syncthreads();
  }
  *count_gt = above;
  return prefix;
}

// The same over all of a token's stored scores.
template <int NT>
__device__ uint32_t radix_kth_global(const IndexerArgs& a, uint32_t* h, uint32_t* tmp, uint32_t* res, int t,
                                     int ncand, uint32_t k, uint32_t* count_gt) {
  const float* srow = a.scores + (size_t)t * a.max_hist_blocks;
  return radix_kth<NT>([srow](int i) { return score_key(srow[i]); }, ncand, k, h, tmp, res, count_gt);
}

// Selection over all scores in one ordered pass (used when a row does not fit
// the LDS structures of either select): keys above tau, then keys equal to tau
// in block order until k are taken; the output comes out ascending.
template <int NT>
__device__ void select_ordered_global(const IndexerArgs& a, uint32_t* h, uint32_t* tmp, uint32_t* res, int t,
                                      int ncand, int32_t* out) {
  const int k = a.topk;
  uint32_t count_gt;
  const uint32_t tau = radix_kth_global<NT>(a, h, tmp, res, t, ncand, (uint32_t)k, &count_gt);
  count_gt = min(count_gt, (uint32_t)k);
  const uint32_t need_eq = (uint32_t)k - count_gt;
  const float* srow = a.scores + (size_t)t * a.max_hist_blocks;
  uint32_t eq_before = 0, sel_before = 0;
  for (int base = 0; base < ncand; base += NT) {
    const int beta = base + threadIdx.x;
    uint32_t key = 0;
    if (beta < ncand) key = score_key(srow[beta]);
    const bool gt = beta < ncand && key > tau;
    const bool eq = beta < ncand && key == tau;
    uint32_t eq_tot, sel_tot;
    const uint32_t eq_rank = eq_before + block_prefix_exclusive<NT>(eq ? 1u : 0u, tmp, &eq_tot);
    const bool take = gt || (eq && eq_rank < need_eq);
    const uint32_t pos = sel_before + block_prefix_exclusive<NT>(take ? 1u : 0u, tmp, &sel_tot);
    if (take && pos < (uint32_t)k) out[pos] = beta;
    eq_before += eq_tot;
    sel_before += sel_tot;
  }
}

// Histogram and classification of one token's scores: a history of at most
// KP * kFinalThreads blocks whose scores are held in registers, KP per thread
// (instantiated for 2 .. 32 so that short histories execute no steps past
// their own). Afterwards sel_bm holds the ids above the threshold bin b1
// (*above of them) and s.tz the threshold-bin entries. Returns kClassified,
// kDone (an invalid token: its output is written) or kFallback (the threshold
// bin does not fit the LDS structures: the caller selects the row in order
// over all scores).
enum ClassifyResult { kClassified, kDone, kFallback };

template <int KP>
__device__ __forceinline__ ClassifyResult finalize_classify(const IndexerArgs& a, FinalizeLds& s, uint32_t* sel_bm, uint32_t* eq_bm, int t,
                                  int ncand, bool valid, int32_t* out, uint32_t* b1_out, uint32_t* above_out) {
  static_assert(KP > 0, "scores held in registers");
  constexpr int kPer = KP;
  constexpr int kGroup = kPer < 8 ? kPer : 8;   // steps whose loads are issued together
  const int k = a.topk;
  const int nw = (ncand + 31) >> 5;   // bitmap words this token needs
  const int jmax = (ncand + kFinalThreads - 1) / kFinalThreads;   // steps j that hold scores (uniform)
  uint32_t kv[kPer];
  {
    // every load of a group is issued (past the history they re-read its last
    // score), so all of them are in flight at once
    const float* srow = a.scores + (size_t)t * a.max_hist_blocks;
    float sv[kPer];
#pragma unroll
    for (int j0 = 0; j0 < kPer; j0 += kGroup) {
      if (j0 < jmax) {
#pragma unroll
        for (int j = j0; j < j0 + kGroup; ++j) sv[j] = srow[min(j * kFinalThreads + (int)threadIdx.x, ncand - 1)];
      }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      kv[j] = j < jmax && j * kFinalThreads + (int)threadIdx.x < ncand ? score_key(sv[j]) : 0u;
    for (int i = threadIdx.x; i < kHistBins; i += kFinalThreads) s.h[i] = 0u;
  }
  if (nw <= a.bitmap_words) {
    for (int i = threadIdx.x; i < nw; i += kFinalThreads) {
      sel_bm[i] = 0u;
      eq_bm[i] = 0u;
    }
  }
  if (threadIdx.x == 0) s.n_tz = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (j < jmax) {
      const int beta = j * kFinalThreads + (int)threadIdx.x;
      if (beta < ncand) atomicAdd(&s.h[kv[j] >> 21], 1u);
    }
  }
  __syncthreads();
  if (!valid) {   // past its sequence's length: selects nothing
    for (int i = threadIdx.x; i < k; i += kFinalThreads) out[i] = -1;
    return kDone;
  }
  select_bin<kFinalThreads>(s.h, kHistBins, (uint32_t)k, s.tmp, s.res);
  const uint32_t b1 = s.res[0];
  const uint32_t above = min(s.res[1], (uint32_t)k - 1u);
  const uint32_t in_bin = s.h[b1];
  if (nw > a.bitmap_words || in_bin > (uint32_t)kTieCap) return kFallback;
  *b1_out = b1;
  *above_out = above;
  // A wave holds 64 consecutive block ids per j: its ballot of "above the
  // threshold bin" is exactly two bitmap words, and the threshold-bin keys
  // take one counter update per wave.
  // Lane j keeps the two words of step j; they are stored once at the end.
  const int lane = threadIdx.x & 63;
  uint32_t n_wave = 0;   // this wave's threshold-bin keys (first pass: count)
  uint32_t word_lo = 0, word_hi = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (j < jmax) {
      const bool in = j * kFinalThreads + (int)threadIdx.x < ncand;
      const uint32_t bin = kv[j] >> 21;
      const uint64_t above_mask = __ballot(in && bin > b1);
      word_lo = lane == j ? (uint32_t)above_mask : word_lo;
      word_hi = lane == j ? (uint32_t)(above_mask >> 32) : word_hi;
      n_wave += (uint32_t)__popcll(__ballot(in && bin == b1));
    }
  }
  if (lane < jmax) {
    const int w = (lane * kFinalThreads + (int)(threadIdx.x - lane)) >> 5;
    if (w < nw) sel_bm[w] = word_lo;
    if (w + 1 < nw) sel_bm[w + 1] = word_hi;
  }
  if (n_wave != 0u) {   // second pass: slots base + rank within the wave
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&s.n_tz, n_wave);
    base = __shfl(base, 0);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (j < jmax) {
        const int beta = j * kFinalThreads + (int)threadIdx.x;
        const bool tz = beta < ncand && (kv[j] >> 21) == b1;
        const uint64_t tz_mask = __ballot(tz);
        const uint32_t slot = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(tz_mask >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)tz_mask, 0u));
        if (tz && slot < (uint32_t)kTieCap) {
          s.tz[slot] = tz_entry(kv[j], (uint32_t)beta);
        }
        base += (uint32_t)__popcll(tz_mask);
      }
    }
  }
  __syncthreads();
  return kClassified;
}

// Per token. The histogram bin b1 that holds the k-th largest score splits the
// scores into "surely chosen" (bins above b1; fewer than k) and the threshold
// bin. Ranking the threshold bin's entries, or two more radix levels over their
// keys, completes the selection: keys above the exact k-th key tau are chosen,
// and keys equal to tau in block order until k are taken. emit_selection writes
// the chosen ids ascending. Used after the MFMA scorers (histories of at most
// kFuseLimit blocks).
__global__ __launch_bounds__(kFinalThreads) void finalize_kernel(IndexerArgs a) {
  __shared__ FinalizeLds s;
  extern __shared__ uint32_t s_bm[];   // [2][bitmap_words]: chosen ids, ids tied at tau
  const int t = blockIdx.x;
  const int k = a.topk;
  // The scores are located from the token's sequence and position; the
  // sequence-length check is consumed after their loads are in flight.
  int b, p;
  const int ncand = min(located_blocks(a, t, &b, &p), a.max_hist_blocks);
  const int len = seq_len_of(a, b);
  int32_t* out = a.sel_idx + (size_t)t * k;
  if (ncand <= k) {
    const int nv = token_valid(a, b, p, len) ? ncand : 0;
    for (int i = threadIdx.x; i < k; i += kFinalThreads) out[i] = i < nv ? i : -1;
    return;
  }
  uint32_t* sel_bm = s_bm;
  uint32_t* eq_bm = s_bm + a.bitmap_words;
  const bool valid = token_valid(a, b, p, len);
  const int jmax = (ncand + kFinalThreads - 1) / kFinalThreads;
  uint32_t b1 = 0, above = 0;
  ClassifyResult r;
  if (ncand > kFuseLimit) r = kFallback;   // (the host never sends such a row here)
  else if (jmax <= 2) r = finalize_classify<2>(a, s, sel_bm, eq_bm, t, ncand, valid, out, &b1, &above);
  else if (jmax <= 4) r = finalize_classify<4>(a, s, sel_bm, eq_bm, t, ncand, valid, out, &b1, &above);
  else if (jmax <= 8) r = finalize_classify<8>(a, s, sel_bm, eq_bm, t, ncand, valid, out, &b1, &above);
  else if (jmax <= 16) r = finalize_classify<16>(a, s, sel_bm, eq_bm, t, ncand, valid, out, &b1, &above);
  else r = finalize_classify<32>(a, s, sel_bm, eq_bm, t, ncand, valid, out, &b1, &above);
  static_assert(kFuseLimit == 32 * kFinalThreads, "the largest instantiation covers every fused history");
  if (r == kFallback) select_ordered_global<kFinalThreads>(a, s.h, s.tmp, s.res, t, ncand, out);
  if (r != kClassified) return;
  const int m = (int)min(s.n_tz, (uint32_t)kTieCap);
  const uint32_t need = (uint32_t)k - above;
  uint32_t need_eq = 0;   // ids tied at the exact threshold, taken in block order
  if (m <= kRankMax) {
    // Few keys in the threshold bin: a key is chosen iff fewer than `need` of
    // them come before it (a larger key, or an equal key of a lower block).
    const int m2 = m & ~1;
    for (int i = threadIdx.x; i < m; i += kFinalThreads) {
      const uint64_t e = s.tz[i];
      uint32_t rank = 0;
#pragma unroll 4
      for (int j = 0; j < m2; j += 2) {
        const ulonglong2 ej = *reinterpret_cast<const ulonglong2*>(&s.tz[j]);
        rank += ej.x > e ? 1u : 0u;
        rank += ej.y > e ? 1u : 0u;
      }
      if (m2 < m) rank += s.tz[m2] > e ? 1u : 0u;
      const uint32_t beta = tz_block(e);
      if (rank < need) atomicOr(&sel_bm[beta >> 5], 1u << (beta & 31));
    }
  } else {
    // exact k-th key inside the threshold bin: two more radix levels
    uint32_t prefix = b1 << 21;
    uint32_t gt_in_bin = 0;
    {
      const int shifts[2] = {10, 0};
      const int widths[2] = {11, 10};
      for (int lvl = 0; lvl < 2; ++lvl) {
        const int sh = shifts[lvl];
        const int nb = 1 << widths[lvl];
        const int hs = sh + widths[lvl];
        for (int i = threadIdx.x; i < kHistBins; i += kFinalThreads) s.h[i] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < m; i += kFinalThreads) {
          const uint32_t key = tz_key(s.tz[i]);
          if ((key >> hs) == (prefix >> hs)) atomicAdd(&s.h[(key >> sh) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        select_bin<kFinalThreads>(s.h, nb, need - gt_in_bin, s.tmp, s.res);
        prefix |= s.res[0] << sh;
        gt_in_bin += s.res[1];
        __syncthreads();
      }
    }
    const uint32_t tau = prefix;
    need_eq = need - min(gt_in_bin, need);
    for (int i = threadIdx.x; i < m; i += kFinalThreads) {
      const uint32_t key = tz_key(s.tz[i]), beta = tz_block(s.tz[i]);
      if (key > tau) atomicOr(&sel_bm[beta >> 5], 1u << (beta & 31));
      else if (key == tau) atomicOr(&eq_bm[beta >> 5], 1u << (beta & 31));
    }
  }
  __syncthreads();   // (the threshold-bin entries are dead from here: their LDS stages the output)
  emit_selection(sel_bm, eq_bm, need_eq, ncand, k, out, s.tmp, reinterpret_cast<int32_t*>(s.tz));
}

// Exact k-th largest (1 <= k <= m) of key_at(0 .. m-1), for key sets that are
// small and crowded (the high end of a row): the bins of each radix level span
// the keys' own range [lo, hi] (2048 bins of 2^sh keys, sh = bit width of the
// range less 11), so that the first level spreads the keys over many bins and
// the later levels (at most two more) only see the keys of the chosen bin.
// After each level the keys of the chosen bin are checked for being one value
// (scores of integer data are: their neighbours lie far apart in key space),
// which ends the search there. *count_gt receives how many keys are strictly
// larger. NT threads.
template <int NT, typename KeyAt>
__device__ uint32_t radix_kth_range(KeyAt key_at, int m, uint32_t k, uint32_t* h, uint32_t* tmp, uint32_t* res,
                                    uint32_t* count_gt) {
  // range of the keys (wave reductions, then across the waves)
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int i = threadIdx.x; i < m; i += NT) {
    const uint32_t x = key_at(i);
    kmin = min(kmin, x);
    kmax = max(kmax, x);
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d));
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();   // tmp may still be read by an earlier scan
  if ((threadIdx.x & 63) == 0) {
    tmp[wave] = kmin;
    tmp[NT / 64 + wave] = kmax;
  }
  __syncthreads();
  kmin = tmp[0];
  kmax = tmp[NT / 64];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    kmin = min(kmin, tmp[w]);
    kmax = max(kmax, tmp[NT / 64 + w]);
  }
  __syncthreads();
  uint32_t base = kmin;                                     // window [base, base + 2^width)
  int width = kmax > kmin ? 32 - __clz(kmax - kmin) : 0;    // kmax - kmin < 2^width
  uint32_t above = 0;
  while (width > 0) {   // (uniform)
    const int sh = max(0, width - 11);
    for (int i = threadIdx.x; i < kHistBins; i += NT) h[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < m; i += NT) {
      const uint32_t d = key_at(i) - base;   // (wraps to a large value below the window)
      if (key_at(i) >= base && (width >= 32 || d < (1u << width))) atomicAdd(&h[d >> sh], 1u);
    }
    __syncthreads();
    select_bin<NT>(h, kHistBins, k - above, tmp, res);
    base += res[0] << sh;
    above += res[1];
    width = sh;
    if (width == 0) break;
    // does the chosen bin [base, base + 2^width) hold a single key value?
    uint32_t bmin = 0xFFFFFFFFu, bmax = 0u;
    for (int i = threadIdx.x; i < m; i += NT) {
      const uint32_t x = key_at(i);
      if (x >= base && (width >= 32 || x - base < (1u << width))) {
        bmin = min(bmin, x);
        bmax = max(bmax, x);
      }
    }
    if (threadIdx.x == 0) {
      tmp[0] = 0xFFFFFFFFu;
      tmp[1] = 0u;
    }
    __syncthreads();
    if (bmin != 0xFFFFFFFFu) {
      atomicMin(&tmp[0], bmin);
      atomicMax(&tmp[1], bmax);
    }
    __syncthreads();
    bmin = tmp[0];
    bmax = tmp[1];
    __syncthreads();
    if (bmin == bmax) {   // (uniform) one value: it is the k-th largest
      base = bmin;
      break;
    }
  }
  *count_gt = above;
  return base;
}

// The same k-th largest when the caller already knows the keys' range
// [kmin, kmax] (no pass over the keys to find it): the histogram pass also
// keeps each bin's smallest and largest key, so the single-value check after a
// level is two reads instead of another pass.
template <int NT, typename KeyAt>
__device__ __forceinline__ uint32_t radix_kth_span(KeyAt key_at, int m, uint32_t k, uint32_t kmin, uint32_t kmax,
                                                   uint32_t* h, uint32_t* hmin, uint32_t* hmax, uint32_t* tmp,
                                                   uint32_t* res, uint32_t* count_gt) {
  uint32_t base = kmin;                                     // window [base, base + 2^width)
  int width = kmax > kmin ? 32 - __clz(kmax - kmin) : 0;    // kmax - kmin < 2^width
  uint32_t above = 0;
  while (width > 0) {   // (uniform)
    const int sh = max(0, width - 11);
    for (int i = threadIdx.x; i < kHistBins; i += NT) {
      h[i] = 0u;
      hmin[i] = 0xFFFFFFFFu;
      hmax[i] = 0u;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < m; i += NT) {
      const uint32_t x = key_at(i);
      const uint32_t d = x - base;   // (wraps to a large value below the window)
      if (x >= base && (width >= 32 || d < (1u << width))) {
        const uint32_t b = d >> sh;
        atomicAdd(&h[b], 1u);
        atomicMin(&hmin[b], x);
        atomicMax(&hmax[b], x);
      }
    }
    __syncthreads();
    select_bin<NT>(h, kHistBins, k - above, tmp, res);
    const uint32_t b = res[0], cnt = res[1];
    const uint32_t bmin = hmin[b], bmax = hmax[b];
    __syncthreads();   // every thread has read res and the bin's extremes
    base += b << sh;
    above += cnt;
    width = sh;
    if (width == 0) break;
    if (bmin == bmax) {   // (uniform) one value: it is the k-th largest
      base = bmin;
      break;
    }
  }
  *count_gt = above;
  return base;
}

// ---------------------------------------------------------------------------
// 4. select (after the per-token scorer)
// ---------------------------------------------------------------------------
// One workgroup per row. The row's candidate lists are read in chunk order, so
// the union U is in ascending block order. tau_U = the k-th largest key of U is
// a lower bound of the row's k-th largest key tau. A chunk whose edge is at or
// below tau_U listed every key >= tau_U it holds; a chunk whose edge lies above
// tau_U (a list that stopped above tau_U, or one that did not fit) is re-read
// from its stored scores. Then F = every key >= tau_U of the row, in block
// order, holds the top k: the keys above tau are chosen and the keys equal to
// tau in block order until k are taken, and the chosen ids come out ascending.
// A row whose lists or F do not fit in LDS takes the ordered select over all
// of its stored scores.
constexpr int kSelThreads = 512;
constexpr int kSelCap = 6144;                     // list entries of one row held in LDS
constexpr int kSelMaxChunks = 1024;               // chunks of one row
constexpr int kSelPer = kSelCap / kSelThreads;    // entries per thread in the ordered pass
constexpr int kSelChunksPer = kSelMaxChunks / kSelThreads;
static_assert(kSelCap < (1 << 16), "the ordered pass packs two counts of F in 32 bits");

struct alignas(16) SelectLds {
  uint32_t key[kSelCap];    // U: the row's lists in chunk (= block) order
  uint32_t id[kSelCap];
  uint32_t fkey[kSelCap];   // F, when some chunk had to be re-read
  uint32_t fid[kSelCap];
  uint32_t h[kHistBins];
  uint32_t hmin[kHistBins];           // smallest and largest key of each bin (tau_U)
  uint32_t hmax[kHistBins];
  uint32_t krange[2];                 // smallest and largest key of U
  uint32_t off[kSelMaxChunks + 1];    // first entry of each chunk's list in U
  uint32_t foff[kSelMaxChunks + 1];   // first entry of each chunk in F (its count, before the scan)
  uint32_t edge[kSelMaxChunks];
  uint32_t tmp[2 * (kSelThreads / 64)];
  uint32_t res[2];
};

// Exclusive scan of v[0 .. n) in place (n <= kSelMaxChunks); v[n] = total.
__device__ void chunk_scan(uint32_t* v, int n, uint32_t* tmp) {
  uint32_t c[kSelChunksPer];
  uint32_t sum = 0;
#pragma unroll
  for (int r = 0; r < kSelChunksPer; ++r) {
    const int i = (int)threadIdx.x * kSelChunksPer + r;
    c[r] = i < n ? v[i] : 0u;
    sum += c[r];
  }
  uint32_t total;
  uint32_t ex = block_prefix_exclusive<kSelThreads>(sum, tmp, &total);
#pragma unroll
  for (int r = 0; r < kSelChunksPer; ++r) {
    const int i = (int)threadIdx.x * kSelChunksPer + r;
    if (i < n) v[i] = ex;
    ex += c[r];
  }
  if (threadIdx.x == 0) v[n] = total;
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(IndexerArgs a) {
  constexpr int kWaves = kSelThreads / 64;
  __shared__ SelectLds s;
  const int t = blockIdx.x;
  const int k = a.topk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C = a.chunk_blocks;
  const int nck_all = (a.max_hist_blocks + C - 1) / C;
  const uint2* meta = a.cand_meta + (size_t)t * nck_all;
  // the row's (count, edge) pairs are read together with its location (the
  // reads are clamped into the row; pairs past the row's chunks are dropped)
  uint2 mv[kSelChunksPer];
#pragma unroll
  for (int r = 0; r < kSelChunksPer; ++r)
    mv[r] = meta[min((int)threadIdx.x * kSelChunksPer + r, min(nck_all, kSelMaxChunks) - 1)];
  int b, p;
  const int ncand = min(located_blocks(a, t, &b, &p), a.max_hist_blocks);
  const int len = seq_len_of(a, b);
  int32_t* out = a.sel_idx + (size_t)t * k;
  const bool valid = token_valid(a, b, p, len);
  if (!valid || ncand <= k) {   // nothing, or every historical block
    const int nv = valid ? ncand : 0;
    for (int i = threadIdx.x; i < k; i += kSelThreads) out[i] = i < nv ? i : -1;
    return;
  }
  const int nck = (ncand + C - 1) / C;
  if (nck > kSelMaxChunks) {
    select_ordered_global<kSelThreads>(a, s.h, s.tmp, s.res, t, ncand, out);
    return;
  }
  const uint2* lists = a.cand + (size_t)t * a.cand_row_stride;
  const float* srow = a.scores + (size_t)t * a.max_hist_blocks;

  // 1. list lengths and edges; first entry of every list in U
#pragma unroll
  for (int r = 0; r < kSelChunksPer; ++r) {
    const int c = (int)threadIdx.x * kSelChunksPer + r;
    if (c < nck) {
      s.off[c] = mv[r].x;
      s.edge[c] = mv[r].y;
    }
  }
  if (threadIdx.x == 0) {
    s.krange[0] = 0xFFFFFFFFu;
    s.krange[1] = 0u;
  }
  __syncthreads();
  chunk_scan(s.off, nck, s.tmp);
  const uint32_t m_u = s.off[nck];
  if (m_u > (uint32_t)kSelCap) {
    select_ordered_global<kSelThreads>(a, s.h, s.tmp, s.res, t, ncand, out);
    return;
  }
  // 2. U in chunk order: thread i copies the lists of chunks i and i + 512,
  // 16 entries (eight 16-byte loads, all issued before any is waited for) at a
  // time; the lists start 16-byte aligned (capacities are multiples of 64).
  // The copy also finds U's key range (for tau_U).
  uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
  for (int c = threadIdx.x; c < nck; c += kSelThreads) {
    const uint32_t o = s.off[c], n = s.off[c + 1] - o;
    const uint4* src = reinterpret_cast<const uint4*>(lists + (size_t)c * a.cand_cap);
    for (uint32_t j0 = 0; j0 < n; j0 += 16) {
      uint4 e[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) e[r] = src[min(j0 / 2 + r, (n - 1) / 2)];   // (clamped into the list)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t j = j0 + 2 * r;
        if (j < n) {
          s.key[o + j] = e[r].x;
          s.id[o + j] = e[r].y;
          lmin = min(lmin, e[r].x);
          lmax = max(lmax, e[r].x);
        }
        if (j + 1 < n) {
          s.key[o + j + 1] = e[r].z;
          s.id[o + j + 1] = e[r].w;
          lmin = min(lmin, e[r].z);
          lmax = max(lmax, e[r].z);
        }
      }
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    lmin = min(lmin, (uint32_t)__shfl_xor((int)lmin, d));
    lmax = max(lmax, (uint32_t)__shfl_xor((int)lmax, d));
  }
  if (lane == 0) {
    atomicMin(&s.krange[0], lmin);
    atomicMax(&s.krange[1], lmax);
  }
  __syncthreads();
  // 3. tau_U (every key, 0, when fewer than k are listed)
  uint32_t gt = 0;
  uint32_t tau = 0;
  if (m_u >= (uint32_t)k) {
    const uint32_t* keys = s.key;
    tau = radix_kth_span<kSelThreads>([keys](int i) { return keys[i]; }, (int)m_u, (uint32_t)k, s.krange[0],
                                       s.krange[1], s.h, s.hmin, s.hmax, s.tmp, s.res, &gt);
  }
  // 4. chunks that may hold unlisted keys >= tau_U
  bool mine = m_u < (uint32_t)k;
  for (int c = threadIdx.x; c < nck; c += kSelThreads) mine |= s.edge[c] > tau;
  const bool reread = __syncthreads_or(mine);
  const uint32_t* fkey = s.key;
  const uint32_t* fid = s.id;
  uint32_t mf = m_u;
  if (reread) {
    const uint32_t tau_u = tau;
    // F's count per chunk: its listed keys >= tau_U, or its stored keys >= tau_U
    for (int c = wave; c < nck; c += kWaves) {
      uint32_t n_f = 0;
      if (s.edge[c] > tau_u) {
        const int lo = c * C, hi = min(ncand, lo + C);
        for (int j = lo + lane; j - lane < hi; j += 64)
          n_f += (uint32_t)__popcll(__ballot(j < hi && score_key(srow[min(j, hi - 1)]) >= tau_u));
      } else {
        const uint32_t o = s.off[c], o1 = s.off[c + 1];
        for (uint32_t j = o + lane; j - lane < o1; j += 64)
          n_f += (uint32_t)__popcll(__ballot(j < o1 && s.key[min(j, o1 - 1)] >= tau_u));
      }
      if (lane == 0) s.foff[c] = n_f;
    }
    __syncthreads();
    chunk_scan(s.foff, nck, s.tmp);
    mf = s.foff[nck];
    if (mf > (uint32_t)kSelCap) {
      select_ordered_global<kSelThreads>(a, s.h, s.tmp, s.res, t, ncand, out);
      return;
    }
    // F in block order
    for (int c = wave; c < nck; c += kWaves) {
      uint32_t pos = s.foff[c];
      if (s.edge[c] > tau_u) {
        const int lo = c * C, hi = min(ncand, lo + C);
        for (int j = lo + lane; j - lane < hi; j += 64) {
          const uint32_t key = score_key(srow[min(j, hi - 1)]);
          const bool in = j < hi && key >= tau_u;
          const uint64_t mask = __ballot(in);
          const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
          if (in) {
            s.fkey[pos + r] = key;
            s.fid[pos + r] = (uint32_t)j;
          }
          pos += (uint32_t)__popcll(mask);
        }
      } else {
        const uint32_t o = s.off[c], o1 = s.off[c + 1];
        for (uint32_t j = o + lane; j - lane < o1; j += 64) {
          const uint32_t jj = min(j, o1 - 1);
          const uint32_t key = s.key[jj];
          const bool in = j < o1 && key >= tau_u;
          const uint64_t mask = __ballot(in);
          const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
          if (in) {
            s.fkey[pos + r] = key;
            s.fid[pos + r] = s.id[jj];
          }
          pos += (uint32_t)__popcll(mask);
        }
      }
    }
    __syncthreads();
    fkey = s.fkey;
    fid = s.fid;
    tau = radix_kth_range<kSelThreads>([fkey](int i) { return fkey[i]; }, (int)mf, (uint32_t)k, s.h, s.tmp, s.res,
                                        &gt);
  }
  // 5. keys above tau, then keys equal to tau in block order until k are
  // taken; thread i owns entries kSelPer*i .. +kSelPer of F (or of U). One scan
  // of packed (above, equal) counts places every entry: a chosen entry goes to
  // (entries above tau before it) + min(entries equal to tau before it, need_eq).
  const uint32_t need_eq = (uint32_t)k - min(gt, (uint32_t)k);
  const int i0 = (int)threadIdx.x * kSelPer;
  uint32_t kk[kSelPer];
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const bool in = i0 + i < (int)mf;
    kk[i] = in ? fkey[i0 + i] : 0u;
    n_gt += (in && kk[i] > tau) ? 1u : 0u;
    n_eq += (in && kk[i] == tau) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t before = block_prefix_exclusive<kSelThreads>(n_gt | n_eq << 16, s.tmp, &tot);
  uint32_t gt_before = before & 0xffffu, eq_before = before >> 16;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const bool in = i0 + i < (int)mf;
    const bool above_tau = in && kk[i] > tau;
    const bool eq = in && kk[i] == tau;
    const uint32_t pos = gt_before + min(eq_before, need_eq);
    if ((above_tau || (eq && eq_before < need_eq)) && pos < (uint32_t)k) out[pos] = (int32_t)fid[i0 + i];
    gt_before += above_tau ? 1u : 0u;
    eq_before += eq ? 1u : 0u;
  }
  const uint32_t taken = (tot & 0xffffu) + min(tot >> 16, need_eq);
  for (int i = (int)min(taken, (uint32_t)k) + (int)threadIdx.x; i < k; i += kSelThreads) out[i] = -1;   // (never: k are taken)
}

}  // namespace

size_t indexer_cand_row_bound(int max_hist_blocks) {
  size_t most = 0;
  for (int c = 64; c <= kCandChunkMax; c <<= 1) {
    const size_t chunks = (size_t)((max_hist_blocks + c - 1) / c);
    most = std::max(most, chunks * (size_t)std::min(c, kChunkCap));
  }
  return most;
}

IndexerWorkspace indexer_workspace_layout(int n_tok, int max_pages_per_seq) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  IndexerWorkspace w;
  const size_t nt = (size_t)(n_tok > 0 ? n_tok : 0);
  const int mhb = (max_pages_per_seq > 0 ? max_pages_per_seq : 0) * kBlocksPerPage;
  const bool lists = mhb > kFuseLimit;   // candidate lists only for histories the finalize cannot hold
  w.scores_off = 0;
  w.meta_off = up(nt * (size_t)mhb * 4);
  w.cand_off = w.meta_off + (lists ? up(nt * (size_t)((mhb + 63) / 64) * 8) : 0);   // chunks are at least 64 blocks
  w.total = w.cand_off + (lists ? up(nt * indexer_cand_row_bound(mhb) * 8) : 0);
  return w;
}

hipError_t launch_indexer_topk(const IndexerArgs& a, hipStream_t stream) {
  if (a.n_tok == 0) return hipSuccess;
  if (a.use_gemm) {
    const int ntt = (a.n_tok + kGemmTokens - 1) / kGemmTokens;
    const int ntiles = (a.max_hist_blocks + kGemmBlocks - 1) / kGemmBlocks;
    // about three workgroups per CU (as many as fit in LDS): split the block
    // tiles when there are few token tiles
    int splits = 1;
    while (splits < ntiles && (long long)ntt * splits < 768) ++splits;
    const int per = (ntiles + splits - 1) / splits;   // <= kGemmMaxTiles: the pass's page ids fit in LDS
    if (a.key_fp8)
      score_gemm_kernel<true><<<dim3((unsigned)ntt, (unsigned)splits), dim3(kThreads), 0, stream>>>(a, per);
    else
      score_gemm_kernel<false><<<dim3((unsigned)ntt, (unsigned)splits), dim3(kThreads), 0, stream>>>(a, per);
    finalize_kernel<<<dim3((unsigned)a.n_tok), dim3(kFinalThreads), (size_t)a.bitmap_words * 2 * 4, stream>>>(a);
    return hipGetLastError();
  }
  if (a.use_mfma16) {   // never with histories over kFuseLimit (the host checks)
    const int nrg = (a.n_tok + kMfmaRows - 1) / kMfmaRows;
    const int nchunk = (a.max_hist_blocks + a.chunk_blocks - 1) / a.chunk_blocks;
    const dim3 grid((unsigned)((long long)nrg * nchunk));
    if (a.key_fp8) score_mfma_kernel<true><<<grid, dim3(kThreads), 0, stream>>>(a);
    else score_mfma_kernel<false><<<grid, dim3(kThreads), 0, stream>>>(a);
    finalize_kernel<<<dim3((unsigned)a.n_tok), dim3(kFinalThreads), (size_t)a.bitmap_words * 2 * 4, stream>>>(a);
    return hipGetLastError();
  }
  const int ngroups = (a.n_tok + a.group_size - 1) / a.group_size;
  const int nchunk = (a.max_hist_blocks + a.chunk_blocks - 1) / a.chunk_blocks;
  const dim3 sgrid((unsigned)((long long)ngroups * nchunk));
  // Histories up to kFuseLimit blocks: finalize selects from the stored scores
  // (held in registers); longer ones: candidate lists and the select pass.
  const bool lists = a.max_hist_blocks > kFuseLimit;
#define SA_SCORE(GS)                                                                                 \
  do {                                                                                               \
    if (lists) {                                                                                     \
      if (a.key_fp8) score_kernel<GS, true, true><<<sgrid, dim3(kThreads), 0, stream>>>(a);          \
      else score_kernel<GS, true, false><<<sgrid, dim3(kThreads), 0, stream>>>(a);                   \
    } else {                                                                                         \
      if (a.key_fp8) score_kernel<GS, false, true><<<sgrid, dim3(kThreads), 0, stream>>>(a);         \
      else score_kernel<GS, false, false><<<sgrid, dim3(kThreads), 0, stream>>>(a);                  \
    }                                                                                                \
  } while (0)
  switch (a.group_size) {
    case 1: SA_SCORE(1); break;
    case 2: SA_SCORE(2); break;
    case 3: SA_SCORE(3); break;
    default: SA_SCORE(4); break;
  }
#undef SA_SCORE
  if (lists) select_kernel<<<dim3((unsigned)a.n_tok), dim3(kSelThreads), 0, stream>>>(a);
  else finalize_kernel<<<dim3((unsigned)a.n_tok), dim3(kFinalThreads), (size_t)a.bitmap_words * 2 * 4, stream>>>(a);
  return hipGetLastError();
}

}  // namespace sa
