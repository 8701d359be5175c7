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
// Pipeline (four launches on the caller's stream):
//  1. zero      clear the per-token histograms and candidate counters.
//  2. score     stream every historical index key of a sequence once and score
//               all of that sequence's query tokens against it (v_dot2 bf16 ->
//               fp32); write fp32 scores and add each score to a 2048-bin
//               histogram of the top 11 bits of its order-preserving key.
//  3. collect   per (token, score chunk): find the histogram bin that holds the
//               k-th largest score and append every score at or above that bin
//               to a small per-token candidate list.
//  4. finalize  per token: exact radix select (11 + 11 + 10 bits) of the k-th
//               largest key among the candidates, ties at that key go to the
//               lower block id, then rank the chosen ids to write them ascending.
//               A token whose candidate list overflowed takes the same radix
//               select over all of its scores instead.

#include <algorithm>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxGroup = 4;

__device__ __forceinline__ u32x4 load16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

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

// Historical block count of token t (0 for a token whose sequence or position
// is out of range).
__device__ __forceinline__ int hist_blocks(const IndexerArgs& a, int t, int* seq_out) {
  const int b = a.q_seq[t];
  const int p = a.q_pos[t];
  *seq_out = b;
  if (b < 0 || b >= a.batch || p < 0) return 0;
  if (p >= a.seq_lens[b] || p >= a.max_pages * kPageTokens) return 0;
  return p >> 3;
}

// ---------------------------------------------------------------------------
// block-wide helpers (256 threads = 4 waves)
// ---------------------------------------------------------------------------

// Exclusive suffix sum over the 256 threads: returns sum of v over threads > tid.
__device__ uint32_t block_suffix_exclusive(uint32_t v, uint32_t* s_tmp /*[4]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(x, off);
    if (lane + off < 64) x += y;
  }
  if (lane == 0) s_tmp[wave] = x;   // wave total
  __syncthreads();
  uint32_t above = 0;
  for (int w = wave + 1; w < 4; ++w) above += s_tmp[w];
  __syncthreads();
  return above + x - v;
}

// Exclusive prefix sum over the 256 threads; *total receives the block total.
__device__ uint32_t block_prefix_exclusive(uint32_t v, uint32_t* s_tmp /*[4]*/, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  uint32_t below = 0, tot = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) below += s_tmp[w];
    tot += s_tmp[w];
  }
  __syncthreads();
  *total = tot;
  return below + x - v;
}

// Among bins h[0..nbins) (a higher bin holds larger keys), find the bin that
// holds the k-th largest element: above < k <= above + h[bin], where above is
// the count in higher bins. Needs sum(h) >= k >= 1 and nbins in {1024, 2048}.
// Result is broadcast through s_res[0] (bin) and s_res[1] (above).
__device__ void select_bin(const uint32_t* h, int nbins, uint32_t k, uint32_t* s_tmp, uint32_t* s_res) {
  if (threadIdx.x == 0) {   // defined result even for inconsistent input
    s_res[0] = 0u;
    s_res[1] = 0u;
  }
  const int per = nbins / kThreads;
  const int b0 = threadIdx.x * per;
  uint32_t part = 0;
  for (int i = 0; i < per; ++i) part += h[b0 + i];
  uint32_t cum = block_suffix_exclusive(part, s_tmp);
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
// 1. zero
// ---------------------------------------------------------------------------
__global__ void zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// 2. score
// ---------------------------------------------------------------------------
// One pass over blocks [lo, hi) of sequence b for NQ query tokens. Four lanes
// share one block key: lane quarter q4 reads 16-byte chunks 4i + q4 (i = 0..7),
// so each quad reads 64 contiguous bytes per load and a wave covers 16 keys.
template <int NQ>
__device__ void score_run(const IndexerArgs& a, int b, const int* tok, const int* hslot, const int* ncb,
                          int lo, int hi, uint32_t (*s_hist)[kHistBins]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q4 = lane & 3;
  const int sub = lane >> 2;
  u32x4 qv[NQ][8];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const uint8_t* qp = a.q_idx + (size_t)tok[j] * kKeyBytes + q4 * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[j][i] = load16(qp + i * 64);
  }
  const int32_t* prow = a.page_table + (size_t)b * a.max_pages;
  for (int base = lo + wave * 16; base < hi; base += 64) {
    const int beta = base + sub;
    const bool in = beta < hi;
    const int page = in ? prow[beta >> 3] : -1;
    const bool ok = in && page >= 0 && page < a.num_pages;
    u32x4 kv[8];
    if (ok) {
      const uint8_t* kp = a.k_idx_cache + ((size_t)page * kBlocksPerPage + (beta & 7)) * kKeyBytes + q4 * 16;
#pragma unroll
      for (int i = 0; i < 8; ++i) kv[i] = load16(kp + i * 64);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) kv[i] = u32x4{0, 0, 0, 0};
    }
    float acc[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int w = 0; w < 4; ++w) s = dot2(kv[i][w], qv[j][i][w], s);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      acc[j] = ok ? s : -INFINITY;   // an unreadable page ranks last
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (in && q4 == (j & 3) && beta < ncb[j]) {
        a.scores[(size_t)tok[j] * a.max_hist_blocks + beta] = acc[j];
        atomicAdd(&s_hist[hslot[j]][score_key(acc[j]) >> 21], 1u);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void score_kernel(IndexerArgs a) {
  __shared__ uint32_t s_hist[kMaxGroup][kHistBins];
  const int nchunk = (a.max_hist_blocks + a.chunk_blocks - 1) / a.chunk_blocks;
  const int chunk = blockIdx.x % nchunk;
  const int grp = blockIdx.x / nchunk;
  const int t0 = grp * a.group_size;
  const int ng = min(a.group_size, a.n_tok - t0);
  int seq[kMaxGroup], ncb[kMaxGroup];
  for (int j = 0; j < kMaxGroup; ++j) {
    ncb[j] = 0;
    seq[j] = -1;
    if (j < ng) ncb[j] = min(hist_blocks(a, t0 + j, &seq[j]), a.max_hist_blocks);
  }
  const int lo = chunk * a.chunk_blocks;
  bool any = false;
  for (int j = 0; j < ng; ++j) any |= ncb[j] > lo;
  if (!any) return;

  for (int i = threadIdx.x; i < ng * kHistBins; i += kThreads) (&s_hist[0][0])[i] = 0u;
  __syncthreads();

  uint32_t done = 0;
  for (int j0 = 0; j0 < ng; ++j0) {
    if ((done >> j0) & 1u) continue;
    int tok[kMaxGroup], hslot[kMaxGroup], cbs[kMaxGroup];
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
    switch (nq) {
      case 1: score_run<1>(a, seq[j0], tok, hslot, cbs, lo, hi, s_hist); break;
      case 2: score_run<2>(a, seq[j0], tok, hslot, cbs, lo, hi, s_hist); break;
      case 3: score_run<3>(a, seq[j0], tok, hslot, cbs, lo, hi, s_hist); break;
      case 4: score_run<4>(a, seq[j0], tok, hslot, cbs, lo, hi, s_hist); break;
      default: break;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ng * kHistBins; i += kThreads) {
    const uint32_t v = (&s_hist[0][0])[i];
    if (v) atomicAdd(&a.hist[(size_t)(t0 + i / kHistBins) * kHistBins + (i % kHistBins)], v);
  }
}

// ---------------------------------------------------------------------------
// 3. collect
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void collect_kernel(IndexerArgs a) {
  __shared__ uint32_t s_h[kHistBins];
  __shared__ uint32_t s_tmp[4];
  __shared__ uint32_t s_res[2];
  const int nck = (a.max_hist_blocks + kCollectChunk - 1) / kCollectChunk;
  const int ck = blockIdx.x % nck;
  const int t = blockIdx.x / nck;
  int b;
  const int ncand = min(hist_blocks(a, t, &b), a.max_hist_blocks);
  const int lo = ck * kCollectChunk;
  if (ncand <= a.topk || lo >= ncand) return;
  const int hi = min(ncand, lo + kCollectChunk);
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) s_h[i] = a.hist[(size_t)t * kHistBins + i];
  __syncthreads();
  select_bin(s_h, kHistBins, (uint32_t)a.topk, s_tmp, s_res);
  const uint32_t b1 = s_res[0];

  const float* srow = a.scores + (size_t)t * a.max_hist_blocks;
  uint2* crow = a.cand + (size_t)t * kCandCap;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = lo + wave * 64; base < hi; base += kThreads) {
    const int beta = base + lane;
    uint32_t key = 0;
    bool take = false;
    if (beta < hi) {
      key = score_key(srow[beta]);
      take = (key >> 21) >= b1;
    }
    const uint64_t m = __ballot(take);
    if (m == 0) continue;
    uint32_t basepos = 0;
    if (lane == 0) basepos = atomicAdd(&a.cand_count[t], (uint32_t)__popcll(m));
    basepos = __shfl(basepos, 0);
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (take && basepos + rank < (uint32_t)kCandCap) crow[basepos + rank] = make_uint2(key, (uint32_t)beta);
  }
}

// ---------------------------------------------------------------------------
// 4. finalize
// ---------------------------------------------------------------------------
struct FinalizeLds {
  uint32_t key[kCandCap];
  uint32_t idx[kCandCap];
  uint32_t h[kHistBins];
  int32_t sel[SA_MAX_TOPK];
  uint32_t tmp[4];
  uint32_t res[2];
  uint32_t n_gt;
  uint32_t n_eq;
};

// Exact k-th largest key over the keys held in LDS (n of them): three radix
// levels. Returns tau; *count_gt receives how many keys are strictly larger.
__device__ uint32_t radix_kth_lds(FinalizeLds& s, int n, uint32_t k, uint32_t* count_gt) {
  uint32_t prefix = 0, above = 0;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int lvl = 0; lvl < 3; ++lvl) {
    const int sh = shifts[lvl];
    const int nb = 1 << widths[lvl];
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) s.h[i] = 0u;
    __syncthreads();
    const int hs = sh + widths[lvl];   // bits above this digit must match the prefix
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t key = s.key[i];
      const bool match = hs >= 32 || (key >> hs) == (prefix >> hs);
      if (match) atomicAdd(&s.h[(key >> sh) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    select_bin(s.h, nb, k - above, s.tmp, s.res);
    prefix |= s.res[0] << sh;
    above += s.res[1];
    __syncthreads();
  }
  *count_gt = above;
  return prefix;
}

// Same radix select over all scores of a token in global memory (fallback for
// candidate-list overflow); level 1 uses the histogram built by the score pass.
__device__ uint32_t radix_kth_global(const IndexerArgs& a, FinalizeLds& s, int t, int ncand, uint32_t k,
                                     uint32_t* count_gt) {
  const float* srow = a.scores + (size_t)t * a.max_hist_blocks;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) s.h[i] = a.hist[(size_t)t * kHistBins + i];
  __syncthreads();
  select_bin(s.h, kHistBins, k, s.tmp, s.res);
  uint32_t prefix = s.res[0] << 21;
  uint32_t above = s.res[1];
  __syncthreads();
  const int shifts[2] = {10, 0};
  const int widths[2] = {11, 10};
  for (int lvl = 0; lvl < 2; ++lvl) {
    const int sh = shifts[lvl];
    const int nb = 1 << widths[lvl];
    const int hs = sh + widths[lvl];
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) s.h[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < ncand; i += kThreads) {
      const uint32_t key = score_key(srow[i]);
      if ((key >> hs) == (prefix >> hs)) atomicAdd(&s.h[(key >> sh) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    select_bin(s.h, nb, k - above, s.tmp, s.res);
    prefix |= s.res[0] << sh;
    above += s.res[1];
    __syncthreads();
  }
  *count_gt = above;
  return prefix;
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(IndexerArgs a) {
  __shared__ FinalizeLds s;
  const int t = blockIdx.x;
  const int k = a.topk;
  int b;
  const int ncand = min(hist_blocks(a, t, &b), a.max_hist_blocks);
  int32_t* out = a.sel_idx + (size_t)t * k;
  if (ncand <= k) {
    for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < ncand ? i : -1;
    return;
  }
  const uint32_t n = a.cand_count[t];
  if (n > (uint32_t)kCandCap) {
    // Overflow: radix select over every score, then an ordered compaction.
    uint32_t count_gt;
    const uint32_t tau = radix_kth_global(a, s, t, ncand, (uint32_t)k, &count_gt);
    count_gt = min(count_gt, (uint32_t)k);
    const uint32_t need_eq = (uint32_t)k - count_gt;
    const float* srow = a.scores + (size_t)t * a.max_hist_blocks;
    uint32_t eq_before = 0, sel_before = 0;
    for (int base = 0; base < ncand; base += kThreads) {
      const int beta = base + threadIdx.x;
      uint32_t key = 0;
      if (beta < ncand) key = score_key(srow[beta]);
      const bool gt = beta < ncand && key > tau;
      const bool eq = beta < ncand && key == tau;
      uint32_t eq_tot, sel_tot;
      const uint32_t eq_rank = eq_before + block_prefix_exclusive(eq ? 1u : 0u, s.tmp, &eq_tot);
      const bool take = gt || (eq && eq_rank < need_eq);
      const uint32_t pos = sel_before + block_prefix_exclusive(take ? 1u : 0u, s.tmp, &sel_tot);
      if (take && pos < (uint32_t)k) out[pos] = beta;
      eq_before += eq_tot;
      sel_before += sel_tot;
    }
    return;
  }
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
    const uint2 c = a.cand[(size_t)t * kCandCap + i];
    s.key[i] = c.x;
    s.idx[i] = c.y;
  }
  if (threadIdx.x == 0) {
    s.n_gt = 0;
    s.n_eq = 0;
  }
  __syncthreads();
  uint32_t count_gt;
  const uint32_t tau = radix_kth_lds(s, (int)n, (uint32_t)k, &count_gt);
  count_gt = min(count_gt, (uint32_t)k);
  const uint32_t need_eq = (uint32_t)k - count_gt;
  // Keys above tau are all chosen; keys equal to tau are parked in h[] (reused)
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
    const uint32_t key = s.key[i];
    if (key > tau) {
      const uint32_t slot = atomicAdd(&s.n_gt, 1u);
      if (slot < (uint32_t)SA_MAX_TOPK) s.sel[slot] = (int32_t)s.idx[i];
    }
    else if (key == tau) s.h[atomicAdd(&s.n_eq, 1u) % kHistBins] = s.idx[i];
  }
  __syncthreads();
  const uint32_t n_eq = s.n_eq;
  if (n_eq <= (uint32_t)kHistBins) {
    for (uint32_t i = threadIdx.x; i < n_eq; i += kThreads) {
      const uint32_t me = s.h[i];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < n_eq; ++j) rank += s.h[j] < me ? 1u : 0u;
      if (rank < need_eq) s.sel[count_gt + rank] = (int32_t)me;
    }
  } else {
    // more ties than the parking space: rank them straight from the candidate list
    for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
      if (s.key[i] != tau) continue;
      const uint32_t me = s.idx[i];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < n; ++j) rank += (s.key[j] == tau && s.idx[j] < me) ? 1u : 0u;
      if (rank < need_eq) s.sel[count_gt + rank] = (int32_t)me;
    }
  }
  __syncthreads();
  // chosen ids are distinct: their rank among themselves is their output slot
  for (int i = threadIdx.x; i < k; i += kThreads) {
    const int32_t me = s.sel[i];
    int r = 0;
    for (int j = 0; j < k; ++j) r += s.sel[j] < me ? 1 : 0;
    out[r] = me;
  }
}

}  // namespace

IndexerWorkspace indexer_workspace_layout(int n_tok, int max_pages_per_seq) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  IndexerWorkspace w;
  const size_t nt = (size_t)(n_tok > 0 ? n_tok : 0);
  const size_t mhb = (size_t)(max_pages_per_seq > 0 ? max_pages_per_seq : 0) * kBlocksPerPage;
  w.hist_off = 0;
  w.count_off = up(nt * kHistBins * 4);
  w.scores_off = w.count_off + up(nt * 4);
  w.cand_off = w.scores_off + up(nt * mhb * 4);
  w.total = w.cand_off + up(nt * kCandCap * 8);
  return w;
}

hipError_t launch_indexer_topk(const IndexerArgs& a, hipStream_t stream) {
  if (a.n_tok == 0) return hipSuccess;
  const size_t nzero = (size_t)a.n_tok * kHistBins + (size_t)a.n_tok;   // hist then counters (adjacent)
  const unsigned zblocks = (unsigned)std::min<size_t>((nzero + 1023) / 1024, 4096);
  // hist and counters are contiguous only up to the padding of the hist region;
  // clear them separately to stay exact.
  zero_kernel<<<zblocks, 1024, 0, stream>>>(a.hist, (size_t)a.n_tok * kHistBins);
  zero_kernel<<<1, 1024, 0, stream>>>(a.cand_count, (size_t)a.n_tok);
  const int ngroups = (a.n_tok + a.group_size - 1) / a.group_size;
  const int nchunk = (a.max_hist_blocks + a.chunk_blocks - 1) / a.chunk_blocks;
  score_kernel<<<dim3((unsigned)((long long)ngroups * nchunk)), dim3(kThreads), 0, stream>>>(a);
  const int nck = (a.max_hist_blocks + kCollectChunk - 1) / kCollectChunk;
  collect_kernel<<<dim3((unsigned)((long long)a.n_tok * nck)), dim3(kThreads), 0, stream>>>(a);
  finalize_kernel<<<dim3((unsigned)a.n_tok), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace sa
