// Block-gather GQA decode attention for gfx950: the sparse layer (selected
// blocks + current block) and the sliding-window layer share one kernel.
//
// What is computed: SGLang blog "Step 5 Preview: Day-0 Inference and RL Support
// with SGLang and Miles", section "Hybrid Attention" (exact attention over the
// tokens of up to 512 chosen earlier blocks plus the current block; three of
// four layers read the latest 512 tokens) and section "Kernels from StepFun"
// (decode attention over the selected blocks only, cut into partitions whose
// partial results are merged).  Shapes: open-weights blog config table (64 query
// heads, 4 KV groups, head dim 192).
//
// Work decomposition.  One workgroup of 4 waves owns one (query token, KV
// group, partition).  The partition's block list (logical block id and
// physical cache unit per slot) is resolved once into LDS.  The waves take
// 32-token chunks (4 blocks) round-robin; each wave keeps its own online-softmax
// state for the 16 heads of the group, and the 4 wave states are merged in LDS
// in a fixed order at the end (deterministic).
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, A: lane l holds row l%16, k-slice
// l/16; B: lane l holds column l%16, same k-slice; D: lane l holds rows
// 4*(l/16)+r, column l%16):
//   scores  S^T[token][head] = K[token][:] . Q[head][:]   (two 16-token halves)
//           A = K rows straight from the cache (16 B per lane per k-step),
//           B = Q of the 16 heads, loaded once.
//   output  O^T[dim][head] += V^T[dim][token] . P^T[token][head]
//           A = V from the cache (the V layout keeps 8 tokens of one dim in 16 B,
//           8 B in the one-byte form),
//           B = P: each lane already holds the 8 probabilities of "its" block for
//           "its" head, so no data moves between lanes.
// Token order inside a chunk is chosen so that the rows of the score half-tiles
// land in exactly the lanes the PV step needs them in (half s, row 4*j + r <->
// block j, token 4*s + r).
//
// Split calls (S > 1) write one partial result per partition. With kMerge the
// partitions of a (token, group) count their arrivals on an integer counter
// once their partial is visible device-wide; the last to arrive resets the
// counter and merges the S partials in the merge kernel's order and with its
// exact arithmetic, so no second launch is needed.

#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxSlots = SA_MAX_TOPK + 1 > SA_MAX_WINDOW / 8 + 2 ? SA_MAX_TOPK + 1 : SA_MAX_WINDOW / 8 + 2;
constexpr int kFillSlots = (kMaxSlots + kThreads - 1) / kThreads * kThreads;   // slot-table rows, whole passes
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegBig = -1.0e30f;   // running-max start: finite, so exp2 of differences never sees inf-inf

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};   // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Decode calls read each K/V block about once: non-temporal loads keep them
// from displacing reusable lines in L2 and the MALL. Calls with many query
// tokens per sequence (a prefill chunk) re-read blocks and use ordinary loads.
template <bool kStream>
__device__ __forceinline__ u32x4 load16_kv(const uint8_t* p) {
  if constexpr (kStream) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}

// Max / sum of v over lanes l, l^16, l^32, l^48 (the 4 lane groups holding one
// head): the row-swap instructions hand each lane {v[l], v[l^16]} (then ^32) in
// one VALU step, without an LDS round trip.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Reductions over the 64 lanes as butterflies (DPP swaps inside rows of 16,
// then row swaps): every lane ends with the same bits. The same order as the
// merge kernel's, so a merge here gives its results bit for bit.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max64(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));    // quad_perm 1,0,3,2
  v = fmaxf(v, dpp_move<0x4E>(v));    // quad_perm 2,3,0,1
  v = fmaxf(v, dpp_move<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_move<0x140>(v));   // row_mirror
  return max_over_groups(v);
}
__device__ __forceinline__ float wave_sum64(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  return sum_over_groups(v);
}

template <bool kStream>
__device__ __forceinline__ u32x2 load8_kv(const uint8_t* p) {
  if constexpr (kStream) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return *reinterpret_cast<const u32x2*>(p);
}

// Eight OCP E4M3 bytes (two words) to eight bf16 (an MFMA operand); exact.
template <bool kHiHalf>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHiHalf));
}
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
               fp8x2_to_bf16x2<true>(w1)};
}

// kFp8: one-byte caches. A K unit is [3 dim-blocks][8 tokens][64 dims], a V
// unit [192 dims][8 tokens] (8 bytes per dim); both are widened exactly to bf16
// right before their MFMA.
// Merge of the S partials of (token t, group g) into the output, by the
// workgroup of the partition that arrived last: wave w computes the weights of
// heads 4w .. 4w+3 (lane s holds partition s), then thread i accumulates dims
// 4*((i % 16) + 16 j), j < 3, of head i / 16 in the merge kernel's order: four
// quarter sums over consecutive partitions, added in quarter order.
__device__ void merge_group(const AttnArgs& a, int t, int g, int S, float* s_w /* [16][64] */,
                            float* s_ml /* [16][2] */) {
  constexpr float kLog2e = 1.44269504088896340736f;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = g * kHeadsPerGroup + 4 * wave + i;
    l[i] = lane < S ? a.part_lse[((size_t)t * S + lane) * kHeads + h] : -INFINITY;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float M = wave_max64(l[i]);
    const bool any = M != -INFINITY;
    const float w = (any && l[i] != -INFINITY) ? __builtin_amdgcn_exp2f((l[i] - M) * kLog2e) : 0.f;
    const float L = wave_sum64(w);
    const int hl = 4 * wave + i;
    s_w[hl * 64 + lane] = w;
    if (lane == 0) {
      s_ml[2 * hl] = M;
      s_ml[2 * hl + 1] = L;
    }
  }
  __syncthreads();
  const int hl = tid >> 4;   // head of the group
  const int head = g * kHeadsPerGroup + hl;
  const float* obase = a.part_o + ((size_t)t * S * kHeads + head) * kHeadDim + 4 * (tid & 15);
  const size_t sstride = (size_t)kHeads * kHeadDim;
  // the partitions in four consecutive quarters of R = ceil(S / 4): each
  // quarter summed in partition order, then ((A0 + A1) + A2) + A3
  const int R = (S + 3) / 4;
  f32x4 qacc[4][3];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq)
#pragma unroll
    for (int j = 0; j < 3; ++j) qacc[qq][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4 v[8][3];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < 3; ++j)
        v[u][j] = *reinterpret_cast<const f32x4*>(obase + (size_t)min(s0 + u, S - 1) * sstride + 64 * j);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // a partition with no weight (empty, or past S) adds nothing
      const float wgt = s0 + u < S ? s_w[hl * 64 + min(s0 + u, 63)] : 0.f;
      const int qs = (s0 + u) / R;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int j = 0; j < 3; ++j)
          qacc[qq][j] = (qs == qq && wgt != 0.f) ? qacc[qq][j] + v[u][j] * wgt : qacc[qq][j];
    }
  }
  f32x4 acc[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    acc[j] = qacc[0][j];
    acc[j] = acc[j] + qacc[1][j];
    acc[j] = acc[j] + qacc[2][j];
    acc[j] = acc[j] + qacc[3][j];
  }
  const float M = s_ml[2 * hl], L = s_ml[2 * hl + 1];
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  uint16_t* orow = a.merge_out + ((size_t)t * kHeads + head) * kHeadDim + 4 * (tid & 15);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    uint2 o;
    o.x = pack_bf16x2(acc[j][0] * inv, acc[j][1] * inv);
    o.y = pack_bf16x2(acc[j][2] * inv, acc[j][3] * inv);
    *reinterpret_cast<uint2*>(orow + 64 * j) = o;
  }
  if (a.merge_lse != nullptr && (tid & 15) == 0)
    a.merge_lse[(size_t)t * kHeads + head] = L > 0.f ? M + __builtin_amdgcn_logf(L) * kLn2 : -INFINITY;
}

template <bool kWindow, bool kStream, bool kFp8, bool kMerge>
__global__ __launch_bounds__(kThreads) void attention_kernel(AttnArgs a) {
  constexpr int kUnit = kFp8 ? kUnitBytes / 2 : kUnitBytes;
  __shared__ int32_t s_unit[kFillSlots];   // entries past the token's list are written and never read
  __shared__ int32_t s_beta[kFillSlots];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_e[kWaves][16];
  __shared__ f32x4 s_o[kWaves][9][64];   // per wave: the 9 output tiles other waves finish

  // Split-major order: the workgroups resident at one time share a partition
  // index, i.e. one slice of every token's (ascending) block list, which keeps
  // the live part of a large cache small enough to stay in L2/MALL when the
  // call is split.
  const int S = a.num_splits;
  const int wg = blockIdx.x;
  const int per_split = a.n_tok * kGroups;
  const int sp = wg / per_split;
  const int g = (wg % per_split) % kGroups;
  const int t = (wg % per_split) / kGroups;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 15;
  const int lg = lane >> 4;

  // ---- token and its attended block list --------------------------------
  // Q, the block ids and the page ids are located from the token's sequence
  // and position alone (every such read stays inside its table); the sequence
  // length only decides whether the token is valid, so no load waits for it.
  const int b = a.q_seq[t];
  const int p = a.q_pos[t];
  const bool in_range = b >= 0 && b < a.batch && p >= 0 && p < a.max_pages * kPageTokens;
  const int seq_len = a.seq_lens[in_range ? b : 0];

  // Q of head 16g + lq (B operand of the score MFMA): k-step i of lane group lg
  // covers dims 64*(i/2) + 16*lg + 8*(i%2) .. +8 (the order of the one-byte K
  // layout; both cache forms sum in this order)
  u32x4 qv[6];
  {
    const uint8_t* qrow = a.q + ((size_t)t * kHeads + g * kHeadsPerGroup + lq) * (kHeadDim * 2);
#pragma unroll
    for (int i = 0; i < 6; ++i) qv[i] = load16(qrow + (64 * (i >> 1) + 16 * lg + 8 * (i & 1)) * 2);
  }

  const int cb = in_range ? (p >> 3) : 0;
  int nslots = 0, lo = 0, b_lo = 0, nsel = 0;
  if (in_range) {
    if (kWindow) {
      lo = max(0, p - a.window + 1);
      b_lo = lo >> 3;
      nslots = cb - b_lo + 1;
    } else {
      nsel = min(a.topk, cb);
      nslots = nsel + 1;
    }
  }
  // This token's own partition count: S, or (split by length) the count its
  // own list length asks for, so that its partition boundaries do not depend
  // on the longest list of the call; its further partitions stay empty.
  const int St = a.split_blocks > 0 ? min(S, max(1, (nslots + a.split_blocks - 1) / a.split_blocks)) : S;
  const bool live = sp < St;
  // sp * nslots < 64 * 514: 32-bit division
  const int s0 = live ? (int)((unsigned)(sp * nslots) / (unsigned)St) : 0;
  const int s1 = live ? (int)((unsigned)((sp + 1) * nslots) / (unsigned)St) : 0;
  const int n_all = s1 - s0;

  // Slot table: every thread issues all of its block-id loads, then all of its
  // page-id loads; each read is clamped into its table (entries past the list
  // are read and dropped), so neither waits behind the other's round trip.
  {
    constexpr int kFill = kFillSlots / kThreads;
    const int32_t* prow = a.page_table + (size_t)(in_range ? b : 0) * a.max_pages;
    const int32_t* srow = kWindow ? nullptr   // (a window call has no block-id table)
        : a.sel_idx + ((size_t)t * (a.sel_per_group ? kGroups : 1) + (a.sel_per_group ? g : 0)) * a.topk;
    int beta[kFill];
    bool ok[kFill];
#pragma unroll
    for (int r = 0; r < kFill; ++r) {
      const int slot = s0 + tid + r * kThreads;
      if (kWindow) {
        beta[r] = b_lo + slot;
        ok[r] = true;
      } else {
        const int v = srow[min(slot, a.topk - 1)];
        beta[r] = slot < nsel ? v : cb;
        ok[r] = (slot >= nsel) | ((v >= 0) & (v < cb));
      }
    }
    int page[kFill];
#pragma unroll
    for (int r = 0; r < kFill; ++r) page[r] = prow[min(max(beta[r], 0) >> 3, a.max_pages - 1)];
#pragma unroll
    for (int r = 0; r < kFill; ++r) {   // unconditional, so that no load is moved behind a branch
      const bool readable = ok[r] & (page[r] >= 0) & (page[r] < a.num_pages);   // no short circuit: no branch
      s_unit[tid + r * kThreads] = readable ? (page[r] * kGroups + g) * kBlocksPerPage + (beta[r] & 7) : -1;
      s_beta[tid + r * kThreads] = ok[r] ? beta[r] : 0;
    }
  }
  const bool valid = in_range && p < seq_len;
  const int n = valid ? n_all : 0;   // an invalid token attends nothing
  __syncthreads();

  // ---- per-wave streaming loop -------------------------------------------
  const float sc = a.scale_log2;
  const int nchunks = (n + 3) >> 2;
  float m_run = kNegBig;
  float l_run = 0.f;   // sum of the bf16-rounded probabilities (normalises O)
  float e_run = 0.f;   // sum of the unrounded probabilities (gives lse)
  f32x4 acc[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K lane offset inside a unit: bf16: dim chunk 2*lg (+8*(i/2) + i%2), token
  // (lq & 3) (+4 for half 1); one-byte: dim-block j (+512 j), token (lq & 3) (+4
  // for half 1), dims 16*lg .. 16*lg+15 of the block -- each load step reads 256
  // contiguous bytes of every unit
  const uint8_t* kbase = kFp8 ? a.k_cache + (lq & 3) * 64 + lg * 16 : a.k_cache + lg * 256 + (lq & 3) * 16;
  // V lane offset inside a unit: dim lq (+16 per output tile), all 8 tokens
  const uint8_t* vbase = a.v_cache + lq * (kFp8 ? 8 : 16);

  u32x4 kr[2][6];      // bf16 K operands
  u32x4 vr[12];        // bf16 V operands
  u32x4 kq[2][3];      // one-byte K: 16 dims (two k-steps) per dim-block and half
  u32x2 vq[12];        // one-byte V: 8 tokens of one dim

  // Loads are branch-free so that the compiler's waits stay precise: a slot
  // with nothing to read (padding, unreadable page) reads unit 0 instead, and
  // its scores are masked to -inf and its V zeroed below.
  auto load_k = [&](int c) {
    const int slot = 4 * c + (lq >> 2);
    const int unit = slot < n ? max(s_unit[slot], 0) : 0;
    const uint8_t* pk = kbase + (size_t)unit * kUnit;
    if constexpr (kFp8) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        kq[0][j] = load16_kv<kStream>(pk + j * 512);
        kq[1][j] = load16_kv<kStream>(pk + j * 512 + 256);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const int off = (8 * (i >> 1) + (i & 1)) * 128;
        kr[0][i] = load16_kv<kStream>(pk + off);
        kr[1][i] = load16_kv<kStream>(pk + off + 64);
      }
    }
  };
  auto load_v = [&](int c) {
    const int slot = 4 * c + lg;
    const int unit = slot < n ? max(s_unit[slot], 0) : 0;
    const uint8_t* pv = vbase + (size_t)unit * kUnit;
    if constexpr (kFp8) {
#pragma unroll
      for (int i = 0; i < 12; ++i) vq[i] = load8_kv<kStream>(pv + i * 128);
    } else {
#pragma unroll
      for (int i = 0; i < 12; ++i) vr[i] = load16_kv<kStream>(pv + i * 256);
    }
  };

  // Chunks of this wave: wave, wave + 4, ... The next chunk's K is issued
  // right after the score MFMAs and its V right after the PV MFMAs. The last
  // chunk is a separate copy of the body without the prefetch, so that every
  // wait covers exactly the data it needs and no load is left in flight at the
  // merge.
  auto chunk = [&](int c, auto prefetch) {
    constexpr bool kPrefetch = decltype(prefetch)::value;
    const int cn = c + kWaves;
    f32x4 st0 = {0.f, 0.f, 0.f, 0.f}, st1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      if constexpr (kFp8) {
        const u32x4 w0 = kq[0][i >> 1], w1 = kq[1][i >> 1];
        const int h = (i & 1) * 2;
        st0 = mfma_bf16(fp8x8_to_bf16x8(w0[h], w0[h + 1]), qv[i], st0);
        st1 = mfma_bf16(fp8x8_to_bf16x8(w1[h], w1[h + 1]), qv[i], st1);
      } else {
        st0 = mfma_bf16(kr[0][i], qv[i], st0);
        st1 = mfma_bf16(kr[1][i], qv[i], st1);
      }
    }
    // keep the refill below the MFMAs that read the K registers: hoisting it
    // would need a second set of them
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPrefetch) load_k(cn);

    // this lane's block (lg) of the chunk and its valid positions
    const int slot = 4 * c + lg;
    const bool blk_ok = slot < n && s_unit[slot] >= 0;
    const int pos0 = (slot < n ? s_beta[slot] : 0) * kBlockTokens;
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = st0[r] * sc;
      x[4 + r] = st1[r] * sc;
    }
    uint32_t okmask = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool ok = blk_ok && (pos0 + k <= p) && (pos0 + k >= lo);
      okmask |= ok ? (1u << k) : 0u;
      x[k] = ok ? x[k] : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = fmaxf(mx, x[k]);
    mx = max_over_groups(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float pr[8];
    float esum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pr[k] = __builtin_amdgcn_exp2f(x[k] - m_new);
      esum += pr[k];
    }
    const u32x4 pb = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                      pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    // the row sum that normalises O uses the same rounded probabilities the PV
    // product sees; the unrounded sum gives lse
    float psum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      psum += __uint_as_float(pb[w] << 16) + __uint_as_float(pb[w] & 0xffff0000u);
    l_run = l_run * alpha + psum;
    e_run = e_run * alpha + esum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 12; ++i) acc[i] *= alpha;

    // Positions outside the attended range (the current block past p, the
    // window's first block before lo, slots that read unit 0 as a stand-in)
    // may hold anything; zero their V so that a zero probability never meets a
    // non-finite value.
    if constexpr (kFp8) {
      // byte mask over the 8 tokens (code 0 is +0)
      uint32_t m8[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) m |= (okmask >> (4 * w + k)) & 1u ? 0xffu << (8 * k) : 0u;
        m8[w] = m;
      }
#pragma unroll
      for (int i = 0; i < 12; ++i)
        acc[i] = mfma_bf16(fp8x8_to_bf16x8(vq[i].x & m8[0], vq[i].y & m8[1]), pb, acc[i]);
    } else {
      if (__any(okmask != 0xffu)) {
        u32x4 vm;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo16 = (okmask >> (2 * w)) & 1u ? 0x0000ffffu : 0u;
          const uint32_t hi16 = (okmask >> (2 * w + 1)) & 1u ? 0xffff0000u : 0u;
          vm[w] = lo16 | hi16;
        }
#pragma unroll
        for (int i = 0; i < 12; ++i) vr[i] &= vm;
      }
#pragma unroll
      for (int i = 0; i < 12; ++i) acc[i] = mfma_bf16(vr[i], pb, acc[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPrefetch) load_v(cn);
  };
  if (wave < nchunks) {
    const int c_last = wave + ((nchunks - 1 - wave) / kWaves) * kWaves;
    load_k(wave);
    load_v(wave);
    // (a do-while: the V refill at the end of each pass is consumed on every
    // path, by the next pass or by the last chunk, so it stays where it is)
    if (wave < c_last) {
      int c = wave;
      do {
        chunk(c, std::true_type{});
        c += kWaves;
      } while (c < c_last);
    }
    chunk(c_last, std::false_type{});
  }

  // ---- merge the 4 wave states (fixed order) and write -------------------
  // Wave w finishes output tiles 3w .. 3w+2: every wave leaves in LDS the 9
  // tiles the other waves finish, then reads the 3 partial tiles it needs from
  // each of them (all reads in flight together).
  const float l_tot = sum_over_groups(l_run);
  const float e_tot = sum_over_groups(e_run);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const int owner = i / 3;
    if (owner != wave) s_o[wave][i - (owner > wave ? 3 : 0)][lane] = acc[i];
  }
  if (lg == 0) {
    s_m[wave][lq] = m_run;
    s_l[wave][lq] = l_tot;
    s_e[wave][lq] = e_tot;
  }
  __syncthreads();

  float mw[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mw[w] = s_m[w][lq];
  // x[w][j]: wave w's partial of tile 3*wave + j (for w == wave a stand-in
  // read, replaced by the registers)
  f32x4 x[kWaves][3];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
#pragma unroll
    for (int j = 0; j < 3; ++j) x[w][j] = s_o[w][min(3 * wave + j - (wave > w ? 3 : 0), 8)][lane];
  }
  f32x4 own[3];
#pragma unroll
  for (int j = 0; j < 3; ++j)
    own[j] = wave == 0 ? acc[j] : wave == 1 ? acc[3 + j] : wave == 2 ? acc[6 + j] : acc[9 + j];
  float M = mw[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[w]);
  float L = 0.f, E = 0.f;
  f32x4 o[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float aw = __builtin_amdgcn_exp2f(mw[w] - M);
    L += s_l[w][lq] * aw;
    E += s_e[w][lq] * aw;
#pragma unroll
    for (int j = 0; j < 3; ++j) o[j] += (w == wave ? own[j] : x[w][j]) * aw;
  }
  const bool any = L > 0.f;
  const float inv = any ? a.v_scale / L : 0.f;   // V scale of a one-byte cache (1 for bf16)
  const float lse = any ? (M + __builtin_amdgcn_logf(E)) * kLn2 : -INFINITY;
  const int head = g * kHeadsPerGroup + lq;

  if (S == 1) {
    uint16_t* orow = a.out + ((size_t)t * kHeads + head) * kHeadDim + 4 * lg + 48 * wave;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      uint2 v;
      v.x = pack_bf16x2(o[j][0] * inv, o[j][1] * inv);
      v.y = pack_bf16x2(o[j][2] * inv, o[j][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * j) = v;
    }
    if (a.out_lse != nullptr && wave == 0 && lg == 0) a.out_lse[(size_t)t * kHeads + head] = lse;
  } else {
    float* orow = a.part_o + (((size_t)t * S + sp) * kHeads + head) * kHeadDim + 4 * lg + 48 * wave;
    float* lrow = a.part_lse + ((size_t)t * S + sp) * kHeads + head;
    if constexpr (!kMerge) {
#pragma unroll
      for (int j = 0; j < 3; ++j) *reinterpret_cast<f32x4*>(orow + 16 * j) = o[j] * inv;
      if (wave == 0 && lg == 0) *lrow = lse;
    } else {
      // The partial is written with device-scope atomic stores, which are
      // visible device-wide once they complete (no L2 write-back needed, as an
      // ordinary store's would be); once every thread's stores have completed
      // the partition counts its arrival. The last of the S partitions resets
      // the counter for the next call, and after a device-scope acquire (an L2
      // invalidate on its own XCD only) merges the S partials.
      __shared__ uint32_t s_last;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const f32x4 v = o[j] * inv;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __hip_atomic_store(reinterpret_cast<uint32_t*>(orow + 16 * j + r), __float_as_uint(v[r]), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      if (wave == 0 && lg == 0)
        __hip_atomic_store(reinterpret_cast<uint32_t*>(lrow), __float_as_uint(lse), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);   // this thread's stores have completed
      __syncthreads();                 // ... and every other thread's
      if (tid == 0) {
        uint32_t* ctr = a.merge_counters + (size_t)t * kGroups + g;
        const uint32_t before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = before == (uint32_t)(S - 1) ? 1u : 0u;
        if (s_last) *ctr = 0u;   // every partition has counted: none touches it again in this call
      }
      __syncthreads();
      if (s_last == 0u) return;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      // s_o is free now: weights [16][64] and (M, L) per head
      merge_group(a, t, g, S, reinterpret_cast<float*>(&s_o[0][0][0]), reinterpret_cast<float*>(&s_o[1][0][0]));
    }
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, bool window_mode, hipStream_t stream) {
  if (a.n_tok == 0) return hipSuccess;
  const long long grid = (long long)a.n_tok * kGroups * a.num_splits;
  const dim3 g((unsigned)grid), b(kThreads);
  const bool merge = a.num_splits > 1 && a.merge_counters != nullptr;
#define SA_ATTN(W, F)                                                                       \
  do {                                                                                      \
    if (merge) {                                                                            \
      if (a.stream_kv) attention_kernel<W, true, F, true><<<g, b, 0, stream>>>(a);          \
      else attention_kernel<W, false, F, true><<<g, b, 0, stream>>>(a);                     \
    } else {                                                                                \
      if (a.stream_kv) attention_kernel<W, true, F, false><<<g, b, 0, stream>>>(a);         \
      else attention_kernel<W, false, F, false><<<g, b, 0, stream>>>(a);                    \
    }                                                                                       \
  } while (0)
  if (window_mode) {
    if (a.kv_fp8) SA_ATTN(true, true);
    else SA_ATTN(true, false);
  } else {
    if (a.kv_fp8) SA_ATTN(false, true);
    else SA_ATTN(false, false);
  }
#undef SA_ATTN
  return hipGetLastError();
}

}  // namespace sa
