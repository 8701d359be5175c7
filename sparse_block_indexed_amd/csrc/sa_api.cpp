// C ABI of libsa.so: host-side validation and launch policy. Every entry point
// only checks its arguments and enqueues kernels on the caller's stream.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "sa_internal.h"

namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kMaxPagesPerSeq = 1 << 20;   // positions stay below 2^26
constexpr int kMaxPoolPages = 1 << 25;     // (page * 4 + group) * 8 + block fits in int32
constexpr int kMaxGroupedTokens = (1 << 29) - 1;   // tokens x 4 query rows fit in int32
constexpr long long kMaxGridThreads = 1LL << 32;    // threads of one grid dimension stay below this

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

sa_status check_desc(const sa_paged_desc& pd) {
  if (pd.page_table == nullptr || pd.seq_lens == nullptr) return SA_ERR_INVALID_ARG;
  if (!aligned(pd.page_table, 4) || !aligned(pd.seq_lens, 4)) return SA_ERR_INVALID_ARG;
  if (pd.batch < 1 || pd.max_pages_per_seq < 1 || pd.num_pages < 1) return SA_ERR_INVALID_ARG;
  if (pd.max_pages_per_seq > kMaxPagesPerSeq || pd.num_pages > kMaxPoolPages) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

sa_status check_tokens(const int32_t* q_seq, const int32_t* q_pos) {
  if (q_seq == nullptr || q_pos == nullptr) return SA_ERR_INVALID_ARG;
  if (!aligned(q_seq, 4) || !aligned(q_pos, 4)) return SA_ERR_INVALID_ARG;
  return SA_OK;
}

sa_status decode_common(const void* q, const void* k_cache, const void* v_cache, const sa_paged_desc& pd,
                        const int32_t* q_seq, const int32_t* q_pos, int n_tok, float softmax_scale,
                        int max_blocks, int num_splits, float* part_o, float* part_lse, uint32_t* merge_counters,
                        void* out, float* out_lse, bool window_mode, const int32_t* sel_idx, int topk, int window,
                        bool kv_fp8, float k_scale, float v_scale, bool sel_per_group, hipStream_t stream) {
  if (n_tok < 0 || num_splits < SA_SPLITS_FILL_GPU) return SA_ERR_INVALID_ARG;
  if (n_tok == 0) return SA_OK;
  if (!(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f)) return SA_ERR_INVALID_ARG;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr) return SA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return SA_ERR_INVALID_ARG;
  sa_status st = check_desc(pd);
  if (st != SA_OK) return st;
  if ((st = check_tokens(q_seq, q_pos)) != SA_OK) return st;
  if (!isfinite(softmax_scale)) return SA_ERR_INVALID_ARG;
  if (num_splits > SA_MAX_SPLITS) return SA_ERR_UNSUPPORTED;
  const int S = sa_resolve_num_splits(n_tok, max_blocks, num_splits);
  // launch limits: fewer than 2^32 threads per grid (attention: 256 per
  // (token, group, partition); merge: 256 per (token, head))
  if ((long long)n_tok * sa::kGroups * S * 256 >= kMaxGridThreads) return SA_ERR_UNSUPPORTED;
  if (S > 1 && (long long)n_tok * sa::kHeads * 256 >= kMaxGridThreads) return SA_ERR_UNSUPPORTED;
  if (S == 1 && out == nullptr) return SA_ERR_INVALID_ARG;
  if (S > 1 && (part_o == nullptr || part_lse == nullptr)) return SA_ERR_INVALID_ARG;
  if (out != nullptr && !aligned(out, 16)) return SA_ERR_INVALID_ARG;
  if (part_o != nullptr && !aligned(part_o, 16)) return SA_ERR_INVALID_ARG;
  if (part_lse != nullptr && !aligned(part_lse, 4)) return SA_ERR_INVALID_ARG;
  if (out_lse != nullptr && !aligned(out_lse, 4)) return SA_ERR_INVALID_ARG;
  if (merge_counters != nullptr && !aligned(merge_counters, 4)) return SA_ERR_INVALID_ARG;

  sa::AttnArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.page_table = pd.page_table;
  a.seq_lens = pd.seq_lens;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.sel_idx = sel_idx;
  a.n_tok = n_tok;
  a.topk = topk;
  a.window = window;
  a.num_splits = S;
  // by length: a token with a shorter list than the longest uses fewer partitions
  a.split_blocks = num_splits == SA_SPLITS_BY_LENGTH ? SA_SPLIT_BLOCKS : 0;
  a.batch = pd.batch;
  a.max_pages = pd.max_pages_per_seq;
  a.num_pages = pd.num_pages;
  // A one-byte cache stores K / k_scale: the scale joins the logit scale.
  a.scale_log2 = softmax_scale * k_scale * kLog2e;
  if (!isfinite(a.scale_log2)) return SA_ERR_INVALID_ARG;
  a.kv_fp8 = kv_fp8;
  a.v_scale = v_scale;
  a.sel_per_group = sel_per_group;
  // Many query tokens per sequence (a prefill chunk) re-read the same blocks:
  // keep them cacheable then; decode-like calls stream them.
  a.stream_kv = n_tok <= 64 * pd.batch;
  a.part_o = S > 1 ? part_o : nullptr;
  a.part_lse = S > 1 ? part_lse : nullptr;
  a.out = S == 1 ? static_cast<uint16_t*>(out) : nullptr;
  a.out_lse = S == 1 ? out_lse : nullptr;
  // split with counters: the last partition of each (token, group) merges in the same launch
  const bool fused = S > 1 && out != nullptr && merge_counters != nullptr;
  a.merge_counters = fused ? merge_counters : nullptr;
  a.merge_out = fused ? static_cast<uint16_t*>(out) : nullptr;
  a.merge_lse = fused ? out_lse : nullptr;
  if (sa::launch_attention(a, window_mode, stream) != hipSuccess) return SA_ERR_HIP;
  if (S > 1 && out != nullptr && !fused) {
    if (sa::launch_merge(part_o, part_lse, n_tok, S, sa::kHeads, sa::kHeadDim, static_cast<uint16_t*>(out),
                         out_lse, stream) != hipSuccess)
      return SA_ERR_HIP;
  }
  return SA_OK;
}

}  // namespace

extern "C" {

const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARG: return "SA_ERR_INVALID_ARG";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
    case SA_STATUS_MAX_ENUM: break;
  }
  return "SA_ERR_UNKNOWN";
}

size_t sa_indexer_topk_workspace_size(int n_tok, int max_pages_per_seq, int topk) {
  (void)topk;
  if (n_tok <= 0 || max_pages_per_seq <= 0) return 0;
  return sa::indexer_workspace_layout(n_tok, max_pages_per_seq).total;
}

int sa_resolve_num_splits(int n_tok, int max_blocks_per_token, int num_splits) {
  if (num_splits > 0) return std::min(num_splits, SA_MAX_SPLITS);
  if (num_splits == SA_SPLITS_BY_LENGTH)   // the longest list's own count (the kernel gives each token its own)
    return std::max(1, std::min((std::max(1, max_blocks_per_token) + SA_SPLIT_BLOCKS - 1) / SA_SPLIT_BLOCKS,
                                SA_MAX_SPLITS));
  if (num_splits != SA_SPLITS_FILL_GPU) return 1;
  // Reach about one workgroup per CU while giving every wave of a workgroup at
  // least one 4-block chunk: a chunk costs about one memory round trip when
  // few workgroups run, so tiny grids want short partitions (a one-token
  // window call: 9.2 us at 2 partitions, 8.1 us at 4), while a split grid that
  // already fills the GPU measured slower than an unsplit one (partial-result
  // traffic and a merge launch).
  const int work = std::max(1, n_tok) * sa::kGroups;
  const int want = (256 + work - 1) / work;
  const int chunks = (std::max(1, max_blocks_per_token) + 3) / 4;
  const int cap = std::max(1, chunks / 4);
  return std::max(1, std::min(std::min(want, cap), SA_MAX_SPLITS));
}

static sa_status indexer_topk_impl(const void* q_idx, const void* k_idx_cache, bool key_fp8, sa_paged_desc pd,
                                   const int32_t* q_seq, const int32_t* q_pos, int n_tok, bool per_group,
                                   int topk, int32_t* sel_idx, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  if (n_tok < 0) return SA_ERR_INVALID_ARG;
  if (n_tok == 0) return SA_OK;
  if (per_group && n_tok > kMaxGroupedTokens) return SA_ERR_UNSUPPORTED;
  // one query row per token, or one per (token, KV group)
  const int n_rows = per_group ? n_tok * sa::kGroups : n_tok;
  if ((long long)n_rows * 512 >= kMaxGridThreads) return SA_ERR_UNSUPPORTED;   // one 512-thread select per row
  if (q_idx == nullptr || k_idx_cache == nullptr || sel_idx == nullptr || workspace == nullptr)
    return SA_ERR_INVALID_ARG;
  if (!aligned(q_idx, 16) || !aligned(k_idx_cache, 16) || !aligned(sel_idx, 4) || !aligned(workspace, 256))
    return SA_ERR_INVALID_ARG;
  sa_status st = check_desc(pd);
  if (st != SA_OK) return st;
  if ((st = check_tokens(q_seq, q_pos)) != SA_OK) return st;
  if (topk < 1 || topk > SA_MAX_TOPK) return SA_ERR_UNSUPPORTED;
  const sa::IndexerWorkspace w = sa::indexer_workspace_layout(n_rows, pd.max_pages_per_seq);
  if (ws_bytes < w.total) return SA_ERR_WORKSPACE;

  sa::IndexerArgs a;
  a.q_idx = static_cast<const uint8_t*>(q_idx);
  a.k_idx_cache = static_cast<const uint8_t*>(k_idx_cache);
  a.page_table = pd.page_table;
  a.seq_lens = pd.seq_lens;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.n_tok = n_rows;
  a.q_shift = per_group ? 2 : 0;
  a.topk = topk;
  a.batch = pd.batch;
  a.max_pages = pd.max_pages_per_seq;
  a.num_pages = pd.num_pages;
  a.max_hist_blocks = pd.max_pages_per_seq * sa::kBlocksPerPage;
  // Query tokens of one sequence are scored in one pass over its keys; the
  // group size guesses how many consecutive tokens share a sequence (any guess
  // is correct, a good one reads each key once).
  a.group_size = std::max(1, std::min(4, n_rows / pd.batch));
  // Many query tokens per sequence (a prefill chunk): the score product is a
  // dense GEMM and runs on MFMA; histories must fit the finalize-only select.
  a.use_gemm = n_rows >= 64 * pd.batch && a.max_hist_blocks <= sa::kFuseLimit;
  // 16 .. 63 query rows per sequence (verify tokens x per-group queries): one
  // MFMA pass scores 16 rows against each key, again for finalize-only histories.
  a.use_mfma16 = !a.use_gemm && n_rows >= 16 * pd.batch && a.max_hist_blocks <= sa::kFuseLimit;
  const int ngroups = a.use_mfma16 ? (n_rows + 15) / 16 : (n_rows + a.group_size - 1) / a.group_size;
  // Few long workgroups: about two per CU (the score kernel's occupancy), so
  // each workgroup's fixed start-up cost is paid about once per CU. The
  // 16-row MFMA scorer keeps one key tile in flight per wave and fits three
  // waves per SIMD: it wants about four workgroups per CU.
  const long long target_wgs = a.use_mfma16 ? 1024 : 512;
  // the per-token scorer keeps its chunk of every row in LDS: at most kCandChunkMax blocks
  int chunk = a.use_mfma16 ? 4096 : sa::kCandChunkMax;
  while (chunk > 64 && (long long)ngroups * ((a.max_hist_blocks + chunk - 1) / chunk) < target_wgs) chunk >>= 1;
  a.chunk_blocks = chunk;
  // launch limit of the score grid (256 threads per workgroup)
  if ((long long)ngroups * ((a.max_hist_blocks + chunk - 1) / chunk) * 256 >= kMaxGridThreads) return SA_ERR_UNSUPPORTED;
  a.bitmap_words = a.max_hist_blocks <= sa::kFuseLimit ? (a.max_hist_blocks + 31) / 32 : 0;
  a.key_fp8 = key_fp8;
  // candidate lists of the per-token scorer: one per (row, chunk)
  a.cand_cap = std::min(chunk, sa::kChunkCap);
  a.cand_row_stride = (size_t)((a.max_hist_blocks + chunk - 1) / chunk) * (size_t)a.cand_cap;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.scores = reinterpret_cast<float*>(ws + w.scores_off);
  a.cand_meta = reinterpret_cast<uint2*>(ws + w.meta_off);
  a.cand = reinterpret_cast<uint2*>(ws + w.cand_off);
  a.sel_idx = sel_idx;
  if (sa::launch_indexer_topk(a, stream) != hipSuccess) return SA_ERR_HIP;
  return SA_OK;
}

sa_status sa_indexer_topk(const void* q_idx, const void* k_idx_cache, sa_paged_desc pd, const int32_t* q_seq,
                          const int32_t* q_pos, int n_tok, int topk, int32_t* sel_idx, void* workspace,
                          size_t ws_bytes, hipStream_t stream) {
  return indexer_topk_impl(q_idx, k_idx_cache, false, pd, q_seq, q_pos, n_tok, false, topk, sel_idx, workspace,
                           ws_bytes, stream);
}

size_t sa_indexer_topk_grouped_workspace_size(int n_tok, int max_pages_per_seq, int topk) {
  (void)topk;
  if (n_tok <= 0 || max_pages_per_seq <= 0 || n_tok > kMaxGroupedTokens) return 0;
  return sa::indexer_workspace_layout(n_tok * sa::kGroups, max_pages_per_seq).total;
}

sa_status sa_indexer_topk_grouped(const void* q_idx, const void* k_idx_cache, int key_format, sa_paged_desc pd,
                                  const int32_t* q_seq, const int32_t* q_pos, int n_tok, int topk,
                                  int32_t* sel_idx, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (key_format != SA_FORMAT_BF16 && key_format != SA_FORMAT_FP8_E4M3) return SA_ERR_UNSUPPORTED;
  return indexer_topk_impl(q_idx, k_idx_cache, key_format == SA_FORMAT_FP8_E4M3, pd, q_seq, q_pos, n_tok, true,
                           topk, sel_idx, workspace, ws_bytes, stream);
}

sa_status sa_indexer_topk_fp8(const void* q_idx, const void* k_idx_cache_fp8, sa_paged_desc pd,
                              const int32_t* q_seq, const int32_t* q_pos, int n_tok, int topk, int32_t* sel_idx,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  return indexer_topk_impl(q_idx, k_idx_cache_fp8, true, pd, q_seq, q_pos, n_tok, false, topk, sel_idx,
                           workspace, ws_bytes, stream);
}

sa_status sa_sparse_decode(const void* q, const void* k_cache, const void* v_cache, sa_paged_desc pd,
                           const int32_t* q_seq, const int32_t* q_pos, const int32_t* sel_idx, int n_tok,
                           int topk, float softmax_scale, int num_splits, float* part_o, float* part_lse,
                           uint32_t* merge_counters, void* out, float* out_lse, hipStream_t stream) {
  if (n_tok > 0) {
    if (sel_idx == nullptr || !aligned(sel_idx, 4)) return SA_ERR_INVALID_ARG;
    if (topk < 1 || topk > SA_MAX_TOPK) return SA_ERR_UNSUPPORTED;
  }
  return decode_common(q, k_cache, v_cache, pd, q_seq, q_pos, n_tok, softmax_scale, topk + 1, num_splits,
                       part_o, part_lse, merge_counters, out, out_lse, false, sel_idx, topk, 0, false, 1.f, 1.f, false, stream);
}

sa_status sa_sparse_decode_fp8kv(const void* q, const void* k_cache_fp8, const void* v_cache_fp8, float k_scale,
                                 float v_scale, sa_paged_desc pd, const int32_t* q_seq, const int32_t* q_pos,
                                 const int32_t* sel_idx, int n_tok, int topk, float softmax_scale, int num_splits,
                                 float* part_o, float* part_lse, uint32_t* merge_counters, void* out, float* out_lse, hipStream_t stream) {
  if (n_tok > 0) {
    if (sel_idx == nullptr || !aligned(sel_idx, 4)) return SA_ERR_INVALID_ARG;
    if (topk < 1 || topk > SA_MAX_TOPK) return SA_ERR_UNSUPPORTED;
  }
  return decode_common(q, k_cache_fp8, v_cache_fp8, pd, q_seq, q_pos, n_tok, softmax_scale, topk + 1, num_splits,
                       part_o, part_lse, merge_counters, out, out_lse, false, sel_idx, topk, 0, true, k_scale, v_scale, false,
                       stream);
}

sa_status sa_sparse_decode_grouped(const void* q, const void* k_cache, const void* v_cache, int kv_format,
                                   float k_scale, float v_scale, sa_paged_desc pd, const int32_t* q_seq,
                                   const int32_t* q_pos, const int32_t* sel_idx, int n_tok, int topk,
                                   float softmax_scale, int num_splits, float* part_o, float* part_lse, uint32_t* merge_counters, void* out,
                                   float* out_lse, hipStream_t stream) {
  if (kv_format != SA_FORMAT_BF16 && kv_format != SA_FORMAT_FP8_E4M3) return SA_ERR_UNSUPPORTED;
  const bool fp8 = kv_format == SA_FORMAT_FP8_E4M3;
  if (n_tok > 0) {
    if (sel_idx == nullptr || !aligned(sel_idx, 4)) return SA_ERR_INVALID_ARG;
    if (topk < 1 || topk > SA_MAX_TOPK) return SA_ERR_UNSUPPORTED;
    if (n_tok > kMaxGroupedTokens) return SA_ERR_UNSUPPORTED;
  }
  return decode_common(q, k_cache, v_cache, pd, q_seq, q_pos, n_tok, softmax_scale, topk + 1, num_splits,
                       part_o, part_lse, merge_counters, out, out_lse, false, sel_idx, topk, 0, fp8, fp8 ? k_scale : 1.f,
                       fp8 ? v_scale : 1.f, true, stream);
}

sa_status sa_swa_decode(const void* q, const void* k_cache, const void* v_cache, sa_paged_desc pd,
                        const int32_t* q_seq, const int32_t* q_pos, int n_tok, int window, float softmax_scale,
                        int num_splits, float* part_o, float* part_lse, uint32_t* merge_counters, void* out, float* out_lse,
                        hipStream_t stream) {
  if (n_tok > 0 && (window < 1 || window > SA_MAX_WINDOW)) return SA_ERR_UNSUPPORTED;
  return decode_common(q, k_cache, v_cache, pd, q_seq, q_pos, n_tok, softmax_scale, window / 8 + 2, num_splits,
                       part_o, part_lse, merge_counters, out, out_lse, true, nullptr, 0, window, false, 1.f, 1.f, false, stream);
}

sa_status sa_swa_decode_fp8kv(const void* q, const void* k_cache_fp8, const void* v_cache_fp8, float k_scale,
                              float v_scale, sa_paged_desc pd, const int32_t* q_seq, const int32_t* q_pos,
                              int n_tok, int window, float softmax_scale, int num_splits, float* part_o,
                              float* part_lse, uint32_t* merge_counters, void* out, float* out_lse, hipStream_t stream) {
  if (n_tok > 0 && (window < 1 || window > SA_MAX_WINDOW)) return SA_ERR_UNSUPPORTED;
  return decode_common(q, k_cache_fp8, v_cache_fp8, pd, q_seq, q_pos, n_tok, softmax_scale, window / 8 + 2,
                       num_splits, part_o, part_lse, merge_counters, out, out_lse, true, nullptr, 0, window, true, k_scale, v_scale,
                       false, stream);
}

sa_status sa_merge(const float* part_o, const float* part_lse, int n_tok, int num_splits, int num_heads,
                   int head_dim, void* out, float* out_lse, hipStream_t stream) {
  if (n_tok < 0) return SA_ERR_INVALID_ARG;
  if (n_tok == 0) return SA_OK;
  if (part_o == nullptr || part_lse == nullptr || out == nullptr) return SA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_heads < 1 || head_dim < 4) return SA_ERR_INVALID_ARG;
  if (num_splits > SA_MAX_SPLITS || num_heads > 1024 || head_dim > 1024 || head_dim % 4 != 0)
    return SA_ERR_UNSUPPORTED;
  if (!aligned(part_o, 16) || !aligned(part_lse, 4) || !aligned(out, 8)) return SA_ERR_INVALID_ARG;
  if (out_lse != nullptr && !aligned(out_lse, 4)) return SA_ERR_INVALID_ARG;
  if ((long long)n_tok * num_heads * 256 >= kMaxGridThreads) return SA_ERR_UNSUPPORTED;   // 256 threads per (token, head)
  if (sa::launch_merge(part_o, part_lse, n_tok, num_splits, num_heads, head_dim, static_cast<uint16_t*>(out),
                       out_lse, stream) != hipSuccess)
    return SA_ERR_HIP;
  return SA_OK;
}

}  // extern "C"
