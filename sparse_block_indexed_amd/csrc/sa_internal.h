// Internal declarations shared by the HIP translation units of libsa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sa.h"

namespace sa {

constexpr int kHeads = SA_NUM_HEADS;
constexpr int kGroups = SA_NUM_GROUPS;
constexpr int kHeadsPerGroup = kHeads / kGroups;
constexpr int kHeadDim = SA_HEAD_DIM;
constexpr int kIdxDim = SA_INDEX_DIM;
constexpr int kBlockTokens = SA_BLOCK_TOKENS;
constexpr int kPageTokens = SA_PAGE_TOKENS;
constexpr int kBlocksPerPage = kPageTokens / kBlockTokens;
constexpr int kUnitBytes = kBlockTokens * kHeadDim * 2;   // one (page, group, block) of K or V
constexpr int kKeyBytes = kIdxDim * 2;                     // one index key

// indexer workspace
constexpr int kHistBins = 2048;       // first radix digit: key bits 31..21
constexpr int kFuseLimit = 16384;     // longest history finalize holds in registers (longer: candidate lists)
constexpr int kCandChunkMax = 2048;   // longest block chunk of one per-token score workgroup
constexpr int kChunkCap = 512;        // candidates one (row, chunk) may list

struct AttnArgs {
  const uint8_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* sel_idx;   // sparse mode only
  int n_tok;
  int topk;                 // sparse mode
  int window;               // window mode
  int num_splits;           // partition extent S of the partial buffers
  int split_blocks;         // > 0: a token uses min(S, ceil(its blocks / split_blocks)) partitions
  int batch;
  int max_pages;
  int num_pages;
  float scale_log2;         // softmax_scale * log2(e)
  bool stream_kv;           // non-temporal K/V loads (blocks read about once per call)
  bool kv_fp8;              // one-byte (OCP E4M3) K/V caches
  bool sel_per_group;       // sel_idx is [n_tok][4][topk] (one set per KV group), else [n_tok][topk]
  float v_scale;            // V = code * v_scale for a one-byte cache (1 for bf16)
  float* part_o;            // used when num_splits > 1
  float* part_lse;
  uint16_t* out;            // used when num_splits == 1
  float* out_lse;
  // num_splits > 1 with the merge in the same launch: per (token, group)
  // arrival counters (zero on entry, left zero), and the merge's outputs
  uint32_t* merge_counters;
  uint16_t* merge_out;
  float* merge_lse;
};

struct IndexerArgs {
  const uint8_t* q_idx;
  const uint8_t* k_idx_cache;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int n_tok;                // query rows (tokens, or tokens x KV groups)
  int q_shift;              // query row r belongs to token r >> q_shift (0: one row per token, 2: per group)
  int topk;
  int batch;
  int max_pages;
  int num_pages;
  int max_hist_blocks;      // max_pages * 8: stride of the score rows
  int group_size;           // query tokens scored per pass over a sequence's keys
  int chunk_blocks;         // blocks per score workgroup
  int bitmap_words;         // LDS bitmap words per finalize workgroup (MFMA scorers)
  bool use_gemm;            // score with the MFMA GEMM kernel (long runs of tokens per sequence)
  bool use_mfma16;          // score 16 query rows per pass with MFMA (16 .. 63 rows per sequence)
  bool key_fp8;             // index keys are one-byte OCP E4M3 codes (else bf16)
  int32_t* sel_idx;
  float* scores;            // [n_tok][max_hist_blocks]
  // per-token scorer: each (row, chunk) lists its local candidates
  int cand_cap;             // list capacity per (row, chunk): min(chunk_blocks, kChunkCap)
  size_t cand_row_stride;   // list entries per row: chunks x cand_cap
  uint2* cand;              // [n_tok][chunks][cand_cap] (key, block), ascending block ids
  uint2* cand_meta;         // [n_tok][chunks] (count, edge key: every key >= edge is listed)
};

struct IndexerWorkspace {
  size_t scores_off, meta_off, cand_off, total;
};

// Candidate-list entries per row the workspace holds for a history of
// max_hist_blocks blocks, over every chunk length the host may pick.
size_t indexer_cand_row_bound(int max_hist_blocks);

IndexerWorkspace indexer_workspace_layout(int n_tok, int max_pages_per_seq);

hipError_t launch_attention(const AttnArgs& a, bool window_mode, hipStream_t stream);
hipError_t launch_merge(const float* part_o, const float* part_lse, int n_tok, int num_splits,
                        int num_heads, int head_dim, uint16_t* out, float* out_lse,
                        hipStream_t stream);
hipError_t launch_indexer_topk(const IndexerArgs& a, hipStream_t stream);

}  // namespace sa
