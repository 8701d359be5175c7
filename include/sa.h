/*
 * sa.h -- C ABI of libsa.so: block-indexed sparse GQA decode for MI355X (gfx950).
 *
 * The operation is the sparse layer and the sliding-window layer of the hybrid
 * attention described in "Step 5 Preview: Day-0 Inference and RL Support with
 * SGLang and Miles" (SGLang blog), sections "Hybrid Attention" and "Kernels from
 * StepFun", with the shapes of the config table in the Step 5 Preview
 * open-weights blog (section "What the config says"):
 *   64 query heads, 4 KV groups (head h reads group h / 16), head dim 192 for K
 *   and V, one 256-dim index key per 8-token block, top 512 blocks, a 512-token
 *   window, and a bf16 cache paged in 64-token pages.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked "device" are HIP device pointers owned by the caller. The
 *   library never allocates, frees or synchronises; all work is enqueued on
 *   `stream` and the call returns before it runs.
 * - The return value reports host-side validation (null pointers, sizes,
 *   alignment, supported shapes, workspace size) and launch errors
 *   (SA_ERR_HIP). Nothing is enqueued when validation fails.
 * - Device-side data (page-table entries, positions, sequence ids, selected
 *   block ids) are not read by the host. A token whose sequence id is outside
 *   [0, batch) or whose position is outside [0, seq_len) gets no attended tokens:
 *   its selection row is all -1 and its output row is zero with lse = -inf. A
 *   page id outside [0, num_pages) or a selected block id outside
 *   [0, floor(p/8)) is skipped. No such value causes an out-of-bounds access.
 * - n_tok == 0 is a valid no-op. A token with no earlier complete block
 *   (p < 8) selects nothing and attends its own block only.
 * - Results are deterministic: the same inputs and arguments give bitwise
 *   identical outputs, and a token's outputs do not depend on the other tokens
 *   of the call unless num_splits is SA_SPLITS_FILL_GPU.
 * - Every call can be captured into a HIP graph: no call records a memset, an
 *   allocation or a synchronisation (what must start at zero is cleared by a
 *   kernel of the call itself).
 * - The library keeps no global state. Calls on different streams may run at
 *   the same time as long as they share no output buffer, partial-result
 *   buffer or indexer workspace.
 * - All arrays are dense and row-major; device pointers must be 16-byte aligned.
 *
 * Cache layouts (this library's storage format; the pages fix none):
 * - K cache  bf16 [num_pages][4 groups][8 blocks][24 dim-chunks][8 tokens][8 dims]
 * - V cache  bf16 [num_pages][4 groups][8 blocks][192 dims][8 tokens]
 * - index-key cache bf16 [num_pages][8 blocks][256]
 * One-byte (OCP FP8 E4M3) forms, same page / block addressing:
 * - K cache  uint8 [num_pages][4 groups][8 blocks][3 dim-blocks][8 tokens][64 dims]
 *   (dim d of a token in dim-block d / 64, at d % 64)
 * - V cache  uint8 [num_pages][4 groups][8 blocks][192 dims][8 tokens]
 * - index-key cache uint8 [num_pages][8 blocks][256]
 *   Token position p of sequence b lives in physical page page_table[b][p / 64],
 *   block (p % 64) / 8 of that page, token p % 8 of that block.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_NUM_HEADS 64
#define SA_NUM_GROUPS 4
#define SA_HEAD_DIM 192
#define SA_INDEX_DIM 256
#define SA_BLOCK_TOKENS 8
#define SA_PAGE_TOKENS 64
#define SA_MAX_TOPK 512
#define SA_MAX_WINDOW 4096
#define SA_MAX_SPLITS 64

/* Partition requests for the num_splits argument of the decode calls. A
 * decode call cuts each (token, KV group)'s attended blocks into partitions
 * whose partial results are merged (SGLang blog, "Kernels from StepFun"):
 *   n > 0                n partitions for every token (at most SA_MAX_SPLITS);
 *   SA_SPLITS_BY_LENGTH  each token's count follows its own attended length
 *                        only: ceil(blocks / SA_SPLIT_BLOCKS) partitions, so a
 *                        token's results never depend on the other tokens of
 *                        the call (the GB300 bring-up, "MTP: the free win and
 *                        the not-quite-free one", records the hazard of verify
 *                        tokens taking a numerically different path);
 *   SA_SPLITS_FILL_GPU   the count follows the size of the call so that the
 *                        grid fills the GPU: fastest, but a token's bits may
 *                        change with the batch it is part of. */
#define SA_SPLITS_BY_LENGTH 0
#define SA_SPLITS_FILL_GPU (-1)
#define SA_SPLIT_BLOCKS 128

/* Storage formats of a cache (index keys or K/V) for the entry points that take one. */
#define SA_FORMAT_BF16 0
#define SA_FORMAT_FP8_E4M3 1

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, misalignment */
  SA_ERR_UNSUPPORTED = 2,   /* a shape or constant outside what the kernels support */
  SA_ERR_WORKSPACE = 3,     /* workspace smaller than the *_workspace_size() answer */
  SA_ERR_HIP = 4,           /* a HIP launch error */
  SA_STATUS_MAX_ENUM = 0x7FFFFFFF   /* not a status: keeps every int code a valid value of the type */
} sa_status;

/* One paged cache, shared by all calls of a layer.
 * page_table: device int32 [batch][max_pages_per_seq], physical page ids.
 * seq_lens:   device int32 [batch], tokens in the cache including the query tokens.
 * A sequence's query tokens are its last positions (an MTP verify token at
 * p + j sees the draft tokens p .. p + j - 1). */
typedef struct {
  const int32_t* page_table;
  const int32_t* seq_lens;
  int batch;
  int max_pages_per_seq;
  int num_pages;
} sa_paged_desc;

/* Human-readable name of a status code (static storage). */
const char* sa_status_string(sa_status s);

/* Bytes of device workspace sa_indexer_topk needs for these sizes. */
size_t sa_indexer_topk_workspace_size(int n_tok, int max_pages_per_seq, int topk);

/*
 * Indexer score + top-k block select.
 * (SGLang blog, "Hybrid Attention": score 8-token block summaries and keep up to
 *  512 historical blocks; "Kernels from StepFun": the indexer scores each query
 *  against compressed history in the paged cache.)
 *
 * For query token t at position p = q_pos[t] of sequence b = q_seq[t], with
 * cb = p / 8, every historical block beta < cb is scored as the fp32 dot product
 * s = sum_d q_idx[t][d] * k_idx_cache[page_table[b][beta / 8]][beta % 8][d]. The
 * min(topk, cb) blocks with the largest s are kept; ties go to the lower block
 * id. The current block is not a candidate (the attention adds it).
 *
 * q_idx        device bf16 [n_tok][256]
 * k_idx_cache  device bf16 [num_pages][8][256]
 * q_seq, q_pos device int32 [n_tok]
 * topk         1 .. 512
 * sel_idx      device int32 [n_tok][topk], out: ascending block ids, -1 padded
 * workspace    device scratch of at least sa_indexer_topk_workspace_size() bytes,
 *              256-byte aligned; its contents on entry do not matter.
 * Exact for index inputs whose partial sums are exact in fp32 (for example
 * small integers); otherwise scores carry fp32 rounding.
 */
sa_status sa_indexer_topk(const void* q_idx, const void* k_idx_cache, sa_paged_desc pd,
                          const int32_t* q_seq, const int32_t* q_pos, int n_tok, int topk,
                          int32_t* sel_idx, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * The same selection with one-byte index keys. (Open-weights blog, "What
 * sparse attention does and doesn't save": index keys at one or two bytes per
 * value; one byte halves the scan that dominates at long context.)
 *
 * k_idx_cache_fp8  device uint8 [num_pages][8][256], OCP FP8 E4M3 codes (sign,
 *                  4 exponent bits with bias 7, 3 mantissa bits; no infinities;
 *                  S.1111.111 is NaN). Keys are widened exactly to bf16 and
 *                  scored like sa_indexer_topk; q_idx stays bf16. Every other
 *                  argument, the workspace size and the result are as for
 *                  sa_indexer_topk. Integers -4..4 are exact in E4M3, so such
 *                  keys give the same selection as their bf16 form.
 */
sa_status sa_indexer_topk_fp8(const void* q_idx, const void* k_idx_cache_fp8, sa_paged_desc pd,
                              const int32_t* q_seq, const int32_t* q_pos, int n_tok, int topk,
                              int32_t* sel_idx, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Per-KV-group selection. (Open-weights blog, "What sparse attention does and
 * doesn't save": each KV group picks its own historical blocks.) The index key
 * stays one per block; each of a token's 4 KV groups brings its own index query
 * and keeps its own top-k blocks, scored and chosen exactly as in
 * sa_indexer_topk.
 *
 * q_idx        device bf16 [n_tok][4][256] (query of token t, group g at [t][g])
 * k_idx_cache  device [num_pages][8][256], bf16 (key_format SA_FORMAT_BF16) or
 *              OCP E4M3 codes (SA_FORMAT_FP8_E4M3, as for sa_indexer_topk_fp8)
 * sel_idx      device int32 [n_tok][4][topk], out: per (token, group) ascending
 *              block ids, -1 padded
 * workspace    at least sa_indexer_topk_grouped_workspace_size() bytes
 * Other arguments as for sa_indexer_topk. Another key_format gives
 * SA_ERR_UNSUPPORTED, as does n_tok >= 2^29.
 */
size_t sa_indexer_topk_grouped_workspace_size(int n_tok, int max_pages_per_seq, int topk);

sa_status sa_indexer_topk_grouped(const void* q_idx, const void* k_idx_cache, int key_format,
                                  sa_paged_desc pd, const int32_t* q_seq, const int32_t* q_pos,
                                  int n_tok, int topk, int32_t* sel_idx, void* workspace,
                                  size_t ws_bytes, hipStream_t stream);

/*
 * sa_indexer_topk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The workspace is a device array inside the library, SA_NOALLOC_SCRATCH_BYTES
 * long, one per GPU the library runs on (held until the process ends); the
 * call allocates nothing. Every other argument and the result are those of
 * sa_indexer_topk. Sizes whose workspace (sa_indexer_topk_workspace_size) is
 * larger than the array give SA_ERR_WORKSPACE (the 128K verify batch, 256 tokens
 * of 131,072-token histories, needs 16 MiB). All calls on one GPU share the
 * array: calls that overlap on one GPU (other streams, other threads) race.
 */
#define SA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

sa_status sa_indexer_topk_noalloc(const void* q_idx, const void* k_idx_cache, sa_paged_desc pd,
                                  const int32_t* q_seq, const int32_t* q_pos, int n_tok, int topk,
                                  int32_t* sel_idx, hipStream_t stream);

/* Partition extent S of a decode call's partial-result buffers for a request
 * (the S of part_o [n_tok][S][64][192]); max_blocks_per_token is the longest
 * attended list a token of the call can have (topk + 1 for the sparse layer,
 * window / 8 + 2 for the window layer).
 *   num_splits > 0       -> min(num_splits, SA_MAX_SPLITS)
 *   SA_SPLITS_BY_LENGTH  -> ceil(max_blocks_per_token / SA_SPLIT_BLOCKS); a token
 *                           with a shorter list uses its own, smaller count and
 *                           leaves its further partitions empty (lse = -inf)
 *   SA_SPLITS_FILL_GPU   -> partitions raised until the grid holds about one
 *                           workgroup per CU, keeping every wave of a workgroup at
 *                           least one 4-block chunk
 * Another negative value returns 1. */
int sa_resolve_num_splits(int n_tok, int max_blocks_per_token, int num_splits);

/*
 * Block-sparse GQA attention over the selected blocks and the current block.
 * (SGLang blog, "Hybrid Attention"; "Kernels from StepFun": decode attention
 *  over only the selected blocks, partitions merged afterwards.)
 *
 * Token t attends the tokens of its selected blocks (sel_idx[t][i] in
 * [0, p / 8)) and of its current block up to p. Head h uses KV group h / 16:
 * logit = softmax_scale * <q[t][h], K[j]>, exact softmax, O = sum w_j V[j].
 *
 * q            device bf16 [n_tok][64][192]
 * k_cache, v_cache  device bf16, layouts above
 * sel_idx      device int32 [n_tok][topk] (as written by sa_indexer_topk)
 * num_splits   partitions per (token, group): n > 0, SA_SPLITS_BY_LENGTH or
 *              SA_SPLITS_FILL_GPU (above); S = sa_resolve_num_splits(n_tok,
 *              topk + 1, num_splits); below SA_SPLITS_FILL_GPU is SA_ERR_INVALID_ARG
 * part_o, part_lse  device fp32 [n_tok][S][64][192], [n_tok][S][64]; needed when
 *              S > 1, ignored (may be NULL) when S == 1. A partition with
 *              lse = -inf attended nothing and its part_o may hold anything
 * merge_counters  device uint32 [n_tok][4] or NULL; used when S > 1 and out is
 *              non-NULL: the last partition of each (token, group) to finish
 *              merges the S partials in the same launch (the order and
 *              arithmetic of sa_merge, so the result is the same bit for bit).
 *              They must be zero before the first call that uses them, and
 *              every such call leaves them zero (allocate and zero once; a
 *              call with more tokens uses words no call has touched, still
 *              zero). Calls that run at the same time need their own. NULL:
 *              the merge is a second launch.
 * out          device bf16 [n_tok][64][192] (round to nearest even) or NULL;
 *              when S > 1 and out is non-NULL the merge is done too, when out
 *              is NULL only the partitions are written
 * out_lse      device fp32 [n_tok][64] natural-log lse, or NULL
 */
sa_status sa_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                           sa_paged_desc pd, const int32_t* q_seq, const int32_t* q_pos,
                           const int32_t* sel_idx, int n_tok, int topk, float softmax_scale,
                           int num_splits, float* part_o, float* part_lse, uint32_t* merge_counters, void* out,
                           float* out_lse, hipStream_t stream);

/*
 * Block-sparse GQA attention with one selection per KV group (as written by
 * sa_indexer_topk_grouped): the 16 heads of group g attend the tokens of the
 * blocks in sel_idx[t][g] and of the current block up to p.
 *
 * sel_idx      device int32 [n_tok][4][topk]
 * kv_format    SA_FORMAT_BF16 (k_scale and v_scale are ignored) or
 *              SA_FORMAT_FP8_E4M3 (one-byte caches and scales as for
 *              sa_sparse_decode_fp8kv); another value gives SA_ERR_UNSUPPORTED
 * Every other argument and every output is as for sa_sparse_decode.
 */
sa_status sa_sparse_decode_grouped(const void* q, const void* k_cache, const void* v_cache,
                                   int kv_format, float k_scale, float v_scale, sa_paged_desc pd,
                                   const int32_t* q_seq, const int32_t* q_pos,
                                   const int32_t* sel_idx, int n_tok, int topk, float softmax_scale,
                                   int num_splits, float* part_o, float* part_lse, uint32_t* merge_counters, void* out,
                                   float* out_lse, hipStream_t stream);

/*
 * Sliding-window GQA attention: token t at position p attends positions
 * max(0, p - window + 1) .. p. (SGLang blog, "Hybrid Attention": three of
 * every four layers read the latest 512 tokens.) Arguments as sa_sparse_decode;
 * window 1 .. SA_MAX_WINDOW; S = sa_resolve_num_splits(n_tok, window / 8 + 2,
 * num_splits).
 */
sa_status sa_swa_decode(const void* q, const void* k_cache, const void* v_cache,
                        sa_paged_desc pd, const int32_t* q_seq, const int32_t* q_pos,
                        int n_tok, int window, float softmax_scale, int num_splits,
                        float* part_o, float* part_lse, uint32_t* merge_counters, void* out, float* out_lse,
                        hipStream_t stream);

/*
 * sa_sparse_decode and sa_swa_decode over one-byte K/V caches. (Open-weights
 * blog, "Fitting it on a node": serving stacks may keep the KV of the
 * full-attention layers in FP8, at some loss of accuracy; one byte per value
 * halves what every decode step gathers. The window form is offered alongside.)
 *
 * k_cache_fp8, v_cache_fp8  device uint8, the one-byte layouts above, OCP FP8
 *              E4M3 codes (bias 7, no infinities, S.1111.111 is NaN).
 * k_scale, v_scale  per-cache dequantisation scales: the attended key is
 *              code * k_scale and the value code * v_scale; both must be finite
 *              and > 0 (else SA_ERR_INVALID_ARG).
 * Every other argument and every output is as for the bf16 entry point; codes
 * are widened exactly to bf16, so K and V enter the products unrounded.
 */
sa_status sa_sparse_decode_fp8kv(const void* q, const void* k_cache_fp8, const void* v_cache_fp8,
                                 float k_scale, float v_scale, sa_paged_desc pd,
                                 const int32_t* q_seq, const int32_t* q_pos, const int32_t* sel_idx,
                                 int n_tok, int topk, float softmax_scale, int num_splits,
                                 float* part_o, float* part_lse, uint32_t* merge_counters, void* out, float* out_lse,
                                 hipStream_t stream);

sa_status sa_swa_decode_fp8kv(const void* q, const void* k_cache_fp8, const void* v_cache_fp8,
                              float k_scale, float v_scale, sa_paged_desc pd,
                              const int32_t* q_seq, const int32_t* q_pos, int n_tok, int window,
                              float softmax_scale, int num_splits, float* part_o, float* part_lse,
                              uint32_t* merge_counters, void* out, float* out_lse, hipStream_t stream);

/*
 * Merge of per-partition results (SGLang blog, "Kernels from StepFun").
 * With M = max_s lse_s: O = sum_s e^(lse_s - M) O_s / sum_s e^(lse_s - M),
 * lse = M + ln sum_s e^(lse_s - M). Partitions with lse = -inf carry no weight
 * and their part_o is not used (it may hold anything, NaN included); if all are
 * empty the output is 0 and lse = -inf. The sum runs in a fixed order (four
 * consecutive quarters of the partitions, each in partition order, then the
 * quarters in order), so the result is deterministic.
 * part_o device fp32 [n_tok][num_splits][num_heads][head_dim]; part_lse
 * [n_tok][num_splits][num_heads]; out device bf16 [n_tok][num_heads][head_dim];
 * out_lse fp32 [n_tok][num_heads] or NULL. head_dim must be a multiple of 4
 * and at most 1024; num_heads at most 1024; num_splits 1 .. SA_MAX_SPLITS;
 * n_tok * num_heads * 256 below 2^32 (one 256-thread workgroup per (token,
 * head)), else SA_ERR_UNSUPPORTED.
 */
sa_status sa_merge(const float* part_o, const float* part_lse, int n_tok, int num_splits,
                   int num_heads, int head_dim, void* out, float* out_lse, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
