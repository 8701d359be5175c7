// A host program that drives libsa.so through its C ABI alone (HIP runtime
// calls and the sa_* entry points; no Python, no PyTorch) and checks results
// that have closed forms:
//   - index keys whose score is the block id (or its negative) select the
//     highest (lowest) block ids; a token without history or with an invalid
//     sequence selects nothing;
//   - a V cache that is constant per KV group gives exactly that constant as
//     the output of every head of the group (window and sparse layers,
//     unsplit and split + merged);
//   - the merge of two partitions with weights 1/4 and 3/4;
//   - host validation: a short workspace, a zero window, status names.
// Prints one line per check; exits 0 when every check passes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "sa.h"

namespace {

int g_failures = 0;

void check(bool ok, const char* what) {
  printf("%s: %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++g_failures;
}

bool hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    printf("FAIL: %s: %s\n", what, hipGetErrorString(e));
    ++g_failures;
    return false;
  }
  return true;
}

// bf16 bits of a float that bf16 holds exactly (every value used here)
uint16_t bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

template <typename T>
T* to_device(const std::vector<T>& h) {
  void* d = nullptr;
  if (!hip_ok(hipMalloc(&d, h.size() * sizeof(T)), "hipMalloc")) return nullptr;
  hip_ok(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy H2D");
  return static_cast<T*>(d);
}

template <typename T>
std::vector<T> to_host(const T* d, size_t n) {
  std::vector<T> h(n);
  hip_ok(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost), "hipMemcpy D2H");
  return h;
}

constexpr int H = SA_NUM_HEADS, G = SA_NUM_GROUPS, D = SA_HEAD_DIM, DI = SA_INDEX_DIM;
constexpr int UNIT = 8 * D;   // bf16 elements of one (page, group, block) unit of K or V

}  // namespace

int main() {
  // Two sequences (300 and 1000 tokens) on a shuffled pool of 21 pages.
  const int batch = 2, max_pages = 16, num_pages = 21;
  const int lens[2] = {300, 1000};
  std::vector<int32_t> page_table(batch * max_pages, -1);
  {
    int next = 0;   // logical page n of the pool -> physical page (5n + 3) mod 21 (a permutation)
    for (int b = 0; b < batch; ++b)
      for (int i = 0; i < (lens[b] + 63) / 64; ++i) page_table[b * max_pages + i] = (5 * next++ + 3) % num_pages;
  }
  std::vector<int32_t> seq_lens(lens, lens + 2);

  // Index keys: block beta of a sequence has key (beta, 0, ..., 0).
  std::vector<uint16_t> kidx((size_t)num_pages * 8 * DI, 0);
  for (int b = 0; b < batch; ++b)
    for (int beta = 0; beta < (lens[b] + 7) / 8; ++beta) {
      const int page = page_table[b * max_pages + beta / 8];
      kidx[((size_t)page * 8 + beta % 8) * DI] = bf16((float)beta);
    }
  // Query tokens: (seq, pos, sign of the index query)
  const int n_tok = 5;
  const int32_t q_seq_h[n_tok] = {0, 1, 1, 1, 7};
  const int32_t q_pos_h[n_tok] = {299, 999, 998, 5, 10};
  const float sign[n_tok] = {1.f, 1.f, -1.f, 1.f, 1.f};
  std::vector<uint16_t> q_idx((size_t)n_tok * DI, 0);
  for (int t = 0; t < n_tok; ++t) q_idx[(size_t)t * DI] = bf16(sign[t]);

  // K: small deterministic values; V: the constant v_g in every element of group g.
  const float v_of_group[G] = {0.5f, 1.25f, -2.f, 3.5f};
  std::vector<uint16_t> kc((size_t)num_pages * G * 8 * UNIT), vc(kc.size());
  uint32_t lcg = 12345u;
  for (size_t i = 0; i < kc.size(); ++i) {
    lcg = lcg * 1664525u + 1013904223u;
    kc[i] = bf16((float)((int)(lcg >> 28) - 8) * 0.125f);   // -1 .. 0.875 in steps of 1/8
  }
  for (int page = 0; page < num_pages; ++page)
    for (int g = 0; g < G; ++g)
      for (int i = 0; i < 8 * UNIT; ++i) vc[((size_t)page * G + g) * 8 * UNIT + i] = bf16(v_of_group[g]);
  std::vector<uint16_t> q((size_t)n_tok * H * D);
  for (size_t i = 0; i < q.size(); ++i) {
    lcg = lcg * 1664525u + 1013904223u;
    q[i] = bf16((float)((int)(lcg >> 28) - 8) * 0.25f);
  }

  int32_t* d_pt = to_device(page_table);
  int32_t* d_sl = to_device(seq_lens);
  int32_t* d_qs = to_device(std::vector<int32_t>(q_seq_h, q_seq_h + n_tok));
  int32_t* d_qp = to_device(std::vector<int32_t>(q_pos_h, q_pos_h + n_tok));
  uint16_t* d_kidx = to_device(kidx);
  uint16_t* d_qidx = to_device(q_idx);
  uint16_t* d_k = to_device(kc);
  uint16_t* d_v = to_device(vc);
  uint16_t* d_q = to_device(q);
  if (g_failures) return 1;
  const sa_paged_desc pd = {d_pt, d_sl, batch, max_pages, num_pages};
  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;

  // ---- indexer ----------------------------------------------------------
  const int topk = 16;
  const size_t ws_bytes = sa_indexer_topk_workspace_size(n_tok, max_pages, topk);
  void* d_ws = nullptr;
  int32_t* d_sel = nullptr;
  hip_ok(hipMalloc(&d_ws, ws_bytes), "hipMalloc workspace");
  hip_ok(hipMalloc((void**)&d_sel, sizeof(int32_t) * n_tok * topk), "hipMalloc sel");
  check(sa_indexer_topk(d_qidx, d_kidx, pd, d_qs, d_qp, n_tok, topk, d_sel, d_ws, ws_bytes - 256, stream) ==
            SA_ERR_WORKSPACE,
        "a workspace one alignment unit short is refused");
  check(sa_indexer_topk(d_qidx, d_kidx, pd, d_qs, d_qp, n_tok, topk, d_sel, d_ws, ws_bytes, stream) == SA_OK,
        "sa_indexer_topk accepted");
  hip_ok(hipStreamSynchronize(stream), "sync indexer");
  const std::vector<int32_t> sel = to_host(d_sel, (size_t)n_tok * topk);
  {
    bool ok = true;
    for (int i = 0; i < topk; ++i) {
      ok &= sel[0 * topk + i] == 37 - topk + i;    // cb = 37: blocks 21 .. 36
      ok &= sel[1 * topk + i] == 124 - topk + i;   // cb = 124: blocks 108 .. 123
      ok &= sel[2 * topk + i] == i;                // negated query: blocks 0 .. 15
      ok &= sel[3 * topk + i] == -1;               // p = 5: no earlier block
      ok &= sel[4 * topk + i] == -1;               // sequence 7 does not exist
    }
    check(ok, "top-16 by block id, by negated block id, empty history, invalid sequence");
  }
  {
    // the entry point for callers that cannot allocate: the same ids, twice in a row
    int32_t* d_sel2 = nullptr;
    hip_ok(hipMalloc((void**)&d_sel2, sizeof(int32_t) * n_tok * topk), "hipMalloc sel2");
    bool ok = true;
    for (int rep = 0; rep < 2; ++rep) {
      ok &= sa_indexer_topk_noalloc(d_qidx, d_kidx, pd, d_qs, d_qp, n_tok, topk, d_sel2, stream) == SA_OK;
      hip_ok(hipStreamSynchronize(stream), "sync noalloc indexer");
      ok &= to_host(d_sel2, (size_t)n_tok * topk) == sel;
    }
    check(ok, "sa_indexer_topk_noalloc gives sa_indexer_topk's ids");
    hipFree(d_sel2);
  }

  // ---- attention with a V constant per group ---------------------------
  float *d_part_o = nullptr, *d_part_lse = nullptr, *d_lse = nullptr;
  uint16_t* d_out = nullptr;
  const int S = 3;
  hip_ok(hipMalloc((void**)&d_part_o, sizeof(float) * n_tok * S * H * D), "hipMalloc part_o");
  hip_ok(hipMalloc((void**)&d_part_lse, sizeof(float) * n_tok * S * H), "hipMalloc part_lse");
  hip_ok(hipMalloc((void**)&d_out, sizeof(uint16_t) * n_tok * H * D), "hipMalloc out");
  hip_ok(hipMalloc((void**)&d_lse, sizeof(float) * n_tok * H), "hipMalloc lse");
  // arrival counters of split calls that merge in the same launch: zeroed once
  uint32_t* d_ctr = nullptr;
  hip_ok(hipMalloc((void**)&d_ctr, sizeof(uint32_t) * n_tok * 4), "hipMalloc counters");
  hip_ok(hipMemset(d_ctr, 0, sizeof(uint32_t) * n_tok * 4), "hipMemset counters");
  const float scale = 1.f / sqrtf((float)D);
  // tokens 0 .. 3 are valid (token 4's sequence does not exist: zero output, lse = -inf)
  auto check_constant_v = [&](const char* what) {
    const std::vector<uint16_t> out = to_host(d_out, (size_t)n_tok * H * D);
    const std::vector<float> lse = to_host(d_lse, (size_t)n_tok * H);
    bool ok = true;
    for (int t = 0; t < n_tok; ++t)
      for (int h = 0; h < H; ++h) {
        const float want = t < 4 ? v_of_group[h / 16] : 0.f;
        for (int d = 0; d < D; ++d) ok &= from_bf16(out[((size_t)t * H + h) * D + d]) == want;
        ok &= t < 4 ? isfinite(lse[t * H + h]) : (isinf(lse[t * H + h]) && lse[t * H + h] < 0);
      }
    check(ok, what);
  };
  check(sa_swa_decode(d_q, d_k, d_v, pd, d_qs, d_qp, n_tok, 0, scale, 1, nullptr, nullptr, nullptr, d_out, d_lse,
                      stream) != SA_OK,
        "window 0 is refused");
  // unsplit; split + merge launch; split merged in the same launch (twice:
  // the counters must be back at zero after each call)
  const int pass_splits[4] = {1, S, S, S};
  for (int pass = 0; pass < 4; ++pass) {
    const int splits = pass_splits[pass];
    uint32_t* ctr = pass >= 2 ? d_ctr : nullptr;
    const char* how = pass >= 2 ? " merged in the same launch" : "";
    char what[160];
    hip_ok(hipMemset(d_out, 0xff, sizeof(uint16_t) * n_tok * H * D), "hipMemset out");
    check(sa_swa_decode(d_q, d_k, d_v, pd, d_qs, d_qp, n_tok, 64, scale, splits, d_part_o, d_part_lse, ctr, d_out,
                        d_lse, stream) == SA_OK,
          "sa_swa_decode accepted");
    hip_ok(hipStreamSynchronize(stream), "sync window");
    snprintf(what, sizeof(what), "window 64, %d partition(s)%s: every head returns its group's constant V", splits,
             how);
    check_constant_v(what);
    hip_ok(hipMemset(d_out, 0xff, sizeof(uint16_t) * n_tok * H * D), "hipMemset out");
    check(sa_sparse_decode(d_q, d_k, d_v, pd, d_qs, d_qp, d_sel, n_tok, topk, scale, splits, d_part_o,
                           d_part_lse, ctr, d_out, d_lse, stream) == SA_OK,
          "sa_sparse_decode accepted");
    hip_ok(hipStreamSynchronize(stream), "sync sparse");
    snprintf(what, sizeof(what), "sparse, %d partition(s)%s: every head returns its group's constant V", splits, how);
    check_constant_v(what);
  }
  {
    std::vector<uint32_t> ctr(n_tok * 4, 1);
    hip_ok(hipMemcpy(ctr.data(), d_ctr, sizeof(uint32_t) * n_tok * 4, hipMemcpyDeviceToHost), "copy counters");
    bool zero = true;
    for (uint32_t c : ctr) zero &= c == 0;
    check(zero, "split calls that merge in the same launch leave their counters at zero");
  }

  // ---- merge: weights 1/4 and 3/4 ---------------------------------------
  {
    const int mh = 2, md = 8;
    std::vector<float> po(2 * mh * md), pl(2 * mh);
    for (int i = 0; i < mh * md; ++i) {
      po[i] = 1.f;             // partition 0
      po[mh * md + i] = 3.f;   // partition 1
    }
    for (int h = 0; h < mh; ++h) {
      pl[h] = 0.f;
      pl[mh + h] = logf(3.f);
    }
    float* d_po = to_device(po);
    float* d_pl = to_device(pl);
    check(sa_merge(d_po, d_pl, 1, 2, mh, md, d_out, d_lse, stream) == SA_OK, "sa_merge accepted");
    hip_ok(hipStreamSynchronize(stream), "sync merge");
    const std::vector<uint16_t> out = to_host(d_out, (size_t)mh * md);
    const std::vector<float> lse = to_host(d_lse, (size_t)mh);
    bool ok = true;
    for (int i = 0; i < mh * md; ++i) ok &= from_bf16(out[i]) == 2.5f;   // (1 + 3 * 3) / 4
    for (int h = 0; h < mh; ++h) ok &= fabsf(lse[h] - logf(4.f)) < 1e-6f;
    check(ok, "merge of (1, lse 0) and (3, lse ln 3) gives 2.5 with lse ln 4");
    hipFree(d_po);
    hipFree(d_pl);
  }
  check(strcmp(sa_status_string(SA_ERR_WORKSPACE), "SA_ERR_WORKSPACE") == 0, "status names");

  hipFree(d_pt);
  hipFree(d_sl);
  hipFree(d_qs);
  hipFree(d_qp);
  hipFree(d_kidx);
  hipFree(d_qidx);
  hipFree(d_k);
  hipFree(d_v);
  hipFree(d_q);
  hipFree(d_ws);
  hipFree(d_sel);
  hipFree(d_part_o);
  hipFree(d_part_lse);
  hipFree(d_ctr);
  hipFree(d_out);
  hipFree(d_lse);
  hipStreamDestroy(stream);
  printf("%s\n", g_failures ? "c-abi closed forms FAILED" : "c-abi closed forms ok");
  return g_failures ? 1 : 0;
}
