// Host validation of every C-ABI entry point, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/c_abi_build.py). Each call
// below is refused (or is a no-op) before any HIP call, so the program needs no
// GPU; the pointers are aligned stand-ins that are never dereferenced. The
// size arithmetic of the checks (grids near 2^32 threads, 2^29 grouped tokens,
// huge workspaces) runs under the sanitizers. Exits 0 when every status is the
// expected one.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sa.h"

namespace {

int g_failures = 0;
int g_checks = 0;

void expect(int got, int want, const char* what) {
  ++g_checks;
  if (got != want) {
    printf("FAIL: %s: got %d (%s), want %d (%s)\n", what, got, sa_status_string((sa_status)got), want,
           sa_status_string((sa_status)want));
    ++g_failures;
  }
}

void* const P = reinterpret_cast<void*>(0x10000);   // aligned stand-in, never dereferenced
void* at(uintptr_t off) { return reinterpret_cast<void*>(0x10000 + off); }
int32_t* const PI = static_cast<int32_t*>(P);
float* const PF = static_cast<float*>(P);

sa_paged_desc desc(int batch = 1, int max_pages = 16, int num_pages = 16, const int32_t* pt = PI) {
  return sa_paged_desc{pt, PI, batch, max_pages, num_pages};
}

}  // namespace

int main() {
  const sa_paged_desc d = desc();
  const size_t ws = sa_indexer_topk_workspace_size(4, 16, 512);
  expect(ws > 0, 1, "workspace size for 4 tokens");
  expect(sa_indexer_topk_workspace_size(0, 16, 512) == 0, 1, "workspace size for 0 tokens");

  // indexer
  expect(sa_indexer_topk(nullptr, nullptr, d, nullptr, nullptr, 0, 512, nullptr, nullptr, 0, nullptr), SA_OK,
         "indexer n_tok 0");
  expect(sa_indexer_topk(P, P, d, PI, PI, -1, 512, PI, P, ws, nullptr), SA_ERR_INVALID_ARG, "indexer n_tok -1");
  expect(sa_indexer_topk(nullptr, P, d, PI, PI, 4, 512, PI, P, ws, nullptr), SA_ERR_INVALID_ARG, "indexer null q");
  expect(sa_indexer_topk(at(8), P, d, PI, PI, 4, 512, PI, P, ws, nullptr), SA_ERR_INVALID_ARG, "indexer misaligned q");
  expect(sa_indexer_topk(P, P, d, PI, PI, 4, 512, PI, at(16), ws, nullptr), SA_ERR_INVALID_ARG,
         "indexer misaligned workspace");
  expect(sa_indexer_topk(P, P, d, PI, PI, 4, 0, PI, P, ws, nullptr), SA_ERR_UNSUPPORTED, "indexer topk 0");
  expect(sa_indexer_topk(P, P, d, PI, PI, 4, 513, PI, P, ws, nullptr), SA_ERR_UNSUPPORTED, "indexer topk 513");
  expect(sa_indexer_topk(P, P, d, PI, PI, 4, 512, PI, P, ws - 1, nullptr), SA_ERR_WORKSPACE, "indexer short ws");
  expect(sa_indexer_topk(P, P, desc(0), PI, PI, 4, 512, PI, P, ws, nullptr), SA_ERR_INVALID_ARG, "indexer batch 0");
  expect(sa_indexer_topk(P, P, desc(1, 16, 16, nullptr), PI, PI, 4, 512, PI, P, ws, nullptr), SA_ERR_INVALID_ARG,
         "indexer null page table");
  expect(sa_indexer_topk(P, P, desc(1, 16, 1 << 26), PI, PI, 4, 512, PI, P, ws, nullptr), SA_ERR_UNSUPPORTED,
         "indexer pool too large");
  expect(sa_indexer_topk(P, P, d, PI, PI, 1 << 23, 512, PI, P, (size_t)1 << 62, nullptr), SA_ERR_UNSUPPORTED,
         "indexer grid limit (tokens)");
  expect(sa_indexer_topk(P, P, desc(1, 1 << 20, 1 << 20), PI, PI, 1 << 16, 512, PI, P, (size_t)1 << 62, nullptr),
         SA_ERR_UNSUPPORTED, "indexer grid limit (8M-block histories)");
  expect(sa_indexer_topk_fp8(P, nullptr, d, PI, PI, 4, 512, PI, P, ws, nullptr), SA_ERR_INVALID_ARG,
         "fp8 indexer null keys");
  expect(sa_indexer_topk_fp8(P, P, d, PI, PI, 4, 512, PI, P, ws - 1, nullptr), SA_ERR_WORKSPACE,
         "fp8 indexer short ws");

  // the indexer with the library's own scratch (refused before any HIP call)
  expect(sa_indexer_topk_noalloc(nullptr, nullptr, d, nullptr, nullptr, 0, 512, nullptr, nullptr), SA_OK,
         "no-alloc indexer n_tok 0");
  expect(sa_indexer_topk_noalloc(nullptr, P, d, PI, PI, 4, 512, PI, nullptr), SA_ERR_INVALID_ARG,
         "no-alloc indexer null q");
  expect(sa_indexer_topk_noalloc(P, P, d, PI, PI, -3, 512, PI, nullptr), SA_ERR_INVALID_ARG,
         "no-alloc indexer n_tok -3");
  expect(sa_indexer_topk_noalloc(P, P, desc(64, 2048, 1 << 20), PI, PI, 1100, 512, PI, nullptr), SA_ERR_WORKSPACE,
         "no-alloc indexer: 1,100 tokens of 128K histories need more than the scratch array");
  expect(sa_indexer_topk_workspace_size(256, 2048, 512) <= SA_NOALLOC_SCRATCH_BYTES, 1,
         "the 128K verify batch fits the scratch array");

  // per-group indexer
  const size_t gws = sa_indexer_topk_grouped_workspace_size(4, 16, 512);
  expect(gws == sa_indexer_topk_workspace_size(16, 16, 512), 1, "grouped workspace covers 4 rows per token");
  expect(sa_indexer_topk_grouped_workspace_size(1 << 29, 16, 512) == 0, 1, "grouped workspace 2^29 tokens");
  expect(sa_indexer_topk_grouped(P, P, 2, d, PI, PI, 4, 512, PI, P, gws, nullptr), SA_ERR_UNSUPPORTED,
         "grouped key format 2");
  expect(sa_indexer_topk_grouped(P, P, 0, d, PI, PI, 4, 512, PI, P, ws, nullptr), SA_ERR_WORKSPACE,
         "grouped per-token workspace is short");
  expect(sa_indexer_topk_grouped(P, P, 0, d, PI, PI, 1 << 29, 512, PI, P, gws, nullptr), SA_ERR_UNSUPPORTED,
         "grouped 2^29 tokens");

  // sparse decode
  const float sc = 0.07f;
  expect(sa_sparse_decode(nullptr, nullptr, nullptr, d, PI, PI, nullptr, 0, 512, sc, 0, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr),
         SA_OK, "sparse n_tok 0");
  expect(sa_sparse_decode(P, P, P, d, PI, PI, nullptr, 4, 512, sc, 1, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_INVALID_ARG, "sparse null selection");
  expect(sa_sparse_decode(P, P, P, d, PI, PI, PI, 4, 600, sc, 1, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_UNSUPPORTED, "sparse topk 600");
  expect(sa_sparse_decode(P, P, P, d, PI, PI, PI, 4, 512, NAN, 1, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_INVALID_ARG, "sparse NaN scale");
  expect(sa_sparse_decode(P, P, P, d, PI, PI, PI, 4, 512, sc, 65, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_UNSUPPORTED, "sparse 65 splits");
  expect(sa_sparse_decode(P, P, P, d, PI, PI, PI, 4, 512, sc, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
         SA_ERR_INVALID_ARG, "sparse unsplit without out");
  expect(sa_sparse_decode(P, P, P, d, PI, PI, PI, 4, 512, sc, 4, nullptr, PF, nullptr, P, nullptr, nullptr),
         SA_ERR_INVALID_ARG, "sparse split without partials");
  expect(sa_sparse_decode(P, at(4), P, d, PI, PI, PI, 4, 512, sc, 1, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_INVALID_ARG, "sparse misaligned K");
  expect(sa_sparse_decode(P, P, P, d, PI, PI, PI, 1 << 22, 512, 0.1f, 1, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_UNSUPPORTED, "sparse grid limit");
  expect(sa_sparse_decode(P, P, P, d, PI, PI, PI, 1 << 18, 512, 0.1f, 2, PF, PF, nullptr, P, nullptr, nullptr),
         SA_ERR_UNSUPPORTED, "sparse merge grid limit");   // 2^18 tokens x 64 heads x 256 threads
  expect(sa_sparse_decode_fp8kv(P, P, P, 0.f, 1.f, d, PI, PI, PI, 4, 512, sc, 1, nullptr, nullptr, nullptr, P, nullptr,
                                nullptr),
         SA_ERR_INVALID_ARG, "fp8 KV zero scale");
  expect(sa_sparse_decode_fp8kv(P, P, P, 1e30f, 1.f, d, PI, PI, PI, 4, 512, 1e30f, 1, nullptr, nullptr, nullptr, P,
                                nullptr, nullptr),
         SA_ERR_INVALID_ARG, "fp8 KV logit scale overflow");
  expect(sa_sparse_decode_grouped(P, P, P, 3, 1.f, 1.f, d, PI, PI, PI, 4, 512, sc, 1, nullptr, nullptr, nullptr, P, nullptr,
                                  nullptr),
         SA_ERR_UNSUPPORTED, "grouped decode KV format 3");
  expect(sa_sparse_decode_grouped(P, P, P, 0, 1.f, 1.f, d, PI, PI, PI, 1 << 29, 512, sc, 1, nullptr, nullptr, nullptr, P,
                                  nullptr, nullptr),
         SA_ERR_UNSUPPORTED, "grouped decode 2^29 tokens");

  // window decode and merge
  expect(sa_swa_decode(P, P, P, d, PI, PI, 0, 512, 0.1f, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), SA_OK,
         "window n_tok 0");
  expect(sa_swa_decode(P, P, P, d, PI, PI, 2, 0, 0.1f, 1, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_UNSUPPORTED, "window 0");
  expect(sa_swa_decode(P, P, P, d, PI, PI, 2, 5000, 0.1f, 1, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_UNSUPPORTED, "window 5000");
  expect(sa_swa_decode_fp8kv(P, P, P, 1.f, INFINITY, d, PI, PI, 2, 512, 0.1f, 1, nullptr, nullptr, nullptr, P, nullptr,
                             nullptr),
         SA_ERR_INVALID_ARG, "fp8 window infinite scale");
  expect(sa_merge(nullptr, nullptr, 0, 1, 64, 192, nullptr, nullptr, nullptr), SA_OK, "merge n_tok 0");
  expect(sa_merge(PF, PF, 2, 0, 64, 192, P, nullptr, nullptr), SA_ERR_INVALID_ARG, "merge 0 splits");
  expect(sa_merge(PF, PF, 2, 65, 64, 192, P, nullptr, nullptr), SA_ERR_UNSUPPORTED, "merge 65 splits");
  expect(sa_merge(PF, PF, 2, 4, 64, 190, P, nullptr, nullptr), SA_ERR_UNSUPPORTED, "merge head dim 190");
  expect(sa_merge(PF, PF, 1 << 18, 2, 64, 192, P, nullptr, nullptr), SA_ERR_UNSUPPORTED, "merge grid limit");

  // split policy and status names
  expect(sa_resolve_num_splits(1, 513, SA_SPLITS_FILL_GPU), 32, "fill the GPU: one 8K token, 32 partitions");
  expect(sa_resolve_num_splits(256, 513, SA_SPLITS_FILL_GPU), 1, "fill the GPU: the 128K verify batch unsplit");
  expect(sa_resolve_num_splits(1, 513, SA_SPLITS_BY_LENGTH), 5, "by length: 513 blocks, 5 partitions");
  expect(sa_resolve_num_splits(256, 513, SA_SPLITS_BY_LENGTH), 5, "by length: the same for any batch");
  expect(sa_resolve_num_splits(64, 66, SA_SPLITS_BY_LENGTH), 1, "by length: a 512 window, unsplit");
  expect(sa_resolve_num_splits(1, 1 << 20, SA_SPLITS_BY_LENGTH), SA_MAX_SPLITS, "by length: clamped");
  expect(sa_resolve_num_splits(4, 513, 100), SA_MAX_SPLITS, "explicit count clamped");
  expect(sa_resolve_num_splits(4, 513, -7), 1, "another negative request");
  expect(sa_sparse_decode(P, P, P, d, PI, PI, PI, 4, 512, sc, -2, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_INVALID_ARG, "sparse num_splits -2");
  expect(sa_swa_decode(P, P, P, d, PI, PI, 2, 512, 0.1f, -2, nullptr, nullptr, nullptr, P, nullptr, nullptr),
         SA_ERR_INVALID_ARG, "window num_splits -2");
  expect(strcmp(sa_status_string((sa_status)99), "SA_ERR_UNKNOWN") == 0, 1, "unknown status name");

  printf("%d checks, %d failed\n%s\n", g_checks, g_failures,
         g_failures ? "c-abi validation FAILED" : "c-abi validation ok");
  return g_failures ? 1 : 0;
}
