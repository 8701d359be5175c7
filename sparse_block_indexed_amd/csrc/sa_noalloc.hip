// sa_indexer_topk_noalloc: the indexer entry point for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). The indexer's workspace (score rows, and
// for long histories the candidate-list headers and lists) lives in a
// file-scope device array of fixed size instead of a caller buffer; every
// other argument and the result are those of sa_indexer_topk, whose kernels
// it runs.
//
// The array exists once per GPU the library runs on and is held until the
// process ends. Its device address is looked up once per device, with that
// device current, and kept; host code uses that address, never the array's
// name (which in host code is only a stand-in for the symbol). Calls that
// overlap on one GPU share the array and therefore race.
#include <mutex>

#include "sa_internal.h"

namespace {

constexpr size_t kScratchBytes = SA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The scratch array's address on the current device (looked up on the first
// call made with that device current).
sa_status current_device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SA_OK;
}

}  // namespace

extern "C" sa_status sa_indexer_topk_noalloc(const void* q_idx, const void* k_idx_cache, sa_paged_desc pd,
                                             const int32_t* q_seq, const int32_t* q_pos, int n_tok, int topk,
                                             int32_t* sel_idx, hipStream_t stream) {
  if (n_tok < 0) return SA_ERR_INVALID_ARG;
  if (n_tok == 0) return SA_OK;
  if (q_idx == nullptr || k_idx_cache == nullptr || sel_idx == nullptr || q_seq == nullptr || q_pos == nullptr)
    return SA_ERR_INVALID_ARG;
  if (pd.max_pages_per_seq < 1) return SA_ERR_INVALID_ARG;
  // the workspace these sizes need must fit the array (checked before any HIP call)
  if (sa_indexer_topk_workspace_size(n_tok, pd.max_pages_per_seq, topk) > kScratchBytes) return SA_ERR_WORKSPACE;
  void* ws = nullptr;
  const sa_status st = current_device_scratch(&ws);
  if (st != SA_OK) return st;
  return sa_indexer_topk(q_idx, k_idx_cache, pd, q_seq, q_pos, n_tok, topk, sel_idx, ws, kScratchBytes, stream);
}
