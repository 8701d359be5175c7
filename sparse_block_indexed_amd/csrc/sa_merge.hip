// Merge of split-K partial attention results (SGLang blog "Step 5 Preview:
// Day-0 Inference and RL Support with SGLang and Miles", section "Kernels from
// StepFun": long histories are cut into partitions and the partial results
// merged).  With M = max_s lse_s:
//   O = sum_s e^(lse_s - M) O_s / sum_s e^(lse_s - M),  lse = M + ln sum_s e^(lse_s - M).
// Partitions are combined in a fixed order, so the result is deterministic.

#include "sa_internal.h"

namespace sa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// One wave per (token, head). Lane s < S holds partition s's lse and weight
// e^(lse_s - M); the wave reduces M and the weight sum, then every lane
// accumulates its 4-dim slices over the partitions in order 0..S-1 with eight
// loads in flight (the weight of partition s is broadcast from lane s).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse, int n_tok, int S,
                                                    int H, int Dh, uint16_t* __restrict__ out,
                                                    float* __restrict__ out_lse) {
  const int lane = threadIdx.x & 63;
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);   // (token, head)
  if (item >= (long long)n_tok * H) return;
  const int h = (int)(item % H);
  const int t = (int)(item / H);
  const float l = lane < S ? part_lse[((size_t)t * S + lane) * H + h] : -INFINITY;
  const float M = wave_max(l);
  const bool any = M != -INFINITY;
  const float w = (any && l != -INFINITY) ? __builtin_amdgcn_exp2f((l - M) * kLog2e) : 0.f;
  const float L = wave_sum(w);   // butterfly: every lane holds the same bits
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const int q4 = Dh / 4;
  for (int d4 = lane; d4 < q4; d4 += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sc = min(s0 + u, S - 1);   // past S: re-read the last partition, weight 0
        v[u] = *reinterpret_cast<const f32x4*>(part_o + (((size_t)t * S + sc) * H + h) * Dh + 4 * d4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(s0 + u, 63)));
        const float wgt = s0 + u < S ? wu : 0.f;
        acc += v[u] * wgt;
      }
    }
    uint2 o;
    o.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    o.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2*>(out + ((size_t)t * H + h) * Dh + 4 * d4) = o;
  }
  if (out_lse != nullptr && lane == 0)
    out_lse[(size_t)t * H + h] = L > 0.f ? M + __builtin_amdgcn_logf(L) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const float* part_o, const float* part_lse, int n_tok, int num_splits, int num_heads,
                        int head_dim, uint16_t* out, float* out_lse, hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  const long long items = (long long)n_tok * num_heads;   // one wave each, four per workgroup
  const unsigned blocks = (unsigned)((items + 3) / 4);
  merge_kernel<<<blocks, 256, 0, stream>>>(part_o, part_lse, n_tok, num_splits, num_heads, head_dim, out, out_lse);
  return hipGetLastError();
}

}  // namespace sa
