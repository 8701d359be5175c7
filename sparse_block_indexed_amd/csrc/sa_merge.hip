// Merge of split-K partial attention results (SGLang blog "Step 5 Preview:
// Day-0 Inference and RL Support with SGLang and Miles", section "Kernels from
// StepFun": long histories are cut into partitions and the partial results
// merged).  With M = max_s lse_s:
//   O = sum_s e^(lse_s - M) O_s / sum_s e^(lse_s - M),  lse = M + ln sum_s e^(lse_s - M).
// Partitions in a fixed order, so the result is deterministic.

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

// One thread per (token, head, 4 consecutive dims).
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse, int n_tok, int S,
                                                    int H, int Dh, uint16_t* __restrict__ out,
                                                    float* __restrict__ out_lse) {
  const int q4 = Dh / 4;
  const long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (long long)n_tok * H * q4) return;
  const int d4 = (int)(item % q4);
  const int h = (int)((item / q4) % H);
  const int t = (int)(item / ((long long)q4 * H));
  const float* lrow = part_lse + (size_t)t * S * H + h;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lrow[(size_t)s * H]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float l = lrow[(size_t)s * H];
      if (l == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f((l - M) * kLog2e);
      const f32x4 o = *reinterpret_cast<const f32x4*>(part_o + (((size_t)t * S + s) * H + h) * Dh + 4 * d4);
      acc += o * w;
      L += w;
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  uint2 v;
  v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2*>(out + ((size_t)t * H + h) * Dh + 4 * d4) = v;
  if (out_lse != nullptr && d4 == 0)
    out_lse[(size_t)t * H + h] = L > 0.f ? M + __builtin_amdgcn_logf(L) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const float* part_o, const float* part_lse, int n_tok, int num_splits, int num_heads,
                        int head_dim, uint16_t* out, float* out_lse, hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  const long long items = (long long)n_tok * num_heads * (head_dim / 4);
  const unsigned blocks = (unsigned)((items + 255) / 256);
  merge_kernel<<<blocks, 256, 0, stream>>>(part_o, part_lse, n_tok, num_splits, num_heads, head_dim, out, out_lse);
  return hipGetLastError();
}

}  // namespace sa
