// Merge of split-K partial attention results (SGLang blog "Step 5 Preview:
// Day-0 Inference and RL Support with SGLang and Miles", section "Kernels from
// StepFun": long histories are cut into partitions and the partial results
// merged).  With M = max_s lse_s:
//   O = sum_s e^(lse_s - M) O_s / sum_s e^(lse_s - M),  lse = M + ln sum_s e^(lse_s - M).
// Partitions are combined in a fixed order (four consecutive quarters, each in
// partition order, then the quarters in order), so the result is deterministic.

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

// Reductions over the 64 lanes as butterflies (DPP swaps inside rows of 16,
// then row swaps): every lane ends with the same bits.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));    // quad_perm 1,0,3,2
  v = fmaxf(v, dpp_move<0x4E>(v));    // quad_perm 2,3,0,1
  v = fmaxf(v, dpp_move<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_move<0x140>(v));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One workgroup of four waves per (token, head). The partitions are cut into
// four consecutive quarters of R = ceil(S / 4) (the last ones may be short or
// empty); wave q sums its quarter's weighted slices in partition order (lane d
// holds the 4-dim slice d, eight loads in flight), and the quarter sums are
// added in quarter order, ((A0 + A1) + A2) + A3, so that a split call waits for
// at most ceil(R / 8) rounds of loads. Every wave reduces M and the weight sum
// over all partitions itself (lane s holds partition s's lse), so no wave waits
// for another before its loads; its first eight slices are read before the
// lse values.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse, int n_tok, int S,
                                                    int H, int Dh, uint16_t* __restrict__ out,
                                                    float* __restrict__ out_lse) {
  __shared__ f32x4 s_acc[4][64];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  // (token, head); the host keeps n_tok * H * 256 below 2^32, so 32-bit division
  const unsigned item = blockIdx.x;
  const int h = (int)(item % (unsigned)H);
  const int t = (int)(item / (unsigned)H);
  const int q4 = Dh / 4;
  const int R = (S + 3) / 4;
  const int s_lo = min(S, q * R), s_hi = min(S, s_lo + R);
  const size_t sstride = (size_t)H * Dh;   // floats from one partition to the next
  const float* obase = part_o + ((size_t)t * S * H + h) * Dh;
  // slices of lanes past the head re-read its last slice and store nothing;
  // partitions past the quarter re-read the last one with weight 0
  auto load8 = [&](f32x4 (&v)[8], int s0, int d4) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const f32x4*>(obase + (size_t)min(s0 + u, S - 1) * sstride + 4 * d4);
  };
  f32x4 v[8];
  load8(v, s_lo, min(lane, q4 - 1));
  const float l = lane < S ? part_lse[((size_t)t * S + lane) * H + h] : -INFINITY;
  const float M = wave_max(l);
  const bool any = M != -INFINITY;
  const float w = (any && l != -INFINITY) ? __builtin_amdgcn_exp2f((l - M) * kLog2e) : 0.f;
  const float L = wave_sum(w);
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  for (int d4b = 0; d4b < q4; d4b += 64) {   // (uniform: every wave reaches the barriers)
    const int d4 = min(d4b + lane, q4 - 1);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = s_lo; s0 < s_hi; s0 += 8) {
      if (d4b > 0 || s0 > s_lo) load8(v, s0, d4);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(s0 + u, 63)));
        // a partition with no weight (empty, or past the quarter) adds nothing:
        // a select, not a product, so that whatever its slot holds (NaN
        // included) stays out
        const float wgt = s0 + u < s_hi ? wu : 0.f;
        acc = wgt != 0.f ? acc + v[u] * wgt : acc;
      }
    }
    s_acc[q][lane] = acc;
    __syncthreads();
    if (q == 0 && d4b + lane < q4) {
      f32x4 sum = s_acc[0][lane];
      sum = sum + s_acc[1][lane];
      sum = sum + s_acc[2][lane];
      sum = sum + s_acc[3][lane];
      uint2 o;
      o.x = pack_bf16x2(sum[0] * inv, sum[1] * inv);
      o.y = pack_bf16x2(sum[2] * inv, sum[3] * inv);
      *reinterpret_cast<uint2*>(out + ((size_t)t * H + h) * Dh + 4 * d4) = o;
    }
    __syncthreads();
  }
  if (out_lse != nullptr && threadIdx.x == 0)
    out_lse[(size_t)t * H + h] = L > 0.f ? M + __builtin_amdgcn_logf(L) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const float* part_o, const float* part_lse, int n_tok, int num_splits, int num_heads,
                        int head_dim, uint16_t* out, float* out_lse, hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  const long long items = (long long)n_tok * num_heads;   // one workgroup each
  const unsigned blocks = (unsigned)items;
  merge_kernel<<<blocks, 256, 0, stream>>>(part_o, part_lse, n_tok, num_splits, num_heads, head_dim, out, out_lse);
  return hipGetLastError();
}

}  // namespace sa
