// Combine: y[t] = sum_j w[t][j] * y_perm[pair_slot[t*k + j]] + y_shared[t].
//
// Chapter 6 'Supernodes' section 6.2.6 (token A: a1 y1 + a6 y6) and section 6.4.1 (the combine
// returns the results, restores token order and sums with the routing weights). Each output
// row gathers its k expert rows; the sum runs in ascending j in fp32, so the result does not
// depend on scheduling and needs no atomics. A pair whose pair_slot is outside [0, T*k)
// contributes nothing.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int CTHR = 256;

template <int ACT>
__global__ void __launch_bounds__(CTHR) combine_kernel(const uint8_t* __restrict__ y_perm,
                                                       const int32_t* __restrict__ pair_slot,
                                                       const float* __restrict__ wts,
                                                       const uint8_t* __restrict__ y_sh,
                                                       uint8_t* __restrict__ y, int H, int k, int P) {
  constexpr int EB = ACT == MOE_F32 ? 4 : 2;  // element bytes
  constexpr int V = 16 / EB;                  // elements per 16-byte chunk
  const int t = blockIdx.x;
  int slot[16];
  float w[16];
  for (int j = 0; j < k; ++j) {
    slot[j] = pair_slot[(size_t)t * k + j];
    w[j] = wts[(size_t)t * k + j];
  }
  for (int c = threadIdx.x; c < H / V; c += CTHR) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      if ((unsigned)slot[j] >= (unsigned)P) continue;
      const u32x4 v = *(const u32x4*)(y_perm + ((size_t)slot[j] * H + (size_t)c * V) * EB);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const float x = (ACT == MOE_F32) ? __uint_as_float(v[i]) : ((i & 1) ? bf16hi(v[i >> 1]) : bf16lo(v[i >> 1]));
        acc[i] += w[j] * x;
      }
    }
    if (y_sh) {
      const u32x4 v = *(const u32x4*)(y_sh + ((size_t)t * H + (size_t)c * V) * EB);
#pragma unroll
      for (int i = 0; i < V; ++i)
        acc[i] += (ACT == MOE_F32) ? __uint_as_float(v[i]) : ((i & 1) ? bf16hi(v[i >> 1]) : bf16lo(v[i >> 1]));
    }
    u32x4 o;
    if (ACT == MOE_F32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    }
    *(u32x4*)(y + ((size_t)t * H + (size_t)c * V) * EB) = o;
  }
}

hipError_t launch_combine(int act, const void* y_perm, const int32_t* pair_slot, const float* w,
                          const void* y_shared, void* y, int T, int H, int k, hipStream_t st) {
  if (k > 16) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  if (act == MOE_F32)
    combine_kernel<MOE_F32><<<T, CTHR, 0, st>>>((const uint8_t*)y_perm, pair_slot, w, (const uint8_t*)y_shared,
                                               (uint8_t*)y, H, k, T * k);
  else
    combine_kernel<MOE_BF16><<<T, CTHR, 0, st>>>((const uint8_t*)y_perm, pair_slot, w, (const uint8_t*)y_shared,
                                                (uint8_t*)y, H, k, T * k);
  return hipGetLastError();
}

}  // namespace moe
