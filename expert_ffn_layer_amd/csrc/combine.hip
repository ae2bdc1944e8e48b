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
constexpr int KMAX = 16;

// One thread per 16-byte chunk of one output row: it loads the token's k slots and weights
// (shared with the row's other threads through the cache), issues the k row loads together,
// then adds them in ascending j.
template <int ACT>
__global__ void __launch_bounds__(CTHR) combine_kernel(const uint8_t* __restrict__ y_perm,
                                                       const int32_t* __restrict__ pair_slot,
                                                       const float* __restrict__ wts,
                                                       const uint8_t* __restrict__ y_sh,
                                                       uint8_t* __restrict__ y, int T, int H, int k, int P) {
  constexpr int EB = ACT == MOE_F32 ? 4 : 2;  // element bytes
  constexpr int V = 16 / EB;                  // elements per 16-byte chunk
  const int cpr = H / V;                      // chunks per row
  const long long id = (long long)blockIdx.x * CTHR + threadIdx.x;
  if (id >= (long long)T * cpr) return;
  const int t = (int)(id / cpr), c = (int)(id - (long long)t * cpr);
  int slot[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    slot[j] = j < k ? pair_slot[(size_t)t * k + j] : -1;
    w[j] = j < k ? wts[(size_t)t * k + j] : 0.0f;
  }
  u32x4 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool ok = (unsigned)slot[j] < (unsigned)P;
    v[j] = ok ? *(const u32x4*)(y_perm + ((size_t)slot[j] * H + (size_t)c * V) * EB) : u32x4{0u, 0u, 0u, 0u};
  }
  u32x4 vs = {0u, 0u, 0u, 0u};
  if (y_sh) vs = *(const u32x4*)(y_sh + ((size_t)t * H + (size_t)c * V) * EB);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if ((unsigned)slot[j] >= (unsigned)P) continue;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float x = (ACT == MOE_F32) ? __uint_as_float(v[j][i]) : ((i & 1) ? bf16hi(v[j][i >> 1]) : bf16lo(v[j][i >> 1]));
      acc[i] += w[j] * x;
    }
  }
  if (y_sh) {
#pragma unroll
    for (int i = 0; i < V; ++i)
      acc[i] += (ACT == MOE_F32) ? __uint_as_float(vs[i]) : ((i & 1) ? bf16hi(vs[i >> 1]) : bf16lo(vs[i >> 1]));
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

hipError_t launch_combine(int act, const void* y_perm, const int32_t* pair_slot, const float* w,
                          const void* y_shared, void* y, int T, int H, int k, hipStream_t st) {
  if (k > KMAX) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  const int V = act == MOE_F32 ? 4 : 8;
  const long long chunks = (long long)T * (H / V);
  const unsigned grid = (unsigned)((chunks + CTHR - 1) / CTHR);
  if (act == MOE_F32)
    combine_kernel<MOE_F32><<<grid, CTHR, 0, st>>>((const uint8_t*)y_perm, pair_slot, w, (const uint8_t*)y_shared,
                                                  (uint8_t*)y, T, H, k, T * k);
  else
    combine_kernel<MOE_BF16><<<grid, CTHR, 0, st>>>((const uint8_t*)y_perm, pair_slot, w, (const uint8_t*)y_shared,
                                                   (uint8_t*)y, T, H, k, T * k);
  return hipGetLastError();
}

}  // namespace moe
