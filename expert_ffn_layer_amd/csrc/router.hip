// Router selection: the k largest scores per token and their renormalised softmax weights
// ('DeepSeek-V4-Pro on NVIDIA H200' step D4: score every routed expert, keep the top k;
// Chapter 6 'Supernodes' section 6.2.6: the routing weights a_e of the combine).
//
// One wave per token. Each lane holds scores e = lane, lane + 64, ... ; k rounds of a
// wave-wide arg-max (ties to the lower index) pick the experts; they are then listed in
// ascending expert index. The weights are exp(l - m) / sum over the chosen of exp(l - m) with
// m the largest score, which equals the softmax over all E renormalised over the chosen k.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int TOPK_MAX = 16;
constexpr int PER_LANE_MAX = 16;  // E <= 1024

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int PL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int ldl,
                                                   const float* __restrict__ bias, int T, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float NEG = -__builtin_huge_valf();
  float v[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int e = lane + 64 * j;
    v[j] = (e < E) ? logits[(size_t)t * ldl + e] + (bias ? bias[e] : 0.0f) : NEG;
  }
  int sel[TOPK_MAX];
  float sv[TOPK_MAX];
  for (int r = 0; r < k; ++r) {
    // lane-local best, then a butterfly arg-max across the wave
    float bv = NEG;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int e = lane + 64 * j;
      if (e < E && better(v[j], e, bv, bi)) { bv = v[j]; bi = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    sel[r] = bi;
    sv[r] = bv;
    if ((bi & 63) == lane) {
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (bi == lane + 64 * j) v[j] = NEG;
    }
  }
  if (lane != 0) return;
  // weights in selection order (sv[0] is the maximum), then list by ascending expert index
  float z = 0.0f, p[TOPK_MAX];
  for (int r = 0; r < k; ++r) {
    p[r] = __expf(sv[r] - sv[0]);
    z += p[r];
  }
  const float inv = 1.0f / z;
  for (int r = 1; r < k; ++r) {  // insertion sort by index, carrying the weight
    const int si = sel[r];
    const float pi = p[r];
    int q = r - 1;
    while (q >= 0 && sel[q] > si) {
      sel[q + 1] = sel[q];
      p[q + 1] = p[q];
      --q;
    }
    sel[q + 1] = si;
    p[q + 1] = pi;
  }
  for (int r = 0; r < k; ++r) {
    idx[(size_t)t * k + r] = sel[r];
    wout[(size_t)t * k + r] = p[r] * inv;
  }
}

hipError_t launch_topk(int /*act_is_f32*/, const float* logits, int ldl, const float* bias, int T, int E,
                       int k, int32_t* idx, float* w, hipStream_t st) {
  if (k > TOPK_MAX || E > 64 * PER_LANE_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  const int pl = (E + 63) / 64;
  if (pl <= 1) topk_kernel<1><<<grid, block, 0, st>>>(logits, ldl, bias, T, E, k, idx, w);
  else if (pl <= 2) topk_kernel<2><<<grid, block, 0, st>>>(logits, ldl, bias, T, E, k, idx, w);
  else if (pl <= 4) topk_kernel<4><<<grid, block, 0, st>>>(logits, ldl, bias, T, E, k, idx, w);
  else if (pl <= 6) topk_kernel<6><<<grid, block, 0, st>>>(logits, ldl, bias, T, E, k, idx, w);
  else if (pl <= 8) topk_kernel<8><<<grid, block, 0, st>>>(logits, ldl, bias, T, E, k, idx, w);
  else topk_kernel<16><<<grid, block, 0, st>>>(logits, ldl, bias, T, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
