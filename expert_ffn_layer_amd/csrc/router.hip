// Router selection: the k largest scores per token and their renormalised softmax weights
// ('DeepSeek-V4-Pro on NVIDIA H200' step D4; Chapter 6 'Supernodes' section 6.2.6), or hash
// routing's table rows ('CANN DeepSeek-V4推理优化', MoE section). One wave per token, four tokens
// per workgroup; the selection of one token is wave_topk (wave_topk.h). The layer's decode batches
// run the same selection fused with the permutation (permute.hip).
#include "common.h"
#include "kernels.h"
#include "wave_topk.h"

namespace moe {

template <int PL, bool HASH>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int ldl, long long part_stride,
                                                   int nparts, const float* __restrict__ bias, int T, int E, int k,
                                                   const int32_t* __restrict__ token_ids,
                                                   const int32_t* __restrict__ table, int vocab,
                                                   int32_t* __restrict__ idx, float* __restrict__ wout) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_topk<PL, HASH>(logits, ldl, part_stride, nparts, bias, t, E, k, token_ids, table, vocab, idx, wout, nullptr);
}

template <bool HASH>
static void launch_topk_t(const float* logits, int ldl, long long ps, int nparts, const float* bias, int T, int E,
                          int k, const int32_t* ids, const int32_t* table, int vocab, int32_t* idx, float* w,
                          hipStream_t st) {
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  const int pl = (E + 63) / 64;
#define MOE_TOPK(PL) topk_kernel<PL, HASH><<<grid, block, 0, st>>>(logits, ldl, ps, nparts, bias, T, E, k, ids, table, vocab, idx, w)
  if (pl <= 1) MOE_TOPK(1);
  else if (pl <= 2) MOE_TOPK(2);
  else if (pl <= 4) MOE_TOPK(4);
  else if (pl <= 6) MOE_TOPK(6);
  else if (pl <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
}

hipError_t launch_topk(const float* logits, int ldl, int nparts, const float* bias, int T, int E, int k,
                       const int32_t* hash_ids, const int32_t* hash_table, int vocab, int32_t* idx, float* w,
                       hipStream_t st) {
  const long long ps = (long long)T * ldl;
  if (k > TOPK_MAX || E > 64 * PER_LANE_MAX) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  if (hash_ids) launch_topk_t<true>(logits, ldl, ps, nparts, bias, T, E, k, hash_ids, hash_table, vocab, idx, w, st);
  else launch_topk_t<false>(logits, ldl, ps, nparts, bias, T, E, k, nullptr, nullptr, 0, idx, w, st);
  return hipGetLastError();
}

}  // namespace moe
