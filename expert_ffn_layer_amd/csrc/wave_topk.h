// The router's selection for one token by one wave: the k largest scores and their
// renormalised softmax weights ('DeepSeek-V4-Pro on NVIDIA H200' step D4: score every routed
// expert, keep the top k; Chapter 6 'Supernodes' section 6.2.6: the routing weights a_e of the
// combine), or hash routing's fixed experts ('CANN DeepSeek-V4推理优化', MoE section).
//
// Each lane holds scores e = lane, lane + 64, ... (the sum of the split-K partial scores, in a
// fixed order). The k-th largest score is found by a bitwise search over order keys with wave
// ballot counts; the experts above it, and the lowest-indexed ones equal to it, are chosen (ties
// to the lower index) and listed in ascending expert index. The weights are exp(l - m) / sum over
// the chosen of exp(l - m) with m the largest score, which equals the softmax over all E
// renormalised over the chosen k. With hash routing the experts are row token_ids[t] of a
// [vocab][k] table, each score fetched from the lane that holds it, and the weights renormalise
// over that set in the same way; entries outside [0, E) (all k for an id outside [0, vocab)) are
// written as expert -1 with weight 0 after the valid ones, and equal experts keep table order.
#pragma once
#include "common.h"

namespace moe {

constexpr int TOPK_MAX = 16;
constexpr int PER_LANE_MAX = 16;  // E <= 1024

// The selection of token t by one wave (t wave-uniform): writes idx[t][0..k) and wout[t][0..k),
// and, when kept is given, the same experts to kept[0..k) (a copy in LDS for the caller). PB:
// split-K parts whose loads are in flight together (PB x PL registers).
template <int PL, bool HASH, int PB = 8>
__device__ __forceinline__ void wave_topk(const float* __restrict__ logits, int ldl, long long part_stride,
                                          int nparts, const float* __restrict__ bias, int t, int E, int k,
                                          const int32_t* __restrict__ token_ids, const int32_t* __restrict__ table,
                                          int vocab, int32_t* __restrict__ idx, float* __restrict__ wout,
                                          int32_t* kept) {
  const int lane = threadIdx.x & 63;
  const float NEG = -__builtin_huge_valf();
  // split-K partial scores, summed in ascending part order; the loads of PB parts of every
  // score are issued together, so the sum costs nparts / PB memory round trips, not nparts
  float v[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) v[j] = 0.0f;
  const float* lt = logits + (size_t)t * ldl;
  for (int p0 = 0; p0 < nparts; p0 += PB) {
    float part[PB][PL];
#pragma unroll
    for (int q = 0; q < PB; ++q) {
      const int p = min(p0 + q, nparts - 1);
#pragma unroll
      for (int j = 0; j < PL; ++j) {
        const int e = min(lane + 64 * j, E - 1);
        part[q][j] = lt[p * part_stride + e];
      }
    }
#pragma unroll
    for (int q = 0; q < PB; ++q)
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (p0 + q < nparts) v[j] += part[q][j];
  }
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? (bias ? v[j] + bias[e] : v[j]) : NEG;
  }
  int sel[TOPK_MAX];
  float sv[TOPK_MAX];
  if constexpr (HASH) {
    const int id = token_ids[t];
    const bool id_ok = id >= 0 && id < vocab;
    int key[TOPK_MAX];
    float m = NEG;
#pragma unroll
    for (int r = 0; r < TOPK_MAX; ++r) {
      sel[r] = -1;
      sv[r] = NEG;
      key[r] = 0x7fffffff;
      if (r < k) {
        int e = id_ok ? table[(size_t)id * k + r] : -1;  // the same address in every lane
        if (e < 0 || e >= E) e = -1;
        float sc = 0.0f;
#pragma unroll
        for (int j = 0; j < PL; ++j)
          if (e >= 0 && (e >> 6) == j) sc = v[j];
        sc = __shfl(sc, e >= 0 ? (e & 63) : 0, 64);  // the score of e lives in lane e % 64
        sel[r] = e;
        sv[r] = e >= 0 ? sc : NEG;
        key[r] = (e >= 0 ? e : E + r) * TOPK_MAX + r;  // valid ones ascending, then table order
        if (e >= 0) m = __builtin_fmaxf(m, sc);
      }
    }
    float z = 0.0f, mine_p = 0.0f;
    int mine_key = 0x7fffffff, mine = -1;
#pragma unroll
    for (int r = 0; r < TOPK_MAX; ++r) {
      if (r < k) {
        const float p = sel[r] >= 0 ? __expf(sv[r] - m) : 0.0f;
        z += p;
        if (r == lane) {
          mine = sel[r];
          mine_p = p;
          mine_key = key[r];
        }
      }
    }
    if (lane < k) {
      int rank = 0;
#pragma unroll
      for (int r = 0; r < TOPK_MAX; ++r)
        if (r < k && key[r] < mine_key) ++rank;
      idx[(size_t)t * k + rank] = mine;
      wout[(size_t)t * k + rank] = mine >= 0 ? mine_p / z : 0.0f;
      if (kept) kept[rank] = mine;
    }
    return;
  }
  // Selection without moving data between lanes. Each score gets an order key (a monotone map of
  // the float to uint32; padding experts get 0, below every real score). The k-th largest key K
  // is built bit by bit from the top: a candidate bit stays when at least k keys reach the
  // candidate, counted with wave ballots. The experts above K are chosen, and the lowest-indexed
  // experts equal to K fill the remaining places (ties to the lower index).
  uint32_t key[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const uint32_t u = __float_as_uint(v[j] + 0.0f);  // -0 -> +0: equal scores, equal keys
    key[j] = lane + 64 * j < E ? ((u >> 31) ? ~u : (u | 0x80000000u)) : 0u;
  }
  uint32_t K = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = K | (1u << b);
    int n = 0;
#pragma unroll
    for (int j = 0; j < PL; ++j) n += __popcll(__ballot(key[j] >= c));
    if (n >= k) K = c;
  }
  uint64_t pick[PL];
  int need = k;
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    pick[j] = __ballot(key[j] > K);
    need -= __popcll(pick[j]);
  }
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    uint64_t eq = __ballot(key[j] == K);
    while (need > 0 && eq) {  // wave-uniform
      const uint64_t low = eq & (~eq + 1);
      pick[j] |= low;
      eq ^= low;
      --need;
    }
  }
  // the largest chosen score, then the weights' sum, both over the chosen in ascending expert
  // index (each score read from the lane that holds it)
  float m = NEG;
#pragma unroll
  for (int j = 0; j < PL; ++j)
    for (uint64_t bits = pick[j]; bits; bits &= bits - 1)
      m = __builtin_fmaxf(m, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), __ffsll((long long)bits) - 1)));
  float z = 0.0f;
#pragma unroll
  for (int j = 0; j < PL; ++j)
    for (uint64_t bits = pick[j]; bits; bits &= bits - 1)
      z += __expf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), __ffsll((long long)bits) - 1)) - m);
  // each chosen expert's lane writes it at its rank among the chosen (ascending index)
  int base = 0;
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    if ((pick[j] >> lane) & 1ull) {
      const int rank = base + __popcll(pick[j] & (lane ? (~0ull >> (64 - lane)) : 0ull));
      idx[(size_t)t * k + rank] = lane + 64 * j;
      wout[(size_t)t * k + rank] = __expf(v[j] - m) / z;
      if (kept) kept[rank] = lane + 64 * j;
    }
    base += __popcll(pick[j]);
  }
}

}  // namespace moe
