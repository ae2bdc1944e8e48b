// Permutation of the (token, expert) pairs into expert-contiguous rows, and the row-block plan
// of the grouped GEMMs.
//
// Chapter 6 'Supernodes' section 6.2.6: the receiver regroups its input rows by expert, runs
// the matrix products, and restores token order by token number. Here that is a stable
// counting sort of the pairs q = t*k + j by expert (ties in ascending q, i.e. token order):
//   1. rank:    per block of PB pairs, each pair's rank among earlier pairs of the block with
//               the same expert (wave ballots, no atomics) and the block's expert histogram;
//   2. scan:    per expert, exclusive prefix over blocks, then over experts -> offsets;
//   3. scatter: slot = offsets[e] + prefix over earlier blocks + rank; pair_slot[q] = slot,
//               slot_token[slot] = q / k.
// Every result is a pure function of topk_idx: the map is the same on every run.
#include "common.h"
#include "kernels.h"
#include "wave_topk.h"

namespace moe {

constexpr int PB = 2048;   // pairs per block
constexpr int PTHR = 256;  // threads per block

int permute_blocks(int P) { return (P + PB - 1) / PB; }

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return lane ? (~0ull >> (64 - lane)) : 0ull; }

__global__ void __launch_bounds__(PTHR) perm_rank_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                         int32_t* __restrict__ rank,
                                                         int32_t* __restrict__ hist) {
  extern __shared__ int32_t sm[];  // run[E], wcnt[4][E]
  int32_t* run = sm;
  int32_t* wcnt = sm + E;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < 5 * E; e += PTHR) sm[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * PB;
  for (int c = 0; c < PB; c += PTHR) {
    const int q = base + c + tid;
    int e = -1;
    if (q < P) {
      e = idx[q];
      if (e < 0 || e >= E) e = -1;
    }
    // rank within the wave among lanes with the same expert, and the wave's counts
    uint64_t pending = __ballot(e >= 0);
    int r_in_wave = 0;
    while (pending) {
      const int leader = __ffsll((long long)pending) - 1;
      const int ek = __builtin_amdgcn_readlane(e, leader);  // leader is wave-uniform
      const uint64_t same = __ballot(e == ek) & pending;
      if (e == ek) r_in_wave = __popcll(same & lanemask_lt(lane));
      if (lane == leader) wcnt[wave * E + ek] = __popcll(same);
      pending &= ~same;
    }
    __syncthreads();
    if (e >= 0) {
      int r = run[e] + r_in_wave;
      for (int w = 0; w < wave; ++w) r += wcnt[w * E + e];
      rank[q] = r;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += PTHR) {
      run[ee] += wcnt[ee] + wcnt[E + ee] + wcnt[2 * E + ee] + wcnt[3 * E + ee];
      wcnt[ee] = wcnt[E + ee] = wcnt[2 * E + ee] = wcnt[3 * E + ee] = 0;
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += PTHR) hist[(size_t)blockIdx.x * E + e] = run[e];
}

// Exclusive scan of n <= 2 * blockDim.x ints held in lds[0..n) (in place); returns the total.
__device__ int block_exclusive_scan(int32_t* lds, int32_t* tmp, int n) {
  const int tid = threadIdx.x, nt = blockDim.x;
  // Hillis-Steele inclusive scan over 2 elements per thread, ping-ponging lds <-> tmp
  int32_t* src = lds;
  int32_t* dst = tmp;
  for (int off = 1; off < n; off <<= 1) {
    for (int i = tid; i < n; i += nt) dst[i] = src[i] + (i >= off ? src[i - off] : 0);
    __syncthreads();
    int32_t* t = src;
    src = dst;
    dst = t;
  }
  const int total = n ? src[n - 1] : 0;
  __syncthreads();
  for (int i = tid; i < n; i += nt) dst[i] = i ? src[i - 1] : 0;
  __syncthreads();
  if (dst != lds)
    for (int i = tid; i < n; i += nt) lds[i] = dst[i];
  __syncthreads();
  return total;
}

// Exclusive scan of one value per thread over the workgroup (up to 16 waves): each wave scans its
// 64 values with lane shuffles, the first wave scans the waves' totals; `wsum` is 16 ints of LDS.
// Returns the thread's exclusive prefix and sets *total to the sum of all values.
__device__ int block_scan_one(int v, int32_t* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < nw ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < nw) wsum[lane] = w;
  }
  __syncthreads();
  const int before = wave ? wsum[wave - 1] : 0;
  *total = wsum[nw - 1];
  __syncthreads();  // wsum free for the next scan
  return before + x - v;
}

__global__ void __launch_bounds__(1024) perm_scan_kernel(int32_t* __restrict__ hist, int NB, int E,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int32_t cnt[1024], tmp[1024];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int running = 0;
    for (int b = 0; b < NB; ++b) {
      const int c = hist[(size_t)b * E + e];
      hist[(size_t)b * E + e] = running;
      running += c;
    }
    cnt[e] = running;
  }
  __syncthreads();
  const int total = block_exclusive_scan(cnt, tmp, E);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    offsets[e] = cnt[e];
    for (int b = 0; b < NB; ++b) hist[(size_t)b * E + e] += cnt[e];
  }
  if (threadIdx.x == 0) offsets[E] = total;
}

__global__ void __launch_bounds__(PTHR) perm_scatter_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                            int k, const int32_t* __restrict__ rank,
                                                            const int32_t* __restrict__ base,
                                                            int32_t* __restrict__ slot_token,
                                                            int32_t* __restrict__ pair_slot) {
  const int q = blockIdx.x * PTHR + threadIdx.x;
  if (q >= P) return;
  const int e = idx[q];
  if (e < 0 || e >= E) {
    pair_slot[q] = -1;
    return;
  }
  const int slot = base[(size_t)(q / PB) * E + e] + rank[q];
  pair_slot[q] = slot;
  slot_token[slot] = q / k;
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* slot_token,
                          int32_t* pair_slot, int32_t* ws_rank, int32_t* ws_hist, hipStream_t st) {
  const int P = T * k;
  const int NB = permute_blocks(P);
  if (E > 1024) return hipErrorInvalidValue;
  perm_rank_kernel<<<NB, PTHR, 5 * E * sizeof(int32_t), st>>>(idx, P, E, ws_rank, ws_hist);
  perm_scan_kernel<<<1, 1024, 0, st>>>(ws_hist, NB, E, offsets);
  perm_scatter_kernel<<<(P + PTHR - 1) / PTHR, PTHR, 0, st>>>(idx, P, E, k, ws_rank, ws_hist, slot_token,
                                                              pair_slot);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Grouped-GEMM plan: the row range [begin, end) of each group (routed expert g from
// expert_offsets, then the shared expert as group E with rows [P, P+T)), and the prefix count
// of row blocks of rb rows per group. Offsets are clamped into [0, P] so malformed input
// cannot produce rows outside the buffers. It also clears `zero` (zero_words words): the zero
// activations the prefill GEMM feeds to the padding rows of a group's last tile.
// ------------------------------------------------------------------------------------------
// block_group[b] = (g << 16) | (b - cum_blocks[g]) for every row block b of group g: the GEMM
// kernels find an item's group and its place in it with one load (no search over cum_blocks).
__device__ __forceinline__ void write_block_group(const int32_t* cum, int G, int32_t* block_group, int tid,
                                                  int nthreads) {
  for (int g = tid; g < G; g += nthreads)
    for (int b = cum[g]; b < cum[g + 1]; ++b) block_group[b] = (g << 16) | (b - cum[g]);
}

__global__ void __launch_bounds__(1024) plan_kernel(const int32_t* __restrict__ off, int E, int P, int T,
                                                     int shared, int rb, int32_t* __restrict__ group_range,
                                                     int32_t* __restrict__ cum_blocks, int32_t* __restrict__ block_group,
                                                     uint32_t* __restrict__ zero, int zero_words) {
  __shared__ int32_t blk[2048], tmp[2048];
  for (int i = threadIdx.x; i < zero_words; i += blockDim.x) zero[i] = 0u;
  const int G = E + (shared ? 1 : 0);
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    int b0, b1;
    if (g < E) {
      b0 = min(max(off[g], 0), P);
      b1 = min(max(off[g + 1], b0), P);
    } else {
      b0 = P;
      b1 = P + T;
    }
    group_range[2 * g] = b0;
    group_range[2 * g + 1] = b1;
    blk[g] = (b1 - b0 + rb - 1) / rb;
  }
  __syncthreads();
  const int total = block_exclusive_scan(blk, tmp, G);
  for (int g = threadIdx.x; g < G; g += blockDim.x) cum_blocks[g] = blk[g];
  if (threadIdx.x == 0) {
    cum_blocks[G] = total;
    blk[G] = total;
  }
  __syncthreads();
  write_block_group(blk, G, block_group, threadIdx.x, blockDim.x);
}

hipError_t launch_plan(const int32_t* expert_offsets, int E, int P, int T, int shared, int rb,
                       int32_t* group_range, int32_t* cum_blocks, int32_t* block_group, uint32_t* zero, int zero_words,
                       hipStream_t st) {
  if (E + 1 > 2048) return hipErrorInvalidValue;
  plan_kernel<<<1, 1024, 0, st>>>(expert_offsets, E, P, T, shared, rb, group_range, cum_blocks, block_group, zero,
                                  zero ? zero_words : 0);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Decode-sized batches (P <= SMALL_P, E <= SMALL_E): the whole permutation, and optionally the
// grouped-GEMM plan, in one workgroup of 16 waves, so a decode step pays one launch instead of
// four. Same ranks as the multi-block path: per chunk of 1024 pairs, the rank among earlier
// pairs of the same expert from wave ballots and per-wave counts, in ascending pair order.
// ------------------------------------------------------------------------------------------
constexpr int SMALL_THR = 1024, SMALL_CHUNKS = 8, SMALL_E = 512;
constexpr int SMALL_P = SMALL_THR * SMALL_CHUNKS;

__global__ void __launch_bounds__(SMALL_THR) permute_small_kernel(
    const int32_t* __restrict__ idx, int P, int k, int E, int T, int shared, int rb,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_token, int32_t* __restrict__ pair_slot,
    int32_t* __restrict__ group_range, int32_t* __restrict__ cum_blocks, int32_t* __restrict__ block_group) {
  __shared__ int32_t wcnt[16 * SMALL_E];
  __shared__ int32_t run[2048], tmp[2048];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 16 * E; i += SMALL_THR) wcnt[i] = 0;
  for (int i = tid; i < E; i += SMALL_THR) run[i] = 0;
  __syncthreads();
  int rank[SMALL_CHUNKS], key[SMALL_CHUNKS];
#pragma unroll
  for (int c = 0; c < SMALL_CHUNKS; ++c) {
    rank[c] = 0;
    key[c] = -1;
    if (c * SMALL_THR < P) {  // uniform
      const int q = c * SMALL_THR + tid;
      int e = -1;
      if (q < P) {
        e = idx[q];
        if (e < 0 || e >= E) e = -1;
      }
      uint64_t pending = __ballot(e >= 0);
      int r_in_wave = 0;
      while (pending) {
        const int leader = __ffsll((long long)pending) - 1;
        const int ek = __builtin_amdgcn_readlane(e, leader);  // leader is wave-uniform
        const uint64_t same = __ballot(e == ek) & pending;
        if (e == ek) r_in_wave = __popcll(same & lanemask_lt(lane));
        if (lane == leader) wcnt[wave * E + ek] = __popcll(same);
        pending &= ~same;
      }
      __syncthreads();
      if (e >= 0) {
        int r = run[e] + r_in_wave;
        for (int w = 0; w < wave; ++w) r += wcnt[w * E + e];
        rank[c] = r;
      }
      key[c] = e;
      __syncthreads();
      for (int ee = tid; ee < E; ee += SMALL_THR) {
        int sum = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
          sum += wcnt[w * E + ee];
          wcnt[w * E + ee] = 0;
        }
        run[ee] += sum;
      }
      __syncthreads();
    }
  }
  const int total = block_exclusive_scan(run, tmp, E);  // run[e] = offsets[e]
  for (int e = tid; e < E; e += SMALL_THR) offsets[e] = run[e];
  if (tid == 0) offsets[E] = total;
#pragma unroll
  for (int c = 0; c < SMALL_CHUNKS; ++c) {
    const int q = c * SMALL_THR + tid;
    if (q < P) {
      if (key[c] >= 0) {
        const int slot = run[key[c]] + rank[c];
        pair_slot[q] = slot;
        slot_token[slot] = q / k;
      } else {
        pair_slot[q] = -1;
      }
    }
  }
  if (!group_range) return;
  // plan: row range and row-block count of each group (routed experts, then the shared one)
  const int G = E + (shared ? 1 : 0);
  __syncthreads();
  for (int g = tid; g < G; g += SMALL_THR) {
    const int b0 = g < E ? run[g] : P;
    const int b1 = g < E ? (g + 1 < E ? run[g + 1] : total) : P + T;
    group_range[2 * g] = b0;
    group_range[2 * g + 1] = b1;
    tmp[g] = (b1 - b0 + rb - 1) / rb;
  }
  __syncthreads();
  const int nblk = block_exclusive_scan(tmp, run, G);
  for (int g = tid; g < G; g += SMALL_THR) cum_blocks[g] = tmp[g];
  if (tid == 0) {
    cum_blocks[G] = nblk;
    tmp[G] = nblk;
  }
  __syncthreads();
  write_block_group(tmp, G, block_group, tid, SMALL_THR);
}

bool permute_small_ok(int P, int E) { return P <= SMALL_P && E <= SMALL_E; }

hipError_t launch_permute_small(const int32_t* idx, int T, int k, int E, int shared, int rb, int32_t* offsets,
                                int32_t* slot_token, int32_t* pair_slot, int32_t* group_range, int32_t* cum_blocks,
                                int32_t* block_group, hipStream_t st) {
  const int P = T * k;
  if (!permute_small_ok(P, E)) return hipErrorInvalidValue;
  permute_small_kernel<<<1, SMALL_THR, 0, st>>>(idx, P, k, E, T, shared, rb, offsets, slot_token, pair_slot,
                                                group_range, cum_blocks, block_group);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Decode batches in one launch: the router's selection, the permutation and the plan.
// Workgroup b selects tokens 16b .. 16b + 15 (one wave each, wave_topk), then ranks its own pairs
// in pair order among its pairs of the same expert (the wave-ballot ranks above) and writes the
// ranks and its expert histogram. The last workgroup to finish -- a completion count in the
// workspace, cleared by the router-score kernel of the same call -- forms the offsets (per expert
// over the workgroups, then over the experts), places every pair at offsets[e] + its workgroup's
// base + its rank, and writes the plan. The map is the same stable counting sort as the other
// paths; only the workgroup that finishes last depends on scheduling, not the result.
// ------------------------------------------------------------------------------------------
constexpr int FTHR = 1024, FTOK = 16;  // threads and tokens per workgroup
constexpr int FPAIRS = FTOK * TOPK_MAX;  // pairs per workgroup at most (4 waves)
constexpr int FUSED_E = 512;
constexpr int FUSED_CELLS = 16384;  // workgroups x experts of the histogram the last workgroup holds

bool topk_permute_ok(int T, int k, int E) {
  return T >= 1 && (long long)T * k <= SMALL_P && E <= FUSED_E && k <= TOPK_MAX &&
         (long long)((T + FTOK - 1) / FTOK) * E <= FUSED_CELLS;
}

template <int PL, bool HASH>
__global__ void __launch_bounds__(FTHR) topk_permute_kernel(
    const float* __restrict__ logits, int ldl, long long part_stride, int nparts, const float* __restrict__ bias,
    int T, int E, int k, const int32_t* __restrict__ token_ids, const int32_t* __restrict__ table, int vocab,
    int32_t* __restrict__ idx, float* __restrict__ wout, int32_t* __restrict__ rank, int32_t* __restrict__ hist,
    uint32_t* __restrict__ done, int shared, int rb, int32_t* __restrict__ offsets, int32_t* __restrict__ slot_token,
    int32_t* __restrict__ pair_slot, int32_t* __restrict__ group_range, int32_t* __restrict__ cum_blocks,
    int32_t* __restrict__ block_group) {
  __shared__ int32_t kept[FPAIRS];            // this workgroup's experts, pair order
  __shared__ int32_t wcnt[4 * FUSED_E];       // per-wave counts of this workgroup's pairs
  __shared__ int32_t cell[FUSED_CELLS];       // last workgroup: base of (workgroup, expert)
  __shared__ int32_t soff[FUSED_E + 2];       // last workgroup: offsets; then the plan's block prefix
  __shared__ int32_t wsum[16];
  __shared__ int last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x, t0 = b * FTOK;
  const int ntok = min(FTOK, T - t0), np = ntok * k;
  const int P = T * k;

  // 1. selection: wave w routes token t0 + w
  if (wave < ntok)
    wave_topk<PL, HASH>(logits, ldl, part_stride, nparts, bias, t0 + wave, E, k, token_ids, table, vocab, idx, wout,
                        kept + wave * k);
  for (int i = tid; i < 4 * E; i += FTHR) wcnt[i] = 0;
  __syncthreads();

  // 2. ranks among this workgroup's pairs of the same expert, in pair order, and its histogram
  int e = -1;
  if (tid < np) {
    e = kept[tid];
    if (e < 0 || e >= E) e = -1;
  }
  int r_in_wave = 0;
  if (wave < 4) {  // wave-uniform: the pairs sit in the first 4 waves
    uint64_t pending = __ballot(e >= 0);
    while (pending) {
      const int leader = __ffsll((long long)pending) - 1;
      const int ek = __builtin_amdgcn_readlane(e, leader);
      const uint64_t same = __ballot(e == ek) & pending;
      if (e == ek) r_in_wave = __popcll(same & lanemask_lt(lane));
      if (lane == leader) wcnt[wave * E + ek] = __popcll(same);
      pending &= ~same;
    }
  }
  __syncthreads();
  if (e >= 0) {
    int r = r_in_wave;
    for (int w = 0; w < wave; ++w) r += wcnt[w * E + e];
    rank[(size_t)t0 * k + tid] = r;
  }
  for (int ee = tid; ee < E; ee += FTHR)
    hist[(size_t)b * E + ee] = wcnt[ee] + wcnt[E + ee] + wcnt[2 * E + ee] + wcnt[3 * E + ee];

  // 3. completion count: this workgroup's selection, ranks and histogram are released device-wide
  // before its increment; the workgroup that counts last acquires everyone's
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(done, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();

  // 4. offsets: per expert, exclusive prefix over the workgroups, then over the experts
  const int nb = gridDim.x;
  for (int i = tid; i < nb * E; i += FTHR) cell[i] = hist[i];
  __syncthreads();
  int tot = 0;
  if (tid < E) {
    for (int bb = 0; bb < nb; ++bb) {
      const int c = cell[bb * E + tid];
      cell[bb * E + tid] = tot;
      tot += c;
    }
  }
  int grand;
  const int off = block_scan_one(tid < E ? tot : 0, wsum, &grand);
  if (tid < E) {
    offsets[tid] = off;
    soff[tid] = off;
  }
  if (tid == 0) {
    offsets[E] = grand;
    soff[E] = grand;
  }
  __syncthreads();

  // 5. every pair to its slot
  for (int q = tid; q < P; q += FTHR) {
    const int eq = idx[q];
    if (eq < 0 || eq >= E) {
      pair_slot[q] = -1;
      continue;
    }
    const int slot = soff[eq] + cell[(q / k / FTOK) * E + eq] + rank[q];
    pair_slot[q] = slot;
    slot_token[slot] = q / k;
  }

  // 6. plan: row range and row-block count of each group (routed experts, then the shared one)
  const int G = E + (shared ? 1 : 0);
  int b0 = 0, b1 = 0;
  if (tid < G) {
    b0 = tid < E ? soff[tid] : P;
    b1 = tid < E ? soff[tid + 1] : P + T;
    group_range[2 * tid] = b0;
    group_range[2 * tid + 1] = b1;
  }
  int nblk;
  const int cum = block_scan_one(tid < G ? (b1 - b0 + rb - 1) / rb : 0, wsum, &nblk);
  if (tid < G) {
    cum_blocks[tid] = cum;
    cell[tid] = cum;
  }
  if (tid == 0) {
    cum_blocks[G] = nblk;
    cell[G] = nblk;
  }
  __syncthreads();
  write_block_group(cell, G, block_group, tid, FTHR);
}

hipError_t launch_topk_permute(const float* logits, int ldl, int nparts, const float* bias, int T, int E, int k,
                               const int32_t* hash_ids, const int32_t* hash_table, int vocab, int32_t* idx, float* w,
                               int32_t* ws_rank, int32_t* ws_hist, uint32_t* done, int shared, int rb,
                               int32_t* offsets, int32_t* slot_token, int32_t* pair_slot, int32_t* group_range,
                               int32_t* cum_blocks, int32_t* block_group, hipStream_t st) {
  if (!topk_permute_ok(T, k, E)) return hipErrorInvalidValue;
  const long long ps = (long long)T * ldl;
  const dim3 grid((unsigned)((T + FTOK - 1) / FTOK)), block(FTHR);
  const int pl = (E + 63) / 64;
#define MOE_TP(PL, HASH)                                                                                         \
  topk_permute_kernel<PL, HASH><<<grid, block, 0, st>>>(logits, ldl, ps, nparts, bias, T, E, k, hash_ids,       \
                                                        hash_table, vocab, idx, w, ws_rank, ws_hist, done, shared, \
                                                        rb, offsets, slot_token, pair_slot, group_range,         \
                                                        cum_blocks, block_group)
  if (hash_ids) {
    if (pl <= 2) MOE_TP(2, true);
    else if (pl <= 4) MOE_TP(4, true);
    else MOE_TP(8, true);
  } else {
    if (pl <= 1) MOE_TP(1, false);
    else if (pl <= 2) MOE_TP(2, false);
    else if (pl <= 4) MOE_TP(4, false);
    else if (pl <= 6) MOE_TP(6, false);
    else MOE_TP(8, false);
  }
#undef MOE_TP
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<(n + 255) / 256, 256, 0, st>>>(p, v, n);
  return hipGetLastError();
}

}  // namespace moe
