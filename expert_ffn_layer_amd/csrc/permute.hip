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
// The row-block plan of the grouped GEMMs from each group's row count cnt[g] (LDS, g < G):
// cum_blocks[g] = the first table entry of group g, cum_blocks[G] = the number of blocks, and the
// table block_group[b] = (g << 16) | (b's place within its group), so a GEMM item finds its group
// and place with one load (no search). Blocks are rb rows. With thick > 0, a group of more than
// rb rows is cut into blocks of `thick` rows instead, and those blocks come first in the table:
// they are the longest items, so they start first. sa, sb, tmp: LDS scratch of G + 1 ints each.
__device__ void write_plan(const int32_t* cnt, int G, int rb, int thick, int32_t* __restrict__ cum_blocks,
                           int32_t* __restrict__ block_group, int32_t* sa, int32_t* sb, int32_t* tmp) {
  const int tid = threadIdx.x, nt = blockDim.x;
  int nthick, nthin;
  if (G <= nt) {
    // one group per thread: two shuffle scans
    const int n = tid < G ? cnt[tid] : 0;
    const bool tk = thick > 0 && n > rb;
    const int a = block_scan_one(tk ? (n + thick - 1) / thick : 0, tmp, &nthick);
    const int b = block_scan_one(tk ? 0 : (n + rb - 1) / rb, tmp, &nthin);
    if (tid < G) {
      sa[tid] = a;
      sb[tid] = b;
    }
    __syncthreads();
  } else {
    for (int g = tid; g < G; g += nt) {
      const int n = cnt[g];
      const bool tk = thick > 0 && n > rb;
      sa[g] = tk ? (n + thick - 1) / thick : 0;
      sb[g] = tk ? 0 : (n + rb - 1) / rb;
    }
    __syncthreads();
    nthick = block_exclusive_scan(sa, tmp, G);
    nthin = block_exclusive_scan(sb, tmp, G);
  }
  for (int g = tid; g < G; g += nt) {
    const int n = cnt[g];
    const bool tk = thick > 0 && n > rb;
    const int first = tk ? sa[g] : nthick + sb[g];
    const int nblk = tk ? (n + thick - 1) / thick : (n + rb - 1) / rb;
    cum_blocks[g] = first;
    for (int i = 0; i < nblk; ++i) block_group[first + i] = (g << 16) | i;
  }
  if (tid == 0) cum_blocks[G] = nthick + nthin;
}

// The plan of the gate/up product (with thick blocks when thick > 0) into cum_a / bg_a, and, when
// thick > 0, the plan of the down product (64-row blocks only: its items are short, and thick ones
// measured slower) into cum_b / bg_b.
// rows: the rows of all groups together (bounds every block count).
__device__ void write_plans(const int32_t* cnt, int G, int rows, int rb, int thick, int32_t* cum_a, int32_t* bg_a,
                            int32_t* cum_b, int32_t* bg_b, int32_t* sa, int32_t* sb, int32_t* tmp) {
  const int tid = threadIdx.x;
  if (G <= (int)blockDim.x && rows / rb + G < 1024) {
    // one group per thread, the three block counts (thick and thin blocks of the first table, thin
    // blocks of the second) packed 10 bits each into one word: one scan. No count, and so no prefix,
    // reaches 1024 (each is at most rows / rb + G).
    const int n = tid < G ? cnt[tid] : 0;
    const bool tk = thick > 0 && n > rb;
    const int ca = tk ? (n + thick - 1) / thick : 0, cb = tk ? 0 : (n + rb - 1) / rb, cc = (n + rb - 1) / rb;
    int tot;
    const int pre = block_scan_one(ca | (cb << 10) | (cc << 20), tmp, &tot);
    const int nthick = tot & 1023, nthin = (tot >> 10) & 1023, nall = (tot >> 20) & 1023;
    if (tid < G) {
      const int first = tk ? (pre & 1023) : nthick + ((pre >> 10) & 1023);
      cum_a[tid] = first;
      for (int i = 0; i < ca + cb; ++i) bg_a[first + i] = (tid << 16) | i;
      if (thick > 0) {
        const int fb = (pre >> 20) & 1023;
        cum_b[tid] = fb;
        for (int i = 0; i < cc; ++i) bg_b[fb + i] = (tid << 16) | i;
      }
    }
    if (tid == 0) {
      cum_a[G] = nthick + nthin;
      if (thick > 0) cum_b[G] = nall;
    }
    return;
  }
  write_plan(cnt, G, rb, thick, cum_a, bg_a, sa, sb, tmp);
  if (thick > 0) {
    __syncthreads();
    write_plan(cnt, G, rb, 0, cum_b, bg_b, sa, sb, tmp);
  }
}

__global__ void __launch_bounds__(1024) plan_kernel(const int32_t* __restrict__ off, int E, int P, int T,
                                                     int shared, int rb, int thick, int32_t* __restrict__ group_range,
                                                     int32_t* __restrict__ cum_blocks, int32_t* __restrict__ block_group,
                                                     int32_t* __restrict__ cum_blocks_b, int32_t* __restrict__ block_group_b,
                                                     uint32_t* __restrict__ zero, int zero_words) {
  __shared__ int32_t cnt[2048], sa[2048], sb[2048], tmp[2048];
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
    cnt[g] = b1 - b0;
  }
  __syncthreads();
  write_plans(cnt, G, P + (shared ? T : 0), rb, thick, cum_blocks, block_group, cum_blocks_b, block_group_b, sa, sb,
              tmp);
}

hipError_t launch_plan(const int32_t* expert_offsets, int E, int P, int T, int shared, int rb, int thick,
                       int32_t* group_range, int32_t* cum_blocks, int32_t* block_group, int32_t* cum_blocks_b,
                       int32_t* block_group_b, uint32_t* zero, int zero_words, hipStream_t st) {
  if (E + 1 > 2048 || (thick > 0 && (!cum_blocks_b || !block_group_b))) return hipErrorInvalidValue;
  plan_kernel<<<1, 1024, 0, st>>>(expert_offsets, E, P, T, shared, rb, thick, group_range, cum_blocks, block_group,
                                  cum_blocks_b, block_group_b, zero, zero ? zero_words : 0);
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
    const int32_t* __restrict__ idx, int P, int k, int E, int T, int shared, int rb, int thick,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_token, int32_t* __restrict__ pair_slot,
    int32_t* __restrict__ group_range, int32_t* __restrict__ cum_blocks, int32_t* __restrict__ block_group,
    int32_t* __restrict__ cum_blocks_b, int32_t* __restrict__ block_group_b) {
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
  // plan: row range and row-block count of each group (routed experts, then the shared one); the
  // per-wave counts are free now and serve as scratch
  const int G = E + (shared ? 1 : 0);
  __syncthreads();
  for (int g = tid; g < G; g += SMALL_THR) {
    const int b0 = g < E ? run[g] : P;
    const int b1 = g < E ? (g + 1 < E ? run[g + 1] : total) : P + T;
    group_range[2 * g] = b0;
    group_range[2 * g + 1] = b1;
    tmp[g] = b1 - b0;
  }
  __syncthreads();
  write_plans(tmp, G, P + (shared ? T : 0), rb, thick, cum_blocks, block_group, cum_blocks_b, block_group_b, wcnt,
              wcnt + 2048, wcnt + 4096);
}

bool permute_small_ok(int P, int E) { return P <= SMALL_P && E <= SMALL_E; }

hipError_t launch_permute_small(const int32_t* idx, int T, int k, int E, int shared, int rb, int thick, int32_t* offsets,
                                int32_t* slot_token, int32_t* pair_slot, int32_t* group_range, int32_t* cum_blocks,
                                int32_t* block_group, int32_t* cum_blocks_b, int32_t* block_group_b, hipStream_t st) {
  const int P = T * k;
  if (!permute_small_ok(P, E) || (group_range && thick > 0 && (!cum_blocks_b || !block_group_b)))
    return hipErrorInvalidValue;
  permute_small_kernel<<<1, SMALL_THR, 0, st>>>(idx, P, k, E, T, shared, rb, thick, offsets, slot_token, pair_slot,
                                                group_range, cum_blocks, block_group, cum_blocks_b, block_group_b);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Decode batches in one launch: the router's selection, the permutation and the plan.
// Workgroup b selects tokens TPW b .. TPW b + TPW - 1 (one wave each, wave_topk), then ranks its
// own pairs in pair order among its pairs of the same expert (the wave-ballot ranks above) and
// writes, per pair, its expert and that rank packed in one word, and its expert histogram. The
// last workgroup to finish -- a completion count in the workspace, cleared by the router-score
// kernel of the same call -- forms the offsets (per expert over the workgroups, then over the
// experts), places every pair at offsets[e] + its workgroup's base + its rank, and writes the
// plan. The map is the same stable counting sort as the other paths; only which workgroup
// finishes last depends on scheduling, not the result.
// ------------------------------------------------------------------------------------------
constexpr int FUSED_E = 512;
constexpr int FUSED_CELLS = 16384;  // workgroups x experts of the histogram the last workgroup holds

// Tokens (waves) per workgroup: 8 for up to 128 tokens (twice the workgroups share the reads of the
// scores), else 16 (fewer histograms for the last workgroup to add up). The last workgroup's
// threads hold one group each in the plan, so 8 needs E + 1 <= 512.
int fused_tpw(int T, int E) { return T <= 128 && E + 1 <= 512 ? 8 : 16; }

bool topk_permute_ok(int T, int k, int E) {
  return T >= 1 && (long long)T * k <= SMALL_P && E <= FUSED_E && k <= TOPK_MAX &&
         (long long)((T + fused_tpw(T, E) - 1) / fused_tpw(T, E)) * E <= FUSED_CELLS;
}

template <int PL, bool HASH, int TPW>
__global__ void __launch_bounds__(64 * TPW) topk_permute_kernel(
    const float* __restrict__ logits, int ldl, long long part_stride, int nparts, const float* __restrict__ bias,
    int T, int E, int k, const int32_t* __restrict__ token_ids, const int32_t* __restrict__ table, int vocab,
    int32_t* __restrict__ idx, float* __restrict__ wout, int32_t* __restrict__ packed, int32_t* __restrict__ hist,
    uint32_t* __restrict__ done, int shared, int rb, int thick, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_token, int32_t* __restrict__ pair_slot, int32_t* __restrict__ group_range,
    int32_t* __restrict__ cum_blocks, int32_t* __restrict__ block_group, int32_t* __restrict__ cum_blocks_b,
    int32_t* __restrict__ block_group_b) {
  constexpr int NT = 64 * TPW;                     // threads
  constexpr int PW = (TPW * TOPK_MAX + 63) / 64;   // waves that hold this workgroup's pairs
  constexpr int QPT = SMALL_P / NT;                // pairs per thread in the last workgroup, at most
  __shared__ int32_t kept[TPW * TOPK_MAX];  // this workgroup's experts, pair order
  __shared__ int32_t wcnt[PW * FUSED_E];    // per-wave counts of this workgroup's pairs
  __shared__ int32_t cell[FUSED_CELLS];     // last workgroup: base of (workgroup, expert)
  __shared__ int32_t soff[FUSED_E + 2];     // last workgroup: offsets
  __shared__ int32_t wsum[16];
  __shared__ int last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x, t0 = b * TPW;
  const int ntok = min(TPW, T - t0), np = ntok * k;
  const int P = T * k;

  // 1. selection: wave w routes token t0 + w, with as many split-K parts in flight as the
  // registers allow (256 per lane at 8 waves per workgroup, 128 at 16)
  constexpr int PB = (TPW == 8 ? 144 : 64) / PL < 32 ? (TPW == 8 ? 144 : 64) / PL : 32;
  if (wave < ntok)
    wave_topk<PL, HASH, PB>(logits, ldl, part_stride, nparts, bias, t0 + wave, E, k, token_ids, table, vocab, idx,
                            wout, kept + wave * k);
  for (int i = tid; i < PW * E; i += NT) wcnt[i] = 0;
  __syncthreads();

  // 2. ranks among this workgroup's pairs of the same expert, in pair order; the pair's expert and
  // rank packed as (e << 16) | rank (-1 for a pair without an expert); the workgroup's histogram
  int e = -1;
  if (tid < np) {
    e = kept[tid];
    if (e < 0 || e >= E) e = -1;
  }
  int r_in_wave = 0;
  if (wave < PW) {  // wave-uniform
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
  if (tid < np) {
    int r = r_in_wave;
    for (int w = 0; w < wave; ++w) r += e >= 0 ? wcnt[w * E + e] : 0;
    packed[(size_t)t0 * k + tid] = e >= 0 ? (e << 16) | r : -1;
  }
  for (int ee = tid; ee < E; ee += NT) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < PW; ++w) c += wcnt[w * E + ee];
    hist[(size_t)b * E + ee] = c;
  }

  // 3. completion count: after the barrier, one thread releases the workgroup's packed pairs and
  // histogram device-wide and counts; the workgroup that counts last acquires everyone's
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const bool l = atomicAdd(done, 1u) == gridDim.x - 1;
    if (l) __threadfence();
    last = l;
  }
  __syncthreads();
  if (!last) return;

  // 4. the pairs (loads issued first, held in registers), then the histogram into LDS
  const int nb = gridDim.x;
  int pq[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int q = tid + i * NT;
    pq[i] = q < P ? packed[q] : -1;
  }
  for (int i = tid; i < nb * E; i += NT) cell[i] = hist[i];
  __syncthreads();
  // offsets: per expert, exclusive prefix over the workgroups, then over the experts
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
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int q = tid + i * NT;
    if (q < P) {
      const int v = pq[i];
      if (v < 0) {
        pair_slot[q] = -1;
      } else {
        const int eq = v >> 16;
        const int slot = soff[eq] + cell[(q / k / TPW) * E + eq] + (v & 0xFFFF);
        pair_slot[q] = slot;
        slot_token[slot] = q / k;
      }
    }
  }

  // 6. plan: row range and row count of each group (routed experts, then the shared one); the
  // histogram cells are free once every pair is placed and serve as scratch
  const int G = E + (shared ? 1 : 0);
  __syncthreads();
  for (int g = tid; g < G; g += NT) {
    const int b0 = g < E ? soff[g] : P;
    const int b1 = g < E ? soff[g + 1] : P + T;
    group_range[2 * g] = b0;
    group_range[2 * g + 1] = b1;
    cell[g] = b1 - b0;
  }
  __syncthreads();
  write_plans(cell, G, P + (shared ? T : 0), rb, thick, cum_blocks, block_group, cum_blocks_b, block_group_b,
              cell + 2048, cell + 4096, cell + 6144);
}

hipError_t launch_topk_permute(const float* logits, int ldl, int nparts, const float* bias, int T, int E, int k,
                               const int32_t* hash_ids, const int32_t* hash_table, int vocab, int32_t* idx, float* w,
                               int32_t* ws_packed, int32_t* ws_hist, uint32_t* done, int shared, int rb, int thick,
                               int32_t* offsets, int32_t* slot_token, int32_t* pair_slot, int32_t* group_range,
                               int32_t* cum_blocks, int32_t* block_group, int32_t* cum_blocks_b, int32_t* block_group_b,
                               hipStream_t st) {
  if (!topk_permute_ok(T, k, E) || (thick > 0 && (!cum_blocks_b || !block_group_b))) return hipErrorInvalidValue;
  const long long ps = (long long)T * ldl;
  const int tpw = fused_tpw(T, E);
  const dim3 grid((unsigned)((T + tpw - 1) / tpw)), block(64 * tpw);
  const int pl = (E + 63) / 64;
#define MOE_TP(PL, HASH, TPW)                                                                                     \
  topk_permute_kernel<PL, HASH, TPW><<<grid, block, 0, st>>>(logits, ldl, ps, nparts, bias, T, E, k, hash_ids,   \
                                                             hash_table, vocab, idx, w, ws_packed, ws_hist, done, \
                                                             shared, rb, thick, offsets, slot_token, pair_slot,   \
                                                             group_range, cum_blocks, block_group, cum_blocks_b,  \
                                                             block_group_b)
#define MOE_TP_PL(TPW)                     \
  if (hash_ids) {                          \
    if (pl <= 2) MOE_TP(2, true, TPW);     \
    else if (pl <= 4) MOE_TP(4, true, TPW); \
    else MOE_TP(8, true, TPW);             \
  } else {                                 \
    if (pl <= 1) MOE_TP(1, false, TPW);    \
    else if (pl <= 2) MOE_TP(2, false, TPW); \
    else if (pl <= 4) MOE_TP(4, false, TPW); \
    else if (pl <= 6) MOE_TP(6, false, TPW); \
    else MOE_TP(8, false, TPW);            \
  }
  if (tpw == 8) {
    MOE_TP_PL(8)
  } else {
    MOE_TP_PL(16)
  }
#undef MOE_TP_PL
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
