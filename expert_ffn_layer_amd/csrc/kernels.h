// Declarations shared by the kernels and the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// EPI_SWIGLU_Q8: SiLU(g) * u rounded to bf16, then written as MXFP8 (codes to out, one e8m0
// exponent per 32 columns to out_scale) for a W4A8 down product
enum { EPI_SWIGLU = 0, EPI_PLAIN = 1, EPI_F32 = 2, EPI_SWIGLU_Q8 = 3 };

// Arguments of a grouped GEMM over a "row space": group g owns rows
// [group_range[2g], group_range[2g+1]). Row r reads activation row
//   gather ? (r < P ? gather[r] : r - P) : r
// (gathered token rows for the routed experts, then the shared expert's rows P.. in token
// order), clamped to [0, act_rows), and writes output row r, or row r - P of out_s when out_s
// is set and r >= P. group_range == nullptr means one group of M rows.
struct GroupedArgs {
  const int32_t* group_range;
  const int32_t* cum_blocks;  // prefix count of row blocks per group (block = RB rows)
  const int32_t* block_group; // per row block b: (group << 16) | (b - cum_blocks[group]), or null
  int G;
  int shared_group;  // group index of the shared expert, or -1
  int P;
  int M;
  const int32_t* gather;
  const void* act;
  int lda;
  int act_rows;
  // weights: routed base + g * mat_bytes, or the shared pointers for the shared group
  const uint8_t* wa_r;
  const uint8_t* wa_s;
  const uint8_t* wb_r;  // second matrix (SwiGLU "up"), else null
  const uint8_t* wb_s;
  const uint8_t* sa_r;
  const uint8_t* sa_s;
  const uint8_t* sb_r;
  const uint8_t* sb_s;
  long long mat_bytes;
  long long scale_bytes;
  int K, N, NTW;
  void* out;
  int ldo;
  void* out_s;
  int ldo_s;
  int ksplit;  // > 1: fp32 output only; workgroup y sums K part y into out + y * M * ldo
  const void* zero_row;  // prefill: K zero activations that rows past a group's end read, or null
  int g_begin, g_end;    // prefill: groups of this launch (g_end <= g_begin: all groups)
  const void* act_scale; // W4A8: e8m0 exponents of the MXFP8 activations, [row][K/32], gathered as act;
                         // Int8 W8A8: fp32 scale per activation row
  void* out_scale;       // EPI_SWIGLU_Q8: e8m0 exponents of the output, [row][N/64] (N = 2 I)
  uint32_t* clear_word;  // decode kernel, fp32 epilogue: a word set to 0 by the launch (the next kernel's completion count)
  int thick_rows;        // decode kernel, SwiGLU epilogue: rows per block of the groups of more than 64 rows (0: 64)
};

// Output features (in units of 16) per decode work item, chosen from the instantiated set so an
// item streams at least about 128 KiB of weights (or the most the set allows): small enough that
// the scheduling granularity stays far below one CU's share of the stream, large enough that the
// per-item setup and reduction stay negligible.
inline int decode_nf(int codec, int epi, int K, int N) {
  if (epi == EPI_F32) return 1;
  const double bpw = codec == 0 ? 4.0 : codec == 1 ? 2.0 : (codec == 2 || codec == 5 || codec == 6) ? 1.03125 : 0.53125;
  const int nmat = epi == EPI_SWIGLU ? 2 : 1;
  // converted formats (fp8, MXFP4) stop at 4 tiles for the plain epilogue: their conversion
  // temporaries make 8 tiles cost a wave of occupancy per SIMD, which streams slower
  const int lo = epi == EPI_SWIGLU ? 1 : 2, hi = epi == EPI_SWIGLU ? 2 : (codec >= 2 ? 4 : 8);
  int nf = lo;
  while (nf < hi && 16.0 * nf * K * bpw * nmat < 128.0 * 1024 && N % (32 * nf) == 0) nf *= 2;
  return nf;
}
hipError_t launch_grouped_decode(int act, int epi, int cr, int cs, const GroupedArgs& a,
                                 int max_row_blocks, hipStream_t st);
hipError_t launch_grouped_prefill(int act, int epi, int cr, int cs, const GroupedArgs& a, int max_tiles,
                                  hipStream_t st);
hipError_t launch_w4a8_prefill(int epi, const GroupedArgs& a, int max_units, hipStream_t st);
// W8A8 MXFP8 shared expert (one group, [g_begin, g_end) = [shared_group, shared_group + 1), of
// `rows` rows): gate/up with the MXFP8-writing SwiGLU epilogue, or down.
hipError_t launch_w8a8_shared(int epi, const GroupedArgs& a, int rows, hipStream_t st);
// Int8 W8A8 over all groups: act holds int8 rows, act_scale their fp32 scales (gathered like the
// rows); gate/up (EPI_SWIGLU, h in bf16) or down (EPI_PLAIN).
hipError_t launch_int8_prefill(int epi, const GroupedArgs& a, int max_units, hipStream_t st);
// bf16 rows -> int8 codes and one fp32 scale per row (Int8 W8A8 activations)
hipError_t launch_quant_int8(const void* src, int rows, int K, int8_t* codes, float* scales, hipStream_t st);
int prefill_row_tile();
bool prefill_supported(int act, int cr, int cs, int K, int N_gateup, int N_down);
bool prefill_scores_supported(int act, int K, int N);
hipError_t launch_prefill_scores(const GroupedArgs& a, hipStream_t st);
// The grouped GEMMs' plan (row range per group, rb-row blocks; with thick > 0, groups of more
// than rb rows in thick-row blocks, listed first, and a second table of rb-row blocks only in
// cum_blocks_b / block_group_b) and the prefill kernel's zero row.
hipError_t launch_plan(const int32_t* expert_offsets, int E, int P, int T, int shared, int rb, int thick,
                       int32_t* group_range, int32_t* cum_blocks, int32_t* block_group, int32_t* cum_blocks_b,
                       int32_t* block_group_b, uint32_t* zero, int zero_words, hipStream_t st);
hipError_t launch_topk(const float* logits, int ldl, int nparts, const float* bias, int T, int E, int k,
                       const int32_t* hash_ids, const int32_t* hash_table, int vocab, int32_t* idx, float* w,
                       hipStream_t st);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* slot_token, int32_t* pair_slot, int32_t* ws_rank,
                          int32_t* ws_hist, hipStream_t st);
int permute_blocks(int P);
bool permute_small_ok(int P, int E);
hipError_t launch_permute_small(const int32_t* idx, int T, int k, int E, int shared, int rb, int thick, int32_t* offsets,
                                int32_t* slot_token, int32_t* pair_slot, int32_t* group_range, int32_t* cum_blocks,
                                int32_t* block_group, int32_t* cum_blocks_b, int32_t* block_group_b, hipStream_t st);
// Decode batches: selection (or hash routing), permutation and plan in one launch. `done` is a
// word of the workspace that must read 0 when the kernel starts (the router-score launch before it
// clears it); ws_packed holds T*k ints, ws_hist ceil(T / 8) x E ints.
bool topk_permute_ok(int T, int k, int E);
hipError_t launch_topk_permute(const float* logits, int ldl, int nparts, const float* bias, int T, int E, int k,
                               const int32_t* hash_ids, const int32_t* hash_table, int vocab, int32_t* idx, float* w,
                               int32_t* ws_packed, int32_t* ws_hist, uint32_t* done, int shared, int rb, int thick,
                               int32_t* offsets, int32_t* slot_token, int32_t* pair_slot, int32_t* group_range,
                               int32_t* cum_blocks, int32_t* block_group, int32_t* cum_blocks_b, int32_t* block_group_b,
                               hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int n, hipStream_t st);
// W4A8: bf16 rows [rows][K] -> MXFP8 codes uint8[rows][K] + e8m0 exponents uint8[rows][K/32].
hipError_t launch_quant_mxfp8(const void* src, int rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_combine(int act, const void* y_perm, const int32_t* pair_slot, const float* w,
                          const void* y_shared, void* y, int T, int H, int k, hipStream_t st);

}  // namespace moe
