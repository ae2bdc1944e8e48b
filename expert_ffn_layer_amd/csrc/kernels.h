// Declarations shared by the kernels and the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum { EPI_SWIGLU = 0, EPI_PLAIN = 1, EPI_F32 = 2 };

// Arguments of a grouped GEMM over a "row space": group g owns rows
// [group_range[2g], group_range[2g+1]). Row r reads activation row
//   gather ? (r < P ? gather[r] : r - P) : r
// (gathered token rows for the routed experts, then the shared expert's rows P.. in token
// order), clamped to [0, act_rows), and writes output row r, or row r - P of out_s when out_s
// is set and r >= P. group_range == nullptr means one group of M rows.
struct GroupedArgs {
  const int32_t* group_range;
  const int32_t* cum_blocks;  // prefix count of row blocks per group (block = RB rows)
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
};

// Output features (in units of 16) per decode work item: a small item (16-32 features) keeps
// the scheduling granularity far below one CU's share of the weight stream.
__host__ __device__ constexpr int decode_nf(int codec, int epi) {
  return epi == EPI_SWIGLU ? (codec == 3 /* MXFP4 */ ? 2 : 1) : (epi == EPI_F32 ? 1 : 2);
}

hipError_t launch_grouped_decode(int act, int epi, int cr, int cs, const GroupedArgs& a,
                                 int max_row_blocks, hipStream_t st);
hipError_t launch_grouped_prefill(int act, int epi, int cr, int cs, const GroupedArgs& a,
                                  hipStream_t st);
hipError_t launch_plan(const int32_t* expert_offsets, int E, int P, int T, int shared, int rb,
                       int32_t* group_range, int32_t* cum_blocks, hipStream_t st);
hipError_t launch_topk(const float* logits, int ldl, int nparts, const float* bias, int T, int E, int k,
                       int32_t* idx, float* w, hipStream_t st);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* slot_token, int32_t* pair_slot, int32_t* ws_rank,
                          int32_t* ws_hist, hipStream_t st);
int permute_blocks(int P);
bool permute_small_ok(int P, int E);
hipError_t launch_permute_small(const int32_t* idx, int T, int k, int E, int shared, int rb, int32_t* offsets,
                                int32_t* slot_token, int32_t* pair_slot, int32_t* group_range, int32_t* cum_blocks,
                                hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int n, hipStream_t st);
hipError_t launch_combine(int act, const void* y_perm, const int32_t* pair_slot, const float* w,
                          const void* y_shared, void* y, int T, int H, int k, hipStream_t st);

}  // namespace moe
