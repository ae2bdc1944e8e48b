// Activation quantisation: bf16 rows -> OCP MXFP8 for W4A8 and W8A8 MXFP8 experts, and -> int8 per
// row for Int8 W8A8 experts.
//
// 'CANN DeepSeek-V4推理优化' (quantisation strategy) runs the routed experts' linear layers as
// W4A8: 4-bit weights times 8-bit activations. On gfx950 the 8-bit side is OCP MXFP8, the format
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies directly: per run of 32 consecutive reduction
// elements an e8m0 exponent X = floor(log2 max|v|) - 8 (8 = the largest E4M3 exponent), clamped
// to [-127, 127] and -127 for an all-zero run, and per element E4M3FN(v * 2^-X), rounded to
// nearest even, saturated at +-448.
//
// Each token row of x is quantised once, in token order: codes uint8[T][K] and exponents
// uint8[T][K/32]; the routed experts' GEMM gathers both by slot_token, as the bf16 path gathers x.
// For the MXFP8 formats the second product's input, h, is quantised in the gate/up GEMM's epilogue
// (a 32-block is one wave's 32 columns of a row); Int8 W8A8 scales a whole row of h, which spans
// many workgroups, so h is written in bf16 and quantised here, row by row, before down.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int QTHREADS = 256;  // int8: 4 waves, one row each

// MXFP8: thread i quantises elements 8i .. 8i + 7 of the row-major [rows][K] matrix (K a multiple
// of 32, so a 32-block is four consecutive threads of one wave, which agree on its exponent by two
// xor shuffles, and block b of the flat matrix is row b / (K / 32), block b % (K / 32)).
__global__ void __launch_bounds__(QTHREADS) quant_mxfp8_kernel(const uint16_t* __restrict__ src, long long n8,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
  const long long i = (long long)blockIdx.x * QTHREADS + threadIdx.x;
  const bool live = i < n8;  // the whole wave takes part in the shuffles
  u32x4 v = {0u, 0u, 0u, 0u};
  if (live) v = *(const u32x4*)(src + 8 * i);
  float f[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf16lo(v[q]);
    f[2 * q + 1] = bf16hi(v[q]);
  }
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[q]));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
  const int X = mxfp8_exponent(amax);
  if (!live) return;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lo |= e4m3_rne_sat(__builtin_amdgcn_ldexpf(f[q], -X)) << (8 * q);
    hi |= e4m3_rne_sat(__builtin_amdgcn_ldexpf(f[4 + q], -X)) << (8 * q);
  }
  *(u32x2*)(codes + 8 * i) = u32x2{lo, hi};
  if ((threadIdx.x & 3) == 0) scales[i >> 2] = (uint8_t)(X + 127);
}

// Int8 W8A8: row `row` of src (bf16, K a multiple of 8, at most 64 * 8 * CH) -> int8 codes and one
// fp32 scale per row. One wave per row, which holds the row in registers (CH chunks of 8 per lane,
// the fewest that cover K, so short rows keep the occupancy up): the largest magnitude by a
// wave-wide xor reduction, then f = 127 / max and s = max / 127 (IEEE fp32 divisions) and
// code = rint(v * f) (fp32 product, ties to even), clamped to +-127. An all-zero row gets s = 0 and
// zero codes. f is formed from the maximum's significand, max = m 2^e, f = 127 / m, and multiplies
// v 2^-e: the exact power-of-two scaling gives the same fp32 value as v * (127 / max) wherever that
// factor is finite, and keeps it finite for rows whose maximum is below about 2^-121.
constexpr int QI8_MAX_CHUNKS = 16;
template <int CH>
__global__ void __launch_bounds__(QTHREADS) quant_int8_kernel(const uint16_t* __restrict__ src, int rows, int K,
                                                              int8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (QTHREADS / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* in = src + (size_t)row * K;
  u32x4 v[CH];
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    const int c = 8 * lane + 512 * q;
    v[q] = c < K ? *(const u32x4*)(in + c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16lo(v[q][i])), __builtin_fabsf(bf16hi(v[q][i]))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
  const int e = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 0;  // amax = m 2^e, m in [0.5, 1)
  const float f = amax > 0.f ? __fdiv_rn(127.0f, __builtin_amdgcn_ldexpf(amax, -e)) : 0.f;
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    const int c = 8 * lane + 512 * q;
    if (c >= K) break;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = (i & 1) ? bf16hi(v[q][i >> 1]) : bf16lo(v[q][i >> 1]);
      const float r =
          __builtin_fminf(__builtin_fmaxf(__builtin_rintf(__fmul_rn(__builtin_amdgcn_ldexpf(x, -e), f)), -127.f), 127.f);
      w[i >> 2] |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * (i & 3));
    }
    *(u32x2*)(codes + (size_t)row * K + c) = u32x2{w[0], w[1]};
  }
  if (lane == 0) scales[row] = __fdiv_rn(amax, 127.0f);
}

}  // namespace

hipError_t launch_quant_int8(const void* src, int rows, int K, int8_t* codes, float* scales, hipStream_t st) {
  if (K % 8 || K > 8 * 64 * QI8_MAX_CHUNKS) return hipErrorInvalidValue;
  const int blocks = (rows + QTHREADS / 64 - 1) / (QTHREADS / 64);
  if (blocks == 0) return hipSuccess;
  const uint16_t* s16 = (const uint16_t*)src;
  if (K <= 512 * 4) quant_int8_kernel<4><<<blocks, QTHREADS, 0, st>>>(s16, rows, K, codes, scales);
  else if (K <= 512 * 8) quant_int8_kernel<8><<<blocks, QTHREADS, 0, st>>>(s16, rows, K, codes, scales);
  else quant_int8_kernel<QI8_MAX_CHUNKS><<<blocks, QTHREADS, 0, st>>>(s16, rows, K, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp8(const void* src, int rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (K % 32) return hipErrorInvalidValue;
  const long long n8 = (long long)rows * K / 8;
  const long long blocks = (n8 + QTHREADS - 1) / QTHREADS;
  if (blocks == 0) return hipSuccess;
  quant_mxfp8_kernel<<<(unsigned)blocks, QTHREADS, 0, st>>>((const uint16_t*)src, n8, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
