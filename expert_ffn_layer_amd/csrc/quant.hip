// Activation quantisation for W4A8 routed experts: bf16 rows -> OCP MXFP8.
//
// 'CANN DeepSeek-V4推理优化' (quantisation strategy) runs the routed experts' linear layers as
// W4A8: 4-bit weights times 8-bit activations. On gfx950 the 8-bit side is OCP MXFP8, the format
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies directly: per run of 32 consecutive reduction
// elements an e8m0 exponent X = floor(log2 max|v|) - 8 (8 = the largest E4M3 exponent), clamped
// to [-127, 127] and -127 for an all-zero run, and per element E4M3FN(v * 2^-X), rounded to
// nearest even, saturated at +-448.
//
// Output layout (what the prefill GEMM's DMA reads):
//   codes  uint8[P][K]: row r of the permuted row space (group g owns rows
//          [group_range[2g], group_range[2g+1])), i.e. the rows of the GEMM's activation operand;
//   scales uint8[R16][K/32][16]: one e8m0 byte per (row, 32-block), grouped by 16-row tiles of the
//          *padded* row space in which group g starts at row 128 * cum_blocks[g]: byte
//          ((pr / 16) * (K / 32) + b) * 16 + pr % 16 holds block b of padded row pr. A GEMM row
//          tile then finds its 16 tokens' exponents of one 128-deep step as 64 contiguous bytes in
//          the order the MFMA's scale operand wants them (lane = token + 16 * block). Padding rows
//          get exponent byte 0 (2^-127; their codes are never read).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int QTHREADS = 256;  // 4 waves, one padded row each per pass
constexpr int QROWS = 16;      // padded rows per workgroup (one GEMM row tile)

// fp32 -> E4M3FN code, round to nearest even, saturating at 448; y is finite.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __builtin_fabsf(y);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid of 2^-9 (8 steps -> the code of 2^-6)
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  const uint32_t ab = __float_as_uint(a);
  int e = (int)(ab >> 23) - 127;  // -6 .. 8
  uint32_t m = (ab >> 20) & 7u;   // top 3 mantissa bits
  const uint32_t rest = ab & 0xFFFFFu, half = 0x80000u;
  if (rest > half || (rest == half && (m & 1u))) ++m;
  if (m == 8u) {
    m = 0;
    ++e;
  }
  return sign | ((uint32_t)(e + 7) << 3) | m;  // a < 448 keeps this at or below 0x7E
}

// One workgroup per 16 padded rows; wave w takes rows w, w + 4, ... Each lane quantises 8
// consecutive elements, so four lanes hold one 32-block and agree on its exponent by two xor
// shuffles.
__global__ void __launch_bounds__(QTHREADS) quant_mxfp8_kernel(const uint16_t* __restrict__ src, int lds_,
                                                               const int32_t* __restrict__ gather,
                                                               const int32_t* __restrict__ group_range,
                                                               const int32_t* __restrict__ cum_blocks, int G,
                                                               int K, int padded_rows, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nblk_total = cum_blocks[G];  // 128-row blocks of the routed groups
  for (int q = wave; q < QROWS; q += QTHREADS / 64) {
    const int pr = blockIdx.x * QROWS + q;
    if (pr >= padded_rows) return;
    // group of this padded row: the last g with cum_blocks[g] <= pr / 128
    const int b128 = pr >> 7;
    int src_row = -1, dst_row = -1;
    if (b128 < nblk_total) {
      int lo = 0, hi = G - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cum_blocks[mid] <= b128) lo = mid; else hi = mid - 1;
      }
      const int i = pr - 128 * cum_blocks[lo];
      const int r0 = group_range[2 * lo], n = group_range[2 * lo + 1] - r0;
      if (i < n) {
        dst_row = r0 + i;
        src_row = gather ? gather[dst_row] : dst_row;
      }
    }
    uint8_t* srow = scales + (size_t)(pr >> 4) * (K / 32) * 16 + (pr & 15);
    for (int c0 = 0; c0 < K; c0 += 512) {
      const int c = c0 + 8 * lane;
      if (c >= K) break;  // K is a multiple of 32: whole 4-lane groups stop together
      if (src_row < 0) {
        if ((lane & 3) == 0) srow[(c >> 5) * 16] = 0;
        continue;
      }
      const u32x4 v = *(const u32x4*)(src + (size_t)src_row * lds_ + c);
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16lo(v[i]);
        f[2 * i + 1] = bf16hi(v[i]);
      }
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
      int X = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 1 - 8 : -127;  // floor(log2 amax) - 8
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= e4m3_rne_sat(__builtin_amdgcn_ldexpf(f[i], -X)) << (8 * i);
        hi |= e4m3_rne_sat(__builtin_amdgcn_ldexpf(f[4 + i], -X)) << (8 * i);
      }
      *(u32x2*)(codes + (size_t)dst_row * K + c) = u32x2{lo, hi};
      if ((lane & 3) == 0) srow[(c >> 5) * 16] = (uint8_t)(X + 127);
    }
  }
}

}  // namespace

size_t mxfp8_padded_rows(int P, int E) { return (size_t)128 * ((P + 127) / 128 + E) + 256; }

hipError_t launch_quant_mxfp8(const void* src, int lds_, const int32_t* gather, const int32_t* group_range,
                              const int32_t* cum_blocks, int G, int K, int padded_rows, uint8_t* codes,
                              uint8_t* scales, hipStream_t st) {
  if (K % 32 || padded_rows % QROWS) return hipErrorInvalidValue;
  const int blocks = padded_rows / QROWS;
  if (blocks == 0) return hipSuccess;
  quant_mxfp8_kernel<<<blocks, QTHREADS, 0, st>>>((const uint16_t*)src, lds_, gather, group_range, cum_blocks, G, K,
                                                 padded_rows, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
