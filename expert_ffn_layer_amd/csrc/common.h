// Shared device definitions of the MoE layer library (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int WAVE = 64;

// ------------------------------------------------------------------------------------------
// Packed weight layout ("packet" layout).
//
// A K x N weight matrix is cut into 16 x KP tiles (16 output features, KP reduction elements),
// each stored as one 1 KiB packet. Packet (nt, kt) sits at byte (nt * KT + kt) * 1024 with
// KT = K / KP, so the K-stream of one group of 16 features is contiguous. Inside a packet,
// lane l (0..63) owns 16 bytes at l * 16: feature n = nt * 16 + l % 16 and the KP/4
// consecutive reduction indices k = kt * KP + (l / 16) * KP / 4 + [0, KP/4). That is exactly
// the A operand of a 16x16 MFMA with the weights as rows, so one 128-bit load per lane fills
// a wave's operand for 16 features with no shuffles.
//   f32   KP = 16  (4 floats per lane, 4 x v_mfma_f32_16x16x4_f32)
//   bf16  KP = 32  (8 bf16,   1 x v_mfma_f32_16x16x32_bf16)
//   fp8   KP = 64  (16 e4m3,  2 x bf16 MFMA after conversion; fp32 scale per 128x128 block,
//                   kept in its logical [K/128][N/128] array)
//   mxfp4 KP = 128 (32 e2m1,  4 x bf16 MFMA after conversion, even k in the low nibble;
//                   the lane's 32 values are one e8m0 block; packed scales: one byte per lane
//                   per packet at (nt * KT + kt) * 64 + l)
// ------------------------------------------------------------------------------------------
constexpr int PACKET_BYTES = 1024;

__host__ __device__ constexpr int kp_of(int fmt) {
  return fmt == MOE_F32 ? 16 : fmt == MOE_BF16 ? 32 : (fmt == MOE_FP8_E4M3_B128 || fmt == MOE_MXFP8_B32_A8 || fmt == MOE_INT8_W8A8) ? 64 : 128;
}

// bf16 bit helpers (raw uint16 storage)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two fp32 -> two bf16 (round to nearest even), packed low/high
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// SiLU(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp) instead of an IEEE
// division sequence; e^-z -> inf for very negative z gives z * 0 = -0, the right limit.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// fp32 -> OCP E4M3FN code, round to nearest even, saturating at +-448 (the sign of y, zero
// included, is kept); y finite.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = __builtin_fabsf(y);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // below 2^-6: grid 2^-9
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

// Shared e8m0 exponent of an OCP MXFP8 block with maximum magnitude amax:
// floor(log2 amax) - 8 (8 = the largest E4M3 exponent), clamped to [-127, 127], -127 for zero.
__device__ __forceinline__ int mxfp8_exponent(float amax) {
  int X = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 9 : -127;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) {
  return __builtin_nontemporal_load(p);
}

}  // namespace moe
