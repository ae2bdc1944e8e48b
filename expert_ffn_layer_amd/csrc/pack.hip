// Prepack: logical row-major K x N matrices -> 1 KiB MFMA-operand packets (see common.h).
// Runs once when the weights are loaded; the layer's kernels only read the packed form.
#include "common.h"

namespace moe {

// One thread writes one lane's 16 bytes of one packet. Reads are strided (one element per
// row); this is a one-time conversion, so it favours obviousness over bandwidth.
template <int FMT>
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t* __restrict__ src,
                                                   const uint8_t* __restrict__ src_scale,
                                                   uint8_t* __restrict__ dst,
                                                   uint8_t* __restrict__ dst_scale, int count,
                                                   int K, int N, int NT, long long total) {
  constexpr int KP = kp_of(FMT);
  constexpr int RUN = KP / 4;
  const int KT = K / KP;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int l = (int)(gid & 63);
  long long p = gid >> 6;  // packet index over (m, nt, kt)
  const int kt = (int)(p % KT);
  const int nt = (int)((p / KT) % NT);
  const int m = (int)(p / ((long long)KT * NT));
  const int n = nt * 16 + (l & 15);
  const int k0 = kt * KP + (l >> 4) * RUN;
  const bool in = n < N;
  u32x4 out = {0u, 0u, 0u, 0u};
  uint32_t* o = (uint32_t*)&out;
  if (FMT == MOE_F32) {
    const float* w = (const float*)src + (size_t)m * K * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = in ? __float_as_uint(w[(size_t)(k0 + i) * N + n]) : 0u;
  } else if (FMT == MOE_BF16) {
    const uint16_t* w = (const uint16_t*)src + (size_t)m * K * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = in ? w[(size_t)(k0 + 2 * i) * N + n] : 0u;
      uint32_t hi = in ? w[(size_t)(k0 + 2 * i + 1) * N + n] : 0u;
      o[i] = lo | (hi << 16);
    }
  } else if (FMT == MOE_FP8_E4M3_B128 || FMT == MOE_MXFP8_B32_A8 || FMT == MOE_INT8_W8A8) {
    const uint8_t* w = src + (size_t)m * K * N;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t b = in ? w[(size_t)(k0 + i) * N + n] : 0u;
      o[i >> 2] |= b << (8 * (i & 3));
    }
    if (FMT == MOE_INT8_W8A8 && kt == 0 && l < 16) {
      // the per-feature scales, one float per (padded) feature: zero past N
      ((float*)dst_scale)[(size_t)m * NT * 16 + n] = in ? ((const float*)src_scale)[(size_t)m * N + n] : 0.0f;
    }
    if (FMT == MOE_MXFP8_B32_A8 && (kt & 1) == 0) {
      // one exponent byte per lane per pair of packets (128 reduction elements): lane l takes
      // the 32-element block (l / 16) of the pair, the run its MFMA operand scale covers
      const int kb = (kt >> 1) * 4 + (l >> 4);
      dst_scale[(p >> 1) * 64 + l] = in ? src_scale[(size_t)m * (K / 32) * N + (size_t)kb * N + n] : 127;
    }
  } else {  // MXFP4
    const uint8_t* w = src + (size_t)m * K * (N / 2);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      uint32_t nib = 0;
      if (in) {
        uint8_t b = w[(size_t)(k0 + i) * (N / 2) + (n >> 1)];
        nib = (n & 1) ? (b >> 4) : (b & 15);
      }
      o[i >> 3] |= nib << (4 * (i & 7));
    }
    uint8_t s = in ? src_scale[(size_t)m * (K / 32) * N + (size_t)(k0 / 32) * N + n] : 127;
    dst_scale[p * 64 + l] = s;
  }
  *(u32x4*)(dst + p * PACKET_BYTES + l * 16) = out;
}

}  // namespace moe

using namespace moe;

extern "C" __attribute__((visibility("hidden"))) hipError_t moe_launch_pack(int fmt, int count, int K, int N, const void* w,
                                      const void* scale, void* packed, void* packed_scale,
                                      hipStream_t stream) {
  const int NT = (N + 255) / 256 * 16;  // features padded to a multiple of 256 with zeros
  const int KT = K / kp_of(fmt);
  long long total = (long long)count * NT * KT * 64;
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
  const uint8_t* s = (const uint8_t*)w;
  const uint8_t* ss = (const uint8_t*)scale;
  uint8_t* d = (uint8_t*)packed;
  uint8_t* ds = (uint8_t*)packed_scale;
  switch (fmt) {
    case MOE_F32: pack_kernel<MOE_F32><<<grid, block, 0, stream>>>(s, ss, d, ds, count, K, N, NT, total); break;
    case MOE_BF16: pack_kernel<MOE_BF16><<<grid, block, 0, stream>>>(s, ss, d, ds, count, K, N, NT, total); break;
    case MOE_FP8_E4M3_B128:
      pack_kernel<MOE_FP8_E4M3_B128><<<grid, block, 0, stream>>>(s, ss, d, ds, count, K, N, NT, total);
      if (packed_scale && scale)
        return hipMemcpyAsync(packed_scale, scale, (size_t)count * (K / 128) * (N / 128) * 4,
                              hipMemcpyDeviceToDevice, stream);
      break;
    case MOE_MXFP4_B32: pack_kernel<MOE_MXFP4_B32><<<grid, block, 0, stream>>>(s, ss, d, ds, count, K, N, NT, total); break;
    case MOE_MXFP8_B32_A8:
      pack_kernel<MOE_MXFP8_B32_A8><<<grid, block, 0, stream>>>(s, ss, d, ds, count, K, N, NT, total);
      break;
    case MOE_INT8_W8A8:
      pack_kernel<MOE_INT8_W8A8><<<grid, block, 0, stream>>>(s, ss, d, ds, count, K, N, NT, total);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
