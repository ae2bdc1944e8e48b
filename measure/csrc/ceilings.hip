// Measurement kernels of the benchmark (not part of the layer): the achievable HBM read rate, the
// matrix-core rates the GPU sustains under its power limit, and a plain copy of known size that
// scales the hardware byte counters of a profiling run.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// A plain 16-byte-per-lane copy: the known-size reference for hardware byte counters.
__global__ void __launch_bounds__(256) copy16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     long long n16) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// A plain streaming read (16 bytes per lane, non-temporal, each byte once): the achievable HBM
// read rate that kernel bandwidths are compared with.
typedef __attribute__((ext_vector_type(4))) unsigned v4u;
__global__ void __launch_bounds__(256) stream_read_kernel(const v4u* __restrict__ src, long long n16,
                                                          unsigned* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * 256 * 8;
  unsigned acc = 0;
  for (long long i = (long long)blockIdx.x * 256 * 8 + threadIdx.x; i < n16; i += stride) {
    v4u v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i + u * 256 < n16 ? __builtin_nontemporal_load(src + i + u * 256) : v4u{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; practically never stores
}


// MFMA burst: the matrix-core rate this GPU sustains under its power limit with GEMM-like data.
// Two waves per SIMD (512 threads, one workgroup per CU), 16 independent accumulators per wave,
// operands rotating over 5 random register sets so consecutive instructions see different data
// (constant operands draw less power and overstate the rate). KIND 0: v_mfma_f32_16x16x32_bf16;
// KIND 1: v_mfma_scale_f32_16x16x128_f8f6f4 with fp4 (e2m1) x fp8 (e4m3) operands; KIND 2: the same
// instruction with fp8 x fp8; KIND 3: v_mfma_i32_16x16x64_i8.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
__device__ __forceinline__ uint32_t burst_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}
template <int KIND>
__global__ void __launch_bounds__(512, 1) mfma_burst_kernel(int iters, unsigned* __restrict__ sink) {
  constexpr int NS = 5;
  const uint32_t t = blockIdx.x * 512 + threadIdx.x;
  f32x4_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (KIND == 0) {
    bf16x8_t a[NS], b[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // sums of uniforms: roughly normal, |v| < 4
        const float ua = (burst_hash(t * 97 + q * 8 + i) & 0xFFFF) * (1.0f / 65536.0f);
        const float ub = (burst_hash(~(t * 89 + q * 8 + i)) & 0xFFFF) * (1.0f / 65536.0f);
        a[q][i] = (__bf16)(4.0f * ua - 2.0f);
        b[q][i] = (__bf16)(4.0f * ub - 2.0f);
      }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j % NS], b[(j * 3 + 1) % NS], acc[j], 0, 0, 0);
    }
  } else if constexpr (KIND == 3) {
    i32x4_t a[NS], b[NS], iacc[16];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[q][i] = (int)burst_hash(t * 97 + q * 8 + i);
        b[q][i] = (int)burst_hash(~(t * 89 + q * 8 + i));
      }
#pragma unroll
    for (int j = 0; j < 16; ++j) iacc[j] = i32x4_t{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        iacc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j % NS], b[(j * 3 + 1) % NS], iacc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f32x4_t{(float)iacc[j][0], (float)iacc[j][1], (float)iacc[j][2], (float)iacc[j][3]};
  } else {
    constexpr int AF = KIND == 2 ? 0 : 4;  // A operand format: fp8 or fp4
    i32x8_t a[NS], b[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t ha = burst_hash(t * 97 + q * 8 + i);
        a[q][i] = KIND == 2 ? (int)(ha & 0xBFBFBFBFu) : (i < 4 ? (int)ha : 0);  // e4m3, or fp4 in 4 dwords
        b[q][i] = (int)(burst_hash(~(t * 89 + q * 8 + i)) & 0xBFBFBFBFu);      // e4m3 without NaN codes
      }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[j % NS], b[(j * 3 + 1) % NS], acc[j], AF, 0, 0,
                                                                  120 + (j & 7), 0, 121);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  if (r == 1234.5f) sink[0] = 1u;  // keeps the products; practically never stores
}

}  // namespace

extern "C" {

// Reads src[0, bytes) once (bytes a multiple of 16); sink: one writable uint32.
int measure_stream_read(const void* src, long long bytes, void* sink, hipStream_t st) {
  if (bytes % 16 || (uintptr_t)src % 16) return -1;
  if (!bytes) return 0;
  stream_read_kernel<<<4096, 256, 0, st>>>((const v4u*)src, bytes / 16, (unsigned*)sink);
  return (int)hipGetLastError();
}

// MFMA burst over `blocks` workgroups of 512 threads, `iters` x 16 MFMAs per wave; kind 0 bf16
// 16x16x32 (16384 FLOP each), kind 1 fp4 x fp8 and kind 2 fp8 x fp8 16x16x128 (65536 FLOP each),
// kind 3 int8 16x16x64 (32768 OP each). sink: one uint32.
int measure_mfma_burst(int kind, int iters, int blocks, void* sink, hipStream_t st) {
  if (iters < 1 || blocks < 1 || kind < 0 || kind > 3) return -1;
  if (kind == 0) mfma_burst_kernel<0><<<blocks, 512, 0, st>>>(iters, (unsigned*)sink);
  else if (kind == 1) mfma_burst_kernel<1><<<blocks, 512, 0, st>>>(iters, (unsigned*)sink);
  else if (kind == 2) mfma_burst_kernel<2><<<blocks, 512, 0, st>>>(iters, (unsigned*)sink);
  else mfma_burst_kernel<3><<<blocks, 512, 0, st>>>(iters, (unsigned*)sink);
  return (int)hipGetLastError();
}

// dst[0, bytes) <- src[0, bytes); bytes a multiple of 16, both pointers 16-byte aligned.
int measure_copy(const void* src, void* dst, long long bytes, hipStream_t st) {
  if (bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16) return -1;
  if (!bytes) return 0;
  copy16_kernel<<<4096, 256, 0, st>>>((const uint4*)src, (uint4*)dst, bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
