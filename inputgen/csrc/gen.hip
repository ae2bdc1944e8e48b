// GPU fill kernels of the seeded input generator. Input machinery only (not part of the MoE
// library): they write the same values as inputgen/philox.py, bit for bit:
//   * Philox4x32-10 (Salmon et al., SC'11); word i of a stream = word i%4 of the block at
//     counter (i/4 mod 2^32, i/4 >> 32, stream, 0) under key (key0, key1);
//   * normal value = integer-interpolated inverse CDF table (Q20), exact in fp32;
//   * N(0, s^2) = z * s (one fp32 multiply, round to nearest even);
//   * stored formats: bf16 (round to nearest even), fp8 e4m3fn with one fp32 scale
//     amax/448 per 128 x 128 block, MXFP4 e2m1 and MXFP8 e4m3fn with one e8m0 exponent per 32 K
//     of a column, int8 with one fp32 scale amax/127 per column.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]), lo0 = 0xD2511F53u * c[0];
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]), lo1 = 0xCD9E8D57u * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// The 4 words of block b of a stream.
__device__ __forceinline__ void block_words(uint64_t b, uint32_t stream, uint32_t k0, uint32_t k1, uint32_t w[4]) {
  w[0] = (uint32_t)b;
  w[1] = (uint32_t)(b >> 32);
  w[2] = stream;
  w[3] = 0u;
  philox(w, k0, k1);
}

__device__ __forceinline__ float normal_of(uint32_t u, const int32_t* __restrict__ T, const int32_t* __restrict__ TT) {
  const uint32_t idx = u >> 20, frac = u & 0xFFFFFu;
  int64_t z;
  if (idx == 0u || idx == 4095u) {
    const uint32_t tl = idx ? 0xFFFFFFFFu - u : u;
    uint32_t sub = tl >> 8;
    sub = sub > 4095u ? 4095u : sub;
    const uint32_t sf = tl & 0xFFu;
    const int64_t s0 = TT[sub], s1 = TT[sub + 1];
    const int64_t zt = s0 + (((s1 - s0) * (int64_t)sf) >> 8);
    z = idx ? -zt : zt;
  } else {
    const int64_t t0 = T[idx], t1 = T[idx + 1];
    z = t0 + (((t1 - t0) * (int64_t)frac) >> 20);
  }
  return __fmul_rn((float)(int32_t)z, 0x1p-20f);
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const float a = fabsf(v);
  const uint32_t bits = __float_as_uint(a);
  int32_t code;
  if (a < 0x1p-6f) {
    code = (int32_t)rintf(a * 512.0f);
  } else {
    code = (int32_t)((bits + 0x7FFFFu + ((bits >> 20) & 1u)) >> 20) - ((127 - 7) << 3);
  }
  code = code > 0x7E ? 0x7E : code;
  if (v < 0.0f && code != 0) code |= 0x80;
  return (uint32_t)code;
}

__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  uint32_t c = 7;
  if (a <= 5.0f) c = 6;
  if (a < 3.5f) c = 5;
  if (a <= 2.5f) c = 4;
  if (a < 1.75f) c = 3;
  if (a <= 1.25f) c = 2;
  if (a < 0.75f) c = 1;
  if (a <= 0.25f) c = 0;
  if (v < 0.0f && c != 0) c |= 8;
  return c;
}

// Dense fill of `count` matrices of n values each (matrix m uses stream stream0 + m), values
// [start, start + n) of each stream. fmt 0 = f32, 1 = bf16. n and start multiples of 4.
__global__ void fill_dense_kernel(void* out, int fmt, uint32_t k0, uint32_t k1, uint32_t stream0, int count,
                                  long long n, long long start, float sigma, const int32_t* T, const int32_t* TT) {
  const long long nb = n / 4;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= nb * count) return;
  const int m = (int)(gid / nb);
  const long long b = gid % nb;
  uint32_t w[4];
  block_words((uint64_t)(start / 4 + b), stream0 + (uint32_t)m, k0, k1, w);
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __fmul_rn(normal_of(w[i], T, TT), sigma);
  const long long o = (long long)m * n + 4 * b;
  if (fmt == 0) {
    float4* p = (float4*)((float*)out + o);
    *p = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2* p = (uint2*)((uint16_t*)out + o);
    *p = make_uint2(bf16_bits(v[0]) | (bf16_bits(v[1]) << 16), bf16_bits(v[2]) | (bf16_bits(v[3]) << 16));
  }
}

// fp8: one workgroup per 128 x 128 block of one K x N matrix. Thread t covers columns
// 4*(t%32) .. +3 of rows t/32 + 8j (j < 16).
__global__ void __launch_bounds__(256) fill_fp8_kernel(uint8_t* codes, float* scales, uint32_t k0, uint32_t k1,
                                                       uint32_t stream0, int K, int N, float sigma,
                                                       const int32_t* T, const int32_t* TT) {
  const int NB = N / 128, KB = K / 128;
  const int m = blockIdx.x / (KB * NB);
  const int kb = (blockIdx.x / NB) % KB, nb = blockIdx.x % NB;
  const int t = threadIdx.x;
  const int c0 = nb * 128 + 4 * (t & 31);
  float v[16][4];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = kb * 128 + (t >> 5) + 8 * j;
    uint32_t w[4];
    block_words(((uint64_t)row * N + c0) / 4, stream0 + (uint32_t)m, k0, k1, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[j][i] = __fmul_rn(normal_of(w[i], T, TT), sigma);
      amax = fmaxf(amax, fabsf(v[j][i]));
    }
  }
  __shared__ float red[256];
  red[t] = amax;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] = fmaxf(red[t], red[t + s]);
    __syncthreads();
  }
  amax = red[0];
  const float sc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (t == 0) scales[(size_t)m * KB * NB + kb * NB + nb] = sc;
  uint8_t* cm = codes + (size_t)m * K * N;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = kb * 128 + (t >> 5) + 8 * j;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= e4m3_code(__fdiv_rn(v[j][i], sc)) << (8 * i);
    *(uint32_t*)(cm + (size_t)row * N + c0) = word;
  }
}

// MXFP4: one thread per (4 consecutive columns, 32-row block) of one K x N matrix.
__global__ void fill_mxfp4_kernel(uint8_t* codes, uint8_t* scales, uint32_t k0, uint32_t k1, uint32_t stream0,
                                  int count, int K, int N, float sigma, const int32_t* T, const int32_t* TT) {
  const long long per = (long long)(N / 4) * (K / 32);
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= per * count) return;
  const int m = (int)(gid / per);
  const int kb = (int)((gid % per) / (N / 4));
  const int c0 = 4 * (int)(gid % (N / 4));
  float v[32][4];
  float amax[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < 32; ++r) {
    uint32_t w[4];
    block_words(((uint64_t)(kb * 32 + r) * N + c0) / 4, stream0 + (uint32_t)m, k0, k1, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[r][i] = __fmul_rn(normal_of(w[i], T, TT), sigma);
      amax[i] = fmaxf(amax[i], fabsf(v[r][i]));
    }
  }
  uint32_t E[4];
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = (int)((__float_as_uint(amax[i]) >> 23) & 0xFF) - 2;
    e = e < 1 ? 1 : (e > 254 ? 254 : e);
    E[i] = amax[i] > 0.0f ? (uint32_t)e : 127u;
    inv[i] = __uint_as_float((254u - E[i]) << 23);
  }
  uint8_t* cm = codes + (size_t)m * K * (N / 2);
  for (int r = 0; r < 32; ++r) {
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = e2m1_code(__fmul_rn(v[r][i], inv[i]));
    *(uint16_t*)(cm + (size_t)(kb * 32 + r) * (N / 2) + c0 / 2) =
        (uint16_t)(c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12));
  }
  *(uint32_t*)(scales + (size_t)m * (K / 32) * N + (size_t)kb * N + c0) = E[0] | (E[1] << 8) | (E[2] << 16) | (E[3] << 24);
}

// MXFP8: one thread per (4 consecutive columns, 32-row block) of one K x N matrix; the exponent
// is floor(log2 amax) - 8 (the largest E4M3 exponent), so codes saturate at 448.
__global__ void fill_mxfp8_kernel(uint8_t* codes, uint8_t* scales, uint32_t k0, uint32_t k1, uint32_t stream0,
                                  int count, int K, int N, float sigma, const int32_t* T, const int32_t* TT) {
  const long long per = (long long)(N / 4) * (K / 32);
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= per * count) return;
  const int m = (int)(gid / per);
  const int kb = (int)((gid % per) / (N / 4));
  const int c0 = 4 * (int)(gid % (N / 4));
  float v[32][4];
  float amax[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < 32; ++r) {
    uint32_t w[4];
    block_words(((uint64_t)(kb * 32 + r) * N + c0) / 4, stream0 + (uint32_t)m, k0, k1, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[r][i] = __fmul_rn(normal_of(w[i], T, TT), sigma);
      amax[i] = fmaxf(amax[i], fabsf(v[r][i]));
    }
  }
  uint32_t E[4];
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = (int)((__float_as_uint(amax[i]) >> 23) & 0xFF) - 8;
    e = e < 1 ? 1 : (e > 254 ? 254 : e);
    E[i] = amax[i] > 0.0f ? (uint32_t)e : 127u;
    inv[i] = __uint_as_float((254u - E[i]) << 23);
  }
  uint8_t* cm = codes + (size_t)m * K * N;
  for (int r = 0; r < 32; ++r) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= e4m3_code(__fmul_rn(v[r][i], inv[i])) << (8 * i);
    *(uint32_t*)(cm + (size_t)(kb * 32 + r) * N + c0) = word;
  }
  *(uint32_t*)(scales + (size_t)m * (K / 32) * N + (size_t)kb * N + c0) = E[0] | (E[1] << 8) | (E[2] << 16) | (E[3] << 24);
}

// Int8 per output channel: one thread per 4 consecutive columns of one K x N matrix, two passes over
// the column (the maximum, then the codes): s = amax / 127, code = rint(w / s), clamped to +-127.
__global__ void fill_int8_kernel(int8_t* codes, float* scales, uint32_t k0, uint32_t k1, uint32_t stream0, int count,
                                 int K, int N, float sigma, const int32_t* T, const int32_t* TT) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)count * (N / 4)) return;
  const int m = (int)(gid / (N / 4));
  const int c0 = 4 * (int)(gid % (N / 4));
  float amax[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < K; ++r) {
    uint32_t w[4];
    block_words(((uint64_t)r * N + c0) / 4, stream0 + (uint32_t)m, k0, k1, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) amax[i] = fmaxf(amax[i], fabsf(__fmul_rn(normal_of(w[i], T, TT), sigma)));
  }
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = amax[i] > 0.0f ? __fdiv_rn(amax[i], 127.0f) : 1.0f;
  int8_t* cm = codes + (size_t)m * K * N;
  for (int r = 0; r < K; ++r) {
    uint32_t w[4];
    block_words(((uint64_t)r * N + c0) / 4, stream0 + (uint32_t)m, k0, k1, w);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float q = rintf(__fdiv_rn(__fmul_rn(normal_of(w[i], T, TT), sigma), sc[i]));
      q = fminf(fmaxf(q, -127.0f), 127.0f);
      word |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * i);
    }
    *(uint32_t*)(cm + (size_t)r * N + c0) = word;
  }
  *(float4*)(scales + (size_t)m * N + c0) = make_float4(sc[0], sc[1], sc[2], sc[3]);
}

}  // namespace

extern "C" {

int gen_fill_dense(void* out, int fmt, uint32_t k0, uint32_t k1, uint32_t stream0, int count, long long n,
                   long long start, float sigma, const int32_t* T, const int32_t* TT, hipStream_t st) {
  if (n % 4 || start % 4) return -1;
  const long long threads = n / 4 * count;
  if (!threads) return 0;
  fill_dense_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(out, fmt, k0, k1, stream0, count, n, start,
                                                                       sigma, T, TT);
  return (int)hipGetLastError();
}

int gen_fill_fp8(uint8_t* codes, float* scales, uint32_t k0, uint32_t k1, uint32_t stream0, int count, int K, int N,
                 float sigma, const int32_t* T, const int32_t* TT, hipStream_t st) {
  if (K % 128 || N % 128) return -1;
  const unsigned blocks = (unsigned)count * (K / 128) * (N / 128);
  if (!blocks) return 0;
  fill_fp8_kernel<<<blocks, 256, 0, st>>>(codes, scales, k0, k1, stream0, K, N, sigma, T, TT);
  return (int)hipGetLastError();
}

int gen_fill_mxfp4(uint8_t* codes, uint8_t* scales, uint32_t k0, uint32_t k1, uint32_t stream0, int count, int K,
                   int N, float sigma, const int32_t* T, const int32_t* TT, hipStream_t st) {
  if (K % 32 || N % 4) return -1;
  const long long threads = (long long)count * (N / 4) * (K / 32);
  if (!threads) return 0;
  fill_mxfp4_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(codes, scales, k0, k1, stream0, count, K, N,
                                                                       sigma, T, TT);
  return (int)hipGetLastError();
}

int gen_fill_mxfp8(uint8_t* codes, uint8_t* scales, uint32_t k0, uint32_t k1, uint32_t stream0, int count, int K,
                   int N, float sigma, const int32_t* T, const int32_t* TT, hipStream_t st) {
  if (K % 32 || N % 4) return -1;
  const long long threads = (long long)count * (N / 4) * (K / 32);
  if (!threads) return 0;
  fill_mxfp8_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(codes, scales, k0, k1, stream0, count, K, N,
                                                                       sigma, T, TT);
  return (int)hipGetLastError();
}

int gen_fill_int8(int8_t* codes, float* scales, uint32_t k0, uint32_t k1, uint32_t stream0, int count, int K, int N,
                  float sigma, const int32_t* T, const int32_t* TT, hipStream_t st) {
  if (N % 4) return -1;
  const long long threads = (long long)count * (N / 4);
  if (!threads) return 0;
  fill_int8_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(codes, scales, k0, k1, stream0, count, K, N,
                                                                      sigma, T, TT);
  return (int)hipGetLastError();
}

}  // extern "C"
