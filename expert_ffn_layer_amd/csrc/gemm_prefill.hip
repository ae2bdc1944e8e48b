// Prefill-regime grouped GEMM: many rows per expert, bound by the matrix cores.
//
// Work item = (group, tile of BM = 128 rows, tile of output features). The four waves of a
// workgroup split the features (64 each: 32 gate + 32 up columns for the SwiGLU GEMM, 64 for the
// plain one) and share the 128-row activation tile. Both operands reach LDS by direct
// global -> LDS DMA (global_load_lds_dwordx4) through a 3- or 4-stage ring of 64-wide reduction
// steps, so the loads of the next stages are in flight for several steps of MFMA work and cost
// no registers. Each 1 KiB DMA lands in MFMA fragment order (a weight packet as stored; an
// activation fragment gathered from 16 rows), so every LDS read is a conflict-free 16-byte read
// at lane * 16. Weights are the A operand of v_mfma_f32_16x16x32_bf16, activations the B
// operand; fp8 packets are converted once per workgroup in registers (e4m3 -> fp32 exact, times
// the 128 x 128 block scale, -> bf16).
//
// Items are ordered so that a run of consecutive items covers up to 8 feature tiles x all row
// tiles of one group, and the workgroup -> item map gives each XCD a contiguous run of items:
// workgroups resident at the same time on one XCD then share weight and activation slices in
// that XCD's L2 (Chapter 6 'Supernodes' section 6.3.2: one weight read serves many rows).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PBM = 128;  // rows per item
constexpr int PBK = 64;   // reduction elements per pipeline stage
constexpr int PWN = 64;   // output features per wave (4 tiles of 16)
constexpr int NXCD = 8;

template <int C>
struct PCodec;

template <>
struct PCodec<MOE_BF16> {
  static constexpr int PK = 2;      // packets per feature tile per stage
  static constexpr int STAGES = 3;  // 48 KiB per stage
  // element offset (within a stage's 64) of the B fragment of half h for lane group g
  __device__ static int boff(int g, int h) { return 8 * g + 32 * h; }
  __device__ static void frags(const u32x4 (&w)[2], float, bf16x8 (&a)[2]) {
    a[0] = __builtin_bit_cast(bf16x8, w[0]);
    a[1] = __builtin_bit_cast(bf16x8, w[1]);
  }
};

// e4m3fn -> fp32 (exact) -> * block scale -> bf16 (round to nearest even)
__device__ __forceinline__ bf16x8 p_fp8x8(uint32_t w0, uint32_t w1, float s) {
  typedef __attribute__((ext_vector_type(2))) float f2;
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
  const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
  const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
  const f2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
  u32x4 r;
  r[0] = pack_bf16x2(a.x * s, a.y * s);
  r[1] = pack_bf16x2(b.x * s, b.y * s);
  r[2] = pack_bf16x2(c.x * s, c.y * s);
  r[3] = pack_bf16x2(d.x * s, d.y * s);
  return __builtin_bit_cast(bf16x8, r);
}

template <>
struct PCodec<MOE_FP8_E4M3_B128> {
  static constexpr int PK = 1;
  static constexpr int STAGES = 4;  // 32 KiB per stage
  __device__ static int boff(int g, int h) { return 16 * g + 8 * h; }
  __device__ static void frags(const u32x4 (&w)[1], float s, bf16x8 (&a)[2]) {
    a[0] = p_fp8x8(w[0][0], w[0][1], s);
    a[1] = p_fp8x8(w[0][2], w[0][3], s);
  }
};

template <int EPI>
struct PEpi {
  static constexpr int NMAT = EPI == EPI_SWIGLU ? 2 : 1;
  static constexpr int WF = PWN / 16 / NMAT;  // feature tiles per matrix per wave
  static constexpr int WGF = 4 * WF * 16;     // output features per workgroup
};

// (group-local item) -> (row tile, feature tile): runs of up to 8 feature tiles over all row
// tiles of the group.
__device__ __forceinline__ void item_tiles(int i, int mt, int ntn, int& m, int& n) {
  const int nb = i / (mt * 8);
  const int rem = i - nb * mt * 8;
  const int width = min(8, ntn - nb * 8);
  m = rem / width;
  n = nb * 8 + rem % width;
}

// s_waitcnt vmcnt(n) (gfx9 encoding; expcnt and lgkmcnt not waited on)
#define MOE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00)

typedef __attribute__((address_space(3))) void lds_void;

template <int C, int EPI>
__global__ void __launch_bounds__(256, 1) grouped_prefill_kernel(GroupedArgs a) {
  using Cd = PCodec<C>;
  constexpr int NMAT = PEpi<EPI>::NMAT;
  constexpr int WF = PEpi<EPI>::WF;
  constexpr int NT = NMAT * WF;  // 16-feature tiles per wave (4)
  constexpr int PK = Cd::PK;
  constexpr int KP = PBK / PK;   // reduction elements per packet
  constexpr int D = Cd::STAGES;
  constexpr int ACT_B = 16 * 1024;            // activation fragments per stage (16 x 1 KiB)
  constexpr int WTS_B = 4 * NT * PK * 1024;   // weight packets per stage (all waves)
  constexpr int STAGE_B = ACT_B + WTS_B;
  constexpr int L = 4 + NT * PK;              // DMA loads per wave per stage
  __shared__ __attribute__((aligned(1024))) uint8_t lds[D * STAGE_B];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (SGPR) so the per-wave scale reads become scalar loads, which do not count
  // against vmcnt and so do not drain the DMA pipeline
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntn = a.NTW;
  // XCD-aware workgroup -> item map: each XCD takes a contiguous run of the item list
  const int per_xcd = gridDim.x / NXCD;
  const int item = (blockIdx.x % NXCD) * per_xcd + blockIdx.x / NXCD;
  const int total = a.cum_blocks[a.G] * ntn;
  if (item >= total) return;
  int lo = 0, hi = a.G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cum_blocks[mid] * ntn <= item) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int mt = a.cum_blocks[g + 1] - a.cum_blocks[g];
  int mtile, ntile;
  item_tiles(item - a.cum_blocks[g] * ntn, mt, ntn, mtile, ntile);
  const int rbeg = a.group_range[2 * g], rend = a.group_range[2 * g + 1];
  const int row0 = rbeg + mtile * PBM;
  const int nr = min(PBM, rend - row0);
  const bool is_shared = g == a.shared_group;
  const uint8_t* w0 = is_shared ? a.wa_s : a.wa_r + (size_t)g * a.mat_bytes;
  const uint8_t* w1 = is_shared ? a.wb_s : (a.wb_r ? a.wb_r + (size_t)g * a.mat_bytes : nullptr);
  const float* s0 = (const float*)(is_shared ? a.sa_s : (a.sa_r ? a.sa_r + (size_t)g * a.scale_bytes : nullptr));
  const float* s1 = (const float*)(is_shared ? a.sb_s : (a.sb_r ? a.sb_r + (size_t)g * a.scale_bytes : nullptr));
  const int KT = a.K / KP;
  const int nsteps = a.K / PBK;
  const int j16 = lane & 15, g4 = lane >> 4;

  // this wave's 16-feature tiles (matrix t / WF) and their packet streams
  int ftile[NT];
  const uint8_t* fbase[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    ftile[t] = (ntile * 4 + wave) * WF + t % WF;
    fbase[t] = (t / WF == 0 ? w0 : w1) + (size_t)ftile[t] * KT * PACKET_BYTES + (size_t)lane * 16;
  }
  // fp8 block scales of this wave: its features of each matrix lie in one 128-wide block, so
  // the scale depends only on the 128-deep reduction block; lane i holds block i (K <= 8192),
  // and the loop picks the current one with a lane read (no memory access in the pipeline)
  const int nblk = ftile[0] >> 3;
  float scv[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const float* sp = m == 0 ? s0 : s1;
    scv[m] = (C == MOE_FP8_E4M3_B128 && lane < (a.K >> 7)) ? sp[lane * (a.N >> 7) + nblk] : 1.0f;
  }

  // activation fragments this wave loads per stage: f = 4 * wave + i -> row tile f / 2, half f % 2;
  // lane l fetches row tile*16 + l%16 at the fragment's reduction offset
  const uint8_t* arow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = (2 * wave + i) * 16 + j16;
    const int r = row0 + (rr < nr ? rr : 0);
    int src = a.gather ? (r < a.P ? a.gather[r] : r - a.P) : r;
    if ((unsigned)src >= (unsigned)a.act_rows) src = 0;
    arow[i] = (const uint8_t*)a.act + (size_t)src * a.lda * 2;
  }

  // issue the DMA of stage `step` (clamped into range) into its LDS slot
  auto dma = [&](int step) {
    const int st = min(step, nsteps - 1);
    uint8_t* base = lds + (step % D) * STAGE_B;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = 4 * wave + i;
      const uint8_t* src = arow[i >> 1] + (size_t)(st * PBK + Cd::boff(g4, i & 1)) * 2;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(base + f * 1024), 16, 0, 0);
    }
    uint8_t* wb = base + ACT_B + wave * (NT * PK * 1024);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int p = 0; p < PK; ++p)
        __builtin_amdgcn_global_load_lds((const void*)(fbase[t] + (size_t)(st * PK + p) * PACKET_BYTES),
                                         (lds_void*)(wb + (t * PK + p) * 1024), 16, 0, 0);
  };

  f32x4 acc[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < D - 1; ++s) dma(s);

  for (int step = 0; step < nsteps; ++step) {
    // this wave's loads of `step` have landed; after the barrier, every wave's have, and no
    // wave still reads the slot the next DMA overwrites (that of step - 1)
    MOE_WAIT_VMCNT((D - 2) * L);
    __builtin_amdgcn_s_barrier();
    dma(step + D - 1);
    const uint8_t* base = lds + (step % D) * STAGE_B;
    const uint8_t* wb = base + ACT_B + wave * (NT * PK * 1024) + lane * 16;
    float sc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
      sc[m] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scv[m]), (step * PBK) >> 7));
    bf16x8 af[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x4 pk[PK];
#pragma unroll
      for (int p = 0; p < PK; ++p) pk[p] = *(const u32x4*)(wb + (t * PK + p) * 1024);
      Cd::frags(pk, sc[t / WF], af[t]);
    }
    const uint8_t* ab = base + lane * 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16x8 b0 = *(const bf16x8*)(ab + (2 * j) * 1024);
      const bf16x8 b1 = *(const bf16x8*)(ab + (2 * j + 1) * 1024);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t][0], b0, acc[t][j], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t][1], b1, acc[t][j], 0, 0, 0);
    }
  }
  MOE_WAIT_VMCNT(0);  // the clamped tail DMAs must land before the workgroup's LDS is released

  // epilogue: lane holds features 4*(lane/16) + i of each 16-feature tile, row j*16 + lane%16
  uint8_t* out;
  int ldo;
  long long rowoff;
  if (a.out_s && row0 >= a.P) {
    out = (uint8_t*)a.out_s;
    ldo = a.ldo_s;
    rowoff = -(long long)a.P;
  } else {
    out = (uint8_t*)a.out;
    ldo = a.ldo;
    rowoff = 0;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rr = j * 16 + j16;
    if (rr >= nr) continue;
    const size_t row = (size_t)((long long)row0 + rr + rowoff);
#pragma unroll
    for (int f = 0; f < WF; ++f) {
      const int n = ftile[f] * 16 + 4 * g4;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = (EPI == EPI_SWIGLU) ? silu(acc[f][j][i]) * acc[WF + f][j][i] : acc[f][j][i];
      *(u32x2*)(out + (row * ldo + n) * 2) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

template <int C, int EPI>
static hipError_t launch_p(const GroupedArgs& a, int max_tiles, hipStream_t st) {
  GroupedArgs b = a;
  b.NTW = a.N / PEpi<EPI>::WGF;
  long long n = (long long)max_tiles * b.NTW;
  n = (n + NXCD - 1) / NXCD * NXCD;
  if (n == 0) return hipSuccess;
  grouped_prefill_kernel<C, EPI><<<(unsigned)n, 256, 0, st>>>(b);
  return hipGetLastError();
}

int prefill_row_tile() { return PBM; }

bool prefill_supported(int act, int cr, int cs, int K, int N_gateup, int N_down) {
  auto ok = [](int c) { return c == MOE_BF16 || c == MOE_FP8_E4M3_B128; };
  return act == MOE_BF16 && ok(cr) && cr == cs && K % PBK == 0 && K <= 64 * 128 &&
         N_gateup % PEpi<EPI_SWIGLU>::WGF == 0 &&
         N_down % PEpi<EPI_PLAIN>::WGF == 0;
}

hipError_t launch_grouped_prefill(int act, int epi, int cr, int cs, const GroupedArgs& a, int max_tiles,
                                  hipStream_t st) {
  if (act != MOE_BF16 || cr != cs || a.K % PBK != 0) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU) {
    if (a.N % PEpi<EPI_SWIGLU>::WGF) return hipErrorInvalidValue;
    if (cr == MOE_BF16) return launch_p<MOE_BF16, EPI_SWIGLU>(a, max_tiles, st);
    if (cr == MOE_FP8_E4M3_B128) return launch_p<MOE_FP8_E4M3_B128, EPI_SWIGLU>(a, max_tiles, st);
  } else if (epi == EPI_PLAIN) {
    if (a.N % PEpi<EPI_PLAIN>::WGF) return hipErrorInvalidValue;
    if (cr == MOE_BF16) return launch_p<MOE_BF16, EPI_PLAIN>(a, max_tiles, st);
    if (cr == MOE_FP8_E4M3_B128) return launch_p<MOE_FP8_E4M3_B128, EPI_PLAIN>(a, max_tiles, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
