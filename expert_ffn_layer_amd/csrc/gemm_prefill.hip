// Prefill-regime grouped GEMM: many rows per expert, bound by the matrix cores.
//
// Work item = (group, tile of BM = 128 rows, tile of output features). The four waves of a
// workgroup split the features (64 each: 32 gate + 32 up columns for the SwiGLU GEMM, 64 for the
// plain one) and share the 128-row activation tile, which is staged in LDS (double-buffered
// over reduction steps of 64, rows padded to 144 bytes so the 16x16 fragment reads are free of
// bank conflicts). The weights stream from global memory straight into each wave's registers in
// the packet layout (one 128-bit load per lane per packet), so every weight byte is converted
// to bf16 exactly once per workgroup, and feed v_mfma_f32_16x16x32_bf16 as the A operand; the
// activations are the B operand. fp8 packets are converted in registers (e4m3 -> fp32 exact,
// times the 128 x 128 block scale, -> bf16).
//
// Items are ordered so that a run of consecutive items covers up to 8 feature tiles x all row
// tiles of one group, and the workgroup -> item map gives each XCD a contiguous run of items:
// workgroups resident at the same time on one XCD then share weight and activation slices in
// that XCD's L2 (Chapter 6 'Supernodes' section 6.3.2: one weight read serves many rows).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PBM = 128;           // rows per item
constexpr int PBK = 64;            // reduction elements per step
constexpr int PWN = 64;            // output features per wave (4 tiles of 16)
constexpr int LDS_ROW = PBK + 8;   // bf16 elements per LDS row (144 bytes)
constexpr int NXCD = 8;

template <int C>
struct PCodec;

template <>
struct PCodec<MOE_BF16> {
  static constexpr int PK = 2;  // packets per feature tile per step
  // byte offset in an LDS row of the B fragment of half h for lane group g
  __device__ static int boff(int g, int h) { return 16 * g + 64 * h; }
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
  __device__ static int boff(int g, int h) { return 32 * g + 16 * h; }
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

template <int C, int EPI>
__global__ void __launch_bounds__(256, 1) grouped_prefill_kernel(GroupedArgs a) {
  using Cd = PCodec<C>;
  constexpr int NMAT = PEpi<EPI>::NMAT;
  constexpr int WF = PEpi<EPI>::WF;
  constexpr int NT = NMAT * WF;  // 16-feature tiles per wave (4)
  constexpr int PK = Cd::PK;
  constexpr int KP = PBK / PK;   // reduction elements per packet
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][PBM * LDS_ROW];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ntn = a.NTW;  // feature tiles of the workgroup width
  // XCD-aware workgroup -> item map: each XCD takes a contiguous run of the item list
  const int per_xcd = gridDim.x / NXCD;
  const int item = (blockIdx.x % NXCD) * per_xcd + blockIdx.x / NXCD;
  const int total = a.cum_blocks[a.G] * ntn;
  if (item >= total) return;
  // group of the item: largest g with cum_blocks[g] * ntn <= item
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
  const int KT = a.K / KP;  // packets along K
  const int nsteps = a.K / PBK;

  // this wave's 16-feature tiles: matrix m, tile index (in units of 16 features)
  int ftile[NT];
  const uint8_t* fbase[NT];
  const float* fscale[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int m = t / WF, f = t % WF;
    ftile[t] = (ntile * 4 + wave) * WF + f;
    fbase[t] = (m == 0 ? w0 : w1) + (size_t)ftile[t] * KT * PACKET_BYTES + (size_t)lane * 16;
    fscale[t] = m == 0 ? s0 : s1;
  }

  // activation rows this thread stages: rows r = tid/8 + 32 i, 16-byte chunk c = tid % 8
  const int c8 = tid & 7;
  const uint8_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (tid >> 3) + 32 * i;
    const int r = row0 + (rr < nr ? rr : 0);
    int src = a.gather ? (r < a.P ? a.gather[r] : r - a.P) : r;
    if ((unsigned)src >= (unsigned)a.act_rows) src = 0;
    arow[i] = (const uint8_t*)a.act + ((size_t)src * a.lda + c8 * 8) * 2;
  }

  f32x4 acc[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 xa[4];  // staged activation chunks of the next step
  // weight packets and scales of two consecutive steps (slot 0: even steps, slot 1: odd steps;
  // static indices keep them in registers and the wait counts exact)
  u32x4 wv0[NT][PK], wv1[NT][PK];
  float sv0[NT], sv1[NT];

  auto load_x = [&](int step) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xa[i] = *(const u32x4*)(arow[i] + (size_t)step * PBK * 2);
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = (tid >> 3) + 32 * i;
      *(u32x4*)((uint8_t*)lds[buf] + rr * (LDS_ROW * 2) + c8 * 16) = xa[i];
    }
  };
  auto load_w = [&](int step, u32x4 (&wv)[NT][PK], float (&sv)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int p = 0; p < PK; ++p)
        wv[t][p] = ld_nt((const u32x4*)(fbase[t] + (size_t)(step * PK + p) * PACKET_BYTES));
      if (C == MOE_FP8_E4M3_B128) {
        const int kb = (step * PBK + (lane >> 4) * 16) >> 7;
        sv[t] = fscale[t][kb * (a.N >> 7) + (ftile[t] >> 3)];
      } else {
        sv[t] = 1.0f;
      }
    }
  };
  const int j16 = lane & 15, g4 = lane >> 4;
  // one reduction step on LDS buffer `buf` with weights (wv, sv), prefetching the next step
  auto step_body = [&](int step, int buf, u32x4 (&wv)[NT][PK], float (&sv)[NT], u32x4 (&wn)[NT][PK],
                       float (&sn)[NT]) {
    // unconditional prefetch (the last step re-reads itself) keeps the wait counts exact
    const int nxt = min(step + 1, nsteps - 1);
    load_x(nxt);
    load_w(nxt, wn, sn);
    // keep the prefetch at the top of the step: the scheduler would otherwise sink it behind
    // the MFMAs, and the next step would stall on it
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 af[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) Cd::frags(wv[t], sv[t], af[t]);
    const uint8_t* lb = (const uint8_t*)lds[buf];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint8_t* rowp = lb + (j * 16 + j16) * (LDS_ROW * 2);
      const bf16x8 b0 = *(const bf16x8*)(rowp + Cd::boff(g4, 0));
      const bf16x8 b1 = *(const bf16x8*)(rowp + Cd::boff(g4, 1));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t][0], b0, acc[t][j], 0, 0, 0);
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t][1], b1, acc[t][j], 0, 0, 0);
      }
    }
    store_x(buf ^ 1);
    __syncthreads();
  };

  // prologue
  load_x(0);
  load_w(0, wv0, sv0);
  store_x(0);
  __syncthreads();
  for (int step = 0; step < nsteps; step += 2) {
    step_body(step, 0, wv0, sv0, wv1, sv1);
    if (step + 1 < nsteps) step_body(step + 1, 1, wv1, sv1, wv0, sv0);
  }

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
  return act == MOE_BF16 && ok(cr) && cr == cs && K % PBK == 0 && N_gateup % PEpi<EPI_SWIGLU>::WGF == 0 &&
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
