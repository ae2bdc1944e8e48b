// Decode-regime grouped GEMM: few rows per expert, bound by streaming the expert weights.
//
// Work item = (group, block of up to 64 rows of that group, tile of 16*NF output features).
// The weights are the MFMA A operand (16 features x KP reduction elements per 1 KiB packet, one
// 128-bit load per lane), the gathered activations the B operand (16 rows), so one
// v_mfma_f32_16x16x32_bf16 (or 16x16x4_f32) consumes a packet with no data shuffles. The four
// waves of a workgroup split the reduction into contiguous parts and, for f32/bf16, each wave
// runs all 1, 2 or 4 row tiles of the block, so every weight packet is loaded once per item
// and feeds one MFMA per row tile (the converted formats split thick blocks' rows over the
// waves instead); the fp32 partial sums are added in LDS in a fixed order. Each selected
// expert's weights are therefore streamed once per block of 64 rows (the within-batch reuse of
// Chapter 6 'Supernodes', section 6.3.2).
//
// Epilogues: SwiGLU (gate and up tiles of the same features, h = SiLU(g) * u,
// Chapter 6 section 6.2.2), plain store in the activation type, or plain fp32 store (router
// scores).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int RB = 64;  // rows per work item

template <int C>
struct Codec;

template <>
struct Codec<MOE_F32> {
  static constexpr int KP = 16, ACT16 = 1;  // activation 16-byte chunks per packet per lane
  static constexpr bool A8 = false;         // MXFP8 activations on the block-scaled MFMA
  static constexpr int WPK = 1;             // 1 KiB weight packets per reduction step
  static constexpr bool I8 = false;         // int8 x int8 with int32 sums, scaled per row and feature
  __device__ static void mma(const u32x4& w, const u32x4* x, float, f32x4& acc) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w[s]), __uint_as_float(x[0][s]), acc, 0, 0, 0);
  }
};

template <>
struct Codec<MOE_BF16> {
  static constexpr int KP = 32, ACT16 = 1;
  static constexpr bool A8 = false;
  static constexpr int WPK = 1;
  static constexpr bool I8 = false;
  __device__ static void mma(const u32x4& w, const u32x4* x, float, f32x4& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                  __builtin_bit_cast(bf16x8, x[0]), acc, 0, 0, 0);
  }
};

// e4m3fn codes -> fp32 (exact, v_cvt_pk_f32_fp8 reads OCP E4M3FN on gfx950) -> * block scale
// -> bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1, float s) {
  typedef __attribute__((ext_vector_type(2))) float f2;
  f2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
  f2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
  f2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
  f2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
  u32x4 r;
  r[0] = pack_bf16x2(a.x * s, a.y * s);
  r[1] = pack_bf16x2(b.x * s, b.y * s);
  r[2] = pack_bf16x2(c.x * s, c.y * s);
  r[3] = pack_bf16x2(d.x * s, d.y * s);
  return __builtin_bit_cast(bf16x8, r);
}

template <>
struct Codec<MOE_FP8_E4M3_B128> {
  static constexpr int KP = 64, ACT16 = 2;
  static constexpr bool A8 = false;
  static constexpr int WPK = 1;
  static constexpr bool I8 = false;
  __device__ static void mma(const u32x4& w, const u32x4* x, float s, f32x4& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w[0], w[1], s),
                                                  __builtin_bit_cast(bf16x8, x[0]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w[2], w[3], s),
                                                  __builtin_bit_cast(bf16x8, x[1]), acc, 0, 0, 0);
  }
};

// 8 e2m1 codes (one dword, element 2b in the low nibble of byte b) -> 8 bf16, times 2^(E-127).
// v_cvt_scalef32_pk_bf16_fp4 is exact here and applies the exponent of `scale`.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return __builtin_bit_cast(bf16x8, r);
}

template <>
struct Codec<MOE_MXFP4_B32> {
  static constexpr int KP = 128, ACT16 = 4;
  static constexpr bool A8 = false;
  static constexpr int WPK = 1;
  static constexpr bool I8 = false;
  __device__ static void mma(const u32x4& w, const u32x4* x, float s, f32x4& acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16(w[i], s),
                                                    __builtin_bit_cast(bf16x8, x[i]), acc, 0, 0, 0);
  }
};

// W4A8: an MXFP4 packet is the fp4 A operand of v_mfma_scale_f32_16x16x128_f8f6f4 as stored (lane
// (f, g): 32 codes of feature f, elements 32g .. 32g + 31, in operand dwords 0-3, with the lane's
// e8m0 byte as its scale). The B operand is the token's MXFP8 row: lane (j, g) holds elements
// 16g .. + 15 and 64 + 16g .. + 15 of the packet's 128 (two 16-byte chunks, 64 bytes apart), and
// its scale byte is the exponent of (token j, block g). One MFMA per packet and row tile.
template <>
struct Codec<MOE_MXFP4_B32_A8> {
  static constexpr int KP = 128, ACT16 = 2;
  static constexpr bool A8 = true;
  static constexpr int WPK = 1;
  static constexpr bool I8 = false;
  __device__ static void mma8(const u32x4* w, const u32x4* x, int sw, int sx, f32x4& acc) {
    const i32x8 a = {(int)w[0][0], (int)w[0][1], (int)w[0][2], (int)w[0][3], 0, 0, 0, 0};
    const i32x8 b = {(int)x[0][0], (int)x[0][1], (int)x[0][2], (int)x[0][3],
                     (int)x[1][0], (int)x[1][1], (int)x[1][2], (int)x[1][3]};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 0, 0, sw, 0, sx);
  }
  __device__ static void mma(const u32x4&, const u32x4*, float, f32x4&) {}  // not reached (mma8)
};

// W8A8 MXFP8 (the shared expert of the hybrid scheme): the same instruction with fp8 A. Measured on
// the hardware, fp8 A takes the fp8 B layout, so the step's two fp8 packets (elements 0..63 and
// 64..127, lane (f, g) holding run 16g of each) are the operand as stored, and the packed
// exponents (one byte per lane per packet pair, at the MXFP4 scale layout's place) its scales.
template <>
struct Codec<MOE_MXFP8_B32_A8> {
  static constexpr int KP = 128, ACT16 = 2;
  static constexpr bool A8 = true;
  static constexpr int WPK = 2;
  static constexpr bool I8 = false;
  __device__ static void mma8(const u32x4* w, const u32x4* x, int sw, int sx, f32x4& acc) {
    const i32x8 a = {(int)w[0][0], (int)w[0][1], (int)w[0][2], (int)w[0][3],
                     (int)w[1][0], (int)w[1][1], (int)w[1][2], (int)w[1][3]};
    const i32x8 b = {(int)x[0][0], (int)x[0][1], (int)x[0][2], (int)x[0][3],
                     (int)x[1][0], (int)x[1][1], (int)x[1][2], (int)x[1][3]};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, sw, 0, sx);
  }
  __device__ static void mma(const u32x4&, const u32x4*, float, f32x4&) {}  // not reached (mma8)
};

// Int8 W8A8: an int8 packet (16 features x 64, laid out as an fp8 packet) and the gathered int8 token
// rows (lane (j, g): 16 bytes of token j, run 16g of the packet's 64) go to v_mfma_i32_16x16x64_i8,
// whose A and B operands share that lane layout, so the codes' products add exactly in int32. The
// sums are scaled by the row's activation scale and the feature's weight scale after the wave's
// reduction range, before the partial sums of the waves are added.
template <>
struct Codec<MOE_INT8_W8A8> {
  static constexpr int KP = 64, ACT16 = 1;
  static constexpr bool A8 = false;
  static constexpr int WPK = 1;
  static constexpr bool I8 = true;
  __device__ static void mma(const u32x4& w, const u32x4* x, float, f32x4& acc) {
    acc = __builtin_bit_cast(f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, w),
                                                                          __builtin_bit_cast(i32x4, x[0]),
                                                                          __builtin_bit_cast(i32x4, acc), 0, 0, 0));
  }
};

// Scale of the lane's packet (nt, kt).
template <int C>
__device__ __forceinline__ float packet_scale(const uint8_t* sc, int N, int KT, int nt, int kt, int lane) {
  if (C == MOE_FP8_E4M3_B128) {
    const int kb = (kt * 64 + (lane >> 4) * 16) >> 7;
    return ((const float*)sc)[kb * (N >> 7) + (nt >> 3)];
  } else if (C == MOE_MXFP4_B32) {
    const uint32_t E = sc[((size_t)nt * KT + kt) * 64 + lane];
    return __uint_as_float(E << 23);
  } else if (C == MOE_MXFP4_B32_A8 || C == MOE_MXFP8_B32_A8) {
    return __int_as_float((int)sc[((size_t)nt * KT + kt) * 64 + lane]);  // the raw e8m0 byte
  }
  return 1.0f;
}

template <int EPI>
struct EpiTraits {
  static constexpr int NMAT = EPI == EPI_SWIGLU ? 2 : 1;
};

// Registers of one pipeline stage: U consecutive packets of each of the NMAT x NF streams,
// the matching activation chunks of the MT row tiles and the packets' scales.
template <int C, int NMAT, int NF, int MT, int U>
struct Stage {
  u32x4 x[U][MT][Codec<C>::ACT16];
  u32x4 w[U][NMAT][NF][Codec<C>::WPK];
  float s[U][NMAT][NF];
  int xs[U][MT];  // W4A8: the lane's activation exponent byte per packet and row tile
};

// Issue the loads of packets kt .. kt+U-1 (indices past kt1-1 re-read packet kt1-1 and are
// not used, so every address stays inside the stream). NTL: weights as non-temporal loads (read
// by this wave only); otherwise plain loads, which the other row groups of the item hit in cache.
template <int C, int ACT, int NMAT, int NF, int MT, int U, bool NTL>
__device__ __forceinline__ void load_stage(Stage<C, NMAT, NF, MT, U>& st, const uint8_t* __restrict__ w0,
                                           const uint8_t* __restrict__ w1, const uint8_t* __restrict__ s0,
                                           const uint8_t* __restrict__ s1, const uint8_t* const (&xrow)[MT],
                                           const uint8_t* const (&xsrow)[MT], int N, int KT, int nt0, int kt,
                                           int kt1, int lane) {
  using Cd = Codec<C>;
  constexpr int AB = (Cd::A8 || Cd::I8) ? 1 : (ACT == MOE_F32 ? 4 : 2);
  constexpr int CHS = Cd::A8 ? 64 : 16;  // bytes between a lane's activation chunks
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = min(kt + u, kt1 - 1);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
      for (int p = 0; p < Cd::WPK; ++p) {
        // WPK consecutive 1 KiB packets per step (the fp8 pair of a 128-deep MXFP8 step)
        const size_t off = (((size_t)(nt0 + f) * KT + k) * Cd::WPK + p) * PACKET_BYTES + (size_t)lane * 16;
        if constexpr (NTL) {
          st.w[u][0][f][p] = ld_nt((const u32x4*)(w0 + off));
          if (NMAT == 2) st.w[u][NMAT - 1][f][p] = ld_nt((const u32x4*)(w1 + off));
        } else {
          st.w[u][0][f][p] = *(const u32x4*)(w0 + off);
          if (NMAT == 2) st.w[u][NMAT - 1][f][p] = *(const u32x4*)(w1 + off);
        }
      }
      st.s[u][0][f] = packet_scale<C>(s0, N, KT, nt0 + f, k, lane);
      if (NMAT == 2) st.s[u][NMAT - 1][f] = packet_scale<C>(s1, N, KT, nt0 + f, k, lane);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int i = 0; i < Cd::ACT16; ++i)
        st.x[u][m][i] = *(const u32x4*)(xrow[m] + (size_t)k * Cd::KP * AB + i * CHS);
      if constexpr (Cd::A8) st.xs[u][m] = xsrow[m][k * 4];
    }
  }
}

template <int C, int NMAT, int NF, int MT, int U>
__device__ __forceinline__ void mma_stage(const Stage<C, NMAT, NF, MT, U>& st, f32x4 (&acc)[MT][NMAT][NF]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          if constexpr (Codec<C>::A8)
            Codec<C>::mma8(st.w[u][m][f], st.x[u][r], __float_as_int(st.s[u][m][f]), st.xs[u][r], acc[r][m][f]);
          else
            Codec<C>::mma(st.w[u][m][f][0], st.x[u][r], st.s[u][m][f], acc[r][m][f]);
        }
}

// The same with the weight operand of packets kt + u >= kt1 replaced by zero codes (which
// decode to 0 in every format), so the MFMAs stay unconditional: no branches around them.
template <int C, int NMAT, int NF, int MT, int U>
__device__ __forceinline__ void mma_stage_masked(const Stage<C, NMAT, NF, MT, U>& st, int kt, int kt1,
                                                 f32x4 (&acc)[MT][NMAT][NF]) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const u32x4 zeros[2] = {zero, zero};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool valid = kt + u < kt1;
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          if constexpr (Codec<C>::A8)
            Codec<C>::mma8(valid ? st.w[u][m][f] : zeros, st.x[u][r], __float_as_int(st.s[u][m][f]), st.xs[u][r],
                           acc[r][m][f]);
          else
            Codec<C>::mma(valid ? st.w[u][m][f][0] : zero, st.x[u][r], st.s[u][m][f], acc[r][m][f]);
        }
  }
}

// Packets per pipeline stage along K, chosen so a stage keeps about 8 weight packets (4 for the
// formats converted in registers, whose temporaries would otherwise cost occupancy) and at most
// 8 activation chunks per lane in flight (4 with several row tiles, whose accumulators and
// activation chunks would otherwise raise the register count of the whole kernel and cost the
// thin items occupancy).
template <int C, int NMAT, int NF, int MT>
constexpr int stage_depth() {
  constexpr int per_stage = (C == MOE_BF16 || C == MOE_F32) ? 8 : 4;
  constexpr int a = per_stage / (NF * NMAT), b = (MT == 1 ? 8 : 4) / (Codec<C>::ACT16 * MT);
  constexpr int u = a < b ? a : b;
  return u < 1 ? 1 : u;
}

// One wave: MT row tiles of 16 rows x (16*NF) features of NMAT matrices over packets
// [kt0, kt1), with the loads of the next stage in flight while the current stage feeds the
// MFMAs. Every weight packet the wave loads feeds all MT row tiles.
template <int C, int ACT, int NMAT, int NF, int MT, bool NTL>
__device__ __forceinline__ void wave_mma(const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                         const uint8_t* __restrict__ s0, const uint8_t* __restrict__ s1,
                                         const uint8_t* const (&xrow)[MT], const uint8_t* const (&xsrow)[MT], int N,
                                         int KT, int nt0, int kt0, int kt1, int lane, f32x4 (&acc)[MT][NMAT][NF]) {
  constexpr int U = stage_depth<C, NMAT, NF, MT>();
  if (kt0 >= kt1) return;
  Stage<C, NMAT, NF, MT, U> A, B;
  load_stage<C, ACT, NMAT, NF, MT, U, NTL>(A, w0, w1, s0, s1, xrow, xsrow, N, KT, nt0, kt0, kt1, lane);
  int kt = kt0;
  // steady state: both stages entirely inside the range, so every load and MFMA is
  // unconditional and the wait counts stay exact (the next stage's loads remain in flight)
  for (; kt + 2 * U < kt1; kt += 2 * U) {
    load_stage<C, ACT, NMAT, NF, MT, U, NTL>(B, w0, w1, s0, s1, xrow, xsrow, N, KT, nt0, kt + U, kt1, lane);
    mma_stage(A, acc);
    load_stage<C, ACT, NMAT, NF, MT, U, NTL>(A, w0, w1, s0, s1, xrow, xsrow, N, KT, nt0, kt + 2 * U, kt1, lane);
    mma_stage(B, acc);
  }
  // remainder (1 .. 2U packets), branch-free: packets past the range are masked to zero
  load_stage<C, ACT, NMAT, NF, MT, U, NTL>(B, w0, w1, s0, s1, xrow, xsrow, N, KT, nt0, kt + U, kt1, lane);
  mma_stage_masked(A, kt, kt1, acc);
  mma_stage_masked(B, kt + U, kt1, acc);
}

// One work item: rows row0 .. row0 + nr - 1 (nr <= 16 * MT * MTP) of group g, features
// ntw * 16 * NF .. + 16 * NF. The four waves form MTP row groups of MT row tiles each and split
// the reduction into KS = 4 / MTP contiguous parts (wave = row group + MTP * part); a wave runs
// all MT row tiles of its group, so within a row group every weight byte is loaded once and
// feeds MT MFMAs. The KS partial sums of row tile r are added in LDS in ascending part order by
// the wave of part r % KS, which then writes the row tile: the result does not depend on
// scheduling.
template <int C, int ACT, int EPI, int NF, int MT, int MTP>
__device__ __forceinline__ void run_item(const GroupedArgs& a, int g, bool is_shared, int row0, int nr, int ntw,
                                         float* red) {
  constexpr int NMAT = EpiTraits<EPI>::NMAT;
  constexpr int KP = Codec<C>::KP;
  constexpr int NREG = NMAT * NF * 4;
  constexpr int KS = 4 / MTP;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int msub = wave % MTP, kpart = wave / MTP;
  const int KT = a.K / KP;
  // reduction range of this workgroup (split-K across workgroups for fp32 partial outputs), then
  // of this wave
  const int KSG = a.ksplit > 1 ? a.ksplit : 1;
  const int ktA = blockIdx.y * KT / KSG, ktB = (blockIdx.y + 1) * KT / KSG;
  const int kt0 = ktA + kpart * (ktB - ktA) / KS, kt1 = ktA + (kpart + 1) * (ktB - ktA) / KS;
  const int nt0 = ntw * NF;
  const int wrow0 = row0 + 16 * MT * msub;  // first row of this wave's row group
  const int wnr = nr - 16 * MT * msub;      // rows of the group (may be <= 0)

  // operand pointers
  const uint8_t* w0 = is_shared ? a.wa_s : a.wa_r + (size_t)g * a.mat_bytes;
  const uint8_t* w1 = is_shared ? a.wb_s : (a.wb_r ? a.wb_r + (size_t)g * a.mat_bytes : nullptr);
  const uint8_t* s0 = is_shared ? a.sa_s : (a.sa_r ? a.sa_r + (size_t)g * a.scale_bytes : nullptr);
  const uint8_t* s1 = is_shared ? a.sb_s : (a.sb_r ? a.sb_r + (size_t)g * a.scale_bytes : nullptr);

  const int rl = lane & 15;
  constexpr int AB = ACT == MOE_F32 ? 4 : 2;
  const uint8_t* xrow[MT];
  const uint8_t* xsrow[MT];  // W4A8: the row's exponent of block (lane / 16) of packet 0
  int srcs[MT];              // Int8: the activation row of each row tile (its scale index)
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int rr = 16 * m + rl;
    const int r = rr < wnr ? wrow0 + rr : row0;
    int src = a.gather ? (r < a.P ? a.gather[r] : r - a.P) : r;
    if ((unsigned)src >= (unsigned)a.act_rows) src = 0;
    srcs[m] = src;
    if constexpr (Codec<C>::I8) {
      // int8 rows of K bytes: the lane's chunk starts at byte 16 (lane / 16) of each 64-byte packet
      xrow[m] = (const uint8_t*)a.act + (size_t)src * a.lda + 16 * (lane >> 4);
      xsrow[m] = nullptr;
    } else if constexpr (Codec<C>::A8) {
      // MXFP8 rows of K bytes: the lane's chunks start at byte 16 (lane / 16) of each packet's 128
      xrow[m] = (const uint8_t*)a.act + (size_t)src * a.lda + 16 * (lane >> 4);
      xsrow[m] = (const uint8_t*)a.act_scale + (size_t)src * (a.K / 32) + (lane >> 4);
    } else {
      xrow[m] = (const uint8_t*)a.act + ((size_t)src * a.lda + (lane >> 4) * (KP / 4)) * AB;
      xsrow[m] = nullptr;
    }
  }

  f32x4 acc[MT][NMAT][NF];
#pragma unroll
  for (int r = 0; r < MT; ++r)
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[r][m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (wnr > 0)
    wave_mma<C, ACT, NMAT, NF, MT, MTP == 1>(w0, w1, s0, s1, xrow, xsrow, a.N, KT, nt0, kt0, kt1, lane, acc);

  if constexpr (Codec<C>::I8) {
    // int32 sums -> fp32 times the row's activation scale and the feature's weight scale (features
    // (nt0 + f) * 16 + 4 (lane / 16) + i of token row 16 r + lane % 16); the whole register
    // vector is reinterpreted (a bit cast of one vector element reads element 0)
    const float* asc = (const float*)a.act_scale;
#pragma unroll
    for (int r = 0; r < MT; ++r) {
      const float rs = asc[srcs[r]];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const f32x4 cs = *(const f32x4*)((const float*)(m == 0 ? s0 : s1) + (nt0 + f) * 16 + 4 * (lane >> 4));
          const i32x4 iv = __builtin_bit_cast(i32x4, acc[r][m][f]);
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (float)iv[i] * rs * cs[i];
          acc[r][m][f] = v;
        }
    }
  }

  // fixed-order reduction of the KS reduction parts, one row tile per round
  if constexpr (KS > 1) {
#pragma unroll
    for (int r = 0; r < MT; ++r) {
      const int owner = r % KS;
      if (kpart != owner) {
        const int slot = msub * (KS - 1) + (kpart < owner ? kpart : kpart - 1);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(slot * NREG + (m * NF + f) * 4 + i) * 64 + lane] = acc[r][m][f][i];
      }
      __syncthreads();
      if (kpart == owner) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float sum = 0.0f;
#pragma unroll
              for (int p = 0; p < KS; ++p) {
                const int slot = msub * (KS - 1) + (p < owner ? p : p - 1);
                sum += p == owner ? acc[r][m][f][i] : red[(slot * NREG + (m * NF + f) * 4 + i) * 64 + lane];
              }
              acc[r][m][f][i] = sum;
            }
      }
      __syncthreads();
    }
  }

  // epilogue: the owner of row tile r writes it; lane holds features
  // n = (nt0+f)*16 + 4*(lane/16) + i of row wrow0 + 16r + rl
#pragma unroll
  for (int r = 0; r < MT; ++r) {
    if (r % KS != kpart || 16 * r + rl >= wnr) continue;
    const int orow = wrow0 + 16 * r + rl;
    uint8_t* out;
    int ldo;
    size_t row;
    if (a.out_s && orow >= a.P) {
      out = (uint8_t*)a.out_s;
      ldo = a.ldo_s;
      row = (size_t)(orow - a.P);
    } else {
      out = (uint8_t*)a.out;
      ldo = a.ldo;
      row = (size_t)orow + (size_t)blockIdx.y * a.M;  // split-K part y of an fp32 output
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = (nt0 + f) * 16 + 4 * (lane >> 4);
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = (EPI == EPI_SWIGLU) ? silu(acc[r][0][f][i]) * acc[r][NMAT - 1][f][i] : acc[r][0][f][i];
      if (EPI == EPI_F32 || ACT == MOE_F32) {
        *(f32x4*)(out + (row * ldo + n) * 4) = f32x4{v[0], v[1], v[2], v[3]};
      } else {
        *(u32x2*)(out + (row * ldo + n) * 2) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

// Row layout of an item of up to 64 rows by its row count: 1, 2 or 4 row tiles, split into MTP row
// groups of MT tiles. Formats with one 16-byte activation chunk per packet (f32, bf16, int8) give each wave as
// many row tiles as 64 accumulator registers allow, so a packet is loaded once per row group
// and feeds MT MFMAs. The converted formats, whose activation chunks per packet are 2x-4x
// larger, split the rows over the waves (each row group loads the packets of its part of K).
// Both keep the kernel's register count, and so the occupancy of the thin items, near that of
// the one-row-tile path. LEAN (the shared expert's path in a kernel whose routed experts use
// another format) always splits rows, so the rarely used path does not set the register count.
template <int C, int ACT, int EPI, int NF, bool LEAN>
constexpr int max_row_tiles() {
  constexpr int ACC = EpiTraits<EPI>::NMAT * NF * 4;  // accumulator registers per row tile
  return (LEAN || Codec<C>::ACT16 != 1) ? 1 : (4 * ACC <= 64 ? 4 : (2 * ACC <= 64 ? 2 : 1));
}

template <int C, int ACT, int EPI, int NF, bool LEAN>
__device__ __forceinline__ void run_rows64(const GroupedArgs& a, int g, bool is_shared, int row0, int nr, int ntw,
                                           float* red) {
  constexpr int MTMAX = max_row_tiles<C, ACT, EPI, NF, LEAN>();
  if (nr <= 16) {
    run_item<C, ACT, EPI, NF, 1, 1>(a, g, is_shared, row0, nr, ntw, red);
  } else if (nr <= 32) {
    if constexpr (MTMAX >= 2) run_item<C, ACT, EPI, NF, 2, 1>(a, g, is_shared, row0, nr, ntw, red);
    else run_item<C, ACT, EPI, NF, 1, 2>(a, g, is_shared, row0, nr, ntw, red);
  } else {
    if constexpr (MTMAX >= 4) run_item<C, ACT, EPI, NF, 4, 1>(a, g, is_shared, row0, nr, ntw, red);
    else if constexpr (MTMAX == 2) run_item<C, ACT, EPI, NF, 2, 2>(a, g, is_shared, row0, nr, ntw, red);
    else run_item<C, ACT, EPI, NF, 1, 4>(a, g, is_shared, row0, nr, ntw, red);
  }
}

// An item of nr rows: up to 64 (one block), or a thick block of a group of more than 64 rows (up to
// 4 x 64 rows), where wave w runs rows 64 w .. 64 w + 63 over the whole reduction: the four waves read
// each weight packet at about the same time, so HBM delivers it once per item instead of once per
// 64 rows. Thick blocks exist only in the SwiGLU kernels with 4 row tiles per wave and one format for
// routed and shared experts (the launcher refuses thick_rows for any other).
template <int C, int ACT, int EPI, int NF, bool LEAN>
__device__ __forceinline__ void run_rows(const GroupedArgs& a, int g, bool is_shared, int row0, int nr, int ntw,
                                         float* red) {
  if constexpr (EPI == EPI_SWIGLU && max_row_tiles<C, ACT, EPI, NF, LEAN>() >= 4) {
    if (nr <= RB) run_rows64<C, ACT, EPI, NF, LEAN>(a, g, is_shared, row0, nr, ntw, red);
    else run_item<C, ACT, EPI, NF, 4, 4>(a, g, is_shared, row0, nr, ntw, red);
  } else {
    run_rows64<C, ACT, EPI, NF, LEAN>(a, g, is_shared, row0, nr, ntw, red);
  }
}

template <int CR, int CS, int ACT, int EPI, int NF>
__global__ void __launch_bounds__(256) grouped_decode_kernel(GroupedArgs a) {
  constexpr int NMAT = EpiTraits<EPI>::NMAT;
  __shared__ float red[3 * NMAT * NF * 4 * 64];
  // (the router-score instantiation only: a store the compiler cannot place apart from the plan
  // arrays would turn the other kernels' uniform plan loads into vector loads)
  if constexpr (EPI == EPI_F32)
    if (a.clear_word && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.clear_word = 0u;
  int rbi = blockIdx.x / a.NTW;
  const int ntw = blockIdx.x % a.NTW;
  if (a.cum_blocks && a.g_end > a.g_begin) {
    // a launch over groups [g_begin, g_end) only: its row blocks follow those of earlier groups
    rbi += a.cum_blocks[a.g_begin];
    if (rbi >= a.cum_blocks[a.g_end]) return;
  }
  int g = 0, blk = rbi;
  if (a.cum_blocks) {
    if (rbi >= a.cum_blocks[a.G]) return;
    if (a.block_group) {
      // one load: group and block within it
      const int gb = a.block_group[rbi];
      g = gb >> 16;
      blk = gb & 0xFFFF;
    } else {
      int lo = 0, hi = a.G - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cum_blocks[mid] <= rbi) lo = mid; else hi = mid - 1;
      }
      g = lo;
      blk = rbi - a.cum_blocks[g];
    }
  } else if (rbi * RB >= a.M) {
    return;
  }
  const int rbeg = a.group_range ? a.group_range[2 * g] : 0;
  const int rend = a.group_range ? a.group_range[2 * g + 1] : a.M;
  // rows per block: 64, or thick_rows for a group of more than 64 rows when the plan cut it so
  const int rbg = (a.thick_rows > RB && rend - rbeg > RB) ? min(a.thick_rows, 4 * RB) : RB;
  const int row0 = rbeg + rbg * blk;
  const int nr = min(rbg, rend - row0);
  if (nr <= 0) return;
  const bool is_shared = g == a.shared_group;
  if (CR == CS || !is_shared)
    run_rows<CR, ACT, EPI, NF, false>(a, g, is_shared, row0, nr, ntw, red);
  else
    run_rows<CS, ACT, EPI, NF, true>(a, g, is_shared, row0, nr, ntw, red);
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------

template <int CR, int CS, int ACT, int EPI, int NF>
static hipError_t launch_t(const GroupedArgs& a, int max_row_blocks, hipStream_t st) {
  // thick blocks: the SwiGLU kernels with 4 row tiles per wave in every path
  if (a.thick_rows && (EPI != EPI_SWIGLU || a.thick_rows > 4 * RB || max_row_tiles<CR, ACT, EPI, NF, false>() < 4 ||
                       (CR != CS && a.shared_group >= 0)))
    return hipErrorInvalidValue;
  GroupedArgs b = a;
  b.NTW = (a.N / 16) / NF;
  dim3 grid((unsigned)(max_row_blocks * b.NTW), (unsigned)(a.ksplit > 1 ? a.ksplit : 1)), block(256);
  if (grid.x == 0) return hipSuccess;
  grouped_decode_kernel<CR, CS, ACT, EPI, NF><<<grid, block, 0, st>>>(b);
  return hipGetLastError();
}

template <int CR, int CS, int ACT, int EPI>
static hipError_t launch_nf(int nf, const GroupedArgs& a, int mrb, hipStream_t st) {
  if constexpr (EPI == EPI_F32) {
    return launch_t<CR, CS, ACT, EPI, 1>(a, mrb, st);
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (nf == 1) return launch_t<CR, CS, ACT, EPI, 1>(a, mrb, st);
    return launch_t<CR, CS, ACT, EPI, 2>(a, mrb, st);
  } else {
    if (nf == 2) return launch_t<CR, CS, ACT, EPI, 2>(a, mrb, st);
    if (nf == 4) return launch_t<CR, CS, ACT, EPI, 4>(a, mrb, st);
    return launch_t<CR, CS, ACT, EPI, 8>(a, mrb, st);
  }
}

template <int ACT, int EPI>
static hipError_t launch_codecs(int cr, int cs, int nf, const GroupedArgs& a, int mrb, hipStream_t st) {
#define MOE_CASE(R, S) \
  if (cr == R && cs == S) return launch_nf<R, S, ACT, EPI>(nf, a, mrb, st);
  if constexpr (ACT == MOE_F32) {
    MOE_CASE(MOE_F32, MOE_F32)
  } else if constexpr (EPI == EPI_F32) {
    MOE_CASE(MOE_BF16, MOE_BF16)
  } else {
    MOE_CASE(MOE_BF16, MOE_BF16)
    MOE_CASE(MOE_BF16, MOE_FP8_E4M3_B128)
    MOE_CASE(MOE_BF16, MOE_MXFP4_B32)
    MOE_CASE(MOE_FP8_E4M3_B128, MOE_BF16)
    MOE_CASE(MOE_FP8_E4M3_B128, MOE_FP8_E4M3_B128)
    MOE_CASE(MOE_FP8_E4M3_B128, MOE_MXFP4_B32)
    MOE_CASE(MOE_MXFP4_B32, MOE_BF16)
    MOE_CASE(MOE_MXFP4_B32, MOE_FP8_E4M3_B128)
    MOE_CASE(MOE_MXFP4_B32, MOE_MXFP4_B32)
    MOE_CASE(MOE_MXFP4_B32_A8, MOE_MXFP4_B32_A8)  // the routed groups of a W4A8 layer
    MOE_CASE(MOE_MXFP8_B32_A8, MOE_MXFP8_B32_A8)  // its W8A8 MXFP8 shared expert
    MOE_CASE(MOE_INT8_W8A8, MOE_INT8_W8A8)
  }
#undef MOE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_grouped_decode(int act, int epi, int cr, int cs, const GroupedArgs& a,
                                 int max_row_blocks, hipStream_t st) {
  // The SwiGLU product takes two tiles per item once the launch's groups average 8 rows or more:
  // the activation chunk of a 16-row tile then feeds twice the weight bytes (one tile per item
  // measured 5% slower on the V3 decode layer, two tiles 10% slower on the Qwen3 one at 4 rows).
  int nf = decode_nf(cr, epi, a.K, a.N);
  if (epi == EPI_SWIGLU && nf == 1 && a.G > 0 && a.M >= 8 * a.G && a.N % 32 == 0) nf = 2;
  if (a.N % (16 * nf) != 0) return hipErrorInvalidValue;
  if (act == MOE_F32) {
    if (epi == EPI_SWIGLU) return launch_codecs<MOE_F32, EPI_SWIGLU>(cr, cs, nf, a, max_row_blocks, st);
    if (epi == EPI_PLAIN) return launch_codecs<MOE_F32, EPI_PLAIN>(cr, cs, nf, a, max_row_blocks, st);
    return launch_codecs<MOE_F32, EPI_F32>(cr, cs, nf, a, max_row_blocks, st);
  }
  if (epi == EPI_SWIGLU) return launch_codecs<MOE_BF16, EPI_SWIGLU>(cr, cs, nf, a, max_row_blocks, st);
  if (epi == EPI_PLAIN) return launch_codecs<MOE_BF16, EPI_PLAIN>(cr, cs, nf, a, max_row_blocks, st);
  return launch_codecs<MOE_BF16, EPI_F32>(cr, cs, nf, a, max_row_blocks, st);
}

}  // namespace moe
