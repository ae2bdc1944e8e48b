// Prefill-regime grouped GEMM: many rows per expert, bound by the matrix cores.
//
// A workgroup of 8 waves (two per SIMD, so one wave's LDS reads, conversions and barrier wait
// overlap the other's MFMAs) computes one work item:
//   full item: 256 rows x 256 matrix columns; waves (wr, wc) = (wave / 4, wave % 4) take rows
//              wr * 128 .. + 128 and columns wc * 64 .. + 64;
//   half item: the last <= 128 rows of a group x 512 matrix columns; wave w takes columns
//              w * 64 .. + 64 of all rows.
// Every wave therefore owns a 128-row x 64-column accumulator tile (for the SwiGLU GEMM, 32 gate
// and the matching 32 up columns, so SiLU(gate) * up is formed in registers). A group of n rows
// is n / 256 full items plus one full or half item for the rest, which wastes no more rows than
// 128-row tiles would.
//
// Both operands reach LDS by direct global -> LDS DMA (global_load_lds_dwordx4) through a ring of
// reduction steps (3 stages, or 2 where a stage is too large), so the loads of the next stages are
// in flight behind the current steps' MFMA work and hold no registers. Each 1 KiB DMA lands in MFMA
// fragment order (a weight packet as stored; an activation fragment gathered from 16 rows), so
// every LDS read is a conflict-free 16-byte read. Weights are the A operand, activations the B
// operand. Per weight format (the PCodec specialisations below):
//   bf16, fp8, MXFP4 with bf16 activations: v_mfma_f32_16x16x32_bf16; fp8 and fp4 packets are
//     converted by the wave that uses them (exactly, with the block scale's exponent);
//   W4A8 and W8A8 MXFP8 with MXFP8 activations: v_mfma_scale_f32_16x16x128_f8f6f4, operands and
//     e8m0 exponents as stored;
//   Int8 W8A8 with int8 activations: v_mfma_i32_16x16x64_i8, exact int32 sums scaled per row and
//     per feature after the last step.
//
// Items are ordered so that a run of consecutive items covers up to 8 column tiles x all full
// row tiles of one group, and the workgroup -> item map gives each XCD a contiguous run of the
// items that exist: workgroups resident at the same time on one XCD then share weight and
// activation slices in that XCD's L2 (Chapter 6 'Supernodes' section 6.3.2: one weight read
// serves many rows).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PTHREADS = 512;
constexpr int PBM = 256;   // rows per full item
constexpr int PRB = 128;   // rows per half item, and the plan's row block
constexpr int PWC = 64;    // matrix columns per wave
constexpr int NXCD = 8;

template <int C>
struct PCodec;

template <>
struct PCodec<MOE_BF16> {
  static constexpr int KP = 32;      // reduction elements per packet
  static constexpr int PBK = 32;     // reduction elements per pipeline step
  static constexpr int H = 1;        // 32-deep MFMA steps per pipeline step
  static constexpr int PK = 1;       // packets per 16-column tile per pipeline step
  static constexpr bool HALF_ONLY = false;  // every item 128 rows x 512 columns
  static constexpr bool FULL_ONLY = false;  // every item 256 rows x 256 columns (one group per launch)
  static constexpr bool SCALE_DMA = false;  // per-packet scales reach LDS with the weights
  static constexpr int ACT_BYTES = 2;       // bytes per activation element
  static constexpr int NSC = 0;             // scale DMA loads per wave per step
  static constexpr int SC_KIB = 0;          // LDS of those scales per stage
  // Activation layout of one 16-row tile per step (H KiB of LDS): DMA unit u, lane l reads
  // 16 bytes of row dma_row(l, u) at byte dma_off(l, u) of the row's step slice and lands them
  // at u * 1024 + 16 * l; the B fragment of MFMA half h is the 16 bytes at read_off(l, h).
  // bf16: lane l holds row l % 16, reduction elements 8 * (l / 16) .. + 8 (the packet's order).
  __device__ static int dma_row(int l, int) { return l & 15; }
  __device__ static int dma_off(int l, int) { return 16 * (l >> 4); }
  __device__ static int read_off(int l, int) { return 16 * l; }
  __device__ static void frags(const u32x4 (&w)[PK], float, bf16x8 (&a)[H]) {
    a[0] = __builtin_bit_cast(bf16x8, w[0]);
  }
};

// fp8 weights: a 128 x 128 block scale s is split as s = 2^e * m with m in [1, 2). The
// conversion e4m3 -> bf16 applies 2^e (v_cvt_scalef32_pk_bf16_fp8 uses only the exponent of its
// scale operand), which is exact: an e4m3 value has 4 significant bits. The mantissa factor m is
// carried by the accumulators instead: at each 128-deep reduction block they are multiplied by
// m_previous / m_current, and the epilogue multiplies by the last block's m. The sum is
// therefore sum_b s_b * (q_b . x_b) with the weights exact and fp32 rounding only.
__device__ __forceinline__ float scale_mantissa(float s) {
  return __int_as_float((__float_as_int(s) & 0x007FFFFF) | 0x3F800000);
}

__device__ __forceinline__ bf16x8 p_fp8x8(uint32_t w0, uint32_t w1, float s) {
  typedef __attribute__((ext_vector_type(2))) __bf16 b2;
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true));
  return __builtin_bit_cast(bf16x8, r);
}

template <>
struct PCodec<MOE_FP8_E4M3_B128> {
  static constexpr int KP = 64;
  static constexpr int PBK = 64;
  static constexpr int H = 2;
  static constexpr int PK = 1;
  static constexpr bool HALF_ONLY = false, FULL_ONLY = false;
  static constexpr bool SCALE_DMA = false;
  static constexpr int ACT_BYTES = 2, NSC = 0, SC_KIB = 0;
  // Lane group g of a packet holds reduction elements 16g .. 16g + 15 and MFMA half h takes the
  // h-th run of 8 of them, so the B fragment of half h for lane (g, row j) is the 16-byte chunk
  // c = 2g + h of row j's 128-byte step slice. DMA unit u moves rows 8u .. 8u + 7 as whole
  // 128-byte lines (lane l: row l / 8, chunk (l % 8) ^ (l / 8) ^ u), so row r of unit u stores
  // chunk c at position c ^ (r % 8) ^ u: the XOR swizzle spreads the 16 lanes of each read phase
  // over all 64 LDS banks.
  __device__ static int dma_row(int l, int u) { return 8 * u + (l >> 3); }
  __device__ static int dma_off(int l, int u) { return 16 * ((l & 7) ^ (l >> 3) ^ u); }
  __device__ static int read_off(int l, int h) {
    const int j = l & 15, g = l >> 4;
    return (j >> 3) * 1024 + (j & 7) * 128 + 16 * ((2 * g + h) ^ (j & 7) ^ (j >> 3));
  }
  __device__ static void frags(const u32x4 (&w)[PK], float s, bf16x8 (&a)[H]) {
    a[0] = p_fp8x8(w[0][0], w[0][1], s);
    a[1] = p_fp8x8(w[0][2], w[0][3], s);
  }
};

// 8 e2m1 codes (one dword, element 2b in the low nibble of byte b) -> 8 bf16 times 2^(E-127):
// v_cvt_scalef32_pk_bf16_fp4 is exact here and applies the exponent of `scale`.
__device__ __forceinline__ bf16x8 p_fp4x8(uint32_t w, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// MXFP4: a packet is 16 features x 128 reduction elements, lane (g, f) holding elements
// 32g .. 32g + 31 as 4 dwords of 8 codes, with one e8m0 exponent per lane. A pipeline step
// is one packet deep, so a 16-row activation tile is 16 rows x 256 bytes per step; to keep the
// stage small every item is 128 rows x 512 columns (2 stages of 72 KiB). MFMA half h takes
// dword h of each lane: elements 32g + 8h .. + 8, i.e. the 16-byte activation chunk
// c = 4g + h of the row. DMA unit u moves rows 4u .. 4u + 3 (lane l: row 4u + l / 16, chunk
// (l % 16) ^ row), so row r stores chunk c at position c ^ r: the XOR swizzle spreads every
// read phase over all 64 LDS banks.
template <>
struct PCodec<MOE_MXFP4_B32> {
  static constexpr int KP = 128;
  static constexpr int PBK = 128;
  static constexpr int H = 4;
  static constexpr int PK = 1;
  static constexpr bool HALF_ONLY = true, FULL_ONLY = false;
  static constexpr bool SCALE_DMA = true;
  static constexpr int ACT_BYTES = 2, NSC = 1, SC_KIB = 8;
  __device__ static int dma_row(int l, int u) { return 4 * u + (l >> 4); }
  __device__ static int dma_off(int l, int u) { return 16 * ((l & 15) ^ (4 * u + (l >> 4))); }
  __device__ static int read_off(int l, int h) {
    const int j = l & 15, g = l >> 4;
    return j * 256 + 16 * ((4 * g + h) ^ j);
  }
  __device__ static void frags(const u32x4 (&w)[PK], float s, bf16x8 (&a)[H]) {
#pragma unroll
    for (int h = 0; h < H; ++h) a[h] = p_fp4x8(w[0][h], s);
  }
};

// W4A8: MXFP4 weight packets times MXFP8 activations, both handed to
// v_mfma_scale_f32_16x16x128_f8f6f4 as stored (no conversion, no rescale: the e8m0 exponents go to
// the instruction's scale operands). One step is one packet deep (128). The operand layouts of that
// instruction (fp4 A, fp8 B, measured on the hardware):
//   A, fp4: lane (f, g) = (l % 16, l / 16) holds 32 codes of feature f. Its pairing with B makes
//           them reduction elements 32g .. 32g + 31 -- exactly a packet lane -- and the lane's own
//           scale byte applies to all 32: the packet's e8m0 byte of that lane.
//   B, fp8: lane (j, g) holds token j: bytes 0..15 are elements 16g .. 16g + 15, bytes 16..31 are
//           elements 64 + 16g .. 64 + 16g + 15, i.e. 16-byte chunks g and 4 + g of the token's
//           128-byte step slice; the exponent of (token j, block b) is taken from lane j + 16b.
// Activations move as whole 128-byte row lines, 8 rows per DMA unit, with the same XOR swizzle as
// the fp8 codec's bf16 lines, so the two chunk reads of a lane are conflict-free. Per stage the LDS
// also holds each wave's 4 tiles x 64 packet exponents and the item's activation exponents, 4
// bytes (the step's 4 blocks) per row, gathered like the rows: both by 4-byte DMAs, one per wave,
// the second covering 4 row tiles from the wave's first (neighbouring waves write the same bytes
// to the overlap).
template <>
struct PCodec<MOE_MXFP4_B32_A8> {
  static constexpr int KP = 128;
  static constexpr int PBK = 128;
  static constexpr int H = 2;  // 1 KiB activation DMA units per 16-row tile per step
  static constexpr int PK = 1;
  static constexpr bool HALF_ONLY = false, FULL_ONLY = false;
  static constexpr bool SCALE_DMA = false;
  static constexpr int ACT_BYTES = 1, NSC = 2, SC_KIB = 4;
  __device__ static int dma_row(int l, int u) { return 8 * u + (l >> 3); }
  __device__ static int dma_off(int l, int u) { return 16 * ((l & 7) ^ (l >> 3) ^ u); }
  // chunk 4h + g of token row j = l % 16
  __device__ static int read_off(int l, int h) {
    const int j = l & 15, g = l >> 4;
    return (j >> 3) * 1024 + (j & 7) * 128 + 16 * ((4 * h + g) ^ (j & 7) ^ (j >> 3));
  }
  // the bf16-operand step is compiled but never reached for this codec (its step returns first)
  __device__ static void frags(const u32x4 (&)[PK], float, bf16x8 (&)[H]) {}
};

// W8A8 MXFP8 (the shared expert of the hybrid MXFP8-MXFP4 scheme): fp8 weight packets times
// MXFP8 activations on the same block-scaled instruction, fp8 x fp8. Measured on the hardware, the
// fp8 A operand has the fp8 B layout: lane (f, g) holds elements 16g .. 16g + 15 in bytes 0..15 and
// 64 + 16g .. + 15 in bytes 16..31, and the exponent of (feature f, block b) comes from lane
// f + 16b. The two packets of a column tile in one step (elements 0..63 and 64..127, lane l holding
// run 16 (l / 16) of each) are therefore the operand as stored, and the packed exponents (one byte
// per lane per pair of packets) its scales. A step takes 2 KiB of weights per column tile, so a
// 128-row x 512-column half item would need 80 KiB per stage: every item is a full one (64 KiB of
// codes and 4 KiB of exponents per stage, two stages), the waves of a row half without rows skip
// the MFMAs, and a launch covers one group. Activations as in the W4A8 codec.
template <>
struct PCodec<MOE_MXFP8_B32_A8> {
  static constexpr int KP = 64;
  static constexpr int PBK = 128;
  static constexpr int H = 2;
  static constexpr int PK = 2;
  static constexpr bool HALF_ONLY = false, FULL_ONLY = true;
  static constexpr bool SCALE_DMA = false;
  static constexpr int ACT_BYTES = 1, NSC = 2, SC_KIB = 4;
  __device__ static int dma_row(int l, int u) { return PCodec<MOE_MXFP4_B32_A8>::dma_row(l, u); }
  __device__ static int dma_off(int l, int u) { return PCodec<MOE_MXFP4_B32_A8>::dma_off(l, u); }
  __device__ static int read_off(int l, int h) { return PCodec<MOE_MXFP4_B32_A8>::read_off(l, h); }
  __device__ static void frags(const u32x4 (&)[PK], float, bf16x8 (&)[H]) {}
};

// Int8 W8A8: int8 weight packets (16 features x 64 K, laid out as fp8 packets) times int8
// activation rows on v_mfma_i32_16x16x64_i8, which adds the products of the codes exactly in int32.
// Its A and B operands take the same lane layout (lane (f, g): 16 bytes of feature or token f), so
// packet lane (f, g) and the activation chunk of the same run pair the same reduction elements,
// whatever order the instruction adds them in. One step is 128 deep: two MFMAs per (row tile,
// column tile), half h on the step's packet h and on chunk 4h + g of the token's 128-byte line (the
// W4A8 activation layout). No scale enters the loop: the epilogue multiplies each sum by its row's
// activation scale and its feature's weight scale. A half item takes 80 KiB per stage (64 KiB of
// packets), so two stages.
template <>
struct PCodec<MOE_INT8_W8A8> {
  static constexpr int KP = 64;
  static constexpr int PBK = 128;
  static constexpr int H = 2;
  static constexpr int PK = 2;
  static constexpr bool HALF_ONLY = false, FULL_ONLY = false;
  static constexpr bool SCALE_DMA = false;
  static constexpr int ACT_BYTES = 1, NSC = 0, SC_KIB = 0;
  __device__ static int dma_row(int l, int u) { return PCodec<MOE_MXFP4_B32_A8>::dma_row(l, u); }
  __device__ static int dma_off(int l, int u) { return PCodec<MOE_MXFP4_B32_A8>::dma_off(l, u); }
  __device__ static int read_off(int l, int h) { return PCodec<MOE_MXFP4_B32_A8>::read_off(l, h); }
  __device__ static void frags(const u32x4 (&)[PK], float, bf16x8 (&)[H]) {}
};

template <int EPI>
struct PEpi {
  static constexpr int NMAT = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q8) ? 2 : 1;
  static constexpr int WF = PWC / 16 / NMAT;   // 16-feature tiles per matrix per wave
  static constexpr int FULL_F = 4 * WF * 16;   // output features of a full item
};

template <int C>
struct PLayout {
  using Cd = PCodec<C>;
  static constexpr int H = Cd::H, PK = Cd::PK;
  // per stage: activation fragments (16 row tiles x H for a full item, 8 x H for a half item)
  // followed by weight packets (16 column tiles x PK, or 32 x PK), then (MXFP4) each wave's
  // 1 KiB of packet scales; in KiB
  static constexpr int FULL_ACT = 16 * H, HALF_ACT = 8 * H;
  static constexpr int FULL_W = 16 * PK, HALF_W = 32 * PK;
  static constexpr int SC_KIB = Cd::SC_KIB;
  static constexpr int ITEM_KIB = Cd::FULL_ONLY ? FULL_ACT + FULL_W
                                 : (!Cd::HALF_ONLY && FULL_ACT + FULL_W > HALF_ACT + HALF_W) ? FULL_ACT + FULL_W
                                                                                           : HALF_ACT + HALF_W;
  static constexpr int SC_OFF = ITEM_KIB * 1024;
  static constexpr int STAGE_KIB = ITEM_KIB + SC_KIB;
  static constexpr int STAGES = (Cd::HALF_ONLY || Cd::FULL_ONLY || 3 * STAGE_KIB > 160) ? 2 : 3;
  // DMA instructions per wave per stage; the shorter kind is padded with repeats of its last
  // load so both kinds issue the same count (the wait counts are compile-time)
  static constexpr int LF = Cd::HALF_ONLY ? 0 : 2 * H + 2 * PK, LH = H + 4 * PK;
  static constexpr int L = (Cd::FULL_ONLY ? LF : (LF > LH ? LF : LH)) + Cd::NSC;
  static_assert(STAGES * STAGE_KIB <= 160, "LDS");
};

// (group-local full item) -> (row tile, column tile): runs of up to 8 column tiles over all
// full row tiles of the group.
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
__global__ void __launch_bounds__(PTHREADS, 1) grouped_prefill_kernel(GroupedArgs a) {
  using Cd = PCodec<C>;
  using Ly = PLayout<C>;
  constexpr int NMAT = PEpi<EPI>::NMAT;
  constexpr int WF = PEpi<EPI>::WF;
  constexpr int NT = NMAT * WF;  // 16-column tiles per wave (4)
  constexpr int H = Cd::H, PK = Cd::PK, PBK = Cd::PBK;
  constexpr int KP = Cd::KP;
  constexpr int D = Ly::STAGES;
  constexpr int STAGE_B = Ly::STAGE_KIB * 1024;
  constexpr int L = Ly::L;
  constexpr int QJ = (L + 7) / 8;  // DMA loads issued per row tile of a step
  __shared__ __attribute__((aligned(1024))) uint8_t lds[D * STAGE_B];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntn = a.NTW;  // full-item column tiles
  // Grouped mode (a plan is given): group g has mt 128-row blocks, i.e. mt / 2 full items and a
  // half item for an odd block, per pair of full-item column tiles (ntn is even), or mt half
  // items with HALF_ONLY; the launch covers groups [g_begin, g_end). Single-group mode (no plan,
  // the router scores): ceil(M / 256) full items per column tile.
  const bool planned = a.cum_blocks != nullptr;
  const int gb = planned && a.g_end > a.g_begin ? a.g_begin : 0;
  const int ge = planned && a.g_end > a.g_begin ? a.g_end : a.G;
  const int ibase = planned ? a.cum_blocks[gb] * (ntn >> 1) : 0;
  // FULL_ONLY (one group per launch): ceil(rows / 256) full items per column tile
  const int total = Cd::FULL_ONLY ? (a.group_range[2 * gb + 1] - a.group_range[2 * gb] + PBM - 1) / PBM * ntn
                    : planned     ? a.cum_blocks[ge] * (ntn >> 1) - ibase
                                  : (a.M + PBM - 1) / PBM * ntn;
  // XCD-aware workgroup -> item map over the items that exist: XCD x (= blockIdx % 8) takes
  // items [x * per_xcd, (x + 1) * per_xcd)
  const int per_xcd = (total + NXCD - 1) / NXCD;
  if ((int)(blockIdx.x / NXCD) >= per_xcd) return;
  const int item = (blockIdx.x % NXCD) * per_xcd + blockIdx.x / NXCD;
  if (item >= total) return;
  int g = 0, row0, ntile, rbeg = 0, rend = a.M;
  bool half = false;
  if (Cd::FULL_ONLY) {
    g = gb;
    rbeg = a.group_range[2 * g];
    rend = a.group_range[2 * g + 1];
    int mtile;
    item_tiles(item, (rend - rbeg + PBM - 1) / PBM, ntn, mtile, ntile);
    row0 = rbeg + mtile * PBM;
  } else if (planned) {
    const int gi = item + ibase;
    // 128-row block gi / (ntn / 2) of the row space: its group and place from the plan's table
    // (one load), else a search over cum_blocks
    int bin;
    if (a.block_group) {
      const int gbk = a.block_group[gi / (ntn >> 1)];
      g = gbk >> 16;
      bin = gbk & 0xFFFF;
    } else {
      int lo = gb, hi = ge - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cum_blocks[mid] * (ntn >> 1) <= gi) lo = mid; else hi = mid - 1;
      }
      g = lo;
      bin = gi / (ntn >> 1) - a.cum_blocks[g];
    }
    rbeg = a.group_range[2 * g];
    rend = a.group_range[2 * g + 1];
    const int mt = (rend - rbeg + PRB - 1) / PRB;  // 128-row blocks of the group
    const int li = bin * (ntn >> 1) + gi % (ntn >> 1);
    if constexpr (Cd::HALF_ONLY) {
      int blk;
      item_tiles(li, mt, ntn >> 1, blk, ntile);
      half = true;
      row0 = rbeg + blk * PRB;
    } else {
      const int mtf = mt >> 1;  // full row tiles
      int mtile;
      half = li >= mtf * ntn;
      if (half) {
        mtile = mtf;
        ntile = li - mtf * ntn;
      } else {
        item_tiles(li, mtf, ntn, mtile, ntile);
      }
      row0 = rbeg + mtile * PBM;
    }
  } else {
    int mtile;
    item_tiles(item, (a.M + PBM - 1) / PBM, ntn, mtile, ntile);
    row0 = mtile * PBM;
  }
  const int nr = min(half ? PRB : PBM, rend - row0);
  const bool is_shared = g == a.shared_group;
  const uint8_t* w0 = is_shared ? a.wa_s : a.wa_r + (size_t)g * a.mat_bytes;
  const uint8_t* w1 = is_shared ? a.wb_s : (a.wb_r ? a.wb_r + (size_t)g * a.mat_bytes : nullptr);
  const uint8_t* ws0 = is_shared ? a.sa_s : (a.sa_r ? a.sa_r + (size_t)g * a.scale_bytes : nullptr);
  const uint8_t* ws1 = is_shared ? a.sb_s : (a.sb_r ? a.sb_r + (size_t)g * a.scale_bytes : nullptr);
  const float* s0 = (const float*)ws0;
  const float* s1 = (const float*)ws1;
  const int KT = a.K / KP;
  const int KTS = a.K / 128;  // W4A8 / W8A8: exponent packets (one per 128-deep step) per column tile
  // reduction steps of this workgroup: split-K part blockIdx.y of ksplit (fp32 partial outputs)
  const int KSG = a.ksplit > 1 ? a.ksplit : 1;
  const int kstep0 = (int)blockIdx.y * (a.K / PBK) / KSG;
  const int nsteps = ((int)blockIdx.y + 1) * (a.K / PBK) / KSG - kstep0;
  const int j16 = lane & 15, g4 = lane >> 4;

  // this wave's place: row half and column slot within the item
  const int wrow = half ? 0 : wave >> 2;
  const int wcol = half ? wave : wave & 3;
  // global wave-column index (units of WF 16-feature tiles per matrix)
  const int gw = half ? ntile * 8 + wave : ntile * 4 + wcol;
  int ftile[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ftile[t] = gw * WF + t % WF;

  // fp8 block scales: this wave's features of each matrix lie in one 128-wide block, so the
  // scale depends only on the 128-deep reduction block; lane i holds block i (K <= 8192), and
  // the loop picks the current one with a lane read (no memory access in the pipeline)
  const int nblk = ftile[0] >> 3;
  float scv[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const float* sp = m == 0 ? s0 : s1;
    scv[m] = (C == MOE_FP8_E4M3_B128 && lane < (a.K >> 7)) ? sp[lane * (a.N >> 7) + nblk] : 1.0f;
  }

  // --- DMA assignment: this wave's L loads per stage, q = 0 .. L - 1 ---
  // full item: activation row tiles 2w, 2w + 1 (x H DMA units), then column tiles 2 * wrow,
  //            2 * wrow + 1 of this wave's slot (the other row half loads the other two);
  // half item: activation row tile w (x H DMA units), then all 4 column tiles of this wave's slot.
  // Load q of stage s reads qsrc[q] + s * qstride[q] into LDS stage offset qdst[q]; the shorter
  // kind repeats its last load (same bytes to the same place) so both issue L loads.
  const uint8_t* qsrc[L];
  int qdst[L], qstride[L];
  const int wts_off = (half ? Ly::HALF_ACT : Ly::FULL_ACT) * 1024;
  constexpr int LSC = Cd::SCALE_DMA ? 1 : 0;  // the last load moves the packet scales
  constexpr bool A8 = C == MOE_MXFP4_B32_A8 || C == MOE_MXFP8_B32_A8;  // the last two loads move the exponents
  constexpr int AFMT = C == MOE_MXFP8_B32_A8 ? 0 : 4;  // A operand format of the block-scaled MFMA: fp8, fp4
  constexpr bool I8 = C == MOE_INT8_W8A8;  // int8 x int8, int32 sums
#pragma unroll
  for (int q = 0; q < L; ++q) {
    const int nact = half ? H : 2 * H;
    const int nw = half ? 4 * PK : 2 * PK;
    const int qq = q < nact + nw ? q : nact + nw - 1;
    if (A8 && q == L - 2) {
      // this wave's 4 column tiles' packet exponents, 64 bytes per tile: a 4-byte DMA, lane l
      // moving bytes 4 (l % 16) .. + 4 of tile l / 16
      const int t = lane >> 4;
      const uint8_t* sp = t / WF == 0 ? ws0 : ws1;
      qsrc[q] = sp + ((size_t)(gw * WF + t % WF) * KTS) * 64 + (size_t)(lane & 15) * 4;
      qdst[q] = Ly::SC_OFF + wave * 256;
      qstride[q] = 64;
    } else if (A8 && q == L - 1) {
      // activation exponents of the step (4 bytes per row) for 4 row tiles from this wave's first:
      // lane l moves row rt0 * 16 + l, gathered like the activation rows; rows past the group's
      // end read the zero row (exponent byte 0 with zero codes)
      const int rt0 = half ? wave : 2 * wave;
      const int rr = rt0 * 16 + lane;
      const int r = row0 + (rr < nr ? rr : 0);
      int src = a.gather ? (r < a.P ? a.gather[r] : r - a.P) : r;
      if ((unsigned)src >= (unsigned)a.act_rows) src = 0;
      qsrc[q] = (rr >= nr && a.zero_row) ? (const uint8_t*)a.zero_row
                                         : (const uint8_t*)a.act_scale + (size_t)src * (a.K / 32);
      qdst[q] = Ly::SC_OFF + 2048 + rt0 * 64;
      qstride[q] = 4;
    } else if (LSC && q == L - 1) {
      // this wave's 4 column tiles' e8m0 bytes of the step's packets (64 per tile): lane l
      // fetches 16 bytes of tile (l % 16) / 4; lanes 16..63 repeat lanes 0..15
      const int t = (lane & 15) >> 2;
      const uint8_t* sp = t / WF == 0 ? ws0 : ws1;
      qsrc[q] = sp + ((size_t)(gw * WF + t % WF) * KT) * 64 + (size_t)(lane & 3) * 16;
      qdst[q] = Ly::SC_OFF + wave * 1024;
      qstride[q] = PK * 64;
    } else if (qq < nact) {
      const int i = qq / H, h = qq % H;
      const int rt = half ? wave : 2 * wave + i;
      const int rr = rt * 16 + Cd::dma_row(lane, h);
      const int r = row0 + (rr < nr ? rr : 0);
      int src = a.gather ? (r < a.P ? a.gather[r] : r - a.P) : r;
      if ((unsigned)src >= (unsigned)a.act_rows) src = 0;
      // rows past the group's end feed zeros when a zero row is given (their results are
      // discarded either way; zero operands keep the padding MFMAs cheap in power)
      const uint8_t* rowp = (rr >= nr && a.zero_row) ? (const uint8_t*)a.zero_row
                                                      : (const uint8_t*)a.act + (size_t)src * a.lda * Cd::ACT_BYTES;
      qsrc[q] = rowp + Cd::dma_off(lane, h);
      qdst[q] = (rt * H + h) * 1024;
      qstride[q] = PBK * Cd::ACT_BYTES;
    } else {
      const int i = (qq - nact) / PK, p = (qq - nact) % PK;
      const int t = half ? i : 2 * wrow + i;
      qsrc[q] = (t / WF == 0 ? w0 : w1) + ((size_t)(gw * WF + t % WF) * KT + p) * PACKET_BYTES + (size_t)lane * 16;
      qdst[q] = wts_off + ((wcol * NT + t) * PK + p) * 1024;
      qstride[q] = PK * PACKET_BYTES;
    }
  }
  auto dma_one = [&](int q, int step) __attribute__((always_inline)) {
    const int st = kstep0 + min(step, nsteps - 1);
    if (A8 && q >= L - 2)
      __builtin_amdgcn_global_load_lds((const void*)(qsrc[q] + (size_t)st * qstride[q]),
                                       (lds_void*)(lds + (step % D) * STAGE_B + qdst[q]), 4, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((const void*)(qsrc[q] + (size_t)st * qstride[q]),
                                       (lds_void*)(lds + (step % D) * STAGE_B + qdst[q]), 16, 0, 0);
  };

  f32x4 acc[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < D - 1; ++s)
#pragma unroll
    for (int q = 0; q < L; ++q) dma_one(q, s);

  int aoff[H];
#pragma unroll
  for (int h = 0; h < H; ++h) aoff[h] = wrow * 8 * H * 1024 + Cd::read_off(lane, h);
  const int wbase = wts_off + wcol * NT * PK * 1024 + lane * 16;
  // fp8: mantissa factor of the current block scale, per matrix (see scale_mantissa)
  constexpr bool SCALED = C == MOE_FP8_E4M3_B128;
  constexpr int SPB = SCALED ? 128 / PBK : 1;  // pipeline steps per scale block
  float mcur[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
    mcur[m] = scale_mantissa(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(scv[m]), (kstep0 * PBK) >> 7)));

  auto step_body = [&](int step, auto first_of_block, auto row_tiles) __attribute__((always_inline)) {
    constexpr bool RESCALE = SCALED && decltype(first_of_block)::value;
    constexpr int MTA = decltype(row_tiles)::value;  // row tiles of this wave that hold group rows
    // this wave's loads of `step` have landed; after the barrier, every wave's have, and no
    // wave still reads the slot the next DMA overwrites (that of step - 1)
    MOE_WAIT_VMCNT((D - 2) * L);
    __builtin_amdgcn_s_barrier();
    const uint8_t* base = lds + (step % D) * STAGE_B;
    float sc[NMAT], rs[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      sc[m] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scv[m]), ((kstep0 + step) * PBK) >> 7));
      if constexpr (RESCALE) {
        const float mn = scale_mantissa(sc[m]);
        rs[m] = mcur[m] * __builtin_amdgcn_rcpf(mn);  // m ratio in (0.5, 2), about 1 ulp
        mcur[m] = mn;
      }
    }
    if constexpr ((A8 || I8) && MTA == 0) {
      // no rows in this wave's half of the item: only its share of the next stage's loads
#pragma unroll
      for (int q = 0; q < L; ++q) dma_one(q, step + D - 1);
      return;
    } else if constexpr (I8) {
      // two int8 MFMAs per (row tile, column tile): packet h of the tile's step and the lane's
      // activation chunk of half h; the int32 sums live in the accumulator registers' bits
      u32x4 aw[NT][2];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) aw[t][h] = *(const u32x4*)(base + wbase + (t * PK + h) * 1024);
      u32x4 b0n = *(const u32x4*)(base + aoff[0]), b1n = *(const u32x4*)(base + aoff[1]);
      constexpr int QA = (L + MTA - 1) / (MTA > 0 ? MTA : 1);
#pragma unroll
      for (int j = 0; j < MTA; ++j) {
        const u32x4 b0 = b0n, b1 = b1n;
        if (j + 1 < MTA) {
          b0n = *(const u32x4*)(base + aoff[0] + (j + 1) * H * 1024);
          b1n = *(const u32x4*)(base + aoff[1] + (j + 1) * H * 1024);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t][j] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, aw[t][0]), __builtin_bit_cast(i32x4, b0),
                                                           __builtin_bit_cast(i32x4, acc[t][j]), 0, 0, 0));
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t][j] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, aw[t][1]), __builtin_bit_cast(i32x4, b1),
                                                           __builtin_bit_cast(i32x4, acc[t][j]), 0, 0, 0));
#pragma unroll
        for (int u = 0; u < QA; ++u)
          if (j * QA + u < L) dma_one(j * QA + u, step + D - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    } else if constexpr (A8) {
      // one block-scaled MFMA per (row tile, column tile): the weights as stored with their e8m0
      // byte (fp4: one packet, codes in operand dwords 0-3; fp8: the step's two packets), the two
      // 16-byte activation chunks of the lane with the row tile's exponent byte
      i32x8 af8[NT];
      int sa[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 pk = *(const u32x4*)(base + wbase + t * PK * 1024);
        if constexpr (PK == 2) {
          const u32x4 pk1 = *(const u32x4*)(base + wbase + (t * PK + 1) * 1024);
          af8[t] = i32x8{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3],
                         (int)pk1[0], (int)pk1[1], (int)pk1[2], (int)pk1[3]};
        } else {
          af8[t] = i32x8{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], 0, 0, 0, 0};
        }
        sa[t] = base[Ly::SC_OFF + wave * 256 + t * 64 + lane];
      }
      // exponent of (token l % 16, block l / 16) of row tile rt: byte rt * 64 + 4 (l % 16) + l / 16
      const uint8_t* sbp = base + Ly::SC_OFF + 2048 + wrow * 8 * 64 + 4 * j16 + (lane >> 4);
      u32x4 b0n = *(const u32x4*)(base + aoff[0]), b1n = *(const u32x4*)(base + aoff[1]);
      int sbn = sbp[0];
      constexpr int QA = (L + MTA - 1) / (MTA > 0 ? MTA : 1);  // DMA loads per row tile
#pragma unroll
      for (int j = 0; j < MTA; ++j) {
        const u32x4 b0 = b0n, b1 = b1n;
        const int sb = sbn;
        if (j + 1 < MTA) {
          b0n = *(const u32x4*)(base + aoff[0] + (j + 1) * H * 1024);
          b1n = *(const u32x4*)(base + aoff[1] + (j + 1) * H * 1024);
          sbn = sbp[(j + 1) * 64];
        }
        const i32x8 bf = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                               (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af8[t], bf, acc[t][j], AFMT, 0, 0, sa[t], 0, sb);
#pragma unroll
        for (int u = 0; u < QA; ++u)
          if (j * QA + u < L) dma_one(j * QA + u, step + D - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    bf16x8 af[NT][H];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x4 pk[PK];
#pragma unroll
      for (int p = 0; p < PK; ++p) pk[p] = *(const u32x4*)(base + wbase + (t * PK + p) * 1024);
      float st = sc[t / WF];
      if constexpr (Cd::SCALE_DMA) st = __uint_as_float((uint32_t)base[Ly::SC_OFF + wave * 1024 + t * 64 + lane] << 23);
      Cd::frags(pk, st, af[t]);
    }
    // the next stage's DMA is spread over the MFMA stream, one load per row tile, so the
    // loads never queue up in front of the matrix work
    bf16x8 bn[H];
#pragma unroll
    for (int h = 0; h < H; ++h) bn[h] = *(const bf16x8*)(base + aoff[h]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x8 b[H];
#pragma unroll
      for (int h = 0; h < H; ++h) b[h] = bn[h];
      if (j + 1 < 8) {
#pragma unroll
        for (int h = 0; h < H; ++h) bn[h] = *(const bf16x8*)(base + aoff[h] + (j + 1) * H * 1024);
      }
      if constexpr (RESCALE) {
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][j] *= rs[t / WF];
      }
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t][h], b[h], acc[t][j], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < QJ; ++u)
        if (j * QJ + u < L) dma_one(j * QJ + u, step + D - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // every instantiation inlined: an outlined copy would pass the captures through scratch memory
  auto run_steps = [&](auto row_tiles) __attribute__((always_inline)) {
    for (int step = 0; step < nsteps; step += SPB) {
      step_body(step, std::true_type{}, row_tiles);
#pragma unroll
      for (int u = 1; u < SPB; ++u) step_body(step + u, std::false_type{}, row_tiles);
    }
  };
  if constexpr (A8 || I8) {
    // W4A8 leaves the row tiles past the group's end out of the MFMA stream, 32 rows at a time:
    // each wave runs the loop compiled for 2, 4, 6 or 8 row tiles, chosen once per item, so the
    // stream has no branches. Their accumulators stay zero and are never stored. (Padding MFMAs
    // of the bf16-operand codecs read zero rows and cost little; fp8 MFMAs cost twice the issue.)
    const int wave_rows = nr - wrow * PRB;  // group rows in this wave's 128-row half
    if (wave_rows > 96) run_steps(std::integral_constant<int, 8>{});
    else if (wave_rows > 64) run_steps(std::integral_constant<int, 6>{});
    else if (wave_rows > 32) run_steps(std::integral_constant<int, 4>{});
    else if (!Cd::FULL_ONLY || wave_rows > 0) run_steps(std::integral_constant<int, 2>{});
    else run_steps(std::integral_constant<int, 0>{});  // FULL_ONLY: the item's rows fit in the other half
  } else {
    run_steps(std::integral_constant<int, 8>{});
  }
  MOE_WAIT_VMCNT(0);  // the clamped tail DMAs must land before the workgroup's LDS is released

  if constexpr (I8) {
    // int32 sums -> fp32, times the row's activation scale (its token's for gathered rows) and the
    // feature's weight scale; rows past the group's end are never stored
    const float* asc = (const float*)a.act_scale;
    float rsc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = wrow * 128 + j * 16 + j16;
      rsc[j] = 0.f;
      if (rr < nr) {
        const int r = row0 + rr;
        const int src = a.gather ? (r < a.P ? a.gather[r] : r - a.P) : r;
        if ((unsigned)src < (unsigned)a.act_rows) rsc[j] = asc[src];
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 cs = *(const f32x4*)((t / WF == 0 ? s0 : s1) + ftile[t] * 16 + 4 * g4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // reinterpret the whole register vector (a bit cast of one vector element read element 0)
        const i32x4 iv = __builtin_bit_cast(i32x4, acc[t][j]);
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (float)iv[i] * rsc[j] * cs[i];
        acc[t][j] = v;
      }
    }
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
  if constexpr (EPI == EPI_PLAIN) {
    // The plain epilogue writes 64 columns x 128 rows of bf16 per wave: through LDS, 64 rows at
    // a time (rows of EPS bytes, padded so the 16 lanes of a write phase hit distinct banks),
    // then out as 16 bytes per lane, one 128-byte line per row, instead of 8-byte pieces.
    constexpr int EPS = 136;
    static_assert(8 * 64 * EPS <= D * STAGE_B, "epilogue staging exceeds the LDS ring");
    __syncthreads();  // every wave is done with the ring
    uint8_t* ep = lds + wave * 64 * EPS;
    const int col0 = ftile[0] * 16;  // this wave's 64 consecutive output columns
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int f = 0; f < WF; ++f) {
          const f32x4 v = acc[f][4 * hh + j];
          *(u32x2*)(ep + (j * 16 + j16) * EPS + (f * 16 + 4 * g4) * 2) =
              u32x2{pack_bf16x2(v[0] * mcur[0], v[1] * mcur[0]), pack_bf16x2(v[2] * mcur[0], v[3] * mcur[0])};
        }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = k * 8 + (lane >> 3);
        const int rr = wrow * 128 + hh * 64 + r;
        const u32x4 v = *(const u32x4*)(ep + r * EPS + (lane & 7) * 16);
        if (rr < nr) {
          const size_t row = (size_t)((long long)row0 + rr + rowoff);
          *(u32x4*)(out + (row * ldo + col0) * 2 + (lane & 7) * 16) = v;
        }
      }
    }
    return;
  }
  if constexpr (EPI == EPI_SWIGLU_Q8) {
    // h = SiLU(g) * u, rounded to bf16 (the type the layer keeps h in), then OCP MXFP8 for the W4A8
    // down product. This wave's 32 h columns of a row (2 tiles x 16) are exactly one 32-block: the
    // lane's 8 values and those of the lanes 16 and 32 apart (same row) make it, so the block
    // maximum takes two xor shuffles. Codes go to out ([row][ldo] bytes), exponents to out_scale
    // ([row][ldo / 32]).
    static_assert(WF == 2, "one MX block per wave and row");
    const int hc0 = ftile[0] * 16;  // this wave's first h column
    uint8_t* osc = (uint8_t*)a.out_scale;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = wrow * 128 + j * 16 + j16;
      float v[2][4];
      float amax = 0.f;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[f][i] = (float)(__bf16)(silu(acc[f][j][i] * mcur[0]) * (acc[WF + f][j][i] * mcur[1]));
          amax = __builtin_fmaxf(amax, __builtin_fabsf(v[f][i]));
        }
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
      const int X = mxfp8_exponent(amax);
      if (rr >= nr) continue;
      const size_t row = (size_t)((long long)row0 + rr + rowoff);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= e4m3_rne_sat(__builtin_amdgcn_ldexpf(v[f][i], -X)) << (8 * i);
        *(uint32_t*)(out + row * ldo + hc0 + 16 * f + 4 * g4) = w;
      }
      if (g4 == 0) osc[row * (ldo / 32) + hc0 / 32] = (uint8_t)(X + 127);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rr = wrow * 128 + j * 16 + j16;
    if (rr >= nr) continue;
    const size_t row = (size_t)((long long)row0 + rr + rowoff);
    if constexpr (EPI == EPI_F32) {
      // fp32 partial scores of split-K part blockIdx.y
      const size_t prow = row + (size_t)blockIdx.y * a.M;
#pragma unroll
      for (int f = 0; f < WF; ++f) {
        const int n = ftile[f] * 16 + 4 * g4;
        *(f32x4*)(out + (prow * ldo + n) * 4) = acc[f][j];
      }
      continue;
    }
#pragma unroll
    for (int f = 0; f < WF; ++f) {
      const int n = ftile[f] * 16 + 4 * g4;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = (EPI == EPI_SWIGLU) ? silu(acc[f][j][i] * mcur[0]) * (acc[WF + f][j][i] * mcur[NMAT - 1])
                                   : acc[f][j][i] * mcur[0];
      *(u32x2*)(out + (row * ldo + n) * 2) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

template <int C, int EPI>
static hipError_t launch_p(const GroupedArgs& a, int max_units, hipStream_t st) {
  GroupedArgs b = a;
  b.NTW = a.N / PEpi<EPI>::FULL_F;
  long long n = (long long)max_units * (b.NTW / 2);
  n = (n + NXCD - 1) / NXCD * NXCD;
  if (n == 0) return hipSuccess;
  grouped_prefill_kernel<C, EPI><<<(unsigned)n, PTHREADS, 0, st>>>(b);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_codec(int c, const GroupedArgs& a, int max_units, hipStream_t st) {
  if (c == MOE_BF16) return launch_p<MOE_BF16, EPI>(a, max_units, st);
  if (c == MOE_FP8_E4M3_B128) return launch_p<MOE_FP8_E4M3_B128, EPI>(a, max_units, st);
  if (c == MOE_MXFP4_B32) return launch_p<MOE_MXFP4_B32, EPI>(a, max_units, st);
  return hipErrorInvalidValue;
}

int prefill_row_tile() { return PRB; }

// Router scores of many tokens: x[M, K] (bf16) times the packed bf16 Wr[K, N] -> fp32
// partials out[ksplit][M][ldo]; N a multiple of 256, K a multiple of 32.
bool prefill_scores_supported(int act, int K, int N) {
  return act == MOE_BF16 && K % PCodec<MOE_BF16>::PBK == 0 && K <= 64 * 128 && N % PEpi<EPI_F32>::FULL_F == 0;
}

hipError_t launch_prefill_scores(const GroupedArgs& a, hipStream_t st) {
  if (a.cum_blocks || a.gather || !prefill_scores_supported(MOE_BF16, a.K, a.N)) return hipErrorInvalidValue;
  GroupedArgs b = a;
  b.NTW = a.N / PEpi<EPI_F32>::FULL_F;
  long long n = (long long)(a.M + PBM - 1) / PBM * b.NTW;
  n = (n + NXCD - 1) / NXCD * NXCD;
  if (n == 0) return hipSuccess;
  const int ks = a.ksplit > 1 ? a.ksplit : 1;
  grouped_prefill_kernel<MOE_BF16, EPI_F32><<<dim3((unsigned)n, (unsigned)ks), PTHREADS, 0, st>>>(b);
  return hipGetLastError();
}

static bool prefill_codec_ok(int c, int K) {
  int pbk = 0;
  if (c == MOE_BF16) pbk = PCodec<MOE_BF16>::PBK;
  else if (c == MOE_FP8_E4M3_B128) pbk = PCodec<MOE_FP8_E4M3_B128>::PBK;
  else if (c == MOE_MXFP4_B32) pbk = PCodec<MOE_MXFP4_B32>::PBK;
  else if (c == MOE_MXFP4_B32_A8) pbk = PCodec<MOE_MXFP4_B32_A8>::PBK;
  else if (c == MOE_MXFP8_B32_A8) pbk = PCodec<MOE_MXFP8_B32_A8>::PBK;
  else if (c == MOE_INT8_W8A8) pbk = PCodec<MOE_INT8_W8A8>::PBK;
  else return false;
  return K % pbk == 0 && K % 128 == 0 && K <= 64 * 128;
}

bool prefill_supported(int act, int cr, int cs, int K, int N_gateup, int N_down) {
  return act == MOE_BF16 && prefill_codec_ok(cr, K) && prefill_codec_ok(cs, K) &&
         N_gateup % (2 * PEpi<EPI_SWIGLU>::FULL_F) == 0 && N_down % (2 * PEpi<EPI_PLAIN>::FULL_F) == 0;
}

// W4A8 routed groups [g_begin, g_end): gate/up with the MXFP8-writing SwiGLU epilogue, or down.
hipError_t launch_w4a8_prefill(int epi, const GroupedArgs& a, int max_units, hipStream_t st) {
  if (!prefill_codec_ok(MOE_MXFP4_B32_A8, a.K) || !a.act_scale) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU_Q8) {
    if (a.N % (2 * PEpi<EPI_SWIGLU_Q8>::FULL_F) || !a.out_scale) return hipErrorInvalidValue;
    return launch_p<MOE_MXFP4_B32_A8, EPI_SWIGLU_Q8>(a, max_units, st);
  }
  if (epi == EPI_PLAIN) {
    if (a.N % (2 * PEpi<EPI_PLAIN>::FULL_F)) return hipErrorInvalidValue;
    return launch_p<MOE_MXFP4_B32_A8, EPI_PLAIN>(a, max_units, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_int8_prefill(int epi, const GroupedArgs& a, int max_units, hipStream_t st) {
  if (!prefill_codec_ok(MOE_INT8_W8A8, a.K) || !a.act_scale) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU) {
    if (a.N % (2 * PEpi<EPI_SWIGLU>::FULL_F)) return hipErrorInvalidValue;
    return launch_p<MOE_INT8_W8A8, EPI_SWIGLU>(a, max_units, st);
  }
  if (epi == EPI_PLAIN) {
    if (a.N % (2 * PEpi<EPI_PLAIN>::FULL_F)) return hipErrorInvalidValue;
    return launch_p<MOE_INT8_W8A8, EPI_PLAIN>(a, max_units, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_w8a8_shared(int epi, const GroupedArgs& a, int rows, hipStream_t st) {
  if (!prefill_codec_ok(MOE_MXFP8_B32_A8, a.K) || !a.act_scale || !a.cum_blocks || !a.group_range ||
      a.g_end != a.g_begin + 1 || rows < 0)
    return hipErrorInvalidValue;
  auto go = [&](auto epi_c) -> hipError_t {
    constexpr int EPI = decltype(epi_c)::value;
    if (a.N % PEpi<EPI>::FULL_F) return hipErrorInvalidValue;
    GroupedArgs b = a;
    b.NTW = a.N / PEpi<EPI>::FULL_F;
    long long n = (long long)(rows + PBM - 1) / PBM * b.NTW;  // the kernel's item count for the group
    n = (n + NXCD - 1) / NXCD * NXCD;
    if (n == 0) return hipSuccess;
    grouped_prefill_kernel<MOE_MXFP8_B32_A8, EPI><<<(unsigned)n, PTHREADS, 0, st>>>(b);
    return hipGetLastError();
  };
  if (epi == EPI_SWIGLU_Q8) return a.out_scale ? go(std::integral_constant<int, EPI_SWIGLU_Q8>{}) : hipErrorInvalidValue;
  if (epi == EPI_PLAIN) return go(std::integral_constant<int, EPI_PLAIN>{});
  return hipErrorInvalidValue;
}

// One launch over all groups when routed and shared experts share a format; else one launch
// per format, over the routed groups [0, shared_group) and over the shared group.
hipError_t launch_grouped_prefill(int act, int epi, int cr, int cs, const GroupedArgs& a, int max_units,
                                  hipStream_t st) {
  if (act != MOE_BF16 || !prefill_codec_ok(cr, a.K) || !prefill_codec_ok(cs, a.K)) return hipErrorInvalidValue;
  if (epi != EPI_SWIGLU && epi != EPI_PLAIN) return hipErrorInvalidValue;
  if (a.N % (2 * (epi == EPI_SWIGLU ? PEpi<EPI_SWIGLU>::FULL_F : PEpi<EPI_PLAIN>::FULL_F))) return hipErrorInvalidValue;
  auto launch = [&](int c, const GroupedArgs& b, int units) {
    return epi == EPI_SWIGLU ? launch_codec<EPI_SWIGLU>(c, b, units, st) : launch_codec<EPI_PLAIN>(c, b, units, st);
  };
  if (cr == cs || a.shared_group < 0) return launch(cr, a, max_units);
  GroupedArgs r = a, sh = a;
  r.g_begin = 0;
  r.g_end = a.shared_group;
  sh.g_begin = a.shared_group;
  sh.g_end = a.shared_group + 1;
  hipError_t e = launch(cr, r, max_units);
  if (e != hipSuccess) return e;
  return launch(cs, sh, (a.M - a.P + PRB - 1) / PRB);
}

}  // namespace moe
