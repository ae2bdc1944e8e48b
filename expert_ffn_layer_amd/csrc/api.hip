// The C ABI (include/moe.h): argument validation, workspace layout and kernel orchestration.
// Host code only; every step of the layer runs in the kernels it enqueues.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "common.h"
#include "kernels.h"

using namespace moe;

extern "C" __attribute__((visibility("hidden"))) hipError_t moe_launch_pack(int fmt, int count, int K, int N, const void* w,
                                                                         const void* scale, void* packed,
                                                                         void* packed_scale, hipStream_t stream);

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t ALIGN = 256;
size_t up(size_t x, size_t a = ALIGN) { return (x + a - 1) / a * a; }
int act_bytes(moe_dtype a) { return a == MOE_F32 ? 4 : 2; }
int pad64(int n) { return (n + 63) / 64 * 64; }
int pad256(int n) { return (n + 255) / 256 * 256; }
constexpr int ROW_BLOCK = 64;

bool valid_fmt(int f) { return f >= MOE_F32 && f <= MOE_INT8_W8A8; }
// storage format: W4A8 weights are stored and packed as MXFP4
moe_dtype stored_fmt(moe_dtype f) { return f == MOE_MXFP4_B32_A8 ? MOE_MXFP4_B32 : f; }

// Bytes of `count` packed K x N matrices and of their packed scales.
moe_status packed_sizes(moe_dtype fmt, int count, int K, int N, size_t* bytes, size_t* sbytes) {
  if (!valid_fmt(fmt)) return fail(MOE_ERR_INVALID_ARG, "unknown weight format %d", (int)fmt);
  fmt = stored_fmt(fmt);
  if (count < 0 || K < 1 || N < 1) return fail(MOE_ERR_INVALID_ARG, "bad matrix size count=%d K=%d N=%d", count, K, N);
  const int KP = kp_of(fmt);
  if (K % KP) return fail(MOE_ERR_INVALID_ARG, "K=%d is not a multiple of %d for format %d", K, KP, (int)fmt);
  if (fmt == MOE_FP8_E4M3_B128 && (K % 128 || N % 128))
    return fail(MOE_ERR_INVALID_ARG, "fp8 block-128 scales need K, N multiples of 128 (K=%d N=%d)", K, N);
  if (fmt == MOE_MXFP4_B32 && N % 2) return fail(MOE_ERR_INVALID_ARG, "MXFP4 packs N=%d in pairs", N);
  if (fmt == MOE_MXFP8_B32_A8 && K % 128)
    return fail(MOE_ERR_INVALID_ARG, "MXFP8 scales are packed per 128 reduction elements (K=%d)", K);
  if (fmt == MOE_INT8_W8A8 && K % 128)
    return fail(MOE_ERR_INVALID_ARG, "INT8 products run 128 reduction elements per step (K=%d)", K);
  const size_t NT = pad256(N) / 16, KT = K / KP;
  *bytes = (size_t)count * NT * KT * PACKET_BYTES;
  if (fmt == MOE_FP8_E4M3_B128)
    *sbytes = (size_t)count * (K / 128) * (N / 128) * 4;
  else if (fmt == MOE_MXFP4_B32)
    *sbytes = (size_t)count * NT * KT * 64;
  else if (fmt == MOE_MXFP8_B32_A8)
    *sbytes = (size_t)count * NT * (K / 128) * 64;
  else if (fmt == MOE_INT8_W8A8)
    *sbytes = (size_t)count * NT * 16 * 4;
  else
    *sbytes = 0;
  return MOE_OK;
}

moe_status check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%d < 0", s->T);
  if (s->H < 128 || s->H % 128) return fail(MOE_ERR_INVALID_ARG, "H=%d must be a positive multiple of 128", s->H);
  if (s->I < 128 || s->I % 128) return fail(MOE_ERR_INVALID_ARG, "I=%d must be a positive multiple of 128", s->I);
  if (s->E < 1 || s->E > 1024) return fail(MOE_ERR_INVALID_ARG, "E=%d outside [1, 1024]", s->E);
  if (s->k < 1 || s->k > s->E || s->k > 16) return fail(MOE_ERR_INVALID_ARG, "k=%d outside [1, min(E, 16)]", s->k);
  if ((long long)s->T * s->k + s->T > 0x7fffffffLL / 2) return fail(MOE_ERR_INVALID_ARG, "T*k too large");
  // The plan's block table keeps a row block's place in its group in 16 bits. A group holds at
  // most T*k rows (hash routing may repeat an expert within a token; the shared group holds T),
  // cut into 64-row blocks on the decode kernel (128 on the prefill one).
  if ((long long)s->T * s->k > 65535LL * ROW_BLOCK)
    return fail(MOE_ERR_UNSUPPORTED, "T*k=%lld: a group of more than %lld rows overflows the plan's block index",
                (long long)s->T * s->k, 65535LL * ROW_BLOCK);
  if (s->I_shared != 0 && s->I_shared != s->I)
    return fail(MOE_ERR_UNSUPPORTED, "I_shared=%d: only 0 or I (=%d) is supported", s->I_shared, s->I);
  if (s->act != MOE_F32 && s->act != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "act must be F32 or BF16");
  if (!valid_fmt(s->w_routed) || (s->I_shared && !valid_fmt(s->w_shared)))
    return fail(MOE_ERR_INVALID_ARG, "unknown weight format");
  if (s->path < MOE_PATH_AUTO || s->path > MOE_PATH_PREFILL) return fail(MOE_ERR_INVALID_ARG, "bad path %d", (int)s->path);
  const bool f32 = s->act == MOE_F32;
  auto ok = [&](moe_dtype w) { return f32 ? w == MOE_F32 : w != MOE_F32; };
  if (!ok(s->w_routed) || (s->I_shared && !ok(s->w_shared)))
    return fail(MOE_ERR_UNSUPPORTED, "F32 weights go with F32 activations, every other format with BF16 ones");
  if (s->I_shared && s->w_shared == MOE_MXFP4_B32_A8)
    return fail(MOE_ERR_UNSUPPORTED, "W4A8 (MOE_MXFP4_B32_A8) applies to the routed experts only");
  if (s->w_routed == MOE_MXFP8_B32_A8)
    return fail(MOE_ERR_UNSUPPORTED, "W8A8 MXFP8 (MOE_MXFP8_B32_A8) applies to the shared expert only");
  if (s->I_shared && s->w_shared == MOE_MXFP8_B32_A8 && s->w_routed != MOE_MXFP4_B32_A8)
    return fail(MOE_ERR_UNSUPPORTED, "a W8A8 MXFP8 shared expert needs W4A8 routed experts (MOE_MXFP4_B32_A8)");
  const bool ri8 = s->w_routed == MOE_INT8_W8A8, si8 = s->I_shared && s->w_shared == MOE_INT8_W8A8;
  if ((ri8 && s->I_shared && !si8) || (si8 && !ri8))
    return fail(MOE_ERR_UNSUPPORTED, "INT8 W8A8 experts: routed and shared both INT8 (or no shared expert)");
  if (s->w_routed == MOE_INT8_W8A8 &&
      (!prefill_supported(s->act, s->w_routed, s->w_routed, s->H, s->I, s->H) ||
       !prefill_supported(s->act, s->w_routed, s->w_routed, s->I, s->I, s->H)))
    return fail(MOE_ERR_UNSUPPORTED,
                "INT8 W8A8 experts need BF16 activations, I a multiple of 256 and H a multiple of 512");
  if (s->w_routed == MOE_MXFP4_B32_A8 &&
      (!prefill_supported(s->act, s->w_routed, s->I_shared ? s->w_shared : s->w_routed, s->H, s->I, s->H) ||
       !prefill_supported(s->act, s->w_routed, s->I_shared ? s->w_shared : s->w_routed, s->I, s->I, s->H)))
    return fail(MOE_ERR_UNSUPPORTED,
                "W4A8 routed experts need BF16 activations, I a multiple of 256 and H a multiple of 512");
  if (s->path == MOE_PATH_PREFILL &&
      (!prefill_supported(s->act, s->w_routed, s->I_shared ? s->w_shared : s->w_routed, s->H, s->I, s->H) ||
       !prefill_supported(s->act, s->w_routed, s->I_shared ? s->w_shared : s->w_routed, s->I, s->I, s->H)))
    return fail(MOE_ERR_UNSUPPORTED,
                "the prefill path needs BF16 activations, BF16 / FP8 / MXFP4 weights, I a multiple of 256 "
                "and H a multiple of 512");
  return MOE_OK;
}

// Split-K factor of the router scores: enough workgroups (about 512) to stream Wr at full rate
// when T is small; every part keeps at least 8 packets of the reduction.
int router_ksplit(const moe_shape& s) {
  if (s.T <= 0) return 1;
  const int rbk = (s.T + ROW_BLOCK - 1) / ROW_BLOCK;
  const int ntw = pad64(s.E) / 16 / decode_nf(s.act, EPI_F32, s.H, pad64(s.E));
  const int KT = s.H / kp_of(s.act);
  int ks = (512 + rbk * ntw - 1) / (rbk * ntw);
  ks = std::min(ks, std::max(1, KT / 8));
  return std::max(ks, 1);
}

// Router scores of many tokens run on the prefill kernel (256 x 256 MFMA tiles, x read once per
// 256 experts), split along H so that about one workgroup per CU is busy; few tokens use the
// decode kernel with router_ksplit.
struct RouterPlan {
  bool prefill;
  int ksplit;
};

RouterPlan router_plan(const moe_shape& s) {
  const int Ep = pad256(s.E);  // the packed router has its features padded to a multiple of 256
  if (s.T >= 2048 && prefill_scores_supported(s.act, s.H, Ep)) {
    const int items = (s.T + 255) / 256 * (Ep / 256);
    int ks = (256 + items - 1) / items;
    ks = std::min(ks, std::max(1, s.H / 32 / 16));  // at least 16 reduction steps per part
    return {true, std::max(ks, 1)};
  }
  return {false, router_ksplit(s)};
}

struct Ws {
  size_t logits, idx, w, offsets, slot_token, pair_slot, rank, hist, fhist, done, group_range, cum_blocks,
      block_group, cum_blocks_b, block_group_b, sh_range, sh_cum, sh_group, sh_cum_b, sh_group_b, zero, h, y_perm,
      y_shared, xq, xs, hq, hs, total;
};

// Decode batches route, permute and plan in one launch after the router scores (on the decode
// kernel, which clears the launch's completion count).
bool use_fused_route(const moe_shape& s) { return !router_plan(s).prefill && topk_permute_ok(s.T, s.k, s.E); }

Ws ws_layout(const moe_shape& s) {
  const size_t P = (size_t)s.T * s.k, S = s.I_shared ? 1 : 0, R = P + S * s.T;
  const size_t ab = act_bytes(s.act);
  Ws w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += up(bytes ? bytes : 1);
    return at;
  };
  w.logits = take((size_t)router_plan(s).ksplit * s.T * pad256(s.E) * 4);
  w.idx = take(P * 4);
  w.w = take(P * 4);
  w.offsets = take(((size_t)s.E + 1) * 4);
  w.slot_token = take(P * 4);
  w.pair_slot = take(P * 4);
  w.rank = take(P * 4);
  w.hist = take((size_t)permute_blocks((int)P) * s.E * 4);
  // the fused route-permute launch: per workgroup of 8 or 16 tokens an expert histogram, and its count
  w.fhist = take(use_fused_route(s) ? (size_t)((s.T + 7) / 8) * s.E * 4 : 0);
  w.done = take(4);
  w.group_range = take(((size_t)s.E + 1) * 8);
  w.cum_blocks = take(((size_t)s.E + 2) * 4);
  // one entry per row block: at most one partial block per group plus the full ones (64-row
  // blocks at decode, 128 at prefill)
  w.block_group = take(((size_t)s.E + 2 + (R + ROW_BLOCK - 1) / ROW_BLOCK) * 4);
  // the down product's table when gate/up runs thick blocks (64-row blocks only)
  w.cum_blocks_b = take(((size_t)s.E + 2) * 4);
  w.block_group_b = take(((size_t)s.E + 2 + (R + ROW_BLOCK - 1) / ROW_BLOCK) * 4);
  // the plan of the shared expert alone, when it runs beside the routed experts (one group)
  const size_t shb = S ? 3 + ((size_t)s.T + ROW_BLOCK - 1) / ROW_BLOCK : 0;
  w.sh_range = take(S * 8);
  w.sh_cum = take(S * 8);
  w.sh_group = take(shb * 4);
  w.sh_cum_b = take(S * 8);
  w.sh_group_b = take(shb * 4);
  w.h = take(R * s.I * ab);
  w.y_perm = take(P * s.H * ab);
  w.y_shared = take(S * s.T * s.H * ab);
  w.zero = take((size_t)std::max(s.H, s.I) * ab);  // zero activations for prefill padding rows
  if (s.w_routed == MOE_MXFP4_B32_A8) {
    // W4A8: MXFP8 codes and exponents of x (token rows) and of the rows of h that the W4A8 and
    // W8A8 products read (the routed rows, then the shared expert's with a W8A8 shared expert)
    const size_t QR = P + (S && s.w_shared == MOE_MXFP8_B32_A8 ? (size_t)s.T : 0);
    w.xq = take((size_t)s.T * s.H);
    w.xs = take((size_t)s.T * (s.H / 32));
    w.hq = take(QR * s.I);
    w.hs = take(QR * (s.I / 32));
  } else if (s.w_routed == MOE_INT8_W8A8) {
    // Int8 W8A8: int8 codes and fp32 per-row scales of x and of every row of h
    w.xq = take((size_t)s.T * s.H);
    w.xs = take((size_t)s.T * 4);
    w.hq = take(R * s.I);
    w.hs = take(R * 4);
  }
  w.total = o;
  return w;
}

moe_status check_ws(const moe_shape& s, void* ws, size_t ws_bytes, Ws* out) {
  *out = ws_layout(s);
  if (!ws && out->total) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < out->total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, out->total);
  if ((uintptr_t)ws % ALIGN) return fail(MOE_ERR_INVALID_ARG, "workspace must be %zu-byte aligned", ALIGN);
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

// The kernels move activations, outputs and packed matrices with 16-byte vector loads and DMA to
// LDS, and scales, index and weight arrays with 4-byte ones: such pointers must be aligned to that
// (every PyTorch allocation is), or the call is refused before any launch.
bool al16(const void* p) { return (uintptr_t)p % 16 == 0; }
bool al4(const void* p) { return (uintptr_t)p % 4 == 0; }
moe_status misaligned(const char* what, int bytes) {
  return fail(MOE_ERR_INVALID_ARG, "%s must be %d-byte aligned", what, bytes);
}

moe_status check_weights(const moe_weights* w, moe_dtype fmt, const char* what) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "%s weights are NULL", what);
  if (!w->gate || !w->up || !w->down) return fail(MOE_ERR_INVALID_ARG, "%s weight pointer is NULL", what);
  if ((fmt == MOE_FP8_E4M3_B128 || fmt == MOE_MXFP4_B32 || fmt == MOE_MXFP4_B32_A8 || fmt == MOE_MXFP8_B32_A8 ||
       fmt == MOE_INT8_W8A8) &&
      (!w->gate_scale || !w->up_scale || !w->down_scale))
    return fail(MOE_ERR_INVALID_ARG, "%s scales are NULL", what);
  if (!al16(w->gate) || !al16(w->up) || !al16(w->down)) return misaligned("packed weights", 16);
  if (!al4(w->gate_scale) || !al4(w->up_scale) || !al4(w->down_scale)) return misaligned("packed scales", 4);
  return MOE_OK;
}

// Hash routing's inputs: the experts of token t are row ids[t] of table[vocab][k].
struct HashRoute {
  const int32_t* ids;
  const int32_t* table;
  int vocab;
};

// The router scores into the workspace (split-K fp32 partials of the padded experts); `clear`:
// a word the decode score kernel sets to 0. Returns the row stride of the partials in *ldl.
moe_status do_scores(const moe_shape& s, const void* x, const void* Wr, void* ws, const Ws& L, hipStream_t st,
                     int* ldl, uint32_t* clear = nullptr) {
  const RouterPlan rp = router_plan(s);
  // scores of the padded experts: 256-wide MFMA tiles on the prefill kernel, 64 on the decode one
  const int Ep = rp.prefill ? pad256(s.E) : pad64(s.E);
  GroupedArgs a{};
  a.group_range = nullptr;
  a.cum_blocks = nullptr;
  a.G = 1;
  a.shared_group = -1;
  a.P = s.T;
  a.M = s.T;
  a.gather = nullptr;
  a.act = x;
  a.lda = s.H;
  a.act_rows = s.T;
  a.wa_r = (const uint8_t*)Wr;
  a.mat_bytes = 0;
  a.K = s.H;
  a.N = Ep;
  a.out = at<float>(ws, L.logits);
  a.ldo = Ep;
  a.ksplit = rp.ksplit;
  a.clear_word = clear;
  if (clear && rp.prefill) return fail(MOE_ERR_HIP, "internal: the prefill score kernel clears no word");
  *ldl = Ep;
  return hip_status(rp.prefill ? launch_prefill_scores(a, st)
                               : launch_grouped_decode(s.act, EPI_F32, s.act, s.act, a, (s.T + ROW_BLOCK - 1) / ROW_BLOCK, st),
                    "router scores");
}

// moe_route (or moe_route_hash, with `hash`) without the argument checks.
moe_status do_route(const moe_shape& s, const void* x, const void* Wr, const float* bias, int32_t* idx,
                    float* w, void* ws, const Ws& L, hipStream_t st, const HashRoute* hash = nullptr) {
  if (s.T == 0) return MOE_OK;
  int ldl;
  moe_status rs = do_scores(s, x, Wr, ws, L, st, &ldl);
  if (rs != MOE_OK) return rs;
  hipError_t e = launch_topk(at<float>(ws, L.logits), ldl, router_plan(s).ksplit, bias, s.T, s.E, s.k,
                             hash ? hash->ids : nullptr, hash ? hash->table : nullptr, hash ? hash->vocab : 0, idx, w, st);
  return hip_status(e, hash ? "hash routing" : "router top-k");
}

// The LDS-tiled MFMA kernel when the experts average at least 64 rows (or when asked for and
// supported: bf16 activations, one weight format for routed and shared experts, bf16 or fp8).
bool use_prefill(const moe_shape& s) {
  const int cs = s.I_shared ? s.w_shared : s.w_routed;
  if (!prefill_supported(s.act, s.w_routed, cs, s.H, s.I, s.H) || !prefill_supported(s.act, s.w_routed, cs, s.I, s.I, s.H))
    return false;
  if (s.path == MOE_PATH_PREFILL) return true;
  if (s.path == MOE_PATH_DECODE) return false;
  return (long long)s.T * s.k >= 64LL * s.E;
}

// Decode batches cut the groups of more than 64 rows into blocks of up to 256 for the gate/up product:
// each wave of such an item runs 64 rows over the whole reduction, so the four waves stream each
// weight tile together (one HBM read, the other three from cache) instead of once per 64-row block.
// Its kernel must run 4 row tiles per wave: f32, bf16 or Int8 weights, the same format for the routed
// and shared experts (one launch). The down product, whose reduction is short, keeps 64-row blocks
// (a plan table of its own).
int decode_thick_rows(const moe_shape& s) {
  if (use_prefill(s)) return 0;
  if (s.I_shared && s.w_shared != s.w_routed) return 0;
  if (s.w_routed != MOE_F32 && s.w_routed != MOE_BF16 && s.w_routed != MOE_INT8_W8A8) return 0;
  return 4 * ROW_BLOCK;
}

// with_plan: also write the grouped-GEMM plan into the workspace (returns whether it did)
moe_status do_permute(const moe_shape& s, const int32_t* idx, int32_t* off, int32_t* st_, int32_t* ps, void* ws,
                      const Ws& L, hipStream_t st, bool with_plan = false, bool* planned = nullptr,
                      bool shared_in_plan = true) {
  if (planned) *planned = false;
  if (s.T == 0) return hip_status(launch_fill_i32(off, 0, s.E + 1, st), "permute (empty)");
  hipError_t e;
  if (permute_small_ok(s.T * s.k, s.E)) {
    e = launch_permute_small(idx, s.T, s.k, s.E, s.I_shared && shared_in_plan ? 1 : 0, ROW_BLOCK, decode_thick_rows(s),
                             off, st_, ps,
                             with_plan ? at<int32_t>(ws, L.group_range) : nullptr, at<int32_t>(ws, L.cum_blocks),
                             at<int32_t>(ws, L.block_group), at<int32_t>(ws, L.cum_blocks_b),
                             at<int32_t>(ws, L.block_group_b), st);
    if (planned) *planned = with_plan;
  } else {
    e = launch_permute(idx, s.T, s.k, s.E, off, st_, ps, at<int32_t>(ws, L.rank), at<int32_t>(ws, L.hist), st);
  }
  return hip_status(e, "permute");
}

moe_status record(hipEvent_t ev, hipStream_t st) {
  return ev ? hip_status(hipEventRecord(ev, st), "event record") : MOE_OK;
}

// Route and permute (and, for the layer, the decode plan). Decode batches run the scores, then the
// selection, permutation and plan in one launch; other shapes route and permute as moe_route and
// moe_permute do. ev (optional): ev[1] is recorded after the scores (fused) or the routing.
moe_status do_route_permute(const moe_shape& s, const void* x, const void* Wr, const float* bias, int32_t* idx,
                            float* w, int32_t* off, int32_t* slot_token, int32_t* pair_slot, void* ws, const Ws& L,
                            hipStream_t st, hipEvent_t const* ev, const HashRoute* hash, bool* planned,
                            bool shared_in_plan = true) {
  moe_status rs;
  *planned = false;
  if (s.T == 0) return do_permute(s, idx, off, slot_token, pair_slot, ws, L, st);
  if (!use_fused_route(s)) {
    if ((rs = do_route(s, x, Wr, bias, idx, w, ws, L, st, hash)) != MOE_OK) return rs;
    if (ev && (rs = record(ev[1], st)) != MOE_OK) return rs;
    return do_permute(s, idx, off, slot_token, pair_slot, ws, L, st, true, planned, shared_in_plan);
  }
  int ldl;
  uint32_t* done = at<uint32_t>(ws, L.done);
  if ((rs = do_scores(s, x, Wr, ws, L, st, &ldl, done)) != MOE_OK) return rs;
  if (ev && (rs = record(ev[1], st)) != MOE_OK) return rs;
  const hipError_t e = launch_topk_permute(
      at<float>(ws, L.logits), ldl, router_plan(s).ksplit, bias, s.T, s.E, s.k, hash ? hash->ids : nullptr,
      hash ? hash->table : nullptr, hash ? hash->vocab : 0, idx, w, at<int32_t>(ws, L.rank), at<int32_t>(ws, L.fhist),
      done, s.I_shared && shared_in_plan ? 1 : 0, ROW_BLOCK, decode_thick_rows(s), off, slot_token, pair_slot,
      at<int32_t>(ws, L.group_range),
      at<int32_t>(ws, L.cum_blocks), at<int32_t>(ws, L.block_group), at<int32_t>(ws, L.cum_blocks_b),
      at<int32_t>(ws, L.block_group_b), st);
  if ((rs = hip_status(e, hash ? "hash routing and permutation" : "router top-k and permutation")) != MOE_OK) return rs;
  *planned = true;
  return MOE_OK;
}

// ev (optional, 3 events): recorded after the plan, after gate/up and after down.
// The launches of one FFN pass (gate/up, then down) on the kernel family the shape selects; the
// per-format rules for the activation operand live here, the argument set-up in do_ffn.
struct FfnPass {
  const moe_shape& s;
  void* ws;
  const Ws& L;
  hipStream_t st;
  bool prefill;
  int P, S;
  int cr;      // the format of the launch's routed groups (the shared one for the shared expert alone)
  int cs;      // the shared expert's format (the routed one when there is none)
  int max_rb;  // row blocks the launch grid covers

  // bf16 activations: one launch over the routed and shared groups
  hipError_t plain(int epi, const GroupedArgs& a) const {
    return prefill ? launch_grouped_prefill(s.act, epi, cr, cs, a, max_rb, st)
                   : launch_grouped_decode(s.act, epi, cr, cs, a, max_rb, st);
  }

  // Int8 W8A8: int8 codes and per-row scales of the activations (rows and gather as in a), one
  // launch over the routed and shared groups; h comes out in bf16
  hipError_t int8(int epi, const GroupedArgs& a, const void* codes, const void* scales) const {
    GroupedArgs ia = a;
    ia.act = codes;
    ia.act_scale = scales;
    return prefill ? launch_int8_prefill(epi, ia, max_rb, st)
                   : launch_grouped_decode(s.act, epi, MOE_INT8_W8A8, MOE_INT8_W8A8, ia, max_rb, st);
  }

  // W4A8: the routed groups multiply MXFP8 codes of the activations (rows of K, gathered through
  // gather, or read in order when it is null). On the prefill kernel gate/up writes h as MXFP8 for
  // the down product; on the decode kernel it writes h in bf16, quantised before down. The shared
  // expert keeps its own launch, on the bf16 activations of base unless it is MXFP8 itself.
  hipError_t w4a8(int epi, const GroupedArgs& base, const void* codes, const void* scales, int K, int rows,
                  const int32_t* gather) const {
    const bool swiglu = epi == EPI_SWIGLU;
    GroupedArgs ra = base;
    ra.gather = gather;
    ra.act = codes;
    ra.lda = K;
    ra.act_rows = rows;
    ra.act_scale = scales;
    ra.g_begin = 0;
    ra.g_end = s.E;
    if (prefill && swiglu) to_mxfp8_h(ra);
    hipError_t r = prefill ? launch_w4a8_prefill(swiglu ? EPI_SWIGLU_Q8 : epi, ra, max_rb, st)
                           : launch_grouped_decode(s.act, epi, MOE_MXFP4_B32_A8, MOE_MXFP4_B32_A8, ra, max_rb, st);
    if (r != hipSuccess || !S) return r;
    GroupedArgs sa = base;
    sa.g_begin = s.E;
    sa.g_end = s.E + 1;
    const int shared_rb = (s.T + ROW_BLOCK - 1) / ROW_BLOCK;
    if (cs != MOE_MXFP8_B32_A8)
      return prefill ? launch_grouped_prefill(s.act, epi, cs, cs, sa, max_rb, st)
                     : launch_grouped_decode(s.act, epi, cs, cs, sa, shared_rb, st);
    // W8A8 MXFP8 shared expert: the same MXFP8 rows of x (token t is row P + t of the group) and
    // of h, whose shared rows follow the routed ones
    sa.act = codes;
    sa.lda = K;
    sa.act_scale = scales;
    sa.gather = swiglu ? gather : nullptr;
    sa.act_rows = swiglu ? rows : P + s.T;
    if (!prefill)
      return launch_grouped_decode(s.act, epi, MOE_MXFP8_B32_A8, MOE_MXFP8_B32_A8, sa, shared_rb, st);
    if (swiglu) to_mxfp8_h(sa);
    return launch_w8a8_shared(swiglu ? EPI_SWIGLU_Q8 : epi, sa, s.T, st);
  }

  // the prefill kernels' gate/up epilogue writes h straight to MXFP8 codes and exponents
  void to_mxfp8_h(GroupedArgs& a) const {
    a.out = at<void>(ws, L.hq);
    a.ldo = s.I;
    a.out_scale = at<void>(ws, L.hs);
  }

  // h (bf16, rows 0..rows-1 of the workspace) to the activation format of the down product;
  // nothing for the formats whose gate/up epilogue already wrote it there
  hipError_t quantise_h(bool a8, bool i8) const {
    if (a8 && !prefill) {
      // the routed rows, and those of a W8A8 MXFP8 shared expert after them
      const int rows = P + (S && cs == MOE_MXFP8_B32_A8 ? s.T : 0);
      return launch_quant_mxfp8(at<void>(ws, L.h), rows, s.I, at<uint8_t>(ws, L.hq), at<uint8_t>(ws, L.hs), st);
    }
    if (i8) return launch_quant_int8(at<void>(ws, L.h), P + S * s.T, s.I, at<int8_t>(ws, L.hq), at<float>(ws, L.hs), st);
    return hipSuccess;
  }
};

// the weights of one product: gate and up (two matrices, the SwiGLU pair) or down (one)
void set_weights(GroupedArgs& a, const moe_weights& r, const moe_weights* sh, bool gate_up, size_t mat_bytes,
                 size_t scale_bytes) {
  a.wa_r = (const uint8_t*)(gate_up ? r.gate : r.down);
  a.wb_r = gate_up ? (const uint8_t*)r.up : nullptr;
  a.sa_r = (const uint8_t*)(gate_up ? r.gate_scale : r.down_scale);
  a.sb_r = gate_up ? (const uint8_t*)r.up_scale : nullptr;
  if (sh) {
    a.wa_s = (const uint8_t*)(gate_up ? sh->gate : sh->down);
    a.wb_s = gate_up ? (const uint8_t*)sh->up : nullptr;
    a.sa_s = (const uint8_t*)(gate_up ? sh->gate_scale : sh->down_scale);
    a.sb_s = gate_up ? (const uint8_t*)sh->up_scale : nullptr;
  }
  a.mat_bytes = (long long)mat_bytes;
  a.scale_bytes = (long long)scale_bytes;
}

// Which groups one do_ffn call runs: all of them, the routed experts alone, or the shared expert
// alone (its own plan: one group of rows P .. P + T - 1, x read in token order).
enum FfnPart { FFN_ALL, FFN_ROUTED, FFN_SHARED };

moe_status do_ffn(const moe_shape& s, const void* x, const int32_t* off, const int32_t* slot_token,
                  const moe_weights& r, const moe_weights* sh, void* y_perm, void* y_shared, void* ws, const Ws& L,
                  hipStream_t st, hipEvent_t const* ev = nullptr, bool plan_ready = false, FfnPart part = FFN_ALL) {
  if (s.T == 0) return MOE_OK;
  const bool only_sh = part == FFN_SHARED;
  if (only_sh && (!s.I_shared || !sh)) return fail(MOE_ERR_INVALID_ARG, "no shared expert");
  const int P = s.T * s.k, S = s.I_shared && part != FFN_ROUTED ? 1 : 0, E = only_sh ? 0 : s.E, G = E + S;
  size_t mb1, sb1, mb2, sb2;
  moe_status ps = packed_sizes(s.w_routed, 1, s.H, s.I, &mb1, &sb1);
  if (ps != MOE_OK) return ps;
  ps = packed_sizes(s.w_routed, 1, s.I, s.H, &mb2, &sb2);
  if (ps != MOE_OK) return ps;
  int32_t* gr = at<int32_t>(ws, only_sh ? L.sh_range : L.group_range);
  int32_t* cb = at<int32_t>(ws, only_sh ? L.sh_cum : L.cum_blocks);
  const bool prefill = use_prefill(s);
  const int rb = prefill ? prefill_row_tile() : ROW_BLOCK;
  hipError_t e = hipSuccess;
  uint32_t* zero = prefill ? at<uint32_t>(ws, L.zero) : nullptr;
  const int zero_words = (int)((size_t)std::max(s.H, s.I) * act_bytes(s.act) / 4);
  int32_t* bg = at<int32_t>(ws, only_sh ? L.sh_group : L.block_group);
  const int thick = decode_thick_rows(s);
  int32_t* cb2 = at<int32_t>(ws, only_sh ? L.sh_cum_b : L.cum_blocks_b);
  int32_t* bg2 = at<int32_t>(ws, only_sh ? L.sh_group_b : L.block_group_b);
  if (!plan_ready || prefill)
    e = launch_plan(off, E, P, s.T, S, rb, thick, gr, cb, bg, cb2, bg2, zero, zero_words, st);
  if (e != hipSuccess) return hip_status(e, "plan");
  moe_status rs;
  if (ev && (rs = record(ev[0], st)) != MOE_OK) return rs;
  const int max_rb = std::min(E, P) + (only_sh ? 0 : (P + rb - 1) / rb) + S * ((s.T + rb - 1) / rb);
  const bool a8 = s.w_routed == MOE_MXFP4_B32_A8, i8 = s.w_routed == MOE_INT8_W8A8;
  if (only_sh && (a8 || i8)) return fail(MOE_ERR_UNSUPPORTED, "the shared expert alone: quantised activations");
  const int cs = s.I_shared ? (int)s.w_shared : (int)s.w_routed;
  // the shared expert alone runs the kernel instantiation that the single-stream launch gives its
  // group: on the decode kernel the (routed, shared) pair of codecs, whose work split the routed
  // format sets; the prefill kernel already runs a shared expert of another format on its own
  const FfnPass f{s, ws, L, st, prefill, P, S, only_sh && prefill ? cs : (int)s.w_routed, S ? cs : (int)s.w_routed,
                  max_rb};

  GroupedArgs a{};
  a.zero_row = zero;
  a.thick_rows = thick;
  a.group_range = gr;
  a.cum_blocks = cb;
  a.block_group = bg;
  a.G = G;
  a.shared_group = S ? E : -1;
  a.P = P;
  a.M = P + S * s.T;
  // gate/up with the SwiGLU epilogue: h = SiLU(x Wg) * (x Wu), x gathered per slot
  a.gather = slot_token;
  a.act = x;
  a.lda = s.H;
  a.act_rows = s.T;
  set_weights(a, r, S ? sh : nullptr, true, mb1, sb1);
  a.K = s.H;
  a.N = s.I;
  a.out = at<void>(ws, L.h);
  a.ldo = s.I;
  a.out_s = nullptr;
  if (only_sh) set_weights(a, *sh, sh, true, mb1, sb1);  // group 0 is the shared expert
  if (a8) {
    // x to MXFP8 once per token; the codes are gathered like x
    e = launch_quant_mxfp8(x, s.T, s.H, at<uint8_t>(ws, L.xq), at<uint8_t>(ws, L.xs), st);
    if (e != hipSuccess) return hip_status(e, "MXFP8 quantisation of x");
    e = f.w4a8(EPI_SWIGLU, a, at<void>(ws, L.xq), at<void>(ws, L.xs), s.H, s.T, slot_token);
  } else if (i8) {
    // x to int8 per token
    e = launch_quant_int8(x, s.T, s.H, at<int8_t>(ws, L.xq), at<float>(ws, L.xs), st);
    if (e != hipSuccess) return hip_status(e, "int8 quantisation of x");
    e = f.int8(EPI_SWIGLU, a, at<void>(ws, L.xq), at<void>(ws, L.xs));
  } else {
    e = f.plain(EPI_SWIGLU, a);
  }
  if (e != hipSuccess) return hip_status(e, "gate/up grouped GEMM");
  if (ev && (rs = record(ev[1], st)) != MOE_OK) return rs;
  e = f.quantise_h(a8, i8);
  if (e != hipSuccess) return hip_status(e, "quantisation of h");

  // down: y = h Wd, the routed rows to y_perm and the shared ones to y_shared (64-row blocks)
  if (thick) {
    a.cum_blocks = cb2;
    a.block_group = bg2;
    a.thick_rows = 0;
  }
  a.gather = nullptr;
  a.act = at<void>(ws, L.h);
  a.lda = s.I;
  a.act_rows = P + S * s.T;
  set_weights(a, only_sh ? *sh : r, S ? sh : nullptr, false, mb2, sb2);
  a.K = s.I;
  a.N = s.H;
  a.out = y_perm;
  a.ldo = s.H;
  a.out_s = S ? y_shared : nullptr;
  a.ldo_s = s.H;
  if (a8) e = f.w4a8(EPI_PLAIN, a, at<void>(ws, L.hq), at<void>(ws, L.hs), s.I, P, nullptr);
  else if (i8) e = f.int8(EPI_PLAIN, a, at<void>(ws, L.hq), at<void>(ws, L.hs));
  else e = f.plain(EPI_PLAIN, a);
  if (e != hipSuccess) return hip_status(e, "down grouped GEMM");
  return ev ? record(ev[2], st) : MOE_OK;
}

// The shared expert beside the routed ones ('CANN DeepSeek-V4推理优化', multi-stream parallelism:
// the shared expert needs no routing, so it runs on a second stream while the router, the
// permutation and the routed experts run on the caller's). Its FFN is the same grouped launch
// restricted to its one group, so every row gets the same arithmetic as in the single-stream
// order. Decode batches only: there the routing is a chain of short latency-bound kernels that
// leaves HBM idle for the shared expert's weights (the V4-Pro decode layer: 0.857 -> 0.836 ms);
// a prefill batch's kernels fill the GPU already, and the overlap measured no gain. Formats with
// quantised activations keep the single-stream order.
bool side_shared(const moe_shape& s) {
  if (!s.I_shared || s.T == 0 || use_prefill(s)) return false;
  const auto plain = [](int f) {
    return f == MOE_F32 || f == MOE_BF16 || f == MOE_FP8_E4M3_B128 || f == MOE_MXFP4_B32;
  };
  return plain(s.w_routed) && plain(s.w_shared);
}

// One second stream and its two events per calling thread and device, made on first use (default
// priority, non-blocking) and kept for the life of the thread. Thread-local, so a thread's fork
// and join events are never recorded by another thread between its record and its wait.
constexpr int MAX_SIDE_DEVICES = 64;
struct SideStream {
  bool made = false;
  hipError_t err = hipSuccess;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
thread_local SideStream t_side[MAX_SIDE_DEVICES];

// The current device's second stream for work on `stream`, or null when `stream` belongs to another
// device (the caller's launches then all stay on `stream`: *st is MOE_OK) or on an error (*st set).
SideStream* side_of_current_device(hipStream_t stream, moe_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_status(e, "hipGetDevice");
    return nullptr;
  }
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) {
      *st = hip_status(e, "hipStreamGetDevice");
      return nullptr;
    }
    if (sdev != dev) {
      *st = MOE_OK;
      return nullptr;
    }
  }
  if (dev < 0 || dev >= MAX_SIDE_DEVICES) {
    *st = fail(MOE_ERR_UNSUPPORTED, "device %d: the second stream covers devices 0..%d", dev, MAX_SIDE_DEVICES - 1);
    return nullptr;
  }
  SideStream& ss = t_side[dev];
  if (!ss.made) {
    ss.made = true;
    ss.err = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
    if (ss.err == hipSuccess) ss.err = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
    if (ss.err == hipSuccess) ss.err = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
  }
  if (ss.err != hipSuccess) {
    *st = hip_status(ss.err, "second stream");
    return nullptr;
  }
  *st = MOE_OK;
  return &ss;
}

// overlap: run a shared expert on the second stream (see side_shared); the timed form and the
// no-allocation entry point keep one stream.
moe_status do_layer(const moe_shape* shape, const void* x, const void* Wr_packed, const float* bias,
                    const moe_weights* routed, const moe_weights* shared, void* y, int32_t* topk_idx_out,
                    float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t st, hipEvent_t const* ev,
                    const HashRoute* hash = nullptr, bool overlap = false) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if ((s = check_weights(routed, shape->w_routed, "routed")) != MOE_OK) return s;
  if (shape->I_shared && (s = check_weights(shared, shape->w_shared, "shared")) != MOE_OK) return s;
  if (shape->T && (!x || !Wr_packed || !y)) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!al16(x) || !al16(Wr_packed) || !al16(y)) return misaligned("x, Wr_packed and y", 16);
  if (!al4(bias) || !al4(topk_idx_out) || !al4(topk_w_out)) return misaligned("bias and the routing outputs", 4);
  if (hash && (!al4(hash->ids) || !al4(hash->table))) return misaligned("token_ids and hash_table", 4);
  Ws L;
  if ((s = check_ws(*shape, ws, ws_bytes, &L)) != MOE_OK) return s;
  if (shape->T == 0) return MOE_OK;
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.idx);
  float* w = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  int32_t* off = at<int32_t>(ws, L.offsets);
  int32_t* slot_token = at<int32_t>(ws, L.slot_token);
  int32_t* pair_slot = at<int32_t>(ws, L.pair_slot);
  void* y_perm = at<void>(ws, L.y_perm);
  void* y_sh = shape->I_shared ? at<void>(ws, L.y_shared) : nullptr;
  if (ev && (s = record(ev[0], st)) != MOE_OK) return s;
  SideStream* ss = nullptr;
  if (overlap && !ev && side_shared(*shape) && !(ss = side_of_current_device(st, &s)) && s != MOE_OK) return s;
  const bool side = ss != nullptr;
  if (side) {
    // fork: the second stream starts after what the caller's stream holds so far, runs the shared
    // expert's plan, gate/up and down, and records the join event
    if ((s = hip_status(hipEventRecord(ss->fork, st), "fork event")) != MOE_OK) return s;
    if ((s = hip_status(hipStreamWaitEvent(ss->s, ss->fork, 0), "fork wait")) != MOE_OK) return s;
    if ((s = do_ffn(*shape, x, off, slot_token, *routed, shared, y_perm, y_sh, ws, L, ss->s, nullptr, false,
                    FFN_SHARED)) != MOE_OK)
      return s;
    if ((s = hip_status(hipEventRecord(ss->join, ss->s), "join event")) != MOE_OK) return s;
  }
  bool planned = false;
  if ((s = do_route_permute(*shape, x, Wr_packed, bias, idx, w, off, slot_token, pair_slot, ws, L, st, ev, hash,
                            &planned, !side)) != MOE_OK)
    return s;
  if (ev && (s = record(ev[2], st)) != MOE_OK) return s;
  if ((s = do_ffn(*shape, x, off, slot_token, *routed, shared, y_perm, y_sh, ws, L, st, ev ? ev + 3 : nullptr,
                  planned, side ? FFN_ROUTED : FFN_ALL)) != MOE_OK)
    return s;
  // join: combine adds the shared expert's rows
  if (side && (s = hip_status(hipStreamWaitEvent(st, ss->join, 0), "join wait")) != MOE_OK) return s;
  s = hip_status(launch_combine(shape->act, y_perm, pair_slot, w, y_sh, y, shape->T, shape->H, shape->k, st),
                 "combine");
  if (s == MOE_OK && ev) s = record(ev[6], st);
  return s;
}

// The workspace of moe_layer_forward_logical: the layer's own workspace, then the packed router,
// routed and shared matrices (moe_pack's layout), each at an ALIGN boundary.
struct PackedSet {
  size_t gate, gate_s, up, up_s, down, down_s;
};
struct LogicalWs {
  size_t wr;
  PackedSet r, sh;
  size_t total;
};

moe_status logical_layout(const moe_shape& s, LogicalWs* out) {
  size_t o = ws_layout(s).total;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += up(bytes ? bytes : 1);
    return at;
  };
  size_t b, sb;
  moe_status st;
  if ((st = packed_sizes(s.act, 1, s.H, s.E, &b, &sb)) != MOE_OK) return st;
  out->wr = take(b);
  auto set = [&](moe_dtype fmt, int count, PackedSet& p) -> moe_status {
    size_t b1, s1, b2, s2;
    moe_status r;
    if ((r = packed_sizes(fmt, count, s.H, s.I, &b1, &s1)) != MOE_OK) return r;
    if ((r = packed_sizes(fmt, count, s.I, s.H, &b2, &s2)) != MOE_OK) return r;
    p.gate = take(b1);
    p.gate_s = take(s1);
    p.up = take(b1);
    p.up_s = take(s1);
    p.down = take(b2);
    p.down_s = take(s2);
    return MOE_OK;
  };
  if ((st = set(s.w_routed, s.E, out->r)) != MOE_OK) return st;
  out->sh = PackedSet{};
  if (s.I_shared && (st = set(s.w_shared, 1, out->sh)) != MOE_OK) return st;
  out->total = o;
  return MOE_OK;
}

// Pack one expert set's logical matrices (gate and up [count][H][I], down [count][I][H]) into p.
moe_status pack_set(const moe_shape& s, moe_dtype fmt, int count, const moe_weights& w, void* ws, const PackedSet& p,
                    moe_weights* packed, hipStream_t st) {
  const moe_dtype f = stored_fmt(fmt);
  const bool scaled = fmt != MOE_F32 && fmt != MOE_BF16;
  const int wal = fmt == MOE_F32 ? 4 : fmt == MOE_BF16 ? 2 : 1;
  if ((uintptr_t)w.gate % wal || (uintptr_t)w.up % wal || (uintptr_t)w.down % wal) return misaligned("logical weights", wal);
  if ((fmt == MOE_FP8_E4M3_B128 || fmt == MOE_INT8_W8A8) && (!al4(w.gate_scale) || !al4(w.up_scale) || !al4(w.down_scale)))
    return misaligned("logical scales", 4);
  struct Job {
    const void *src, *src_s;
    size_t dst, dst_s;
    int K, N;
  } jobs[3] = {{w.gate, w.gate_scale, p.gate, p.gate_s, s.H, s.I},
               {w.up, w.up_scale, p.up, p.up_s, s.H, s.I},
               {w.down, w.down_scale, p.down, p.down_s, s.I, s.H}};
  for (const Job& j : jobs) {
    const hipError_t e = moe_launch_pack(f, count, j.K, j.N, j.src, scaled ? j.src_s : nullptr, at<void>(ws, j.dst),
                                         scaled ? at<void>(ws, j.dst_s) : nullptr, st);
    if (e != hipSuccess) return hip_status(e, "pack");
  }
  packed->gate = at<void>(ws, p.gate);
  packed->up = at<void>(ws, p.up);
  packed->down = at<void>(ws, p.down);
  packed->gate_scale = scaled ? at<void>(ws, p.gate_s) : nullptr;
  packed->up_scale = scaled ? at<void>(ws, p.up_s) : nullptr;
  packed->down_scale = scaled ? at<void>(ws, p.down_s) : nullptr;
  return MOE_OK;
}

// ------------------------------------------------------------------------------------------
// The library's own scratch memory, for callers that cannot allocate: moe_layer_forward_noalloc
// runs the layer with this array as its workspace. Each GPU holds its own copy for the life of the
// process; the host side finds that copy's address once per device and passes it to the kernels.
// ------------------------------------------------------------------------------------------
constexpr size_t SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[MAX_DEVICES];

// The device address of the current device's scratch array (found on the first call per device,
// with that device current), or null with the error set.
void* scratch_of_current_device(moe_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_status(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= MAX_DEVICES) {
    *st = fail(MOE_ERR_UNSUPPORTED, "device %d: the library's scratch covers devices 0..%d", dev, MAX_DEVICES - 1);
    return nullptr;
  }
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] { slot.err = hipGetSymbolAddress((void**)&slot.ptr, HIP_SYMBOL(scratch)); });
  if (slot.err != hipSuccess || !slot.ptr) {
    *st = hip_status(slot.err != hipSuccess ? slot.err : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    return nullptr;
  }
  *st = MOE_OK;
  return slot.ptr;
}

}  // namespace

extern "C" {

__attribute__((visibility("hidden"))) hipError_t moe_launch_pack(int fmt, int count, int K, int N, const void* w, const void* scale, void* packed,
                           void* packed_scale, hipStream_t stream);

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "unknown moe_status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_pack_size(moe_dtype fmt, int32_t count, int32_t K, int32_t N, size_t* packed_bytes,
                         size_t* packed_scale_bytes) {
  if (!packed_bytes || !packed_scale_bytes) return fail(MOE_ERR_INVALID_ARG, "NULL size pointer");
  return packed_sizes(fmt, count, K, N, packed_bytes, packed_scale_bytes);
}

moe_status moe_pack(moe_dtype fmt, int32_t count, int32_t K, int32_t N, const void* w, const void* scale,
                    void* packed, void* packed_scale, moe_stream_t stream) {
  size_t b, sb;
  moe_status s = packed_sizes(fmt, count, K, N, &b, &sb);
  if (s != MOE_OK) return s;
  if (count == 0) return MOE_OK;
  if (!w || !packed) return fail(MOE_ERR_INVALID_ARG, "NULL matrix pointer");
  if (sb && (!scale || !packed_scale)) return fail(MOE_ERR_INVALID_ARG, "NULL scale pointer");
  if (!al16(packed)) return misaligned("packed", 16);
  if (!al4(packed_scale)) return misaligned("packed_scale", 4);
  const int wal = fmt == MOE_F32 ? 4 : fmt == MOE_BF16 ? 2 : 1;  // the source's element size
  if ((uintptr_t)w % wal) return misaligned("w", wal);
  if ((fmt == MOE_FP8_E4M3_B128 || fmt == MOE_INT8_W8A8) && !al4(scale)) return misaligned("scale", 4);
  return hip_status(moe_launch_pack(stored_fmt(fmt), count, K, N, w, scale, packed, packed_scale, (hipStream_t)stream),
                    "pack");
}

moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_layout(*shape).total;
  return MOE_OK;
}

moe_status moe_route(const moe_shape* shape, const void* x, const void* Wr_packed, const float* bias,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (shape->T && (!x || !Wr_packed || !topk_idx || !topk_w)) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!al16(x) || !al16(Wr_packed)) return misaligned("x and Wr_packed", 16);
  if (!al4(bias) || !al4(topk_idx) || !al4(topk_w)) return misaligned("bias, topk_idx and topk_w", 4);
  Ws L;
  if ((s = check_ws(*shape, ws, ws_bytes, &L)) != MOE_OK) return s;
  return do_route(*shape, x, Wr_packed, bias, topk_idx, topk_w, ws, L, (hipStream_t)stream);
}

moe_status moe_route_hash(const moe_shape* shape, const void* x, const void* Wr_packed, const float* bias,
                          const int32_t* token_ids, const int32_t* hash_table, int32_t vocab, int32_t* topk_idx,
                          float* topk_w, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (vocab < 1) return fail(MOE_ERR_INVALID_ARG, "vocab=%d < 1", vocab);
  if (shape->T && (!x || !Wr_packed || !token_ids || !hash_table || !topk_idx || !topk_w))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!al16(x) || !al16(Wr_packed)) return misaligned("x and Wr_packed", 16);
  if (!al4(bias) || !al4(token_ids) || !al4(hash_table) || !al4(topk_idx) || !al4(topk_w))
    return misaligned("bias, token_ids, hash_table, topk_idx and topk_w", 4);
  Ws L;
  if ((s = check_ws(*shape, ws, ws_bytes, &L)) != MOE_OK) return s;
  const HashRoute h{token_ids, hash_table, vocab};
  return do_route(*shape, x, Wr_packed, bias, topk_idx, topk_w, ws, L, (hipStream_t)stream, &h);
}

moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx, int32_t* expert_offsets,
                       int32_t* slot_token, int32_t* pair_slot, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (!expert_offsets || (shape->T && (!topk_idx || !slot_token || !pair_slot)))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!al4(topk_idx) || !al4(expert_offsets) || !al4(slot_token) || !al4(pair_slot))
    return misaligned("the index arrays", 4);
  Ws L;
  if ((s = check_ws(*shape, ws, ws_bytes, &L)) != MOE_OK) return s;
  return do_permute(*shape, topk_idx, expert_offsets, slot_token, pair_slot, ws, L, (hipStream_t)stream);
}

moe_status moe_route_permute(const moe_shape* shape, const void* x, const void* Wr_packed, const float* bias,
                             int32_t* topk_idx, float* topk_w, int32_t* expert_offsets, int32_t* slot_token,
                             int32_t* pair_slot, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (!expert_offsets || (shape->T && (!x || !Wr_packed || !topk_idx || !topk_w || !slot_token || !pair_slot)))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!al16(x) || !al16(Wr_packed)) return misaligned("x and Wr_packed", 16);
  if (!al4(bias) || !al4(topk_idx) || !al4(topk_w) || !al4(expert_offsets) || !al4(slot_token) || !al4(pair_slot))
    return misaligned("bias, the routing outputs and the index arrays", 4);
  Ws L;
  if ((s = check_ws(*shape, ws, ws_bytes, &L)) != MOE_OK) return s;
  bool planned;
  return do_route_permute(*shape, x, Wr_packed, bias, topk_idx, topk_w, expert_offsets, slot_token, pair_slot, ws, L,
                          (hipStream_t)stream, nullptr, nullptr, &planned);
}

moe_status moe_grouped_ffn(const moe_shape* shape, const void* x, const int32_t* expert_offsets,
                           const int32_t* slot_token, const moe_weights* routed, const moe_weights* shared,
                           void* y_perm, void* y_shared, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if ((s = check_weights(routed, shape->w_routed, "routed")) != MOE_OK) return s;
  if (shape->I_shared && (s = check_weights(shared, shape->w_shared, "shared")) != MOE_OK) return s;
  if (shape->T && (!x || !expert_offsets || !slot_token || !y_perm || (shape->I_shared && !y_shared)))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!al16(x) || !al16(y_perm) || !al16(y_shared)) return misaligned("x, y_perm and y_shared", 16);
  if (!al4(expert_offsets) || !al4(slot_token)) return misaligned("expert_offsets and slot_token", 4);
  Ws L;
  if ((s = check_ws(*shape, ws, ws_bytes, &L)) != MOE_OK) return s;
  return do_ffn(*shape, x, expert_offsets, slot_token, *routed, shared, y_perm, y_shared, ws, L, (hipStream_t)stream);
}

moe_status moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* pair_slot, const float* topk_w,
                       const void* y_shared, void* y, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (shape->T && (!y_perm || !pair_slot || !topk_w || !y)) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!al16(y_perm) || !al16(y_shared) || !al16(y)) return misaligned("y_perm, y_shared and y", 16);
  if (!al4(pair_slot) || !al4(topk_w)) return misaligned("pair_slot and topk_w", 4);
  return hip_status(launch_combine(shape->act, y_perm, pair_slot, topk_w, y_shared, y, shape->T, shape->H, shape->k,
                                   (hipStream_t)stream),
                    "combine");
}

moe_status moe_layer_forward(const moe_shape* shape, const void* x, const void* Wr_packed, const float* bias,
                             const moe_weights* routed, const moe_weights* shared, void* y, int32_t* topk_idx_out,
                             float* topk_w_out, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return do_layer(shape, x, Wr_packed, bias, routed, shared, y, topk_idx_out, topk_w_out, ws, ws_bytes,
                  (hipStream_t)stream, nullptr, nullptr, true);
}

moe_status moe_logical_workspace_size(const moe_shape* shape, size_t* bytes) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  LogicalWs L;
  if ((s = logical_layout(*shape, &L)) != MOE_OK) return s;
  *bytes = L.total;
  return MOE_OK;
}

moe_status moe_layer_forward_logical(const moe_shape* shape, const void* x, const void* Wr, const float* bias,
                                     const moe_weights* routed, const moe_weights* shared, void* y,
                                     int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                                     moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if ((s = check_weights(routed, shape->w_routed, "routed")) != MOE_OK) return s;
  if (shape->I_shared && (s = check_weights(shared, shape->w_shared, "shared")) != MOE_OK) return s;
  if (!Wr) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if ((uintptr_t)Wr % (shape->act == MOE_F32 ? 4 : 2)) return misaligned("Wr", shape->act == MOE_F32 ? 4 : 2);
  LogicalWs L;
  if ((s = logical_layout(*shape, &L)) != MOE_OK) return s;
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  if ((uintptr_t)ws % ALIGN) return fail(MOE_ERR_INVALID_ARG, "workspace must be %zu-byte aligned", ALIGN);
  if (shape->T == 0) return MOE_OK;
  const hipStream_t st = (hipStream_t)stream;
  // the router, the routed experts and the shared one into moe_pack's layout, then the layer
  hipError_t e = moe_launch_pack(shape->act, 1, shape->H, shape->E, Wr, nullptr, at<void>(ws, L.wr), nullptr, st);
  if (e != hipSuccess) return hip_status(e, "pack");
  moe_weights pr{}, ps{};
  if ((s = pack_set(*shape, shape->w_routed, shape->E, *routed, ws, L.r, &pr, st)) != MOE_OK) return s;
  if (shape->I_shared && (s = pack_set(*shape, shape->w_shared, 1, *shared, ws, L.sh, &ps, st)) != MOE_OK) return s;
  return do_layer(shape, x, at<void>(ws, L.wr), bias, &pr, shape->I_shared ? &ps : nullptr, y, topk_idx_out,
                  topk_w_out, ws, ws_layout(*shape).total, st, nullptr, nullptr, true);
}

moe_status moe_layer_forward_noalloc(const moe_shape* shape, const void* x, const void* Wr_packed, const float* bias,
                                     const moe_weights* routed, const moe_weights* shared, void* y,
                                     int32_t* topk_idx_out, float* topk_w_out, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  const size_t need = ws_layout(*shape).total;
  if (need > SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "this shape needs %zu bytes of workspace; the library's own scratch holds %zu "
                "(use moe_layer_forward with a workspace)",
                need, SCRATCH_BYTES);
  void* ws = scratch_of_current_device(&s);
  if (!ws) return s;
  return do_layer(shape, x, Wr_packed, bias, routed, shared, y, topk_idx_out, topk_w_out, ws, SCRATCH_BYTES,
                  (hipStream_t)stream, nullptr);
}

moe_status moe_layer_forward_hash(const moe_shape* shape, const void* x, const void* Wr_packed, const float* bias,
                                  const int32_t* token_ids, const int32_t* hash_table, int32_t vocab,
                                  const moe_weights* routed, const moe_weights* shared, void* y,
                                  int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                                  moe_stream_t stream) {
  if (vocab < 1) return fail(MOE_ERR_INVALID_ARG, "vocab=%d < 1", vocab);
  if (shape && shape->T && (!token_ids || !hash_table)) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  const HashRoute h{token_ids, hash_table, vocab};
  return do_layer(shape, x, Wr_packed, bias, routed, shared, y, topk_idx_out, topk_w_out, ws, ws_bytes,
                  (hipStream_t)stream, nullptr, &h, true);
}

moe_status moe_layer_forward_timed(const moe_shape* shape, const void* x, const void* Wr_packed, const float* bias,
                                   const moe_weights* routed, const moe_weights* shared, void* y,
                                   int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                                   moe_stream_t stream, moe_event_t* events) {
  if (!events) return fail(MOE_ERR_INVALID_ARG, "events is NULL");
  for (int i = 0; i < MOE_TIMED_EVENTS; ++i)
    if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "event %d is NULL", i);
  return do_layer(shape, x, Wr_packed, bias, routed, shared, y, topk_idx_out, topk_w_out, ws, ws_bytes,
                  (hipStream_t)stream, (hipEvent_t const*)events);
}

moe_status moe_quantize_mxfp8(const void* x, int32_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                              moe_stream_t stream) {
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows=%d < 0", rows);
  if (K < 32 || K % 32) return fail(MOE_ERR_INVALID_ARG, "K=%d must be a positive multiple of 32", K);
  if ((long long)rows * K > (1LL << 40)) return fail(MOE_ERR_INVALID_ARG, "rows * K too large");
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if ((uintptr_t)x % 16 || (uintptr_t)codes % 8)
    return fail(MOE_ERR_INVALID_ARG, "x must be 16-byte and codes 8-byte aligned");
  return hip_status(launch_quant_mxfp8(x, rows, K, codes, scales, (hipStream_t)stream), "MXFP8 quantisation");
}

moe_status moe_quantize_int8(const void* x, int32_t rows, int32_t K, int8_t* codes, float* scales,
                             moe_stream_t stream) {
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows=%d < 0", rows);
  if (K < 8 || K % 8 || K > 8192)
    return fail(MOE_ERR_INVALID_ARG, "K=%d must be a positive multiple of 8, at most 8192", K);
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if ((uintptr_t)x % 16 || (uintptr_t)codes % 8 || (uintptr_t)scales % 4)
    return fail(MOE_ERR_INVALID_ARG, "x must be 16-byte, codes 8-byte and scales 4-byte aligned");
  return hip_status(launch_quant_int8(x, rows, K, codes, scales, (hipStream_t)stream), "int8 quantisation");
}

}  // extern "C"
