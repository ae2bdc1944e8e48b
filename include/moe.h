/*
 * moe.h — C ABI of a single-GPU Mixture-of-Experts expert-FFN layer for AMD MI355X (gfx950).
 *
 * The layer (sources: "Chapter 6 Supernodes" of the AI-infra book = [ch6];
 * "DeepSeek-V4-Pro on NVIDIA H200" report = [V4]):
 *   route    scores l[t][e] = x[t] . Wr[:, e] (+ b[e]); the k largest per token; weights =
 *            softmax over all E renormalised over the k chosen            [ch6 §6.2.6; V4 D4]
 *   permute  regroup the (token, expert) pairs by expert, stable in token order, and keep the
 *            map back to token order                             [ch6 §6.2.6, receiver side]
 *   FFN      each expert e on its rows X_e: Y_e = [SiLU(X_e Wg_e) (.) (X_e Wu_e)] Wd_e
 *                                                                 [ch6 §6.2.2, SwiGLU; V4 D6]
 *   shared   an always-active expert of the same form, weight 1           [V4 §0.1.2, §3.2]
 *   combine  y[t] = sum_j w[t][j] Y[pair_slot[t k + j]] + Y_shared[t]    [ch6 §6.2.6, §6.4.1]
 *
 * Conventions (all functions):
 *   - Every pointer argument is device memory owned by the caller, except the moe_shape /
 *     moe_weights structs, which are host memory read during the call only.
 *   - Functions validate their arguments on the host, then only enqueue kernels on `stream`
 *     and return. MOE_OK means "enqueued"; results are valid in stream order (the same
 *     contract the chapter describes for collective calls, [ch6 §6.4.3]). No function
 *     synchronises, allocates or frees memory, or copies data-dependent sizes to the host.
 *   - Scratch memory comes from the caller's workspace `ws` (moe_workspace_size); the library
 *     keeps no mutable global state, so calls on different streams with different
 *     workspaces may run concurrently.
 *   - Errors are returned as codes, never thrown; on an error nothing has been enqueued,
 *     except MOE_ERR_HIP (a launch failed; moe_last_error() has the runtime's message).
 *   - Row-major everywhere. Activations x, y are [T][H] in the `act` type.
 *   - Alignment: activations, outputs (x, y, y_perm, y_shared), the packed router and packed
 *     weight matrices are 16-byte aligned; packed scales, bias, index and routing-weight arrays
 *     4-byte aligned (any PyTorch allocation is). A misaligned pointer is MOE_ERR_INVALID_ARG.
 *
 * Weights are read in the packed layout written by moe_pack (once, at weight-load time): see
 * moe_pack for the layout and for which logical matrix each argument is.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* a hipStream_t; NULL = the null stream */
typedef struct ihipEvent_t* moe_event_t;   /* a hipEvent_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,       /* null required pointer, bad size, bad dtype */
  MOE_ERR_UNSUPPORTED = 2,       /* a valid but unimplemented combination */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                /* a kernel launch failed */
} moe_status;

typedef enum {
  MOE_F32 = 0,            /* float32 */
  MOE_BF16 = 1,           /* bfloat16 */
  MOE_FP8_E4M3_B128 = 2,  /* OCP E4M3FN codes + one fp32 scale per 128 x 128 block */
  MOE_MXFP4_B32 = 3,      /* OCP e2m1 codes + one e8m0 exponent per 32 reduction elements */
  MOE_MXFP4_B32_A8 = 4,   /* W4A8 routed experts ('CANN DeepSeek-V4推理优化', quantisation
                             strategy: the routed experts' linear layers run W4A8). Weights are
                             stored, packed and sized exactly as MOE_MXFP4_B32; the activations of
                             both products (x before gate/up, h before down) are quantised to OCP
                             MXFP8 (E4M3FN codes, round to nearest even, saturating at 448, with
                             one e8m0 exponent floor(log2 max|v|) - 8 per 32 reduction elements)
                             and multiplied by the block-scaled fp4 x fp8 matrix instruction.
                             Only as w_routed, with BF16 activations, I a multiple of 256 and H of
                             512; on either path (thin batches take the decode kernel). */
  MOE_MXFP8_B32_A8 = 5,   /* W8A8 MXFP8 shared expert of the hybrid MXFP8-MXFP4 scheme (same
                             passage: the shared expert's linear layers run W8A8, weights and
                             activations both MXFP8). Weights: OCP E4M3FN codes + one e8m0
                             exponent per 32 reduction elements, w = e4m3(c) * 2^(E-127). The
                             activations are quantised to MXFP8 as for MOE_MXFP4_B32_A8 and both
                             operands go to the block-scaled fp8 x fp8 matrix instruction. Only
                             as w_shared, with w_routed = MOE_MXFP4_B32_A8; on either path. */
  MOE_INT8_W8A8 = 6       /* Int8 W8A8 experts (same page, Int8 quantisation strategy: the routed
                             and shared experts' linear layers run W8A8, weights statically
                             quantised per output channel, activations dynamically per token).
                             Weights: int8 codes + one fp32 scale per output feature, w = c * s[n].
                             Each row of x and of h (after its bf16 rounding) is quantised in fp32:
                             f = 127 / max|v|, s = max|v| / 127, code = rint(v * f) (ties to even,
                             clamped to +-127; f taken from max|v|'s significand, as
                             moe_quantize_int8 states); an all-zero row has s = 0. The products accumulate
                             the codes exactly in int32 on the int8 matrix instruction, then scale
                             by s_row * s[n]. As w_routed, with no shared expert or an INT8 one;
                             BF16 activations, I a multiple of 256 and H of 512; on either path. */
} moe_dtype;

typedef enum {
  MOE_PATH_AUTO = 0,      /* prefill when T * k >= 64 * E and the prefill kernel takes the
                             shape, else decode */
  MOE_PATH_DECODE = 1,    /* weight-streaming grouped GEMM (few rows per expert) */
  MOE_PATH_PREFILL = 2    /* LDS-tiled MFMA grouped GEMM (many rows per expert): BF16
                             activations, BF16 / FP8 / MXFP4 / W4A8 / W8A8 MXFP8 / INT8 weights, I
                             a multiple of 256, H a multiple of 512; MOE_ERR_UNSUPPORTED otherwise.
                             */
} moe_path;

typedef struct {
  int32_t T;          /* tokens, >= 0 (0: the calls enqueue nothing) */
  int32_t H;          /* hidden size, multiple of 128 */
  int32_t E;          /* routed experts, 1..1024 */
  int32_t k;          /* experts per token, 1..min(E, 16) */
  int32_t I;          /* expert intermediate size, multiple of 128 */
  int32_t I_shared;   /* shared expert intermediate size: 0 = no shared expert, else == I */
  moe_dtype act;      /* MOE_F32 or MOE_BF16: x, Wr, y and the intermediates */
  moe_dtype w_routed; /* MOE_F32 (with act MOE_F32) or BF16 / FP8 / MXFP4 / MXFP4_B32_A8 /
                         INT8_W8A8 (with act BF16) */
  moe_dtype w_shared; /* MOE_F32 (with act MOE_F32) or BF16 / FP8 / MXFP4 (with act BF16);
                         MXFP8_B32_A8 beside MXFP4_B32_A8 routed experts; INT8_W8A8 beside
                         INT8_W8A8 routed experts (the only shared format they take) */
  moe_path path;
} moe_shape;

/* Packed weights of one kind (routed: E experts back to back; shared: one expert). */
typedef struct {
  const void* gate;        /* packed W_gate (logical [H][I] per expert) */
  const void* up;          /* packed W_up   (logical [H][I]) */
  const void* down;        /* packed W_down (logical [I][H]) */
  const void* gate_scale;  /* packed scales, NULL for F32 / BF16 */
  const void* up_scale;
  const void* down_scale;
} moe_weights;

/* Readable name of a status code (static string). */
const char* moe_status_string(moe_status s);

/* Detail text of the last error returned on this thread (static storage, thread-local). */
const char* moe_last_error(void);

/*
 * moe_pack_size / moe_pack — convert `count` logical K x N matrices (back to back) from the
 * row-major layout in which the chapter writes them (W[k][n]: k indexes the reduction, n the
 * output feature; [ch6 §6.2.2]) to the packed layout the kernels stream.
 *
 * Logical (source) formats, per matrix:
 *   MOE_F32   float[K][N]                MOE_BF16  uint16[K][N] (bf16 bits)
 *   MOE_FP8_E4M3_B128  uint8[K][N] codes + float[K/128][N/128] scales (w = e4m3(c) * s)
 *   MOE_MXFP4_B32      uint8[K][N/2] codes, even n in the low nibble + uint8[K/32][N] e8m0
 *                      exponents (w = e2m1(c) * 2^(E-127)); MOE_MXFP4_B32_A8 the same
 *   MOE_MXFP8_B32_A8   uint8[K][N] codes + uint8[K/32][N] e8m0 exponents (w = e4m3(c) * 2^(E-127))
 *   MOE_INT8_W8A8      int8[K][N] codes + float[N] scales (w = c * s[n])
 * Packed layout: 1 KiB packets of 16 features x KP reduction elements (KP = 16, 32, 64, 128 for
 * F32, BF16, FP8 / MXFP8 / INT8, MXFP4), packet (nt, kt) at byte (nt*(K/KP) + kt)*1024, lane l of a
 * packet holding feature nt*16 + l%16 and reduction run kt*KP + (l/16)*KP/4 + [0, KP/4). FP8
 * scales are copied unchanged; MXFP4 scales are regrouped one byte per lane per packet, and
 * MXFP8 scales one byte per lane per pair of packets (128 reduction elements): byte
 * (nt*(K/128) + kt2)*64 + l is the exponent of feature nt*16 + l%16, reduction elements
 * kt2*128 + (l/16)*32 + [0, 32). INT8 scales are copied per matrix into pad256(N) floats, zero
 * past N.
 * N is padded up to a multiple of 256 with zero features (only the router, N = E, needs it).
 * Requirements: K a multiple of KP (and of 128 for FP8, MXFP8 and INT8), N a multiple of 16 (128
 * for FP8, 2 for MXFP4) before padding. `packed_scale` may be NULL for F32 / BF16.
 * Router: pack Wr[H][E] as one K = H, N = E matrix in the `act` format.
 */
moe_status moe_pack_size(moe_dtype fmt, int32_t count, int32_t K, int32_t N,
                         size_t* packed_bytes, size_t* packed_scale_bytes);
moe_status moe_pack(moe_dtype fmt, int32_t count, int32_t K, int32_t N, const void* w,
                    const void* scale, void* packed, void* packed_scale, moe_stream_t stream);

/* Scratch bytes moe_layer_forward / moe_grouped_ffn / moe_permute / moe_route need for
 * `shape` (the same workspace serves any of them). */
moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes);

/*
 * moe_route — router scores, top-k and weights [ch6 §6.2.6; V4 D4].
 *   x        [T][H] act          Wr_packed  packed Wr (K = H, N = E, act format)
 *   bias     float[E] or NULL: added to the scores (selection and weights)
 *   topk_idx int32[T][k] out: chosen experts in ascending index; an exact tie at the k-th
 *            place goes to the lower index
 *   topk_w   float[T][k] out: exp(l - m) / sum over the chosen of exp(l - m), m = max score
 */
moe_status moe_route(const moe_shape* shape, const void* x, const void* Wr_packed,
                     const float* bias, int32_t* topk_idx, float* topk_w, void* ws,
                     size_t ws_bytes, moe_stream_t stream);

/*
 * moe_route_hash — hash routing ('CANN DeepSeek-V4推理优化', MoE section: the first layers pick
 * their experts by hash, the later ones by the learned router). The experts of token t are row
 * token_ids[t] of hash_table; the weights are moe_route's, renormalised over that set.
 *   token_ids  int32[T], values in [0, vocab)
 *   hash_table int32[vocab][k]: the k experts of each id, values in [0, E)
 *   topk_idx   int32[T][k] out: the row's valid experts in ascending index (equal ones in table
 *              order), then -1 for each entry outside [0, E) (all k for an id outside [0, vocab))
 *   topk_w     float[T][k] out: exp(l - m) / sum of exp(l - m) over the row's valid experts,
 *              m = their largest score (the router's scores, bias included); 0 for -1 entries
 * Pairs with expert -1 are skipped by moe_permute and add nothing in moe_combine. Other
 * arguments, ownership and errors as moe_route; MOE_ERR_INVALID_ARG for vocab < 1.
 */
moe_status moe_route_hash(const moe_shape* shape, const void* x, const void* Wr_packed,
                          const float* bias, const int32_t* token_ids, const int32_t* hash_table,
                          int32_t vocab, int32_t* topk_idx, float* topk_w, void* ws,
                          size_t ws_bytes, moe_stream_t stream);

/*
 * moe_permute — stable counting sort of the pairs q = t*k + j by expert [ch6 §6.2.6].
 *   topk_idx       int32[T*k] in: values in [0, E) (entries outside are skipped)
 *   expert_offsets int32[E+1] out: rows of expert e are [off[e], off[e+1]); off[E] = the number
 *                  of pairs with a valid expert (T*k when none is skipped)
 *   slot_token     int32[T*k] out: token of each row (slot); entries from off[E] on are not
 *                  written
 *   pair_slot      int32[T*k] out: row of each pair, -1 for a skipped pair
 * Deterministic: no atomics decide an order.
 */
moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx,
                       int32_t* expert_offsets, int32_t* slot_token, int32_t* pair_slot,
                       void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_route_permute — moe_route followed by moe_permute, with the same outputs bit for bit
 * ('DeepSeek-V4-Pro on NVIDIA H200' §9.2: launch and synchronisation cost eats the gain of small
 * kernels; 'CANN DeepSeek-V4推理优化', fused-kernel section: a fused gating top-k). Decode
 * batches (T*k <= 8192, E <= 512, fewer than 2048 tokens) run as the router-score kernel and one
 * more launch: its workgroups select 8 or 16 tokens each and rank their own pairs by expert, and
 * the last workgroup to finish (a completion count in ws, cleared by the score kernel) forms the
 * offsets and places every pair. Other shapes run moe_route's and moe_permute's kernels.
 *   topk_idx, topk_w               out, as moe_route
 *   expert_offsets, slot_token, pair_slot   out, as moe_permute
 * Arguments, ownership and errors as moe_route and moe_permute.
 */
moe_status moe_route_permute(const moe_shape* shape, const void* x, const void* Wr_packed,
                             const float* bias, int32_t* topk_idx, float* topk_w,
                             int32_t* expert_offsets, int32_t* slot_token, int32_t* pair_slot,
                             void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_grouped_ffn — every expert's SwiGLU on its rows, plus the shared expert on all tokens
 * [ch6 §6.2.2; V4 D6].
 *   x              [T][H] act
 *   expert_offsets, slot_token: from moe_permute
 *   routed         packed routed weights (E experts)
 *   shared         packed shared weights, or NULL when I_shared == 0
 *   y_perm         [T*k][H] act out: row r = FFN_e(x[slot_token[r]]) for the e owning r (rows
 *                  from expert_offsets[E] on, those of skipped pairs, are not written)
 *   y_shared       [T][H] act out (NULL when I_shared == 0)
 * The intermediate h = SiLU(x Wg) (.) (x Wu) is kept in `ws` in the act type (for the MXFP8 and
 * INT8 formats also, or only, as the codes and scales the down product reads); accumulation fp32.
 */
moe_status moe_grouped_ffn(const moe_shape* shape, const void* x, const int32_t* expert_offsets,
                           const int32_t* slot_token, const moe_weights* routed,
                           const moe_weights* shared, void* y_perm, void* y_shared, void* ws,
                           size_t ws_bytes, moe_stream_t stream);

/*
 * moe_combine — y[t] = sum_{j<k} topk_w[t][j] * y_perm[pair_slot[t*k+j]] + y_shared[t], summed
 * in ascending j in fp32, one gather per output row, no atomics [ch6 §6.2.6, §6.4.1].
 *   y_perm     [T*k][H] act, pair_slot int32[T*k], topk_w float[T][k] (from moe_grouped_ffn,
 *              moe_permute and moe_route); a pair whose pair_slot is outside [0, T*k) adds nothing
 *   y_shared   [T][H] act, or NULL
 *   y          [T][H] act out
 */
moe_status moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* pair_slot,
                       const float* topk_w, const void* y_shared, void* y, moe_stream_t stream);

/*
 * moe_layer_forward — route, permute, grouped FFN and combine in one call (V4 §8.3: router
 * top-k, grouped expert weight reads, Linear-1/activation/Linear-2, combine).
 *   y              [T][H] act out
 *   topk_idx_out   int32[T][k] or NULL; topk_w_out float[T][k] or NULL (copies of the routing)
 * Routing and permutation run as moe_route_permute; for decode batches its second launch also
 * writes the grouped GEMMs' plan.
 * Decode batches with a shared expert in a bf16-activation format run that expert ('CANN
 * DeepSeek-V4推理优化', multi-stream parallelism) on a second stream the library owns, one per
 * calling thread and device, made on the thread's first such call (when `stream` belongs to the
 * current device; otherwise everything stays on `stream`): it waits for an event recorded on
 * `stream` at entry, and `stream` waits for its end before the combine. The call still only
 * enqueues, results are bit-identical to the single-stream order (moe_layer_forward_timed), and
 * capturing `stream` in a HIP graph captures both streams' work.
 */
moe_status moe_layer_forward(const moe_shape* shape, const void* x, const void* Wr_packed,
                             const float* bias, const moe_weights* routed,
                             const moe_weights* shared, void* y, int32_t* topk_idx_out,
                             float* topk_w_out, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_layer_forward_logical — moe_layer_forward on weights in the layout in which the pages write
 * them ('第 6 章 超節點' §6.2.2: x·W_g and x·W_u with W_g, W_u [H][I], then ·W_d with W_d [I][H],
 * row-major; the router's W_r [H][E]) instead of moe_pack's layout. Each call first packs the
 * router, the routed experts and the shared one into the workspace (moe_pack's kernels, on
 * `stream`), then runs moe_layer_forward on the packed copies, with the same results. This reads
 * and writes every weight once more per call, so a layer that runs more than once is faster packed
 * once with moe_pack and run with moe_layer_forward.
 *   Wr        act [H][E] row-major (bf16 bits or float)
 *   routed    gate, up: [E][H][I]; down: [E][I][H]; scales: moe_pack's source scale layout of
 *             each matrix, back to back per expert (NULL for F32 / BF16)
 *   shared    the same for one expert, or NULL when I_shared == 0
 *   ws        moe_logical_workspace_size(shape) bytes (the layer's workspace followed by the
 *             packed matrices), 256-byte aligned
 *   Other arguments, ownership, results and errors as moe_layer_forward; pointers are caller-owned
 *   device memory, read only.
 */
moe_status moe_logical_workspace_size(const moe_shape* shape, size_t* bytes);
moe_status moe_layer_forward_logical(const moe_shape* shape, const void* x, const void* Wr,
                                     const float* bias, const moe_weights* routed,
                                     const moe_weights* shared, void* y, int32_t* topk_idx_out,
                                     float* topk_w_out, void* ws, size_t ws_bytes,
                                     moe_stream_t stream);

/*
 * moe_layer_forward_noalloc — moe_layer_forward with the library's own scratch memory as the
 * workspace, for callers that cannot allocate device memory (code under HIP graph capture that
 * owns no workspace, tight serving loops, harnesses that forbid hipMalloc). It allocates nothing
 * and calls no allocating routine: the scratch is a 64 MiB array in the library's device code,
 * one copy per GPU, held until the process ends; its address is looked up on the first call on
 * each device (with that device current).
 *   Arguments, ownership, results and errors as moe_layer_forward (bit-identical outputs), with
 *   `stream` belonging to the current device; every launch goes to `stream` (no second stream). A shape whose moe_workspace_size exceeds 64 MiB
 *   (e.g. prefill batches) is refused with MOE_ERR_WORKSPACE_TOO_SMALL before any launch.
 *   Every call on a GPU uses that GPU's one scratch array: calls that overlap in time on one GPU
 *   (other streams, other threads) race and give undefined results; calls in one stream are
 *   ordered. Nothing in the scratch needs to start at zero: each call rewrites what it reads.
 */
moe_status moe_layer_forward_noalloc(const moe_shape* shape, const void* x, const void* Wr_packed,
                                     const float* bias, const moe_weights* routed,
                                     const moe_weights* shared, void* y, int32_t* topk_idx_out,
                                     float* topk_w_out, moe_stream_t stream);

/*
 * moe_layer_forward_hash — moe_layer_forward with moe_route_hash in place of moe_route
 * (arguments as those two).
 */
moe_status moe_layer_forward_hash(const moe_shape* shape, const void* x, const void* Wr_packed,
                                  const float* bias, const int32_t* token_ids,
                                  const int32_t* hash_table, int32_t vocab,
                                  const moe_weights* routed, const moe_weights* shared, void* y,
                                  int32_t* topk_idx_out, float* topk_w_out, void* ws,
                                  size_t ws_bytes, moe_stream_t stream);

/*
 * moe_layer_forward_timed — moe_layer_forward that also records `events` (MOE_TIMED_EVENTS
 * caller-created HIP events) on `stream` around its kernels, for per-stage timing:
 *   [0] start   [1] after route   [2] after permute   [3] after the grouped-GEMM plan
 *   [4] after the gate/up grouped GEMM   [5] after the down grouped GEMM   [6] after combine
 * Decode batches (T*k <= 8192, E <= 512, fewer than 2048 tokens) run the top-k selection, the
 * permutation and the plan as one kernel after the router scores: there [1] follows the scores
 * and [2] that kernel. Every launch goes to `stream`, a shared expert in the grouped launches of
 * the routed ones, so the intervals are those of one stream. Same results as moe_layer_forward.
 * With T == 0 nothing is recorded.
 */
#define MOE_TIMED_EVENTS 7
moe_status moe_layer_forward_timed(const moe_shape* shape, const void* x, const void* Wr_packed,
                                   const float* bias, const moe_weights* routed,
                                   const moe_weights* shared, void* y, int32_t* topk_idx_out,
                                   float* topk_w_out, void* ws, size_t ws_bytes,
                                   moe_stream_t stream, moe_event_t* events);

/*
 * moe_quantize_mxfp8 — the activation quantisation of the MXFP8 formats (MOE_MXFP4_B32_A8,
 * MOE_MXFP8_B32_A8; 'CANN DeepSeek-V4推理优化', quantisation strategy: 8-bit activations of the
 * W4A8 and W8A8 linear layers), as the layer applies it to each row of x before gate/up.
 *   x        bf16 [rows][K], row-major; K a multiple of 32
 *   codes    uint8 [rows][K] out: E4M3FN(x * 2^-X), round to nearest even, saturating at +-448,
 *            the sign of zero kept
 *   scales   uint8 [rows][K/32] out: X + 127 for each run of 32 consecutive elements of a row,
 *            X = floor(log2 max|v|) - 8 clamped to [-127, 127], and -127 for an all-zero run
 * x is 16-byte aligned and codes 8-byte aligned. rows == 0 enqueues nothing. MOE_ERR_INVALID_ARG
 * for rows < 0, K < 32 or not a multiple of 32, rows * K above 2^40, a NULL pointer or a
 * misaligned one.
 */
moe_status moe_quantize_mxfp8(const void* x, int32_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                              moe_stream_t stream);

/*
 * moe_quantize_int8 — the per-token activation quantisation of MOE_INT8_W8A8 (same page, Int8
 * quantisation strategy: activations quantised dynamically per token), as the layer applies it to
 * each row of x before gate/up and of h before down.
 *   x        bf16 [rows][K], row-major; K a multiple of 8, at most 8192
 *   codes    int8 [rows][K] out: rint(v * f) with f = 127 / max|v| (fp32 division and product,
 *            ties to even), clamped to +-127; zero for an all-zero row. f is formed from the
 *            maximum's significand (max|v| = m 2^e: f = 127 / m applied to v 2^-e), the same fp32
 *            value wherever 127 / max|v| is finite, and finite for any row
 *   scales   float [rows] out: max|v| / 127 (fp32 division); 0 for an all-zero row
 * x is 16-byte, codes 8-byte and scales 4-byte aligned. rows == 0 enqueues nothing.
 * MOE_ERR_INVALID_ARG for rows < 0, K outside those limits, a NULL pointer or a misaligned one.
 */
moe_status moe_quantize_int8(const void* x, int32_t rows, int32_t K, int8_t* codes, float* scales,
                             moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
