/*
 * The oracle: a plain, slow, obviously correct CPU implementation of one Mixture-of-Experts
 * expert-FFN layer. TEST INFRASTRUCTURE ONLY: it is compiled and called by the tests, by the
 * smoke check and by the CPU-baseline leg of the benchmark, never by the library. It shares no
 * source with the HIP library.
 *
 * Arithmetic is fp64 throughout. Stored weights are decoded element by element with this
 * file's own decoders, from the same bytes the GPU reads, in the logical row-major layout:
 *   W_gate, W_up : [H][I]   W_down : [I][H]   (one matrix per expert, experts back to back)
 *   f32   float[K][N]
 *   bf16  uint16[K][N]                                   (bit patterns)
 *   fp8   uint8[K][N] OCP E4M3FN + float[K/128][N/128]   (w = e4m3(code) * s)
 *   mxfp4 uint8[K][N/2] e2m1, even n in the low nibble + uint8[K/32][N] e8m0
 *                                                        (w = e2m1(code) * 2^(E-127))
 *   mxfp4a8  stored as mxfp4; the routed experts' activations are quantised to MXFP8 before
 *            each of their products (W4A8, see oracle_mxfp8_quantize)
 *   mxfp8a8  uint8[K][N] OCP E4M3FN + uint8[K/32][N] e8m0     (w = e4m3(code) * 2^(E-127));
 *            the expert's activations are quantised to MXFP8 before each of its products
 *            (W8A8 MXFP8, the shared expert of the hybrid MXFP8-MXFP4 scheme)
 *   int8     int8[K][N] + float[N], one scale per output channel  (w = code * s[n]);
 *            the expert's activations are quantised to int8 per token before each of its
 *            products (Int8 W8A8, see oracle_int8_quantize)
 *
 * What it computes, step by step (sources: "AI infra book, ch. 6 Supernodes" (bojieli.github.io
 * ai-infra-book ch. 6) = [ch6]; "DeepSeek-V4-Pro on NVIDIA H200" report = [V4]):
 *   1. router scores l[t][e] = sum_h x[t][h] Wr[h][e] (+ b[e])       [ch6 §6.2.6; V4 step D4]
 *   2. the k largest scores per token, ties to the lower expert index, listed in ascending
 *      expert index                                                  [V4 step D4 "top-6"]
 *   2'. or, with hash routing, the k experts are row token_id[t] of a [vocab][k] table; entries
 *      outside [0, E) are dropped                          [CANN DeepSeek-V4 page, MoE section]
 *   3. weights: softmax over all E scores, renormalised over the k selected
 *      (a1, a6 of the token-A example)                               [ch6 §6.2.6]
 *   4. permutation: rows regrouped by expert, stable in token order  [ch6 §6.2.6, receiver side]
 *   5. each expert: Y = [SiLU(X Wg) (.) (X Wu)] Wd                    [ch6 §6.2.2, SwiGLU display]
 *   6. the shared expert: the same FFN on every token, weight 1      [V4 §0.1.2, §3.2]
 *   7. combine: y[t] = sum_j w[t][j] y_perm[pair_slot[t k + j]] + y_sh[t]
 *                                                                    [ch6 §6.2.6, §6.4.1]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2, OR_MXFP4 = 3, OR_MXFP4_A8 = 4, OR_MXFP8_A8 = 5, OR_INT8 = 6 };

/* storage format of a weight format (W4A8 stores its weights as MXFP4) */
static int stored(int fmt) { return fmt == OR_MXFP4_A8 ? OR_MXFP4 : fmt; }

/* ---------------------------------------------------------------------------------------- */
/* decoders                                                                                  */
/* ---------------------------------------------------------------------------------------- */

double oracle_decode_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; S.1111.111 = NaN. */
double oracle_decode_e4m3fn(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* subnormal: m/8 * 2^-6 */
  else
    v = ldexp(8.0 + m, e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

/* OCP e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit. */
double oracle_decode_e2m1(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(2.0 + m, e - 2); /* (1 + m/2) * 2^(e-1) */
  return s ? -v : v;
}

/* OCP e8m0: 2^(E-127); E = 255 is NaN. */
double oracle_decode_e8m0(uint8_t E) {
  if (E == 255) return NAN;
  return ldexp(1.0, (int)E - 127);
}

static double act_at(const void* p, int act, size_t i) {
  return act == OR_F32 ? (double)((const float*)p)[i] : oracle_decode_bf16(((const uint16_t*)p)[i]);
}

/* Element W[k][n] of a stored K x N matrix. */
static double w_at(const void* w, const void* scale, int fmt, int K, int N, int k, int n) {
  size_t i = (size_t)k * N + n;
  switch (stored(fmt)) {
    case OR_F32: return (double)((const float*)w)[i];
    case OR_BF16: return oracle_decode_bf16(((const uint16_t*)w)[i]);
    case OR_FP8: {
      double s = (double)((const float*)scale)[(size_t)(k / 128) * (N / 128) + n / 128];
      return oracle_decode_e4m3fn(((const uint8_t*)w)[i]) * s;
    }
    case OR_MXFP4: {
      uint8_t byte = ((const uint8_t*)w)[(size_t)k * (N / 2) + n / 2];
      uint8_t code = (n & 1) ? (byte >> 4) : (byte & 15);
      uint8_t E = ((const uint8_t*)scale)[(size_t)(k / 32) * N + n];
      return oracle_decode_e2m1(code) * oracle_decode_e8m0(E);
    }
    case OR_MXFP8_A8: {
      uint8_t E = ((const uint8_t*)scale)[(size_t)(k / 32) * N + n];
      return oracle_decode_e4m3fn(((const uint8_t*)w)[i]) * oracle_decode_e8m0(E);
    }
    case OR_INT8: return (double)((const int8_t*)w)[i] * (double)((const float*)scale)[n];
  }
  return NAN;
}

/* Bytes of one stored K x N matrix and of its scales. */
static size_t w_bytes(int fmt, int K, int N) {
  switch (stored(fmt)) {
    case OR_F32: return (size_t)K * N * 4;
    case OR_BF16: return (size_t)K * N * 2;
    case OR_FP8: return (size_t)K * N;
    case OR_MXFP4: return (size_t)K * N / 2;
    case OR_MXFP8_A8:
    case OR_INT8: return (size_t)K * N;
  }
  return 0;
}
static size_t s_bytes(int fmt, int K, int N) {
  switch (stored(fmt)) {
    case OR_FP8: return (size_t)(K / 128) * (N / 128) * 4;
    case OR_MXFP4:
    case OR_MXFP8_A8: return (size_t)(K / 32) * N;
    case OR_INT8: return (size_t)N * 4;
  }
  return 0;
}

/* Decode a whole stored matrix to fp64 (for tests of the decoders and the generator). */
int oracle_decode_matrix(int fmt, int K, int N, const void* w, const void* scale, double* out) {
  for (int k = 0; k < K; ++k)
    for (int n = 0; n < N; ++n) out[(size_t)k * N + n] = w_at(w, scale, fmt, K, N, k, n);
  return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* the row-vector times matrix product every step is made of: out[n] = sum_k u[k] W[k][n]    */
/* ---------------------------------------------------------------------------------------- */

int oracle_row_matmul(int K, int N, int fmt, const void* w, const void* scale, const double* u,
                      double* out) {
  for (int n = 0; n < N; ++n) out[n] = 0.0;
  for (int k = 0; k < K; ++k) {
    double uk = u[k];
    for (int n = 0; n < N; ++n) out[n] += uk * w_at(w, scale, fmt, K, N, k, n);
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* steps 1-3: router                                                                         */
/* ---------------------------------------------------------------------------------------- */

int oracle_route(int T, int H, int E, int k, int act, const void* x, const void* Wr,
                 const float* bias, int32_t* topk_idx, double* topk_w, double* logits_out) {
  if (T < 0 || H < 1 || E < 1 || k < 1 || k > E) return 1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) if (T > 1)
  for (int t = 0; t < T; ++t) {
    double* l = (double*)malloc(sizeof(double) * E);
    char* chosen = (char*)calloc(E, 1);
    double* u = (double*)malloc(sizeof(double) * H);
    if (!l || !chosen || !u) {
      bad = 1;
    } else {
      for (int h = 0; h < H; ++h) u[h] = act_at(x, act, (size_t)t * H + h);
      oracle_row_matmul(H, E, act == OR_F32 ? OR_F32 : OR_BF16, Wr, NULL, u, l);
      if (bias)
        for (int e = 0; e < E; ++e) l[e] += (double)bias[e];
      if (logits_out) memcpy(logits_out + (size_t)t * E, l, sizeof(double) * E);
      /* k rounds of "largest not yet chosen"; scanning upward with '>' keeps the lower index
         on an exact tie */
      for (int r = 0; r < k; ++r) {
        int best = -1;
        for (int e = 0; e < E; ++e)
          if (!chosen[e] && (best < 0 || l[e] > l[best])) best = e;
        chosen[best] = 1;
      }
      /* softmax over all E, then renormalise over the chosen k */
      double m = l[0];
      for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
      double z_all = 0.0, z_sel = 0.0;
      for (int e = 0; e < E; ++e) z_all += exp(l[e] - m);
      for (int e = 0; e < E; ++e)
        if (chosen[e]) z_sel += exp(l[e] - m) / z_all;
      int j = 0;
      for (int e = 0; e < E; ++e)
        if (chosen[e]) {
          topk_idx[(size_t)t * k + j] = e;
          topk_w[(size_t)t * k + j] = (exp(l[e] - m) / z_all) / z_sel;
          ++j;
        }
    }
    free(l);
    free(chosen);
    free(u);
  }
  return bad ? 2 : 0;
}

/* ---------------------------------------------------------------------------------------- */
/* hash routing                                                                              */
/*                                                                                          */
/* [CANN] "CANN DeepSeek-V4推理优化", MoE section: the first layers choose experts by hash      */
/* routing, the later ones by the learned router. Read plainly: the k experts of a token are */
/* a fixed function of its token id (row id of a [vocab][k] table), independent of x; the   */
/* weights stay those of the router (step 3) renormalised over that set. Output order: the   */
/* valid entries (in [0, E)) ascending by expert index, equal indices in table order, then   */
/* the invalid ones (or all k for an id outside [0, vocab)) as index -1 with weight 0.        */
/* ---------------------------------------------------------------------------------------- */

int oracle_route_hash(int T, int H, int E, int k, int act, const void* x, const void* Wr,
                      const float* bias, const int32_t* token_ids, const int32_t* table, int vocab,
                      int32_t* topk_idx, double* topk_w) {
  if (T < 0 || H < 1 || E < 1 || k < 1 || k > 16 || vocab < 0) return 1;
  double* l = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * E);
  if (!l) return 2;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * k);
  double* w = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * k);
  int rc = (!idx || !w) ? 2 : oracle_route(T, H, E, k, act, x, Wr, bias, idx, w, l);
  for (int t = 0; t < T && !rc; ++t) {
    const double* lt = l + (size_t)t * E;
    const int id = token_ids[t];
    int e_of[16], key[16];
    for (int r = 0; r < k; ++r) {
      const int e = (id >= 0 && id < vocab) ? table[(size_t)id * k + r] : -1;
      e_of[r] = (e >= 0 && e < E) ? e : -1;
      key[r] = (e_of[r] >= 0 ? e_of[r] : E + r) * 16 + r; /* unique: table order breaks ties */
    }
    double m = -INFINITY, z = 0.0;
    for (int r = 0; r < k; ++r)
      if (e_of[r] >= 0 && lt[e_of[r]] > m) m = lt[e_of[r]];
    for (int r = 0; r < k; ++r)
      if (e_of[r] >= 0) z += exp(lt[e_of[r]] - m);
    for (int r = 0; r < k; ++r) {
      int rank = 0;
      for (int q = 0; q < k; ++q) rank += key[q] < key[r];
      topk_idx[(size_t)t * k + rank] = e_of[r];
      topk_w[(size_t)t * k + rank] = e_of[r] >= 0 ? exp(lt[e_of[r]] - m) / z : 0.0;
    }
  }
  free(l);
  free(idx);
  free(w);
  return rc;
}

/* ---------------------------------------------------------------------------------------- */
/* step 4: permutation (a stable counting sort of the pairs q = t*k + j by expert)           */
/* ---------------------------------------------------------------------------------------- */

int oracle_permute(int T, int k, int E, const int32_t* topk_idx, int32_t* expert_offsets,
                   int32_t* slot_token, int32_t* pair_slot) {
  int P = T * k;
  int32_t* fill = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
  if (!fill) return 2;
  for (int e = 0; e <= E; ++e) expert_offsets[e] = 0;
  for (int q = 0; q < P; ++q) {
    int e = topk_idx[q];
    if (e == -1) continue; /* "no expert" (hash routing's invalid entries): skipped */
    if (e < 0 || e >= E) {
      free(fill);
      return 1;
    }
    expert_offsets[e + 1] += 1;
  }
  for (int e = 0; e < E; ++e) expert_offsets[e + 1] += expert_offsets[e];
  for (int e = 0; e < E; ++e) fill[e] = expert_offsets[e];
  for (int q = 0; q < P; ++q) {
    if (topk_idx[q] == -1) {
      pair_slot[q] = -1;
      continue;
    }
    int slot = fill[topk_idx[q]]++;
    slot_token[slot] = q / k;
    pair_slot[q] = slot;
  }
  free(fill);
  return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* step 5/6: one expert's SwiGLU FFN on M rows                                               */
/* ---------------------------------------------------------------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* ---------------------------------------------------------------------------------------- */
/* W4A8: activations quantised to MXFP8 for the routed experts' products                     */
/*                                                                                          */
/* [CANN] "CANN DeepSeek-V4推理优化", quantisation strategy: the routed experts' linear layers */
/* run W4A8, 4-bit weights times 8-bit activations. The 8-bit activation format read here is */
/* OCP MXFP8 (OCP Microscaling Formats v1.0): each run of 32 consecutive reduction elements   */
/* shares an e8m0 exponent X = floor(log2 max|v|) - 8 (8 is the largest E4M3 exponent),      */
/* clamped to [-127, 127] and -127 for an all-zero run; each element is stored as           */
/* E4M3FN(v / 2^X), rounded to nearest even and saturated at +-448.                         */
/* ---------------------------------------------------------------------------------------- */

/* E4M3FN code of v, round to nearest even, saturating (the sign of v, zero included, kept). */
static uint8_t e4m3_encode(double v) {
  const uint8_t s = signbit(v) ? 0x80 : 0;
  const double a = fabs(v);
  if (!(a < 448.0)) return s | 0x7E;
  if (a < ldexp(1.0, -6)) return s | (uint8_t)nearbyint(ldexp(a, 9)); /* grid 2^-9; 8 -> 0x08 */
  int e = ilogb(a);                                                    /* -6 .. 8 */
  double m = nearbyint((ldexp(a, -e) - 1.0) * 8.0);                    /* 0 .. 8 */
  if (m == 8.0) {
    e += 1;
    m = 0.0;
  }
  int code = ((e + 7) << 3) | (int)m;
  if (code > 0x7E) code = 0x7E; /* 464 <= a < 480 would round to the NaN pattern */
  return s | (uint8_t)code;
}

/* K values (K a multiple of 32) -> K E4M3FN codes and K/32 e8m0 exponents. */
int oracle_mxfp8_quantize(int K, const double* v, uint8_t* codes, uint8_t* scales) {
  if (K % 32) return 1;
  for (int b = 0; b < K / 32; ++b) {
    double amax = 0.0;
    for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs(v[32 * b + j]));
    int X = amax > 0.0 ? ilogb(amax) - 8 : -127;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    scales[b] = (uint8_t)(X + 127);
    for (int j = 0; j < 32; ++j) codes[32 * b + j] = e4m3_encode(ldexp(v[32 * b + j], -X));
  }
  return 0;
}

/* v -> the value its MXFP8 encoding stands for (quantise, then decode), in place. */
static int mxfp8_roundtrip(int K, double* v) {
  uint8_t* c = (uint8_t*)malloc(K);
  uint8_t* e = (uint8_t*)malloc(K / 32 + 1);
  int rc = (!c || !e) ? 2 : oracle_mxfp8_quantize(K, v, c, e);
  for (int i = 0; i < K && !rc; ++i) v[i] = oracle_decode_e4m3fn(c[i]) * oracle_decode_e8m0(e[i / 32]);
  free(c);
  free(e);
  return rc;
}

/* ---------------------------------------------------------------------------------------- */
/* Int8 W8A8: activations quantised to int8 per token                                       */
/*                                                                                          */
/* [CANN] "CANN DeepSeek-V4推理优化", Int8 quantisation strategy: the routed and shared      */
/* experts' linear layers run W8A8, weights statically quantised to int8 per output channel, */
/* activations dynamically to int8 per token. Per token (one row of K values), in fp32: the  */
/* largest magnitude a, the factor f = 127 / a and the scale s = a / 127 (fp32 divisions),    */
/* and each code q = v * f (fp32 product) rounded to the nearest integer, ties to even,     */
/* clamped to [-127, 127]; the row then stands for q * s. An all-zero row has s = 0, q = 0.  */
/* f is formed with a's binary exponent taken out: a = m 2^e (m in [0.5, 1)), f = 127 / m   */
/* and q = rint((v 2^-e) * f). Scaling by 2^-e is exact, so this is the same fp32 number as  */
/* v * (127 / a) wherever 127 / a is finite, and it stays defined for rows whose maximum is  */
/* so small (below about 2^-121) that 127 / a overflows fp32.                                 */
/* The rows quantised here (bf16 values, or h after its bf16 rounding) are exact in fp32,    */
/* so this decision is the same on any IEEE machine.                                        */
/* ---------------------------------------------------------------------------------------- */

int oracle_int8_quantize(int K, const double* v, int8_t* codes, float* scale) {
  float a = 0.0f;
  for (int i = 0; i < K; ++i) {
    const float x = (float)v[i];
    if ((double)x != v[i]) return 1; /* the row must be exact in fp32 */
    a = fmaxf(a, fabsf(x));
  }
  if (a == 0.0f) {
    memset(codes, 0, (size_t)K);
    *scale = 0.0f;
    return 0;
  }
  int e;
  const float m = frexpf(a, &e);                  /* a = m 2^e exactly */
  volatile float f = 127.0f / m, s = a / 127.0f; /* fp32 roundings, not extended precision */
  for (int i = 0; i < K; ++i) {
    volatile float p = ldexpf((float)v[i], -e) * f;
    float q = rintf(p);
    if (q > 127.0f) q = 127.0f;
    if (q < -127.0f) q = -127.0f;
    codes[i] = (int8_t)q;
  }
  *scale = s;
  return 0;
}

/* v -> the value its int8 encoding stands for, in place. */
static int int8_roundtrip(int K, double* v) {
  int8_t* c = (int8_t*)malloc(K);
  float s = 0.0f;
  int rc = !c ? 2 : oracle_int8_quantize(K, v, c, &s);
  for (int i = 0; i < K && !rc; ++i) v[i] = (double)c[i] * (double)s;
  free(c);
  return rc;
}

/* v rounded to the nearest bfloat16 (8 significant bits), ties to even. */
static double bf16_round(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e = ilogb(v);
  if (e < -126) e = -126;
  return ldexp(nearbyint(ldexp(v, 7 - e)), e - 7);
}

/* W4A8 (fmt mxfp4a8) and W8A8 MXFP8 (fmt mxfp8a8): the row is quantised to MXFP8 before gate/up;
 * h = SiLU(g) * v is rounded to bf16, the type the layer keeps it in between the two products,
 * then quantised to MXFP8 before down. Int8 W8A8 (fmt int8): the same with the per-token int8
 * quantisation. Other formats multiply the rows as given. */
int oracle_expert_ffn(int H, int I, int M, int fmt, const void* wg, const void* sg,
                      const void* wu, const void* su, const void* wd, const void* sd,
                      const double* u, double* y) {
  int bad = 0;
  const int a8 = fmt == OR_MXFP4_A8 || fmt == OR_MXFP8_A8, i8 = fmt == OR_INT8;
#pragma omp parallel for schedule(dynamic, 1) if (M > 1)
  for (int m = 0; m < M; ++m) {
    double* g = (double*)malloc(sizeof(double) * I);
    double* v = (double*)malloc(sizeof(double) * I);
    double* uq = (double*)malloc(sizeof(double) * H);
    if (!g || !v || !uq) {
      bad = 1;
    } else {
      memcpy(uq, u + (size_t)m * H, sizeof(double) * H);
      if (a8 && mxfp8_roundtrip(H, uq)) bad = 1;
      if (i8 && int8_roundtrip(H, uq)) bad = 1;
      oracle_row_matmul(H, I, fmt, wg, sg, uq, g);
      oracle_row_matmul(H, I, fmt, wu, su, uq, v);
      for (int i = 0; i < I; ++i) g[i] = silu(g[i]) * v[i];
      if (a8 || i8) {
        for (int i = 0; i < I; ++i) g[i] = bf16_round(g[i]);
        if (a8 ? mxfp8_roundtrip(I, g) : int8_roundtrip(I, g)) bad = 1;
      }
      oracle_row_matmul(I, H, fmt, wd, sd, g, y + (size_t)m * H);
    }
    free(g);
    free(v);
    free(uq);
  }
  return bad ? 2 : 0;
}

/* ---------------------------------------------------------------------------------------- */
/* step 7: combine one token                                                                  */
/* ---------------------------------------------------------------------------------------- */

int oracle_combine_token(int H, int k, const double* w, const double* yk, const double* ysh,
                         double* y) {
  for (int n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int j = 0; j < k; ++j) acc += w[j] * yk[(size_t)j * H + n];
    y[n] = acc + (ysh ? ysh[n] : 0.0);
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* the whole layer, steps 1-7                                                                */
/* ---------------------------------------------------------------------------------------- */

/* steps 4-7 from a given routing (topk_idx, topk_w) */
static int layer_after_route(int T, int H, int E, int k, int I, int act, const void* x, int fmt_r,
                             const void* rg, const void* rsg, const void* ru, const void* rsu,
                             const void* rd, const void* rsd, int has_shared, int fmt_s,
                             const void* sg, const void* ssg, const void* su, const void* ssu,
                             const void* sd, const void* ssd, const int32_t* topk_idx,
                             const double* topk_w, int32_t* expert_offsets, int32_t* slot_token,
                             int32_t* pair_slot, double* y) {
  int P = T * k, rc;
  rc = oracle_permute(T, k, E, topk_idx, expert_offsets, slot_token, pair_slot);
  if (rc) return rc;
  size_t gw = w_bytes(fmt_r, H, I), gs = s_bytes(fmt_r, H, I);
  size_t dw = w_bytes(fmt_r, I, H), ds = s_bytes(fmt_r, I, H);
  double* xin = (double*)malloc(sizeof(double) * (size_t)(P > T ? P : T) * H);
  double* yperm = (double*)malloc(sizeof(double) * (size_t)P * H);
  double* ysh = has_shared ? (double*)malloc(sizeof(double) * (size_t)T * H) : NULL;
  if (!xin || !yperm || (has_shared && !ysh)) return 2;
  /* rows of each expert's group, gathered in slot order (the expert_offsets[E] pairs with one) */
  for (int r = 0; r < expert_offsets[E]; ++r)
    for (int h = 0; h < H; ++h) xin[(size_t)r * H + h] = act_at(x, act, (size_t)slot_token[r] * H + h);
  for (int e = 0; e < E && !rc; ++e) {
    int r0 = expert_offsets[e], M = expert_offsets[e + 1] - r0;
    if (M == 0) continue;
    rc = oracle_expert_ffn(H, I, M, fmt_r, (const char*)rg + e * gw, rsg ? (const char*)rsg + e * gs : NULL,
                           (const char*)ru + e * gw, rsu ? (const char*)rsu + e * gs : NULL,
                           (const char*)rd + e * dw, rsd ? (const char*)rsd + e * ds : NULL,
                           xin + (size_t)r0 * H, yperm + (size_t)r0 * H);
  }
  if (has_shared && !rc) {
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h) xin[(size_t)t * H + h] = act_at(x, act, (size_t)t * H + h);
    rc = oracle_expert_ffn(H, I, T, fmt_s, sg, ssg, su, ssu, sd, ssd, xin, ysh);
  }
  if (!rc) {
    double* yk = (double*)malloc(sizeof(double) * (size_t)k * H);
    if (!yk) rc = 2;
    for (int t = 0; t < T && !rc; ++t) {
      for (int j = 0; j < k; ++j) {
        const int32_t ps = pair_slot[(size_t)t * k + j];
        if (ps >= 0)
          memcpy(yk + (size_t)j * H, yperm + (size_t)ps * H, sizeof(double) * H);
        else /* a pair without an expert (hash routing's invalid entries) adds nothing */
          memset(yk + (size_t)j * H, 0, sizeof(double) * H);
      }
      oracle_combine_token(H, k, topk_w + (size_t)t * k, yk, ysh ? ysh + (size_t)t * H : NULL,
                           y + (size_t)t * H);
    }
    free(yk);
  }
  free(xin);
  free(yperm);
  free(ysh);
  return rc;
}

int oracle_layer(int T, int H, int E, int k, int I, int act, const void* x, const void* Wr,
                 const float* bias, int fmt_r, const void* rg, const void* rsg, const void* ru,
                 const void* rsu, const void* rd, const void* rsd, int has_shared, int fmt_s,
                 const void* sg, const void* ssg, const void* su, const void* ssu,
                 const void* sd, const void* ssd, int32_t* topk_idx, double* topk_w,
                 int32_t* expert_offsets, int32_t* slot_token, int32_t* pair_slot, double* y) {
  int rc = oracle_route(T, H, E, k, act, x, Wr, bias, topk_idx, topk_w, NULL);
  if (rc) return rc;
  return layer_after_route(T, H, E, k, I, act, x, fmt_r, rg, rsg, ru, rsu, rd, rsd, has_shared, fmt_s, sg,
                           ssg, su, ssu, sd, ssd, topk_idx, topk_w, expert_offsets, slot_token, pair_slot, y);
}

/* the whole layer with hash routing (steps 1-3 replaced by oracle_route_hash) */
int oracle_layer_hash(int T, int H, int E, int k, int I, int act, const void* x, const void* Wr,
                      const float* bias, const int32_t* token_ids, const int32_t* table, int vocab,
                      int fmt_r, const void* rg, const void* rsg, const void* ru, const void* rsu,
                      const void* rd, const void* rsd, int has_shared, int fmt_s, const void* sg,
                      const void* ssg, const void* su, const void* ssu, const void* sd,
                      const void* ssd, int32_t* topk_idx, double* topk_w, int32_t* expert_offsets,
                      int32_t* slot_token, int32_t* pair_slot, double* y) {
  int rc = oracle_route_hash(T, H, E, k, act, x, Wr, bias, token_ids, table, vocab, topk_idx, topk_w);
  if (rc) return rc;
  return layer_after_route(T, H, E, k, I, act, x, fmt_r, rg, rsg, ru, rsu, rd, rsd, has_shared, fmt_s, sg,
                           ssg, su, ssu, sd, ssd, topk_idx, topk_w, expert_offsets, slot_token, pair_slot, y);
}
