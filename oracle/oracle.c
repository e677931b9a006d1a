/*
 * oracle.c -- plain, slow CPU oracle for weight-only low-bit dequantize-and-multiply.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may link, load or call this
 * file; only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no source with the HIP kernels and includes none of their headers.
 *
 * Sources (the web pages this is written from):
 *   [CCQ]  "CCQ: Convolutional Code for Extreme Low-bit Quantization in LLMs" (arXiv 2507.07145).
 *   [WINT2] FastDeploy documentation page "WINT2 Quantization".
 *   [E6.4] coursefy lesson E6.4 "GPTQ and AWQ" (INT4 packing exercise, affine formulas,
 *          worked example).
 *
 * Arithmetic rules:
 *   - bf16 <-> f32 conversions are written out here (round-to-nearest-even, NaN -> 0x7FC0).
 *   - Decode follows the pages' formulas in fp32 exactly as stated, one rounding per
 *     operation; the fp32 fused multiply-add of the code-cluster stage is an explicit fmaf.
 *     Build with -ffp-contract=off so no other multiply-add is fused.
 *   - Every sum of products (GEMM, MoE) is accumulated in fp64 and rounded once to bf16:
 *     the plain definition y = bf16(sum_k x_k * w_k).
 *   - OpenMP only splits independent outputs between threads; it never changes the order
 *     in which one output is summed.
 *
 * Readings where the pages leave a step open are listed next to the code that takes them.
 * Parity status: stage 1 of the code-cluster decode (the fp32 fma + rounding) has no worked
 * example on the pages; it is pinned by invariants and an exact-rational re-statement only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------------------------ */
/* bf16                                                                                        */
/* ------------------------------------------------------------------------------------------ */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round an fp32 value to bf16, ties to even.  NaN becomes the canonical quiet NaN 0x7FC0. */
static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Round an fp64 value straight to bf16 (one rounding, ties to even), never via fp32. */
static uint16_t f64_to_bf16(double d) {
  if (isnan(d)) return 0x7FC0;
  if (d == 0.0 || isinf(d)) return f32_to_bf16((float)d); /* exact */
  uint16_t sign = signbit(d) ? 0x8000 : 0;
  double a = fabs(d);
  int e;
  (void)frexp(a, &e);         /* a = m * 2^e, m in [0.5, 1) */
  int q = e - 8;              /* bf16 keeps 8 significant bits */
  if (q < -133) q = -133;     /* bf16 subnormal spacing is 2^-133 */
  double r = nearbyint(ldexp(a, -q)) ; /* exact scaling, then round-half-even to an integer */
  double v = ldexp(r, q);
  if (v >= 0x1p128) return (uint16_t)(sign | 0x7F80);
  float fv = (float)v;        /* exact: v has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &fv, 4);
  return (uint16_t)(sign | (u >> 16));
}

ORC_API void orc_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

ORC_API void orc_f64_to_bf16(const double* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* [E6.4] "Do it in code": INT4 packing helpers, nominal size, RTN; "Math and notation":     */
/* affine quantization.                                                                        */
/* ------------------------------------------------------------------------------------------ */

/* Two signed codes per byte: the first code of each pair in the low nibble, the second in
 * the high nibble; an odd count is padded with a 0 code.  Returns 0, or -4 if any code is
 * outside -8..7 (the exercise raises ValueError there) -- in that case nothing is written. */
ORC_API int32_t orc_pack_int4(const int32_t* codes, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i)
    if (codes[i] < -8 || codes[i] > 7) return -4;
  for (int64_t b = 0; b < (n + 1) / 2; ++b) {
    int32_t lo = codes[2 * b];
    int32_t hi = (2 * b + 1 < n) ? codes[2 * b + 1] : 0;
    out[b] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
  }
  return 0;
}

/* The first n signed codes back, each 4-bit field sign-extended. */
ORC_API void orc_unpack_int4(const uint8_t* data, int64_t n, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    int32_t nib = (data[i >> 1] >> (4 * (i & 1))) & 0xF;
    out[i] = nib >= 8 ? nib - 16 : nib;
  }
}

/* Nominal packed size M = N*b/8 bytes (scales excluded), rounded up to whole bytes. */
ORC_API int64_t orc_packed_size(int64_t n_codes, int32_t bits) {
  return (n_codes * (int64_t)bits + 7) / 8;
}

/* Plain round-to-nearest 4-bit quantization, returned dequantized:
 * clip(round(w/scale), -8, 7) * scale with ties to even (numpy's round), in fp64. */
ORC_API void orc_rtn(const double* w, int64_t n, double scale, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    double q = nearbyint(w[i] / scale);
    if (q < -8) q = -8;
    if (q > 7) q = 7;
    out[i] = q * scale;
  }
}

/* Affine quantization q = clip(round(x/s) + z, qmin, qmax) (ties to even), fp64. */
ORC_API void orc_affine_quant(const double* x, int64_t n, double s, int32_t z, int32_t qmin,
                              int32_t qmax, int32_t* q) {
  for (int64_t i = 0; i < n; ++i) {
    double v = nearbyint(x[i] / s) + (double)z;
    if (v < qmin) v = qmin;
    if (v > qmax) v = qmax;
    q[i] = (int32_t)v;
  }
}

/* Affine reconstruction x_hat = s * (q - z), fp64. */
ORC_API void orc_affine_dequant(const int32_t* q, int64_t n, double s, int32_t z, double* xhat) {
  for (int64_t i = 0; i < n; ++i) xhat[i] = s * (double)(q[i] - z);
}

/* ------------------------------------------------------------------------------------------ */
/* [CCQ] section 3.1: convolutional-code codebook (L, N, S) and bit-shift decoding.            */
/* ------------------------------------------------------------------------------------------ */

/* Total bits of one convolutional code: T = L + (N - 1) * S. */
ORC_API int32_t orc_ccq_total_bits(int32_t L, int32_t N, int32_t S) { return L + (N - 1) * S; }

/* Shift of state i: state i of a code starts (N - 1 - i) * S bits above bit 0, so the first
 * state sits in the highest bits (it was the first stored; later transitions are appended
 * below it).  Fills shifts[0..N-1]. */
ORC_API void orc_ccq_shifts(int32_t L, int32_t N, int32_t S, int32_t* shifts) {
  (void)L;
  for (int32_t i = 0; i < N; ++i) shifts[i] = (N - 1 - i) * S;
}

/* Bit-shift decode of one code into its N states of L bits each. */
ORC_API void orc_ccq_states(uint32_t code, int32_t L, int32_t N, int32_t S, int32_t* states) {
  uint32_t mask = (L >= 32) ? 0xFFFFFFFFu : ((1u << L) - 1u);
  for (int32_t i = 0; i < N; ++i) states[i] = (int32_t)((code >> ((N - 1 - i) * S)) & mask);
}

/* Equivalent bits per weight, [CCQ] section 3.4 Eq. (bpw): T*ceil(g/N)/g when g = 1 (mod N)
 * (the scale lives in the last code's spare bits), T*(g/N)/g + scale_bits/g when N divides g.
 * With the code cluster T is the 8 bits of the clustered code.  Returns -1 otherwise. */
ORC_API double orc_ccq_bpw(int32_t T, int32_t g, int32_t N, int32_t scale_bits) {
  if (g % N == 1) return (double)T * (double)((g + N - 1) / N) / (double)g;
  if (g % N == 0) return (double)T * (double)(g / N) / (double)g + (double)scale_bits / (double)g;
  return -1.0;
}

/* ------------------------------------------------------------------------------------------ */
/* Packed weight descriptor (the oracle's own; one [n, k] matrix per expert).                  */
/*   format 1: INT4 codes u8[E][n][k/2] (low nibble = even k, two's complement), scales bf16   */
/*             [E][n][k/64] (group 64) or [E][n] (group 0 = per channel), zero point 0.        */
/*   format 2: 2-bit affine codes u8[E][n][k/4] (lowest two bits = k%4 == 0), scales bf16      */
/*             [E][n][k/64], zeros u8 [E][n][k/64].                                            */
/*   format 3: CCQ (L,N,S) = (6,4,3) with code cluster: codes u8[E][n][k/4] (one clustered     */
/*             code per 4 weights), qscale u8[E][n][ceil(k/128)] (two 4-bit group scales per   */
/*             byte, low nibble = even group), super/code_scale/code_zero f32 [E][n], zp.       */
/*   format 4: CCQ (4,3,2) without code cluster, 2.75 bpw: 22 u8 code words per 64-weight     */
/*             group, codes u8[E][n][k/64*22]; the last word's low 4 bits hold the group's    */
/*             quantized scale; super f32 [E][n], zp.                                         */
/*   format 5: CCQ hybrid (3,3,2)+(3,4,2), 2.5 bpw: 10 u16 code words per group (little      */
/*             endian), codes u8[E][n][k/64*20]; the last word's low 13 bits hold the group's */
/*             quantized scale; super f32 [E][n], zp.                                         */
/*   format 6: WINT8, one signed byte per weight (two's complement), codes i8[E][n][k];       */
/*             scales bf16 [E][n][k/64] (group 64) or [E][n] (group 0, per output channel).   */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
  int32_t format;
  int32_t group;
  int64_t experts;
  int64_t n;
  int64_t k;
  const uint8_t* codes;
  const uint16_t* scales;
  const uint8_t* zeros;
  const uint8_t* qscale;
  const float* super_scale;
  const float* code_scale;
  const float* code_zero;
  int32_t zp;
} orc_weight;

enum { ORC_INT4 = 1, ORC_AFFINE2 = 2, ORC_CCQ = 3, ORC_CCQ432 = 4, ORC_CCQ_HYBRID = 5, ORC_INT8 = 6 };

/* [E6.4] "Do it in code" (sign-extended 4-bit field) and "Math and notation" (x_hat = s(q-z)
 * with z = 0): W_hat = bf16(f32(q) * f32(s)). */
static uint16_t decode_int4(const orc_weight* w, int64_t e, int64_t n, int64_t k) {
  int64_t row = e * w->n + n;
  uint8_t byte = w->codes[row * (w->k / 2) + (k >> 1)];
  int32_t nib = (byte >> (4 * (k & 1))) & 0xF;
  int32_t q = nib >= 8 ? nib - 16 : nib;
  float s = (w->group == 0) ? bf16_to_f32(w->scales[row])
                            : bf16_to_f32(w->scales[row * (w->k / w->group) + k / w->group]);
  float d = (float)q * s;
  return f32_to_bf16(d);
}

/* WINT8 (FastDeploy "Quantization" precision list: INT8 weights, BF16 activations) read with the
 * [E6.4] formula x_hat = s(q - z), z = 0, at b = 8: W_hat = bf16(f32(q) * f32(s)), q the byte as
 * a signed 8-bit integer.  Reading: the scale granularity follows INT4 (group 64 or per channel). */
static uint16_t decode_int8(const orc_weight* w, int64_t e, int64_t n, int64_t k) {
  int64_t row = e * w->n + n;
  int32_t q = (int32_t)(int8_t)w->codes[row * w->k + k];
  float s = (w->group == 0) ? bf16_to_f32(w->scales[row])
                            : bf16_to_f32(w->scales[row * (w->k / w->group) + k / w->group]);
  float d = (float)q * s;
  return f32_to_bf16(d);
}

/* [E6.4] "Math and notation": x_hat = s * (q - z) for a 2-bit code, per-group s and z.
 * Reading: the lowest two bits of a byte hold the first of its four weights (the same
 * lowest-first order the INT4 exercise uses for nibbles). */
static uint16_t decode_affine2(const orc_weight* w, int64_t e, int64_t n, int64_t k) {
  int64_t row = e * w->n + n;
  int64_t groups = w->k / 64;
  uint8_t byte = w->codes[row * (w->k / 4) + (k >> 2)];
  int32_t q = (byte >> (2 * (k & 3))) & 3;
  int32_t z = w->zeros[row * groups + k / 64];
  float s = bf16_to_f32(w->scales[row * groups + k / 64]);
  float d = (float)(q - z) * s;
  return f32_to_bf16(d);
}

/* [CCQ] section 3.3, Eq. (code cluster), inverted: the clustered byte C' expands to a code
 * C = round(C' * code_scale + code_zero).  Readings: one fp32 fused multiply-add, then round
 * half to even, then clamp into the T = 15-bit code range [0, 2^15 - 1].  This is the first
 * of the two dequantization stages of section 3.5. */
ORC_API uint32_t orc_ccq_expand(uint32_t cprime, float code_scale, float code_zero) {
  float t = fmaf((float)cprime, code_scale, code_zero);
  float r = nearbyintf(t);
  r = fmaxf(r, 0.0f);
  r = fminf(r, 32767.0f);
  return (uint32_t)r;
}

/* [CCQ] section 3.5, "Dequantization with Code Cluster", with the (6,4,3) row of the
 * dequantization-configuration table: weight bit-shifts (9,6,3,0), weight mask 0x3F, scale
 * mask 0xF.  For weight index k of a row:
 *   s      = ((s_q >> s_shift) & 0xF) * s_super           (fp32 multiply)
 *   C      = expand(W_q[k / 4])                            (stage 1)
 *   u      = (C >> shift[k % 4]) & 0x3F                    (stage 2)
 *   W_hat  = bf16((u - zp) * s)                            (fp32 multiply, then bf16)
 * Readings: s_q holds two 4-bit group scales per byte (even group in the low nibble, so
 * s_shift = 4 * (group & 1)); super, code scale and code zero are per output channel; the
 * two multiplies are done in the order written, each rounded to fp32. */
static uint16_t decode_ccq(const orc_weight* w, int64_t e, int64_t n, int64_t k) {
  int64_t row = e * w->n + n;
  int64_t groups = w->k / 64;
  int64_t qs_bytes = (groups + 1) / 2;
  int64_t g = k / 64;
  uint32_t sq = (w->qscale[row * qs_bytes + (g >> 1)] >> (4 * (g & 1))) & 0xFu;
  float s = (float)sq * w->super_scale[row];
  uint32_t cp = w->codes[row * (w->k / 4) + (k >> 2)];
  uint32_t C = orc_ccq_expand(cp, w->code_scale[row], w->code_zero[row]);
  static const int32_t shift[4] = {9, 6, 3, 0};
  int32_t u = (int32_t)((C >> shift[k & 3]) & 0x3Fu);
  float d = (float)(u - w->zp) * s;
  return f32_to_bf16(d);
}

/* [CCQ] section 3.5, "Dequantization without Code Cluster", with the (4,3,2) and hybrid
 * (3,3,2)(3,4,2) rows of the dequantization-configuration table, and section 3.4 (scale
 * compression: the group's quantized scale sits in the redundant bits of its last code word).
 * For weight index i of a 64-weight group whose code words are W[0 .. P-1]:
 *   s      = (W[P-1] & s_mask) * s_super                    (fp32 multiply)
 *   u      = (W[i / p_w] >> shift[i % p_w]) & w_mask
 *   W_hat  = bf16((u - zp) * s)                             (fp32 multiply, then bf16)
 * with p_w the number of shifts.  (4,3,2): u8 words, P = 22, shifts (4,2,0), w_mask 0xF,
 * s_mask 0xF.  Hybrid: u16 words, P = 10, shifts (13,11,9,6,4,2,0), w_mask 0x7, s_mask
 * 0x1FFF.  Readings: a group's words are stored consecutively and groups consecutively along
 * the row; u16 words are little endian; the states of a word are taken in the order of the
 * shift list (the first state uses the highest shift). */
static uint32_t alg2_word(const orc_weight* w, int64_t row, int64_t g, int64_t j) {
  if (w->format == ORC_CCQ432) return w->codes[row * (w->k / 64) * 22 + g * 22 + j];
  const uint8_t* b = w->codes + row * (w->k / 64) * 20 + g * 20 + 2 * j;
  return (uint32_t)b[0] | ((uint32_t)b[1] << 8);
}

static uint16_t decode_alg2(const orc_weight* w, int64_t e, int64_t n, int64_t k) {
  static const int32_t sh432[3] = {4, 2, 0};
  static const int32_t shhyb[7] = {13, 11, 9, 6, 4, 2, 0};
  const int hyb = w->format == ORC_CCQ_HYBRID;
  const int32_t P = hyb ? 10 : 22, pw = hyb ? 7 : 3;
  const uint32_t wmask = hyb ? 0x7u : 0xFu, smask = hyb ? 0x1FFFu : 0xFu;
  const int32_t* shift = hyb ? shhyb : sh432;
  int64_t row = e * w->n + n;
  int64_t g = k / 64, i = k % 64;
  float s = (float)(alg2_word(w, row, g, P - 1) & smask) * w->super_scale[row];
  int32_t u = (int32_t)((alg2_word(w, row, g, i / pw) >> shift[i % pw]) & wmask);
  float d = (float)(u - w->zp) * s;
  return f32_to_bf16(d);
}

static uint16_t decode_one(const orc_weight* w, int64_t e, int64_t n, int64_t k) {
  switch (w->format) {
    case ORC_INT4: return decode_int4(w, e, n, k);
    case ORC_INT8: return decode_int8(w, e, n, k);
    case ORC_AFFINE2: return decode_affine2(w, e, n, k);
    case ORC_CCQ432:
    case ORC_CCQ_HYBRID: return decode_alg2(w, e, n, k);
    default: return decode_ccq(w, e, n, k);
  }
}

static int check_weight(const orc_weight* w) {
  if (w->k <= 0 || w->n <= 0 || w->k % 64 != 0) return -1;
  if (w->format == ORC_INT4 || w->format == ORC_INT8) return (w->group == 64 || w->group == 0) ? 0 : -1;
  if (w->format == ORC_AFFINE2 || w->format == ORC_CCQ || w->format == ORC_CCQ432 ||
      w->format == ORC_CCQ_HYBRID)
    return w->group == 64 ? 0 : -1;
  return -1;
}

/* Decode rows [n0, n1) of expert e to bf16, row-major [n1 - n0][k]. */
ORC_API int32_t orc_dequantize(const orc_weight* w, int64_t e, int64_t n0, int64_t n1,
                               uint16_t* out) {
  if (check_weight(w) || e < 0 || e >= w->experts || n0 < 0 || n1 > w->n || n0 > n1) return -1;
  int64_t k = w->k;
#pragma omp parallel for schedule(static)
  for (int64_t n = n0; n < n1; ++n)
    for (int64_t kk = 0; kk < k; ++kk) out[(n - n0) * k + kk] = decode_one(w, e, n, kk);
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Dense product: y = x * W_hat^T, bf16 operands, fp64 sum, one rounding to bf16.              */
/* [WINT2]: weights are decoded to BF16 and the arithmetic is carried out on BF16 values.      */
/* ------------------------------------------------------------------------------------------ */

/* x bf16 [m][k], w bf16 [n][k] (already decoded), y bf16 [m][n]; y64 (optional) receives the
 * unrounded fp64 sums. */
ORC_API void orc_gemm_bf16(const uint16_t* x, int64_t m, int64_t k, const uint16_t* w, int64_t n,
                           uint16_t* y, double* y64) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int64_t kk = 0; kk < k; ++kk)
        acc += (double)bf16_to_f32(x[i * k + kk]) * (double)bf16_to_f32(w[j * k + kk]);
      if (y) y[i * n + j] = f64_to_bf16(acc);
      if (y64) y64[i * n + j] = acc;
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Mixture-of-experts expert FFN.                                                              */
/* Routing: pairs p = t*topk + j (token t, slot j) grouped by expert id, stable in p.          */
/* ------------------------------------------------------------------------------------------ */

/* Counting sort of the pair indices by expert: offsets[e] = number of pairs routed to experts
 * below e (offsets[E] = t*topk); sorted_pairs lists the pair indices of expert 0 first, then
 * expert 1, ..., each in increasing p.  Returns -1 (and writes nothing) for an id outside
 * [0, E). */
ORC_API int32_t orc_moe_route(const int32_t* ids, int64_t t, int32_t topk, int32_t experts,
                              int32_t* offsets, int32_t* sorted_pairs) {
  int64_t pairs = t * (int64_t)topk;
  for (int64_t p = 0; p < pairs; ++p)
    if (ids[p] < 0 || ids[p] >= experts) return -1;
  int64_t* count = (int64_t*)calloc((size_t)experts + 1, sizeof(int64_t));
  for (int64_t p = 0; p < pairs; ++p) count[ids[p]]++;
  offsets[0] = 0;
  for (int32_t e = 0; e < experts; ++e) offsets[e + 1] = offsets[e] + (int32_t)count[e];
  for (int32_t e = 0; e < experts; ++e) count[e] = offsets[e];
  for (int64_t p = 0; p < pairs; ++p) sorted_pairs[count[ids[p]]++] = (int32_t)p;
  free(count);
  return 0;
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* For the tokens listed in `tokens` (n_tok of them; all of them if tokens == NULL):
 *   for each slot j, e = ids[t][j]:
 *     g = W_gate[e] x_t, u = W_up[e] x_t                       (fp64 sums of bf16 products)
 *     h = bf16(SiLU(g) * u)                                    (one rounding; BF16 operand)
 *     d_j = W_down[e] h                                        (fp64)
 *   y_t = bf16(sum_j weights[t][j] * d_j)                      (fp64, slots in order j = 0..)
 * Routing weights are used as given.  Duplicate ids in a row simply add.  x bf16 [t][hidden],
 * y bf16 [n_tok][hidden] (row i belongs to tokens[i]).  gate/up are [E][inter][hidden] and
 * down is [E][hidden][inter].  Each expert's matrices are decoded once (fully, by the decode
 * functions above) and reused by every pair routed to it; that only changes which work is
 * shared, never the arithmetic of any output. */
ORC_API int32_t orc_moe_ffn(const uint16_t* x, int64_t t, int64_t hidden, const int32_t* ids,
                            const float* weights, int32_t topk, int32_t experts,
                            const orc_weight* gate, const orc_weight* up,
                            const orc_weight* down, int64_t inter, const int32_t* tokens,
                            int64_t n_tok, uint16_t* y) {
  if (check_weight(gate) || check_weight(up) || check_weight(down)) return -1;
  if (gate->n != inter || up->n != inter || gate->k != hidden || up->k != hidden ||
      down->n != hidden || down->k != inter)
    return -1;
  if (gate->experts < experts || up->experts < experts || down->experts < experts) return -1;
  if (tokens == NULL) n_tok = t;
  for (int64_t i = 0; i < n_tok; ++i) {
    int64_t tt = tokens ? tokens[i] : i;
    if (tt < 0 || tt >= t) return -1;
    for (int32_t j = 0; j < topk; ++j)
      if (ids[tt * topk + j] < 0 || ids[tt * topk + j] >= experts) return -1;
  }
  double* d = (double*)calloc((size_t)(n_tok * topk * hidden), sizeof(double));
  uint16_t* wg = (uint16_t*)malloc((size_t)(inter * hidden) * 2);
  uint16_t* wu = (uint16_t*)malloc((size_t)(inter * hidden) * 2);
  uint16_t* wd = (uint16_t*)malloc((size_t)(hidden * inter) * 2);
  uint16_t* hbuf = (uint16_t*)malloc((size_t)inter * 2);
  if (!d || !wg || !wu || !wd || !hbuf) {
    free(d); free(wg); free(wu); free(wd); free(hbuf);
    return -2;
  }
  for (int32_t e = 0; e < experts; ++e) {
    int used = 0;
    for (int64_t i = 0; i < n_tok && !used; ++i) {
      int64_t tt = tokens ? tokens[i] : i;
      for (int32_t j = 0; j < topk; ++j) used |= ids[tt * topk + j] == e;
    }
    if (!used) continue;
    orc_dequantize(gate, e, 0, inter, wg);
    orc_dequantize(up, e, 0, inter, wu);
    orc_dequantize(down, e, 0, hidden, wd);
    for (int64_t i = 0; i < n_tok; ++i) {
      int64_t tt = tokens ? tokens[i] : i;
      for (int32_t j = 0; j < topk; ++j) {
        if (ids[tt * topk + j] != e) continue;
        const uint16_t* xt = x + tt * hidden;
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < inter; ++r) {
          double g = 0.0, u = 0.0;
          for (int64_t c = 0; c < hidden; ++c) {
            double xv = (double)bf16_to_f32(xt[c]);
            g += xv * (double)bf16_to_f32(wg[r * hidden + c]);
            u += xv * (double)bf16_to_f32(wu[r * hidden + c]);
          }
          hbuf[r] = f64_to_bf16(silu(g) * u);
        }
        double* dj = d + (i * topk + j) * hidden;
#pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < hidden; ++c) {
          double acc = 0.0;
          for (int64_t r = 0; r < inter; ++r)
            acc += (double)bf16_to_f32(hbuf[r]) * (double)bf16_to_f32(wd[c * inter + r]);
          dj[c] = acc;
        }
      }
    }
  }
  for (int64_t i = 0; i < n_tok; ++i) {
    int64_t tt = tokens ? tokens[i] : i;
    for (int64_t c = 0; c < hidden; ++c) {
      double acc = 0.0;
      for (int32_t j = 0; j < topk; ++j)
        acc += (double)weights[tt * topk + j] * d[(i * topk + j) * hidden + c];
      y[i * hidden + c] = f64_to_bf16(acc);
    }
  }
  free(d); free(wg); free(wu); free(wd); free(hbuf);
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Quantizers (offline side; they make the packed test weights).                               */
/* ------------------------------------------------------------------------------------------ */

/* INT4 round-to-nearest ([E6.4] "Do it in code", rtn; [CCQ] section 2.1 RTN with min-max
 * scale): per group of 64 along k (group = 64) or per row (group = 0),
 *   s = bf16(absmax / 7),  q = clip(round_half_even(w / s), -8, 7)  (fp32, stored s),
 * packed two per byte, low nibble first.  A group of zeros gets s = 0 and codes 0. */
ORC_API int32_t orc_quant_int4(const float* w, int64_t n, int64_t k, int32_t group,
                               uint8_t* codes, uint16_t* scales) {
  if (k % 64 || (group != 64 && group != 0)) return -1;
  int64_t gsz = group ? group : k;
  int64_t groups = k / gsz;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < groups; ++g) {
      const float* src = w + r * k + g * gsz;
      float amax = 0.0f;
      for (int64_t i = 0; i < gsz; ++i) amax = fmaxf(amax, fabsf(src[i]));
      uint16_t sb = f32_to_bf16(amax / 7.0f);
      scales[r * groups + g] = sb;
      float s = bf16_to_f32(sb);
      for (int64_t i = 0; i < gsz; ++i) {
        int32_t q = 0;
        if (s != 0.0f) {
          float v = nearbyintf(src[i] / s);
          if (v < -8.0f) v = -8.0f;
          if (v > 7.0f) v = 7.0f;
          q = (int32_t)v;
        }
        int64_t kk = g * gsz + i;
        uint8_t* b = codes + r * (k / 2) + (kk >> 1);
        if ((kk & 1) == 0)
          *b = (uint8_t)(q & 0xF);
        else
          *b = (uint8_t)(*b | ((q & 0xF) << 4));
      }
    }
  }
  return 0;
}

/* WINT8 round-to-nearest: s = bf16(absmax / 127) per group of 64 (or per row for group 0),
 * q = clip(round_half_even(w / s), -128, 127) (the [E6.4] affine quantizer with z = 0 at b = 8);
 * a zero group gets q = 0. */
ORC_API int32_t orc_quant_int8(const float* w, int64_t n, int64_t k, int32_t group,
                               int8_t* codes, uint16_t* scales) {
  if (k % 64 || (group != 64 && group != 0)) return -1;
  int64_t gsz = group ? group : k;
  int64_t groups = k / gsz;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < groups; ++g) {
      const float* src = w + r * k + g * gsz;
      float amax = 0.0f;
      for (int64_t i = 0; i < gsz; ++i) amax = fmaxf(amax, fabsf(src[i]));
      uint16_t sb = f32_to_bf16(amax / 127.0f);
      scales[r * groups + g] = sb;
      float s = bf16_to_f32(sb);
      for (int64_t i = 0; i < gsz; ++i) {
        int32_t q = 0;
        if (s != 0.0f) {
          float v = nearbyintf(src[i] / s);
          if (v < -128.0f) v = -128.0f;
          if (v > 127.0f) v = 127.0f;
          q = (int32_t)v;
        }
        codes[r * k + g * gsz + i] = (int8_t)q;
      }
    }
  }
  return 0;
}

/* 2-bit affine ("WINT2-Standard") with the [E6.4] affine formulas, per group of 64:
 *   s = bf16((max - min) / 3), z = clip(round(-min / s), 0, 3),
 *   q = clip(round(w / s) + z, 0, 3), four codes per byte, lowest bits first. */
ORC_API int32_t orc_quant_affine2(const float* w, int64_t n, int64_t k, uint8_t* codes,
                                  uint16_t* scales, uint8_t* zeros) {
  if (k % 64) return -1;
  int64_t groups = k / 64;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    memset(codes + r * (k / 4), 0, (size_t)(k / 4));
    for (int64_t g = 0; g < groups; ++g) {
      const float* src = w + r * k + g * 64;
      float mn = src[0], mx = src[0];
      for (int i = 1; i < 64; ++i) {
        mn = fminf(mn, src[i]);
        mx = fmaxf(mx, src[i]);
      }
      uint16_t sb = f32_to_bf16((mx - mn) / 3.0f);
      float s = bf16_to_f32(sb);
      int32_t z = 0;
      if (s != 0.0f) {
        float zf = nearbyintf(-mn / s);
        z = (int32_t)fminf(fmaxf(zf, 0.0f), 3.0f);
      }
      scales[r * groups + g] = sb;
      zeros[r * groups + g] = (uint8_t)z;
      for (int i = 0; i < 64; ++i) {
        int32_t q = 0;
        if (s != 0.0f) {
          float v = nearbyintf(src[i] / s) + (float)z;
          q = (int32_t)fminf(fmaxf(v, 0.0f), 3.0f);
        }
        int64_t kk = g * 64 + i;
        codes[r * (k / 4) + (kk >> 2)] |= (uint8_t)(q << (2 * (kk & 3)));
      }
    }
  }
  return 0;
}

/* [CCQ] Algorithm "Convolutional Code Quantization" for one vector of N = 4 weights with the
 * (6,4,3) configuration: the codebook row of code C is its four states (bit-shift decode),
 * scaled by the group scale after removing the zero point, and the stored code is the argmin
 * of the squared distance over all 2^15 codes.  Computed exactly by dynamic programming over
 * the trellis: the code's 15 bits are five 3-bit digits b4..b0 (b4 highest) and state j is
 * the digit pair (b_{4-j}, b_{3-j}), so the cost is a chain sum f0(b4,b3) + f1(b3,b2) +
 * f2(b2,b1) + f3(b1,b0).  The minimum is taken from the low end so that, among equal totals,
 * the smallest code wins.  Returns the code; *cost receives its squared error. */
ORC_API uint32_t orc_ccq_search(const double* v, double scale, int32_t zp, double* cost) {
  double f[4][64];
  for (int j = 0; j < 4; ++j)
    for (int u = 0; u < 64; ++u) {
      double r = v[j] - (double)(u - zp) * scale;
      f[j][u] = r * r;
    }
  /* best[j][a]: cheapest cost of states j..3 given that state j's high digit is a, with the
   * argmin low digit kept in arg[j][a] (smallest digit on ties). */
  double best[4][8];
  int arg[4][8];
  for (int a = 0; a < 8; ++a) {
    best[3][a] = INFINITY;
    for (int b = 0; b < 8; ++b) {
      double c = f[3][a * 8 + b];
      if (c < best[3][a]) { best[3][a] = c; arg[3][a] = b; }
    }
  }
  for (int j = 2; j >= 0; --j)
    for (int a = 0; a < 8; ++a) {
      best[j][a] = INFINITY;
      for (int b = 0; b < 8; ++b) {
        double c = f[j][a * 8 + b] + best[j + 1][b];
        if (c < best[j][a]) { best[j][a] = c; arg[j][a] = b; }
      }
    }
  int b4 = 0;
  for (int a = 1; a < 8; ++a)
    if (best[0][a] < best[0][b4]) b4 = a;
  int digits[5];
  digits[0] = b4;
  for (int j = 0; j < 4; ++j) digits[j + 1] = arg[j][digits[j]];
  uint32_t code = 0;
  for (int i = 0; i < 5; ++i) code = (code << 3) | (uint32_t)digits[i];
  if (cost) *cost = best[0][b4];
  return code;
}

/* Squared error of decoding `code` against v with the given scale, states summed in order. */
static double ccq_code_cost(uint32_t code, const double* v, double scale, int32_t zp) {
  double c = 0.0;
  for (int j = 0; j < 4; ++j) {
    int32_t u = (int32_t)((code >> (9 - 3 * j)) & 0x3Fu);
    double r = v[j] - (double)(u - zp) * scale;
    c += r * r;
  }
  return c;
}

/* Squared error of a group of 64 weights decoded from its 16 codes at scale s:
 * sum over i = 0..63, in order, of (w_i - (u_i - zp) * s)^2 with u_i the bit-shift state of
 * weight i ([CCQ] section 3.4, the quantization-error equation of a group). */
static double ccq_group_error(const float* wg, const uint32_t* codes, double s, int32_t zp) {
  double e = 0.0;
  for (int i = 0; i < 64; ++i) {
    int32_t u = (int32_t)((codes[i / 4] >> (9 - 3 * (i % 4))) & 0x3Fu);
    double r = (double)wg[i] - (double)(u - zp) * s;
    e += r * r;
  }
  return e;
}

/* One group of 64 weights of the (6,4,3) configuration:
 *   1. trellis search (orc_ccq_search) of its 16 vectors at the decode scale fl(sq * super);
 *   2. update != 0: [CCQ] section 3.4 "Scale Optimization".  With the searched codes fixed,
 *      the group error sum_i (W_i - W^q_i S)^2 (W^q_i = state - zp, the decoded value) is
 *      least at S* = sum_i W_i W^q_i / sum_i (W^q_i)^2 (the derivative set to zero, sums over
 *      i = 0..g-1 in order).  Readings: S* goes through the same 4-bit compression as the
 *      first scale (sq2 = clip(round(S* / super), 1, 15)); the group is searched again at
 *      fl(sq2 * super), and the new scale and codes are kept only when the group error
 *      (ccq_group_error) drops.  One update, no iteration; skipped when S* is not positive.
 * codes[16] receives the 15-bit codes, *sq_out the group's 4-bit scale; returns the group's
 * squared error. */
ORC_API double orc_ccq_encode_group(const float* wg, float super, uint32_t sq, int32_t zp,
                                    int32_t update, uint32_t* codes, uint32_t* sq_out) {
  double s = (double)((float)sq * super);
  for (int c = 0; c < 16; ++c) {
    double v[4];
    for (int j = 0; j < 4; ++j) v[j] = (double)wg[4 * c + j];
    codes[c] = orc_ccq_search(v, s, zp, NULL);
  }
  double err = ccq_group_error(wg, codes, s, zp);
  *sq_out = sq;
  if (!update) return err;
  double num = 0.0, den = 0.0;
  for (int i = 0; i < 64; ++i) {
    double q = (double)((int32_t)((codes[i / 4] >> (9 - 3 * (i % 4))) & 0x3Fu) - zp);
    num += (double)wg[i] * q;
    den += q * q;
  }
  if (!(den > 0.0 && num > 0.0)) return err;
  double sqd = nearbyint((num / den) / (double)super);
  if (sqd < 1) sqd = 1;
  if (sqd > 15) sqd = 15;
  uint32_t sq2 = (uint32_t)sqd;
  if (sq2 == sq) return err;
  double s2 = (double)((float)sq2 * super);
  uint32_t c2[16];
  for (int c = 0; c < 16; ++c) {
    double v[4];
    for (int j = 0; j < 4; ++j) v[j] = (double)wg[4 * c + j];
    c2[c] = orc_ccq_search(v, s2, zp, NULL);
  }
  double e2 = ccq_group_error(wg, c2, s2, zp);
  if (e2 < err) {
    memcpy(codes, c2, sizeof(c2));
    *sq_out = sq2;
    return e2;
  }
  return err;
}

/* CCQ (6,4,3) with code cluster, per output row (group 64 along k):
 *   1. group scale s_g = absmax_g / (2^(L-1) - 1) = absmax_g / 31            ([CCQ] Alg. 1)
 *   2. scale compression ([CCQ] section 3.4): super = max_g s_g / 15 per row,
 *      s_q = clip(round(s_g / super), 1, 15) (4 bits), decode scale s = s_q * super (fp32)
 *   3. trellis search of every 4-weight vector against the scaled codebook, group by group
 *      (orc_ccq_encode_group); with refine bit 1 (value 2) each group's scale is then
 *      optimized ([CCQ] section 3.4, "Scale Optimization")
 *   4. code cluster ([CCQ] section 3.3 Eq.): per row, beta = min C, alpha = (max C - min C)/255
 *      (alpha = 1 for a constant row), C' = clip(round((C - beta) / alpha), 0, 255)
 *   5. refine bit 0 (value 1) (reading: the cluster restricts the code space, so re-pick each
 *      C' as the best of the row's 256 decodable codes; decode parity does not depend on it).
 * zp is the weight zero point (reading: 2^(L-1) = 32).  full (optional, u16 [n][k/4])
 * receives the codes of step 3, before the cluster. */
ORC_API int32_t orc_quant_ccq(const float* w, int64_t n, int64_t k, int32_t zp, int32_t refine,
                              uint8_t* codes, uint8_t* qscale, float* super_scale,
                              float* code_scale, float* code_zero, uint16_t* full_out) {
  if (k % 64) return -1;
  int64_t groups = k / 64;
  int64_t qs_bytes = (groups + 1) / 2;
  int64_t vecs = k / 4;
  uint32_t* full = (uint32_t*)malloc((size_t)(n * vecs) * sizeof(uint32_t));
  float* sdec = (float*)malloc((size_t)(n * groups) * sizeof(float));
  if (!full || !sdec) {
    free(full); free(sdec);
    return -2;
  }
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < n; ++r) {
    const float* row = w + r * k;
    double smax = 0.0;
    for (int64_t g = 0; g < groups; ++g) {
      double amax = 0.0;
      for (int i = 0; i < 64; ++i) amax = fmax(amax, fabs((double)row[g * 64 + i]));
      smax = fmax(smax, amax / 31.0);
    }
    float sup = (float)(smax / 15.0);
    if (!(sup > 0.0f)) sup = 1.0f;
    super_scale[r] = sup;
    memset(qscale + r * qs_bytes, 0, (size_t)qs_bytes);
    uint32_t cmin = 0x7FFF, cmax = 0;
    for (int64_t g = 0; g < groups; ++g) {
      double amax = 0.0;
      for (int i = 0; i < 64; ++i) amax = fmax(amax, fabs((double)row[g * 64 + i]));
      double sqd = nearbyint((amax / 31.0) / (double)sup);
      if (sqd < 1) sqd = 1;
      if (sqd > 15) sqd = 15;
      uint32_t sq;
      uint32_t* gc = full + r * vecs + g * 16;
      orc_ccq_encode_group(row + g * 64, sup, (uint32_t)sqd, zp, refine & 2, gc, &sq);
      qscale[r * qs_bytes + (g >> 1)] |= (uint8_t)(sq << (4 * (g & 1)));
      sdec[r * groups + g] = (float)sq * sup;
      for (int c = 0; c < 16; ++c) {
        if (gc[c] < cmin) cmin = gc[c];
        if (gc[c] > cmax) cmax = gc[c];
      }
    }
    if (full_out)
      for (int64_t c = 0; c < vecs; ++c) full_out[r * vecs + c] = (uint16_t)full[r * vecs + c];
    float alpha = (cmax > cmin) ? (float)((double)(cmax - cmin) / 255.0) : 1.0f;
    float beta = (float)cmin;
    code_scale[r] = alpha;
    code_zero[r] = beta;
    for (int64_t c = 0; c < vecs; ++c) {
      double cp = nearbyint(((double)full[r * vecs + c] - (double)beta) / (double)alpha);
      if (cp < 0) cp = 0;
      if (cp > 255) cp = 255;
      uint32_t best = (uint32_t)cp;
      if (refine & 1) {
        double v[4];
        for (int j = 0; j < 4; ++j) v[j] = (double)row[c * 4 + j];
        double s = (double)sdec[r * groups + (c * 4) / 64];
        double bc = INFINITY;
        for (uint32_t cand = 0; cand < 256; ++cand) {
          double cc = ccq_code_cost(orc_ccq_expand(cand, alpha, beta), v, s, zp);
          if (cc < bc) { bc = cc; best = cand; }
        }
      }
      codes[r * vecs + c] = (uint8_t)best;
    }
  }
  free(full);
  free(sdec);
  return 0;
}

/* [CCQ] section 3.1 (Algorithm "Convolutional Code Quantization"), section 3.2 (hybrid
 * encoding) and section 3.4 (scale optimization, scale compression into redundant bits), for
 * the two configurations that need no code cluster, per output row with groups of 64 along k:
 *   fmt ORC_CCQ432:     (L,N,S) = (4,3,2): 22 u8 codes per group, 3 weights per code
 *                       (weights 3i .. 3i+2 in code i); the last code holds weight 63 in its
 *                       high state and the 4-bit quantized scale in its low 4 bits.
 *   fmt ORC_CCQ_HYBRID: (3,3,2) followed by (3,4,2) in one u16 word: 7 weights per word
 *                       (weights 7i .. 7i+6 in word i: three 3-bit states at bits 15..9, then
 *                       four at bits 8..0); the last word holds weight 63 in bits 15..13 and
 *                       the 13-bit quantized scale in bits 12..0.
 * Steps (readings stated where the pages leave a choice):
 *   1. group scale s_g = absmax_g / (2^(L-1) - 1) (7 for L = 4, 3 for L = 3); zp = 2^(L-1)
 *      is the caller's (8 or 4);
 *   2. scale compression: super = max_g s_g / s_mask per row (s_mask = 15 or 8191; a row of
 *      zeros gets super = 1), s_q = clip(round(s_g / super), 1, s_mask), s = fl(s_q * super);
 *   3. codebook search: every code of a configuration decodes by bit shifts to N states; the
 *      stored code is the argmin over all 2^T codes of sum_j (v_j - (state_j - zp) * s)^2,
 *      ties to the smallest code (exhaustive: at most 2^9 candidates);
 *   4. the last code of a group: its states past weight 63 are padding and its remaining
 *      bits carry s_q, so only weight 63's state is searched;
 *   5. refine != 0: one pass of the least-squares scale update S* = sum W Wq / sum Wq^2 over
 *      the group's decoded states Wq = state - zp (section 3.4), re-quantized as in step 2,
 *      re-searched, and kept only when the group's squared error drops.
 * codes: u8[n][k/64 * 22] or u8[n][k/64 * 20] (u16 little endian); super_scale f32[n]. */
static double alg2_search(int hyb, const double* v, int nv, double s, int32_t zp,
                          uint32_t* best_code) {
  /* nv = number of real weights in v (the code's remaining states are padding). */
  const int L = hyb ? 3 : 4;
  double total = 0.0;
  uint32_t word = 0;
  /* the parts of one stored word: (bits, states, shift of the lowest state) */
  int parts = hyb ? 2 : 1;
  int pos = 0;
  for (int p = 0; p < parts; ++p) {
    int N = hyb ? (p == 0 ? 3 : 4) : 3;
    int T = L + (N - 1) * 2;
    int base = hyb ? (p == 0 ? 9 : 0) : 0;
    uint32_t bc = 0;
    double bcost = INFINITY;
    for (uint32_t c = 0; c < (1u << T); ++c) {
      double cost = 0.0;
      for (int j = 0; j < N; ++j) {
        if (pos + j >= nv) break;
        int32_t u = (int32_t)((c >> (2 * (N - 1 - j))) & ((1u << L) - 1u));
        double r = v[pos + j] - (double)(u - zp) * s;
        cost += r * r;
      }
      if (cost < bcost) { bcost = cost; bc = c; }
    }
    word |= bc << base;
    total += bcost;
    pos += N;
  }
  *best_code = word;
  return total;
}

/* Encode one group (64 weights) with decode scale s; returns the squared error. */
static double alg2_encode_group(int hyb, const float* wg, double s, int32_t zp, uint32_t sq,
                                uint32_t* words) {
  const int per = hyb ? 7 : 3, P = hyb ? 10 : 22;
  double err = 0.0;
  for (int i = 0; i < P; ++i) {
    double v[7];
    int nv = 0;
    for (int j = 0; j < per; ++j)
      if (i * per + j < 64) v[nv++] = (double)wg[i * per + j];
    uint32_t code;
    if (i < P - 1) {
      err += alg2_search(hyb, v, nv, s, zp, &code);
    } else {
      /* weight 63 alone in the high state; the scale fills the low bits */
      const int L = hyb ? 3 : 4, top = hyb ? 13 : 4;
      double bcost = INFINITY;
      uint32_t bu = 0;
      for (uint32_t u = 0; u < (1u << L); ++u) {
        double r = v[0] - (double)((int32_t)u - zp) * s;
        if (r * r < bcost) { bcost = r * r; bu = u; }
      }
      err += bcost;
      code = (bu << top) | sq;
    }
    words[i] = code;
  }
  return err;
}

ORC_API int32_t orc_quant_alg2(const float* w, int64_t n, int64_t k, int32_t fmt, int32_t zp,
                               int32_t refine, uint8_t* codes, float* super_scale) {
  if (k % 64 || (fmt != ORC_CCQ432 && fmt != ORC_CCQ_HYBRID)) return -1;
  const int hyb = fmt == ORC_CCQ_HYBRID;
  const int64_t G = k / 64;
  const int P = hyb ? 10 : 22, bytes = hyb ? 20 : 22;
  const double lev = hyb ? 3.0 : 7.0;
  const uint32_t smask = hyb ? 0x1FFFu : 0xFu;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < n; ++r) {
    const float* row = w + r * k;
    double smax = 0.0;
    for (int64_t g = 0; g < G; ++g) {
      double amax = 0.0;
      for (int i = 0; i < 64; ++i) amax = fmax(amax, fabs((double)row[g * 64 + i]));
      smax = fmax(smax, amax / lev);
    }
    float sup = (float)(smax / (double)smask);
    if (!(sup > 0.0f)) sup = 1.0f;
    super_scale[r] = sup;
    for (int64_t g = 0; g < G; ++g) {
      const float* wg = row + g * 64;
      double amax = 0.0;
      for (int i = 0; i < 64; ++i) amax = fmax(amax, fabs((double)wg[i]));
      double sqd = nearbyint((amax / lev) / (double)sup);
      if (sqd < 1) sqd = 1;
      if (sqd > (double)smask) sqd = (double)smask;
      uint32_t sq = (uint32_t)sqd;
      uint32_t words[22];
      double err = alg2_encode_group(hyb, wg, (double)((float)sq * sup), zp, sq, words);
      if (refine) {
        /* least-squares scale for the chosen states (section 3.4, scale optimization) */
        const int per = hyb ? 7 : 3;
        static const int32_t sh432[3] = {4, 2, 0};
        static const int32_t shhyb[7] = {13, 11, 9, 6, 4, 2, 0};
        double num = 0.0, den = 0.0;
        for (int i = 0; i < 64; ++i) {
          uint32_t u = (words[i / per] >> (hyb ? shhyb[i % per] : sh432[i % per])) &
                       (hyb ? 0x7u : 0xFu);
          double q = (double)((int32_t)u - zp);
          num += (double)wg[i] * q;
          den += q * q;
        }
        if (den > 0.0 && num > 0.0) {
          double s2 = nearbyint((num / den) / (double)sup);
          if (s2 < 1) s2 = 1;
          if (s2 > (double)smask) s2 = (double)smask;
          uint32_t sq2 = (uint32_t)s2;
          if (sq2 != sq) {
            uint32_t w2[22];
            double e2 = alg2_encode_group(hyb, wg, (double)((float)sq2 * sup), zp, sq2, w2);
            if (e2 < err) {
              err = e2;
              memcpy(words, w2, sizeof(words));
            }
          }
        }
      }
      uint8_t* dst = codes + r * G * bytes + g * bytes;
      for (int i = 0; i < P; ++i) {
        if (hyb) {
          dst[2 * i] = (uint8_t)(words[i] & 0xFFu);
          dst[2 * i + 1] = (uint8_t)(words[i] >> 8);
        } else {
          dst[i] = (uint8_t)words[i];
        }
      }
    }
  }
  return 0;
}
