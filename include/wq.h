/*
 * wq.h -- C ABI of libwq.so: weight-only low-bit dequantize-and-multiply on AMD MI355X (gfx950).
 *
 * What the library computes (sources are the web pages the method is described on):
 *   - Weights are stored offline as packed low-bit codes and decoded in real time to BF16,
 *     the arithmetic being carried out on BF16 values with fp32 accumulation
 *     (FastDeploy "WINT2 Quantization", opening paragraph).
 *   - Formats:
 *       WQ_FMT_INT4         two signed 4-bit codes per byte, the first in the low nibble,
 *                           sign-extended (coursefy lesson E6.4 "GPTQ and AWQ", "Do it in
 *                           code"); x_hat = s * q with a bf16 scale per group of 64 along k,
 *                           or per output channel (group = 0).
 *       WQ_FMT_INT2_AFFINE  plain 2-bit codes, four per byte, lowest two bits first;
 *                           x_hat = s * (q - z) (lesson E6.4, "Math and notation") with a bf16
 *                           scale and a u8 zero point per group of 64.
 *       WQ_FMT_CCQ2         convolutional-code quantization (L,N,S) = (6,4,3) with code
 *                           cluster, one byte per 4 weights ("CCQ: Convolutional Code for
 *                           Extreme Low-bit Quantization in LLMs", section 3.3 and section 3.5,
 *                           algorithm "Dequantization with Code Cluster", table of dequantization
 *                           configurations).  Per weight:
 *                             C  = clamp(round_half_even(fmaf(C', code_scale, code_zero)), 0, 32767)
 *                             u  = (C >> (9 - 3*(k%4))) & 0x3F
 *                             s  = f32(s_q) * super_scale           (s_q: 4-bit group scale)
 *                             x_hat = bf16(f32(u - zp) * s)
 *       WQ_FMT_CCQ432       convolutional code (L,N,S) = (4,3,2) without code cluster, 2.75 bpw
 *       WQ_FMT_CCQ_HYBRID   hybrid convolutional code (3,3,2)+(3,4,2) in 16-bit words, 2.5 bpw
 *                           (CCQ paper, section 3.2 hybrid encoding, section 3.4 scale
 *                           compression, section 3.5 algorithm "Dequantization without Code
 *                           Cluster" and the table of dequantization configurations).  A group
 *                           of 64 weights is P code words W[0..P-1]; weight i of the group is
 *                             u  = (W[i / p] >> shift[i % p]) & w_mask
 *                             s  = f32(W[P-1] & s_mask) * super_scale
 *                             x_hat = bf16(f32(u - zp) * s)
 *                           (4,3,2): u8 words, P = 22, p = 3, shifts 4,2,0, w_mask 0xF,
 *                           s_mask 0xF.  Hybrid: u16 words, P = 10, p = 7, shifts
 *                           13,11,9,6,4,2,0, w_mask 0x7, s_mask 0x1FFF.  The last word carries
 *                           weight 63 in its top state and the group scale in its low bits.
 *       WQ_FMT_INT8         WINT8: one signed byte per weight (two's complement); x_hat = s * q
 *                           with a bf16 scale per group of 64 along k or per output channel
 *                           (group = 0) (FastDeploy "Quantization" precision list: INT8 weights,
 *                           BF16 activations; lesson E6.4 "Math and notation" at b = 8).
 *
 * Layouts (every matrix is W[n][k], k contiguous, y = x W^T; an MoE tensor adds a leading
 * expert dimension; group = 64 along k; G = k / 64):
 *   INT4:   codes u8[E][n][k/2]; scales bf16[E][n][G] (group 64) or bf16[E][n] (group 0).
 *   AFFINE: codes u8[E][n][k/4]; scales bf16[E][n][G]; zeros u8[E][n][G].
 *   CCQ2:   codes u8[E][n][k/4]; qscale u8[E][n][(G+1)/2], two 4-bit group scales per byte,
 *           the even group in the low nibble; super_scale, code_scale, code_zero f32[E][n];
 *           zp (32 for the symmetric 6-bit states).
 *   CCQ432: codes u8[E][n][G*22] (each group's 22 words consecutive, groups in k order);
 *           super_scale f32[E][n]; zp (8 for the 4-bit states).
 *   CCQ_HYBRID: codes u8[E][n][G*20] (each group's 10 u16 words, little endian);
 *           super_scale f32[E][n]; zp (4 for the 3-bit states).
 *   INT8:   codes i8[E][n][k]; scales bf16[E][n][G] (group 64) or bf16[E][n] (group 0).
 *
 * Conventions for every call below:
 *   - Every pointer inside wq_weight and every tensor argument of a compute call is DEVICE
 *     memory owned by the caller; the library never frees or retains it.  Only the
 *     wq_weight struct itself is read on the host, during the call.
 *   - Compute calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream)
 *     and never synchronize the host.  The library allocates no device memory in them.
 *   - Arguments are validated on the host before anything is launched; a negative status
 *     means nothing was launched and no output was touched.  wq_last_error() then gives a
 *     human-readable detail (thread-local).
 *   - Results are deterministic: no floating-point atomics; identical calls give identical
 *     bits.
 *   - Scales (bf16 scales, CCQ super/code scales) must be finite and the scales non-negative;
 *     wq_gemm / wq_moe_ffn need a CCQ zero point of 0 or a power of two (the kernels form
 *     (u - zp) * s as fma(u, s, -zp * s), the same single rounding when zp * s is exact) and
 *     2-bit affine zero points below 256.  The decoded weights the products use are the
 *     same bits wq_dequantize returns, except that a weight the definition makes -0 (a zero
 *     group scale times a negative state offset) enters the products as +0, which no sum
 *     starting from +0 can tell apart.
 *   - The products (wq_gemm, wq_moe_gate_up, wq_moe_down, wq_moe_ffn) also require every scale
 *     to be below 2^100 in magnitude: they rescale it by up to 2^24 on its way into the decode
 *     (wq_dequantize has no such limit).  Real weights sit many orders of magnitude below it.
 *   - Sizes are element counts (int64).  Device pointers must be 16-byte aligned.  The products
 *     address one expert's arrays and one activation row with 32-bit byte offsets: they return
 *     WQ_ERR_UNSUPPORTED for k >= 2^30 or when one expert's codes exceed 2^31 - 24 bytes.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WQ_OK = 0,
  WQ_ERR_ARG = -1,         /* null pointer, bad size or shape                         */
  WQ_ERR_UNSUPPORTED = -2, /* format / group / size combination not supported          */
  WQ_ERR_ALIGN = -3,       /* a device pointer is not 16-byte aligned                  */
  WQ_ERR_RANGE = -4,       /* an INT4 code outside -8..7 (wq_pack_int4)                 */
  WQ_ERR_WORKSPACE = -5,   /* workspace smaller than wq_moe_workspace_bytes()           */
  WQ_ERR_HIP = -6          /* the HIP runtime reported an error at launch               */
} wq_status;

typedef enum {
  WQ_FMT_INT4 = 1,
  WQ_FMT_INT2_AFFINE = 2,
  WQ_FMT_CCQ2 = 3,
  WQ_FMT_CCQ432 = 4,
  WQ_FMT_CCQ_HYBRID = 5,
  WQ_FMT_INT8 = 6
} wq_format;

/* A packed weight tensor [experts][n][k] in device memory (see layouts above). */
typedef struct {
  int32_t format;            /* wq_format                                                  */
  int32_t group;             /* 64, or 0 = per output channel (INT4 and INT8)              */
  int64_t experts;           /* 1 for a dense matrix                                       */
  int64_t n;                 /* output channels per expert                                 */
  int64_t k;                 /* input channels; a multiple of 64                           */
  const uint8_t* codes;
  const uint16_t* scales;    /* bf16 bits; INT4, INT8 and AFFINE                           */
  const uint8_t* zeros;      /* AFFINE                                                     */
  const uint8_t* qscale;     /* CCQ2                                                       */
  const float* super_scale;  /* CCQ2, CCQ432, CCQ_HYBRID                                   */
  const float* code_scale;   /* CCQ2                                                       */
  const float* code_zero;    /* CCQ2                                                       */
  int32_t zp;                /* CCQ weight zero point (all three CCQ formats)              */
} wq_weight;

/* Decode every weight to bf16, out[e][n][k] (device, bf16 bits).  Bit-exact with the
 * formulas above (CCQ paper section 3.5; lesson E6.4 "Math and notation"). */
wq_status wq_dequantize(const wq_weight* w, uint16_t* out, void* stream);

/* Dense weight-only product y[m][n] = bf16(sum_k x[m][k] * x_hat[n][k]) with bf16 operands
 * and fp32 accumulation (FastDeploy "WINT2 Quantization"; the pages' GEMV and grouped-GEMM
 * operator benchmarks).  x bf16 [m][k], y bf16 [m][n], w->experts must be 1.  m == 0 is a
 * no-op.  Small m (<= 32) runs the decode kernels that stream the packed weights once;
 * larger m runs the MFMA kernel with LDS-staged dequantized tiles, except group-64 INT8,
 * which runs the decode kernels at every m (in launches of at most 65535 x 32 rows). */
wq_status wq_gemm(const uint16_t* x, int64_t m, const wq_weight* w, uint16_t* y, void* stream);

/* ---- Mixture-of-experts expert FFN --------------------------------------------------------
 * The pages' deployment is an MoE model whose expert weights are the low-bit ones (FastDeploy
 * "WINT2 Quantization": supported architecture MoE; the w4w2 layer map quantizes the experts),
 * and their grouped-GEMM benchmark routes each token to 8 of 256 experts through a grouped
 * weight-only product of the tokens gathered per expert (CCQ paper, section 5 "Inference
 * Performance", the grouped-GEMM operator table).  The calls below are that path: routing
 * groups the (token, slot) pairs by expert, the grouped gate+up product with SiLU(gate) * up,
 * the grouped down product, and the routing-weighted sum back per token. */

/* Bytes of device workspace wq_moe_ffn needs for t tokens, top-k routing over `experts`
 * experts, hidden size `hidden` and expert intermediate size `inter` (expert offsets, the
 * sorted pair list, h and d of the stages below, and above 4096 pairs the routing table of
 * wq_moe_route_workspace_bytes).  0 for invalid sizes. */
size_t wq_moe_workspace_bytes(int64_t t, int32_t topk, int32_t experts, int64_t hidden,
                              int64_t inter);

/* Bytes of device workspace that lets wq_moe_route sort t*topk pairs in chunks, one
 * workgroup per chunk (a per-chunk table of counts per expert); 0 when the sort takes no
 * workspace (at most 4096 pairs) or for invalid sizes. */
size_t wq_moe_route_workspace_bytes(int64_t t, int32_t topk, int32_t experts);

/* Group the (token, slot) pairs p = t*topk + j by expert (sort by expert id, stable in p):
 * expert_offsets[e] = number of pairs routed to experts < e (expert_offsets[experts] =
 * t*topk); sorted_pairs[expert_offsets[e] ...] lists expert e's pairs in increasing p.
 * topk_ids int32 [t][topk] must lie in [0, experts); the device drops a pair whose id lies
 * outside (it lands in no expert's list and nothing is written out of bounds), and the
 * outputs of its token are then unspecified.  ws: NULL (ws_bytes 0) sorts in one workgroup;
 * device memory of at least wq_moe_route_workspace_bytes bytes (caller-owned, nothing in it
 * needs to be initialized) lets a long array be sorted in chunks over many workgroups, with the
 * same result.  A non-NULL ws smaller than that returns WQ_ERR_WORKSPACE, a NULL ws with a
 * non-zero size WQ_ERR_ARG.  At most 512 experts and 2^30 pairs. */
wq_status wq_moe_route(const int32_t* topk_ids, int64_t t, int32_t topk, int32_t experts,
                       int32_t* expert_offsets, int32_t* sorted_pairs, void* ws,
                       size_t ws_bytes, void* stream);

/* MoE expert FFN with routed tokens grouped per expert:
 *   y[t] = bf16( sum_{j<topk} topk_weights[t][j] * W_down[e] h_{t,j} ),  e = topk_ids[t][j],
 *   h_{t,j} = bf16( SiLU(W_gate[e] x_t) * (W_up[e] x_t) )
 * x bf16 [t][hidden], y bf16 [t][hidden]; gate and up are [E][inter][hidden], down is
 * [E][hidden][inter]; the slot sum runs in order j = 0..topk-1 in fp32.  Routing weights are
 * used as given.  ws must hold wq_moe_workspace_bytes(t, topk, E, hidden, inter) bytes (device
 * memory, caller-owned, nothing in it needs to be initialized).  The expert products are the
 * weight-only grouped GEMMs of the CCQ paper's section 5 (BF16 activations against the
 * experts' decoded low-bit weights); SiLU(gate) * up between them is the expert FFN of the
 * deployed MoE models, with h rounded to bf16 because every product takes BF16 operands
 * (FastDeploy "WINT2 Quantization": BF16 arithmetic). */
wq_status wq_moe_ffn(const uint16_t* x, int64_t t, int64_t hidden, const int32_t* topk_ids,
                     const float* topk_weights, int32_t topk, const wq_weight* gate,
                     const wq_weight* up, const wq_weight* down, uint16_t* y, void* ws,
                     size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: wq_moe_ffn with its workspace taken from a
 * library-owned device array of WQ_NOALLOC_SCRATCH_BYTES (32 MiB), which every GPU the library
 * runs on holds from the first call on it until the process ends.  The caller still passes x,
 * the routing arrays, the weights and y.  The call itself allocates nothing (no hipMalloc, no
 * library allocation).  A call whose workspace (wq_moe_workspace_bytes) exceeds the array
 * returns WQ_ERR_WORKSPACE without launching: at hidden 8192 and inter 3584 that is above 840
 * (token, slot) pairs, 105 tokens at top-8.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two host threads) race, and must be ordered by
 * the caller.  Arguments and results are otherwise those of wq_moe_ffn. */
#define WQ_NOALLOC_SCRATCH_BYTES (32u << 20)
wq_status wq_moe_ffn_noalloc(const uint16_t* x, int64_t t, int64_t hidden,
                             const int32_t* topk_ids, const float* topk_weights, int32_t topk,
                             const wq_weight* gate, const wq_weight* up, const wq_weight* down,
                             uint16_t* y, void* stream);

/* The stages of wq_moe_ffn, for callers that route elsewhere or time the stages separately
 * (wq_moe_ffn = wq_moe_route + wq_moe_gate_up + wq_moe_down + wq_moe_combine).  The routing
 * arrays are those wq_moe_route produces; npairs = t * topk.  wq_moe_gate_up and wq_moe_down
 * are the two grouped products of the CCQ paper's grouped-GEMM table (section 5; its shapes
 * "groups x output x input" 256 x 1024 x 7168 are gate+up, two 512-row matrices against a
 * 7168-wide token, and 256 x 7168 x 512 the down product).
 * wq_moe_gate_up: h[r] = bf16(SiLU(W_gate[e] x_tok) * (W_up[e] x_tok)) for every sorted
 *   position r (expert e, pair p = sorted_pairs[r], token p / topk); h bf16 [npairs][inter].
 * wq_moe_down: d[p] = W_down[e] h[r] in fp32 for every sorted position r, stored by pair id
 *   p = sorted_pairs[r]; d f32 [npairs][hidden].
 * wq_moe_combine: y[t] = bf16(sum_j topk_weights[t][j] * d[t*topk + j]) (fp32, j in order). */
wq_status wq_moe_gate_up(const uint16_t* x, int64_t t, const int32_t* expert_offsets,
                         const int32_t* sorted_pairs, int32_t topk, const wq_weight* gate,
                         const wq_weight* up, uint16_t* h, void* stream);
wq_status wq_moe_down(const uint16_t* h, int64_t t, int32_t topk, const int32_t* expert_offsets,
                      const int32_t* sorted_pairs, const wq_weight* down, float* d, void* stream);
wq_status wq_moe_combine(const float* d, const float* topk_weights, int64_t t, int32_t topk,
                         int64_t hidden, uint16_t* y, void* stream);

/* CCQ (6,4,3) code-cluster encoder (CCQ paper, algorithm "Convolutional Code Quantization" of
 * section 3.1, section 3.3 Eq. 1, section 3.4 scale optimization (Eq. 2-4) and scale
 * compression): fp32 weights w[n][k] (device, row-major; an MoE tensor is n = experts x rows)
 * -> the WQ_FMT_CCQ2 arrays of the layout above (codes u8[n][k/4], qscale u8[n][(k/64+1)/2],
 * super_scale, code_scale, code_zero f32[n], all device memory owned by the caller).  Per row,
 * groups of 64:
 *   s_g = absmax_g / 31; super = f32(max_g s_g / 15) (1 for a zero row);
 *   s_q = clip(round(s_g / super), 1, 15); s = f32(s_q) * super;
 *   C = the 15-bit code minimizing sum_j (v_j - (u_j - zp) s)^2 over the vector's 4 weights
 *       (u_j: states at shifts 9, 6, 3, 0; ties to the smallest code);
 *   refine bit 1 (value 2), scale optimization: with a group's codes fixed, S* = sum_i w_i q_i /
 *       sum_i q_i^2 (q_i = u_i - zp over the group's 64 weights in order); when S* > 0 and
 *       s_q2 = clip(round(S* / super), 1, 15) differs from s_q, the group is searched again at
 *       f32(s_q2) * super and takes s_q2 and the new codes if its error sum_i (w_i - q_i s)^2
 *       drops;
 *   beta = min C, alpha = f32((max C - min C) / 255) (1 if all codes are equal);
 *   C' = clip(round((C - beta) / alpha), 0, 255), or, with refine bit 0 (value 1), the C' in
 *       0..255 whose decoded code (round(fmaf(C', alpha, beta)) clamped to [0, 2^15 - 1]) costs
 *       least (ties to the smallest C').
 * Costs, ratios and roundings to integers are taken in fp64 (round half to even), so the
 * outputs are a function of w alone.  Requires k % 64 == 0, k <= 131072 (one workgroup keeps
 * a row's codes in LDS), zp in 0..127, refine in 0..3, w 16-byte aligned.  Asynchronous on
 * `stream`, no allocation. */
wq_status wq_quantize_ccq(const float* w, int64_t n, int64_t k, int32_t zp, int32_t refine,
                          uint8_t* codes, uint8_t* qscale, float* super_scale, float* code_scale,
                          float* code_zero, void* stream);

/* Host helpers for the INT4 storage format (lesson E6.4, "Do it in code"); host memory.
 * wq_pack_int4: two codes per byte, the first in the low nibble, an odd count padded with 0;
 *   out must hold (n+1)/2 bytes; WQ_ERR_RANGE (nothing written) for a code outside -8..7.
 * wq_unpack_int4: the first n codes, sign-extended; data holds at least (n+1)/2 bytes.
 * wq_packed_size: nominal bytes of n_codes codes of `bits` bits (n*bits/8, rounded up);
 *   -1 for negative n, bits outside 1..32, or a bit count n*bits beyond int64. */
wq_status wq_pack_int4(const int32_t* codes, int64_t n, uint8_t* out);
wq_status wq_unpack_int4(const uint8_t* data, int64_t n, int32_t* out);
int64_t wq_packed_size(int64_t n_codes, int32_t bits);

/* Name of a status code, and the detail of the calling thread's last failure (the text stays
 * valid until that thread's next failing call; wq_last_error_detail is the same call under a
 * second name). */
const char* wq_status_string(int32_t status);
const char* wq_last_error(void);
const char* wq_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
