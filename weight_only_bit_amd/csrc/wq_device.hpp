// wq_device.hpp -- device-side building blocks for gfx950: bf16 rounding, the packed-code
// decode unit, and the MFMA operand types.
//
// Every decode path produces the weight value x_hat rounded to bf16 exactly as the format
// defines it (the pages decode the weights to BF16 before the BF16 arithmetic); the MFMA
// kernels and the dequantize kernel give identical bits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

enum { FMT_INT4 = 1, FMT_AFFINE2 = 2, FMT_CCQ2 = 3, FMT_CCQ432 = 4, FMT_CCQH = 5, FMT_INT8 = 6 };

// The CCQ formats without code cluster: the group scale rides in the last code word.
__host__ __device__ constexpr bool is_alg2(int f) { return f == FMT_CCQ432 || f == FMT_CCQH; }
// Code bytes of one 64-weight group: 22 u8 words ((4,3,2)) or 10 u16 words (hybrid).
__host__ __device__ constexpr int alg2_group_bytes(int f) { return f == FMT_CCQ432 ? 22 : 20; }

// Device view of a packed weight [experts][n][k] (pointers already offset to expert 0).
struct DevWeight {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint8_t* zeros;
  const uint8_t* qscale;
  const float* super_scale;
  const float* code_scale;
  const float* code_zero;
  int64_t n, k;
  int32_t group;  // 64 or 0 (per channel)
  int32_t zp;
};

// ---------------------------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two fp32 values -> packed bf16 pair, low half first (v_cvt_pk_bf16_f32: round half to even;
// a NaN keeps its sign and payload bits).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// fp32 -> bf16 bits, round half to even; NaN -> 0x7FC0.  On any other input the conversion
// instruction gives (u + 0x7FFF + ((u >> 16) & 1)) >> 16 of the bit pattern u; a NaN is
// replaced by the canonical one.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t b = cvt_pk_bf16(f, f) & 0xFFFFu;
  return f != f ? 0x7FC0u : b;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  uint32_t p = cvt_pk_bf16(lo, hi);
  if (lo != lo) p = (p & 0xFFFF0000u) | 0x7FC0u;
  if (hi != hi) p = (p & 0x0000FFFFu) | 0x7FC00000u;
  return p;
}

// ---------------------------------------------------------------------------------------------
// CCQ (6,4,3) code cluster, stage 1 ("CCQ", section 3.5: the first of the two dequantization
// operations widens the stored byte to the 15-bit convolutional code):
//   C = clamp(round_half_even(fmaf(C', code_scale, code_zero)), 0, 2^15 - 1)
// The clamp is applied before rounding (equivalent: the bounds are integers).  Adding
// 1.5 * 2^23 to a value in [0, 2^15) rounds it half-to-even to an integer that lands in the
// low mantissa bits, so the returned float's bit pattern is 0x4B400000 + C: bits 0..14 are C.
// ---------------------------------------------------------------------------------------------
template <bool CLAMP = true>
__device__ __forceinline__ uint32_t ccq_expand_bits(float cprime, float cscale, float czero) {
  float t = __builtin_fmaf(cprime, cscale, czero);
  if (CLAMP) t = __builtin_amdgcn_fmed3f(t, 0.0f, 32767.0f);
  return __float_as_uint(t + 12582912.0f);
}

// True when no byte of a row can expand outside [0, 32767] (so the clamp is the identity):
// fmaf is monotonic in C', so checking C' = 0 and C' = 255 covers the row.
__device__ __forceinline__ bool ccq_row_needs_no_clamp(float cscale, float czero) {
  const float a = __builtin_fmaf(0.0f, cscale, czero), b = __builtin_fmaf(255.0f, cscale, czero);
  return fminf(a, b) >= 0.0f && fmaxf(a, b) <= 32767.0f;
}

// ---------------------------------------------------------------------------------------------
// Fast exact decode for the MFMA kernels.  Each helper turns the packed bytes one lane holds
// (16 consecutive weights of one row) into 8 dwords of bf16 pairs in k order, equal bit for
// bit to the format's x_hat:
//   value = bf16(fl((c - z) * s))
//
// The arithmetic runs on v_fma_mix_f32, which reads one operand as the low or high f16 half
// of a dword, widens it exactly and fuses it into an fp32 FMA.  A code field c (< 1024) that
// sits alone in a 16-bit half is, read as f16, the subnormal c * 2^-24; with the scale
// pre-multiplied by 2^24 (exact) the mixed FMA forms the exact product c * s and rounds
//   c * s - z * s
// once -- the single rounding of the exact (c - z) * s whenever z * s is exact in fp32 (z a
// power of two -- the CCQ zero point 32 -- or z * s with few enough bits: the 2-bit affine
// zero point times a bf16 scale, INT4's 8 * s).  So one instruction converts and scales a
// weight, and 16-bit packed shifts place two codes per dword.  A field that lies wholly in
// bits 0..9 of its half need not be shifted down: masked in place at bit p it reads as the
// subnormal c * 2^(p - 24), and the scale passed with it is s * 2^(24 - p) (an exact power-of-two
// rescaling), so the product is again exactly c * s.  Only fields reaching into the f16
// exponent bits (10..14) or the sign bit are shifted.  For c == z the result is +0
// where the two-step form gives 0 * s: the same bits for s >= 0 (scales are non-negative).
// For s == 0 (a zero group-scale field) and c < z the two-step form gives -0 and this one +0;
// no product can tell them apart (every accumulation starts at +0).
// Requires f16 subnormals to be kept (the default float mode) and |s| < 2^100.
// ---------------------------------------------------------------------------------------------

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr float kTwo24 = 16777216.0f;

// Both 16-bit halves of x shifted right by sh (v_pk_lshrrev_b16).
__device__ __forceinline__ uint32_t pk_shr16(uint32_t x, uint16_t sh) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, x) >> (u16x2){sh, sh});
}

// fl(h * a + b) with h the low / high f16 half of x (v_fma_mix_f32 op_sel).
__device__ __forceinline__ float mix_lo(uint32_t x, float a, float b) {
  return __builtin_fmaf((float)__builtin_bit_cast(f16x2_t, x).x, a, b);
}
__device__ __forceinline__ float mix_hi(uint32_t x, float a, float b) {
  return __builtin_fmaf((float)__builtin_bit_cast(f16x2_t, x).y, a, b);
}

// CCQ: one dword = 4 clustered bytes = 16 weights.  cs24 = code_scale * 2^24, s24 = s * 2^24
// with s = f32(s_q) * super, mzs = -zp * s.  Stage 1 uses the same mixed FMA: the byte C'
// read as a subnormal times cs24 is the exact C' * code_scale, so t = fmaf(C', code_scale,
// code_zero) bit for bit.  CLAMP = false only when ccq_row_needs_no_clamp holds for the row.
template <bool CLAMP = true>
__device__ __forceinline__ void ccq_decode16(uint32_t w, float cs24, float cz, float s24,
                                             float mzs, uint32_t (&p)[8]) {
  const uint32_t ev = w & 0x00FF00FFu;  // bytes 0, 2
  const uint32_t od = pk_shr16(w, 8);    // bytes 1, 3 (one packed shift, nothing above them)
  float t[4] = {mix_lo(ev, cs24, cz), mix_lo(od, cs24, cz), mix_hi(ev, cs24, cz),
                mix_hi(od, cs24, cz)};
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (CLAMP) t[b] = __builtin_amdgcn_fmed3f(t[b], 0.0f, 32767.0f);
  const float s21 = s24 * 0.125f;
  float r[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // P = C of byte 2h (low half) | C of byte 2h + 1 (high half): the magic-number add of
    // ccq_expand_bits leaves C in bits 0..14, and the second add writes only its low 16 bits
    // into the high half of the first result (SDWA destination select, other half kept).
    uint32_t P = __float_as_uint(t[2 * h] + 12582912.0f);
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD"
        : "+v"(P)
        : "v"(t[2 * h + 1]), "v"(12582912.0f));
    // bit-shift decode: 6-bit states at shifts 9, 6, 3, 0 of each half; the state at shift 3
    // (bits 3..8) is read in place with the scale s * 2^21
    const uint32_t q0 = pk_shr16(P, 9);  // C < 2^15: no bits above the field
    const uint32_t q1 = pk_shr16(P, 6) & 0x003F003Fu;
    const uint32_t q2 = P & 0x01F801F8u;
    const uint32_t q3 = P & 0x003F003Fu;
    r[8 * h + 0] = mix_lo(q0, s24, mzs);
    r[8 * h + 1] = mix_lo(q1, s24, mzs);
    r[8 * h + 2] = mix_lo(q2, s21, mzs);
    r[8 * h + 3] = mix_lo(q3, s24, mzs);
    r[8 * h + 4] = mix_hi(q0, s24, mzs);
    r[8 * h + 5] = mix_hi(q1, s24, mzs);
    r[8 * h + 6] = mix_hi(q2, s21, mzs);
    r[8 * h + 7] = mix_hi(q3, s24, mzs);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = cvt_pk_bf16(r[2 * i], r[2 * i + 1]);
}

// INT4: two dwords = 16 signed nibbles (first weight in the low nibble).  XOR 8 biases a
// two's-complement nibble q to q + 8 in 0..15, so value = fl((q + 8) * s - 8 s);
// s24 = s * 2^24, m8s = -8 s.  The second nibble of each half (bits 4..7) is read in place
// with the scale s * 2^20.
__device__ __forceinline__ void int4_decode16(uint32_t w0, uint32_t w1, float s24, float m8s,
                                              uint32_t (&p)[8]) {
  const float sc[4] = {s24, s24 * 0.0625f, s24, s24};
  float r[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t d = (h ? w1 : w0) ^ 0x88888888u;  // halves: nibbles 0..3 and 4..7
    const uint32_t q[4] = {d & 0x000F000Fu, d & 0x00F000F0u, pk_shr16(d, 8) & 0x000F000Fu,
                           pk_shr16(d, 12)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[8 * h + i] = mix_lo(q[i], sc[i], m8s);
      r[8 * h + 4 + i] = mix_hi(q[i], sc[i], m8s);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = cvt_pk_bf16(r[2 * i], r[2 * i + 1]);
}

// INT8: 16 signed bytes (k order).  XOR 0x80 biases a byte q to q + 128 in 0..255 (< 1024, so
// an f16 subnormal), value = fl((q + 128) s - 128 s); s24 = s * 2^24, m128s = -128 s.
__device__ __forceinline__ void int8_decode16(const u32x4& w, float s24, float m128s,
                                              uint32_t (&p)[8]) {
  float r[16];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = w[d] ^ 0x80808080u;
    const uint32_t ev = x & 0x00FF00FFu;  // bytes 0, 2
    const uint32_t od = pk_shr16(x, 8);   // bytes 1, 3
    r[4 * d + 0] = mix_lo(ev, s24, m128s);
    r[4 * d + 1] = mix_lo(od, s24, m128s);
    r[4 * d + 2] = mix_hi(ev, s24, m128s);
    r[4 * d + 3] = mix_hi(od, s24, m128s);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = cvt_pk_bf16(r[2 * i], r[2 * i + 1]);
}

// 2-bit affine: one dword = 16 codes (first in the lowest two bits); value = fl(q s - z s)
// with z s exact (8-bit z times a bf16 scale); s24 = s * 2^24, mzs = -z s.  Codes 0..4 of each
// half (bits 0..9) are read in place at bit 2i with the scale s * 2^(24 - 2i); codes 5..7 are
// read at bits 4, 6, 8 of the half shifted right by 6.
__device__ __forceinline__ void affine2_decode16(uint32_t w, float s24, float mzs,
                                                 uint32_t (&p)[8]) {
  const float sc[5] = {s24, s24 * 0.25f, s24 * 0.0625f, s24 * 0.015625f, s24 * 0.00390625f};
  const uint32_t t = pk_shr16(w, 6);
  // q[i]: codes i (low half) and 8 + i (high half)
  const uint32_t q[8] = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u,
                         w & 0x03000300u, t & 0x00300030u, t & 0x00C000C0u, t & 0x03000300u};
  const int si[8] = {0, 1, 2, 3, 4, 2, 3, 4};
  float r[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r[i] = mix_lo(q[i], sc[si[i]], mzs);
    r[8 + i] = mix_hi(q[i], sc[si[i]], mzs);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = cvt_pk_bf16(r[2 * j], r[2 * j + 1]);
}

// CCQ without code cluster ("CCQ", section 3.5, "Dequantization without Code Cluster"): one
// 64-weight group -> 32 dwords of bf16 pairs in k order.  The group's code bytes start at byte
// 0 of c[0] (little endian); fin24 = super * 2^24, mzp24 = -zp / 2^24 (zp a power of two or 0,
// so -zp * s is exact).  s = fl(s_q * super) is formed as fl(s_q * fin24) = s * 2^24 exactly.
//
// (4,3,2): byte b (< 21) holds weights 3b, 3b+1, 3b+2 as its states at shifts 4, 2, 0; byte 21
// holds weight 63 in its high nibble and s_q in its low nibble.  Each 16-bit half of a dword
// holds bytes 4d, 4d+1 (low) and 4d+2, 4d+3 (high): the even byte's states are read in place
// (bits 4, 2, 0 of the half), the odd byte's at bits 6, 4, 2 of the half shifted right by 6.
__device__ __forceinline__ void ccq432_decode64(const uint32_t (&c)[6], float fin24, float mzp24,
                                                uint32_t (&p)[32]) {
  const float s24 = (float)((c[5] >> 8) & 0xFu) * fin24;
  const float mzs = s24 * mzp24;
  const float s22 = s24 * 0.25f, s20 = s24 * 0.0625f, s18 = s24 * 0.015625f;
  float v[66];
#pragma unroll
  for (int d = 0; d < 6; ++d) {
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) {
      const uint32_t x = odd ? pk_shr16(c[d], 6) : c[d];  // the byte at bit 2 odd, 0 even
      const int b = 4 * d + odd;  // byte in the low half; b + 2 in the high half
      const uint32_t q0 = x & (odd ? 0x03C003C0u : 0x00F000F0u);
      const uint32_t q1 = x & (odd ? 0x00F000F0u : 0x003C003Cu);
      const uint32_t q2 = x & (odd ? 0x003C003Cu : 0x000F000Fu);
      const float a0 = odd ? s18 : s20, a1 = odd ? s20 : s22, a2 = odd ? s22 : s24;
      if (3 * b < 64) v[3 * b] = mix_lo(q0, a0, mzs);
      if (3 * b + 1 < 64) v[3 * b + 1] = mix_lo(q1, a1, mzs);
      if (3 * b + 2 < 64) v[3 * b + 2] = mix_lo(q2, a2, mzs);
      if (3 * b + 6 < 64) v[3 * b + 6] = mix_hi(q0, a0, mzs);
      if (3 * b + 7 < 64) v[3 * b + 7] = mix_hi(q1, a1, mzs);
      if (3 * b + 8 < 64) v[3 * b + 8] = mix_hi(q2, a2, mzs);
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) p[i] = cvt_pk_bf16(v[2 * i], v[2 * i + 1]);
}

// Hybrid (3,3,2)+(3,4,2): u16 word j (< 9) holds weights 7j .. 7j+6 as its states at shifts
// 13, 11, 9, 6, 4, 2, 0; word 9 holds weight 63 at shift 13 and s_q in bits 0..12.  Dword d
// holds words 2d (low half) and 2d+1 (high half).  The states at shifts 6, 4, 2, 0 are read in
// place; those at 13, 11, 9 at bits 6, 4, 2 of the halves shifted right by 7.
__device__ __forceinline__ void ccqh_decode64(const uint32_t (&c)[5], float fin24, float mzp24,
                                              uint32_t (&p)[32]) {
  const float s24 = (float)((c[4] >> 16) & 0x1FFFu) * fin24;
  const float mzs = s24 * mzp24;
  // field position in the (shifted) half and the matching scale s * 2^(24 - position)
  constexpr uint32_t mask[7] = {0x01C001C0u, 0x00700070u, 0x001C001Cu, 0x01C001C0u,
                                0x00700070u, 0x001C001Cu, 0x00070007u};
  const float sc[4] = {s24, s24 * 0.25f, s24 * 0.0625f, s24 * 0.015625f};
  constexpr int si[7] = {3, 2, 1, 3, 2, 1, 0};
  float v[70];
#pragma unroll
  for (int d = 0; d < 5; ++d) {
    const uint32_t t = pk_shr16(c[d], 7);
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const uint32_t q = (j < 3 ? t : c[d]) & mask[j];
      const int w = 14 * d + j;
      if (w < 64) v[w] = mix_lo(q, sc[si[j]], mzs);
      if (w + 7 < 64) v[w + 7] = mix_hi(q, sc[si[j]], mzs);
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) p[i] = cvt_pk_bf16(v[2 * i], v[2 * i + 1]);
}

// ---------------------------------------------------------------------------------------------
// Reference-form exact decode of one weight (dequantize kernel): the two-step form of the
// format definitions, rounded with the same bf16 conversion.
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float int4_value(uint32_t nib, float s) {
  const int32_t q = (int32_t)(nib ^ 8u) - 8;  // sign-extend the 4-bit field
  return (float)q * s;
}

__device__ __forceinline__ float affine2_value(uint32_t q, uint32_t z, float s) {
  return (float)((int32_t)q - (int32_t)z) * s;
}

// u: 6-bit state, s = f32(s_q) * super (already rounded to fp32).
__device__ __forceinline__ float ccq_value(uint32_t u, int32_t zp, float s) {
  return (float)((int32_t)u - zp) * s;
}

// ---------------------------------------------------------------------------------------------
// MFMA
// ---------------------------------------------------------------------------------------------

// D[16x16] += A[16x32] * B[32x16], bf16 operands, fp32 accumulate.  Lane l supplies row l%16
// of A and column l%16 of B, each over k-slots 8*(l/16) .. 8*(l/16)+7; it receives
// D[4*(l/16) + r][l%16] for r = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D[32x32] += A[32x16] * B[16x32]: lane l supplies row l%32 of A / column l%32 of B over
// k-slots 8*(l/32) .. +7; it receives D[8*(r/4) + 4*(l/32) + (r%4)][l%32] for r = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// SiLU(v) = v / (1 + e^-v) with the hardware exponential and reciprocal (about one ulp each;
// h is rounded to bf16 right after, 2^-9 relative).
__device__ __forceinline__ float silu_f32(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

}  // namespace wq
