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

enum { FMT_INT4 = 1, FMT_AFFINE2 = 2, FMT_CCQ2 = 3 };

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

// fp32 -> bf16 bits, round half to even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
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

// Two fp32 values -> packed bf16 pair (round half to even), low half first.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ---------------------------------------------------------------------------------------------
// Fast exact decode for the MFMA kernels.  Each helper turns the packed bytes one lane holds
// for a 64-weight group (16 consecutive weights of one row) into 8 dwords of bf16 pairs in k
// order, equal bit for bit to the format's x_hat:
//   value = bf16(fl((c - z) * s))  computed as  bf16(fma(f32(c), s, -z*s))
// which is the same single rounding of the same exact product whenever z*s is exact in fp32
// (z a power of two -- the CCQ zero point 32 -- or z*s with few enough bits -- the 2-bit
// affine zero point times a bf16 scale, and INT4's 8 * s).  For c == z the fma gives +0 where
// the two-step form gives 0 * s: the same bits for s >= 0 (scales are non-negative).
// ---------------------------------------------------------------------------------------------

// CCQ: one dword = 4 clustered bytes = 16 weights.  s = f32(s_q) * super, mzs = -zp * s.
// CLAMP = false only when ccq_row_needs_no_clamp holds for the row.
template <bool CLAMP = true>
__device__ __forceinline__ void ccq_decode16(uint32_t w, float cs, float cz, float s, float mzs,
                                             uint32_t (&p)[8]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t R = ccq_expand_bits<CLAMP>((float)((w >> (8 * b)) & 0xFFu), cs, cz);
    float f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)  // bit-shift decode: shifts 9, 6, 3, 0; mask 0x3F
      f[j] = __builtin_fmaf((float)((R >> (9 - 3 * j)) & 0x3Fu), s, mzs);
    p[2 * b] = cvt_pk_bf16(f[0], f[1]);
    p[2 * b + 1] = cvt_pk_bf16(f[2], f[3]);
  }
}

// a & b, opaque to the optimizer: keeps a masked dword whole so each byte is converted by
// one v_cvt_f32_ubyteN instead of a bit-field extract plus a convert.
__device__ __forceinline__ uint32_t and_opaque(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// INT4: two dwords = 16 signed nibbles (first weight in the low nibble).  XOR 8 biases a
// two's-complement nibble q to q + 8 in 0..15, so value = fma(f32(q + 8), s, -8 s).
__device__ __forceinline__ void int4_decode16(uint32_t w0, uint32_t w1, float s,
                                              uint32_t (&p)[8]) {
  const float m8s = -8.0f * s;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t d = (h ? w1 : w0) ^ 0x88888888u;
    const uint32_t ev = and_opaque(d, 0x0F0F0F0Fu);       // nibbles 0,2,4,6 -> bytes 0..3
    const uint32_t od = and_opaque(d >> 4, 0x0F0F0F0Fu);  // nibbles 1,3,5,7
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float a = __builtin_fmaf((float)((ev >> (8 * b)) & 0xFFu), s, m8s);
      const float c = __builtin_fmaf((float)((od >> (8 * b)) & 0xFFu), s, m8s);
      p[4 * h + b] = cvt_pk_bf16(a, c);
    }
  }
}

// 2-bit affine: one dword = 16 codes (first in the lowest two bits); value = fma(f32(q), s,
// -z s) with z s exact (8-bit z times a bf16 scale).
__device__ __forceinline__ void affine2_decode16(uint32_t w, float s, float mzs,
                                                 uint32_t (&p)[8]) {
  uint32_t q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = and_opaque(w >> (2 * i), 0x03030303u);  // byte b: code 4b + i
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __builtin_fmaf((float)((q[i] >> (8 * b)) & 0xFFu), s, mzs);
    p[2 * b] = cvt_pk_bf16(f[0], f[1]);
    p[2 * b + 1] = cvt_pk_bf16(f[2], f[3]);
  }
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

__device__ __forceinline__ float silu_f32(float v) { return v / (1.0f + __expf(-v)); }

}  // namespace wq
