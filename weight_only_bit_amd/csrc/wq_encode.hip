// wq_encode.hip -- the CCQ (6,4,3) code-cluster encoder on the GPU: fp32 weights -> packed
// codes, 4-bit group scales, per-row super scale, code scale and code zero.
//
// "CCQ: Convolutional Code for Extreme Low-bit Quantization in LLMs": section 3.1 and the
// algorithm "Convolutional Code Quantization" (codebook search per 4-weight vector), section
// 3.3 Eq. 1 (code cluster), section 3.4 (scale optimization, Eq. 2-4, and scale compression
// against a per-row super scale).
// Per output row, groups of 64 along k:
//   group scale  s_g = absmax_g / 31;  super = fl32(max_g s_g / 15) (1 for a zero row)
//   s_q = clip(round(s_g / super), 1, 15);  s = fl32(s_q * super)
//   code C of each vector = argmin over the 2^15 codes of sum_j (v_j - (u_j - zp) s)^2, where
//     u_j is state j of C (shifts 9, 6, 3, 0); ties go to the smallest code
//   with the scale update: per group, with its codes fixed, S* = sum_i w_i q_i / sum_i q_i^2
//     (q_i = u_i - zp, i = 0..63 in order), s_q2 = clip(round(S* / super), 1, 15); when s_q2
//     differs the group is searched again at fl32(s_q2 * super) and the new scale and codes
//     replace the old ones if the group error sum_i (w_i - q_i s)^2 drops (S* > 0 only)
//   beta = min C, alpha = fl32((max C - min C) / 255) (1 when all codes are equal)
//   C' = clip(round((C - beta) / alpha), 0, 255), or with re-pick the cheapest of the 256
//     codes the row can decode (C' -> clamp(round(fmaf(C', alpha, beta)), 0, 2^15 - 1)).
// Every decision is taken in fp64 (costs, ratios, rounding to integers), so the codes depend
// only on the weights, never on a summation order the hardware picks.
//
// One workgroup per row.  The argmin is exact by dynamic programming over the code's five
// 3-bit digits d4..d0 (state j = (d_{4-j}, d_{3-j})): the cost is a chain f0(d4,d3) +
// f1(d3,d2) + f2(d2,d1) + f3(d1,d0), so best_j(a) = min_b f_j(8a + b) + best_{j+1}(b), summed
// right to left and each minimum taken at its smallest argument.
#include <hip/hip_runtime.h>

#include "wq_kernels.hpp"

namespace wq {
namespace {

constexpr int ENC_THREADS = 256;

// Squared error of state u for weight v at scale s, zero point zp.
__device__ __forceinline__ double state_cost(double v, int u, int zp, double s) {
  const double r = v - (double)(u - zp) * s;
  return r * r;
}

// The cheapest 15-bit code for the vector v at scale s (ties to the smallest code).  The scale
// is passed through an empty asm per state so that the 64 products (u - zp) s are formed again
// for each state instead of being kept live across all four (register pressure).
__device__ uint32_t search_code(const double (&v)[4], double s, int zp) {
  double best[8], nxt[8];
  uint32_t arg[4];  // arg[j]: 8 argmin digits of 3 bits (digit for each a)
  // state 3: best over the low digit b for each high digit a
  arg[3] = 0;
  double s3 = s;
  asm volatile("" : "+v"(s3));
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    double bc = INFINITY;
    uint32_t bb = 0;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const double c = state_cost(v[3], a * 8 + b, zp, s3);
      if (c < bc) {
        bc = c;
        bb = (uint32_t)b;
      }
    }
    best[a] = bc;
    arg[3] |= bb << (3 * a);
  }
#pragma unroll
  for (int j = 2; j >= 0; --j) {
    arg[j] = 0;
    double sj = s;
    asm volatile("" : "+v"(sj));
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      double bc = INFINITY;
      uint32_t bb = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const double c = state_cost(v[j], a * 8 + b, zp, sj) + best[b];
        if (c < bc) {
          bc = c;
          bb = (uint32_t)b;
        }
      }
      nxt[a] = bc;
      arg[j] |= bb << (3 * a);
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) best[a] = nxt[a];
  }
  uint32_t d = 0;
#pragma unroll
  for (int a = 1; a < 8; ++a)
    if (best[a] < best[d]) d = (uint32_t)a;
  uint32_t code = d;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    d = (arg[j] >> (3 * d)) & 7u;
    code = (code << 3) | d;
  }
  return code;
}

// Stage 1 of the decode: the code the clustered byte cp stands for.
__device__ __forceinline__ uint32_t expand_code(uint32_t cp, float alpha, float beta) {
  float t = __builtin_fmaf((float)cp, alpha, beta);
  t = __builtin_rintf(t);
  t = fmaxf(t, 0.0f);
  t = fminf(t, 32767.0f);
  return (uint32_t)t;
}

// Cost of decoding code C against v.
__device__ __forceinline__ double code_cost(uint32_t C, const double (&v)[4], double s, int zp) {
  double c = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) c += state_cost(v[j], (int)((C >> (9 - 3 * j)) & 0x3Fu), zp, s);
  return c;
}

// Squared error of a group's 64 weights x[0..63] decoded from its 16 codes at scale s, summed
// in weight order (the order the update's decisions are defined in).
__device__ double group_error(const float* __restrict__ x, const uint16_t* codes, double s, int zp) {
  double e = 0.0;
  for (int i = 0; i < 64; ++i) {
    const int u = (int)((codes[i >> 2] >> (9 - 3 * (i & 3))) & 0x3Fu);
    const double r = (double)x[i] - (double)(u - zp) * s;
    e += r * r;
  }
  return e;
}

// Block-wide reductions (256 threads; red holds one slot per wave).
__device__ __forceinline__ double block_max(double x, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  const double r = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, uint32_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
  }
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = lo;
    red[4 + (threadIdx.x >> 6)] = hi;
  }
  __syncthreads();
  lo = min(min(red[0], red[1]), min(red[2], red[3]));
  hi = max(max(red[4], red[5]), max(red[6], red[7]));
  __syncthreads();
}

// LDS layout: group absmax f64 [G], group scales s f32 [G], full codes u16 [V], expand table
// u16 [256], 4-bit group scales u8 [G], then (scale update only) the updated scales u8 [G]
// and the re-searched codes u16 [V]; reduction slots last.
struct EncLds {
  int64_t amax, sgrp, full, table, sq, sq2, full2, red, bytes;
};
__host__ __device__ inline EncLds enc_lds(int64_t k, bool update) {
  const int64_t G = k / 64, V = k / 4;
  EncLds L;
  L.amax = 0;
  L.sgrp = 8 * G;
  L.full = 12 * G;
  L.table = L.full + 2 * V;
  L.sq = L.table + 512;
  L.sq2 = L.sq + G;
  L.full2 = (L.sq2 + G + 1) & ~(int64_t)1;
  const int64_t end = update ? L.full2 + 2 * V : L.sq + G;
  L.red = (end + 15) & ~(int64_t)15;
  L.bytes = L.red + 4 * 8 + 8 * 4;
  return L;
}

template <bool REPICK, bool UPDATE>
__global__ __launch_bounds__(ENC_THREADS) void ccq_encode_kernel(const float* __restrict__ w,
                                                                 int64_t k, int32_t zp,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ qscale,
                                                                 float* __restrict__ super_out,
                                                                 float* __restrict__ cs_out,
                                                                 float* __restrict__ cz_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t G = k / 64, V = k / 4, QB = (G + 1) / 2;
  const EncLds L = enc_lds(k, UPDATE);
  double* amax = reinterpret_cast<double*>(lds + L.amax);      // [G]
  float* sgrp = reinterpret_cast<float*>(lds + L.sgrp);        // [G]
  uint16_t* full = reinterpret_cast<uint16_t*>(lds + L.full);  // [V]
  uint16_t* table = reinterpret_cast<uint16_t*>(lds + L.table);  // [256]
  uint8_t* sqv = lds + L.sq;                                   // [G]
  uint8_t* sq2v = lds + L.sq2;                                 // [G] (update)
  uint16_t* full2 = reinterpret_cast<uint16_t*>(lds + L.full2);  // [V] (update)
  double* redd = reinterpret_cast<double*>(lds + L.red);
  uint32_t* redu = reinterpret_cast<uint32_t*>(redd + 4);
  const float* x = w + row * k;

  // 1. group absmax and the row's largest group scale
  double smax = 0.0;
  for (int64_t g = tid; g < G; g += ENC_THREADS) {
    const float4* p = reinterpret_cast<const float4*>(x + g * 64);
    double a = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 q = p[i];
      a = fmax(a, fabs((double)q.x));
      a = fmax(a, fabs((double)q.y));
      a = fmax(a, fabs((double)q.z));
      a = fmax(a, fabs((double)q.w));
    }
    amax[g] = a;
    smax = fmax(smax, a / 31.0);
  }
  smax = block_max(smax, redd);
  float sup = (float)(smax / 15.0);
  if (!(sup > 0.0f)) sup = 1.0f;

  // 2. 4-bit group scales
  for (int64_t g = tid; g < G; g += ENC_THREADS) {
    double sqd = rint((amax[g] / 31.0) / (double)sup);
    sqd = sqd < 1.0 ? 1.0 : (sqd > 15.0 ? 15.0 : sqd);
    const uint32_t sq = (uint32_t)sqd;
    sgrp[g] = (float)sq * sup;
    sqv[g] = (uint8_t)sq;
  }
  if (tid == 0) super_out[row] = sup;
  __syncthreads();

  // 3. codebook search of every vector
  for (int64_t c = tid; c < V; c += ENC_THREADS) {
    const float4 q = reinterpret_cast<const float4*>(x)[c];
    const double v[4] = {(double)q.x, (double)q.y, (double)q.z, (double)q.w};
    full[c] = (uint16_t)search_code(v, (double)sgrp[c >> 4], zp);
  }
  __syncthreads();

  // 3b. scale optimization: least-squares scale of each group with its codes fixed,
  // re-quantized to 4 bits; groups whose scale changes are searched again
  if constexpr (UPDATE) {
    for (int64_t g = tid; g < G; g += ENC_THREADS) {
      const float* xg = x + g * 64;
      const uint16_t* cg = full + g * 16;
      double num = 0.0, den = 0.0;
      for (int i = 0; i < 64; ++i) {
        const double q = (double)((int)((cg[i >> 2] >> (9 - 3 * (i & 3))) & 0x3Fu) - zp);
        num += (double)xg[i] * q;
        den += q * q;
      }
      uint32_t sq2 = 0;
      if (den > 0.0 && num > 0.0) {
        double sqd = rint((num / den) / (double)sup);
        sqd = sqd < 1.0 ? 1.0 : (sqd > 15.0 ? 15.0 : sqd);
        sq2 = (uint32_t)sqd;
        if (sq2 == sqv[g]) sq2 = 0;
      }
      sq2v[g] = (uint8_t)sq2;
    }
    __syncthreads();
    for (int64_t c = tid; c < V; c += ENC_THREADS) {
      const uint32_t sq2 = sq2v[c >> 4];
      if (sq2 == 0) continue;
      const float4 q = reinterpret_cast<const float4*>(x)[c];
      const double v[4] = {(double)q.x, (double)q.y, (double)q.z, (double)q.w};
      full2[c] = (uint16_t)search_code(v, (double)((float)sq2 * sup), zp);
    }
    __syncthreads();
    for (int64_t g = tid; g < G; g += ENC_THREADS) {
      const uint32_t sq2 = sq2v[g];
      if (sq2 == 0) continue;
      const float s2 = (float)sq2 * sup;
      const double e0 = group_error(x + g * 64, full + g * 16, (double)sgrp[g], zp);
      const double e2 = group_error(x + g * 64, full2 + g * 16, (double)s2, zp);
      if (e2 < e0) {
        for (int c = 0; c < 16; ++c) full[g * 16 + c] = full2[g * 16 + c];
        sqv[g] = (uint8_t)sq2;
        sgrp[g] = s2;
      }
    }
    __syncthreads();
  }

  // 4. stored group scales (two per byte, even group in the low nibble) and the code range
  for (int64_t b = tid; b < QB; b += ENC_THREADS) {
    const uint32_t lo4 = sqv[2 * b];
    const uint32_t hi4 = (2 * b + 1 < G) ? sqv[2 * b + 1] : 0u;
    qscale[row * QB + b] = (uint8_t)(lo4 | (hi4 << 4));
  }
  uint32_t lo = 0x7FFFu, hi = 0u;
  for (int64_t c = tid; c < V; c += ENC_THREADS) {
    lo = min(lo, (uint32_t)full[c]);
    hi = max(hi, (uint32_t)full[c]);
  }
  block_minmax(lo, hi, redu);

  // 5. code cluster
  const float alpha = hi > lo ? (float)((double)(hi - lo) / 255.0) : 1.0f;
  const float beta = (float)lo;
  if (tid == 0) {
    cs_out[row] = alpha;
    cz_out[row] = beta;
  }
  if constexpr (REPICK) {
    table[tid] = (uint16_t)expand_code((uint32_t)tid, alpha, beta);  // 256 threads, 256 codes
    __syncthreads();
  }
  for (int64_t c = tid; c < V; c += ENC_THREADS) {
    double cp = rint(((double)full[c] - (double)beta) / (double)alpha);
    cp = cp < 0.0 ? 0.0 : (cp > 255.0 ? 255.0 : cp);
    uint32_t best = (uint32_t)cp;
    if constexpr (REPICK) {
      const float4 q = reinterpret_cast<const float4*>(x)[c];
      const double v[4] = {(double)q.x, (double)q.y, (double)q.z, (double)q.w};
      const double s = (double)sgrp[c >> 4];
      double bc = INFINITY;
      for (uint32_t cand = 0; cand < 256; ++cand) {
        const double cc = code_cost(table[cand], v, s, zp);
        if (cc < bc) {
          bc = cc;
          best = cand;
        }
      }
    }
    codes[row * V + c] = (uint8_t)best;
  }
}

}  // namespace

size_t ccq_encode_lds_bytes(int64_t k, int refine) {
  return (size_t)enc_lds(k, (refine & 2) != 0).bytes;
}

hipError_t launch_ccq_encode(const float* w, int64_t n, int64_t k, int32_t zp, int refine,
                             uint8_t* codes, uint8_t* qscale, float* super_scale,
                             float* code_scale, float* code_zero, hipStream_t stream) {
  const size_t lds = ccq_encode_lds_bytes(k, refine);
  typedef void (*Kern)(const float*, int64_t, int32_t, uint8_t*, uint8_t*, float*, float*, float*);
  static const Kern kerns[4] = {ccq_encode_kernel<false, false>, ccq_encode_kernel<true, false>,
                                ccq_encode_kernel<false, true>, ccq_encode_kernel<true, true>};
  const int variant = refine & 3;
  static std::atomic<uint64_t> lds_set[4];  // per variant, one bit per device
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kerns[variant]), 160 * 1024,
                                    lds_set[variant]);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kerns[variant], dim3((unsigned)n), dim3(ENC_THREADS), lds, stream, w, k, zp,
                     codes, qscale, super_scale, code_scale, code_zero);
  return hipGetLastError();
}

}  // namespace wq
