// wq_misc.hip -- exact dequantize, MoE routing (sort pairs by expert) and the routing-
// weighted combine.
#include <hip/hip_runtime.h>

#include "wq_kernels.hpp"

namespace wq {
namespace {

// ---------------------------------------------------------------------------------------------
// Dequantize: one thread per 16 consecutive weights of a row (one 64-bit or 32-bit code load,
// two 16-byte stores), bit-exact with the format definitions:
//   INT4:   bf16(f32(q) * s)                 (lesson E6.4: x_hat = s q, zero point 0)
//   AFFINE: bf16(f32(q - z) * s)             (lesson E6.4: x_hat = s (q - z))
//   CCQ2:   s = f32(s_q) * super; C = expand(C'); u = (C >> shift) & 0x3F;
//           bf16(f32(u - zp) * s)           (CCQ, "Dequantization with Code Cluster")
// ---------------------------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const DevWeight w, int64_t rows,
                                                      uint16_t* __restrict__ out) {
  const int64_t blocks_per_row = w.k / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * blocks_per_row) return;
  const int64_t row = idx / blocks_per_row;
  const int64_t blk = idx % blocks_per_row;
  const int64_t k0 = blk * 16;
  const int64_t G = w.k / 64;
  const int64_t g = k0 >> 6;
  float v[16];
  if constexpr (FMT == FMT_INT4) {
    const u32x2 c = *reinterpret_cast<const u32x2*>(w.codes + row * (w.k / 2) + (k0 >> 1));
    const float s = bf16_bits_to_f32(w.group ? w.scales[row * G + g] : w.scales[row]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t word = i < 8 ? c.x : c.y;
      v[i] = int4_value((word >> (4 * (i & 7))) & 0xFu, s);
    }
  } else if constexpr (FMT == FMT_AFFINE2) {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(w.codes + row * (w.k / 4) + (k0 >> 2));
    const float s = bf16_bits_to_f32(w.scales[row * G + g]);
    const uint32_t z = w.zeros[row * G + g];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = affine2_value((c >> (2 * i)) & 3u, z, s);
  } else {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(w.codes + row * (w.k / 4) + (k0 >> 2));
    const uint32_t sq = (w.qscale[row * ((G + 1) / 2) + (g >> 1)] >> (4 * (g & 1))) & 0xFu;
    const float s = (float)sq * w.super_scale[row];
    const float cs = w.code_scale[row], cz = w.code_zero[row];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t C = ccq_expand_bits((float)((c >> (8 * b)) & 0xFFu), cs, cz) & 0x7FFFu;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * b + j] = ccq_value((C >> (9 - 3 * j)) & 0x3Fu, w.zp, s);
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + row * w.k + k0);
  dst[0] = (u32x4){cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]), cvt_pk_bf16(v[4], v[5]),
                   cvt_pk_bf16(v[6], v[7])};
  dst[1] = (u32x4){cvt_pk_bf16(v[8], v[9]), cvt_pk_bf16(v[10], v[11]), cvt_pk_bf16(v[12], v[13]),
                   cvt_pk_bf16(v[14], v[15])};
}

// ---------------------------------------------------------------------------------------------
// Routing: one workgroup of 1024 threads.
//   pass 1: per-expert counts (LDS integer atomics; the totals do not depend on order);
//   scan:   offsets = exclusive prefix sum of the counts;
//   pass 2: 1024 pairs per round; a pair's slot is offsets[e] + (pairs of e in earlier rounds)
//           + (pairs of e in earlier waves of this round) + (its rank among the lanes of its
//           wave with the same expert), which keeps the pairs of an expert in increasing p.
// ---------------------------------------------------------------------------------------------
constexpr int ROUTE_THREADS = 1024;
constexpr int ROUTE_WAVES = ROUTE_THREADS / 64;

__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(const int32_t* __restrict__ ids,
                                                              int64_t npairs, int32_t experts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted) {
  extern __shared__ int32_t sm[];
  int32_t* cnt = sm;                     // [experts]
  int32_t* run = cnt + experts;          // [experts] next free slot per expert
  int32_t* wc = run + experts;           // [ROUTE_WAVES][experts]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < experts; i += ROUTE_THREADS) cnt[i] = 0;
  for (int i = tid; i < ROUTE_WAVES * experts; i += ROUTE_THREADS) wc[i] = 0;
  __syncthreads();
  // Ids outside [0, experts) are dropped (never counted or placed) so a bad routing table
  // cannot make any kernel write out of bounds.
  for (int64_t p = tid; p < npairs; p += ROUTE_THREADS) {
    const int32_t e = ids[p];
    if (e >= 0 && e < experts) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int32_t s = 0;
    for (int e = 0; e < experts; ++e) {
      offsets[e] = s;
      run[e] = s;
      s += cnt[e];
    }
    offsets[experts] = s;
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = 0; base < npairs; base += ROUTE_THREADS) {
    const int64_t p = base + tid;
    int32_t e = (p < npairs) ? ids[p] : -1;
    if (e >= experts) e = -1;
    bool done = e < 0;
    int32_t rank = 0;
    // Peel off one expert value at a time, led by the lowest pending lane.
    while (true) {
      const uint64_t pending = __ballot(!done);
      if (pending == 0) break;
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int32_t el = __shfl(e, leader);
      const bool mine = !done && e == el;
      const uint64_t m = __ballot(mine);
      if (mine) {
        rank = __popcll(m & lt_mask);
        done = true;
      }
      if (lane == leader) wc[wave * experts + el] = __popcll(m);
    }
    __syncthreads();
    for (int ex = tid; ex < experts; ex += ROUTE_THREADS) {
      int32_t r = run[ex];
      for (int w = 0; w < ROUTE_WAVES; ++w) {
        const int32_t c = wc[w * experts + ex];
        wc[w * experts + ex] = r;
        r += c;
      }
      run[ex] = r;
    }
    __syncthreads();
    if (e >= 0) sorted[wc[wave * experts + e] + rank] = (int32_t)p;
    __syncthreads();
    for (int i = tid; i < ROUTE_WAVES * experts; i += ROUTE_THREADS) wc[i] = 0;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// Combine: y[t][c] = bf16( sum_j w[t][j] * d[t*topk + j][c] ), slots summed in order j with
// fp32 fused multiply-adds.  One thread per 4 columns.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ d,
                                                      const float* __restrict__ wts, int64_t t,
                                                      int32_t topk, int64_t hidden,
                                                      uint16_t* __restrict__ y) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t quads = hidden / 4;
  if (q >= t * quads) return;
  const int64_t tok = q / quads;
  const int64_t c = (q % quads) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const float w = wts[tok * topk + j];
    const f32x4 v = *reinterpret_cast<const f32x4*>(d + (tok * topk + j) * hidden + c);
    acc.x = __builtin_fmaf(w, v.x, acc.x);
    acc.y = __builtin_fmaf(w, v.y, acc.y);
    acc.z = __builtin_fmaf(w, v.z, acc.z);
    acc.w = __builtin_fmaf(w, v.w, acc.w);
  }
  u32x2 o = {pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w)};
  *reinterpret_cast<u32x2*>(y + tok * hidden + c) = o;
}

}  // namespace

hipError_t launch_dequant(int fmt, const DevWeight& w, int64_t experts, uint16_t* out,
                          hipStream_t stream) {
  const int64_t rows = experts * w.n;
  const int64_t threads = rows * (w.k / 16);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (fmt == FMT_INT4)
    hipLaunchKernelGGL(dequant_kernel<FMT_INT4>, grid, dim3(256), 0, stream, w, rows, out);
  else if (fmt == FMT_AFFINE2)
    hipLaunchKernelGGL(dequant_kernel<FMT_AFFINE2>, grid, dim3(256), 0, stream, w, rows, out);
  else
    hipLaunchKernelGGL(dequant_kernel<FMT_CCQ2>, grid, dim3(256), 0, stream, w, rows, out);
  return hipGetLastError();
}

hipError_t launch_route(const int32_t* ids, int64_t npairs, int32_t experts, int32_t* offsets,
                        int32_t* sorted_pairs, hipStream_t stream) {
  const size_t lds = sizeof(int32_t) * (size_t)experts * (2 + ROUTE_WAVES);
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(ROUTE_THREADS), lds, stream, ids, npairs,
                     experts, offsets, sorted_pairs);
  return hipGetLastError();
}

hipError_t launch_combine(const float* d, const float* weights, int64_t t, int32_t topk,
                          int64_t hidden, uint16_t* y, hipStream_t stream) {
  const int64_t threads = t * (hidden / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, d, weights, t, topk, hidden, y);
  return hipGetLastError();
}

}  // namespace wq
