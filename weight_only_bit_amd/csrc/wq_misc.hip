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
//   INT8:   bf16(f32(q) * s)                 (the same formula for a signed byte)
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
  } else if constexpr (FMT == FMT_INT8) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(w.codes + row * w.k + k0);
    const float s = bf16_bits_to_f32(w.group ? w.scales[row * G + g] : w.scales[row]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int32_t q = (int32_t)(int8_t)(uint8_t)(c[i >> 2] >> (8 * (i & 3)));
      v[i] = (float)q * s;
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

// CCQ without code cluster ("CCQ", section 3.5, "Dequantization without Code Cluster", with the
// (4,3,2) and (3,3,2)(3,4,2) rows of the configuration table): one thread per 16 weights of a
// group; each weight is read from its own code word,
//   s = f32(W[P-1] & s_mask) * super;  u = (W[i / p] >> shift[i % p]) & w_mask;
//   x_hat = bf16(f32(u - zp) * s).
template <int FMT>
__global__ __launch_bounds__(256) void dequant_alg2_kernel(const DevWeight w, int64_t rows,
                                                           uint16_t* __restrict__ out) {
  constexpr bool HYB = FMT == FMT_CCQH;
  constexpr int P = HYB ? 10 : 22, PW = HYB ? 7 : 3, GB = alg2_group_bytes(FMT);
  constexpr uint32_t WMASK = HYB ? 0x7u : 0xFu, SMASK = HYB ? 0x1FFFu : 0xFu;
  const int64_t quarters = w.k / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * quarters) return;
  const int64_t row = idx / quarters;
  const int64_t k0 = (idx % quarters) * 16;
  const int64_t g = k0 >> 6;
  const uint8_t* grp = w.codes + row * (w.k / 64) * GB + g * GB;
  auto word = [&](int j) -> uint32_t {
    return HYB ? (uint32_t)grp[2 * j] | ((uint32_t)grp[2 * j + 1] << 8) : (uint32_t)grp[j];
  };
  const float s = (float)(word(P - 1) & SMASK) * w.super_scale[row];
  float v[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int i = (int)(k0 & 63) + t;
    const int j = i % PW;  // state within the word: shifts 13,11,9,6,4,2,0 or 4,2,0
    const int sh = HYB ? (j < 3 ? 13 - 2 * j : 12 - 2 * j) : 4 - 2 * j;
    v[t] = ccq_value((word(i / PW) >> sh) & WMASK, w.zp, s);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + row * w.k + k0);
  dst[0] = (u32x4){cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]), cvt_pk_bf16(v[4], v[5]),
                   cvt_pk_bf16(v[6], v[7])};
  dst[1] = (u32x4){cvt_pk_bf16(v[8], v[9]), cvt_pk_bf16(v[10], v[11]), cvt_pk_bf16(v[12], v[13]),
                   cvt_pk_bf16(v[14], v[15])};
}

// ---------------------------------------------------------------------------------------------
// Routing: a stable counting sort of the pairs by expert.  One workgroup of T threads sorts a
// contiguous range of pairs.  Thread t owns the contiguous pairs [t c, (t + 1) c) of the range
// (c = ceil(range / T)) and a private row of E counters in LDS (T * E <= 32768 int32, 128 KB):
//   pass 1: each thread counts its pairs per expert in its own row (no atomics);
//   scan:   column sums give the range's expert totals; with the whole array as the range their
//           exclusive scan gives the expert offsets, for a chunk of a longer array the chunk's
//           first slot per expert comes from a table (below); each counter is then replaced by
//           that slot + (pairs of e owned by threads t' < t);
//   pass 2: each thread walks its pairs again in order and places pair p at its counter,
//           incrementing it -- so an expert's pairs land in increasing p.
// Long arrays (more than two chunks of ROUTE_CHUNK_MIN pairs) are cut into chunks sorted by
// one workgroup each: route_count_kernel writes each chunk's count per expert to a table,
// route_scan_kernel turns the table into each chunk's first slot per expert (the column's
// exclusive prefix plus the expert's offset) and writes the offsets, and route_kernel places
// every chunk -- chunks in order, so the sort stays stable.
// Ids outside [0, E) are dropped (never counted or placed), so a bad routing table cannot
// make any kernel write out of bounds.
// ---------------------------------------------------------------------------------------------
constexpr int ROUTE_MAX_THREADS = 1024;
constexpr int ROUTE_LDS_COUNTERS = 32768;

int route_threads(int32_t experts) {
  int t = ROUTE_LDS_COUNTERS / experts;
  if (t > ROUTE_MAX_THREADS) t = ROUTE_MAX_THREADS;
  int p = 64;
  while (p * 2 <= t) p *= 2;  // a power of two, at least one wave
  return p;
}

// chunk_first: null to sort the whole array in one workgroup (which then also writes the
// offsets), else the [chunks][E] table of each chunk's first slot per expert, workgroup b
// sorting pairs [b chunk, (b + 1) chunk).
__global__ __launch_bounds__(ROUTE_MAX_THREADS) void route_kernel(const int32_t* __restrict__ ids,
                                                                  int64_t npairs, int32_t experts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted,
                                                                  const int32_t* __restrict__ chunk_first,
                                                                  int64_t chunk) {
  extern __shared__ int32_t sm[];
  const int T = blockDim.x;
  const int E = experts;
  int32_t* cnt = sm;                   // [T][E]
  const int S = T >= E ? T / E : 1;    // scan segments per expert
  const int R = T / S;                 // counter rows per segment
  int32_t* part = cnt + T * E;         // [S][E] segment sums
  int32_t* base = part + S * E;        // [E] first slot of each expert in this range
  const int tid = threadIdx.x;
  const int64_t q0 = chunk_first ? (int64_t)blockIdx.x * chunk : 0;
  const int64_t q1 = chunk_first ? (q0 + chunk < npairs ? q0 + chunk : npairs) : npairs;
  const int64_t c = (q1 - q0 + T - 1) / T;
  const int64_t p0 = q0 + (int64_t)tid * c;
  const int64_t p1 = p0 + c < q1 ? p0 + c : q1;

  for (int i = tid; i < T * E; i += T) cnt[i] = 0;
  __syncthreads();
  int32_t* row = cnt + tid * E;
  // pairs in batches of RB: the batch's id loads are issued together, one memory round trip per
  // batch (ids past the thread's range read as -1, which no expert matches)
  constexpr int RB = 8;
  for (int64_t p = p0; p < p1; p += RB) {
    int32_t v[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) v[j] = p + j < p1 ? ids[p + j] : -1;
#pragma unroll
    for (int j = 0; j < RB; ++j)
      if (v[j] >= 0 && v[j] < E) row[v[j]] += 1;
  }
  __syncthreads();
  // segment sums: (expert e, segment g) covers counter rows g R .. g R + R - 1
  for (int idx = tid; idx < S * E; idx += T) {
    const int e = idx % E, g = idx / E;
    int32_t sum = 0;
    for (int r = g * R; r < g * R + R; ++r) sum += cnt[r * E + e];
    part[g * E + e] = sum;
  }
  __syncthreads();
  if (chunk_first) {  // this chunk's first slots, from the table
    for (int e = tid; e < E; e += T) base[e] = chunk_first[(int64_t)blockIdx.x * E + e];
  } else if (tid < 64) {  // expert totals and their exclusive scan (lane l: a block of experts)
    const int per = (E + 63) / 64;
    const int e0 = tid * per;
    int32_t local = 0;
    for (int e = e0; e < e0 + per && e < E; ++e) {
      int32_t tot = 0;
      for (int g = 0; g < S; ++g) tot += part[g * E + e];
      base[e] = tot;
      local += tot;
    }
    int32_t incl = local;  // inclusive scan of the lane sums
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t v = __shfl_up(incl, d);
      if (tid >= d) incl += v;
    }
    int32_t run = incl - local;
    for (int e = e0; e < e0 + per && e < E; ++e) {
      const int32_t tot = base[e];
      base[e] = run;
      offsets[e] = run;
      run += tot;
    }
    if (tid == 63) offsets[E] = incl;
  }
  __syncthreads();
  // counters -> first slot of each (thread, expert)
  for (int idx = tid; idx < S * E; idx += T) {
    const int e = idx % E, g = idx / E;
    int32_t run = base[e];
    for (int gg = 0; gg < g; ++gg) run += part[gg * E + e];
    for (int r = g * R; r < g * R + R; ++r) {
      const int32_t v = cnt[r * E + e];
      cnt[r * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  for (int64_t p = p0; p < p1; p += RB) {
    int32_t v[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) v[j] = p + j < p1 ? ids[p + j] : -1;
#pragma unroll
    for (int j = 0; j < RB; ++j)
      if (v[j] >= 0 && v[j] < E) sorted[row[v[j]]++] = (int32_t)(p + j);
  }
}

// Chunks of a long routing array: at least ROUTE_CHUNK_MIN pairs each, at most
// ROUTE_MAX_CHUNKS of them (the table is chunks x E int32, at most 1 MB).
constexpr int64_t ROUTE_CHUNK_MIN = 2048;
constexpr int64_t ROUTE_MAX_CHUNKS = 512;

int64_t route_chunk(int64_t npairs) {
  const int64_t c = (npairs + ROUTE_MAX_CHUNKS - 1) / ROUTE_MAX_CHUNKS;
  return c > ROUTE_CHUNK_MIN ? c : ROUTE_CHUNK_MIN;
}

// Workgroup b: the per-expert counts of pairs [b chunk, (b + 1) chunk) into table row b.
__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ ids,
                                                          int64_t npairs, int32_t experts,
                                                          int64_t chunk, int32_t* __restrict__ table) {
  __shared__ int32_t hist[ROUTE_LDS_COUNTERS / 64];  // experts <= 512
  const int E = experts;
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t q0 = (int64_t)blockIdx.x * chunk;
  const int64_t q1 = q0 + chunk < npairs ? q0 + chunk : npairs;
  for (int64_t p = q0 + threadIdx.x; p < q1; p += 256) {
    const int32_t e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) table[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup of 512 threads (thread e: expert e): each table column becomes its exclusive
// prefix over the chunks plus the expert's offset; the offsets are the exclusive scan of the
// expert totals, offsets[E] the number of pairs placed.
__global__ __launch_bounds__(512) void route_scan_kernel(int32_t* __restrict__ table,
                                                         int32_t chunks, int32_t experts,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int32_t sc[2][512];
  const int e = threadIdx.x;
  const int E = experts;
  int32_t total = 0;
  constexpr int CB = 8;  // chunks per batch of loads
  if (e < E) {
    for (int b0 = 0; b0 < chunks; b0 += CB) {
      int32_t v[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) v[j] = b0 + j < chunks ? table[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < CB; ++j)
        if (b0 + j < chunks) {
          table[(int64_t)(b0 + j) * E + e] = total;
          total += v[j];
        }
    }
  }
  sc[0][e] = total;  // 0 for e >= E
  __syncthreads();
  int src = 0;
  for (int d = 1; d < 512; d <<= 1) {  // inclusive scan over the experts
    const int32_t v = sc[src][e] + (e >= d ? sc[src][e - d] : 0);
    sc[src ^ 1][e] = v;
    src ^= 1;
    __syncthreads();
  }
  const int32_t first = sc[src][e] - total;
  if (e < E) {
    offsets[e] = first;
    for (int b0 = 0; b0 < chunks; b0 += CB) {
      int32_t v[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) v[j] = b0 + j < chunks ? table[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < CB; ++j)
        if (b0 + j < chunks) table[(int64_t)(b0 + j) * E + e] = v[j] + first;
    }
  }
  if (e == E - 1) offsets[E] = first + total;
}

// ---------------------------------------------------------------------------------------------
// Routing of few pairs (at most ROUTE_SMALL_PAIRS, a decode step): the counter rows above cost
// more than the pairs themselves.  One thread per pair; wave c holds the pairs 64 c .. 64 c + 63.
// Each lane finds the lanes of its wave with the same expert from ten ballots over the bits of
// its id (E <= 512; dropped pairs carry the id E, which no expert matches), so its rank among
// them is a population count of the lower lanes.  The first lane of each such group writes the
// group's size to the wave's row of an LDS histogram; per expert, the rows' exclusive prefix over
// waves plus the expert's offset is the slot of the wave's first pair of that expert.  Equal ids
// therefore keep increasing p -- the stable order of the kernel above.
// ---------------------------------------------------------------------------------------------
constexpr int ROUTE_SMALL_PAIRS = 1024;
constexpr int ROUTE_MAX_EXPERTS = ROUTE_LDS_COUNTERS / 64;  // 512

__global__ __launch_bounds__(1024) void route_small_kernel(const int32_t* __restrict__ ids,
                                                           int32_t npairs, int32_t experts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted) {
  __shared__ int32_t s_hist[ROUTE_SMALL_PAIRS / 64 * ROUTE_MAX_EXPERTS];  // [wave][expert]
  __shared__ int32_t s_base[ROUTE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int T = blockDim.x;  // 64 * ceil(npairs / 64), at least 64
  const int lane = tid & 63;
  const int c = tid >> 6;
  const int nc = T >> 6;
  const int E = experts;
  int e = E;
  if (tid < npairs) {
    const int v = ids[tid];
    if (v >= 0 && v < E) e = v;
  }
  for (int i = tid; i < nc * ROUTE_MAX_EXPERTS; i += T) s_hist[i] = 0;
  uint64_t same = ~0ull;  // lanes of this wave with the same id
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  const int within = __popcll(same & ((1ull << lane) - 1ull));
  __syncthreads();
  if (e < E && within == 0) s_hist[c * ROUTE_MAX_EXPERTS + e] = __popcll(same);
  __syncthreads();
  for (int x = tid; x < E; x += T) {  // per expert: prefix over waves, total
    int32_t run = 0;
    for (int w = 0; w < nc; ++w) {
      const int32_t v = s_hist[w * ROUTE_MAX_EXPERTS + x];
      s_hist[w * ROUTE_MAX_EXPERTS + x] = run;
      run += v;
    }
    s_base[x] = run;
  }
  __syncthreads();
  // exclusive scan of the totals (wave 0; lane l takes a block of experts)
  if (tid < 64) {
    const int per = (E + 63) / 64;
    const int e0 = tid * per;
    int32_t local = 0;
    for (int x = e0; x < e0 + per && x < E; ++x) local += s_base[x];
    int32_t incl = local;
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t v = __shfl_up(incl, d);
      if (tid >= d) incl += v;
    }
    int32_t run = incl - local;
    for (int x = e0; x < e0 + per && x < E; ++x) {
      const int32_t tot = s_base[x];
      s_base[x] = run;
      offsets[x] = run;
      run += tot;
    }
    if (tid == 63) offsets[E] = incl;
  }
  __syncthreads();
  if (e < E) sorted[s_base[e] + s_hist[c * ROUTE_MAX_EXPERTS + e] + within] = tid;
}

// ---------------------------------------------------------------------------------------------
// Combine: y[t][c] = bf16( sum_j w[t][j] * d[t*topk + j][c] ), slots summed in order j with
// fp32 fused multiply-adds.  One thread per 4 columns; the slots' rows are loaded 8 at a time
// before their multiply-adds, so a thread has up to 8 loads in flight.
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
  for (int j0 = 0; j0 < topk; j0 += 8) {
    float w[8];
    f32x4 v[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int64_t j = j0 + jj;
      if (j < topk) {
        w[jj] = wts[tok * topk + j];
        v[jj] = *reinterpret_cast<const f32x4*>(d + (tok * topk + j) * hidden + c);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj < topk) {
        acc.x = __builtin_fmaf(w[jj], v[jj].x, acc.x);
        acc.y = __builtin_fmaf(w[jj], v[jj].y, acc.y);
        acc.z = __builtin_fmaf(w[jj], v[jj].z, acc.z);
        acc.w = __builtin_fmaf(w[jj], v[jj].w, acc.w);
      }
    }
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
  else if (fmt == FMT_INT8)
    hipLaunchKernelGGL(dequant_kernel<FMT_INT8>, grid, dim3(256), 0, stream, w, rows, out);
  else if (fmt == FMT_CCQ432)
    hipLaunchKernelGGL(dequant_alg2_kernel<FMT_CCQ432>, grid, dim3(256), 0, stream, w, rows, out);
  else if (fmt == FMT_CCQH)
    hipLaunchKernelGGL(dequant_alg2_kernel<FMT_CCQH>, grid, dim3(256), 0, stream, w, rows, out);
  else
    hipLaunchKernelGGL(dequant_kernel<FMT_CCQ2>, grid, dim3(256), 0, stream, w, rows, out);
  return hipGetLastError();
}

int64_t route_table_entries(int64_t npairs, int32_t experts) {
  if (npairs <= 2 * ROUTE_CHUNK_MIN || experts <= 0) return 0;
  const int64_t chunk = route_chunk(npairs);
  return (npairs + chunk - 1) / chunk * experts;
}

hipError_t launch_route(const int32_t* ids, int64_t npairs, int32_t experts, int32_t* offsets,
                        int32_t* sorted_pairs, int32_t* table, hipStream_t stream) {
  if (experts <= 0 || experts > ROUTE_LDS_COUNTERS / 64) return hipErrorInvalidValue;
  if (npairs <= ROUTE_SMALL_PAIRS) {
    const int64_t t = npairs < 64 ? 64 : (npairs + 63) / 64 * 64;
    hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3((unsigned)t), 0, stream, ids,
                       (int32_t)npairs, experts, offsets, sorted_pairs);
    return hipGetLastError();
  }
  const int T = route_threads(experts);
  const int S = T >= experts ? T / experts : 1;
  const size_t lds = sizeof(int32_t) * ((size_t)T * experts + (size_t)S * experts + experts);
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&route_kernel),
                                    (int)(sizeof(int32_t) * (ROUTE_LDS_COUNTERS + 2 * 1024 + 512)),
                                    lds_set);
  if (e != hipSuccess) return e;
  if (table && route_table_entries(npairs, experts) > 0) {
    const int64_t chunk = route_chunk(npairs);
    const int64_t chunks = (npairs + chunk - 1) / chunk;  // <= ROUTE_MAX_CHUNKS
    hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)chunks), dim3(256), 0, stream, ids,
                       npairs, experts, chunk, table);
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(512), 0, stream, table, (int32_t)chunks,
                       experts, offsets);
    hipLaunchKernelGGL(route_kernel, dim3((unsigned)chunks), dim3(T), lds, stream, ids, npairs,
                       experts, offsets, sorted_pairs, (const int32_t*)table, chunk);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(T), lds, stream, ids, npairs, experts, offsets,
                     sorted_pairs, (const int32_t*)nullptr, (int64_t)0);
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
