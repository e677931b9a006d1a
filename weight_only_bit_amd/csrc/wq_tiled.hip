// wq_tiled.hip -- weight-only GEMM for many activation rows (prefill): LDS-staged exact-bf16
// weight tiles feeding bf16 MFMA.
//
// One workgroup = 4 waves computes a 128 (activation rows) x 128 (output channels) tile; K
// advances one 64-weight group per step.  Per step:
//   * the packed codes of the 128 x 64 weight tile are decoded once, by all 256 threads, to
//     the exact bf16 weights (the same bits wq_dequantize produces) and written to LDS; each
//     decoded weight is then used by 128 activation rows;
//   * the 128 x 64 bf16 activation tile is copied to LDS (gathered rows for MoE);
//   * each wave multiplies a 64 x 64 quarter with v_mfma_f32_32x32x16_bf16 (2 x 2 tiles x 4
//     k-steps), fp32 accumulation.
// LDS is double-buffered: the next step's packed bytes and activations are loaded into
// registers before the current MFMAs are issued, and decoded/stored after them, so the
// decode's VALU work overlaps the matrix-core work.
//
// MoE gate+up: the 128 weight rows of a tile are 64 gate rows and the matching 64 up rows, so
// each lane holds gate and up results for the same (row, channel) and applies SiLU(g) * u in
// the epilogue.  MoE tiles are enumerated per expert (ceil(rows / 128) row tiles each); a
// workgroup finds its expert from the expert offsets.
#include <hip/hip_runtime.h>

#include "wq_kernels.hpp"

namespace wq {
namespace {

constexpr int BM = 128;            // activation rows per tile
constexpr int BN = 128;            // weight rows (output channels) per tile
constexpr int BK = 64;             // k per step (one group)
constexpr int LPITCH = BK * 2 + 16;  // LDS row pitch in bytes (pad: conflict-free 16 B reads)
constexpr int TILE_BYTES = 128 * LPITCH;

// Packed bytes one thread decodes per step: 32 weights of one weight row.
template <int FMT>
struct PRaw {
  u32x4 codes;     // INT4: 16 bytes; 2-bit formats: first 8 bytes used
  uint32_t scale;  // CCQ: scale byte; INT4 g64 / affine: bf16 bits
  uint32_t zero;
};

struct RowInfo {
  const uint8_t* codes;  // row start
  const uint16_t* scales;
  const uint8_t* zeros;
  const uint8_t* qscale;
  float cs, cz, fin;
};

template <int FMT>
__device__ __forceinline__ RowInfo row_info(const DevWeight& w, int64_t e, int64_t row) {
  RowInfo r{};
  const int64_t n = w.n, k = w.k, G = k / 64, grow = e * n + row;
  r.fin = 1.0f;
  if (FMT == FMT_INT4) {
    r.codes = w.codes + grow * (k / 2);
    if (w.group)
      r.scales = w.scales + grow * G;
    else
      r.fin = bf16_bits_to_f32(w.scales[grow]);
  } else if (FMT == FMT_AFFINE2) {
    r.codes = w.codes + grow * (k / 4);
    r.scales = w.scales + grow * G;
    r.zeros = w.zeros + grow * G;
  } else {
    r.codes = w.codes + grow * (k / 4);
    r.qscale = w.qscale + grow * ((G + 1) / 2);
    r.cs = w.code_scale[grow];
    r.cz = w.code_zero[grow];
    r.fin = w.super_scale[grow];
  }
  return r;
}

// Step `g` (group g), half `hf` (weights 32 hf .. 32 hf + 31 of the group) of one row.
template <int FMT>
__device__ __forceinline__ void pload(PRaw<FMT>& p, const RowInfo& r, int64_t g, int hf) {
  if (FMT == FMT_INT4) {
    p.codes = *reinterpret_cast<const u32x4*>(r.codes + g * 32 + hf * 16);
    p.scale = r.scales ? (uint32_t)r.scales[g] : 0u;
  } else if (FMT == FMT_AFFINE2) {
    const u32x2 c = *reinterpret_cast<const u32x2*>(r.codes + g * 16 + hf * 8);
    p.codes = (u32x4){c.x, c.y, 0u, 0u};
    p.scale = r.scales[g];
    p.zero = r.zeros[g];
  } else {
    const u32x2 c = *reinterpret_cast<const u32x2*>(r.codes + g * 16 + hf * 8);
    p.codes = (u32x4){c.x, c.y, 0u, 0u};
    p.scale = r.qscale[g >> 1];
  }
}

// Decode 32 weights into 16 bf16 pairs (k order).
template <int FMT>
__device__ __forceinline__ void pdecode(const PRaw<FMT>& p, const RowInfo& r, int64_t g,
                                        float zpf, uint32_t (&o)[16]) {
  uint32_t a[8], b[8];
  if (FMT == FMT_INT4) {
    const float s = r.scales ? bf16_bits_to_f32(p.scale & 0xFFFFu) : r.fin;
    int4_decode16(p.codes.x, p.codes.y, s, a);
    int4_decode16(p.codes.z, p.codes.w, s, b);
  } else if (FMT == FMT_AFFINE2) {
    const float s = bf16_bits_to_f32(p.scale & 0xFFFFu);
    const float mzs = -(float)(p.zero & 0xFFu) * s;
    affine2_decode16(p.codes.x, s, mzs, a);
    affine2_decode16(p.codes.y, s, mzs, b);
  } else {
    const float s = (float)((p.scale >> (4 * (g & 1))) & 0xFu) * r.fin;
    ccq_decode16(p.codes.x, r.cs, r.cz, s, -zpf * s, a);
    ccq_decode16(p.codes.y, r.cs, r.cz, s, -zpf * s, b);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o[i] = a[i];
    o[8 + i] = b[i];
  }
}

template <int FMT, int MODE>
__global__ __launch_bounds__(256) void tiled_kernel(const TiledArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // buffers: A tiles at lds + buf * TILE_BYTES, decoded weight tiles after them
  auto As = [&](int buf) { return lds + buf * TILE_BYTES; };
  auto Bs = [&](int buf) { return lds + (2 + buf) * TILE_BYTES; };
  __shared__ int32_t s_tile[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave quarter: rows 64 wm, columns 64 wn

  // ---- which rows: dense row tile, or (expert, row tile) from the expert offsets ----
  int64_t e = 0, row0, rows;
  if constexpr (MODE == MODE_DENSE) {
    row0 = (int64_t)blockIdx.y * BM;
    rows = args.M - row0 < BM ? args.M - row0 : BM;
  } else {
    if (tid == 0) {
      int64_t acc = 0;
      int found = -1;
      int64_t before = 0;
      for (int ex = 0; ex < args.experts; ++ex) {
        const int64_t c = args.offsets[ex + 1] - args.offsets[ex];
        const int64_t nt = (c + BM - 1) / BM;
        if ((int64_t)blockIdx.y < acc + nt) {
          found = ex;
          before = acc;
          break;
        }
        acc += nt;
      }
      s_tile[0] = found;
      s_tile[1] = (int32_t)((int64_t)blockIdx.y - before);
    }
    __syncthreads();
    if (s_tile[0] < 0) return;
    e = s_tile[0];
    const int64_t base = args.offsets[e];
    const int64_t cnt = args.offsets[e + 1] - base;
    row0 = base + (int64_t)s_tile[1] * BM;
    rows = base + cnt - row0 < BM ? base + cnt - row0 : BM;
  }

  // ---- weight rows this workgroup covers ----
  const int64_t N = args.N;
  const int64_t K = args.K;
  const int64_t steps = K / BK;
  // Weight tile row i (0..127): dense/down: channel n0 + i; gate+up: i < 64 -> gate row
  // n0 + i, else up row n0 + i - 64 (n0 = 64 * blockIdx.x).
  const int64_t n0 = (MODE == MODE_GATEUP) ? (int64_t)blockIdx.x * 64 : (int64_t)blockIdx.x * BN;

  // decode role: thread -> (tile row dr, half hf)
  const int dr = tid >> 1, hf = tid & 1;
  int64_t wrow;
  const DevWeight* wsrc;
  if constexpr (MODE == MODE_GATEUP) {
    wrow = n0 + (dr & 63);
    wsrc = (dr < 64) ? &args.w0 : &args.w1;
  } else {
    wrow = n0 + dr;
    wsrc = &args.w0;
  }
  const bool wvalid = wrow < N;
  const RowInfo ri = row_info<FMT>(*wsrc, e, wvalid ? wrow : N - 1);
  const float zpf = (float)args.w0.zp;

  // activation copy role: thread -> (tile row ar, half ah): 64 bytes
  const int ar = tid >> 1, ah = tid & 1;
  const uint16_t* arow = nullptr;
  if (ar < rows) {
    const int64_t r = row0 + ar;
    if constexpr (MODE == MODE_GATEUP)
      arow = args.a + (int64_t)(args.sorted_pairs[r] / args.topk) * args.a_stride;
    else
      arow = args.a + r * args.a_stride;
  }

  PRaw<FMT> pr;
  u32x4 xa[4];
  auto load_step = [&](int64_t g) {
    pload<FMT>(pr, ri, g, hf);
    if (arow) {
      const u32x4* src = reinterpret_cast<const u32x4*>(arow + g * BK + ah * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto store_step = [&](int64_t g, int buf) {
    uint32_t o[16];
    pdecode<FMT>(pr, ri, g, zpf, o);
    u32x4* bd = reinterpret_cast<u32x4*>(Bs(buf) + dr * LPITCH + hf * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) bd[i] = (u32x4){o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
    u32x4* ad = reinterpret_cast<u32x4*>(As(buf) + ar * LPITCH + ah * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = xa[i];
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // MFMA operand rows: A row 64 wm + 32 i + (lane % 32); B row (weight tile row):
  //   dense/down: 64 wn + 32 j + (lane % 32); gate+up: j = 0 -> gate row 32 wn + lane % 32,
  //   j = 1 -> the matching up row 64 + 32 wn + lane % 32.
  const int l32 = lane & 31, kh = lane >> 5;
  int arow_l[2], brow_l[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) arow_l[i] = 64 * wm + 32 * i + l32;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    brow_l[j] = (MODE == MODE_GATEUP) ? (64 * j + 32 * wn + l32) : (64 * wn + 32 * j + l32);

  load_step(0);
  store_step(0, 0);
  __syncthreads();
  for (int64_t g = 0; g < steps; ++g) {
    const int buf = (int)(g & 1);
    const bool more = g + 1 < steps;
    if (more) load_step(g + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 A[2], B[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        A[i] = *reinterpret_cast<const u32x4*>(As(buf) + arow_l[i] * LPITCH + (ks * 16 + kh * 8) * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        B[j] = *reinterpret_cast<const u32x4*>(Bs(buf) + brow_l[j] * LPITCH + (ks * 16 + kh * 8) * 2);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(A[i], B[j], acc[i][j]);
    }
    if (more) store_step(g + 1, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds D[8 (r/4) + 4 kh + r % 4][l32] of each 32 x 32 tile ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (m >= rows) continue;
      const int64_t grow = row0 + m;
      if constexpr (MODE == MODE_GATEUP) {
        const int64_t n = n0 + 32 * wn + l32;
        if (n >= N) continue;
        uint16_t* h = reinterpret_cast<uint16_t*>(args.out);
        h[grow * args.out_stride + n] = (uint16_t)f32_to_bf16_bits(silu_f32(acc[i][0][r]) * acc[i][1][r]);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t n = n0 + 64 * wn + 32 * j + l32;
          if (n >= N) continue;
          if constexpr (MODE == MODE_DENSE) {
            uint16_t* y = reinterpret_cast<uint16_t*>(args.out);
            y[grow * args.out_stride + n] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
          } else {
            float* d = reinterpret_cast<float*>(args.out);
            d[(int64_t)args.sorted_pairs[grow] * args.out_stride + n] = acc[i][j][r];
          }
        }
      }
    }
  }
}

template <int FMT, int MODE>
hipError_t launch_t(const TiledArgs& a, int64_t row_tiles, hipStream_t s) {
  constexpr size_t lds_bytes = 4 * (size_t)TILE_BYTES;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&tiled_kernel<FMT, MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t cols = (MODE == MODE_GATEUP) ? (a.N + 63) / 64 : (a.N + BN - 1) / BN;
  dim3 grid((unsigned)cols, (unsigned)row_tiles);
  hipLaunchKernelGGL((tiled_kernel<FMT, MODE>), grid, dim3(256), lds_bytes, s, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int fmt, const TiledArgs& a, int64_t row_tiles, hipStream_t s) {
  switch (fmt) {
    case FMT_INT4: return launch_t<FMT_INT4, MODE>(a, row_tiles, s);
    case FMT_AFFINE2: return launch_t<FMT_AFFINE2, MODE>(a, row_tiles, s);
    default: return launch_t<FMT_CCQ2, MODE>(a, row_tiles, s);
  }
}

}  // namespace

int tiled_rows() { return BM; }

hipError_t launch_tiled(int fmt, int mode, const TiledArgs& args, int64_t row_tiles,
                        hipStream_t stream) {
  if (row_tiles <= 0) return hipSuccess;
  if (mode == MODE_DENSE) return launch_mode<MODE_DENSE>(fmt, args, row_tiles, stream);
  if (mode == MODE_GATEUP) return launch_mode<MODE_GATEUP>(fmt, args, row_tiles, stream);
  return launch_mode<MODE_DOWN>(fmt, args, row_tiles, stream);
}

}  // namespace wq
