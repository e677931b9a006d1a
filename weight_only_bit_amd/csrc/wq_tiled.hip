// wq_tiled.hip -- weight-only GEMM for many activation rows (prefill): LDS-staged exact-bf16
// weight tiles feeding bf16 MFMA.
//
// One workgroup = 8 waves computes a 256 (activation rows) x 128 (output channels) tile; K
// advances one 64-weight group per step.  Per step:
//   * the packed codes of the 128 x 64 weight tile are decoded once, by all 512 threads, to
//     the exact bf16 weights (the same bits wq_dequantize produces) and written to LDS; each
//     decoded weight is then used by 256 activation rows -- enough reuse that the decode's
//     VALU work (about 4.5 instructions per CCQ weight) stays below the MFMA time;
//   * the 256 x 64 bf16 activation tile is copied to LDS (gathered rows for MoE);
//   * each wave multiplies a 64 x 64 block with v_mfma_f32_32x32x16_bf16 (2 x 2 tiles x 4
//     k-steps), fp32 accumulation; waves whose rows are all past the end of a ragged tile skip
//     their MFMAs.
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

constexpr int BM = 256;            // activation rows per tile
constexpr int BN = 128;            // weight rows (output channels) per tile
constexpr int BK = 64;             // k per step (one group)
constexpr int NTHREADS = 512;      // 8 waves: 4 along rows x 2 along channels
constexpr int LPITCH = BK * 2 + 16;  // LDS row pitch in bytes (pad: conflict-free 16 B reads)
constexpr int A_BYTES = BM * LPITCH;
constexpr int B_BYTES = BN * LPITCH;

// Packed bytes one thread decodes per step: 16 weights (a quarter group) of one weight row.
template <int FMT>
struct PRaw {
  u32x2 codes;     // INT4: 8 bytes; 2-bit formats: first 4 bytes used
  uint32_t scale;  // CCQ: scale byte; INT4 g64 / affine: bf16 bits
  uint32_t zero;
};

struct RowInfo {
  const uint8_t* codes;  // row start
  const uint16_t* scales;
  const uint8_t* zeros;
  const uint8_t* qscale;
  float cs24, cz, fin24;  // CCQ code scale and super / INT4 per-channel scale, times 2^24
};

template <int FMT>
__device__ __forceinline__ RowInfo row_info(const DevWeight& w, int64_t e, int64_t row) {
  RowInfo r{};
  const int64_t n = w.n, k = w.k, G = k / 64, grow = e * n + row;
  r.fin24 = kTwo24;
  if (FMT == FMT_INT4) {
    r.codes = w.codes + grow * (k / 2);
    if (w.group)
      r.scales = w.scales + grow * G;
    else
      r.fin24 = bf16_bits_to_f32(w.scales[grow]) * kTwo24;
  } else if (FMT == FMT_AFFINE2) {
    r.codes = w.codes + grow * (k / 4);
    r.scales = w.scales + grow * G;
    r.zeros = w.zeros + grow * G;
  } else {
    r.codes = w.codes + grow * (k / 4);
    r.qscale = w.qscale + grow * ((G + 1) / 2);
    r.cs24 = w.code_scale[grow] * kTwo24;
    r.cz = w.code_zero[grow];
    r.fin24 = w.super_scale[grow] * kTwo24;
  }
  return r;
}

// Step `g` (group g), quarter `qt` (weights 16 qt .. 16 qt + 15 of the group) of one row.
template <int FMT>
__device__ __forceinline__ void pload(PRaw<FMT>& p, const RowInfo& r, int64_t g, int qt) {
  if (FMT == FMT_INT4) {
    p.codes = *reinterpret_cast<const u32x2*>(r.codes + g * 32 + qt * 8);
    p.scale = r.scales ? (uint32_t)r.scales[g] : 0u;
  } else if (FMT == FMT_AFFINE2) {
    p.codes.x = *reinterpret_cast<const uint32_t*>(r.codes + g * 16 + qt * 4);
    p.scale = r.scales[g];
    p.zero = r.zeros[g];
  } else {
    p.codes.x = *reinterpret_cast<const uint32_t*>(r.codes + g * 16 + qt * 4);
    p.scale = r.qscale[g >> 1];
  }
}

// Decode 16 weights into 8 bf16 pairs (k order).  mzp24 = -zp / 2^24 (CCQ).
template <int FMT>
__device__ __forceinline__ void pdecode(const PRaw<FMT>& p, const RowInfo& r, int64_t g,
                                        float mzp24, uint32_t (&o)[8]) {
  if (FMT == FMT_INT4) {
    const float s24 = r.scales ? bf16_bits_to_f32(p.scale & 0xFFFFu) * kTwo24 : r.fin24;
    int4_decode16(p.codes.x, p.codes.y, s24, s24 * (-8.0f / kTwo24), o);
  } else if (FMT == FMT_AFFINE2) {
    const float s = bf16_bits_to_f32(p.scale & 0xFFFFu);
    affine2_decode16(p.codes.x, s * kTwo24, -(float)(p.zero & 0xFFu) * s, o);
  } else {
    const float s24 = (float)((p.scale >> (4 * (g & 1))) & 0xFu) * r.fin24;
    ccq_decode16(p.codes.x, r.cs24, r.cz, s24, s24 * mzp24, o);
  }
}

template <int FMT, int MODE>
__global__ __launch_bounds__(NTHREADS) void tiled_kernel(const TiledArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // buffers: two activation tiles, then two decoded weight tiles
  auto As = [&](int buf) { return lds + buf * A_BYTES; };
  auto Bs = [&](int buf) { return lds + 2 * A_BYTES + buf * B_BYTES; };
  __shared__ int32_t s_tile[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave block: rows 64 wm (0..3), channels 64 wn

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

  // decode role: thread -> (weight tile row dr, quarter qt of the group)
  const int dr = tid >> 2, qt = tid & 3;
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
  const float mzp24 = -(float)args.w0.zp / kTwo24;

  // activation copy role: thread -> (tile row ar, half ah): 64 bytes
  const int ar = tid >> 1, ah = tid & 1;
  const bool wave_active = 64 * wm < rows;  // some of this wave's rows are real
  const uint16_t* arow = nullptr;
  if (ar < rows) {
    const int64_t r = row0 + ar;
    if constexpr (MODE == MODE_GATEUP)
      arow = args.a + (int64_t)(args.sorted_pairs[r] / args.topk) * args.a_stride;
    else
      arow = args.a + r * args.a_stride;
  }

  // One step's global data held in registers between its load and its LDS store.
  struct Stage {
    PRaw<FMT> pr;
    u32x4 xa[4];
  };
  auto load_step = [&](Stage& st, int64_t g) {
    pload<FMT>(st.pr, ri, g, qt);
    if (arow) {
      const u32x4* src = reinterpret_cast<const u32x4*>(arow + g * BK + ah * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.xa[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) st.xa[i] = (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto store_step = [&](const Stage& st, int64_t g, int buf) {
    uint32_t o[8];
    pdecode<FMT>(st.pr, ri, g, mzp24, o);
    u32x4* bd = reinterpret_cast<u32x4*>(Bs(buf) + dr * LPITCH + qt * 32);
    bd[0] = (u32x4){o[0], o[1], o[2], o[3]};
    bd[1] = (u32x4){o[4], o[5], o[6], o[7]};
    u32x4* ad = reinterpret_cast<u32x4*>(As(buf) + ar * LPITCH + ah * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = st.xa[i];
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

  auto mfma_step = [&](int buf) {
    if (!wave_active) return;
    u32x4 A[BK / 16][2], B[BK / 16][2];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        A[ks][i] = *reinterpret_cast<const u32x4*>(As(buf) + arow_l[i] * LPITCH + (ks * 16 + kh * 8) * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        B[ks][j] = *reinterpret_cast<const u32x4*>(Bs(buf) + brow_l[j] * LPITCH + (ks * 16 + kh * 8) * 2);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(A[ks][i], B[ks][j], acc[i][j]);
  };

  // Pipeline: while step g is multiplied from LDS buffer g & 1, step g + 1 (loaded one
  // iteration earlier) is decoded into the other buffer and step g + 2 is being loaded.
  Stage s0, s1;
  load_step(s0, 0);
  if (steps > 1) load_step(s1, 1);
  store_step(s0, 0, 0);
  __syncthreads();
  auto iter = [&](Stage& nxt, Stage& fut, int64_t g) {
    const int buf = (int)(g & 1);
    if (g + 2 < steps) load_step(fut, g + 2);  // `fut` was stored to LDS last iteration
    mfma_step(buf);
    if (g + 1 < steps) store_step(nxt, g + 1, buf ^ 1);
    __syncthreads();
  };
  for (int64_t g = 0; g < steps; g += 2) {
    iter(s1, s0, g);
    if (g + 1 < steps) iter(s0, s1, g + 1);
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
  constexpr size_t lds_bytes = 2 * (size_t)(A_BYTES + B_BYTES);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&tiled_kernel<FMT, MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t cols = (MODE == MODE_GATEUP) ? (a.N + 63) / 64 : (a.N + BN - 1) / BN;
  dim3 grid((unsigned)cols, (unsigned)row_tiles);
  hipLaunchKernelGGL((tiled_kernel<FMT, MODE>), grid, dim3(NTHREADS), lds_bytes, s, a);
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
