// wq_skinny.hip -- decode-streaming weight-only GEMM for few activation rows (<= 32 per pass).
//
// Every packed weight byte is read from HBM once per pass and decoded in registers straight
// into MFMA B-operand fragments (exact bf16 weights, see wq_device.hpp); nothing decoded goes
// through LDS or memory.
//
// Work layout (one workgroup = 4 waves of 64):
//   * a wave owns a 16-row tile of output channels (n) and, with KSPLIT = 4, a quarter of K;
//   * the activation rows (16 or 32) are staged in LDS in 512-column chunks, double-buffered,
//     shared by the 4 waves (16-byte row padding keeps the fragment reads conflict-free);
//   * packed codes and group scales of the next chunk are prefetched into registers while the
//     current chunk is multiplied;
//   * per 64-weight group a lane decodes 16 weights of its row (one CCQ dword, two INT4 dwords
//     or one 2-bit dword) into two 8-value B fragments and issues two 16x16x32 MFMAs per
//     16-row activation tile; fp32 accumulation; one bf16 rounding in the epilogue.
#include <hip/hip_runtime.h>

#include "wq_kernels.hpp"

namespace wq {
namespace {

constexpr int KCT = 512;  // activation columns per LDS chunk (all K-parts together)

template <int FMT>
struct Raw;  // packed bytes + group metadata of one 64-weight group, one lane
template <>
struct Raw<FMT_INT4> {
  u32x2 codes;
  uint32_t scale;
};
template <>
struct Raw<FMT_AFFINE2> {
  uint32_t codes;
  uint32_t scale;
  uint32_t zero;
};
template <>
struct Raw<FMT_CCQ2> {
  uint32_t codes;
  uint32_t qs;
};

// Per-lane, per-matrix row constants.
struct RowConst {
  const uint8_t* codes;    // row start
  const uint16_t* scales;  // row start (INT4 g64 / AFFINE)
  const uint8_t* zeros;    // row start (AFFINE)
  const uint8_t* qscale;   // row start (CCQ)
  float cs, cz;            // CCQ code scale / zero
  float fin;               // CCQ super scale / INT4 per-channel scale (else 1)
};

__device__ __forceinline__ DevWeight at_expert(const DevWeight& w, int fmt, int64_t e) {
  DevWeight r = w;
  const int64_t G = w.k / 64;
  const int64_t rows = e * w.n;
  if (fmt == FMT_INT4) {
    r.codes = w.codes + rows * (w.k / 2);
    r.scales = w.scales + (w.group ? rows * G : rows);
  } else if (fmt == FMT_AFFINE2) {
    r.codes = w.codes + rows * (w.k / 4);
    r.scales = w.scales + rows * G;
    r.zeros = w.zeros + rows * G;
  } else {
    r.codes = w.codes + rows * (w.k / 4);
    r.qscale = w.qscale + rows * ((G + 1) / 2);
    r.super_scale = w.super_scale + rows;
    r.code_scale = w.code_scale + rows;
    r.code_zero = w.code_zero + rows;
  }
  return r;
}

template <int FMT>
__device__ __forceinline__ RowConst row_const(const DevWeight& w, int64_t row) {
  RowConst c;
  const int64_t G = w.k / 64;
  c.cs = 0.f;
  c.cz = 0.f;
  c.fin = 1.0f;
  c.scales = nullptr;
  c.zeros = nullptr;
  c.qscale = nullptr;
  if (FMT == FMT_INT4) {
    c.codes = w.codes + row * (w.k / 2);
    if (w.group)
      c.scales = w.scales + row * G;
    else
      c.fin = bf16_bits_to_f32(w.scales[row]);
  } else if (FMT == FMT_AFFINE2) {
    c.codes = w.codes + row * (w.k / 4);
    c.scales = w.scales + row * G;
    c.zeros = w.zeros + row * G;
  } else {
    c.codes = w.codes + row * (w.k / 4);
    c.qscale = w.qscale + row * ((G + 1) / 2);
    c.cs = w.code_scale[row];
    c.cz = w.code_zero[row];
    c.fin = w.super_scale[row];
  }
  return c;
}

// Load one group's packed data for this lane: weights k0 + 16*kb .. +15 of its row.
template <int FMT>
__device__ __forceinline__ void load_raw(Raw<FMT>& r, const RowConst& c, int64_t k0, int kb,
                                         bool per_channel) {
  const int64_t g = k0 >> 6;
  if constexpr (FMT == FMT_INT4) {
    r.codes = *reinterpret_cast<const u32x2*>(c.codes + (k0 >> 1) + kb * 8);
    r.scale = per_channel ? 0u : (uint32_t)c.scales[g];
  } else if constexpr (FMT == FMT_AFFINE2) {
    r.codes = *reinterpret_cast<const uint32_t*>(c.codes + (k0 >> 2) + kb * 4);
    r.scale = c.scales[g];
    r.zero = c.zeros[g];
  } else {
    r.codes = *reinterpret_cast<const uint32_t*>(c.codes + (k0 >> 2) + kb * 4);
    r.qs = c.qscale[g >> 1];
  }
}

template <int FMT, int MT, int NWN, int KSPLIT, int MODE>
__global__ __launch_bounds__(256) void skinny_kernel(const SkinnyArgs args) {
  constexpr int KCW = KCT / KSPLIT;  // columns per wave per chunk
  constexpr int GPC = KCW / 64;      // groups per wave per chunk
  constexpr int ROWS = MT * 16;
  constexpr int PITCH = KCT * 2 + 16;  // bytes per LDS row (16 B pad: conflict-free reads)
  constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
  constexpr int BLOCKS = ROWS * (KCT / 16);  // 16-element blocks per chunk
  constexpr int BPT = BLOCKS / 256;          // blocks staged per thread
  static_assert(BPT * 256 == BLOCKS, "staging must divide evenly");
  static_assert(NWN * KSPLIT == 4, "4 waves per workgroup");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  uint8_t(*lds)[ROWS * PITCH] = reinterpret_cast<uint8_t(*)[ROWS * PITCH]>(lds_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % NWN;
  const int kw = wave / NWN;
  const int nl = lane & 15;
  const int kb = lane >> 4;

  const int64_t N = args.N, K = args.K;
  const int64_t Kpp = K / KSPLIT;
  const int nchunks = (int)((Kpp + KCW - 1) / KCW);

  // Rows of this workgroup's activation block.
  int64_t m_base, m_total;
  if constexpr (MODE == MODE_DENSE) {
    m_base = (int64_t)blockIdx.z * ROWS;
    m_total = args.M - m_base;
    if (m_total > ROWS) m_total = ROWS;
  } else {
    const int e = blockIdx.y;
    m_base = args.offsets[e];
    m_total = args.offsets[e + 1] - m_base;
    if (m_total <= 0) return;
  }

  // Weights of this wave's 16-row tile.
  DevWeight W0 = args.w0, W1 = args.w1;
  if constexpr (MODE != MODE_DENSE) {
    W0 = at_expert(args.w0, FMT, blockIdx.y);
    if constexpr (NMAT == 2) W1 = at_expert(args.w1, FMT, blockIdx.y);
  }
  const int64_t n0 = ((int64_t)blockIdx.x * NWN + wn) * 16;
  const int64_t nrow = n0 + nl;
  const bool nvalid = nrow < N;
  const int64_t nr = nvalid ? nrow : (N - 1);
  RowConst rc[NMAT];
  rc[0] = row_const<FMT>(W0, nr);
  if constexpr (NMAT == 2) rc[1] = row_const<FMT>(W1, nr);
  const bool per_channel = (FMT == FMT_INT4) && (W0.group == 0);

  const float zpf = (float)W0.zp;

  // m super-tiles (one for dense; as many as the expert needs for MoE).
  for (int64_t ms = 0; ms < m_total; ms += ROWS) {
    const int64_t rows_here = (m_total - ms) < ROWS ? (m_total - ms) : ROWS;

    // Source row pointers of the blocks this thread stages (fixed across chunks).
    const uint16_t* srow[BPT];
    int sblk[BPT];
    int srowi[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int b = tid + 256 * i;
      const int row = b / (KCT / 16);
      sblk[i] = b % (KCT / 16);
      srowi[i] = row;
      srow[i] = nullptr;
      if (row < rows_here) {
        const int64_t r = m_base + ms + row;
        if constexpr (MODE == MODE_GATEUP)
          srow[i] = args.a + (int64_t)(args.sorted_pairs[r] / args.topk) * args.a_stride;
        else
          srow[i] = args.a + r * args.a_stride;
      }
    }

    u32x4 xr[BPT][2];
    auto stage_load = [&](int c) {
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        const int part = sblk[i] / (KCW / 16);
        const int64_t kin = (int64_t)c * KCW + (sblk[i] % (KCW / 16)) * 16;
        if (srow[i] != nullptr && kin < Kpp) {
          const u32x4* p = reinterpret_cast<const u32x4*>(srow[i] + part * Kpp + kin);
          xr[i][0] = p[0];
          xr[i][1] = p[1];
        } else {
          xr[i][0] = (u32x4){0, 0, 0, 0};
          xr[i][1] = (u32x4){0, 0, 0, 0};
        }
      }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        u32x4* d = reinterpret_cast<u32x4*>(&lds[buf][srowi[i] * PITCH + sblk[i] * 32]);
        d[0] = xr[i][0];
        d[1] = xr[i][1];
      }
    };

    f32x4 acc[NMAT][MT];
#pragma unroll
    for (int q = 0; q < NMAT; ++q)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[q][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    Raw<FMT> rawA[NMAT][GPC], rawB[NMAT][GPC];
    const int64_t kpart0 = (int64_t)kw * Kpp;
    auto load_chunk = [&](Raw<FMT>(&r)[NMAT][GPC], int c) {
#pragma unroll
      for (int gi = 0; gi < GPC; ++gi) {
        const int64_t kin = (int64_t)c * KCW + gi * 64;
        if (kin < Kpp) {
#pragma unroll
          for (int q = 0; q < NMAT; ++q) load_raw<FMT>(r[q][gi], rc[q], kpart0 + kin, kb, per_channel);
        }
      }
    };

    auto compute_chunk = [&](Raw<FMT>(&r)[NMAT][GPC], int c, int buf) {
#pragma unroll
      for (int gi = 0; gi < GPC; ++gi) {
        const int64_t kin = (int64_t)c * KCW + gi * 64;
        if (kin >= Kpp) break;
        // A fragments: rows t*16 + nl, block (kw part, group gi, kb), halves h
        u32x4 A[MT][2];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint8_t* base = &lds[buf][(t * 16 + nl) * PITCH + (kw * (KCW / 16) + gi * 4 + kb) * 32];
          A[t][0] = *reinterpret_cast<const u32x4*>(base);
          A[t][1] = *reinterpret_cast<const u32x4*>(base + 16);
        }
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
          const Raw<FMT>& rw = r[q][gi];
          uint32_t p[8];
          if constexpr (FMT == FMT_CCQ2) {
            const int64_t g = (kpart0 + kin) >> 6;
            const float s = (float)((rw.qs >> (4 * (g & 1))) & 0xFu) * rc[q].fin;
            ccq_decode16(rw.codes, rc[q].cs, rc[q].cz, s, -zpf * s, p);
          } else if constexpr (FMT == FMT_INT4) {
            const float s = per_channel ? rc[q].fin : bf16_bits_to_f32(rw.scale);
            int4_decode16(rw.codes.x, rw.codes.y, s, p);
          } else {
            const float s = bf16_bits_to_f32(rw.scale);
            affine2_decode16(rw.codes, s, -(float)rw.zero * s, p);
          }
          const u32x4 B0 = {p[0], p[1], p[2], p[3]};
          const u32x4 B1 = {p[4], p[5], p[6], p[7]};
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            acc[q][t] = mfma16x16x32(A[t][0], B0, acc[q][t]);
            acc[q][t] = mfma16x16x32(A[t][1], B1, acc[q][t]);
          }
        }
      }
    };

    // Prologue: chunk 0's weights and activations.
    load_chunk(rawA, 0);
    stage_load(0);
    stage_store(0);
    __syncthreads();

    auto step = [&](Raw<FMT>(&cur)[NMAT][GPC], Raw<FMT>(&nxt)[NMAT][GPC], int c, int buf) {
      const bool more = (c + 1) < nchunks;
      if (more) {
        load_chunk(nxt, c + 1);
        stage_load(c + 1);
      }
      compute_chunk(cur, c, buf);
      if (more) stage_store(buf ^ 1);
      __syncthreads();
    };
    for (int c = 0; c < nchunks; c += 2) {
      step(rawA, rawB, c, 0);
      if (c + 1 < nchunks) step(rawB, rawA, c + 1, 1);
    }

    // Sum the K-parts in order (waves kw = 1..KSPLIT-1 into kw = 0) through LDS.
    if constexpr (KSPLIT > 1) {
      f32x4* red = reinterpret_cast<f32x4*>(&lds[0][0]);
      if (kw > 0) {
#pragma unroll
        for (int q = 0; q < NMAT; ++q)
#pragma unroll
          for (int t = 0; t < MT; ++t)
            red[(((kw - 1) * NWN + wn) * NMAT * MT + q * MT + t) * 64 + lane] = acc[q][t];
      }
      __syncthreads();
      if (kw == 0) {
#pragma unroll
        for (int p = 1; p < KSPLIT; ++p)
#pragma unroll
          for (int q = 0; q < NMAT; ++q)
#pragma unroll
            for (int t = 0; t < MT; ++t)
              acc[q][t] += red[(((p - 1) * NWN + wn) * NMAT * MT + q * MT + t) * 64 + lane];
      }
      __syncthreads();
    }

    // Epilogue: lane holds rows t*16 + 4*kb + i (i = 0..3) of column nrow.
    if (kw == 0 && nvalid) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = t * 16 + 4 * kb + i;
          if (m >= rows_here) continue;
          const int64_t r = m_base + ms + m;
          if constexpr (MODE == MODE_DENSE) {
            uint16_t* y = reinterpret_cast<uint16_t*>(args.out);
            y[r * args.out_stride + nrow] = (uint16_t)f32_to_bf16_bits(acc[0][t][i]);
          } else if constexpr (MODE == MODE_GATEUP) {
            const float gv = acc[0][t][i];
            const float uv = acc[1][t][i];
            uint16_t* h = reinterpret_cast<uint16_t*>(args.out);
            h[r * args.out_stride + nrow] = (uint16_t)f32_to_bf16_bits(silu_f32(gv) * uv);
          } else {
            float* d = reinterpret_cast<float*>(args.out);
            const int64_t pair = args.sorted_pairs[r];
            d[pair * args.out_stride + nrow] = acc[0][t][i];
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int FMT, int MT, int NWN, int KSPLIT, int MODE>
hipError_t launch_one(const SkinnyArgs& a, int64_t gy, int64_t gz, hipStream_t s) {
  constexpr size_t lds_bytes = 2 * (size_t)(MT * 16) * (KCT * 2 + 16);
  static bool attr_set = false;  // per instantiation; the attribute is per-function state
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&skinny_kernel<FMT, MT, NWN, KSPLIT, MODE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t ntiles = (a.N + 15) / 16;
  dim3 grid((unsigned)((ntiles + NWN - 1) / NWN), (unsigned)gy, (unsigned)gz);
  hipLaunchKernelGGL((skinny_kernel<FMT, MT, NWN, KSPLIT, MODE>), grid, dim3(256), lds_bytes, s, a);
  return hipGetLastError();
}

template <int FMT, int MODE>
hipError_t launch_fmt(int mt, int ksplit, const SkinnyArgs& a, int64_t gy, int64_t gz,
                      hipStream_t s) {
  if (ksplit == 4) {
    if (mt == 1) return launch_one<FMT, 1, 1, 4, MODE>(a, gy, gz, s);
    return launch_one<FMT, 2, 1, 4, MODE>(a, gy, gz, s);
  }
  if (mt == 1) return launch_one<FMT, 1, 4, 1, MODE>(a, gy, gz, s);
  return launch_one<FMT, 2, 4, 1, MODE>(a, gy, gz, s);
}

template <int MODE>
hipError_t launch_mode(int fmt, int mt, int ksplit, const SkinnyArgs& a, int64_t gy, int64_t gz,
                       hipStream_t s) {
  switch (fmt) {
    case FMT_INT4: return launch_fmt<FMT_INT4, MODE>(mt, ksplit, a, gy, gz, s);
    case FMT_AFFINE2: return launch_fmt<FMT_AFFINE2, MODE>(mt, ksplit, a, gy, gz, s);
    default: return launch_fmt<FMT_CCQ2, MODE>(mt, ksplit, a, gy, gz, s);
  }
}

}  // namespace

hipError_t launch_skinny(int fmt, int mode, int m_tiles, int ksplit, const SkinnyArgs& args,
                         int64_t grid_y, int64_t grid_z, hipStream_t stream) {
  if (mode == MODE_DENSE) return launch_mode<MODE_DENSE>(fmt, m_tiles, ksplit, args, grid_y, grid_z, stream);
  if (mode == MODE_GATEUP) return launch_mode<MODE_GATEUP>(fmt, m_tiles, 1, args, grid_y, grid_z, stream);
  return launch_mode<MODE_DOWN>(fmt, m_tiles, 1, args, grid_y, grid_z, stream);
}

}  // namespace wq
