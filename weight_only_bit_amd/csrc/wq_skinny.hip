// wq_skinny.hip -- decode-streaming weight-only GEMM for few activation rows (<= 32 per pass).
//
// Every packed weight byte is read from HBM once per pass and decoded in registers straight
// into MFMA B-operand fragments (exact bf16 weights, see wq_device.hpp); nothing decoded goes
// through LDS or memory.  The decode is VALU work (about 2.8 instructions per CCQ weight), so
// the layout aims at keeping every SIMD's VALU busy:
//
//   * one workgroup = 4 waves of 64; each wave decodes ONE weight matrix for a 16-row tile of
//     output channels (MoE gate+up: two waves take gate tiles, two take the matching up tiles;
//     their results meet in LDS for the SiLU(gate) * up epilogue);
//   * packed codes and group scales are read with buffer loads from a per-wave resource (the
//     lane's row offset is computed once; the step offset is a scalar), one chunk ahead of the
//     decode.  Each lane loads 16 contiguous bytes of its row per step -- one 64-weight group
//     of 2-bit codes or half a group of INT4 -- and the 4 lanes of a row take consecutive
//     pieces, so a wave's load covers 64 contiguous bytes of each of its 16 rows and a lane
//     needs one group scale per step.  (With exact bf16 weights the MFMA k-slots need not
//     follow group boundaries.)
//   * the activation rows (16 or 32) are staged in LDS in 512-column chunks, double-buffered
//     and shared by the 4 waves; a 16-byte row pad keeps the A-fragment reads conflict-free;
//   * per step a lane decodes its 64 (INT4: 32) weights 16 at a time into 8-value B fragments,
//     each feeding one 16x16x32 MFMA per 16-row activation tile; fp32 accumulation, one bf16
//     rounding in the epilogue;
//   * dense products with few output tiles split K over the 4 waves (summed in LDS, in order).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "wq_kernels.hpp"

namespace wq {
namespace {

constexpr int KCT_BASE = 512;  // activation columns per LDS chunk (all K-parts together)
constexpr int FMT_INT4PC = 8;  // INT4 with one scale per output channel (kernel variant)
constexpr int FMT_INT8PC = 9;  // INT8 with one scale per output channel (kernel variant)

__host__ __device__ constexpr bool is_int4(int f) { return f == FMT_INT4 || f == FMT_INT4PC; }
__host__ __device__ constexpr bool is_int8(int f) { return f == FMT_INT8 || f == FMT_INT8PC; }

// Weights one lane decodes per step: 16 bytes of codes, or one group of the CCQ formats
// without code cluster (22 or 20 bytes).
template <int FMT>
__host__ __device__ constexpr int lane_weights() { return is_int8(FMT) ? 16 : is_int4(FMT) ? 32 : 64; }

// Columns per wave per LDS chunk: at least one step (4 lanes x lane_weights).
template <int FMT, int KSPLIT>
__host__ __device__ constexpr int chunk_cols() {
  return (KCT_BASE / KSPLIT) > 4 * lane_weights<FMT>() ? KCT_BASE / KSPLIT : 4 * lane_weights<FMT>();
}

// Packed data of one step for one lane: 16 bytes of its row and its group's scale.
template <int FMT>
struct Raw {
  u32x4 codes;
  uint32_t scale;  // CCQ: the byte holding the 4-bit group scale; INT4 g64 / affine: bf16 bits
  uint32_t zero;   // affine zero point
  u32x2 extra;     // (4,3,2): code bytes 16..23 of the aligned window; hybrid: bytes 16..19
};

// A byte range of one expert's array.  A load at step offset `off` goes through a resource
// whose base is advanced by `off` (scalar arithmetic) and whose range shrinks by it, so the
// range check covers the whole offset and a load past the array reads zeros.
// Sizes are below 2^31 (the host checks one expert's arrays and k), so the range arithmetic is
// 32-bit and stays on the scalar unit.
struct BufView {
  const uint8_t* base;
  int32_t bytes;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc32(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes > 0 ? bytes : 0,
                                           0x00020000);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t at(const BufView& b, int32_t off) {
  return make_rsrc32(b.base + off, b.bytes - off);
}

__device__ __forceinline__ BufView view(const void* base, int64_t bytes) {
  return BufView{reinterpret_cast<const uint8_t*>(base), (int32_t)(bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0ll : bytes)};
}

// Per-wave view of one weight matrix (one expert); loads go through buffer resources, so an
// offset outside the matrix reads zeros instead of faulting.
template <int FMT>
struct WaveW {
  BufView codes, scales, zeros;
  int32_t row_codes;   // byte offset of this lane's row and 16-weight slice in codes
  int32_t row_scales;  // byte offset of this lane's row in scales / qscale
  int32_t row_zeros;
  uint32_t qshift;     // CCQ: 0 or 4, the nibble of the scale byte that is this lane's group;
                       // (4,3,2): 0 or 16, the bit offset of the group in its first dword
  float cs, cz;        // CCQ code scale / code zero of this lane's row
  float fin;           // CCQ super scale / INT4 per-channel scale of this lane's row
};

// gb: first group of the wave's K range (its steps start at k = 64 gb).
template <int FMT>
__device__ __forceinline__ WaveW<FMT> wave_weight(const DevWeight& w, int64_t e, int64_t row,
                                                  int kb, int32_t gb) {
  WaveW<FMT> v;
  const int64_t n = w.n, k = w.k, G = k / 64;
  v.qshift = 0;
  v.cs = v.cz = 0.f;
  v.fin = 1.0f;
  v.row_scales = v.row_zeros = 0;
  v.zeros = v.scales = view(w.codes, 0);
  if constexpr (is_int4(FMT)) {
    v.codes = view(w.codes + e * n * (k / 2), n * (k / 2));
    v.row_codes = (int32_t)(row * (k / 2) + gb * 32 + kb * 16);
    if constexpr (FMT == FMT_INT4) {  // lane kb's 32 weights of step j lie in group gb + 2 j + kb / 2
      v.scales = view(w.scales + e * n * G, n * G * 2);
      v.row_scales = (int32_t)(row * G * 2 + (gb + (kb >> 1)) * 2);
    } else {
      v.fin = bf16_bits_to_f32(w.scales[e * n + row]);
    }
  } else if constexpr (is_int8(FMT)) {
    // a step is one group: lane kb holds weights 16 kb .. 16 kb + 15 of group gb + j
    v.codes = view(w.codes + e * n * k, n * k);
    v.row_codes = (int32_t)(row * k + gb * 64 + kb * 16);
    if constexpr (FMT == FMT_INT8) {
      v.scales = view(w.scales + e * n * G, n * G * 2);
      v.row_scales = (int32_t)(row * G * 2 + gb * 2);
    } else {
      v.fin = bf16_bits_to_f32(w.scales[e * n + row]);
    }
  } else if constexpr (FMT == FMT_AFFINE2) {
    v.codes = view(w.codes + e * n * (k / 4), n * (k / 4));
    v.row_codes = (int32_t)(row * (k / 4) + gb * 16 + kb * 16);  // group gb + 4 j + kb
    v.scales = view(w.scales + e * n * G, n * G * 2);
    v.row_scales = (int32_t)(row * G * 2 + (gb + kb) * 2);
    v.zeros = view(w.zeros + e * n * G, n * G);
    v.row_zeros = (int32_t)(row * G + gb + kb);
  } else if constexpr (is_alg2(FMT)) {
    // A group is 22 (or 20) bytes: lane kb's group gb + 4 j + kb starts at an even byte.  Loads
    // read the dword-aligned window that holds it (the resource starts at the expert's first
    // dword and ends at the dword holding its last byte, so the window stays in that dword).
    constexpr int GB = alg2_group_bytes(FMT);
    const uint8_t* eb = w.codes + e * n * G * GB;
    const int64_t lead = (int64_t)(reinterpret_cast<uintptr_t>(eb) & 3u);
    v.codes = view(eb - lead, (lead + n * G * GB + 3) & ~(int64_t)3);
    const int64_t off = lead + row * G * GB + (int64_t)(gb + kb) * GB;
    v.qshift = 8u * (uint32_t)(off & 3);
    v.row_codes = (int32_t)(off & ~(int64_t)3);
    v.fin = w.super_scale[e * n + row];
  } else {
    const int64_t qb = (G + 1) / 2;
    v.codes = view(w.codes + e * n * (k / 4), n * (k / 4));
    v.row_codes = (int32_t)(row * (k / 4) + gb * 16 + kb * 16);  // group gb + 4 j + kb
    v.scales = view(w.qscale + e * n * qb, n * qb);
    v.row_scales = (int32_t)(row * qb + ((gb + kb) >> 1));  // two 4-bit scales per byte
    v.qshift = 4u * (uint32_t)((gb + kb) & 1);
    v.cs = w.code_scale[e * n + row];
    v.cz = w.code_zero[e * n + row];
    v.fin = w.super_scale[e * n + row];
  }
  return v;
}

// Load step st of the wave's K range (k = 64 gb + st * 4 * lane_weights) for this lane's row.
// st is wave-uniform and goes in the scalar offset.
template <int FMT>
__device__ __forceinline__ void load_raw(Raw<FMT>& r, const WaveW<FMT>& v, int32_t st) {
  if constexpr (is_alg2(FMT)) {  // a step advances 4 groups: 88 or 80 bytes, dword aligned
    constexpr int STEP = 4 * alg2_group_bytes(FMT);
    r.codes = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(at(v.codes, st * STEP), v.row_codes, 0, 0));
    if constexpr (FMT == FMT_CCQ432)
      r.extra = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(at(v.codes, st * STEP), v.row_codes + 16, 0, 0));
    else
      r.extra.x = __builtin_amdgcn_raw_buffer_load_b32(at(v.codes, st * STEP), v.row_codes + 16, 0, 0);
    return;
  }
  r.codes = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(at(v.codes, st * 64), v.row_codes, 0, 0));
  if constexpr (FMT == FMT_INT8) {
    r.scale = __builtin_amdgcn_raw_buffer_load_b16(at(v.scales, st * 2), v.row_scales, 0, 0);
  } else if constexpr (FMT == FMT_INT4) {
    r.scale = __builtin_amdgcn_raw_buffer_load_b16(at(v.scales, st * 4), v.row_scales, 0, 0);
  } else if constexpr (FMT == FMT_AFFINE2) {
    r.scale = __builtin_amdgcn_raw_buffer_load_b16(at(v.scales, st * 8), v.row_scales, 0, 0);
    r.zero = __builtin_amdgcn_raw_buffer_load_b8(at(v.zeros, st * 4), v.row_zeros, 0, 0);
  } else if constexpr (FMT == FMT_CCQ2) {
    r.scale = __builtin_amdgcn_raw_buffer_load_b8(at(v.scales, st * 2), v.row_scales, 0, 0);
  }
}

// One step of one lane: decode its packed data rw (WPL weights of its row) into B fragments and
// multiply them with the A fragments at abase (LDS: the lane's activation row at the step's
// first column of this lane; tile t of 16 rows at abase + t * tpitch) into acc.
template <int FMT, int MT, bool CLAMP>
__device__ __forceinline__ void step_mma(const Raw<FMT>& rw, const WaveW<FMT>& W, float cs24,
                                         float fin24, float mzp24, const uint8_t* abase,
                                         int tpitch, f32x4 (&acc)[MT]) {
  constexpr int WPL = lane_weights<FMT>();
  if constexpr (is_alg2(FMT)) {
    uint32_t p[32];
    if constexpr (FMT == FMT_CCQ432) {
      // shift the window so that the group starts at byte 0
      const uint32_t w6[6] = {rw.codes[0], rw.codes[1], rw.codes[2], rw.codes[3],
                              rw.extra.x, rw.extra.y};
      uint32_t c[6];
#pragma unroll
      for (int i = 0; i < 5; ++i) c[i] = __builtin_amdgcn_alignbit(w6[i + 1], w6[i], W.qshift);
      c[5] = w6[5] >> W.qshift;
      ccq432_decode64(c, fin24, mzp24, p);
    } else {
      const uint32_t c[5] = {rw.codes[0], rw.codes[1], rw.codes[2], rw.codes[3], rw.extra.x};
      ccqh_decode64(c, fin24, mzp24, p);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 B0 = {p[8 * q], p[8 * q + 1], p[8 * q + 2], p[8 * q + 3]};
      const u32x4 B1 = {p[8 * q + 4], p[8 * q + 5], p[8 * q + 6], p[8 * q + 7]};
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const u32x4 A0 = *reinterpret_cast<const u32x4*>(abase + t * tpitch + q * 32);
        const u32x4 A1 =
            *reinterpret_cast<const u32x4*>(abase + t * tpitch + q * 32 + 16);
        acc[t] = mfma16x16x32(A0, B0, acc[t]);
        acc[t] = mfma16x16x32(A1, B1, acc[t]);
      }
    }
    return;
  }
  // s24 = s * 2^24 (the decode helpers' scaled form), mzs = -z * s
  float s24 = 0.0f, mzs = 0.0f;
  if constexpr (FMT == FMT_CCQ2) {
    s24 = (float)((rw.scale >> W.qshift) & 0xFu) * fin24;  // = fl(s_q * super) * 2^24
    mzs = s24 * mzp24;
  } else if constexpr (FMT == FMT_INT4) {
    s24 = bf16_bits_to_f32(rw.scale & 0xFFFFu) * kTwo24;
    mzs = s24 * (-8.0f / kTwo24);
  } else if constexpr (FMT == FMT_INT4PC) {
    s24 = fin24;
    mzs = fin24 * (-8.0f / kTwo24);
  } else if constexpr (FMT == FMT_INT8) {
    s24 = bf16_bits_to_f32(rw.scale & 0xFFFFu) * kTwo24;
    mzs = s24 * (-128.0f / kTwo24);
  } else if constexpr (FMT == FMT_INT8PC) {
    s24 = fin24;
    mzs = fin24 * (-128.0f / kTwo24);
  } else {
    const float s = bf16_bits_to_f32(rw.scale & 0xFFFFu);
    s24 = s * kTwo24;
    mzs = -(float)(rw.zero & 0xFFu) * s;
  }
  // 16 weights (two MFMAs) at a time
#pragma unroll
  for (int q = 0; q < WPL / 16; ++q) {
    uint32_t p[8];
    if constexpr (FMT == FMT_CCQ2) {
      ccq_decode16<CLAMP>(rw.codes[q], cs24, W.cz, s24, mzs, p);
    } else if constexpr (is_int4(FMT)) {
      int4_decode16(rw.codes[2 * q], rw.codes[2 * q + 1], s24, mzs, p);
    } else if constexpr (is_int8(FMT)) {
      int8_decode16(rw.codes, s24, mzs, p);
    } else {
      affine2_decode16(rw.codes[q], s24, mzs, p);
    }
    const u32x4 B0 = {p[0], p[1], p[2], p[3]};
    const u32x4 B1 = {p[4], p[5], p[6], p[7]};
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const u32x4 A0 = *reinterpret_cast<const u32x4*>(abase + t * tpitch + q * 32);
      const u32x4 A1 = *reinterpret_cast<const u32x4*>(abase + t * tpitch + q * 32 + 16);
      acc[t] = mfma16x16x32(A0, B0, acc[t]);
      acc[t] = mfma16x16x32(A1, B1, acc[t]);
    }
  }
}

template <int FMT, int MT, int MODE, int KSPLIT>
__global__ __launch_bounds__(256) void skinny_kernel(const SkinnyArgs args) {
  constexpr int WPL = lane_weights<FMT>();     // weights per lane per step
  constexpr int SSK = 4 * WPL;                 // k per step
  constexpr int KCW = chunk_cols<FMT, KSPLIT>();  // columns per wave per chunk
  constexpr int KCT = KCW * KSPLIT;
  constexpr int SPC = KCW / SSK;               // steps per wave per chunk
  constexpr int ROWS = MT * 16;
  constexpr int PITCH = KCT * 2 + 16;  // bytes per LDS row
  static_assert(MODE == MODE_DENSE || KSPLIT == 1, "K split is for dense products");
  constexpr int TPW = (KSPLIT == 4) ? 1 : (MODE == MODE_GATEUP ? 2 : 4);  // tiles per workgroup

  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  uint8_t(*lds)[ROWS * PITCH] = reinterpret_cast<uint8_t(*)[ROWS * PITCH]>(lds_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15;
  const int kb = lane >> 4;
  const int kw = (KSPLIT == 4) ? wave : 0;
  const int mat = (MODE == MODE_GATEUP) ? (wave >> 1) : 0;
  const int tile_in_wg = (KSPLIT == 4) ? 0 : (MODE == MODE_GATEUP ? (wave & 1) : wave);

  const int64_t N = args.N;
  const int32_t Kpp = (int32_t)(args.K / KSPLIT);  // K < 2^31 (checked on the host)
  const int nchunks = (Kpp + KCW - 1) / KCW;

  int64_t m_base, m_total, e = 0;
  if constexpr (MODE == MODE_DENSE) {
    m_base = (int64_t)blockIdx.z * ROWS;
    m_total = args.M - m_base;
    if (m_total > ROWS) m_total = ROWS;
  } else {
    e = blockIdx.y;
    m_base = args.offsets[e];
    m_total = args.offsets[e + 1] - m_base;
    if (m_total <= 0) return;
  }

  const int64_t n0 = ((int64_t)blockIdx.x * TPW + tile_in_wg) * 16;
  const int64_t nrow = n0 + nl;
  const bool nvalid = nrow < N;
  const int64_t nr = nvalid ? nrow : (N - 1);
  const int32_t g_part0 = (kw * Kpp) >> 6;  // first group of this wave's K part
  const WaveW<FMT> W = wave_weight<FMT>(mat ? args.w1 : args.w0, e, nr, kb, g_part0);
  // Decode constants in the 2^24-scaled form of the decode helpers (exact power-of-two
  // scalings): a zero point that is a power of two keeps -zp * s exact.
  const float cs24 = W.cs * kTwo24, fin24 = W.fin * kTwo24;
  const float mzp24 = -(float)args.w0.zp / kTwo24;

  // CCQ rows whose codes can never leave [0, 2^15 - 1] skip the clamp (one instruction per
  // byte); the choice is uniform over the wave.
  bool no_clamp = false;
  if constexpr (FMT == FMT_CCQ2) no_clamp = __all(ccq_row_needs_no_clamp(W.cs, W.cz));
  auto run = [&](auto clamp_tag) {
    constexpr bool CLAMP = decltype(clamp_tag)::value;
  for (int64_t ms = 0; ms < m_total; ms += ROWS) {
    const int64_t rows_here = (m_total - ms) < ROWS ? (m_total - ms) : ROWS;

    // Staging: every wave-wide load brings one 1 KiB segment of one activation row's chunk
    // (lane l: bytes 16 l .. 16 l + 15), so each load reads through a wave-uniform buffer
    // resource: base = the row's chunk start, range = the rest of the row.  The chunk advance is
    // scalar arithmetic and the lane's byte offset is fixed, and bytes past the row's end read
    // as zeros.  Rows past rows_here read the pass's first row (their results are never
    // stored).  With a K split, columns past a part's end read the next part's data and are
    // zeroed when stored.  Every load in the chunk loop is unconditional, so the compiler's
    // waits before a chunk's decode count exactly the next chunk's loads and leave them in
    // flight.
    constexpr int SEGS = KCT / 512;             // 1 KiB segments per row chunk
    constexpr int LPW = ROWS * SEGS / 4;        // segment loads per wave per chunk
    static_assert(LPW * 4 == ROWS * SEGS, "segments must divide over the waves");
    const uint16_t* srow[LPW];  // wave-uniform row pointers
    int32_t svoff[LPW];         // lane's byte offset in the row chunk (fixed)
    int32_t skin[LPW];          // lane's column offset inside its K part's chunk
    int32_t sidx[LPW];          // source row (dense, down) or sorted-pair index (gate+up)
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int row = (wave * LPW + j) / SEGS;
      sidx[j] = (int32_t)(m_base + ms + (row < rows_here ? row : 0));
    }
    if constexpr (MODE == MODE_GATEUP) {
      int32_t tok[LPW];  // every index load issued before the first is used
#pragma unroll
      for (int j = 0; j < LPW; ++j) tok[j] = args.sorted_pairs[sidx[j]];
#pragma unroll
      for (int j = 0; j < LPW; ++j)
        srow[j] = args.a + (int64_t)(__builtin_amdgcn_readfirstlane(tok[j]) / args.topk) * args.a_stride;
    } else {
#pragma unroll
      for (int j = 0; j < LPW; ++j) srow[j] = args.a + (int64_t)sidx[j] * args.a_stride;
    }
    // down: the pair ids of the lane's output rows, loaded before the chunk loop so that the
    // epilogue's stores wait for no memory round trip
    int32_t pid[MT][4];
    if constexpr (MODE == MODE_DOWN) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = t * 16 + 4 * kb + i;
          pid[t][i] = args.sorted_pairs[m_base + ms + (m < rows_here ? m : 0)];
        }
    }
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int seg = (wave * LPW + j) % SEGS;
      const int col = seg * 512 + 8 * lane;  // LDS column of the lane's 8 elements
      const int part = col / KCW;
      skin[j] = col % KCW;
      svoff[j] = (int32_t)((uint32_t)(part * Kpp + skin[j]) * 2u);  // < 2 K
    }
    u32x4 xr[LPW];
    auto stage_load = [&](int c) {
      const int32_t c0 = c * KCW;  // K < 2^30 (checked on the host)
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc32(srow[j] + c0, ((int32_t)args.K - c0) * 2);
        xr[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, svoff[j], 0, 0));
      }
    };
    auto stage_store = [&](int c, int buf) {
      if constexpr (KSPLIT > 1) {
        if ((c + 1) * KCW > Kpp) {  // last chunk of a K part that ends inside it
#pragma unroll
          for (int j = 0; j < LPW; ++j)
            if (c * KCW + skin[j] >= Kpp) xr[j] = (u32x4){0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int g = wave * LPW + j;
        *reinterpret_cast<u32x4*>(&lds[buf][(g / SEGS) * PITCH + (g % SEGS) * 1024 + 16 * lane]) =
            xr[j];
      }
    };

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    Raw<FMT> rawA[SPC], rawB[SPC];
    // Steps past the K part are loaded too (buffer loads: in range or zero) and never decoded.
    auto load_chunk = [&](Raw<FMT>(&r)[SPC], int c) {
#pragma unroll
      for (int j = 0; j < SPC; ++j) load_raw<FMT>(r[j], W, c * SPC + j);
    };
    auto compute_chunk = [&](Raw<FMT>(&r)[SPC], int c, int buf) {
#pragma unroll
      for (int j = 0; j < SPC; ++j) {
        if (c * KCW + j * SSK >= Kpp) break;
        // lane's A fragments: row t*16 + nl, columns kw*KCW + j*SSK + kb*WPL + 8h
        step_mma<FMT, MT, CLAMP>(r[j], W, cs24, fin24, mzp24,
                                 &lds[buf][nl * PITCH + (kw * KCW + j * SSK + kb * WPL) * 2],
                                 16 * PITCH, acc);
      }
    };

    load_chunk(rawA, 0);
    stage_load(0);
    stage_store(0, 0);
    __syncthreads();
    auto step = [&](Raw<FMT>(&cur)[SPC], Raw<FMT>(&nxt)[SPC], int c, int buf) {
      const bool more = (c + 1) < nchunks;
      const int cn = more ? c + 1 : c;  // past the last chunk: reload it, store nothing
      // Staging loads first: they are waited for at the end of this chunk, and vmcnt retires
      // in order, so the weight loads issued after them stay in flight into the next chunk.
      stage_load(cn);
      load_chunk(nxt, cn);
      compute_chunk(cur, c, buf);
      if (more) stage_store(cn, buf ^ 1);
      __syncthreads();
    };
    int c = 0;
    for (; c + 1 < nchunks; c += 2) {
      step(rawA, rawB, c, 0);
      step(rawB, rawA, c + 1, 1);
    }
    if (c < nchunks) step(rawA, rawB, c, 0);

    // Results that meet in LDS: K parts summed in order (dense) or the up tile handed to the
    // gate wave of the same tile (gate+up).
    f32x4* red = reinterpret_cast<f32x4*>(&lds[0][0]);
    if constexpr (KSPLIT > 1) {
      if (kw > 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) red[((kw - 1) * MT + t) * 64 + lane] = acc[t];
      }
      __syncthreads();
      if (kw == 0) {
#pragma unroll
        for (int p = 1; p < KSPLIT; ++p)
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[t] += red[((p - 1) * MT + t) * 64 + lane];
      }
      __syncthreads();
    }
    f32x4 up[MT];
    if constexpr (MODE == MODE_GATEUP) {
      if (mat == 1) {
#pragma unroll
        for (int t = 0; t < MT; ++t) red[(tile_in_wg * MT + t) * 64 + lane] = acc[t];
      }
      __syncthreads();
      if (mat == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) up[t] = red[(tile_in_wg * MT + t) * 64 + lane];
      }
      __syncthreads();
    }

    // Epilogue: lane holds rows t*16 + 4*kb + i (i = 0..3) of column nrow.
    const bool writer = (KSPLIT > 1) ? (kw == 0) : (mat == 0);
    if (writer && nvalid) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = t * 16 + 4 * kb + i;
          if (m >= rows_here) continue;
          const int64_t r = m_base + ms + m;
          if constexpr (MODE == MODE_DENSE) {
            uint16_t* y = reinterpret_cast<uint16_t*>(args.out);
            y[r * args.out_stride + nrow] = (uint16_t)f32_to_bf16_bits(acc[t][i]);
          } else if constexpr (MODE == MODE_GATEUP) {
            uint16_t* h = reinterpret_cast<uint16_t*>(args.out);
            h[r * args.out_stride + nrow] =
                (uint16_t)f32_to_bf16_bits(silu_f32(acc[t][i]) * up[t][i]);
          } else {
            float* d = reinterpret_cast<float*>(args.out);
            d[(int64_t)pid[t][i] * args.out_stride + nrow] = acc[t][i];
          }
        }
      }
    }
  }
  };
  if (no_clamp)
    run(std::integral_constant<bool, false>{});
  else
    run(std::integral_constant<bool, true>{});
}

// ---------------------------------------------------------------------------------------------
// Single-staging kernel: products of at most 16 activation rows per pass whose rows fit in LDS
// whole -- a dense product of few rows, or an MoE product of few routed tokens (each expert's
// rows in passes).  The chunked kernel above pays a memory round trip per chunk (staging loads,
// LDS store, barrier); at these sizes that chain, not bandwidth or decode, sets the call time.
// Here the activations are staged once per pass and a wave issues the weight loads of up to GNSB
// steps before its first decode, so a pass costs about one round trip plus the decode.  One
// workgroup per 16 output channels (and expert); its KS waves (4, or 16 when there are few
// output tiles) split K into parts of Kpp columns -- gate+up: half of the waves take the gate
// matrix and half the up matrix -- summed in LDS in order.  LDS: the pass's activation rows
// (pitch 2 K + 16 bytes), then a 128-byte zero block that the lanes of a step running past their
// part read instead; lanes of padding rows (nl >= rows of the pass) read row 0 and their results
// are never stored.
// ---------------------------------------------------------------------------------------------
constexpr int GEMV_LDS_MAX = 135168;  // 132 KiB: 16 rows of K = 4096 (one workgroup per CU)

// Steps whose packed data a lane holds at once (2048 columns of a wave's part with 4 waves, 512
// with 16: their parts are shorter and their register budget a quarter).
template <int FMT, int KS>
__host__ __device__ constexpr int gemv_steps() {
  return KS == 4 ? (is_int8(FMT) || is_int4(FMT) ? 16 : 8) : (is_int8(FMT) || is_int4(FMT) ? 4 : 2);
}

template <int FMT, int KS, int MODE>
__global__ __launch_bounds__(64 * KS) void gemv_kernel(const SkinnyArgs args, int32_t pass_rows) {
  constexpr int WPL = lane_weights<FMT>();
  constexpr int SSK = 4 * WPL;
  constexpr int GNSB = gemv_steps<FMT, KS>();
  constexpr int NT = 64 * KS;               // threads
  constexpr int XB = KS == 4 ? 16 : 4;      // 16-byte activation blocks per thread per round
  constexpr int NMAT = MODE == MODE_GATEUP ? 2 : 1;  // gate+up: half of the waves per matrix
  constexpr int KP = KS / NMAT;                        // K parts per matrix
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  __shared__ int32_t s_row[16];  // MoE: the pass's token (gate+up) or pair (down) per row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mat = kw / KP;
  const int part = kw % KP;
  const int nl = lane & 15;
  const int kb = lane >> 4;
  const int64_t N = args.N;
  const int32_t Kpp = (int32_t)(args.K / KP);        // a multiple of 64 (checked on the host)
  const int32_t ns = (Kpp + SSK - 1) / SSK;          // steps per wave
  const int32_t pitch = (int32_t)(args.K * 2 + 16);  // bytes per LDS activation row
  const int32_t bpr = (int32_t)(args.K / 8);         // 16-byte blocks per activation row

  int64_t e = 0, m_base = 0, m_total = args.M;  // dense: M <= pass_rows (checked on the host)
  if constexpr (MODE != MODE_DENSE) {
    e = blockIdx.y;
    m_base = args.offsets[e];
    m_total = args.offsets[e + 1] - m_base;
    if (m_total <= 0) return;
  }

  const int64_t nrow = (int64_t)blockIdx.x * 16 + nl;
  const bool nvalid = nrow < N;
  const WaveW<FMT> W =
      wave_weight<FMT>(mat ? args.w1 : args.w0, e, nvalid ? nrow : (N - 1), kb, (part * Kpp) >> 6);
  const float cs24 = W.cs * kTwo24, fin24 = W.fin * kTwo24;
  const float mzp24 = -(float)args.w0.zp / kTwo24;

  // Weight loads of the first GNSB steps (steps past the part are not loaded), issued before the
  // activation staging so that every load is in flight before the first wait.
  Raw<FMT> raw[GNSB];
#pragma unroll
  for (int j = 0; j < GNSB; ++j)
    if (j < ns) load_raw<FMT>(raw[j], W, j);

  const float inv = 1.0f / (float)bpr;
  uint8_t* zero_blk = lds_raw + pass_rows * pitch;
  auto run = [&](auto clamp_tag) {
    constexpr bool CLAMP = decltype(clamp_tag)::value;
    for (int64_t ms = 0; ms < m_total; ms += pass_rows) {
      const int32_t M = (int32_t)(m_total - ms < pass_rows ? m_total - ms : pass_rows);
      if (ms > 0) __syncthreads();  // the previous pass's LDS reads and sums are done
      if constexpr (MODE != MODE_DENSE) {
        if (tid < M) {
          const int32_t pr = args.sorted_pairs[m_base + ms + tid];
          s_row[tid] = MODE == MODE_GATEUP ? pr / args.topk : pr;
        }
        __syncthreads();
      }
      // Staged in rounds of XB blocks per thread (64 KiB per round).  Block b =
      // row r, column block c.  r = trunc((b + 1/2) * fl(1 / bpr)) in fp32 is floor(b / bpr):
      // the exact quotient lies at least 1 / (2 bpr) from an integer, and the fp32 error, a few
      // ulp of a value below 2^9 (b < 16384, bpr >= 32), stays far below that margin.
      const int32_t nblk = M * bpr;
      for (int32_t base = 0; base < nblk; base += XB * NT) {
        auto split = [&](int i, int32_t& r, int32_t& c) {
          const int32_t b = base + tid + NT * i;
          r = (int32_t)(((float)b + 0.5f) * inv);
          c = b - r * bpr;
        };
        u32x4 xr[XB];
#pragma unroll
        for (int i = 0; i < XB; ++i) {
          int32_t r, c;
          split(i, r, c);
          if (r < M) {
            int64_t src = ms + r;  // dense x row / MoE h row (sorted pair order)
            if constexpr (MODE == MODE_GATEUP) src = s_row[r];
            else if constexpr (MODE == MODE_DOWN) src = m_base + ms + r;
            xr[i] = *reinterpret_cast<const u32x4*>(args.a + src * args.a_stride + (int64_t)c * 8);
          }
        }
#pragma unroll
        for (int i = 0; i < XB; ++i) {
          int32_t r, c;
          split(i, r, c);
          if (r < M) *reinterpret_cast<u32x4*>(lds_raw + r * pitch + c * 16) = xr[i];
        }
      }
      if (tid < 8) reinterpret_cast<u32x4*>(zero_blk)[tid] = (u32x4){0, 0, 0, 0};
      __syncthreads();

      const uint8_t* arow = lds_raw + (nl < M ? nl : 0) * pitch + (part * Kpp + kb * WPL) * 2;
      f32x4 acc[1] = {(f32x4){0.f, 0.f, 0.f, 0.f}};
      for (int32_t s0 = 0; s0 < ns; s0 += GNSB) {
        if (s0 > 0 || (ms > 0 && ns > GNSB)) {  // a later block, or block 0 again
#pragma unroll
          for (int j = 0; j < GNSB; ++j)
            if (s0 + j < ns) load_raw<FMT>(raw[j], W, s0 + j);
        }
#pragma unroll
        for (int j = 0; j < GNSB; ++j) {
          const int32_t st = s0 + j;
          if (st >= ns) break;
          // this lane's first column of the step inside its part; past the part it reads zeros
          const bool inside = st * SSK + kb * WPL < Kpp;
          step_mma<FMT, 1, CLAMP>(raw[j], W, cs24, fin24, mzp24,
                                  inside ? arow + st * SSK * 2 : zero_blk, 0, acc);
        }
      }

      // K parts summed in order by wave 0 (gate+up: gate parts, then up parts), which writes the
      // rows 4 kb + i of its column.
      __syncthreads();
      f32x4* red = reinterpret_cast<f32x4*>(lds_raw);
      if (kw > 0) red[(kw - 1) * 64 + lane] = acc[0];
      __syncthreads();
      if (kw == 0 && nvalid) {
        f32x4 g = acc[0];
#pragma unroll
        for (int p = 1; p < KP; ++p) g += red[(p - 1) * 64 + lane];
        f32x4 u = g;
        if constexpr (MODE == MODE_GATEUP) {
          u = red[(KP - 1) * 64 + lane];
#pragma unroll
          for (int p = 1; p < KP; ++p) u += red[(KP - 1 + p) * 64 + lane];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * kb + i;
          if (m >= M) continue;
          if constexpr (MODE == MODE_DENSE) {
            uint16_t* y = reinterpret_cast<uint16_t*>(args.out);
            y[(ms + m) * args.out_stride + nrow] = (uint16_t)f32_to_bf16_bits(g[i]);
          } else if constexpr (MODE == MODE_GATEUP) {
            uint16_t* h = reinterpret_cast<uint16_t*>(args.out);
            h[(m_base + ms + m) * args.out_stride + nrow] =
                (uint16_t)f32_to_bf16_bits(silu_f32(g[i]) * u[i]);
          } else {
            float* d = reinterpret_cast<float*>(args.out);
            d[(int64_t)s_row[m] * args.out_stride + nrow] = g[i];
          }
        }
      }
    }
  };
  bool no_clamp = false;
  if constexpr (FMT == FMT_CCQ2) no_clamp = __all(ccq_row_needs_no_clamp(W.cs, W.cz));
  if (no_clamp)
    run(std::integral_constant<bool, false>{});
  else
    run(std::integral_constant<bool, true>{});
}

template <int FMT, int KS, int MODE>
hipError_t launch_gemv_ks(const SkinnyArgs& a, int64_t gy, int32_t pass_rows, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};  // per instantiation, one bit per device
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemv_kernel<FMT, KS, MODE>),
                                    GEMV_LDS_MAX, lds_set);
  if (e != hipSuccess) return e;
  int64_t lds = (int64_t)pass_rows * (2 * a.K + 16) + 128;
  if (lds < (KS - 1) * 1024) lds = (KS - 1) * 1024;  // the K-part sums reuse it
  hipLaunchKernelGGL((gemv_kernel<FMT, KS, MODE>), dim3((unsigned)((a.N + 15) / 16), (unsigned)gy),
                     dim3(64 * KS), (size_t)lds, s, a, pass_rows);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gemv_fmt(int mode, const SkinnyArgs& a, int ks, int64_t gy, int32_t pass_rows,
                           hipStream_t s) {
  if constexpr (is_alg2(FMT)) {  // a whole-group decode needs more registers than 16 waves leave
    if (mode == MODE_GATEUP) return launch_gemv_ks<FMT, 4, MODE_GATEUP>(a, gy, pass_rows, s);
    if (mode == MODE_DOWN) return launch_gemv_ks<FMT, 4, MODE_DOWN>(a, gy, pass_rows, s);
    return launch_gemv_ks<FMT, 4, MODE_DENSE>(a, gy, pass_rows, s);
  } else {
    if (mode == MODE_GATEUP)
      return ks == 16 ? launch_gemv_ks<FMT, 16, MODE_GATEUP>(a, gy, pass_rows, s)
                      : launch_gemv_ks<FMT, 4, MODE_GATEUP>(a, gy, pass_rows, s);
    if (mode == MODE_DOWN)
      return ks == 16 ? launch_gemv_ks<FMT, 16, MODE_DOWN>(a, gy, pass_rows, s)
                      : launch_gemv_ks<FMT, 4, MODE_DOWN>(a, gy, pass_rows, s);
    return ks == 16 ? launch_gemv_ks<FMT, 16, MODE_DENSE>(a, gy, pass_rows, s)
                    : launch_gemv_ks<FMT, 4, MODE_DENSE>(a, gy, pass_rows, s);
  }
}

template <int FMT, int MT, int MODE, int KSPLIT>
hipError_t launch_one(const SkinnyArgs& a, int64_t gy, int64_t gz, hipStream_t s) {
  constexpr int KCT = chunk_cols<FMT, KSPLIT>() * KSPLIT;
  constexpr size_t lds_bytes = 2 * (size_t)(MT * 16) * (KCT * 2 + 16);
  constexpr int TPW = (KSPLIT == 4) ? 1 : (MODE == MODE_GATEUP ? 2 : 4);
  static std::atomic<uint64_t> lds_set{0};  // per instantiation, one bit per device
  hipError_t e = ensure_dynamic_lds(
      reinterpret_cast<const void*>(&skinny_kernel<FMT, MT, MODE, KSPLIT>), (int)lds_bytes, lds_set);
  if (e != hipSuccess) return e;
  const int64_t ntiles = (a.N + 15) / 16;
  dim3 grid((unsigned)((ntiles + TPW - 1) / TPW), (unsigned)gy, (unsigned)gz);
  hipLaunchKernelGGL((skinny_kernel<FMT, MT, MODE, KSPLIT>), grid, dim3(256), lds_bytes, s, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(int mode, int mt, int ksplit, const SkinnyArgs& a, int64_t gy, int64_t gz,
                      hipStream_t s) {
  if (mode == MODE_DENSE) {
    if (ksplit == 4)
      return mt == 1 ? launch_one<FMT, 1, MODE_DENSE, 4>(a, gy, gz, s)
                     : launch_one<FMT, 2, MODE_DENSE, 4>(a, gy, gz, s);
    return mt == 1 ? launch_one<FMT, 1, MODE_DENSE, 1>(a, gy, gz, s)
                   : launch_one<FMT, 2, MODE_DENSE, 1>(a, gy, gz, s);
  }
  if (mode == MODE_GATEUP)
    return mt == 1 ? launch_one<FMT, 1, MODE_GATEUP, 1>(a, gy, gz, s)
                   : launch_one<FMT, 2, MODE_GATEUP, 1>(a, gy, gz, s);
  return mt == 1 ? launch_one<FMT, 1, MODE_DOWN, 1>(a, gy, gz, s)
                 : launch_one<FMT, 2, MODE_DOWN, 1>(a, gy, gz, s);
}

hipError_t dispatch_gemv(int fmt, int mode, const SkinnyArgs& args, int ks, int64_t gy,
                         int32_t pass_rows, hipStream_t stream) {
  switch (fmt) {
    case FMT_INT4:
      if (args.w0.group == 0) return launch_gemv_fmt<FMT_INT4PC>(mode, args, ks, gy, pass_rows, stream);
      return launch_gemv_fmt<FMT_INT4>(mode, args, ks, gy, pass_rows, stream);
    case FMT_AFFINE2: return launch_gemv_fmt<FMT_AFFINE2>(mode, args, ks, gy, pass_rows, stream);
    case FMT_INT8:
      if (args.w0.group == 0) return launch_gemv_fmt<FMT_INT8PC>(mode, args, ks, gy, pass_rows, stream);
      return launch_gemv_fmt<FMT_INT8>(mode, args, ks, gy, pass_rows, stream);
    case FMT_CCQ432: return launch_gemv_fmt<FMT_CCQ432>(mode, args, ks, gy, pass_rows, stream);
    case FMT_CCQH: return launch_gemv_fmt<FMT_CCQH>(mode, args, ks, gy, pass_rows, stream);
    default: return launch_gemv_fmt<FMT_CCQ2>(mode, args, ks, gy, pass_rows, stream);
  }
}

}  // namespace

hipError_t launch_skinny(int fmt, int mode, int m_tiles, int ksplit, const SkinnyArgs& args,
                         int64_t grid_y, int64_t grid_z, hipStream_t stream) {
  switch (fmt) {
    case FMT_INT4:
      if (args.w0.group == 0)
        return launch_fmt<FMT_INT4PC>(mode, m_tiles, ksplit, args, grid_y, grid_z, stream);
      return launch_fmt<FMT_INT4>(mode, m_tiles, ksplit, args, grid_y, grid_z, stream);
    case FMT_AFFINE2:
      return launch_fmt<FMT_AFFINE2>(mode, m_tiles, ksplit, args, grid_y, grid_z, stream);
    case FMT_INT8:
      if (args.w0.group == 0)
        return launch_fmt<FMT_INT8PC>(mode, m_tiles, ksplit, args, grid_y, grid_z, stream);
      return launch_fmt<FMT_INT8>(mode, m_tiles, ksplit, args, grid_y, grid_z, stream);
    case FMT_CCQ432:
      return launch_fmt<FMT_CCQ432>(mode, m_tiles, ksplit, args, grid_y, grid_z, stream);
    case FMT_CCQH:
      return launch_fmt<FMT_CCQH>(mode, m_tiles, ksplit, args, grid_y, grid_z, stream);
    default: return launch_fmt<FMT_CCQ2>(mode, m_tiles, ksplit, args, grid_y, grid_z, stream);
  }
}

int gemv_pass_rows(int64_t k) {
  if (k <= 0 || k % 256 != 0 || k >= (1ll << 30)) return 0;
  const int64_t r = (GEMV_LDS_MAX - 128) / (2 * k + 16);
  return (int)(r > 16 ? 16 : r);
}

bool gemv_fits(int64_t m, int64_t n, int64_t k) {
  return m >= 1 && m <= gemv_pass_rows(k) && (n + 15) / 16 <= 0x7FFFFFFF;
}

hipError_t launch_gemv(int fmt, const SkinnyArgs& args, hipStream_t stream) {
  if (!gemv_fits(args.M, args.N, args.K)) return hipErrorInvalidValue;
  // 16 waves per output tile when 4 would leave at least half of the 1024 SIMDs idle (each
  // part a multiple of 64 columns); with 8 the compiler runs out of registers
  const int64_t ntiles = (args.N + 15) / 16;
  const int ks = (ntiles * 16 <= 2048 && args.K % 1024 == 0 && !is_alg2(fmt)) ? 16 : 4;
  return dispatch_gemv(fmt, MODE_DENSE, args, ks, 1, (int32_t)args.M, stream);
}

int gemv_moe_split(int fmt, int mode, int64_t active_experts, int64_t n, int64_t k) {
  const int nmat = mode == MODE_GATEUP ? 2 : 1;
  if (gemv_pass_rows(k) < 1 || k % (64 * (4 / nmat)) != 0) return 0;
  const int64_t wgs = active_experts * ((n + 15) / 16);
  const bool ks16 = k % (64 * (16 / nmat)) == 0 && !is_alg2(fmt);
  if (wgs > (ks16 ? 1024 : 256)) return 0;
  return ks16 ? 16 : 4;
}

hipError_t launch_gemv_moe(int fmt, int mode, const SkinnyArgs& args, int64_t experts, int ks,
                           hipStream_t stream) {
  const int nmat = mode == MODE_GATEUP ? 2 : 1;
  const int rows = gemv_pass_rows(args.K);
  if ((mode != MODE_GATEUP && mode != MODE_DOWN) || (ks != 4 && ks != 16) || rows < 1 ||
      (ks == 16 && is_alg2(fmt)) ||
      args.K % (64 * (ks / nmat)) != 0 || experts < 1 || experts > 65535)
    return hipErrorInvalidValue;
  return dispatch_gemv(fmt, mode, args, ks, experts, rows, stream);
}

}  // namespace wq
