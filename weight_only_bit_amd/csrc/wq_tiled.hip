// wq_tiled.hip -- weight-only GEMM for many activation rows (prefill): exact-bf16 weights
// decoded straight into MFMA operands, activations staged in LDS by direct-to-LDS copies.
//
// One workgroup = 4 waves (one per SIMD) computes a 256 (activation rows) x 256 (weight rows)
// tile; K advances one 64-weight group per step.
//   * Weights: each wave owns 64 weight rows (MoE gate+up: 32 gate rows and the matching 32 up
//     rows).  Lane (n, h) decodes 32 consecutive weights of each of its two rows per step
//     (k = 32 h .. 32 h + 31 of the group) to the exact bf16 values -- the same bits
//     wq_dequantize produces -- directly into v_mfma_f32_32x32x16_bf16 B fragments.  The MFMA
//     k-slots of slice s take k = 32 h + 8 s + i (i < 8): any fixed order of the k-sum is the
//     same product, and this one makes every lane's weights contiguous.  Each packed code is
//     decoded exactly once per workgroup and serves 256 activation rows, so the decode (about
//     3.3 VALU instructions per CCQ weight) runs in the shadow of the MFMAs of the same wave.
//   * Activations: the 256 x 64 bf16 tile of each step is copied HBM -> LDS with
//     global_load_lds_dwordx4 (no registers, no LDS store instructions) three steps ahead
//     into a ring of four 32 KB buffers; rows are 128 bytes with the 16-byte pieces XOR-
//     swizzled by row pair (piece p of row r sits in slot p ^ ((r / 2) % 8)).  A 128-bit LDS
//     read serves 16 lanes per cycle from 64 banks (256 bytes), so the fragment read -- 32
//     consecutive rows, one piece -- is conflict free when each pair of rows (one 256-byte
//     bank line) uses its own slot: measured, this layout streams about 3x faster than a
//     swizzle by row (r % 8), which puts rows r and r + 8 of one cycle on the same banks.
//     MoE rows are gathered by token.
//   * Each wave multiplies all 256 rows by its 64 weight rows: 8 x 2 tiles of 32 x 32, four
//     k-slices per step, fp32 accumulation in 256 accumulation registers.  The next slice's
//     fragments are read while the current slice's MFMAs run, and the first slice of the next
//     step is read right after the step's barrier, under the last slice's MFMAs.
// Waves of a ragged tile still run every MFMA (rows past the end read the tile's first row);
// their results are not stored.
//
// The CCQ formats without code cluster ((4,3,2) and the hybrid) keep a group's scale in its last
// code word, so a group cannot be split between lanes cheaply.  There lane l copies and decodes
// the whole group of wave row l (64 weights), and v_permlane32_swap hands each lane half the
// other half's k-range: after the swap lane (n, h) holds k = 32 h .. 32 h + 31 of rows n and
// 32 + n, the same fragments as above.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "wq_kernels.hpp"

namespace wq {
namespace {

constexpr int BM = 256;        // activation rows per full tile (8 MFMA row blocks of 32)
constexpr int BN = 256;        // weight rows per tile (4 waves x 64)
constexpr int BK = 64;         // k per step (one group)
constexpr int NTHREADS = 256;  // 4 waves
constexpr int NSTAGE = 4;      // activation LDS ring
constexpr int A_STAGE = BM * BK * 2;  // 32 KB, 128-byte rows, no padding (XOR swizzle)

__shared__ __attribute__((aligned(16))) uint8_t sA0[A_STAGE];
__shared__ __attribute__((aligned(16))) uint8_t sA1[A_STAGE];
__shared__ __attribute__((aligned(16))) uint8_t sA2[A_STAGE];
__shared__ __attribute__((aligned(16))) uint8_t sA3[A_STAGE];

template <int ST>
__device__ __forceinline__ uint8_t* a_stage() {
  static_assert(ST >= 0 && ST < NSTAGE, "stage");
  if constexpr (ST == 0) return sA0;
  else if constexpr (ST == 1) return sA1;
  else if constexpr (ST == 2) return sA2;
  else return sA3;
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding: vmcnt bits 3:0 and 15:14).
#define WQ_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt((((n) & 0xF) | (((n) >> 4) << 14)) | (0x7 << 4) | (0xF << 8))

// Packed bytes one lane decodes per step for one weight row: 32 weights (the CCQ formats
// without code cluster: the 64 weights of one row).
template <int FMT>
struct Codes {
  u32x4 c;         // 2-bit formats: c.x, c.y (8 bytes); INT4 and (4,3,2) / hybrid: 16 bytes
  uint32_t scale;  // CCQ: scale byte; INT4 / affine: bf16 bits
  uint32_t zero;   // affine zero point
  u32x2 t;         // (4,3,2): bytes 16..23 of the aligned window; hybrid: bytes 16..19
  u32x4 c2;        // INT8: the second 16 bytes of the lane's 32 weights
};

// Where one weight row's packed data lives; the row is copied to LDS by one lane of its wave.
struct RowSrc {
  const uint8_t* codes;    // row start
  const uint8_t* scale;    // INT4 / affine: scales row (bf16, byte address); CCQ: qscale row
  const uint8_t* zeros;    // affine zero points row
  int32_t gstep;           // bytes between groups' scales: 2 (INT4 g64, affine) or 0 (INT4
                           // per channel); CCQ: unused (two 4-bit scales per byte)
};

template <int FMT>
__device__ __forceinline__ RowSrc row_src(const DevWeight& w, int64_t e, int64_t row) {
  RowSrc r{};
  const int64_t n = w.n, k = w.k, G = k / 64, grow = e * n + row;
  if (FMT == FMT_INT8) {  // per output channel (group-64 INT8 runs the decode-streaming kernels)
    r.codes = w.codes + grow * k;
  } else if (FMT == FMT_INT4) {
    r.codes = w.codes + grow * (k / 2);
    if (w.group) {
      r.scale = reinterpret_cast<const uint8_t*>(w.scales + grow * G);
      r.gstep = 2;
    } else {
      r.scale = reinterpret_cast<const uint8_t*>(w.scales + grow);
      r.gstep = 0;
    }
  } else if (FMT == FMT_AFFINE2) {
    r.codes = w.codes + grow * (k / 4);
    r.scale = reinterpret_cast<const uint8_t*>(w.scales + grow * G);
    r.zeros = w.zeros + grow * G;
    r.gstep = 2;
  } else if (is_alg2(FMT)) {
    r.codes = w.codes + grow * G * alg2_group_bytes(FMT);
  } else {
    r.codes = w.codes + grow * (k / 4);
    r.scale = w.qscale + grow * ((G + 1) / 2);
  }
  return r;
}

// Per-row constants of the CCQ decode (code scale and super scale times 2^24, code zero).
struct RowConst {
  float cs24, cz, fin24;
};

// The lane's 32 weights of one row as 16 bf16 pairs (k order).  mzp24 = -zp / 2^24 (CCQ).
template <int FMT>
__device__ __forceinline__ void cdecode(const Codes<FMT>& p, const RowConst& r, int64_t g,
                                        float mzp24, uint32_t (&o)[16]) {
  uint32_t a[8], b[8];
  if (FMT == FMT_INT8) {
    const float m128s = r.fin24 * (-128.0f / kTwo24);
    int8_decode16(p.c, r.fin24, m128s, a);
    int8_decode16(p.c2, r.fin24, m128s, b);
  } else if (FMT == FMT_INT4) {
    const float s24 = bf16_bits_to_f32(p.scale & 0xFFFFu) * kTwo24;
    const float m8s = s24 * (-8.0f / kTwo24);
    int4_decode16(p.c.x, p.c.y, s24, m8s, a);
    int4_decode16(p.c.z, p.c.w, s24, m8s, b);
  } else if (FMT == FMT_AFFINE2) {
    const float s = bf16_bits_to_f32(p.scale & 0xFFFFu);
    const float s24 = s * kTwo24, mzs = -(float)(p.zero & 0xFFu) * s;
    affine2_decode16(p.c.x, s24, mzs, a);
    affine2_decode16(p.c.y, s24, mzs, b);
  } else {
    const float s24 = (float)((p.scale >> (4 * (g & 1))) & 0xFu) * r.fin24;
    ccq_decode16(p.c.x, r.cs24, r.cz, s24, s24 * mzp24, a);
    ccq_decode16(p.c.y, r.cs24, r.cz, s24, s24 * mzp24, b);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o[i] = a[i];
    o[8 + i] = b[i];
  }
}

// Packed-data LDS ring, per wave and stage: codes (64 rows x 16 bytes, INT4: two such halves),
// then one dword per row for the scale, then (affine) one for the zero point.  (4,3,2) and
// hybrid: the first 16 bytes of each row's group window, then one (hybrid) or two ((4,3,2))
// dwords per row for the rest.
// INT8 (per channel): each row's 64 bytes as four 16-byte pieces (piece i at 1024 i), no scale
// (the row's scale is read once); two stages fill the 160 KB with the activation ring exactly.
template <int FMT>
struct CodeRing {
  static constexpr int CODE_BYTES = (FMT == FMT_INT8 ? 4 : FMT == FMT_INT4 ? 2 : 1) * 64 * 16;
  static constexpr int WAVE_BYTES =
      CODE_BYTES + (FMT == FMT_INT8 ? 0 : 256 * ((FMT == FMT_AFFINE2 || FMT == FMT_CCQ432) ? 2 : 1));
  static constexpr int STAGE_BYTES = 4 * WAVE_BYTES;
  static constexpr int DEPTH = (FMT == FMT_INT4 || FMT == FMT_INT8) ? 2 : 4;  // fits 160 KB with A
  static constexpr int AHEAD = DEPTH - 1 > 2 ? DEPTH - 1 : 2;  // steps between copy and decode
  // memory instructions per step per lane: codes, scale, zero / window pieces
  static constexpr int VMEM = FMT == FMT_INT8 ? 4
                             : is_alg2(FMT) ? (FMT == FMT_CCQ432 ? 3 : 2)
                                            : (FMT == FMT_INT4 ? 2 : 1) + 1 + (FMT == FMT_AFFINE2 ? 1 : 0);
};

// Row tiles.  An expert's (or the dense matrix's) rows are covered by full 256-row tiles; the
// remainder rem = rows % 256 goes to one tile of the smallest of 256, 128, 64 or 32 rows that
// holds it.  Kernel instances are per tile size (MT = rows / 32 MFMA row blocks): a launch
// with MT = 8 covers the full tiles and remainders above 128, the others one remainder each.
__host__ __device__ constexpr int tail_mt(int64_t rem) {
  return rem > 128 ? 8 : rem > 64 ? 4 : rem > 32 ? 2 : 1;
}
// Tiles of size class MT among `count` rows, and the first row of tile i of that class.
__device__ __forceinline__ int64_t class_tiles(int MT, int64_t count) {
  const int64_t rem = count % BM;
  if (MT == 8) return count / BM + (rem > 128 ? 1 : 0);
  return (rem > 0 && tail_mt(rem) == MT) ? 1 : 0;
}
__device__ __forceinline__ int64_t class_row0(int MT, int64_t count, int64_t i) {
  return MT == 8 ? i * BM : (count / BM) * BM;
}

// Per-format LDS ring of packed data (declared by the kernel, shared by its tile sizes).
struct CodeStages {
  uint8_t* s[4];
};

// One tile: rows row0 .. row0 + rows - 1 (at most 32 MT) of expert e, weight-row tile ctile.
template <int FMT, int MODE, int MT>
__device__ __forceinline__ void tile_body(const TiledArgs& args, const CodeStages& cs, int64_t e,
                                          int64_t row0, int64_t rows, int64_t ctile) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31, kh = lane >> 5;
  constexpr int64_t NCOLS_PER_TILE = (MODE == MODE_GATEUP) ? BN / 2 : BN;

  const int64_t N = args.N;
  const int64_t steps = args.K / BK;
  const int64_t last = steps - 1;
  const int64_t n0 = ctile * NCOLS_PER_TILE;

  // ---- weight rows ----
  // Decode: lane (l32, kh) decodes rows j = 0, 1:
  //   dense/down: channel n0 + 64 wave + 32 j + l32
  //   gate+up: j = 0 -> gate row n0 + 32 wave + l32, j = 1 -> the matching up row
  // i.e. "wave row" 32 j + l32 of the wave's 64 rows.  Copy: lane l copies wave row l.
  // The rows' constants are loaded here and scaled only after the prologue has issued its
  // packed-data copies: an operation on a loaded value makes the wave wait for the load first.
  using Ring = CodeRing<FMT>;
  int64_t wrow[2];
  RowConst rc[2];
  float rl[2][3] = {{0.f, 0.f, 0.f}, {0.f, 0.f, 0.f}};  // CCQ: code scale, code zero, super scale
  uint32_t rb[2] = {0u, 0u};                             // INT8: the row's scale (bf16 bits)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    wrow[j] = (MODE == MODE_GATEUP) ? n0 + 32 * wave + l32 : n0 + 64 * wave + 32 * j + l32;
    if constexpr (FMT == FMT_CCQ2) {
      const DevWeight& w = (MODE == MODE_GATEUP && j == 1) ? args.w1 : args.w0;
      const int64_t grow = e * w.n + (wrow[j] < N ? wrow[j] : N - 1);
      rl[j][0] = w.code_scale[grow];
      rl[j][1] = w.code_zero[grow];
      rl[j][2] = w.super_scale[grow];
    } else if constexpr (FMT == FMT_INT8) {  // the row's one scale
      const DevWeight& w = (MODE == MODE_GATEUP && j == 1) ? args.w1 : args.w0;
      const int64_t grow = e * w.n + (wrow[j] < N ? wrow[j] : N - 1);
      rb[j] = w.scales[grow];
    }
  }
  const float mzp24 = -(float)args.w0.zp / kTwo24;
  RowSrc rs;
  float own_super = 0.f;  // (4,3,2) / hybrid: super scale of wave row `lane`
  float own_fin24 = 0.f;  // ... times 2^24
  {
    const int jj = lane >> 5;  // wave row `lane` = 32 jj + (lane % 32)
    const int64_t r = (MODE == MODE_GATEUP) ? n0 + 32 * wave + (lane & 31)
                                            : n0 + 64 * wave + lane;
    const DevWeight& w = (MODE == MODE_GATEUP && jj == 1) ? args.w1 : args.w0;
    rs = row_src<FMT>(w, e, r < N ? r : N - 1);
    if constexpr (is_alg2(FMT)) own_super = w.super_scale[e * w.n + (r < N ? r : N - 1)];
  }
  auto scale_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (FMT == FMT_CCQ2) rc[j] = RowConst{rl[j][0] * kTwo24, rl[j][1], rl[j][2] * kTwo24};
      else if constexpr (FMT == FMT_INT8) rc[j] = RowConst{0.f, 0.f, bf16_bits_to_f32(rb[j]) * kTwo24};
      else rc[j] = RowConst{0.f, 0.f, 0.f};
    }
    own_fin24 = own_super * kTwo24;
  };

  // ---- activation copy role ----
  // Copy instruction i of wave w fills rows 32 i + 8 w .. + 7 of a stage (1 KB: lane l lands
  // at byte 16 l); lane l's row is r = 32 i + 8 w + l / 8 and its slot l % 8 receives piece
  // (l % 8) ^ ((r / 2) % 8) = (l % 8) ^ ((4 w + l / 16) % 8) of that row.  Rows past the end of a ragged tile read the tile's first
  // row; their results are never stored.
  // Gate+up rows are tokens: the pair ids are loaded here and turned into row addresses only
  // after the prologue has issued its packed-data copies, which need no wait for them.
  const uint16_t* csrc[MT];
  int32_t pair[MT];
  const int piece = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int r = 32 * i + 8 * wave + (lane >> 3);
    const int64_t gr = row0 + (r < rows ? r : 0);
    if constexpr (MODE == MODE_GATEUP) pair[i] = args.sorted_pairs[gr];
    else csrc[i] = args.a + gr * args.a_stride + piece * 8;
  }
  auto copy_a = [&](int64_t g, auto stc) __attribute__((always_inline)) {
    uint8_t* base = a_stage<decltype(stc)::value>();
#pragma unroll
    for (int i = 0; i < MT; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(csrc[i] + g * BK),
          (__attribute__((address_space(3))) void*)(base + (32 * i + 8 * wave) * 128), 16, 0, 0);
  };

  // ---- A fragments: rows m = 32 i + l32 (i < 8), slice s -> piece 4 kh + s, in slot
  // (4 kh + s) ^ ((m / 2) % 8) = (4 kh + s) ^ ((l32 / 2) % 8) ----
  auto read_a = [&](u32x4(&A)[MT], int s, auto stc) __attribute__((always_inline)) {
    const uint8_t* base = a_stage<decltype(stc)::value>();
    const int p = 4 * kh + s;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = 32 * i + l32;
      A[i] = *reinterpret_cast<const u32x4*>(base + m * 128 + ((p ^ ((l32 >> 1) & 7)) << 4));
    }
  };

  f32x16 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // B fragments of one step: slice s, row j -> 4 dwords (weights 32 kh + 8 s .. + 7).
  uint32_t Bw[2][2][16];  // [parity][j][16 dwords]
  auto mma = [&](const u32x4(&A)[MT], const uint32_t(&B)[2][16], int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 b = {B[j][4 * s], B[j][4 * s + 1], B[j][4 * s + 2], B[j][4 * s + 3]};
        acc[i][j] = mfma32x32x16(A[i], b, acc[i][j]);
      }
  };

  // ---- packed data: copied to this wave's part of an LDS ring, Ring::AHEAD steps ahead ----
  auto c_stage = [&](auto stc) __attribute__((always_inline)) {
    constexpr int CS = decltype(stc)::value;
    return cs.s[CS] + wave * Ring::WAVE_BYTES;
  };
  auto copy_codes = [&](int64_t g, auto stc) __attribute__((always_inline)) {
    uint8_t* base = c_stage(stc);
    if constexpr (is_alg2(FMT)) {
      // the dword-aligned window holding group g (a (4,3,2) group may start 2 bytes into a
      // dword; its window's last dword then holds the group's last 2 bytes)
      const uint8_t* p = rs.codes + g * alg2_group_bytes(FMT);
      if constexpr (FMT == FMT_CCQ432)
        p = reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(p) & ~(uintptr_t)3);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(p),
                                       (__attribute__((address_space(3))) void*)(base), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(p + 16),
                                       (__attribute__((address_space(3))) void*)(base + 1024), 4, 0, 0);
      if constexpr (FMT == FMT_CCQ432)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(p + 20),
                                         (__attribute__((address_space(3))) void*)(base + 1280), 4, 0, 0);
      return;
    }
    if constexpr (FMT == FMT_INT8) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(rs.codes + g * 64 + 16 * i),
            (__attribute__((address_space(3))) void*)(base + 1024 * i), 16, 0, 0);
      return;
    }
    if constexpr (FMT == FMT_INT4) {
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(rs.codes + g * 32),
                                       (__attribute__((address_space(3))) void*)(base), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(rs.codes + g * 32 + 16),
                                       (__attribute__((address_space(3))) void*)(base + 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(rs.scale + g * rs.gstep),
                                       (__attribute__((address_space(3))) void*)(base + Ring::CODE_BYTES), 2, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(rs.codes + g * 16),
                                       (__attribute__((address_space(3))) void*)(base), 16, 0, 0);
      if constexpr (FMT == FMT_AFFINE2) {
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(rs.scale + g * 2),
                                         (__attribute__((address_space(3))) void*)(base + Ring::CODE_BYTES), 2, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(rs.zeros + g),
                                         (__attribute__((address_space(3))) void*)(base + Ring::CODE_BYTES + 256), 1, 0, 0);
      } else {
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(rs.scale + (g >> 1)),
                                         (__attribute__((address_space(3))) void*)(base + Ring::CODE_BYTES), 1, 0, 0);
      }
    }
  };
  // The lane's packed data for its rows j = 0, 1 (wave rows 32 j + l32), half kh.  These LDS
  // reads are written out with their own wait: the copies that filled the buffer may have
  // been issued a loop trip earlier, and for such copies the compiler's own wait would be for
  // every outstanding memory instruction (the copies of the next steps included).  The caller
  // waits for the copy itself (vmcnt) first.  The outputs are early-clobber: a read's result
  // may land while a later read of the block has not yet issued, so no result register may
  // share a register with an address.
  auto read_codes = [&](Codes<FMT>(&cc)[2], auto stc) __attribute__((always_inline)) {
    const uint8_t* base = c_stage(stc);
    if constexpr (is_alg2(FMT)) {  // the lane's own row: 16 + 4 (+ 4) bytes
      const uint32_t oa = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(
          base + lane * 16);
      const uint32_t ta = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(
          base + 1024 + lane * 4);
      u32x4 c0;
      uint32_t t0, t1;
      if constexpr (FMT == FMT_CCQ432) {
        asm volatile(
            "ds_read_b128 %0, %3\n\t"
            "ds_read_b32 %1, %4\n\t"
            "ds_read_b32 %2, %4 offset:256\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(c0), "=&v"(t0), "=&v"(t1)
            : "v"(oa), "v"(ta)
            : "memory");
      } else {
        asm volatile(
            "ds_read_b128 %0, %2\n\t"
            "ds_read_b32 %1, %3\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(c0), "=&v"(t0)
            : "v"(oa), "v"(ta)
            : "memory");
        t1 = 0u;
      }
      cc[0].c = c0;
      cc[0].t = (u32x2){t0, t1};
      return;
    }
    if constexpr (FMT == FMT_INT8) {  // rows j = 0, 1: pieces 2 kh and 2 kh + 1
      const uint32_t ia = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(
          base + kh * 2048 + l32 * 16);
      u32x4 a0, a1, b0, b1;
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %4 offset:1024\n\t"
          "ds_read_b128 %2, %4 offset:512\n\t"
          "ds_read_b128 %3, %4 offset:1536\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1)
          : "v"(ia)
          : "memory");
      cc[0].c = a0;
      cc[0].c2 = a1;
      cc[1].c = b0;
      cc[1].c2 = b1;
      return;
    }
    const uint32_t ca = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(
        base + (FMT == FMT_INT4 ? kh * 1024 + l32 * 16 : l32 * 16 + kh * 8));
    const uint32_t sa = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(
        base + Ring::CODE_BYTES + l32 * 4);
    if constexpr (FMT == FMT_INT4) {
      u32x4 c0, c1;
      uint32_t s0, s1;
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %4 offset:512\n\t"
          "ds_read_b32 %2, %5\n\t"
          "ds_read_b32 %3, %5 offset:128\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(c0), "=&v"(c1), "=&v"(s0), "=&v"(s1)
          : "v"(ca), "v"(sa)
          : "memory");
      cc[0].c = c0;
      cc[1].c = c1;
      cc[0].scale = s0;
      cc[1].scale = s1;
    } else if constexpr (FMT == FMT_AFFINE2) {
      u32x2 c0, c1;
      uint32_t s0, s1, z0, z1;
      asm volatile(
          "ds_read_b64 %0, %6\n\t"
          "ds_read_b64 %1, %6 offset:512\n\t"
          "ds_read_b32 %2, %7\n\t"
          "ds_read_b32 %3, %7 offset:128\n\t"
          "ds_read_b32 %4, %7 offset:256\n\t"
          "ds_read_b32 %5, %7 offset:384\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(c0), "=&v"(c1), "=&v"(s0), "=&v"(s1), "=&v"(z0), "=&v"(z1)
          : "v"(ca), "v"(sa)
          : "memory");
      cc[0].c = (u32x4){c0.x, c0.y, 0u, 0u};
      cc[1].c = (u32x4){c1.x, c1.y, 0u, 0u};
      cc[0].scale = s0;
      cc[1].scale = s1;
      cc[0].zero = z0;
      cc[1].zero = z1;
    } else {
      u32x2 c0, c1;
      uint32_t s0, s1;
      asm volatile(
          "ds_read_b64 %0, %4\n\t"
          "ds_read_b64 %1, %4 offset:512\n\t"
          "ds_read_b32 %2, %5\n\t"
          "ds_read_b32 %3, %5 offset:128\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(c0), "=&v"(c1), "=&v"(s0), "=&v"(s1)
          : "v"(ca), "v"(sa)
          : "memory");
      cc[0].c = (u32x4){c0.x, c0.y, 0u, 0u};
      cc[1].c = (u32x4){c1.x, c1.y, 0u, 0u};
      cc[0].scale = s0;
      cc[1].scale = s1;
    }
  };
  auto clamp_step = [&](int64_t g) __attribute__((always_inline)) { return g < last ? g : last; };
  // (4,3,2) / hybrid: decode the lane's whole group, then swap lane halves so that lane
  // (n, h) holds k = 32 h .. 32 h + 31 of wave rows n (j = 0) and 32 + n (j = 1).
  auto decode_rows = [&](const Codes<FMT>(&cc)[2], int64_t g, uint32_t(&dst)[2][16])
      __attribute__((always_inline)) {
    if constexpr (is_alg2(FMT)) {
      uint32_t p[32];
      if constexpr (FMT == FMT_CCQ432) {
        const uint32_t sh =
            8u * (((uint32_t)reinterpret_cast<uintptr_t>(rs.codes) + 22u * (uint32_t)g) & 3u);
        const uint32_t w6[6] = {cc[0].c.x, cc[0].c.y, cc[0].c.z, cc[0].c.w, cc[0].t.x, cc[0].t.y};
        uint32_t c[6];
#pragma unroll
        for (int i = 0; i < 5; ++i) c[i] = __builtin_amdgcn_alignbit(w6[i + 1], w6[i], sh);
        c[5] = w6[5] >> sh;
        ccq432_decode64(c, own_fin24, mzp24, p);
      } else {
        const uint32_t c[5] = {cc[0].c.x, cc[0].c.y, cc[0].c.z, cc[0].c.w, cc[0].t.x};
        ccqh_decode64(c, own_fin24, mzp24, p);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // lower lanes keep p[i] and receive the upper lane's p[i]; upper lanes keep p[16 + i]
        // and receive the lower lane's p[16 + i]
        const auto r = __builtin_amdgcn_permlane32_swap(p[i], p[16 + i], false, false);
        dst[0][i] = r[0];
        dst[1][i] = r[1];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) cdecode<FMT>(cc[j], rc[j], g, mzp24, dst[j]);
    }
  };
  auto decode_step = [&](int64_t g, auto cstc, uint32_t(&dst)[2][16]) __attribute__((always_inline)) {
    Codes<FMT> cc[2];
    read_codes(cc, cstc);
    decode_rows(cc, g, dst);
  };
  constexpr int CD = Ring::DEPTH;

  // ---- prologue: steps 0 and 1 of the activations and 0..AHEAD-1 of the packed data in
  // flight, step 0 decoded and visible.  The packed data (from HBM, addresses known at once)
  // goes first; the activation copies may wait for the pair ids that locate their rows. ----
  copy_codes(0, std::integral_constant<int, 0>{});
  copy_codes(clamp_step(1), std::integral_constant<int, 1 % CD>{});
  if constexpr (Ring::AHEAD > 2) copy_codes(clamp_step(2), std::integral_constant<int, 2 % CD>{});
  __builtin_amdgcn_sched_barrier(0);
  scale_rows();
  if constexpr (MODE == MODE_GATEUP) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
      csrc[i] = args.a + (int64_t)(pair[i] / args.topk) * args.a_stride + piece * 8;
  }
  copy_a(0, std::integral_constant<int, 0>{});
  copy_a(clamp_step(1), std::integral_constant<int, 1>{});
  __builtin_amdgcn_s_waitcnt(0);  // everything issued so far
  __syncthreads();
  decode_step(0, std::integral_constant<int, 0>{}, Bw[0]);
  u32x4 X[MT], Y[MT];
  read_a(X, 0, std::integral_constant<int, 0>{});

  // ---- main loop: iteration g multiplies step g (LDS stage g % 4, B parity g % 2) ----
  //   wait for step g + 1's packed data; issue the packed data of step g + AHEAD; on even g the
  //   activation copies of steps g + 2 and g + 3 (two after each of the first MFMAs); slices
  //   0..2 (slice 0 was read last iteration), the next slices' reads and the decode of step
  //   g + 1; on odd g, once this wave's copies of steps g + 1 and g + 2 have landed, the
  //   barrier; read slice 0 of step g + 1 under slice 3 of step g.
  // The barrier comes every second step.  Even iteration g copies into the stages of steps
  // g - 2 and g - 1, whose last reads every wave made, and saw return, before the barrier that
  // ended iteration g - 1; a stage's copies are known landed in every wave at the barrier after
  // the odd iteration that follows them, before any wave reads that stage (step g + 1 of an
  // even g was copied two iterations earlier).  The packed data goes to this wave's own stage
  // of step g + AHEAD - CD, read at the start of an earlier iteration.
  auto iter = [&](int64_t g, auto stc) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    constexpr int PB = ST & 1;
    constexpr bool EVEN = PB == 0;
    // This wave's packed data of step g + 1 has landed once at most the memory instructions
    // issued after it are outstanding: on odd g the last iteration's (its packed data and 2 MT
    // activation copies; with the packed data only two steps ahead, just the copies); on even g
    // the wait before the last barrier covered it, unless it was issued in that odd iteration
    // itself (two steps ahead).
    if constexpr (!EVEN)
      WQ_WAIT_VMCNT(Ring::AHEAD >= 3 ? Ring::VMEM + 2 * MT : 2 * MT);
    else if constexpr (Ring::AHEAD < 3)
      WQ_WAIT_VMCNT(0);
    // slice 0's fragments (read under the previous iteration's last MFMAs) are complete; saying
    // so here spares the first MFMA a wait that would also cover the reads issued below
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
    Codes<FMT> cc[2];
    read_codes(cc, std::integral_constant<int, (ST + 1) % CD>{});
    copy_codes(clamp_step(g + Ring::AHEAD), std::integral_constant<int, (ST + Ring::AHEAD) % CD>{});
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (EVEN) {
      copy_a(clamp_step(g + 2), std::integral_constant<int, (ST + 2) & 3>{});
      copy_a(clamp_step(g + 3), std::integral_constant<int, (ST + 3) & 3>{});
    }
    read_a(Y, 1, stc);
    mma(X, Bw[PB], 0);
    read_a(X, 2, stc);
    mma(Y, Bw[PB], 1);
    read_a(Y, 3, stc);
    decode_rows(cc, clamp_step(g + 1), Bw[PB ^ 1]);
    mma(X, Bw[PB], 2);
    // 0x100 LDS read, 0x8 MFMA, 0x2 VALU, 0x20 VMEM read (the activation copies).  The copies
    // go under the first MFMAs of slice 0, before slice 1's fragment reads: the compiler counts
    // them among the LDS events, and no copy between a read and the wait for it keeps every
    // wait of the step down to the reads issued after the one it needs.
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (EVEN) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 40 / MT, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 40 / MT, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 40 / MT, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 40 / MT, 0);
    }
    if constexpr (!EVEN) {
      // this wave's copies of steps g + 1 and g + 2 have landed once at most this iteration's
      // packed data is outstanding, and every LDS read of this wave has returned before it
      // arrives: a stage read before this barrier may be overwritten by any wave's copies in
      // the next iteration
      WQ_WAIT_VMCNT(Ring::VMEM);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_sched_barrier(0);
    read_a(X, 0, std::integral_constant<int, (ST + 1) & 3>{});
    mma(Y, Bw[PB], 3);
    __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * MT, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  int64_t g = 0;
  for (; g + 3 < steps; g += 4) {
    iter(g, std::integral_constant<int, 0>{});
    iter(g + 1, std::integral_constant<int, 1>{});
    iter(g + 2, std::integral_constant<int, 2>{});
    iter(g + 3, std::integral_constant<int, 3>{});
  }
  if (g < steps) iter(g, std::integral_constant<int, 0>{});
  if (g + 1 < steps) iter(g + 1, std::integral_constant<int, 1>{});
  if (g + 2 < steps) iter(g + 2, std::integral_constant<int, 2>{});
  __builtin_amdgcn_s_waitcnt(0);  // no copy may still be writing LDS when the wave exits

  // ---- epilogue: lane holds D[m][wrow[j]] for m = 32 i + 8 q + 4 kh + t, r = 4 q + t, of each
  // 32 x 32 tile i.  For dense products whose output rows and columns allow 16-byte pieces, the
  // tile goes through LDS (the activation stages, free once every wave has passed the barrier
  // below: every copy has landed and every read returned) and leaves in 16-byte stores, two
  // rows per wave at a time -- 8 times fewer store instructions than storing each lane's bf16
  // values.  Otherwise each lane stores its own values: row m's address is a per-lane base plus
  // m x the row stride, a uniform (scalar) product; down rows go to their pair's row of d (pair
  // ids staged in activation stage 0, four consecutive rows per read). ----
  const bool full_rows = rows == 32 * MT;
  using OutT = typename std::conditional<MODE == MODE_DOWN, float, uint16_t>::type;
  constexpr int EB = (int)sizeof(OutT);
  constexpr int PIECE = 16 / EB;                             // elements per 16-byte piece
  constexpr int TC = (MODE == MODE_GATEUP) ? BN / 2 : BN;    // output columns of the tile
  constexpr int ROWB = TC * EB;                               // bytes of one output row
  constexpr int BLKB = 32 * ROWB;                             // one 32-row block
  constexpr int BPS = A_STAGE / BLKB;                         // blocks per activation stage
  constexpr int BPR = NSTAGE * BPS;                           // blocks per round
  constexpr int CPR = ROWB / 16;                              // pieces per row
  static_assert(BPS >= 1 && A_STAGE % BLKB == 0, "output blocks must tile the stages");
  const int64_t stride = args.out_stride;
  // Dense products only: the MoE epilogues measured no faster this way (gate+up writes an
  // eighth of a dense tile's bytes per lane, down's fp32 rows are scattered by pair id).
  const bool staged = MODE == MODE_DENSE && (N % PIECE == 0) && (stride % PIECE == 0);
  // down only (never staged): the address of each tile row's row of d (its pair's row)
  uint64_t* s_row = reinterpret_cast<uint64_t*>(a_stage<0>());
  (void)s_row;
  if (MODE == MODE_DOWN || staged) __syncthreads();  // every wave is done with the LDS rings
  if constexpr (MODE == MODE_DOWN) {
    for (int m = tid; m < 32 * MT; m += NTHREADS)
      s_row[m] = reinterpret_cast<uint64_t>(
          reinterpret_cast<float*>(args.out) +
          (int64_t)args.sorted_pairs[row0 + (m < rows ? m : 0)] * stride);
  }
  if (staged) {
    auto blk_ptr = [&](int b) __attribute__((always_inline)) {  // block b of a round
      const int st = b / BPS;
      uint8_t* sb = st == 0 ? a_stage<0>() : st == 1 ? a_stage<1>() : st == 2 ? a_stage<2>() : a_stage<3>();
      return sb + (b % BPS) * BLKB;
    };
    // rows 4..7 of every 8 are written 32 columns over, so the two row quads of one write
    // (kh = 0, 1) use different banks; the pieces move whole
    auto swz = [](int r) __attribute__((always_inline)) { return ((r >> 2) & 1) * 32; };
#pragma unroll
    for (int i0 = 0; i0 < MT; i0 += BPR) {
#pragma unroll
      for (int i = i0; i < MT && i < i0 + BPR; ++i) {
        OutT* blk = reinterpret_cast<OutT*>(blk_ptr(i - i0));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 8 * (r >> 2) + 4 * kh + (r & 3);  // row in the block
          if constexpr (MODE == MODE_GATEUP) {
            const int c = (32 * wave + l32) ^ swz(rr);
            blk[rr * TC + c] = (uint16_t)f32_to_bf16_bits(silu_f32(acc[i][0][r]) * acc[i][1][r]);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int c = (64 * wave + 32 * j + l32) ^ swz(rr);
              if constexpr (MODE == MODE_DOWN) blk[rr * TC + c] = acc[i][j][r];
              else blk[rr * TC + c] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
            }
          }
        }
      }
      __syncthreads();
      const int nblk = (MT - i0) < BPR ? (MT - i0) : BPR;
      for (int pc = tid; pc < nblk * 32 * CPR; pc += NTHREADS) {
        const int rr_all = pc / CPR, ch = pc % CPR;
        const int m = 32 * i0 + rr_all;
        const int64_t col = n0 + (int64_t)ch * PIECE;
        if ((!full_rows && m >= rows) || col >= N) continue;
        const int rr = rr_all & 31;
        const uint8_t* src = blk_ptr(rr_all >> 5) + rr * ROWB + ((ch * 16) ^ (swz(rr) * EB));
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        OutT* dst;
        if constexpr (MODE == MODE_DOWN)
          dst = reinterpret_cast<OutT*>(s_row[m]) + col;
        else
          dst = reinterpret_cast<OutT*>(args.out) + (row0 + m) * stride + col;
        *reinterpret_cast<u32x4*>(dst) = v;
      }
      if (i0 + BPR < MT) __syncthreads();  // the next round overwrites the stages
    }
    return;
  }
  // Full tiles whose rows all exist and whose wave's columns all lie inside N (uniform per
  // wave) store without per-element checks; ragged ones check every row and column.
  constexpr int WCOLS = (MODE == MODE_GATEUP) ? 32 : 64;  // output columns of one wave
  const bool wave_cols = n0 + WCOLS * (wave + 1) <= N;
  if constexpr (MODE == MODE_DOWN) {
    __syncthreads();
    auto store_rows = [&](auto checked) __attribute__((always_inline)) {
      constexpr bool CK = decltype(checked)::value;
      const bool in0 = wrow[0] < N, in1 = wrow[1] < N;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        // the addresses of the lane's 16 rows of block i (rows 32 i + 8 q + 4 kh + t), read
        // before the block's first store
        uint64_t ra[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m0 = 32 * i + 8 * q + 4 * kh;
          const u64x2 a01 = *reinterpret_cast<const u64x2*>(s_row + m0);
          const u64x2 a23 = *reinterpret_cast<const u64x2*>(s_row + m0 + 2);
          ra[q][0] = a01.x;
          ra[q][1] = a01.y;
          ra[q][2] = a23.x;
          ra[q][3] = a23.y;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m0 = 32 * i + 8 * q + 4 * kh;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (CK && m0 + t >= rows) continue;
            // a global-memory pointer (the generic form would compile to flat stores)
            __attribute__((address_space(1))) float* drow =
                reinterpret_cast<__attribute__((address_space(1))) float*>(ra[q][t]);
            if (!CK || in0) drow[wrow[0]] = acc[i][0][4 * q + t];
            if (!CK || in1) drow[wrow[1]] = acc[i][1][4 * q + t];
          }
        }
      }
    };
    if (full_rows && wave_cols) store_rows(std::false_type{});
    else store_rows(std::true_type{});
  } else {
    uint16_t* out = reinterpret_cast<uint16_t*>(args.out);
    auto value = [&](int i, int j, int r) __attribute__((always_inline)) {
      if constexpr (MODE == MODE_GATEUP) return silu_f32(acc[i][0][r]) * acc[i][1][r];
      else return acc[i][j][r];
    };
    // Fast path: row m = 32 i + 8 (r / 4) + 4 kh + r % 4 of the tile at a uniform row address
    // (rows 32 i + 8 (r / 4) + r % 4) plus the lane's byte offset 2 (4 kh stride + n), which
    // fits 32 bits when 4 stride + N < 2^30.
    if (full_rows && wave_cols && 4 * stride + N < (1ll << 30)) {
#pragma unroll
      for (int j = 0; j < (MODE == MODE_GATEUP ? 1 : 2); ++j) {
        const uint32_t loff = (uint32_t)(2 * (4 * kh * stride + wrow[j]));
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int mc = 32 * i + 8 * (r >> 2) + (r & 3);
            uint8_t* rowp = reinterpret_cast<uint8_t*>(out + (row0 + mc) * stride);
            *reinterpret_cast<uint16_t*>(rowp + loff) = (uint16_t)f32_to_bf16_bits(value(i, j, r));
          }
        }
      }
    } else {
      uint16_t* base = out + (row0 + 4 * kh) * stride;
#pragma unroll
      for (int j = 0; j < (MODE == MODE_GATEUP ? 1 : 2); ++j) {
        const int64_t n = wrow[j];
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int mc = 32 * i + 8 * (r >> 2) + (r & 3);  // m - 4 kh: the uniform part of the row
            if (!full_rows && mc + 4 * kh >= rows) continue;
            base[(int64_t)mc * stride + n] = (uint16_t)f32_to_bf16_bits(value(i, j, r));
          }
        }
      }
    }
  }
}

template <int FMT, int MODE>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void tiled_kernel(const TiledArgs args) {
  using Ring = CodeRing<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t sC0[Ring::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sC1[Ring::STAGE_BYTES];
  uint8_t* sC2 = sC0;  // stages 2 and 3 exist only for four-stage rings
  uint8_t* sC3 = sC1;
  if constexpr (Ring::DEPTH > 2) {
    __shared__ __attribute__((aligned(16))) uint8_t sC2_[Ring::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sC3_[Ring::STAGE_BYTES];
    sC2 = sC2_;
    sC3 = sC3_;
  }
  const int lane = threadIdx.x & 63;

  // ---- which tile: XCD-aware order ----
  // Workgroups are handed to the 8 XCDs round-robin (workgroup w runs on XCD w % 8).  Row tile
  // r goes to XCD r % 8, and each XCD walks all column tiles of one row tile before the next,
  // so the workgroups running together on an XCD share their activation tile through its L2.
  constexpr int64_t NCOLS_PER_TILE = (MODE == MODE_GATEUP) ? BN / 2 : BN;
  const int64_t ncols = (args.N + NCOLS_PER_TILE - 1) / NCOLS_PER_TILE;
  const int64_t wg = blockIdx.x;
  const int64_t li = wg >> 3;
  const int64_t rtile = (li / ncols) * 8 + (wg & 7);
  const int64_t ctile = li % ncols;

  // ---- the row tile: index rtile in the list [tiles of 256 rows][remainders of 128][64][32]
  // (each class in expert order), then its expert and rows ----
  int mt;
  int64_t e = 0, row0, rows;
  if constexpr (MODE == MODE_DENSE) {
    const int64_t nfull = class_tiles(8, args.M), rem = args.M % BM;
    if (rtile < nfull) {
      mt = 8;
      row0 = rtile * BM;
    } else {
      if (rtile > nfull || rem == 0 || rem > 128) return;
      mt = tail_mt(rem);
      row0 = (args.M / BM) * BM;
    }
    rows = args.M - row0 < BM ? args.M - row0 : BM;
  } else {
    // Every wave finds the tile itself (the same uniform result in each, no LDS, no barrier):
    // per-expert tile counts of each size class, scanned 64 experts at a time.  With at most
    // 64 experts the counts are loaded once.
    int64_t idx = rtile;
    int found_e = -1, found_c = 0, local = 0;
    auto find = [&](int32_t nt, int cls, int eb) __attribute__((always_inline)) {
      int32_t incl = nt;
      for (int d = 1; d < 64; d <<= 1) {
        const int32_t v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
      }
      const int32_t total = __shfl(incl, 63);
      if (idx < total) {
        const uint64_t m = __ballot(idx >= incl - nt && idx < incl);
        const int src = __ffsll((unsigned long long)m) - 1;
        found_e = eb + src;
        found_c = cls;
        local = (int)(idx - __shfl(incl - nt, src));
      } else {
        idx -= total;
      }
    };
    if (args.experts <= 64) {
      const int64_t cnt = lane < args.experts ? args.offsets[lane + 1] - args.offsets[lane] : 0;
      for (int ci = 0; ci < 4 && found_e < 0; ++ci)
        find((int32_t)class_tiles(8 >> ci, cnt), 8 >> ci, 0);
    } else {
      for (int ci = 0; ci < 4 && found_e < 0; ++ci) {
        const int cls = 8 >> ci;
        for (int eb = 0; eb < args.experts && found_e < 0; eb += 64) {
          const int ex = eb + lane;
          const int32_t nt =
              ex < args.experts ? (int32_t)class_tiles(cls, args.offsets[ex + 1] - args.offsets[ex]) : 0;
          find(nt, cls, eb);
        }
      }
    }
    found_e = __builtin_amdgcn_readfirstlane(found_e);
    if (found_e < 0) return;
    e = found_e;
    mt = __builtin_amdgcn_readfirstlane(found_c);
    local = __builtin_amdgcn_readfirstlane(local);
    const int64_t base = args.offsets[e];
    const int64_t cnt = args.offsets[e + 1] - base;
    row0 = base + class_row0(mt, cnt, local);
    rows = base + cnt - row0 < BM ? base + cnt - row0 : BM;
  }
  const CodeStages cs{{sC0, sC1, sC2, sC3}};
  switch (mt) {
    case 8: tile_body<FMT, MODE, 8>(args, cs, e, row0, rows, ctile); break;
    case 4: tile_body<FMT, MODE, 4>(args, cs, e, row0, rows < 128 ? rows : 128, ctile); break;
    case 2: tile_body<FMT, MODE, 2>(args, cs, e, row0, rows < 64 ? rows : 64, ctile); break;
    default: tile_body<FMT, MODE, 1>(args, cs, e, row0, rows < 32 ? rows : 32, ctile); break;
  }
}

// One launch: the tile list holds the full tiles and every remainder tile (MoE: row_tiles
// bounds their number, sum_e ceil(rows_e / 256); workgroups past the list exit at once).
template <int FMT, int MODE>
hipError_t launch_t(const TiledArgs& a, int64_t row_tiles, hipStream_t s) {
  const int64_t tiles = (MODE == MODE_DENSE) ? a.M / BM + 1 : row_tiles;
  if (tiles <= 0) return hipSuccess;
  constexpr int64_t per_tile = (MODE == MODE_GATEUP) ? BN / 2 : BN;
  const int64_t cols = (a.N + per_tile - 1) / per_tile;
  const int64_t wgs = (tiles + 7) / 8 * 8 * cols;  // row tiles padded to the 8 XCDs
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid((unsigned)wgs);
  hipLaunchKernelGGL((tiled_kernel<FMT, MODE>), grid, dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int fmt, const TiledArgs& a, int64_t row_tiles, hipStream_t s) {
  switch (fmt) {
    case FMT_INT4: return launch_t<FMT_INT4, MODE>(a, row_tiles, s);
    case FMT_AFFINE2: return launch_t<FMT_AFFINE2, MODE>(a, row_tiles, s);
    case FMT_CCQ2: return launch_t<FMT_CCQ2, MODE>(a, row_tiles, s);
    case FMT_INT8:
      if (a.w0.group != 0) return hipErrorInvalidValue;  // per channel only
      return launch_t<FMT_INT8, MODE>(a, row_tiles, s);
    case FMT_CCQ432: return launch_t<FMT_CCQ432, MODE>(a, row_tiles, s);
    case FMT_CCQH: return launch_t<FMT_CCQH, MODE>(a, row_tiles, s);
    default: return hipErrorInvalidValue;
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
