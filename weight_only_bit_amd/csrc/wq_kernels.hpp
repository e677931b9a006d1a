// wq_kernels.hpp -- kernel argument structs and launcher declarations shared by the HIP
// translation units of libwq.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "wq_device.hpp"

namespace wq {

// Raise a kernel's dynamic-LDS limit on the current device, once per device: the attribute is
// per-device state, and `done` holds one bit per device already set (ids below 64; higher ids
// set it on every call).  Safe to call from several host threads.
inline hipError_t ensure_dynamic_lds(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Arguments of the decode-streaming ("skinny") MFMA kernels.
struct SkinnyArgs {
  DevWeight w0;                 // dense W / MoE gate / MoE down
  DevWeight w1;                 // MoE up (gate+up mode only)
  const uint16_t* a;            // activations: dense x [M][K]; MoE x [T][K]; MoE h [P][K]
  int64_t a_stride;             // elements per activation row
  void* out;                    // dense y bf16 [M][N]; MoE h bf16 [P][N]; MoE d f32 [P][N]
  int64_t out_stride;           // elements per output row
  int64_t M;                    // dense rows
  int64_t N, K;
  const int32_t* offsets;       // MoE: expert_offsets [E+1]
  const int32_t* sorted_pairs;  // MoE: pair ids grouped by expert
  int32_t topk;
};

enum { MODE_DENSE = 0, MODE_GATEUP = 1, MODE_DOWN = 2 };

// Launch the skinny kernel for format `fmt`; m_tiles = 1 or 2 (16 or 32 activation rows per
// pass); ksplit = 1 or 4 (waves of a workgroup split K); grid_y = experts (MoE) or 1;
// grid_z = row super-tiles (dense).
hipError_t launch_skinny(int fmt, int mode, int m_tiles, int ksplit, const SkinnyArgs& args,
                         int64_t grid_y, int64_t grid_z, hipStream_t stream);

// Single-staging products: activation rows staged in LDS whole, rows x (2 K + 16) + 128 bytes
// at most 132 KiB, K % 256 == 0.  gemv_pass_rows(k): rows of one pass (at most 16, 0 if none).
int gemv_pass_rows(int64_t k);
// Dense products of 1 .. gemv_pass_rows(k) rows: one launch, the waves of a workgroup split K.
bool gemv_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv(int fmt, const SkinnyArgs& args, hipStream_t stream);
// MoE gate+up / down over `experts` (grid y), each expert's routed rows in passes of
// gemv_pass_rows(K).  gemv_moe_split: the waves per workgroup (4 or 16) for a launch whose
// routed work touches at most `active_experts` experts, or 0 when the chunked kernel is the
// better choice (many workgroups) or K does not split.
int gemv_moe_split(int fmt, int mode, int64_t active_experts, int64_t n, int64_t k);
hipError_t launch_gemv_moe(int fmt, int mode, const SkinnyArgs& args, int64_t experts, int ks,
                           hipStream_t stream);

hipError_t launch_dequant(int fmt, const DevWeight& w, int64_t experts, uint16_t* out,
                          hipStream_t stream);

// Entries (int32) of the per-chunk routing table a long routing array uses, 0 when the pairs
// are sorted without one.  launch_route with table == nullptr always sorts in one workgroup.
int64_t route_table_entries(int64_t npairs, int32_t experts);
hipError_t launch_route(const int32_t* ids, int64_t npairs, int32_t experts, int32_t* offsets,
                        int32_t* sorted_pairs, int32_t* table, hipStream_t stream);

hipError_t launch_combine(const float* d, const float* weights, int64_t t, int32_t topk,
                          int64_t hidden, uint16_t* y, hipStream_t stream);

// Arguments of the LDS-staged MFMA GEMM (many activation rows).
struct TiledArgs {
  DevWeight w0, w1;             // as SkinnyArgs
  const uint16_t* a;            // activations (rows as in SkinnyArgs)
  int64_t a_stride;
  void* out;
  int64_t out_stride;
  int64_t M, N, K;              // M: dense rows
  const int32_t* offsets;       // MoE expert offsets [E+1]
  const int32_t* sorted_pairs;
  int32_t topk;
  int32_t experts;
};

// CCQ (6,4,3) code-cluster encoder: one workgroup per row of w [n][k] (fp32).  refine: bit 0
// re-picks each clustered code among the row's decodable codes, bit 1 optimizes group scales.
size_t ccq_encode_lds_bytes(int64_t k, int refine);
hipError_t launch_ccq_encode(const float* w, int64_t n, int64_t k, int32_t zp, int refine,
                             uint8_t* codes, uint8_t* qscale, float* super_scale,
                             float* code_scale, float* code_zero, hipStream_t stream);

// Rows of one tile of the tiled kernel.
int tiled_rows();

// row_tiles: dense: ceil(M / tiled_rows()); MoE: an upper bound of sum_e ceil(rows_e /
// tiled_rows()) (extra workgroups exit).
hipError_t launch_tiled(int fmt, int mode, const TiledArgs& args, int64_t row_tiles,
                        hipStream_t stream);

}  // namespace wq
