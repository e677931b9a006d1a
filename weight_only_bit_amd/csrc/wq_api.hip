// wq_api.hip -- the C ABI of libwq.so (declared in include/wq.h): host-side validation,
// kernel selection and launches.  No compute happens on the host; nothing here allocates
// device memory or synchronizes.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/wq.h"
#include "wq_kernels.hpp"

namespace {

thread_local std::string g_last_error;

wq_status fail(wq_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
wq_status fail(wq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

wq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return WQ_OK;
  return fail(WQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Weights the tiled (many-row) kernels implement: every format but group-64 INT8, whose
// packed data (64 bytes per row per step plus scales) leaves no LDS for a staging ring next to
// the activation ring; it runs the decode-streaming kernels for every row count.
bool has_tiled(const wq_weight* w) {
  return w->format != WQ_FMT_INT8 || w->group == 0;
}

bool is_ccq(int32_t f) {
  return f == WQ_FMT_CCQ2 || f == WQ_FMT_CCQ432 || f == WQ_FMT_CCQ_HYBRID;
}

// Bytes of one packed row of k weights.
int64_t row_code_bytes(const wq_weight* w) {
  switch (w->format) {
    case WQ_FMT_INT4: return w->k / 2;
    case WQ_FMT_INT8: return w->k;
    case WQ_FMT_CCQ432: return w->k / 64 * 22;
    case WQ_FMT_CCQ_HYBRID: return w->k / 64 * 20;
    default: return w->k / 4;
  }
}

// Largest byte range of one expert's array that the decode kernels' 32-bit buffer resources
// cover (the (4,3,2) / hybrid code views add up to 6 bytes of dword alignment to it).
constexpr int64_t kMaxExpertBytes = 0x7FFFFFF0ll - 8;

// The product kernels decode CCQ weights as fma(u, s, -zp*s), exact when zp*s is exact: zp
// must then be zero or a power of two (the formats' zero points are 32, 8 and 4).
// The product kernels also address one expert's arrays, and one activation row, with 32-bit
// byte offsets: every array of one expert must lie within kMaxExpertBytes.  The codes are
// the largest array of every format (scales, zeros and the per-row arrays are smaller).
wq_status check_product_zp(const wq_weight* w, const char* what) {
  if (is_ccq(w->format) && (w->zp & (w->zp - 1)) != 0)
    return fail(WQ_ERR_UNSUPPORTED, "%s: products need a CCQ zero point of 0 or a power of two", what);
  if (w->k >= (1ll << 30))
    return fail(WQ_ERR_UNSUPPORTED, "%s: products need k below 2^30", what);
  const int64_t row_bytes = row_code_bytes(w);
  if (w->n * row_bytes > kMaxExpertBytes)
    return fail(WQ_ERR_UNSUPPORTED, "%s: one expert's codes must not exceed %lld bytes", what,
                (long long)kMaxExpertBytes);
  return WQ_OK;
}

// Validate a packed-weight descriptor; `what` names it in error messages.
wq_status check_weight(const wq_weight* w, const char* what) {
  if (!w) return fail(WQ_ERR_ARG, "%s: null descriptor", what);
  if (w->n <= 0 || w->k <= 0 || w->experts <= 0)
    return fail(WQ_ERR_ARG, "%s: n, k and experts must be positive", what);
  if (w->k % 64 != 0) return fail(WQ_ERR_UNSUPPORTED, "%s: k = %lld is not a multiple of 64", what, (long long)w->k);
  if (w->n > (1ll << 31) || w->k > (1ll << 31))
    return fail(WQ_ERR_UNSUPPORTED, "%s: n and k must be below 2^31", what);
  if (!w->codes) return fail(WQ_ERR_ARG, "%s: null codes", what);
  if (!aligned16(w->codes)) return fail(WQ_ERR_ALIGN, "%s: codes not 16-byte aligned", what);
  switch (w->format) {
    case WQ_FMT_INT4:
      if (w->group != 64 && w->group != 0)
        return fail(WQ_ERR_UNSUPPORTED, "%s: INT4 group must be 64 or 0 (per channel)", what);
      if (!w->scales) return fail(WQ_ERR_ARG, "%s: null scales", what);
      if (!aligned16(w->scales)) return fail(WQ_ERR_ALIGN, "%s: scales not 16-byte aligned", what);
      break;
    case WQ_FMT_INT8:
      if (w->group != 64 && w->group != 0)
        return fail(WQ_ERR_UNSUPPORTED, "%s: INT8 group must be 64 or 0 (per channel)", what);
      if (!w->scales) return fail(WQ_ERR_ARG, "%s: null scales", what);
      if (!aligned16(w->scales)) return fail(WQ_ERR_ALIGN, "%s: scales not 16-byte aligned", what);
      break;
    case WQ_FMT_INT2_AFFINE:
      if (w->group != 64) return fail(WQ_ERR_UNSUPPORTED, "%s: affine 2-bit needs group 64", what);
      if (!w->scales || !w->zeros) return fail(WQ_ERR_ARG, "%s: null scales or zeros", what);
      if (!aligned16(w->scales) || !aligned16(w->zeros))
        return fail(WQ_ERR_ALIGN, "%s: scales/zeros not 16-byte aligned", what);
      break;
    case WQ_FMT_CCQ2:
      if (w->group != 64) return fail(WQ_ERR_UNSUPPORTED, "%s: CCQ needs group 64", what);
      if (!w->qscale || !w->super_scale || !w->code_scale || !w->code_zero)
        return fail(WQ_ERR_ARG, "%s: null CCQ scale arrays", what);
      if (!aligned16(w->qscale) || !aligned16(w->super_scale) || !aligned16(w->code_scale) ||
          !aligned16(w->code_zero))
        return fail(WQ_ERR_ALIGN, "%s: CCQ scale arrays not 16-byte aligned", what);
      if (w->zp < 0 || w->zp > 127)
        return fail(WQ_ERR_UNSUPPORTED, "%s: CCQ zero point must lie in 0..127", what);
      break;
    case WQ_FMT_CCQ432:
    case WQ_FMT_CCQ_HYBRID:
      if (w->group != 64) return fail(WQ_ERR_UNSUPPORTED, "%s: CCQ needs group 64", what);
      if (!w->super_scale) return fail(WQ_ERR_ARG, "%s: null super_scale", what);
      if (!aligned16(w->super_scale))
        return fail(WQ_ERR_ALIGN, "%s: super_scale not 16-byte aligned", what);
      if (w->zp < 0 || w->zp > 127)
        return fail(WQ_ERR_UNSUPPORTED, "%s: CCQ zero point must lie in 0..127", what);
      break;
    default:
      return fail(WQ_ERR_UNSUPPORTED, "%s: unknown format %d", what, w->format);
  }
  return WQ_OK;
}

wq::DevWeight dev_weight(const wq_weight* w) {
  wq::DevWeight d;
  d.codes = w->codes;
  d.scales = w->scales;
  d.zeros = w->zeros;
  d.qscale = w->qscale;
  d.super_scale = w->super_scale;
  d.code_scale = w->code_scale;
  d.code_zero = w->code_zero;
  d.n = w->n;
  d.k = w->k;
  d.group = w->group;
  d.zp = w->zp;
  return d;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct MoeWs {
  int32_t* offsets;
  int32_t* sorted;
  int32_t* route_table;  // null when the routing sort takes no table
  uint16_t* h;
  float* d;
  size_t bytes;
};

MoeWs moe_layout(void* ws, int64_t t, int32_t topk, int32_t experts, int64_t hidden, int64_t inter) {
  MoeWs L;
  const size_t pairs = (size_t)t * (size_t)topk;
  size_t off = 0;
  char* b = static_cast<char*>(ws);
  L.offsets = reinterpret_cast<int32_t*>(b + off);
  off = align_up(off + sizeof(int32_t) * ((size_t)experts + 1));
  L.sorted = reinterpret_cast<int32_t*>(b + off);
  off = align_up(off + sizeof(int32_t) * pairs);
  const int64_t table = wq::route_table_entries((int64_t)pairs, experts);
  L.route_table = table > 0 ? reinterpret_cast<int32_t*>(b + off) : nullptr;
  off = align_up(off + sizeof(int32_t) * (size_t)table);
  L.h = reinterpret_cast<uint16_t*>(b + off);
  off = align_up(off + sizeof(uint16_t) * pairs * (size_t)inter);
  L.d = reinterpret_cast<float*>(b + off);
  off = align_up(off + sizeof(float) * pairs * (size_t)hidden);
  L.bytes = off;
  return L;
}

constexpr int32_t kMaxExperts = 512;
// Up to this many activation rows the decode-streaming kernels run; above it the tiled ones.
constexpr int64_t kSkinnyMaxRows = 32;
// MoE layers whose experts average at least this many routed rows use the tiled kernels.
constexpr double kMoeTiledRows = 32.0;
// Largest grid z extent one launch uses.
constexpr int64_t kMaxGridZ = 65535;

}  // namespace

extern "C" {

const char* wq_status_string(int32_t st) {
  switch (st) {
    case WQ_OK: return "WQ_OK";
    case WQ_ERR_ARG: return "WQ_ERR_ARG";
    case WQ_ERR_UNSUPPORTED: return "WQ_ERR_UNSUPPORTED";
    case WQ_ERR_ALIGN: return "WQ_ERR_ALIGN";
    case WQ_ERR_RANGE: return "WQ_ERR_RANGE";
    case WQ_ERR_WORKSPACE: return "WQ_ERR_WORKSPACE";
    case WQ_ERR_HIP: return "WQ_ERR_HIP";
    default: return "WQ_ERR_UNKNOWN";
  }
}

const char* wq_last_error(void) { return g_last_error.c_str(); }

const char* wq_last_error_detail(void) { return g_last_error.c_str(); }

wq_status wq_pack_int4(const int32_t* codes, int64_t n, uint8_t* out) {
  if (n < 0 || (n > 0 && (!codes || !out))) return fail(WQ_ERR_ARG, "wq_pack_int4: bad arguments");
  for (int64_t i = 0; i < n; ++i)
    if (codes[i] < -8 || codes[i] > 7)
      return fail(WQ_ERR_RANGE, "wq_pack_int4: code %d at index %lld outside -8..7", codes[i], (long long)i);
  for (int64_t b = 0; b < (n + 1) / 2; ++b) {
    const int32_t first = codes[2 * b];
    const int32_t second = (2 * b + 1 < n) ? codes[2 * b + 1] : 0;
    out[b] = (uint8_t)((first & 0xF) | ((second & 0xF) << 4));
  }
  return WQ_OK;
}

wq_status wq_unpack_int4(const uint8_t* data, int64_t n, int32_t* out) {
  if (n < 0 || (n > 0 && (!data || !out))) return fail(WQ_ERR_ARG, "wq_unpack_int4: bad arguments");
  for (int64_t i = 0; i < n; ++i) {
    const int32_t v = (data[i >> 1] >> (4 * (i & 1))) & 0xF;
    out[i] = (v ^ 8) - 8;
  }
  return WQ_OK;
}

int64_t wq_packed_size(int64_t n_codes, int32_t bits) {
  if (n_codes < 0 || bits < 1 || bits > 32) return -1;
  if (n_codes > (INT64_MAX - 7) / bits) return -1;  // the bit count would overflow
  return (n_codes * (int64_t)bits + 7) / 8;
}

wq_status wq_dequantize(const wq_weight* w, uint16_t* out, void* stream) {
  wq_status st = check_weight(w, "wq_dequantize");
  if (st != WQ_OK) return st;
  if (!out) return fail(WQ_ERR_ARG, "wq_dequantize: null output");
  if (!aligned16(out)) return fail(WQ_ERR_ALIGN, "wq_dequantize: output not 16-byte aligned");
  return hip_status(wq::launch_dequant(w->format, dev_weight(w), w->experts, out,
                                       static_cast<hipStream_t>(stream)),
                    "wq_dequantize launch");
}

wq_status wq_quantize_ccq(const float* w, int64_t n, int64_t k, int32_t zp, int32_t refine,
                          uint8_t* codes, uint8_t* qscale, float* super_scale, float* code_scale,
                          float* code_zero, void* stream) {
  if (n <= 0 || k <= 0) return fail(WQ_ERR_ARG, "wq_quantize_ccq: n and k must be positive");
  if (k % 64 != 0) return fail(WQ_ERR_UNSUPPORTED, "wq_quantize_ccq: k = %lld is not a multiple of 64", (long long)k);
  if (k > 131072) return fail(WQ_ERR_UNSUPPORTED, "wq_quantize_ccq: k = %lld above 131072", (long long)k);
  if (n > 0x7FFFFFFFll) return fail(WQ_ERR_UNSUPPORTED, "wq_quantize_ccq: n must be below 2^31");
  if (zp < 0 || zp > 127) return fail(WQ_ERR_UNSUPPORTED, "wq_quantize_ccq: zero point must lie in 0..127");
  if (refine < 0 || refine > 3) return fail(WQ_ERR_ARG, "wq_quantize_ccq: refine is a mask of 1 and 2");
  if (!w || !codes || !qscale || !super_scale || !code_scale || !code_zero)
    return fail(WQ_ERR_ARG, "wq_quantize_ccq: null pointer");
  if (!aligned16(w)) return fail(WQ_ERR_ALIGN, "wq_quantize_ccq: w not 16-byte aligned");
  return hip_status(wq::launch_ccq_encode(w, n, k, zp, refine, codes, qscale, super_scale,
                                          code_scale, code_zero, static_cast<hipStream_t>(stream)),
                    "wq_quantize_ccq launch");
}

wq_status wq_gemm(const uint16_t* x, int64_t m, const wq_weight* w, uint16_t* y, void* stream) {
  wq_status st = check_weight(w, "wq_gemm");
  if (st != WQ_OK) return st;
  if ((st = check_product_zp(w, "wq_gemm")) != WQ_OK) return st;
  if (m < 0) return fail(WQ_ERR_ARG, "wq_gemm: negative m");
  if (w->experts != 1) return fail(WQ_ERR_ARG, "wq_gemm: a dense weight has experts == 1");
  if (m == 0) return WQ_OK;
  if (!x || !y) return fail(WQ_ERR_ARG, "wq_gemm: null x or y");
  if (!aligned16(x) || !aligned16(y)) return fail(WQ_ERR_ALIGN, "wq_gemm: x or y not 16-byte aligned");
  if (m > (1ll << 31)) return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: m must be below 2^31");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m > kSkinnyMaxRows && has_tiled(w)) {
    wq::TiledArgs t{};
    t.w0 = dev_weight(w);
    t.w1 = t.w0;
    t.a = x;
    t.a_stride = w->k;
    t.out = y;
    t.out_stride = w->n;
    t.M = m;
    t.N = w->n;
    t.K = w->k;
    const int64_t bm = wq::tiled_rows();
    return hip_status(wq::launch_tiled(w->format, wq::MODE_DENSE, t, (m + bm - 1) / bm, s),
                      "wq_gemm launch");
  }
  wq::SkinnyArgs a{};
  a.w0 = dev_weight(w);
  a.w1 = a.w0;
  a.a = x;
  a.a_stride = w->k;
  a.out = y;
  a.out_stride = w->n;
  a.M = m;
  a.N = w->n;
  a.K = w->k;
  const int mt = (m <= 16) ? 1 : 2;
  const int64_t rows = 16 * mt;
  const int64_t n_tiles = (w->n + 15) / 16;
  // Split K across the 4 waves when 4-tile workgroups would leave the 256 CUs idle.
  const int ksplit = (n_tiles / 4 < 512 && w->k % 256 == 0) ? 4 : 1;
  // Few rows whose activations fit in LDS whole: the single-staging kernel (lower latency).
  if (ksplit == 4 && wq::gemv_fits(m, w->n, w->k))
    return hip_status(wq::launch_gemv(w->format, a, s), "wq_gemm launch");
  // One launch covers at most kMaxGridZ row blocks (the grid's z extent); more rows (group-64
  // INT8 runs this kernel for every row count) take further launches on the same stream.
  const int64_t chunk = kMaxGridZ * rows;
  for (int64_t r0 = 0; r0 < m; r0 += chunk) {
    const int64_t mr = m - r0 < chunk ? m - r0 : chunk;
    a.a = x + r0 * w->k;
    a.out = y + r0 * w->n;
    a.M = mr;
    st = hip_status(wq::launch_skinny(w->format, wq::MODE_DENSE, mt, ksplit, a, 1,
                                      (mr + rows - 1) / rows, s),
                    "wq_gemm launch");
    if (st != WQ_OK) return st;
  }
  return WQ_OK;
}

size_t wq_moe_workspace_bytes(int64_t t, int32_t topk, int32_t experts, int64_t hidden,
                              int64_t inter) {
  if (t < 0 || topk <= 0 || experts <= 0 || hidden <= 0 || inter <= 0) return 0;
  return moe_layout(nullptr, t, topk, experts, hidden, inter).bytes;
}

size_t wq_moe_route_workspace_bytes(int64_t t, int32_t topk, int32_t experts) {
  if (t < 0 || topk <= 0 || experts <= 0 || experts > kMaxExperts || (int64_t)t * topk > (1ll << 30))
    return 0;
  return sizeof(int32_t) * (size_t)wq::route_table_entries(t * topk, experts);
}

wq_status wq_moe_route(const int32_t* topk_ids, int64_t t, int32_t topk, int32_t experts,
                       int32_t* expert_offsets, int32_t* sorted_pairs, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!ws && ws_bytes) return fail(WQ_ERR_ARG, "wq_moe_route: a workspace size without a workspace");
  if (t < 0 || topk <= 0 || experts <= 0) return fail(WQ_ERR_ARG, "wq_moe_route: bad sizes");
  if (experts > kMaxExperts) return fail(WQ_ERR_UNSUPPORTED, "wq_moe_route: at most %d experts", kMaxExperts);
  if ((int64_t)t * topk > (1ll << 30)) return fail(WQ_ERR_UNSUPPORTED, "wq_moe_route: too many pairs");
  const size_t need = wq_moe_route_workspace_bytes(t, topk, experts);
  if (ws && ws_bytes < need)
    return fail(WQ_ERR_WORKSPACE, "wq_moe_route: workspace %zu < %zu bytes", ws_bytes, need);
  if (!expert_offsets || (t > 0 && (!topk_ids || !sorted_pairs)))
    return fail(WQ_ERR_ARG, "wq_moe_route: null pointer");
  if (ws && !aligned16(ws)) return fail(WQ_ERR_ALIGN, "wq_moe_route: ws must be 16-byte aligned");
  return hip_status(wq::launch_route(topk_ids, t * topk, experts, expert_offsets, sorted_pairs,
                                     ws && need ? static_cast<int32_t*>(ws) : nullptr,
                                     static_cast<hipStream_t>(stream)),
                    "wq_moe_route launch");
}

namespace {

// Shared checks of the gate/up pair and the down matrix of one MoE layer.
wq_status check_moe_weights(const wq_weight* gate, const wq_weight* up, const wq_weight* down,
                            const char* what) {
  wq_status st;
  if (gate && (st = check_weight(gate, what)) != WQ_OK) return st;
  if (up && (st = check_weight(up, what)) != WQ_OK) return st;
  if (down && (st = check_weight(down, what)) != WQ_OK) return st;
  if (gate && (st = check_product_zp(gate, what)) != WQ_OK) return st;
  if (down && (st = check_product_zp(down, what)) != WQ_OK) return st;
  const wq_weight* any = gate ? gate : down;
  if (any->experts > kMaxExperts) return fail(WQ_ERR_UNSUPPORTED, "%s: at most %d experts", what, kMaxExperts);
  if (gate && up) {
    if (up->experts != gate->experts || up->n != gate->n || up->k != gate->k)
      return fail(WQ_ERR_ARG, "%s: gate and up must both be [E][inter][hidden]", what);
    if (gate->format != up->format || gate->group != up->group || gate->zp != up->zp)
      return fail(WQ_ERR_UNSUPPORTED, "%s: gate and up must share format, group and zp", what);
  }
  if (gate && down && (down->experts != gate->experts || down->n != gate->k || down->k != gate->n))
    return fail(WQ_ERR_ARG, "%s: down must be [E][hidden][inter] for gate/up [E][inter][hidden]", what);
  return WQ_OK;
}

int moe_row_tiles(int64_t t, int32_t topk, int64_t experts) {
  // 16 activation rows per pass while experts average at most 8 routed rows, else 32.
  return ((double)t * topk / (double)experts <= 8.0) ? 1 : 2;
}

// The single-staging kernel for MoE products of at most 16 tokens (so an expert's rows, one per
// token routed to it, take one pass of up to 16 rows when they fit) with few workgroups: the
// waves per workgroup, or 0 for the chunked kernel.
int moe_gemv_split(int mode, const wq_weight* w, int64_t t, int32_t topk) {
  if (t > 16) return 0;
  const int64_t active = t * topk < w->experts ? t * topk : w->experts;
  return wq::gemv_moe_split(w->format, mode, active, w->n, w->k);
}

bool moe_tiled(const wq_weight* w, int64_t t, int32_t topk) {
  return has_tiled(w) && (double)t * topk / (double)w->experts >= kMoeTiledRows;
}

int64_t moe_tile_bound(int64_t t, int32_t topk, int64_t experts) {
  const int64_t bm = wq::tiled_rows();
  return (t * topk + bm - 1) / bm + experts;
}

wq::TiledArgs moe_tiled_args(const int32_t* offsets, const int32_t* sorted, int32_t topk,
                             int64_t experts) {
  wq::TiledArgs a{};
  a.offsets = offsets;
  a.sorted_pairs = sorted;
  a.topk = topk;
  a.experts = (int32_t)experts;
  return a;
}

hipError_t run_gate_up(const uint16_t* x, int64_t t, const int32_t* offsets, const int32_t* sorted,
                       int32_t topk, const wq_weight* gate, const wq_weight* up, uint16_t* h,
                       hipStream_t s) {
  if (moe_tiled(gate, t, topk)) {
    wq::TiledArgs a = moe_tiled_args(offsets, sorted, topk, gate->experts);
    a.w0 = dev_weight(gate);
    a.w1 = dev_weight(up);
    a.a = x;
    a.a_stride = gate->k;
    a.out = h;
    a.out_stride = gate->n;
    a.N = gate->n;
    a.K = gate->k;
    return wq::launch_tiled(gate->format, wq::MODE_GATEUP, a, moe_tile_bound(t, topk, gate->experts), s);
  }
  wq::SkinnyArgs a{};
  a.offsets = offsets;
  a.sorted_pairs = sorted;
  a.topk = topk;
  a.w0 = dev_weight(gate);
  a.w1 = dev_weight(up);
  a.a = x;
  a.a_stride = gate->k;
  a.out = h;
  a.out_stride = gate->n;
  a.N = gate->n;
  a.K = gate->k;
  if (const int ks = moe_gemv_split(wq::MODE_GATEUP, gate, t, topk))
    return wq::launch_gemv_moe(gate->format, wq::MODE_GATEUP, a, gate->experts, ks, s);
  return wq::launch_skinny(gate->format, wq::MODE_GATEUP, moe_row_tiles(t, topk, gate->experts), 1,
                           a, gate->experts, 1, s);
}

hipError_t run_down(const uint16_t* h, int64_t t, int32_t topk, const int32_t* offsets,
                    const int32_t* sorted, const wq_weight* down, float* d, hipStream_t s) {
  if (moe_tiled(down, t, topk)) {
    wq::TiledArgs a = moe_tiled_args(offsets, sorted, topk, down->experts);
    a.w0 = dev_weight(down);
    a.w1 = a.w0;
    a.a = h;
    a.a_stride = down->k;
    a.out = d;
    a.out_stride = down->n;
    a.N = down->n;
    a.K = down->k;
    return wq::launch_tiled(down->format, wq::MODE_DOWN, a, moe_tile_bound(t, topk, down->experts), s);
  }
  wq::SkinnyArgs a{};
  a.offsets = offsets;
  a.sorted_pairs = sorted;
  a.topk = topk;
  a.w0 = dev_weight(down);
  a.w1 = a.w0;
  a.a = h;
  a.a_stride = down->k;
  a.out = d;
  a.out_stride = down->n;
  a.N = down->n;
  a.K = down->k;
  if (const int ks = moe_gemv_split(wq::MODE_DOWN, down, t, topk))
    return wq::launch_gemv_moe(down->format, wq::MODE_DOWN, a, down->experts, ks, s);
  return wq::launch_skinny(down->format, wq::MODE_DOWN, moe_row_tiles(t, topk, down->experts), 1,
                           a, down->experts, 1, s);
}

}  // namespace

wq_status wq_moe_gate_up(const uint16_t* x, int64_t t, const int32_t* expert_offsets,
                         const int32_t* sorted_pairs, int32_t topk, const wq_weight* gate,
                         const wq_weight* up, uint16_t* h, void* stream) {
  if (!gate || !up) return fail(WQ_ERR_ARG, "wq_moe_gate_up: null descriptor");
  wq_status st = check_moe_weights(gate, up, nullptr, "wq_moe_gate_up");
  if (st != WQ_OK) return st;
  if (t < 0 || topk <= 0) return fail(WQ_ERR_ARG, "wq_moe_gate_up: bad sizes");
  if (t == 0) return WQ_OK;
  if ((int64_t)t * topk > (1ll << 30)) return fail(WQ_ERR_UNSUPPORTED, "wq_moe_gate_up: too many pairs");
  if (!x || !expert_offsets || !sorted_pairs || !h) return fail(WQ_ERR_ARG, "wq_moe_gate_up: null pointer");
  if (!aligned16(x) || !aligned16(h)) return fail(WQ_ERR_ALIGN, "wq_moe_gate_up: x and h must be 16-byte aligned");
  return hip_status(run_gate_up(x, t, expert_offsets, sorted_pairs, topk, gate, up, h,
                                static_cast<hipStream_t>(stream)),
                    "wq_moe_gate_up launch");
}

wq_status wq_moe_down(const uint16_t* h, int64_t t, int32_t topk, const int32_t* expert_offsets,
                      const int32_t* sorted_pairs, const wq_weight* down, float* d, void* stream) {
  if (!down) return fail(WQ_ERR_ARG, "wq_moe_down: null descriptor");
  wq_status st = check_moe_weights(nullptr, nullptr, down, "wq_moe_down");
  if (st != WQ_OK) return st;
  if (t < 0 || topk <= 0) return fail(WQ_ERR_ARG, "wq_moe_down: bad sizes");
  if (t == 0) return WQ_OK;
  if ((int64_t)t * topk > (1ll << 30)) return fail(WQ_ERR_UNSUPPORTED, "wq_moe_down: too many pairs");
  if (!h || !expert_offsets || !sorted_pairs || !d) return fail(WQ_ERR_ARG, "wq_moe_down: null pointer");
  if (!aligned16(h) || !aligned16(d)) return fail(WQ_ERR_ALIGN, "wq_moe_down: h and d must be 16-byte aligned");
  return hip_status(run_down(h, t, topk, expert_offsets, sorted_pairs, down, d,
                             static_cast<hipStream_t>(stream)),
                    "wq_moe_down launch");
}

wq_status wq_moe_combine(const float* d, const float* topk_weights, int64_t t, int32_t topk,
                         int64_t hidden, uint16_t* y, void* stream) {
  if (t < 0 || topk <= 0 || hidden <= 0) return fail(WQ_ERR_ARG, "wq_moe_combine: bad sizes");
  if (hidden % 4 != 0) return fail(WQ_ERR_UNSUPPORTED, "wq_moe_combine: hidden must be a multiple of 4");
  if (t == 0) return WQ_OK;
  if (!d || !topk_weights || !y) return fail(WQ_ERR_ARG, "wq_moe_combine: null pointer");
  if (!aligned16(d) || !aligned16(y)) return fail(WQ_ERR_ALIGN, "wq_moe_combine: d and y must be 16-byte aligned");
  return hip_status(wq::launch_combine(d, topk_weights, t, topk, hidden, y, static_cast<hipStream_t>(stream)),
                    "wq_moe_combine launch");
}

}  // extern "C"

namespace {

// The body of wq_moe_ffn once a workspace is at hand: validation, then the four stages.
// `what` names the entry point in error messages; a null ws means the caller's ws was null.
wq_status moe_ffn_in(const char* what, const uint16_t* x, int64_t t, int64_t hidden,
                     const int32_t* topk_ids, const float* topk_weights, int32_t topk,
                     const wq_weight* gate, const wq_weight* up, const wq_weight* down,
                     uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  if (!gate || !up || !down) return fail(WQ_ERR_ARG, "%s: null descriptor", what);
  wq_status st = check_moe_weights(gate, up, down, what);
  if (st != WQ_OK) return st;
  if (t < 0 || topk <= 0 || hidden <= 0) return fail(WQ_ERR_ARG, "%s: bad sizes", what);
  if (gate->k != hidden) return fail(WQ_ERR_ARG, "%s: gate/up k must equal hidden", what);
  if (hidden % 4 != 0) return fail(WQ_ERR_UNSUPPORTED, "%s: hidden must be a multiple of 4", what);
  if (t == 0) return WQ_OK;
  if (!x || !topk_ids || !topk_weights || !y || !ws) return fail(WQ_ERR_ARG, "%s: null pointer", what);
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws))
    return fail(WQ_ERR_ALIGN, "%s: x, y and ws must be 16-byte aligned", what);
  if ((int64_t)t * topk > (1ll << 30)) return fail(WQ_ERR_UNSUPPORTED, "%s: too many pairs", what);
  const int64_t E = gate->experts, I = gate->n;
  MoeWs L = moe_layout(ws, t, topk, (int32_t)E, hidden, I);
  if (ws_bytes < L.bytes)
    return fail(WQ_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", what, ws_bytes, L.bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = wq::launch_route(topk_ids, t * topk, (int32_t)E, L.offsets, L.sorted,
                                  L.route_table, s);
  if (e != hipSuccess) return hip_status(e, "moe ffn route");
  e = run_gate_up(x, t, L.offsets, L.sorted, topk, gate, up, L.h, s);
  if (e != hipSuccess) return hip_status(e, "moe ffn gate/up");
  e = run_down(L.h, t, topk, L.offsets, L.sorted, down, L.d, s);
  if (e != hipSuccess) return hip_status(e, "moe ffn down");
  return hip_status(wq::launch_combine(L.d, topk_weights, t, topk, hidden, y, s), "moe ffn combine");
}

}  // namespace

extern "C" {

wq_status wq_moe_ffn(const uint16_t* x, int64_t t, int64_t hidden, const int32_t* topk_ids,
                     const float* topk_weights, int32_t topk, const wq_weight* gate,
                     const wq_weight* up, const wq_weight* down, uint16_t* y, void* ws,
                     size_t ws_bytes, void* stream) {
  return moe_ffn_in("wq_moe_ffn", x, t, hidden, topk_ids, topk_weights, topk, gate, up, down, y,
                    ws, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// wq_moe_ffn_noalloc: wq_moe_ffn with its workspace in `scratch`, a file-scope device array of
// WQ_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its device address is
// taken once per device with hipGetSymbolAddress (with that device current) and kept in
// g_scratch_dev; kernels only ever receive that address.  Every call on one GPU shares that
// GPU's array (calls that overlap on one GPU race).  Nothing in it needs clearing: each call
// writes every workspace element it reads (offsets, the sorted pairs, h and d of its pairs).
// ---------------------------------------------------------------------------------------------
namespace {

static __device__ __align__(256) uint8_t scratch[WQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_dev[kMaxDevices];

// The current device's address of `scratch` (looked up on the device's first call).
wq_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "wq_moe_ffn_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(WQ_ERR_UNSUPPORTED, "wq_moe_ffn_noalloc: device id %d is %d or more", dev, kMaxDevices);
  void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "wq_moe_ffn_noalloc: hipGetSymbolAddress");
    if (!p) return fail(WQ_ERR_HIP, "wq_moe_ffn_noalloc: no device address for the scratch array");
    g_scratch_dev[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return WQ_OK;
}

}  // namespace

extern "C" wq_status wq_moe_ffn_noalloc(const uint16_t* x, int64_t t, int64_t hidden,
                                        const int32_t* topk_ids, const float* topk_weights,
                                        int32_t topk, const wq_weight* gate, const wq_weight* up,
                                        const wq_weight* down, uint16_t* y, void* stream) {
  if (!gate) return fail(WQ_ERR_ARG, "wq_moe_ffn_noalloc: null descriptor");
  const size_t need = wq_moe_workspace_bytes(t, topk, (int32_t)gate->experts, hidden, gate->n);
  if (need > (size_t)WQ_NOALLOC_SCRATCH_BYTES)
    return fail(WQ_ERR_WORKSPACE,
                "wq_moe_ffn_noalloc: this call needs %zu bytes of workspace, above the %zu-byte "
                "scratch array (use wq_moe_ffn with a workspace)",
                need, (size_t)WQ_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  wq_status st = scratch_address(&ws);
  if (st != WQ_OK) return st;
  return moe_ffn_in("wq_moe_ffn_noalloc", x, t, hidden, topk_ids, topk_weights, topk, gate, up,
                    down, y, ws, (size_t)WQ_NOALLOC_SCRATCH_BYTES, stream);
}
