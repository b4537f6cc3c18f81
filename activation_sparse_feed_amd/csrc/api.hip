// C ABI of the activation-sparse gated FFN (declared in include/sffn.h):
// argument validation on the host, workspace carving and kernel launches.
// Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sffn.h"
#include "launch.h"
#include "route.cuh"

namespace {

using namespace sffn;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
size_t elt_bytes(int dtype) { return dtype == SFFN_BF16 ? 2 : 4; }

// Shape checks shared by every call.
int32_t check_shape(const sffn_shape* s) {
  if (s == nullptr) return SFFN_ERR_ARG;
  if (s->T < 0 || s->d_model <= 0 || s->d_ff <= 0 || s->cap < 0 || s->tile <= 0)
    return SFFN_ERR_ARG;
  if (s->dtype != SFFN_F32 && s->dtype != SFFN_BF16) return SFFN_ERR_ARG;
  if (s->tile != 128) return SFFN_ERR_UNSUPPORTED;
  if (s->d_ff % 128 != 0 || s->d_ff > 65535) return SFFN_ERR_UNSUPPORTED;
  if (s->d_model % 8 != 0 || s->d_model < 8 || s->d_model > 8192) return SFFN_ERR_UNSUPPORTED;
  if (s->cap > 128) return SFFN_ERR_UNSUPPORTED;
  return SFFN_OK;
}

bool ptrs_ok(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr || !aligned16(p)) return false;
  return true;
}

size_t dense_ws(const sffn_shape* s) {
  size_t n = align256((size_t)s->T * s->d_ff * elt_bytes(s->dtype));
  if (dense_skinny_ok(s->dtype, s->T, s->d_model, s->d_ff))
    n += align256(dense_skinny_partial_bytes(s->d_model, s->d_ff));
  return n;
}

size_t pack_ws(const sffn_shape* s) {
  return align256((size_t)s->T * 4) + align256((size_t)s->d_ff * 4) +
         gate_workspace_bytes(s->dtype, s->T, s->d_model, s->d_ff);
}

// The buffer-load GEMMs address an activation matrix, and the down weight,
// with 32-bit byte offsets.
bool act_bytes_too_large(const sffn_shape* s) {
  return (uint64_t)s->T * (uint64_t)s->d_model * elt_bytes(s->dtype) >= (1ull << 31) ||
         (uint64_t)s->d_ff * (uint64_t)s->d_model * elt_bytes(s->dtype) >= (1ull << 31);
}

bool routed_fast_path(const sffn_shape* s) {
  return s->dtype == SFFN_BF16 && s->d_model % 32 == 0;
}

size_t hybrid_ws(const sffn_shape* s) {
  size_t n = route_workspace_bytes(s->T) + align256((size_t)s->T * s->d_ff * elt_bytes(s->dtype));
  if (routed_fast_path(s)) n += align256(routed_partial_bytes(s->T, s->d_model, s->d_ff));
  return n;
}

// twell_pack_l1: the pack workspace, then the per-(row, tile) L1 sums and the
// reduction's block sums.
size_t pack_l1_ws(const sffn_shape* s) {
  return pack_ws(s) + align256((size_t)s->T * (s->d_ff / 128) * 4) + align256(l1_ws_bytes());
}

// The general backward (float32, bf16 widths not a multiple of 512): the
// complete lists' arrays (count, idx, val at capacity backward_general_cap())
// after twell_pack's workspace, then the backward's own.
size_t backward_general_lists_bytes(const sffn_shape* s) {
  const size_t nt = (size_t)s->d_ff / 128, cap = (size_t)backward_general_cap();
  return align256((size_t)s->T * nt * 2) + align256((size_t)s->T * nt * cap * 2) +
         align256((size_t)s->T * nt * cap * elt_bytes(s->dtype));
}

size_t backward_ws(const sffn_shape* s, int max_routed) {
  if (backward_general(s->dtype, s->d_model))
    return pack_ws(s) + backward_general_lists_bytes(s) +
           backward_general_workspace_bytes(s->T, s->d_ff);
  return align256((size_t)s->T * 4) + align256((size_t)s->d_ff * 4) +
         backward_workspace_bytes(s->T, s->d_ff, s->d_model, s->cap, max_routed);
}

size_t convert_ws(const sffn_shape* s) {
  return align256((size_t)s->T * 4) + align256((size_t)s->d_ff * 4);
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? SFFN_OK : SFFN_ERR_HIP; }

}  // namespace

// Scratch memory of twell_pack_noalloc: a static device array instead of a
// caller workspace, for callers that cannot allocate.  Every GPU the library
// runs on holds its own copy until the process ends.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_addr[kMaxDevices];  // device address of `scratch`, per device, set once

// Device address of the scratch array on the device that runs `stream`.  The
// array's name is only a host-side handle: kernels must be given this address.
int32_t device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return SFFN_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_addr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SFFN_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return SFFN_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return SFFN_ERR_HIP;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return SFFN_OK;
}

// Guard band of the activity decision (see the TwELL epilogue), with
// u = 2^-24 and S = sum_k |x_k w_k| <= ||x|| ||w||.
// bf16: one v_mfma_f32_16x16x32_bf16 was measured (sffn_probe_mfma_step) to
// err by at most u (8 max_k |a_k b_k| + 2 |result|): its 32 products are
// aligned to the largest and truncated a little below float32 precision, then
// added to the accumulator with one rounding.  Over the K/32 chained
// instructions the truncations add up to at most 8 u S (every product is in
// one instruction) and the roundings to 2 u (K/32) S; the bias add is one more
// rounding.  The band 4 u (K/32 + 2) ||x|| ||w|| + 4 u |b| covers that total,
// 2 u (K/32) + 9 u, for every K >= 32.
// float32: one FMA rounding per k, K u S; the band 4 u (K + 2) covers it.
GuardBand guard_band(const sffn_shape* s) {
  const float u4 = 0x1p-22f;
  if (s->dtype == SFFN_BF16) return GuardBand{u4 * (float)(s->d_model / 32 + 2), u4};
  return GuardBand{u4 * (float)(s->d_model + 2), u4};
}

}  // namespace

extern "C" {

int32_t twell_weight_norms(const sffn_shape* shape, const void* wg_t, float* wg_norms,
                           void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (!ptrs_ok({wg_t, wg_norms})) return SFFN_ERR_ARG;
  return hip_status(launch_row_norms(shape->dtype, wg_t, shape->d_ff, wg_norms, nullptr, 0,
                                     nullptr, shape->d_model, (hipStream_t)stream));
}

namespace {

// twell_pack, with the L1 regulariser's per-(row, tile) sums when l1_part is set.
int32_t pack_impl(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                  const float* wg_norms, uint16_t* count, uint16_t* idx, void* val,
                  void* workspace, float* l1_part, size_t* l1_n, hipStream_t s) {
  float* xn = (float*)workspace;
  float* wn = (float*)((char*)workspace + align256((size_t)shape->T * 4));
  void* gws = (char*)wn + align256((size_t)shape->d_ff * 4);
  const int rows_x = gate_needs_xnorm(shape->dtype, shape->T, shape->d_model) ? shape->T : 0;
  const int rows_w = wg_norms ? 0 : shape->d_ff;
  hipError_t e = launch_row_norms(shape->dtype, x, rows_x, xn, wg_t, rows_w, wn, shape->d_model, s);
  if (e != hipSuccess) return SFFN_ERR_HIP;
  return hip_status(launch_gate_twell(shape->dtype, x, wg_t, b_g, xn, wg_norms ? wg_norms : wn,
                                      count, idx, val, shape->T, shape->d_model, shape->d_ff,
                                      shape->cap, guard_band(shape), gws, l1_part, l1_n, s));
}

int32_t check_pack(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                   const float* wg_norms, uint16_t* count, uint16_t* idx, void* val) {
  if (!ptrs_ok({x, wg_t, count}) || (b_g && !aligned16(b_g)) || (wg_norms && !aligned16(wg_norms)))
    return SFFN_ERR_ARG;
  if (shape->cap > 0 && !ptrs_ok({idx, val})) return SFFN_ERR_ARG;
  return SFFN_OK;
}

}  // namespace

int32_t twell_pack(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                   const float* wg_norms, uint16_t* count, uint16_t* idx, void* val,
                   void* workspace, size_t ws_bytes, void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (shape->T == 0) return SFFN_OK;
  st = check_pack(shape, x, wg_t, b_g, wg_norms, count, idx, val);
  if (st != SFFN_OK) return st;
  if (workspace == nullptr || !aligned16(workspace) || ws_bytes < pack_ws(shape))
    return SFFN_ERR_WORKSPACE;
  if (act_bytes_too_large(shape)) return SFFN_ERR_UNSUPPORTED;
  return pack_impl(shape, x, wg_t, b_g, wg_norms, count, idx, val, workspace, nullptr, nullptr,
                   (hipStream_t)stream);
}

int32_t twell_pack_noalloc(const sffn_shape* shape, const void* x, const void* wg_t,
                           const float* b_g, const float* wg_norms, uint16_t* count,
                           uint16_t* idx, void* val, void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (shape->T == 0) return SFFN_OK;
  st = check_pack(shape, x, wg_t, b_g, wg_norms, count, idx, val);
  if (st != SFFN_OK) return st;
  if (act_bytes_too_large(shape)) return SFFN_ERR_UNSUPPORTED;
  if (pack_ws(shape) > kNoAllocScratchBytes) return SFFN_ERR_TOO_LARGE;
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  st = device_scratch(s, &ws);
  if (st != SFFN_OK) return st;
  return pack_impl(shape, x, wg_t, b_g, wg_norms, count, idx, val, ws, nullptr, nullptr, s);
}

size_t twell_pack_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int32_t twell_pack_l1(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                      const float* wg_norms, uint16_t* count, uint16_t* idx, void* val,
                      float lambda, float* l1_value, void* workspace, size_t ws_bytes,
                      void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (!ptrs_ok({l1_value}) || !(lambda == lambda)) return SFFN_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (shape->T == 0) {
    return hip_status(launch_l1_zero(l1_value, s));  // the mean over no tokens: 0
  }
  st = check_pack(shape, x, wg_t, b_g, wg_norms, count, idx, val);
  if (st != SFFN_OK) return st;
  if (workspace == nullptr || !aligned16(workspace) || ws_bytes < pack_l1_ws(shape))
    return SFFN_ERR_WORKSPACE;
  if (act_bytes_too_large(shape)) return SFFN_ERR_UNSUPPORTED;
  float* part = (float*)((char*)workspace + pack_ws(shape));
  const size_t n = (size_t)shape->T * (shape->d_ff / 128);
  void* red = (char*)part + align256(n * 4);
  size_t parts = n;
  st = pack_impl(shape, x, wg_t, b_g, wg_norms, count, idx, val, workspace, part, &parts, s);
  if (st != SFFN_OK) return st;
  return hip_status(launch_l1_reduce(part, parts, (double)lambda / (double)shape->T, red, l1_value,
                                     s));
}

int32_t sparse_ffn_fwd(const sffn_shape* shape, const void* x, const void* wu_t, const void* wd,
                       const uint16_t* count, const uint16_t* idx, const void* val, void* y,
                       void* workspace, size_t ws_bytes, void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (shape->T == 0) return SFFN_OK;
  if (!ptrs_ok({x, wu_t, wd, count, y})) return SFFN_ERR_ARG;
  if (shape->cap > 0 && !ptrs_ok({idx, val})) return SFFN_ERR_ARG;
  const int nt = shape->d_ff / 128;
  const size_t need = sparse_workspace_bytes(shape->dtype, shape->T, nt, shape->d_model, shape->cap);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || ws_bytes < need))
    return SFFN_ERR_WORKSPACE;
  return hip_status(launch_sparse_updown(shape->dtype, x, wu_t, wd, count, idx, val, y,
                                         workspace, shape->T, shape->d_model, nt, shape->cap,
                                         (hipStream_t)stream));
}

int32_t sparse_ffn_fwd_union(const sffn_shape* shape, const void* x, const void* wu_t,
                             const void* wd, const uint16_t* count, const uint16_t* idx,
                             const void* val, void* y, void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (!union_supported(shape->dtype, shape->d_model, shape->cap)) return SFFN_ERR_UNSUPPORTED;
  if (shape->T == 0) return SFFN_OK;
  if (!ptrs_ok({x, wu_t, wd, count, y})) return SFFN_ERR_ARG;
  if (shape->cap > 0 && !ptrs_ok({idx, val})) return SFFN_ERR_ARG;
  return hip_status(launch_sparse_union(x, wu_t, wd, count, idx, val, y, shape->T,
                                        shape->d_model, shape->d_ff / 128, shape->cap,
                                        (hipStream_t)stream));
}

int32_t hybrid_route(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                     const void* wu_t, const void* wd, const uint16_t* count, int32_t* routed,
                     int32_t* n_routed, void* workspace, size_t ws_bytes, void* y, void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (shape->T == 0) return SFFN_OK;
  if (!ptrs_ok({x, wg_t, wu_t, wd, count, routed, n_routed, y}) || (b_g && !aligned16(b_g)))
    return SFFN_ERR_ARG;
  if (workspace == nullptr || !aligned16(workspace) || ws_bytes < hybrid_ws(shape))
    return SFFN_ERR_WORKSPACE;
  if (act_bytes_too_large(shape)) return SFFN_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const int T = shape->T, K = shape->d_model, N = shape->d_ff;
  void* h = (char*)workspace + route_workspace_bytes(T);
  hipError_t e = hipSuccess;
  if (routed_fast_path(shape)) {
    // the MFMA fallback's gate+up kernel compacts the routed rows itself:
    // from the TwELL counts (few tokens) or from the routed-row mask
    const bool fused_route = T <= kRouteBlock;
    uint16_t* mask = (uint16_t*)workspace;
    if (!fused_route) {
      e = launch_route_mask(count, T, N / 128, shape->cap, mask, s);
      if (e != hipSuccess) return SFFN_ERR_HIP;
    }
    float* partial = (float*)((char*)h + align256((size_t)T * N * elt_bytes(shape->dtype)));
    return hip_status(launch_routed_ffn(x, wg_t, b_g, wu_t, wd, h, y, partial, T, routed,
                                        n_routed, fused_route ? count : nullptr,
                                        fused_route ? nullptr : mask, N / 128, shape->cap, K, N,
                                        s));
  }
  e = launch_route(count, T, N / 128, shape->cap, routed, n_routed, workspace, s);
  if (e != hipSuccess) return SFFN_ERR_HIP;
  e = launch_dense_gateup(shape->dtype, x, wg_t, b_g, wu_t, h, T, routed, n_routed, K, N, s);
  if (e != hipSuccess) return SFFN_ERR_HIP;
  e = launch_down(shape->dtype, h, wd, y, T, routed, n_routed, N, K, s);
  return hip_status(e);
}

int32_t dense_ffn_ref(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                      const void* wu_t, const void* wd, void* workspace, size_t ws_bytes, void* y,
                      void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (shape->T == 0) return SFFN_OK;
  if (!ptrs_ok({x, wg_t, wu_t, wd, y}) || (b_g && !aligned16(b_g))) return SFFN_ERR_ARG;
  if (workspace == nullptr || !aligned16(workspace) || ws_bytes < dense_ws(shape))
    return SFFN_ERR_WORKSPACE;
  if (act_bytes_too_large(shape)) return SFFN_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const int T = shape->T, K = shape->d_model, N = shape->d_ff;
  if (dense_skinny_ok(shape->dtype, T, K, N)) {
    float* partial = (float*)((char*)workspace + align256((size_t)T * N * elt_bytes(shape->dtype)));
    return hip_status(launch_dense_skinny(x, wg_t, b_g, wu_t, wd, workspace, partial, y, T, K, N, s));
  }
  hipError_t e = launch_dense_gateup(shape->dtype, x, wg_t, b_g, wu_t, workspace, T, nullptr,
                                     nullptr, K, N, s);
  if (e != hipSuccess) return SFFN_ERR_HIP;
  return hip_status(launch_down(shape->dtype, workspace, wd, y, T, nullptr, nullptr, N, K, s));
}

int32_t gate_preact(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                    float* z, void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (shape->T == 0) return SFFN_OK;
  if (!ptrs_ok({x, wg_t, z}) || (b_g && !aligned16(b_g))) return SFFN_ERR_ARG;
  if (!preact_supported(shape->dtype, shape->d_model) || act_bytes_too_large(shape))
    return SFFN_ERR_UNSUPPORTED;
  return hip_status(launch_gate_preact(x, wg_t, b_g, z, shape->T, shape->d_model, shape->d_ff,
                                       nullptr, nullptr, (hipStream_t)stream));
}

namespace {

// Row norms for the converters' guard band: x always, wg_t unless given.
int32_t convert_norms(const sffn_shape* s, const void* x, const void* wg_t, const float* wg_norms,
                      void* workspace, float** xn, const float** wn, hipStream_t stream) {
  *xn = (float*)workspace;
  float* wbuf = (float*)((char*)workspace + align256((size_t)s->T * 4));
  *wn = wg_norms ? wg_norms : wbuf;
  return hip_status(launch_row_norms(s->dtype, x, s->T, *xn, wg_t, wg_norms ? 0 : s->d_ff, wbuf,
                                     s->d_model, stream));
}

int32_t check_convert(const sffn_shape* s, const float* z, const void* x, const void* wg_t,
                      const float* b_g, const float* wg_norms, void* workspace, size_t ws_bytes) {
  if (!ptrs_ok({z, x, wg_t}) || (b_g && !aligned16(b_g)) || (wg_norms && !aligned16(wg_norms)))
    return SFFN_ERR_ARG;
  if (workspace == nullptr || !aligned16(workspace) || ws_bytes < convert_ws(s))
    return SFFN_ERR_WORKSPACE;
  if (!preact_supported(s->dtype, s->d_model) || act_bytes_too_large(s))
    return SFFN_ERR_UNSUPPORTED;
  return SFFN_OK;
}

}  // namespace

int32_t twell_from_preact(const sffn_shape* shape, const float* z, const void* x,
                          const void* wg_t, const float* b_g, const float* wg_norms,
                          uint16_t* count, uint16_t* idx, void* val, void* workspace,
                          size_t ws_bytes, void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (shape->T == 0) return SFFN_OK;
  if (!ptrs_ok({count}) || (shape->cap > 0 && !ptrs_ok({idx, val}))) return SFFN_ERR_ARG;
  st = check_convert(shape, z, x, wg_t, b_g, wg_norms, workspace, ws_bytes);
  if (st != SFFN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  float* xn;
  const float* wn;
  st = convert_norms(shape, x, wg_t, wg_norms, workspace, &xn, &wn, s);
  if (st != SFFN_OK) return st;
  return hip_status(launch_twell_convert(z, x, wg_t, b_g, xn, wn, count, idx, val, shape->T,
                                         shape->d_model, shape->d_ff, shape->cap,
                                         guard_band(shape), s));
}

int32_t ell_from_preact(const sffn_shape* shape, int32_t width, const float* z, const void* x,
                        const void* wg_t, const float* b_g, const float* wg_norms,
                        uint16_t* ell_count, uint16_t* ell_idx, void* ell_val, void* workspace,
                        size_t ws_bytes, void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (width < 0 || width > shape->d_ff) return SFFN_ERR_ARG;
  if (shape->T == 0) return SFFN_OK;
  if (!ptrs_ok({ell_count}) || (width > 0 && !ptrs_ok({ell_idx, ell_val}))) return SFFN_ERR_ARG;
  st = check_convert(shape, z, x, wg_t, b_g, wg_norms, workspace, ws_bytes);
  if (st != SFFN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  float* xn;
  const float* wn;
  st = convert_norms(shape, x, wg_t, wg_norms, workspace, &xn, &wn, s);
  if (st != SFFN_OK) return st;
  return hip_status(launch_ell_convert(z, x, wg_t, b_g, xn, wn, width, ell_count, ell_idx,
                                       ell_val, shape->T, shape->d_model, shape->d_ff,
                                       guard_band(shape), nullptr, nullptr, s));
}

int32_t sparse_ffn_bwd(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                       const void* wu_t, const void* wd, const float* wg_norms,
                       const uint16_t* count, const uint16_t* idx, const void* val,
                       const int32_t* routed, const int32_t* n_routed, int32_t max_routed,
                       const void* gy, float l1_lambda, void* gx, float* gwg_t, float* gwu_t,
                       float* gwd, float* gb, void* workspace, size_t ws_bytes, void* stream) {
  int32_t st = check_shape(shape);
  if (st != SFFN_OK) return st;
  if (!(l1_lambda == l1_lambda) || max_routed < 0 || max_routed > shape->T) return SFFN_ERR_ARG;
  if (shape->T == 0) return SFFN_OK;
  if (!ptrs_ok({x, wg_t, wu_t, wd, count, routed, n_routed, gy, gx, gwg_t, gwu_t, gwd}) ||
      (b_g && !aligned16(b_g)) || (wg_norms && !aligned16(wg_norms)) || (gb && !aligned16(gb)))
    return SFFN_ERR_ARG;
  if (shape->cap > 0 && !ptrs_ok({idx, val})) return SFFN_ERR_ARG;
  if (workspace == nullptr || !aligned16(workspace) || ws_bytes < backward_ws(shape, max_routed))
    return SFFN_ERR_WORKSPACE;
  if (!backward_supported(shape->dtype, shape->d_model) || act_bytes_too_large(shape))
    return SFFN_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const float l1g = (float)((double)l1_lambda / (double)shape->T);
  if (backward_general(shape->dtype, shape->d_model)) {
    // complete activity lists of every row: twell_pack's kernels at the full
    // capacity (rows within the forward's capacity get their forward entries,
    // routed rows their complete lists; routed, n_routed and max_routed are
    // not needed)
    sffn_shape full = *shape;
    full.cap = backward_general_cap();
    const size_t nt = (size_t)shape->d_ff / 128, cap = (size_t)full.cap;
    char* p = (char*)workspace + pack_ws(shape);
    uint16_t* count2 = (uint16_t*)p;
    p += align256((size_t)shape->T * nt * 2);
    uint16_t* idx2 = (uint16_t*)p;
    p += align256((size_t)shape->T * nt * cap * 2);
    void* val2 = p;
    p += align256((size_t)shape->T * nt * cap * elt_bytes(shape->dtype));
    st = pack_impl(&full, x, wg_t, b_g, wg_norms, count2, idx2, val2, workspace, nullptr,
                   nullptr, s);
    if (st != SFFN_OK) return st;
    return hip_status(launch_backward_general(shape->dtype, x, wg_t, wu_t, wd, count2, idx2, val2,
                                              gy, gx, gwg_t, gwu_t, gwd, gb, shape->T,
                                              shape->d_model, shape->d_ff, l1g, p, s));
  }
  float* xn = (float*)workspace;
  float* wbuf = (float*)((char*)workspace + align256((size_t)shape->T * 4));
  void* bws = (char*)wbuf + align256((size_t)shape->d_ff * 4);
  hipError_t e = launch_row_norms(shape->dtype, x, shape->T, xn, wg_t, wg_norms ? 0 : shape->d_ff,
                                  wbuf, shape->d_model, s);
  if (e != hipSuccess) return SFFN_ERR_HIP;
  return hip_status(launch_backward(x, wg_t, b_g, wu_t, wd, xn, wg_norms ? wg_norms : wbuf, count,
                                    idx, val, routed, n_routed, gy, gx, gwg_t, gwu_t, gwd, gb,
                                    shape->T, shape->d_model, shape->d_ff, shape->cap, l1g,
                                    max_routed, guard_band(shape), bws, s));
}

size_t sparse_ffn_bwd_workspace_bytes(const sffn_shape* shape, int32_t max_routed) {
  if (check_shape(shape) != SFFN_OK || max_routed < 0 || max_routed > shape->T) return 0;
  return backward_ws(shape, max_routed);
}

size_t sffn_workspace_bytes(const sffn_shape* shape, int32_t which) {
  if (check_shape(shape) != SFFN_OK) return 0;
  switch (which) {
    case SFFN_WS_HYBRID: return hybrid_ws(shape);
    case SFFN_WS_DENSE: return dense_ws(shape);
    case SFFN_WS_SPARSE:
      return sparse_workspace_bytes(shape->dtype, shape->T, shape->d_ff / 128, shape->d_model,
                                    shape->cap);
    case SFFN_WS_PACK: return pack_ws(shape);
    case SFFN_WS_CONVERT: return convert_ws(shape);
    case SFFN_WS_PACK_L1: return pack_l1_ws(shape);
    case SFFN_WS_BACKWARD: return backward_ws(shape, shape->T);
    default: return 0;
  }
}

const char* sffn_strerror(int32_t status) {
  switch (status) {
    case SFFN_OK: return "success";
    case SFFN_ERR_ARG: return "invalid argument (null or misaligned pointer, bad size)";
    case SFFN_ERR_UNSUPPORTED: return "shape or parameter outside the supported range";
    case SFFN_ERR_WORKSPACE: return "workspace missing or too small";
    case SFFN_ERR_HIP: return "HIP launch or runtime error";
    case SFFN_ERR_TOO_LARGE:
      return "shape needs more scratch than twell_pack_noalloc holds (use twell_pack)";
    default: return "unknown sffn status";
  }
}

}  // extern "C"
