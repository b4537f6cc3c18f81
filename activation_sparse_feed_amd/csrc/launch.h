// Internal launchers of the sffn kernels (host side, C++ linkage).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sffn {

// Guard band of the TwELL activity decision: an entry is re-evaluated exactly
// when |z32| <= coef_xw * ||x_t|| * ||w_j|| + coef_b * |b_j|.
struct GuardBand {
  float coef_xw;
  float coef_b;
};

// Gate GEMM + TwELL epilogue.  gate_ws: gate_workspace_bytes() bytes (partial
// tiles of the few-token split-K kernels); xnorm is not read when
// gate_needs_xnorm() is false (those kernels compute the norms of x from the
// operands they load).
size_t gate_workspace_bytes(int dtype, int T, int K, int N);
bool gate_needs_xnorm(int dtype, int T, int K);
hipError_t launch_gate_twell(int dtype, const void* x, const void* wg_t, const float* b_g,
                             const float* xnorm, const float* wnorm, uint16_t* count,
                             uint16_t* idx, void* val, int T, int K, int N, int cap,
                             GuardBand gb, void* gate_ws, float* l1_part, size_t* l1_n,
                             hipStream_t stream);

// L1 regulariser value: *out = scale * (sum of the n per-(row, tile) sums in
// part), summed in float64 in a fixed order (two launches; ws: l1_ws_bytes()).
size_t l1_ws_bytes();
hipError_t launch_l1_zero(float* out, hipStream_t stream);
hipError_t launch_l1_reduce(const float* part, size_t n, double scale, void* ws, float* out,
                            hipStream_t stream);

// Separate-conversion baseline (bf16, K a multiple of 32): the gate GEMM
// storing the float32 pre-activation z [T, N] (bias added), and converters
// from z to TwELL and to a row-wise ELLPACK of the given width (ecount [T],
// eidx / eval [T, width]).  Same activity decision as launch_gate_twell.
// With rowmap / n_rows_dev (both may be null): output row m < *n_rows_dev is
// x row rowmap[m] (the backward's routed rows); max_rows (>= 0) caps the
// mapped rows (the output holds that many rows), else T.
bool preact_supported(int dtype, int K);
hipError_t launch_gate_preact(const void* x, const void* wg_t, const float* b_g, float* z, int T,
                              int K, int N, const int* rowmap, const int* n_rows_dev,
                              hipStream_t stream, int max_rows = -1);
hipError_t launch_twell_convert(const float* z, const void* x, const void* wg_t, const float* b_g,
                                const float* xnorm, const float* wnorm, uint16_t* count,
                                uint16_t* idx, void* val, int T, int K, int N, int cap,
                                GuardBand gb, hipStream_t stream);
hipError_t launch_ell_convert(const float* z, const void* x, const void* wg_t, const float* b_g,
                              const float* xnorm, const float* wnorm, int width,
                              uint16_t* ecount, uint16_t* eidx, void* eval, int T, int K, int N,
                              GuardBand gb, const int* rowmap, const int* n_rows_dev,
                              hipStream_t stream, int max_rows = -1);

// Backward through TwELL and the hybrid routing (bf16, d_model % 512 == 0,
// d_model <= 4096): gx [T, D] bf16, float32 weight gradients [N, D] and gb
// [N] (may be null).  l1g is added to gz of every active entry.  R: routed
// rows the workspace holds (backward_workspace_bytes(..., R)); if the forward
// routed more, gb and the first row of gx are set to NaN.  xnorm: ||x_t|| of every row; wnorm: ||wg_t[j]||.  ws:
// backward_workspace_bytes().
bool backward_supported(int dtype, int d_model);
// The general backward (float32, and bf16 widths not a multiple of 512; up
// to d_model 2048): from complete activity lists of every row (twell_pack at
// capacity backward_general_cap()): count [T, N/128], idx and val
// [T, N/128, cap] (val in the element type); workspace
// backward_general_workspace_bytes(T, N).
bool backward_general(int dtype, int d_model);
int backward_general_cap();
size_t backward_general_workspace_bytes(int T, int N);
hipError_t launch_backward_general(int dtype, const void* x, const void* wg_t, const void* wu_t,
                                   const void* wd, const uint16_t* count, const uint16_t* idx,
                                   const void* val, const void* gy, void* gx, float* gwg_t,
                                   float* gwu_t, float* gwd, float* gb, int T, int D, int N,
                                   float l1g, void* ws, hipStream_t stream);
size_t backward_workspace_bytes(int T, int N, int D, int cap, int R);

// The routed rows' backward on MFMA tiles (backward_routed.hip): launched when
// at least kDenseRoutedTokens tokens and room for kDenseRoutedRows routed
// rows; it takes the routed rows when the device-side count reaches
// kDenseRoutedRows (the per-entry kernels take them otherwise).
constexpr int kDenseRoutedRows = 1024;
constexpr int kDenseRoutedTokens = 8192;
inline bool routed_dense_launch(int T, int R) {
  return T >= kDenseRoutedTokens && R >= kDenseRoutedRows;
}
size_t routed_dense_workspace_bytes(int N, int D, int R);
// stage 0: gathers, u and ga, per-entry gradients, gx of the routed rows
// (after the routed rows' complete lists exist); stage 1: the weight
// gradients and gb, added to what the column walk wrote (after it).
hipError_t launch_backward_routed_dense(const void* x, const void* gy, const void* wg_t,
                                        const void* wu_t, const void* wd, const int32_t* routed,
                                        const int32_t* n_routed, const uint16_t* ecount,
                                        const uint16_t* eidx, const void* eval, void* gx,
                                        float* gwg_t, float* gwu_t, float* gwd, float* gb,
                                        int T, int D, int N, int R, float l1g, void* ws,
                                        int stage, hipStream_t stream);
hipError_t launch_backward(const void* x, const void* wg_t, const float* b_g, const void* wu_t,
                           const void* wd, const float* xnorm, const float* wnorm,
                           const uint16_t* count, const uint16_t* idx, const void* val,
                           const int32_t* routed, const int32_t* n_routed, const void* gy,
                           void* gx, float* gwg_t, float* gwu_t, float* gwd, float* gb, int T,
                           int D, int N, int cap, float l1g, int R, GuardBand band, void* ws,
                           hipStream_t stream);

// Row norms of a [rows_a, K] and a [rows_b, K] matrix in one launch.
hipError_t launch_row_norms(int dtype, const void* a, int rows_a, float* out_a, const void* b,
                            int rows_b, float* out_b, int K, hipStream_t stream);

// h[m, :] = ReLU(x[row(m)] wg_t^T + b) * (x[row(m)] wu_t^T) for m < rows, where
// row(m) = rowmap[m] (rowmap != nullptr) and rows = *n_rows_dev (n_rows_dev !=
// nullptr) else rows = M.
hipError_t launch_dense_gateup(int dtype, const void* x, const void* wg_t, const float* b_g,
                               const void* wu_t, void* h, int M, const int* rowmap,
                               const int* n_rows_dev, int K, int N, hipStream_t stream);

// y[row(m), :] = h[m, :] wd for m < rows (same row rules as above).
hipError_t launch_down(int dtype, const void* h, const void* wd, void* y, int M,
                       const int* rowmap, const int* n_rows_dev, int K, int N,
                       hipStream_t stream);

// Dense FFN of the routed rows (hybrid fallback), row count on the device:
// h [T, d_ff] (first n_routed rows used) and partial (routed_partial_bytes)
// are workspace; y rows routed[m] are written.  bf16, d_model and d_ff
// multiples of 32.  The gate+up kernel finds the routed rows and writes
// routed and n_routed for the kernels after it: with route_count
// (T <= kRouteBlock) from the TwELL counts, else from route_mask (the
// route_flags mask, launch_route_mask).
size_t routed_partial_bytes(int T, int d_model, int d_ff);
hipError_t launch_routed_ffn(const void* x, const void* wg_t, const float* b_g, const void* wu_t,
                             const void* wd, void* h, void* y, float* partial, int T,
                             int32_t* routed, int32_t* n_routed, const uint16_t* route_count,
                             const uint16_t* route_mask, int route_nt, int route_cap,
                             int d_model, int d_ff, hipStream_t stream);

// Dense gated FFN for few tokens (split-K weight streams): bf16, M <= 32,
// d_model and d_ff multiples of 128.  h [M, d_ff] and partial
// (dense_skinny_partial_bytes) are workspace.
bool dense_skinny_ok(int dtype, int M, int d_model, int d_ff);
size_t dense_skinny_partial_bytes(int d_model, int d_ff);
hipError_t launch_dense_skinny(const void* x, const void* wg_t, const float* b_g, const void* wu_t,
                               const void* wd, void* h, float* partial, void* y, int M,
                               int d_model, int d_ff, hipStream_t stream);

// Number of column splits of the fused sparse kernel for this shape.
int sparse_splits(int T, int n_tiles, int d_model);
size_t sparse_workspace_bytes(int dtype, int T, int n_tiles, int d_model, int cap);

hipError_t launch_sparse_updown(int dtype, const void* x, const void* wu_t, const void* wd,
                                const uint16_t* count, const uint16_t* idx, const void* val,
                                void* y, void* ws, int T, int K, int n_tiles, int cap,
                                hipStream_t stream);

// The column-union variant of the fused kernel (union.hip): bf16, d_model in
// {512, 1024, 2048, 4096}, cap <= 32.
bool union_supported(int dtype, int d_model, int cap);
hipError_t launch_sparse_union(const void* x, const void* wu_t, const void* wd,
                               const uint16_t* count, const uint16_t* idx, const void* val,
                               void* y, int T, int K, int n_tiles, int cap, hipStream_t stream);

// Routing scan: the routed-row mask (one 16-bit word per 16 rows, at the
// start of ws), then the ascending compaction into routed and n_routed.
size_t route_workspace_bytes(int T);
int route_mask_words(int T);
hipError_t launch_route(const uint16_t* count, int T, int n_tiles, int cap, int32_t* routed,
                        int32_t* n_routed, void* ws, hipStream_t stream);
// The mask alone (route_mask_words(T) words), for launch_routed_ffn.
hipError_t launch_route_mask(const uint16_t* count, int T, int n_tiles, int cap, uint16_t* mask,
                             hipStream_t stream);

}  // namespace sffn
