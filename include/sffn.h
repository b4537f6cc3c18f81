/*
 * sffn.h -- C ABI of the activation-sparse gated FFN forward on AMD MI355X (gfx950).
 *
 * The method ("Sparser, Faster, Lighter Transformer Language Models", as
 * described by the pwwt.cn article, sections 01-03, the kongchang.com article,
 * sections "TwELL" and "custom CUDA kernels", and the neo-ai.one article):
 *
 *   gated FFN   y = (ReLU(x W_g + b_g) * (x W_u)) W_d           (pwwt.cn 01)
 *   TwELL       the gate projection's epilogue writes the ReLU survivors of
 *               each row, tile by tile over 1D column tiles, as small ELLPACK
 *               lists (column index + value), with no separate conversion
 *               kernel                                            (pwwt.cn 02)
 *   fused       one kernel computes the up projection only on the packed
 *               nonzeros, scales by the gate value and accumulates the down
 *               projection, never storing h                       (pwwt.cn 02)
 *   hybrid      rows whose nonzeros do not fit the compact format are routed
 *               to a dense fallback on the matrix cores           (pwwt.cn 03)
 *
 * Conventions shared by every call:
 *   - All buffer pointers are DEVICE pointers, 16-byte aligned.  Shapes and
 *     scalars are passed by value or through the host struct sffn_shape.
 *   - Every call is asynchronous on the given HIP stream (hipStream_t passed
 *     as void*; NULL means the default stream).  The library never allocates,
 *     frees or synchronises.  The caller owns all memory, workspace included,
 *     except the static scratch array of twell_pack_noalloc (see there).
 *   - Layouts (row-major):
 *       x, y                  [T, d_model]
 *       wg_t, wu_t, wd        [d_ff, d_model]; row j holds the d_model weights
 *                             of FFN neuron j (gate column j, up column j,
 *                             down row j)
 *       b_g                   [d_ff] float32 gate bias, may be NULL (zero)
 *       count                 uint16 [T, n_tiles], n_tiles = d_ff / tile
 *       idx                   uint16 [T, n_tiles, cap]: global column index j
 *       val                   dtype  [T, n_tiles, cap]
 *   - dtype (sffn_shape.dtype) applies to x, the weights, val, y and the
 *     internal h of the dense paths: SFFN_F32 or SFFN_BF16.  Accumulation is
 *     always float32; outputs are rounded to dtype with round-to-nearest-even.
 *   - Preconditions (else SFFN_ERR_ARG or SFFN_ERR_UNSUPPORTED, detected on the
 *     host before anything is launched, nothing written):
 *       tile == 128; d_ff % 128 == 0; 128 <= d_ff <= 65535;
 *       0 <= cap <= 128; d_model % 8 == 0; 8 <= d_model <= 8192;
 *       0 <= T; T == 0 is a no-op returning SFFN_OK;
 *       T * d_model * sizeof(dtype) < 2^31 and d_ff * d_model * sizeof(dtype)
 *       < 2^31 (twell_pack, hybrid_route, dense_ffn_ref).
 *     Inputs must be finite (no Inf/NaN).
 *   - Errors: every call returns an sffn_status.  A failed launch returns
 *     SFFN_ERR_HIP; device faults surface at the caller's next synchronisation.
 */
#ifndef SFFN_H
#define SFFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SFFN_OK = 0,
  SFFN_ERR_ARG = -1,         /* null/misaligned pointer, negative or inconsistent size */
  SFFN_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement */
  SFFN_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than sffn_workspace_bytes */
  SFFN_ERR_HIP = -4,         /* a HIP launch or runtime call failed */
  SFFN_ERR_TOO_LARGE = -5    /* twell_pack_noalloc: shape needs more than its scratch */
} sffn_status;

typedef enum { SFFN_F32 = 0, SFFN_BF16 = 1 } sffn_dtype;

/* Which call a workspace query is for. */
typedef enum {
  SFFN_WS_HYBRID = 0,
  SFFN_WS_DENSE = 1,
  SFFN_WS_SPARSE = 2,
  SFFN_WS_PACK = 3,
  SFFN_WS_CONVERT = 4,
  SFFN_WS_PACK_L1 = 5,
  SFFN_WS_BACKWARD = 6
} sffn_ws_kind;

typedef struct {
  int32_t T;       /* tokens (rows of x and y) */
  int32_t d_model; /* model width */
  int32_t d_ff;    /* FFN width (number of gate/up/down neurons) */
  int32_t tile;    /* TwELL column-tile width; must be 128 */
  int32_t cap;     /* TwELL capacity: slots per (row, tile) */
  int32_t dtype;   /* sffn_dtype */
} sffn_shape;

/*
 * twell_weight_norms -- Euclidean norm of every row of wg_t (float32 [d_ff]),
 * an input of twell_pack's exact-sign guard band.  The gate weights do not
 * change between calls, so a caller can compute these once per weight matrix
 * and pass them to every twell_pack call.  No workspace.
 */
int32_t twell_weight_norms(const sffn_shape* shape, const void* wg_t, float* wg_norms,
                           void* stream);

/*
 * twell_pack -- gate projection with the TwELL epilogue (pwwt.cn article,
 * section 02: the format is produced directly in the gate GEMM's epilogue).
 *
 *   z[t, j] = sum_k x[t, k] * wg_t[j, k] + b_g[j]        (float32 accumulation)
 *   active  = z > 0 (strict), decided on the EXACT value of z: entries whose
 *             float32 result lies within a rigorous bound of the accumulation
 *             error around zero (proportional to ||x_t|| ||wg_t[j]||) are
 *             re-evaluated exactly in the epilogue.
 *   For each row t and tile k (columns 128k .. 128k+127):
 *     count[t, k]   = number of active columns in the tile (uncapped, <= 128)
 *     idx[t, k, s]  = s-th active column, ascending, global index j, for
 *                     s < min(count, cap)
 *     val[t, k, s]  = z at that column, rounded to dtype
 *   Slots s >= min(count, cap) are left unwritten (unspecified).
 *
 * x: [T, d_model] dtype; wg_t: [d_ff, d_model] dtype; b_g: [d_ff] f32 or NULL;
 * wg_norms: the output of twell_weight_norms for this wg_t, or NULL (then they
 * are computed inside the call); count/idx/val: outputs as laid out above.
 * workspace: at least sffn_workspace_bytes(shape, SFFN_WS_PACK) bytes (row
 * norms of x, and of wg_t when wg_norms is NULL; for few tokens, also the
 * partial tiles of the split-K gate kernels).  No initial contents needed.
 * Calls that share a workspace must be stream-ordered.
 */
int32_t twell_pack(const sffn_shape* shape, const void* x, const void* wg_t,
                   const float* b_g, const float* wg_norms, uint16_t* count, uint16_t* idx,
                   void* val, void* workspace, size_t ws_bytes, void* stream);

/*
 * twell_pack_noalloc -- twell_pack without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same computation,
 * kernels and outputs as twell_pack (bit for bit); the workspace is a static
 * device array of twell_pack_noalloc_max_bytes() bytes (32 MiB) inside the
 * library, one per GPU, held until the process ends.  Nothing is allocated
 * or freed by the call (the first call on a device looks the array's address
 * up; later calls reuse it).  Shapes whose twell_pack workspace
 * (sffn_workspace_bytes(shape, SFFN_WS_PACK)) exceeds that size return
 * SFFN_ERR_TOO_LARGE before anything is launched.  All calls on one GPU share
 * the array: calls that overlap in time on one GPU (on different streams or
 * host threads) race and must not be issued; calls ordered on one stream are
 * safe.  The scratch needs no initial contents.  Arguments and errors
 * otherwise as twell_pack; the device is the one that runs `stream`.
 */
int32_t twell_pack_noalloc(const sffn_shape* shape, const void* x, const void* wg_t,
                           const float* b_g, const float* wg_norms, uint16_t* count,
                           uint16_t* idx, void* val, void* stream);

/* Size in bytes of twell_pack_noalloc's static scratch array. */
size_t twell_pack_noalloc_max_bytes(void);

/*
 * twell_pack_l1 -- twell_pack plus the L1 activation regulariser that drives
 * the sparsity in training (pwwt.cn article, section 04: a light L1 penalty on
 * the FFN activations; the besthub.dev page), summed in the same gate
 * epilogue from the same z as the TwELL lists:
 *
 *   *l1_value = lambda / T * sum_t sum_j ReLU(z[t, j])      (float32, device)
 *
 * Every active entry counts, also those past the capacity.  The gate kernels
 * sum in float32 in a fixed order (the 256-row kernel over its whole tile of
 * up to 256 x 128 entries, at most about 30 additions deep; the others per
 * row and tile), and those partial sums are added in float64 in a fixed
 * order, so the value is deterministic.  The
 * gradient of the term with respect to z is lambda / T on exactly the active
 * entries (the uncapped TwELL support) and 0 elsewhere; sparse_ffn_bwd adds it
 * when given the same lambda.  T == 0 writes 0.  Outputs and arguments otherwise as
 * twell_pack; lambda must not be NaN (else SFFN_ERR_ARG); workspace: at least
 * sffn_workspace_bytes(shape, SFFN_WS_PACK_L1) bytes, no initial contents.
 */
int32_t twell_pack_l1(const sffn_shape* shape, const void* x, const void* wg_t,
                      const float* b_g, const float* wg_norms, uint16_t* count, uint16_t* idx,
                      void* val, float lambda, float* l1_value, void* workspace, size_t ws_bytes,
                      void* stream);

/*
 * sparse_ffn_fwd -- fused up(.)gate -> down over the TwELL nonzeros (pwwt.cn
 * article, section 02).  For every row t with count[t, k] <= cap for all k:
 *
 *   y[t, :] = sum over k, s < count[t, k] of
 *               val[t,k,s] * (x[t, :] . wu_t[idx[t,k,s], :]) * wd[idx[t,k,s], :]
 *
 * accumulated in float32 and written once, rounded to dtype.  Rows with any
 * count above cap are not touched (hybrid_route writes them).
 * workspace: at least sffn_workspace_bytes(shape, SFFN_WS_SPARSE) bytes of
 * device memory, no initial contents needed (every call initialises what it
 * uses, so nothing is carried from one call to the next, also after a call
 * that failed).  May be NULL when that size is 0.  Calls that share a
 * workspace must be stream-ordered.
 */
int32_t sparse_ffn_fwd(const sffn_shape* shape, const void* x, const void* wu_t,
                       const void* wd, const uint16_t* count, const uint16_t* idx,
                       const void* val, void* y, void* workspace, size_t ws_bytes,
                       void* stream);

/*
 * sparse_ffn_fwd_union -- the same sum as sparse_ffn_fwd, computed with the
 * organisation of the pages' fused kernel (pwwt.cn article, section 02): per
 * block of consecutive tokens, the active columns the block shares within a
 * column tile are deduplicated, and the wu_t and wd rows of each distinct
 * column are read from global memory once per block into LDS, where every
 * token of the block that uses the column reads them.  A measured alternative
 * to sparse_ffn_fwd (which walks each token's entries against rows served by
 * the caches); y agrees with it to float32 rounding of the down projection,
 * not bit for bit.  Rows with any count above cap are not touched.
 * Supported: dtype SFFN_BF16, d_model in {512, 1024, 2048, 4096},
 * cap <= 32 (else SFFN_ERR_UNSUPPORTED, nothing written).  No workspace; no
 * state between calls.
 */
int32_t sparse_ffn_fwd_union(const sffn_shape* shape, const void* x, const void* wu_t,
                             const void* wd, const uint16_t* count, const uint16_t* idx,
                             const void* val, void* y, void* stream);

/*
 * hybrid_route -- route overflowing rows to a dense fallback (pwwt.cn article,
 * section 03: rare high-activity tokens go to a dense backup path on the
 * matrix cores).
 *
 *   routed[0 .. n_routed) = ascending rows t with count[t, k] > cap for some k
 *   *n_routed             = their number (written on the device; no host sync)
 *   for each routed row:  y[t, :] = (ReLU(x_t W_g + b_g) * (x_t W_u)) W_d,
 *                         gate recomputed from x, h rounded to dtype.
 * Rows that are not routed are not touched.  routed: int32 [T] (entries past
 * n_routed unspecified); n_routed: one int32.  workspace: at least
 * sffn_workspace_bytes(shape, SFFN_WS_HYBRID) bytes (side buffer for the
 * routed rows' h, the split-K partials of their down projection and the
 * routing scan).  No initial contents needed.  Calls that share a workspace
 * must be stream-ordered.
 */
int32_t hybrid_route(const sffn_shape* shape, const void* x, const void* wg_t,
                     const float* b_g, const void* wu_t, const void* wd,
                     const uint16_t* count, int32_t* routed, int32_t* n_routed,
                     void* workspace, size_t ws_bytes, void* y, void* stream);

/*
 * sparse_ffn_bwd -- backward of the sparse forward (training through TwELL
 * and the hybrid routing: pwwt.cn article, sections 03-04), optionally with
 * the L1 activation regulariser of the same training recipe (section 04:
 * the penalty lambda / T * sum_t sum_j ReLU(z[t, j]) whose value
 * twell_pack_l1 computes).  For the upstream gradient gy = dL/dy, the
 * regulariser weight l1_lambda (0 for none) and the forward's count/idx/val
 * (from twell_pack) and routed/n_routed (from hybrid_route), by the chain
 * rule on the gated FFN:
 *
 *   gx[t, :]    = sum_j gz[t,j] wg_t[j, :] + gu[t,j] wu_t[j, :]     (dtype)
 *   gwg_t[j, :] = sum_t gz[t,j] x[t, :]      gwu_t[j, :] = sum_t gu[t,j] x[t, :]
 *   gwd[j, :]   = sum_t a[t,j] gy[t, :]      gb[j] = sum_t gz[t,j]  (float32)
 *
 * over the active entries only (gz = ga u + l1_lambda / T, gu = ga h,
 * a = h u with ga = gy_t . wd[j], u = x_t . wu_t[j]; ReLU' is 0 elsewhere,
 * so the regulariser adds l1_lambda / T to gz on exactly the active entries,
 * those past the capacity included).  l1_lambda must not be NaN (else
 * SFFN_ERR_ARG).  Rows within
 * capacity use their TwELL entries (h = val); routed rows use complete
 * activity lists rebuilt from x with twell_pack's GEMM and exact activity
 * decision (h rounded to bf16 like val).  With at least 8192 tokens and 1024
 * routed rows (the count read on the device), the routed rows' products run as
 * dense bf16 matrix-core tiles instead, with their gz, gu and a rounded to
 * bf16 before the products (as a dense bf16 backward rounds them).  Every sum
 * runs in a fixed order: the result is deterministic.  Every element of the outputs is written
 * (weight-gradient rows of inactive columns are zero); gb may be NULL.
 *
 * bf16 with d_model <= 4096 or float32 with d_model <= 2048 (else
 * SFFN_ERR_UNSUPPORTED), plus twell_pack's size limits.  Float32 and bf16
 * widths that are not a multiple of 512 take the general path: the entries
 * of every row from complete activity lists that it rebuilds with
 * twell_pack's own kernels at the full capacity of 128 per tile (the same
 * exact activity decision; routed rows included, so routed, n_routed and
 * max_routed are not read, and the workspace does not depend on
 * max_routed).  gy, gx: [T, d_model]
 * dtype; gwg_t, gwu_t, gwd: float32 [d_ff, d_model]; gb: float32 [d_ff].
 * wg_norms as for twell_pack (or NULL); routed and n_routed of the same
 * forward.  max_routed (0 <= max_routed <= T, else SFFN_ERR_ARG) bounds the
 * routed rows the workspace holds: T always suffices; a caller that reads
 * n_routed after the forward can pass it and keep the workspace small.  If the
 * forward routed more rows than max_routed, those rows are not processed and
 * gb (when given) and the first row of gx are set to NaN.  workspace: at
 * least sparse_ffn_bwd_workspace_bytes(shape, max_routed) bytes (about
 * 20 max_routed d_ff + 32 max_routed d_model bytes for the routed rows plus
 * about 20 T n_tiles cap bytes for the TwELL entries; about 40 T d_ff bytes
 * on the general path), no initial contents; calls sharing it must be
 * stream-ordered.
 */
int32_t sparse_ffn_bwd(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                       const void* wu_t, const void* wd, const float* wg_norms,
                       const uint16_t* count, const uint16_t* idx, const void* val,
                       const int32_t* routed, const int32_t* n_routed, int32_t max_routed,
                       const void* gy, float l1_lambda, void* gx, float* gwg_t, float* gwu_t,
                       float* gwd, float* gb, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes of sparse_ffn_bwd for this shape and routed-row bound
 * (0 if the shape is invalid or max_routed is outside 0..T);
 * sffn_workspace_bytes(shape, SFFN_WS_BACKWARD) is this with max_routed = T. */
size_t sparse_ffn_bwd_workspace_bytes(const sffn_shape* shape, int32_t max_routed);

/*
 * dense_ffn_ref -- the dense gated FFN used as the speed-up reference
 * (pwwt.cn article, section 01 formula, computed densely on the matrix cores):
 *   h = ReLU(x wg_t^T + b_g) * (x wu_t^T)  rounded to dtype, in workspace;
 *   y = h wd, float32 accumulation, rounded to dtype.
 * workspace: at least sffn_workspace_bytes(shape, SFFN_WS_DENSE) bytes.
 */
int32_t dense_ffn_ref(const sffn_shape* shape, const void* x, const void* wg_t,
                      const float* b_g, const void* wu_t, const void* wd,
                      void* workspace, size_t ws_bytes, void* y, void* stream);

/*
 * Separate-conversion baseline.  The pwwt.cn article (sections 01 and 02)
 * argues that writing the whole gate activation and converting it to a sparse
 * format afterwards costs an extra launch, a global-memory write and read and
 * a synchronisation, and that the classic row-wise ELLPACK (one list per row,
 * padded to a common width; kongchang.com article, "ELLPACK" passage) fits
 * tiled GEMMs poorly.  These three calls build that design so both claims can
 * be measured against twell_pack.  They are not on the fused forward path.
 * bf16 only, d_model % 32 == 0 (else SFFN_ERR_UNSUPPORTED), plus the size
 * limits of twell_pack.
 *
 * gate_preact -- z[t, j] = sum_k x[t, k] * wg_t[j, k] + b_g[j], float32,
 * row-major [T, d_ff] (T * d_ff * 4 bytes, caller-owned).  The accumulation is
 * twell_pack's own for T > 64 (for fewer tokens twell_pack splits the sum
 * over K; the float32 values may then differ in the last bits, the activity
 * decision does not).  No workspace.
 */
int32_t gate_preact(const sffn_shape* shape, const void* x, const void* wg_t, const float* b_g,
                    float* z, void* stream);

/*
 * twell_from_preact -- TwELL from a z written by gate_preact for the same x,
 * wg_t and b_g: count/idx/val exactly as twell_pack defines them (activity on
 * the exact value of z, through the same guard band and exact re-evaluation).
 * wg_norms as for twell_pack (or NULL).  workspace: at least
 * sffn_workspace_bytes(shape, SFFN_WS_CONVERT) bytes (row norms), no initial
 * contents; calls sharing it must be stream-ordered.
 */
int32_t twell_from_preact(const sffn_shape* shape, const float* z, const void* x,
                          const void* wg_t, const float* b_g, const float* wg_norms,
                          uint16_t* count, uint16_t* idx, void* val, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * ell_from_preact -- classic row-wise ELLPACK of ReLU(z), z from gate_preact:
 *   ell_count[t]     = active columns of row t (uncapped; uint16 [T])
 *   ell_idx[t, s]    = s-th active column of the row, ascending, for
 *                      s < min(ell_count[t], width)  (uint16 [T, width])
 *   ell_val[t, s]    = z at that column, rounded to bf16 (bf16 [T, width])
 * Slots past min(ell_count[t], width) are left unwritten.  The classic format
 * pads every row to the longest one: width = max_t ell_count[t] keeps every
 * entry.  0 <= width <= d_ff (else SFFN_ERR_ARG); ell_idx and ell_val may be
 * NULL when width == 0.  shape->cap is not used.  Activity, wg_norms and
 * workspace as for twell_from_preact.
 */
int32_t ell_from_preact(const sffn_shape* shape, int32_t width, const float* z, const void* x,
                        const void* wg_t, const float* b_g, const float* wg_norms,
                        uint16_t* ell_count, uint16_t* ell_idx, void* ell_val, void* workspace,
                        size_t ws_bytes, void* stream);

/*
 * Peak probes: measured denominators for the roofline fractions (the
 * published MI355X peaks are 8 TB/s of HBM and 2.5 PFLOP/s of dense bf16
 * MFMA; these report what kernels of the hot path's kind reach on this GPU).
 *
 * sffn_probe_hbm -- one grid-stride pass over `bytes` bytes of src with
 * 16-byte loads, four in flight per lane, `workgroups` workgroups of 256
 * threads.  dst != NULL: copies src to dst (bytes read + bytes written);
 * dst == NULL: reads only.  Time it with events around the call; use buffers
 * much larger than the 256 MB Infinity Cache to measure HBM.  src and dst
 * device pointers, 16-byte aligned, not overlapping; bytes % 16 == 0;
 * workgroups > 0 (else SFFN_ERR_ARG).  bytes == 0 is a no-op.
 */
int32_t sffn_probe_hbm(const void* src, void* dst, size_t bytes, int32_t workgroups,
                       void* stream);

/*
 * sffn_probe_mfma -- `workgroups` workgroups of 256 threads; every wave issues
 * iters x 16 independent v_mfma_f32_16x16x32_bf16 (16384 flops each) on
 * operands of ones: 4 * 16 * 16384 * iters flops per workgroup (use at least
 * 8 workgroups per CU: several waves per SIMD).  out: float32
 * [workgroups * 256], each set to 2048 * iters (exact), a check that every
 * MFMA ran.  out != NULL, workgroups > 0, 0 < iters < 8192 (else
 * SFFN_ERR_ARG).
 */
int32_t sffn_probe_mfma(float* out, int32_t workgroups, int32_t iters, void* stream);

/*
 * sffn_probe_cached -- `workgroups` workgroups of 256 threads each read the
 * same window [src, src + window_bytes) `reps` times with 16-byte loads, eight
 * in flight per lane (workgroups * reps * window_bytes bytes in all).  With a
 * window that fits the L2 of an XCD (a few MiB) this is the rate at which the
 * vector-memory path brings cached data into the CUs: the ceiling of a kernel
 * that gathers rows it re-reads from the cache.  src 16-byte aligned,
 * window_bytes a positive multiple of 16, reps > 0, workgroups > 0 (else
 * SFFN_ERR_ARG).
 */
int32_t sffn_probe_cached(const void* src, size_t window_bytes, int32_t reps, int32_t workgroups,
                          void* stream);

/*
 * sffn_probe_gather -- for every i < nrows, one wave reads row rows[i] of
 * matrix a and of matrix b (rows of row_bytes bytes, row-major, 16-byte loads,
 * the whole row in flight): a row gather like the sparse kernel's, without
 * its arithmetic (2 * nrows * row_bytes bytes).  row_bytes one of 1024, 2048,
 * 4096, 8192, 16384; rows: int32 device array of valid row indices; a, b
 * 16-byte aligned; nrows >= 0 (else SFFN_ERR_ARG; 0 is a no-op).
 */
int32_t sffn_probe_gather(const void* a, const void* b, const int32_t* rows, int32_t nrows,
                          int32_t row_bytes, void* stream);

/*
 * sffn_probe_mfma_step -- one v_mfma_f32_16x16x32_bf16 per wave on operand
 * registers given by the caller, so that a test can compare the instruction
 * with the exact C + A.B.  The TwELL epilogue's guard band (twell_pack)
 * assumes that each such instruction's float32 result carries at most a few
 * unit roundoffs of error relative to |C| + sum |a_k b_k|; this probe lets
 * that assumption be checked on the hardware.  For wave w (0 <= w < waves)
 * and lane l (0..63): a[(64w + l) * 8 .. + 8] and b[...] are the lane's
 * eight bf16 A and B operand values (uint16 bit patterns), c[(64w + l) * 4
 * .. + 4] its four float32 accumulator inputs, and d[(64w + l) * 4 .. + 4]
 * receives the four accumulator outputs.  The lane layout is the
 * instruction's own (lane l holds row l % 16 of A, column l % 16 of B, and
 * k = 8 (l / 16) .. 8 (l / 16) + 7 of both; its outputs are column l % 16,
 * rows 4 (l / 16) .. 4 (l / 16) + 3).  Device pointers, 16-byte aligned,
 * sized for `waves` waves; waves > 0 (else SFFN_ERR_ARG).
 */
int32_t sffn_probe_mfma_step(const void* a, const void* b, const float* c, float* d,
                             int32_t waves, void* stream);

/*
 * sffn_probe_bf16_round -- out[i] = the float32 -> bfloat16 rounding that
 * every kernel of this library applies when it stores a bfloat16 result
 * (round to nearest, ties to even; NaN stays NaN), for i < n, so that a test
 * can compare it with a host rounding of the same inputs.  in: float32 [n],
 * out: uint16 bit patterns [n], device pointers; NULL pointers are
 * SFFN_ERR_ARG; n == 0 is a no-op.
 */
int32_t sffn_probe_bf16_round(const float* in, uint16_t* out, size_t n, void* stream);

/* Workspace bytes needed by one call for this shape (0 if the shape is invalid). */
size_t sffn_workspace_bytes(const sffn_shape* shape, int32_t which);

/* Static, NUL-terminated description of a status code. */
const char* sffn_strerror(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* SFFN_H */
