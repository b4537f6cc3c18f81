// Separate-conversion baseline (not on the fused forward path): the gate
// GEMM storing the float32 pre-activation, and standalone conversions of it to
// TwELL and to a classic row-wise ELLPACK.  Declared in launch.h; the C entry
// points are gate_preact, twell_from_preact and ell_from_preact.
#include <climits>

#include "common.cuh"
#include "exact.cuh"
#include "gemm_v2.cuh"
#include "launch.h"
#include "twell_emit.cuh"

namespace sffn {

namespace {

// ---------------------------------------------------------------------------
// Separate-conversion baseline: the design the pwwt.cn article (sections 01
// and 02) argues against, kept to measure that claim.  The gate GEMM stores
// the whole float32 pre-activation z, then standalone kernels read it back
// and build TwELL, or a classic row-wise ELLPACK (one list per row over all
// columns, padded to a common width: the "traditional ELLPACK" of the same
// section 01 and of the kongchang.com article).  The GEMM is the TwELL
// kernel's own main loop (GateGemm), so z holds exactly the float32 values the
// fused epilogue sees and the converters reach the same exact activity
// decision with the same guard band; it also runs the same mix of 256 x 256
// and 256 x 128 tiles, so the two designs differ only after the main loop.

// One tile of z[m, j] = acc + b_g[j] (float32, row-major [rows, N]) for the
// x rows rowmap[m] (rowmap null: row m), m < mv.  G: GateGemmWide or GateGemm
// (the TwELL kernel's own tiles, for the baseline) or RowsGemm (64-row tiles,
// for a few mapped rows).  All chain 16x16x32 MFMAs over K, K / 32 roundings:
// the same guard band holds.
using RowsGemm = Gemm2<1, kTile, false, 64, 4, false, 64, 4, 4>;

template <class G>
__device__ __forceinline__ void preact_tile(const GateArgs& a, uint8_t* lds, float* z,
                                            const int* rowmap, int mv, int m0, int n0) {
  G g;
  const uint16_t* B[1] = {(const uint16_t*)a.wg};
  g.init((const uint16_t*)a.x, (size_t)a.T, rowmap, m0, mv, B, n0, a.N, a.K);
  g.run_pipe(lds, a.K);
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  const int wm = w % G::WAVES_M, wn = w / G::WAVES_M;
#pragma unroll
  for (int fn = 0; fn < G::FN; ++fn) {
    const int col = n0 + wn * G::WN + fn * 16 + (lane & 15);
    const bool cv = col < a.N;
    const float bb = (a.b && cv) ? a.b[col] : 0.f;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * G::WM + fm * 16 + 4 * (lane >> 4) + r;
        if (cv && m < mv) z[(size_t)m * a.N + col] = g.acc[0][fm][fn][r] + bb;
      }
  }
}

// Mapped rows (the routed rows of the backward), 64-row tiles.  wide_from:
// the row count from which gate_preact_rows_wide takes the rows instead (this
// kernel then returns), or INT_MAX when that kernel is not launched.
__global__ __launch_bounds__(64 * RowsGemm::NWAVES) void gate_preact_rows(
    GateArgs a, float* z, const int* rowmap, const int* n_rows_dev, int max_rows,
    int wide_from) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[RowsGemm::LDS_BYTES];
  // the active tiles are the first ones, spread over the XCDs in dispatch
  // order (the XCD-aware map would put them all on one)
  const int ntn = a.N / RowsGemm::BN;
  const int mi = (int)blockIdx.x / ntn, ni = (int)blockIdx.x - mi * ntn;
  const int m0 = mi * RowsGemm::BM;
  const int mv = uniform(min(*n_rows_dev, max_rows));
  if (m0 >= mv || mv >= wide_from) return;
  preact_tile<RowsGemm>(a, lds, z, rowmap, mv, m0, ni * RowsGemm::BN);
}

// Many mapped rows (kRowsWideFrom or more): the TwELL kernel's 256 x 256 tiles
// (256 x 128 for an odd last column tile), numbered by the actual row count
// through the XCD-aware map so that the working tiles come first and spread
// over the XCDs.  The 64-row tiles run these at about 0.46 PFLOP/s.
constexpr int kRowsWideFrom = 1024;

__global__ __launch_bounds__(64 * GateGemm::NWAVES) void gate_preact_rows_wide(
    GateArgs a, float* z, const int* rowmap, const int* n_rows_dev, int max_rows) {
  constexpr size_t kLds = GateGemm::LDS_BYTES > GateGemmWide::LDS_BYTES ? GateGemm::LDS_BYTES
                                                                         : GateGemmWide::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  const int mv = uniform(min(*n_rows_dev, max_rows));
  if (mv < kRowsWideFrom) return;
  const int mt = (mv + GateGemm::BM - 1) / GateGemm::BM;
  const int nt = a.N / kTile, wide_nt = nt / 2, narrow_nt = nt - 2 * wide_nt;
  const int bid = (int)blockIdx.x, n_wide = mt * wide_nt;
  int mi, ni;
  if (bid < n_wide) {
    tile_of(bid, mt, wide_nt, &mi, &ni);
    preact_tile<GateGemmWide>(a, lds, z, rowmap, mv, mi * GateGemmWide::BM,
                              ni * GateGemmWide::BN);
  } else if (bid - n_wide < mt * narrow_nt) {
    tile_of(bid - n_wide, mt, narrow_nt, &mi, &ni);
    preact_tile<GateGemm>(a, lds, z, rowmap, mv, mi * GateGemm::BM,
                          wide_nt * GateGemmWide::BN + ni * GateGemm::BN);
  }
}

// All rows: the TwELL kernel's grid (wide tiles, then narrow ones).
__global__ __launch_bounds__(64 * GateGemm::NWAVES) void gate_preact_bf16(GateArgs a, float* z,
                                                                         int wide_nt,
                                                                         int narrow_nt) {
  constexpr size_t kLds = GateGemm::LDS_BYTES > GateGemmWide::LDS_BYTES ? GateGemm::LDS_BYTES
                                                                         : GateGemmWide::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  const int mt = (a.T + GateGemm::BM - 1) / GateGemm::BM;
  const int n_wide = mt * wide_nt;
  const int bid = (int)blockIdx.x;
  int mi, ni;
  if (bid < n_wide) {
    tile_of(bid, mt, wide_nt, &mi, &ni);
    preact_tile<GateGemmWide>(a, lds, z, nullptr, a.T, mi * GateGemmWide::BM,
                              ni * GateGemmWide::BN);
  } else {
    tile_of(bid - n_wide, mt, narrow_nt, &mi, &ni);
    preact_tile<GateGemm>(a, lds, z, nullptr, a.T, mi * GateGemm::BM,
                          wide_nt * GateGemmWide::BN + ni * GateGemm::BN);
  }
}

// TwELL from z: one wavefront per (16 rows, column tile), all 32 row loads
// of its z block in flight at once (the conversion streams z from HBM; no LDS
// staging, no workgroup barrier).  Rows with an entry inside the guard band
// are deferred and emitted after the exact re-evaluation, re-reading their z
// row (rare, and still in cache).
constexpr int kConvRows = 16;

__global__ __launch_bounds__(256) void twell_convert_bf16(GateArgs a, const float* z) {
  __shared__ uint32_t exact_lds[4 * kExactLdsWords];
  const int w = uniform((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int nt = a.N / kTile;
  const int item = (int)blockIdx.x * 4 + w;
  const int kt = item % nt;
  const int r0 = (item / nt) * kConvRows;
  if (r0 >= a.T) return;
  const int n0 = kt * kTile;
  const int rows = min(kConvRows, a.T - r0);
  float zv[kConvRows][2];
#pragma unroll
  for (int r = 0; r < kConvRows; ++r) {
    const float* zr = z + (size_t)(r0 + min(r, rows - 1)) * a.N + n0;
    zv[r][0] = zr[lane];
    zv[r][1] = zr[64 + lane];
  }
  const float nxl = lane < rows ? a.xnorm[r0 + lane] : 0.f;
  RowCtx c;
  c.nt = nt;
  c.kt = kt;
  c.m0 = 0;
  c.n0 = n0;
  c.r0 = 0;
  c.b0 = a.b ? a.b[n0 + lane] : 0.f;
  c.b1 = a.b ? a.b[n0 + 64 + lane] : 0.f;
  c.nw0 = a.wnorm[n0 + lane];
  c.nw1 = a.wnorm[n0 + 64 + lane];
  c.band_scale = 1.0f;
  const float e0 = a.gb.coef_b * fabsf(c.b0), e1 = a.gb.coef_b * fabsf(c.b1);
  uint32_t deferred = 0;
#pragma unroll
  for (int r = 0; r < kConvRows; ++r) {
    if (r < rows) {
      const float nx = __shfl(nxl, r, kWave);
      const uint64_t f = __ballot(!(fabsf(zv[r][0]) > a.gb.coef_xw * nx * c.nw0 + e0)) |
                         __ballot(!(fabsf(zv[r][1]) > a.gb.coef_xw * nx * c.nw1 + e1));
      if (f) deferred |= 1u << r;
      else emit_row<uint16_t>(a, c, r0 + r, zv[r][0] > 0.f, zv[r][1] > 0.f, zv[r][0], zv[r][1]);
    }
  }
  const uint16_t* wg = (const uint16_t*)a.wg;
  while (deferred) {
    const int r = __builtin_ctz(deferred);
    deferred &= deferred - 1;
    const int t = r0 + r;
    const float* zr = z + (size_t)t * a.N + n0;
    float z0 = zr[lane], z1 = zr[64 + lane];
    const float nx = __shfl(nxl, r, kWave);
    uint64_t f0 = __ballot(!(fabsf(z0) > a.gb.coef_xw * nx * c.nw0 + e0));
    uint64_t f1 = __ballot(!(fabsf(z1) > a.gb.coef_xw * nx * c.nw1 + e1));
    bool act0 = z0 > 0.f, act1 = z1 > 0.f;
    while (f0 | f1) {
      int col;
      if (f0) { col = __builtin_ctzll(f0); f0 &= f0 - 1; }
      else    { col = 64 + __builtin_ctzll(f1); f1 &= f1 - 1; }
      const float bc = a.b ? a.b[n0 + col] : 0.f;
      const ExactResult e = exact_gate_value<uint16_t, 2>(
          (const uint16_t*)a.x + (size_t)t * a.K, wg + (size_t)(n0 + col) * a.K, bc, a.K,
          exact_lds + w * kExactLdsWords);
      if (col < 64) {
        if (lane == col) { act0 = e.sign > 0; z0 = (float)e.value; }
      } else {
        if (lane == col - 64) { act1 = e.sign > 0; z1 = (float)e.value; }
      }
    }
    emit_row<uint16_t>(a, c, t, act0, act1, z0, z1);
  }
}

// Classic row-wise ELLPACK from z: one wavefront per row walks the column
// tiles in order with a running slot count across tiles, U tiles of loads in
// flight per round, emitted straight from registers; a tile with an entry
// inside the guard band first gets its exact re-evaluation.  ecount[t] = active columns of the row
// (uncapped); slots s < min(ecount, width) hold the ascending columns and
// their values.
__device__ __forceinline__ void ell_emit(uint16_t* eidx, uint16_t* eval, size_t ebase, int width,
                                         int col0, bool act0, bool act1, float z0, float z1,
                                         int& running) {
  const int lane = lane_id();
  const uint64_t m0 = __ballot(act0), m1 = __ballot(act1);
  const int s0 = running + lanes_below(m0);
  if (act0 && s0 < width) {
    eidx[ebase + s0] = (uint16_t)(col0 + lane);
    eval[ebase + s0] = f32_to_bf16(z0);
  }
  const int s1 = running + __popcll(m0) + lanes_below(m1);
  if (act1 && s1 < width) {
    eidx[ebase + s1] = (uint16_t)(col0 + 64 + lane);
    eval[ebase + s1] = f32_to_bf16(z1);
  }
  running += __popcll(m0) + __popcll(m1);
}

// Row m of z and of the output is x row rowmap[m] (rowmap null: m), for
// m < rows (n_rows_dev null: T; else the count on the device).
// The exact re-evaluation of one tile's flagged entries (|z| not above the
// band d), out of line so the unrolled round keeps one copy of it.
struct TileFix {
  float z0, z1;
  int a0, a1;
};

__device__ __noinline__ TileFix ell_fix_tile(const uint16_t* xrow, const uint16_t* wg,
                                             const float* b, int K, int c0, float z0, float z1,
                                             float d0, float d1, uint32_t* exact_lds) {
  const int lane = lane_id();
  TileFix f{z0, z1, z0 > 0.f, z1 > 0.f};
  uint64_t fl[2] = {__ballot(!(fabsf(z0) > d0)), __ballot(!(fabsf(z1) > d1))};
  while (fl[0] | fl[1]) {
    const int h = fl[0] ? 0 : 1;
    const int L = __builtin_ctzll(fl[h]);
    fl[h] &= fl[h] - 1;
    const int col = c0 + 64 * h + L;
    const ExactResult e = exact_gate_value<uint16_t, 2>(xrow, wg + (size_t)col * K,
                                                        b ? b[col] : 0.f, K, exact_lds);
    if (lane == L) {
      if (h == 0) { f.a0 = e.sign > 0; f.z0 = (float)e.value; }
      else        { f.a1 = e.sign > 0; f.z1 = (float)e.value; }
    }
  }
  return f;
}

template <int U>
__global__ __launch_bounds__(256) void ell_convert_bf16(GateArgs a, const float* z, int width,
                                                        uint16_t* ecount, uint16_t* eidx,
                                                        uint16_t* eval, const int* rowmap,
                                                        const int* n_rows_dev, int max_rows) {
  __shared__ uint32_t exact_lds[4 * kExactLdsWords];
  const int w = uniform((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int m = (int)blockIdx.x * 4 + w;
  const int mv = uniform(n_rows_dev ? min(*n_rows_dev, max_rows) : max_rows);
  if (m >= mv) return;
  const int t = uniform(rowmap ? rowmap[m] : m);
  const int nt = a.N / kTile;
  const float nx = a.xnorm[t];
  const float* zr = z + (size_t)m * a.N;
  const size_t ebase = (size_t)m * width;
  int running = 0;
  for (int k0 = 0; k0 < nt; k0 += U) {
    float zv[U][2], dv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = min(k0 + u, nt - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = kk * kTile + 64 * h + lane;
        zv[u][h] = zr[col];
        dv[u][h] = a.gb.coef_xw * nx * a.wnorm[col] + (a.b ? a.gb.coef_b * fabsf(a.b[col]) : 0.f);
      }
    }
    uint32_t fm = 0;  // tiles of the round with an entry inside the guard band
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + u < nt &&
          __ballot(!(fabsf(zv[u][0]) > dv[u][0]) || !(fabsf(zv[u][1]) > dv[u][1])))
        fm |= 1u << u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u >= nt) break;
      float z0 = zv[u][0], z1 = zv[u][1];
      bool a0 = z0 > 0.f, a1 = z1 > 0.f;
      if ((fm >> u) & 1u) {  // rare: exact re-evaluation of the tile's flagged entries
        const TileFix f = ell_fix_tile((const uint16_t*)a.x + (size_t)t * a.K,
                                       (const uint16_t*)a.wg, a.b, a.K, (k0 + u) * kTile, z0, z1,
                                       dv[u][0], dv[u][1], exact_lds + w * kExactLdsWords);
        z0 = f.z0;
        z1 = f.z1;
        a0 = f.a0 != 0;
        a1 = f.a1 != 0;
      }
      ell_emit(eidx, eval, ebase, width, (k0 + u) * kTile, a0, a1, z0, z1, running);
    }
  }
  if (lane == 0) ecount[m] = (uint16_t)running;
}

}  // namespace

hipError_t launch_gate_preact(const void* x, const void* wg_t, const float* b_g, float* z, int T,
                              int K, int N, const int* rowmap, const int* n_rows_dev,
                              hipStream_t stream, int max_rows) {
  GateArgs a{x, wg_t, b_g, nullptr, nullptr, nullptr, nullptr, nullptr, T, K, N, 0, GuardBand{}};
  if (rowmap) {
    if (!n_rows_dev) return hipErrorInvalidValue;
    const int rows = max_rows >= 0 ? min(max_rows, T) : T;
    if (rows == 0) return hipSuccess;
    // the 256-row kernel only where it can matter (below 8192 tokens its
    // extra launch would cost more than the few routed rows' tiles gain)
    const bool wide = rows >= kRowsWideFrom && T >= 8192 && N % kTile == 0;
    // with the 256-row kernel launched, the 64-row one takes fewer than
    // kRowsWideFrom rows: no larger grid (its workgroups that return at once
    // still cost their dispatch)
    const int narrow_rows = wide ? kRowsWideFrom : rows;
    const dim3 g((unsigned)(((narrow_rows + RowsGemm::BM - 1) / RowsGemm::BM) * (N / RowsGemm::BN)));
    hipLaunchKernelGGL(gate_preact_rows, g, dim3(64 * RowsGemm::NWAVES), 0, stream, a, z, rowmap,
                       n_rows_dev, rows, wide ? kRowsWideFrom : INT_MAX);
    if (wide) {
      const int nt = N / kTile;
      const dim3 gw((unsigned)(((rows + GateGemm::BM - 1) / GateGemm::BM) * (nt / 2 + nt % 2)));
      hipLaunchKernelGGL(gate_preact_rows_wide, gw, dim3(64 * GateGemm::NWAVES), 0, stream, a, z,
                         rowmap, n_rows_dev, rows);
    }
  } else {
    int wide_nt, narrow_nt;
    gate_tile_split(T, N, &wide_nt, &narrow_nt);
    const dim3 g((unsigned)(((T + GateGemm::BM - 1) / GateGemm::BM) * (wide_nt + narrow_nt)));
    hipLaunchKernelGGL(gate_preact_bf16, g, dim3(64 * GateGemm::NWAVES), 0, stream, a, z, wide_nt,
                       narrow_nt);
  }
  return hipGetLastError();
}

bool preact_supported(int dtype, int K) { return dtype == 1 && K % GateGemm::BK == 0; }

hipError_t launch_twell_convert(const float* z, const void* x, const void* wg_t, const float* b_g,
                                const float* xnorm, const float* wnorm, uint16_t* count,
                                uint16_t* idx, void* val, int T, int K, int N, int cap,
                                GuardBand gb, hipStream_t stream) {
  GateArgs a{x, wg_t, b_g, count, idx, val, xnorm, wnorm, T, K, N, cap, gb};
  const long items = (long)((T + kConvRows - 1) / kConvRows) * (N / kTile);
  hipLaunchKernelGGL(twell_convert_bf16, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream,
                     a, z);
  return hipGetLastError();
}

hipError_t launch_ell_convert(const float* z, const void* x, const void* wg_t, const float* b_g,
                              const float* xnorm, const float* wnorm, int width,
                              uint16_t* ecount, uint16_t* eidx, void* eval, int T, int K, int N,
                              GuardBand gb, const int* rowmap, const int* n_rows_dev,
                              hipStream_t stream, int max_rows) {
  GateArgs a{x, wg_t, b_g, nullptr, nullptr, nullptr, xnorm, wnorm, T, K, N, 0, gb};
  const int rows = max_rows >= 0 ? min(max_rows, T) : T;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(ell_convert_bf16<16>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     a, z, width, ecount, eidx, (uint16_t*)eval, rowmap, n_rows_dev, rows);
  return hipGetLastError();
}


}  // namespace sffn
