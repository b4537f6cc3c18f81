// Shared pieces of the TwELL builders: the gate kernels' arguments, the row
// walk that turns a staged z tile into TwELL lists (guard band, exact
// re-evaluation, ballot compaction), and the 256-row gate GEMM configuration.
// Included by the fused gate kernels (twell_gate.hip) and by the
// separate-conversion baseline (convert.hip), so both decide activity the
// same way and the baseline's GEMM accumulates exactly like the fused one.
#pragma once

#include "common.cuh"
#include "exact.cuh"
#include "gemm_v2.cuh"
#include "launch.h"

namespace sffn {

namespace {

constexpr int kTile = 128;
constexpr int kZld = kTile + 4;  // LDS row stride of the staged z half-tile (floats)

struct GateArgs {
  const void* x;
  const void* wg;
  const float* b;
  uint16_t* count;
  uint16_t* idx;
  void* val;
  const float* xnorm;  // ||x_t||, [T]
  const float* wnorm;  // ||wg_t[j]||, [N]
  int T, K, N, cap;
  GuardBand gb;
  float* l1_part;  // [T, n_tiles] sums of ReLU(z) over each (row, tile), or null
};

// Copy the row norms of a tile into LDS (rows past T read as 0).
__device__ __forceinline__ void load_tile_norms(const GateArgs& a, int m0, int bm, int n0,
                                                float* rn_a, float* rn_b) {
  for (int i = threadIdx.x; i < bm; i += blockDim.x) rn_a[i] = (m0 + i < a.T) ? a.xnorm[m0 + i] : 0.f;
  for (int i = threadIdx.x; i < kTile; i += blockDim.x) rn_b[i] = a.wnorm[n0 + i];
}

// Rows [r0, r0 + nrows) of the tile are staged in zs (row stride zld, float32
// or bfloat16 bits); the four waves take every fourth row.  Rows whose
// entries are all outside the guard band are emitted at once; rows with an
// entry inside it are listed in `defer` (LDS, 1 + nrows ints) and emitted in a
// second pass after their flagged entries were re-evaluated exactly, so the
// slow path runs on a few rows spread over all waves instead of stalling the
// row walk.
__device__ __forceinline__ float zget(const float* zs, int i) { return zs[i]; }
__device__ __forceinline__ float zget(const uint16_t* zs, int i) { return bf16_to_f32(zs[i]); }

struct RowCtx {
  int nt, kt, m0, n0, r0;
  float b0, b1, nw0, nw1, band_scale;
};

// Activity of the two entries of this lane in row rr, and the guard-band flags.
template <typename ZT>
__device__ __forceinline__ void row_state(const GateArgs& a, const RowCtx& c, const ZT* zs,
                                          int zld, const float* rn_a, int rr, float& z0, float& z1,
                                          uint64_t& f0, uint64_t& f1) {
  const int lane = lane_id();
  z0 = zget(zs, rr * zld + lane);
  z1 = zget(zs, rr * zld + 64 + lane);
  const float nx = rn_a[c.r0 + rr];
  const float d0 = c.band_scale * (a.gb.coef_xw * nx * c.nw0 + a.gb.coef_b * fabsf(c.b0));
  const float d1 = c.band_scale * (a.gb.coef_xw * nx * c.nw1 + a.gb.coef_b * fabsf(c.b1));
  f0 = __ballot(!(fabsf(z0) > d0));
  f1 = __ballot(!(fabsf(z1) > d1));
}

// Compaction of one row: ascending active columns into the first cap slots.
template <typename T>
__device__ __forceinline__ void emit_row(const GateArgs& a, const RowCtx& c, int t, bool act0,
                                         bool act1, float z0, float z1) {
  const int lane = lane_id();
  const uint64_t m0m = __ballot(act0);
  const uint64_t m1m = __ballot(act1);
  const int c0 = __popcll(m0m);
  const size_t base = ((size_t)t * c.nt + c.kt) * a.cap;
  if (act0) {
    const int s = lanes_below(m0m);
    if (s < a.cap) {
      a.idx[base + s] = (uint16_t)(c.n0 + lane);
      Elt<T>::store1(a.val, base + s, z0);
    }
  }
  if (act1) {
    const int s = c0 + lanes_below(m1m);
    if (s < a.cap) {
      a.idx[base + s] = (uint16_t)(c.n0 + 64 + lane);
      Elt<T>::store1(a.val, base + s, z1);
    }
  }
  if (lane == 0) a.count[(size_t)t * c.nt + c.kt] = (uint16_t)(c0 + __popcll(m1m));
  if (a.l1_part) {  // L1 regulariser: the row's ReLU sum over this tile, fixed order
    const float s = wave_sum((act0 ? z0 : 0.f) + (act1 ? z1 : 0.f));
    if (lane == 0) a.l1_part[(size_t)t * c.nt + c.kt] = s;
  }
}

// bias_lds (optional): the tile's 128 bias values already staged in LDS.
template <typename T, typename ZT, int EXACT_U = 2>
__device__ void twell_rows(const GateArgs& a, const ZT* zs, int zld, int nrows, float band_scale,
                           const float* rn_a, const float* rn_b, int r0, int m0, int n0,
                           int* defer, uint32_t* exact_lds, const float* bias_lds = nullptr) {
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  RowCtx c;
  c.nt = a.N / kTile;
  c.kt = n0 / kTile;
  c.m0 = m0;
  c.n0 = n0;
  c.r0 = r0;
  if (bias_lds) {
    c.b0 = bias_lds[lane];
    c.b1 = bias_lds[64 + lane];
  } else {
    c.b0 = a.b ? a.b[n0 + lane] : 0.f;
    c.b1 = a.b ? a.b[n0 + 64 + lane] : 0.f;
  }
  c.nw0 = rn_b[lane];
  c.nw1 = rn_b[64 + lane];
  c.band_scale = band_scale;
  if (threadIdx.x == 0) defer[0] = 0;
  __syncthreads();
  for (int rr = w; rr < nrows; rr += 4) {
    const int t = m0 + r0 + rr;
    if (t >= a.T) break;
    float z0, z1;
    uint64_t f0, f1;
    row_state(a, c, zs, zld, rn_a, rr, z0, z1, f0, f1);
    if (f0 | f1) {
      if (lane == 0) defer[1 + atomicAdd(&defer[0], 1)] = rr;
      continue;
    }
    emit_row<T>(a, c, t, z0 > 0.f, z1 > 0.f, z0, z1);
  }
  __syncthreads();
  const int nd = defer[0];
  const T* x = (const T*)a.x;
  const T* wg = (const T*)a.wg;
  for (int i = w; i < nd; i += 4) {
    const int rr = uniform(defer[1 + i]);
    const int t = m0 + r0 + rr;
    float z0, z1;
    uint64_t f0, f1;
    row_state(a, c, zs, zld, rn_a, rr, z0, z1, f0, f1);
    bool act0 = z0 > 0.f, act1 = z1 > 0.f;
    while (f0 | f1) {
      int col;
      if (f0) { col = __builtin_ctzll(f0); f0 &= f0 - 1; }
      else    { col = 64 + __builtin_ctzll(f1); f1 &= f1 - 1; }
      const float bc = a.b ? a.b[n0 + col] : 0.f;
      const ExactResult e = exact_gate_value<T, EXACT_U>(x + (size_t)t * a.K,
                                                wg + (size_t)(n0 + col) * a.K, bc, a.K,
                                                exact_lds + w * kExactLdsWords);
      if (col < 64) {
        if (lane == col) { act0 = e.sign > 0; z0 = (float)e.value; }
      } else {
        if (lane == col - 64) { act1 = e.sign > 0; z1 = (float)e.value; }
      }
    }
    emit_row<T>(a, c, t, act0, act1, z0, z1);
  }
}

// Configuration of the 256-row gate GEMM (gate_twell_bf16_v2 and gate_preact_bf16).
constexpr int kGateBK = 32;      // K depth of one pipeline stage
constexpr int kGateStages = 4;   // LDS ring depth
constexpr int kGateWaves = 8;    // waves per workgroup (two per SIMD)
using GateGemm = Gemm2<1, 128, false, kGateBK, 1, false, 256, kGateStages, kGateWaves, true>;
static_assert(GateGemm::WN == kTile, "each wave holds one TwELL column tile");
// 256 x 256 tiles of the same kernel: eight waves as 4 x 2, each 64 rows x one
// TwELL tile (a quarter fewer LDS fragment bytes per MFMA than 32 x 128).
using GateGemmWide = Gemm2<1, 256, false, kGateBK, 2, false, 256, kGateStages, kGateWaves, true>;
static_assert(GateGemmWide::WN == kTile, "each wave holds one TwELL column tile");

// Columns of 256-wide tiles (wide_nt, counted in 256-column tiles) and of
// 128-wide tiles after them (narrow_nt) for the 256-row gate kernels, one
// workgroup per CU.  Wide tiles everywhere, unless the last round of them
// would hold at most half a round (then that remainder, rounded up to whole
// columns of tiles, runs as twice as many narrow tiles, each half as long).
// Any split gives the same results; this only sets the schedule.
constexpr int kGateCUs = 256;
inline void gate_tile_split(int T, int N, int* wide_nt, int* narrow_nt) {
  const int mt = (T + GateGemm::BM - 1) / GateGemm::BM;
  const int nt = N / kTile;
  int wide = nt / 2;
  const long rem = ((long)mt * wide) % kGateCUs;
  if (rem != 0 && rem <= kGateCUs / 2) wide = max(0, wide - (int)((rem + mt - 1) / mt));
  *wide_nt = wide;
  *narrow_nt = nt - 2 * wide;
}

}  // namespace

}  // namespace sffn
