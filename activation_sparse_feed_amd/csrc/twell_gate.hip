// Gate projection with the TwELL epilogue.
//
// One workgroup computes a tile of 128 or 256 tokens x 128 columns of
// z = x wg_t^T + b_g, i.e. exactly one TwELL column tile for those rows, so
// every (row, tile) list is built inside one workgroup with no atomics and no
// second kernel (the format is produced in the GEMM epilogue: pwwt.cn article,
// section 02; 1D column tiles: same section, and the neo-ai.one article on
// TwELL).  The row norms of the guard band come from a small norms pass.
//
// Epilogue of the 128-row kernels, per row (one wavefront per row, two
// columns per lane):
//   1. guard band: entries with |z32| <= coef_xw ||x_t|| ||w_j|| + coef_b |b_j|
//      are re-evaluated exactly (exact.cuh), so activity is the sign of the
//      exact z;
//   2. activity masks by wave ballot; slot = popcount of active lanes below,
//      which lists the active columns in ascending order;
//   3. slots below cap receive (global column, value rounded to dtype); the
//      uncapped count is written by lane 0.
#include "common.cuh"
#include "exact.cuh"
#include "gemm_core.cuh"
#include "gemm_v2.cuh"
#include "launch.h"
#include "twell_emit.cuh"

namespace sffn {

namespace {

// bf16, d_model % 8 == 0: 128 x 128 tiles on the register-staged main loop.
// The whole z tile (bias added) is staged in LDS as bfloat16, the value TwELL
// stores anyway; the guard band is widened by 2^-7 to cover that rounding.
constexpr int kZld16 = kTile + 8;

__global__ __launch_bounds__(256) void gate_twell_bf16(GateArgs a) {
  using G = MfmaGemm<1, kTile, false>;
  static_assert(G::LDS_BYTES >= (size_t)36864 + 4 * kExactLdsWords * 4, "epilogue staging fits");
  __shared__ __attribute__((aligned(16))) uint16_t lds[G::LDS_BYTES / 2];
  const int nt = a.N / kTile;
  const int m0 = (blockIdx.x / nt) * G::BM;
  const int n0 = (blockIdx.x % nt) * kTile;
  G g;
  const uint16_t* B[1] = {(const uint16_t*)a.wg};
  g.init((const uint16_t*)a.x, a.K, nullptr, m0, a.T, B, a.K, n0, a.N);
  g.run(lds, a.K);
  uint16_t* zs = lds;
  float* rn_a = (float*)(lds + 128 * kZld16);
  float* rn_b = rn_a + 128;
  load_tile_norms(a, m0, 128, n0, rn_a, rn_b);
  g.for_each([&](int, int row, int col, float v) {
    const float bb = a.b ? a.b[n0 + col] : 0.f;
    zs[row * kZld16 + col] = f32_to_bf16(v + bb);
  });
  __syncthreads();
  twell_rows<uint16_t>(a, zs, kZld16, 128, 1.0f + 0x1p-7f, rn_a, rn_b, 0, m0, n0,
                       (int*)(rn_b + 128), (uint32_t*)((uint8_t*)lds + 36864));
}

// bf16, d_model % 32 == 0: 256-row tiles on the buffer-load main loop, TwELL
// built straight from the MFMA accumulators; eight waves, two per SIMD, one
// workgroup per CU.  Two tile shapes in one grid: 256 x 256 (GateGemmWide,
// waves as 4 x 2, each 64 rows x one TwELL tile) wherever they fill whole
// rounds of the CUs, and 256 x 128 (GateGemm, waves as 8 x 1, each 32 rows x
// the TwELL tile) for a remainder that would leave a last round of wide tiles
// at most half full.  The wide tile reads 12 KB of LDS fragments per wave and
// K step for 64 x 128 outputs where the narrow one reads 10 KB for 32 x 128.
// (256 x 256 tiles of four waves as 2 x 2, one wave per SIMD, let the buffer
// loads stall the MFMA stream: slower.)
//
// A wave holds rows WM wm + 16 fm + 4 g + r and columns WN wn + 16 fn + i of
// the workgroup tile, for lane 16 g + i and accumulator (fm, fn, r).  For a
// fixed (fm, r), one ballot per fn gives, in its 16-bit segment g, the
// activity of columns 16 fn .. 16 fn + 15 of the wave's TwELL tile in row
// 16 fm + 4 g + r.  A column's slot is the number of active columns before it
// in its row: the popcounts of the row's segments of lower fn plus the active
// lanes below it in its own segment; the row's count is the sum over fn.  All
// of it stays inside the wave.
//
// Guard band: each entry is first tested against a bound for its whole row
// (largest column norm and bias of the wave's tile); only entries inside it
// get the per-entry band, and only those inside that are re-evaluated exactly.
constexpr int kEpiExactChunks = 4;  // exact re-evaluation: 16-byte chunks per lane loaded together

template <class G>
struct AccEpi {
  int m0, n0, nt, kt, wm, lane, gi, li;  // n0: first column of the wave's TwELL tile
  float cw, cb;
  float bias[G::FN], nw[G::FN];
  const float* rn_a;
  uint32_t* exact_lds;  // this wave's exact-stage area
  float l1;             // L1 regulariser: this lane's ReLU sum over its rows and columns
  // Stores: wave-uniform bases (the wave's first row, its TwELL tile) and this
  // lane's 32-bit byte offsets from them, so that each store takes one
  // scalar base and one vector offset.
  uint16_t* idx_w;
  uint16_t* val_w;
  uint16_t* cnt_w;
  uint32_t lane_b;      // bytes from the bases of idx/val to the lane's row group (rows + 4 gi)
  uint32_t lane_cb;     // bytes from cnt_w to the lane's row group's count
  uint32_t below;       // bits of the lanes before this one in its 16-lane segment
};

// One accumulator row group (fm, r): 4 rows of the wave, all 128 columns of
// its TwELL tile.  Template indices keep every accumulator access static (no
// spill of the accumulator array to scratch).
template <class G, int FM, int R>
__device__ __forceinline__ void epi_group(const GateArgs& a, G& g, AccEpi<G>& c) {
  constexpr int FN = G::FN;
  const int row = c.wm * G::WM + FM * 16 + 4 * c.gi + R;
  const int t = c.m0 + row;
  const bool valid = t < a.T;
  const float nx = c.rn_a[row];
  const float dmax = c.cw * nx + c.cb;
  float v[FN];
  bool fl = false;
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    v[fn] = g.acc[0][FM][fn][R] + c.bias[fn];
    fl |= valid && !(fabsf(v[fn]) > dmax);
  }
  if (__ballot(fl)) {
    // rare: per-entry band, exact re-evaluation inside it
    for (int fn = 0; fn < FN; ++fn) {
      const float d = a.gb.coef_xw * nx * c.nw[fn] + a.gb.coef_b * fabsf(c.bias[fn]);
      uint64_t fb = __ballot(valid && !(fabsf(v[fn]) > d));
      while (fb) {
        const int L = __builtin_ctzll(fb);
        fb &= fb - 1;
        const int lrow = c.wm * G::WM + FM * 16 + 4 * (L >> 4) + R;
        const int lcol = fn * 16 + (L & 15);
        const float bl = a.b ? a.b[c.n0 + lcol] : 0.f;
        const ExactResult e = exact_gate_value<uint16_t, kEpiExactChunks>(
            (const uint16_t*)a.x + (size_t)(c.m0 + lrow) * a.K,
            (const uint16_t*)a.wg + (size_t)(c.n0 + lcol) * a.K, bl, a.K, c.exact_lds);
        // activity is v > 0 from here on: a positive exact z that float32
        // cannot hold stays positive (its bfloat16 value is 0 either way)
        if (c.lane == L) v[fn] = e.sign > 0 ? fmaxf((float)e.value, 0x1p-149f) : (float)e.value;
      }
    }
  }
  // the group's rows (FM * 16 + R + 4 gi of the wave): byte offsets of the
  // lane's row in idx / val and in count
  const uint32_t rb = c.lane_b + (uint32_t)((FM * 16 + R) * c.nt * a.cap * 2);
  const uint32_t cb = c.lane_cb + (uint32_t)((FM * 16 + R) * c.nt * 2);
  int running = 0;
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const bool act = v[fn] > 0.f;
    const uint64_t m = __ballot(act);
    // at low density most 16-column groups of the four rows hold no active
    // entry: a uniform branch skips their slot arithmetic (the epilogue is
    // bound by VALU issue, all eight waves reaching it together)
    if (m == 0) continue;
    const uint32_t seg = (uint32_t)(m >> (16 * c.gi)) & 0xffffu;
    const int slot = running + __builtin_popcount(seg & c.below);
    if (act && valid && slot < a.cap) {
      const uint32_t o = rb + 2u * (uint32_t)slot;
      *(uint16_t*)((char*)c.idx_w + o) = (uint16_t)(c.n0 + fn * 16 + c.li);
      *(uint16_t*)((char*)c.val_w + o) = f32_to_bf16(v[fn]);
    }
    running += __builtin_popcount(seg);
  }
  if (c.li == 0 && valid) *(uint16_t*)((char*)c.cnt_w + cb) = (uint16_t)running;
  if (a.l1_part) {  // L1 regulariser, fixed order: per lane over its rows,
    float s = 0.f;     // one value per workgroup after the walk
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) s += v[fn] > 0.f ? v[fn] : 0.f;
    if (valid) c.l1 += s;
  }
}

template <class G, int FM, int R>
struct EpiLoop {
  __device__ static __forceinline__ void run(const GateArgs& a, G& g, AccEpi<G>& c) {
    epi_group<G, FM, R>(a, g, c);
    if constexpr (R + 1 < 4) EpiLoop<G, FM, R + 1>::run(a, g, c);
    else if constexpr (FM + 1 < G::FM) EpiLoop<G, FM + 1, 0>::run(a, g, c);
  }
};

// One output tile (rows m0.., columns n0..) of configuration G: main loop,
// then the TwELL epilogue from the accumulators.  Every wave's TwELL tile lies
// inside [0, N) (the launcher never lets a tile hang over the last column).
// epi: LDS outside the pipeline for the tile's row norms [BM], column norms
// [BN] and biases [BN]; they are loaded while the first stages are in flight.
template <class G>
__device__ __forceinline__ void gate_tile(const GateArgs& a, uint8_t* lds, float* epi, int m0,
                                          int n0) {
  const int nt = a.N / kTile;
  float* rn_a = epi;            // [BM]
  float* rn_b = rn_a + G::BM;   // [BN]
  float* bias_s = rn_b + G::BN;  // [BN]
  G g;
  const uint16_t* B[1] = {(const uint16_t*)a.wg};
  g.init((const uint16_t*)a.x, (size_t)a.T, nullptr, m0, a.T, B, n0, a.N, a.K);
  static_assert(G::BM <= 64 * G::NWAVES && G::BN <= 64 * G::NWAVES, "one element per thread");
  g.run_pipe(lds, a.K, [&] {
    const int i = (int)threadIdx.x;
    const float xn = (i < G::BM && m0 + i < a.T) ? a.xnorm[m0 + i] : 0.f;
    const float wn = i < G::BN ? a.wnorm[n0 + i] : 0.f;
    const float bb = (i < G::BN && a.b) ? a.b[n0 + i] : 0.f;
    if (i < G::BM) rn_a[i] = xn;
    if (i < G::BN) {
      rn_b[i] = wn;
      bias_s[i] = bb;
    }
  });

  // epilogue LDS (the pipeline stages are free after run_pipe's barrier):
  // one exact-stage area per wave
  constexpr int kExactOff = 0;
  static_assert(G::LDS_BYTES >= kExactOff + G::NWAVES * kExactLdsWords * 4, "epilogue LDS fits");
  const int w = uniform((int)(threadIdx.x >> 6));
  const int wn = w / G::WAVES_M;
  AccEpi<G> c;
  c.m0 = m0;
  c.n0 = n0 + wn * G::WN;
  c.nt = nt;
  c.kt = c.n0 / kTile;
  c.rn_a = rn_a;
  c.lane = lane_id();
  c.wm = w % G::WAVES_M;
  c.exact_lds = (uint32_t*)(lds + kExactOff) + w * kExactLdsWords;
  c.gi = c.lane >> 4;
  c.li = c.lane & 15;
  c.cw = 0.f;
  c.cb = 0.f;
  c.l1 = 0.f;
  {
    const size_t r0 = (size_t)(m0 + c.wm * G::WM);  // the wave's first row
    c.idx_w = a.idx + (r0 * nt + c.kt) * a.cap;
    c.val_w = (uint16_t*)a.val + (r0 * nt + c.kt) * a.cap;
    c.cnt_w = a.count + r0 * nt + c.kt;
    c.lane_b = (uint32_t)(4 * c.gi * nt * a.cap * 2);
    c.lane_cb = (uint32_t)(4 * c.gi * nt * 2);
    c.below = (1u << c.li) - 1u;
  }
#pragma unroll
  for (int fn = 0; fn < G::FN; ++fn) {
    const int col = fn * 16 + c.li;
    c.bias[fn] = bias_s[wn * G::WN + col];
    c.nw[fn] = rn_b[wn * G::WN + col];
    c.cw = fmaxf(c.cw, a.gb.coef_xw * c.nw[fn]);
    c.cb = fmaxf(c.cb, a.gb.coef_b * fabsf(c.bias[fn]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    c.cw = fmaxf(c.cw, __shfl_xor(c.cw, o, kWave));
    c.cb = fmaxf(c.cb, __shfl_xor(c.cb, o, kWave));
  }
  EpiLoop<G, 0, 0>::run(a, g, c);
  if (a.l1_part) {  // L1 regulariser: the workgroup's sum, fixed order, one store
    float* red = (float*)(lds + kExactOff + G::NWAVES * kExactLdsWords * 4);
    static_assert(G::LDS_BYTES >= kExactOff + G::NWAVES * (kExactLdsWords + 1) * 4, "fits");
    const float s = wave_sum_uniform(c.l1);
    if (c.lane == 0) red[w] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = 0.f;
      for (int i = 0; i < G::NWAVES; ++i) t += red[i];
      a.l1_part[blockIdx.x] = t;
    }
  }
}

// The grid: the first mt * wide_nt workgroups take 256 x 256 tiles
// (GateGemmWide) of columns [0, 256 wide_nt), the rest 256 x 128 tiles
// (GateGemm) of the columns after.  The wide tiles read a quarter fewer LDS
// bytes per MFMA; the narrow ones fill what would otherwise be a part-empty
// last round of wide tiles.
__global__ __launch_bounds__(64 * kGateWaves, 1) void gate_twell_bf16_v2(
    GateArgs a, int wide_nt, int narrow_nt) {
  static_assert(GateGemm::NWAVES == GateGemmWide::NWAVES, "one block size");
  static_assert(GateGemm::BM == GateGemmWide::BM, "one row tiling");
  constexpr size_t kLds = GateGemm::LDS_BYTES > GateGemmWide::LDS_BYTES ? GateGemm::LDS_BYTES
                                                                         : GateGemmWide::LDS_BYTES;
  // one LDS object: the pipeline stages, then the epilogue's norms and biases
  // (a second __shared__ array would cost the compiler its proof that the
  // fragment reads do not alias the buffer loads in flight)
  constexpr size_t kEpiFloats = GateGemmWide::BM + 2 * GateGemmWide::BN;
  static_assert(GateGemmWide::BN >= GateGemm::BN, "epilogue area sized by the wide tile");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds + kEpiFloats * 4];
  float* epi = (float*)(lds + kLds);
  const int mt = (a.T + GateGemm::BM - 1) / GateGemm::BM;
  const int n_wide = mt * wide_nt;
  const int bid = (int)blockIdx.x;
  int mi, ni;
  if (bid < n_wide) {
    tile_of(bid, mt, wide_nt, &mi, &ni);
    gate_tile<GateGemmWide>(a, lds, epi, mi * GateGemmWide::BM, ni * GateGemmWide::BN);
  } else {
    tile_of(bid - n_wide, mt, narrow_nt, &mi, &ni);
    gate_tile<GateGemm>(a, lds, epi, mi * GateGemm::BM,
                        wide_nt * GateGemmWide::BN + ni * GateGemm::BN);
  }
}

__global__ __launch_bounds__(256) void gate_twell_f32(GateArgs a) {
  using G = ValuGemm<1, kTile, false, false>;
  constexpr size_t kZBytes = 35840;  // >= (64 * kZld + 256 + 65) * 4, 256-aligned
  static_assert(kZBytes >= (64 * kZld + 256 + 65) * 4, "staging");
  constexpr size_t kBytes = (G::LDS_BYTES > kZBytes ? G::LDS_BYTES : kZBytes) + 4 * kExactLdsWords * 4;
  __shared__ __attribute__((aligned(16))) float lds[kBytes / 4];
  const int nt = a.N / kTile;
  const int m0 = (blockIdx.x / nt) * G::BM;
  const int n0 = (blockIdx.x % nt) * kTile;
  G g;
  const float* B[1] = {(const float*)a.wg};
  g.run(lds, (const float*)a.x, a.K, nullptr, m0, a.T, B, a.K, n0, a.N, a.K);
  float* zs = lds;
  float* rn_a = zs + 64 * kZld;
  float* rn_b = rn_a + 128;
  load_tile_norms(a, m0, 128, n0, rn_a, rn_b);
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
    g.for_each([&](int, int row, int col, float v) {
      if ((row >> 6) == half) {
        const float bb = a.b ? a.b[n0 + col] : 0.f;
        zs[(row - half * 64) * kZld + col] = v + bb;
      }
    });
    __syncthreads();
    twell_rows<float>(a, zs, kZld, 64, 1.0f, rn_a, rn_b, half * 64, m0, n0,
                      (int*)(rn_b + 128), (uint32_t*)((uint8_t*)lds + kBytes - 4 * kExactLdsWords * 4));
  }
}

// Few tokens (T <= 64, e.g. decode, or up to 128 with d_model % 64 == 0): the
// gate GEMM is a stream of wg_t, and a grid of one workgroup per column tile
// (or per 256-row tile) would leave most CUs idle.  Two kernels:
//
// gate_skinny_partial: workgroup = (column tile kt, K split s) of S splits;
// its four waves take consecutive quarters of the split's K range (at most
// kSkinnySteps MFMA K steps each), so the 128 rows of wg_t of one tile are
// read by 4S waves with no overlap.  Each wave issues the loads of all its
// steps at once, straight from global memory into MFMA operand registers (a
// 16-row x 64-byte fragment per load; consecutive steps read the two halves of
// the same cache lines), then runs the MFMAs; x rows past T repeat row 0 and are never emitted.  The
// waves also accumulate the sums of squares of the x values they load, which
// over the 4S waves of a tile cover every element of the T rows once, so the
// row norms of the guard band come out of this pass.  The four waves' tiles
// are summed in LDS, (w0 + w2) + (w1 + w3), and the workgroup writes that
// partial (fragment order) and its row sums of squares to the workspace.
//
// gate_skinny_epilogue: one workgroup per (tile, 16-row fragment) sums the S
// partials in split order, adds the bias, stages z in LDS and builds the TwELL
// lists with the row walk of the fp32 kernel (guard band, exact
// re-evaluation with all of a row's loads in flight at once).  The kernel
// boundary orders the partial writes before their reads, so no fence or
// counter is needed, and the sums are in a fixed order: deterministic.
constexpr int kSkinnyFN = kTile / 16;
constexpr int kSkinnySteps = 4;  // max K steps of 32 per wave

template <int MF>
struct Skinny {
  static constexpr int ROWS = 16 * MF;
  static constexpr int NFRAG = MF * kSkinnyFN;
  // floats per partial: NFRAG fragments of 64 lanes x 4, then ROWS sums of squares
  static constexpr int PART = NFRAG * 256 + ROWS;
  static constexpr int RED_BYTES = 2 * NFRAG * 64 * 16 + 4 * ROWS * 4;
};

template <int MF>
__global__ __launch_bounds__(256) void gate_skinny_partial(GateArgs a, float* partial, int S) {
  using SK = Skinny<MF>;
  constexpr int FN = kSkinnyFN;
  constexpr int ST = kSkinnySteps;
  __shared__ __attribute__((aligned(16))) uint8_t lds[SK::RED_BYTES];
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  const int kt = (int)blockIdx.x / S;
  const int s = (int)blockIdx.x - kt * S;
  const int n0 = kt * kTile;
  const int nk = a.K / 32;
  const int sp = s * 4 + w, nsp = S * 4;
  const int k_lo = (int)(((long)sp * nk) / nsp);
  const int nst = (int)(((long)(sp + 1) * nk) / nsp) - k_lo;  // <= ST (host guarantees)
  const int r = lane & 15, g = lane >> 4;

  const uint16_t* bp = (const uint16_t*)a.wg + (size_t)(n0 + r) * a.K + (size_t)k_lo * 32 + 8 * g;
  const size_t bstride = (size_t)16 * a.K;  // next fragment: 16 rows down
  u32x4_t bf[ST][FN], af[ST][MF];
#pragma unroll
  for (int i = 0; i < ST; ++i) {
    if (i < nst) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) bf[i][fn] = ldg16(bp + fn * bstride + i * 32);
#pragma unroll
      for (int fm = 0; fm < MF; ++fm) {
        // rows past T read row 0: MFMA output rows depend only on their own A
        // row, and those rows are never emitted
        const int row = 16 * fm + r;
        af[i][fm] = ldg16((const uint16_t*)a.x + (size_t)(row < a.T ? row : 0) * a.K +
                          (size_t)(k_lo + i) * 32 + 8 * g);
      }
    }
  }
  f32x4_t acc[MF][FN];
  float sq[MF];
#pragma unroll
  for (int fm = 0; fm < MF; ++fm) {
    sq[fm] = 0.f;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < ST; ++i) {
    if (i < nst) {
#pragma unroll
      for (int fm = 0; fm < MF; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, af[i][fm]), __builtin_bit_cast(bf16x8_t, bf[i][fn]),
              acc[fm][fn], 0, 0, 0);
        const u32x4_t v = af[i][fm];
        sq[fm] = dot2_bf16(v.x, v.x, dot2_bf16(v.y, v.y, dot2_bf16(v.z, v.z, dot2_bf16(v.w, v.w, sq[fm]))));
      }
    }
  }
  // row sums of squares: lanes r, r+16, r+32, r+48 hold row 16 fm + r
#pragma unroll
  for (int fm = 0; fm < MF; ++fm) {
    sq[fm] += __shfl_xor(sq[fm], 16, kWave);
    sq[fm] += __shfl_xor(sq[fm], 32, kWave);
  }

  // ---- workgroup reduction in LDS: (w0 + w2) + (w1 + w3)
  f32x4_t* red = (f32x4_t*)lds;                            // [2][NFRAG][64]
  float* redsq = (float*)(lds + 2 * SK::NFRAG * 64 * 16);  // [4][ROWS]
  if (g == 0) {
#pragma unroll
    for (int fm = 0; fm < MF; ++fm) redsq[w * SK::ROWS + 16 * fm + r] = sq[fm];
  }
  if (w >= 2) {
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) red[((w - 2) * SK::NFRAG + fm * FN + fn) * 64 + lane] = acc[fm][fn];
  }
  __syncthreads();
  if (w < 2) {
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] += red[(w * SK::NFRAG + fm * FN + fn) * 64 + lane];
  }
  __syncthreads();
  if (w == 1) {
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) red[(fm * FN + fn) * 64 + lane] = acc[fm][fn];
  }
  __syncthreads();
  if (w != 0) return;
  float* mine = partial + ((size_t)kt * S + s) * SK::PART;
#pragma unroll
  for (int fm = 0; fm < MF; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const f32x4_t v = acc[fm][fn] + red[(fm * FN + fn) * 64 + lane];
      *(f32x4_t*)(mine + (size_t)((fm * FN + fn) * 64 + lane) * 4) = v;
    }
  for (int i = lane; i < SK::ROWS; i += kWave)
    mine[SK::NFRAG * 256 + i] =
        (redsq[i] + redsq[2 * SK::ROWS + i]) + (redsq[SK::ROWS + i] + redsq[3 * SK::ROWS + i]);
}

template <int MF>
constexpr int kStreamBK = 64;     // K depth of a stage of the streaming kernel
constexpr int kStreamWgs8 = 256;  // workgroups of the streaming kernel above 64 tokens

// gate_skinny_stream (d_model % 64 == 0): the same partials from a workgroup
// that streams its tile's wg_t rows over its split's K range through an LDS
// ring (the buffer-load pipeline with an A tile of the 16 MF token rows; every
// load instruction fetches 1 KB of whole cache lines).  The four waves take 32
// columns each, so their tiles are disjoint: no reduction across waves, and
// one workgroup per (tile, split) with S chosen so that the grid fits the chip
// at once (about one workgroup per CU).  Wave 0 also sums the squares of the x values it feeds to the MFMA.
template <int MF>
using StreamGemm = Gemm2<1, kTile, false, kStreamBK<MF>, 4, false, 16 * MF, 4, 4>;

template <int MF>
__global__ __launch_bounds__(256) void gate_skinny_stream(GateArgs a, float* partial, int S) {
  using SK = Skinny<MF>;
  using G = StreamGemm<MF>;
  static_assert(G::FM == MF && G::FN == 2, "wave tile: all token rows, 32 columns");
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES];
  const int kt = (int)blockIdx.x / S;
  const int s = (int)blockIdx.x - kt * S;
  const int nc = a.K / 64;  // 64-wide K chunks
  const int c_lo = (int)(((long)s * nc) / S), c_hi = (int)(((long)(s + 1) * nc) / S);
  const int k_lo = c_lo * 64;
  G g;
  const uint16_t* B[1] = {(const uint16_t*)a.wg + k_lo};
  g.init((const uint16_t*)a.x + k_lo, (size_t)a.T, nullptr, 0, a.T, B, kt * kTile, a.N,
         (c_hi - c_lo) * 64, a.K, k_lo);
  g.template run_pipe<true>(lds, (c_hi - c_lo) * 64);
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  float* mine = partial + ((size_t)kt * S + s) * SK::PART;
  // fragment (fm, fn) of wave w is fragment (fm, 2 w + fn) of the tile
#pragma unroll
  for (int fm = 0; fm < MF; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
      *(f32x4_t*)(mine + (size_t)((fm * kSkinnyFN + 2 * w + fn) * 64 + lane) * 4) = g.acc[0][fm][fn];
  if (w == 0) {
#pragma unroll
    for (int fm = 0; fm < MF; ++fm) {
      float q = g.sqa[fm];
      q += __shfl_xor(q, 16, kWave);
      q += __shfl_xor(q, 32, kWave);
      if (lane < 16) mine[SK::NFRAG * 256 + 16 * fm + lane] = q;
    }
  }
}

template <int MF>
__global__ __launch_bounds__(256) void gate_skinny_epilogue(GateArgs a, const float* partial,
                                                            int S) {
  using SK = Skinny<MF>;
  constexpr int FN = kSkinnyFN;
  constexpr int EPI_BYTES = (16 * kZld + SK::ROWS + 2 * kTile + 17) * 4 + 4 * kExactLdsWords * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[EPI_BYTES];
  const int kt = (int)blockIdx.x / MF;
  const int fm = (int)blockIdx.x - kt * MF;  // this workgroup's 16 rows: 16 fm ..
  const int n0 = kt * kTile;
  if (16 * fm >= a.T) return;
  float* zs = (float*)lds;           // [16][kZld]
  float* rn_a = zs + 16 * kZld;      // [ROWS], entries 16 fm .. 16 fm + 15 used
  float* rn_b = rn_a + SK::ROWS;     // [128]
  float* bias_s = rn_b + kTile;      // [128]
  int* defer = (int*)(bias_s + kTile); // [1 + 16]
  uint32_t* exact_lds = (uint32_t*)(lds + EPI_BYTES - 4 * kExactLdsWords * 4);
  const float* part0 = partial + (size_t)kt * S * SK::PART + (size_t)fm * FN * 256;
  // Every load of the workgroup is issued before the first is used (one
  // memory round trip for the first eight splits): the bias and column norms,
  // the partial row sums of squares (threads 0..15) and the partial z.  Split
  // indices past S are clamped and their terms masked, so the code is straight.
  // The FN fragments of row fragment fm are 2 float4 per thread; thread tid
  // sums entries tid and tid + 256 of the S partials in split order.
  const int col0 = 16 * ((int)threadIdx.x >> 6) + ((int)threadIdx.x & 15);  // entry tid; entry tid + 256 is col0 + 64
  float bb[2] = {0.f, 0.f};
  if (a.b) {
    bb[0] = a.b[n0 + col0];
    bb[1] = a.b[n0 + col0 + 64];
  }
  const float wn = a.wnorm[n0 + ((int)threadIdx.x & (kTile - 1))];
  const bool sq_thread = threadIdx.x < 16;
  const float* sq0 = partial + (size_t)kt * S * SK::PART + SK::NFRAG * 256 + 16 * fm + (threadIdx.x & 15);
  f32x4_t v[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  float t = 0.f;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4_t ld[8][2];
    float q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int su = min(s0 + u, S - 1);
#pragma unroll
      for (int m = 0; m < 2; ++m)
        ld[u][m] = *(const f32x4_t*)(part0 + (size_t)su * SK::PART + (size_t)(threadIdx.x + 256 * m) * 4);
      q[u] = sq0[(size_t)su * SK::PART];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool in = s0 + u < S;
#pragma unroll
      for (int m = 0; m < 2; ++m) v[m] += in ? ld[u][m] : zero4;
      t += in ? q[u] : 0.f;  // sums of squares: the masked terms are +0
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int p = threadIdx.x + 256 * m;  // fn * 64 + fragment lane
    const int fl = p & 63;
    const int col = col0 + 64 * m;
#pragma unroll
    for (int i = 0; i < 4; ++i) zs[(4 * (fl >> 4) + i) * kZld + col] = v[m][i] + bb[m];
  }
  if (sq_thread) rn_a[16 * fm + threadIdx.x] = sqrtf(t);
  if (threadIdx.x < kTile) rn_b[threadIdx.x] = wn;
  if (((threadIdx.x >> 4) & 3) == 0) {  // one thread per column of 0..63
    bias_s[col0] = bb[0];
    bias_s[col0 + 64] = bb[1];
  }
  __syncthreads();
  twell_rows<uint16_t, float, 8>(a, (const float*)zs, kZld, 16, 1.0f, rn_a, rn_b, 16 * fm, 0, n0,
                                 defer, exact_lds, bias_s);
}

// Splits of the few-token gate: at least enough that no wave has more than
// kSkinnySteps K steps, and about kSkinnyWgs workgroups when the K
// range allows it (one step per wave at most that many splits).
constexpr int kSkinnyWgs = 512;
int skinny_splits(int K, int N) {
  const int nt = N / kTile;
  const int nk = K / 32;
  const int s_min = (nk + 4 * kSkinnySteps - 1) / (4 * kSkinnySteps);
  const int s_max = max(1, nk / 4);
  int S = max(kSkinnyWgs / nt, s_min);
  S = min(S, max(s_max, s_min));
  return max(S, 1);
}

bool use_stream(int K) { return K % 64 == 0; }
// 65 to 128 tokens: the streaming kernel only (the register-staged partial
// kernel would need twice its registers for 8 row fragments)
bool use_skinny(int dtype, int T, int K) {
  return dtype == 1 && K % 32 == 0 && (T <= 64 || (T <= 128 && use_stream(K)));
}

// Splits of the streaming kernel: about one workgroup per CU (kStreamWgs
// in all; fewer, longer streams also leave fewer partials to sum), at most one
// per 64-wide K chunk.
constexpr int kStreamWgs = 256;
int stream_splits(int K, int N, int T) {
  const int nt = N / kTile;
  const int wgs = T > 64 ? kStreamWgs8 : kStreamWgs;
  return max(1, min(wgs / nt, K / 64));
}

int few_token_splits(int K, int N, int T) {
  return use_stream(K) ? stream_splits(K, N, T) : skinny_splits(K, N);
}


}  // namespace

size_t gate_workspace_bytes(int dtype, int T, int K, int N) {
  if (!use_skinny(dtype, T, K)) return 0;
  const int nt = N / kTile;
  const int S = few_token_splits(K, N, T);
  const size_t part = T <= 32 ? Skinny<2>::PART : T <= 64 ? Skinny<4>::PART : Skinny<8>::PART;
  return (size_t)nt * S * part * 4;
}

bool gate_needs_xnorm(int dtype, int T, int K) { return !use_skinny(dtype, T, K); }

hipError_t launch_gate_twell(int dtype, const void* x, const void* wg_t, const float* b_g,
                             const float* xnorm, const float* wnorm, uint16_t* count,
                             uint16_t* idx, void* val, int T, int K, int N, int cap,
                             GuardBand gb, void* gate_ws, float* l1_part, size_t* l1_n,
                             hipStream_t stream) {
  GateArgs a{x, wg_t, b_g, count, idx, val, xnorm, wnorm, T, K, N, cap, gb, l1_part};
  const int nt = N / kTile;
  if (l1_n) *l1_n = (size_t)T * nt;  // one sum per (row, tile), except the 256-row kernel
  if (use_skinny(dtype, T, K)) {
    // Guard band for this summation order: the MFMA steps of a split (at most
    // kSkinnySteps per wave and two adds across the waves for the partial
    // kernel; the whole split, ceil(nc / S) 64-wide chunks, for the streaming
    // kernel), S partials and the bias.  With the measured MFMA error (product
    // truncation at most 8u of sum |x_k w_k| over the whole sum, 2u of
    // rounding per instruction) the total is below u (2 steps + S + 11)
    // ||x|| ||w||, which 4u (steps + S + 2) covers.
    const bool strm = use_stream(K);
    const int S = few_token_splits(K, N, T);
    const int steps = strm ? 2 * ((K / 64 + S - 1) / S) : kSkinnySteps + 2;
    a.gb.coef_xw = 0x1p-22f * (float)(steps + S + 2);
    float* partial = (float*)gate_ws;
    const dim3 gp((unsigned)(nt * S)), blk(256);
    if (T <= 32) {
      if (strm) hipLaunchKernelGGL(gate_skinny_stream<2>, gp, blk, 0, stream, a, partial, S);
      else hipLaunchKernelGGL(gate_skinny_partial<2>, gp, blk, 0, stream, a, partial, S);
      hipLaunchKernelGGL(gate_skinny_epilogue<2>, dim3((unsigned)(nt * 2)), blk, 0, stream, a, partial, S);
    } else if (T <= 64) {
      if (strm) hipLaunchKernelGGL(gate_skinny_stream<4>, gp, blk, 0, stream, a, partial, S);
      else hipLaunchKernelGGL(gate_skinny_partial<4>, gp, blk, 0, stream, a, partial, S);
      hipLaunchKernelGGL(gate_skinny_epilogue<4>, dim3((unsigned)(nt * 4)), blk, 0, stream, a, partial, S);
    } else {  // use_skinny: d_model % 64 == 0 here
      hipLaunchKernelGGL(gate_skinny_stream<8>, gp, blk, 0, stream, a, partial, S);
      hipLaunchKernelGGL(gate_skinny_epilogue<8>, dim3((unsigned)(nt * 8)), blk, 0, stream, a, partial, S);
    }
  } else if (dtype == 1 && K % GateGemm::BK == 0) {
    int wide_nt, narrow_nt;
    gate_tile_split(T, N, &wide_nt, &narrow_nt);
    const int mt = (T + GateGemm::BM - 1) / GateGemm::BM;
    const dim3 g2((unsigned)(mt * (wide_nt + narrow_nt)));
    hipLaunchKernelGGL(gate_twell_bf16_v2, g2, dim3(64 * GateGemm::NWAVES), 0, stream, a, wide_nt,
                       narrow_nt);
    if (l1_n) *l1_n = g2.x;  // one sum per workgroup
  } else if (dtype == 1) {
    hipLaunchKernelGGL(gate_twell_bf16, dim3((unsigned)(((T + 127) / 128) * nt)), dim3(256), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL(gate_twell_f32, dim3((unsigned)(((T + 127) / 128) * nt)), dim3(256), 0,
                       stream, a);
  }
  return hipGetLastError();
}


}  // namespace sffn
