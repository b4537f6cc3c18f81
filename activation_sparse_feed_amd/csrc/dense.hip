// Dense gated FFN on the matrix cores: the same-GPU speed-up reference and the
// dense fallback of the hybrid route (pwwt.cn article, section 03: rows that
// overflow the compact format go to a dense path on the matrix units).
//
//   gate+up: h[m, n] = ReLU(z[m, n]) * u[m, n], z = x wg_t^T + b, u = x wu_t^T,
//            both projections share the A tile (one kernel, two accumulators);
//            h is rounded to dtype.
//   down:    y[m, :] = h[m, :] wd, wd [d_ff, d_model] transposed into the
//            K-contiguous LDS layout by the loader.
// Both take an optional row map (gather of x rows / scatter of y rows) and an
// optional device-side row count, so the hybrid route runs them on the routed
// rows without a host synchronisation.
#include <algorithm>

#include "common.cuh"
#include "gemm_core.cuh"
#include "gemm_v2.cuh"
#include "launch.h"
#include "route.cuh"

namespace sffn {

namespace {

struct DenseArgs {
  const void* a;       // A matrix [*, K]
  const void* b0;      // B matrices
  const void* b1;
  const float* bias;
  void* out;
  const int* rowmap;
  const int* n_rows_dev;
  int M, K, N;
  // routed gate+up only: when route_count is set, each workgroup finds the
  // routed rows of the M <= 256 rows itself from the TwELL counts (no row map
  // or device count is read) and workgroup 0 writes them to routed_out and
  // n_routed_out for the down kernels.
  const uint16_t* route_count = nullptr;
  int route_nt = 0, route_cap = 0;
  int32_t* routed_out = nullptr;
  int32_t* n_routed_out = nullptr;
  // routed gate+up only: when route_mask is set (many tokens), each workgroup
  // finds its tiles' routed rows in the route_flags mask of route_groups
  // words and writes its share of routed_out (and workgroup 0 n_routed_out);
  // the row map and device count are then left to the kernels after it.
  const uint16_t* route_mask = nullptr;
  int route_groups = 0;
  // fused route only: per-output-tile split counters of the down GEMM, zeroed
  // by workgroup 0 of the routed gate+up before the down GEMM runs
  int* tile_count = nullptr;
  int tile_count_n = 0;
  // routed rows: the eight-wave kernels (gateup_routed_wide, down_routed_wide)
  // were launched too and take every count above kRoutedBigRows
  int routed_wide = 0;
};

__device__ __forceinline__ int rows_valid(const DenseArgs& a) {
  return a.n_rows_dev ? *a.n_rows_dev : a.M;
}

// ---------------------------------------------------------------- gate + up
__global__ __launch_bounds__(256) void gateup_bf16(DenseArgs a) {
  using G = MfmaGemm<2, 64, false>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[G::LDS_BYTES / 2];
  const int nt = a.N / 64;
  const int m0 = (blockIdx.x / nt) * G::BM;
  const int n0 = (blockIdx.x % nt) * 64;
  const int mv = rows_valid(a);
  if (m0 >= mv) return;
  G g;
  const uint16_t* B[2] = {(const uint16_t*)a.b0, (const uint16_t*)a.b1};
  g.init((const uint16_t*)a.a, a.K, a.rowmap, m0, mv, B, a.K, n0, a.N);
  g.run(lds, a.K);
  // acc[0] = z tile, acc[1] = u tile, identical layouts
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  uint16_t* h = (uint16_t*)a.out;
#pragma unroll
  for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn) {
      const int col = n0 + wn * G::WN + fn * 16 + (lane & 15);
      const float bb = a.bias ? a.bias[col] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + fm * 16 + 4 * (lane >> 4) + r;
        if (m < mv) {
          const float z = g.acc[0][fm][fn][r] + bb;
          const float hv = z > 0.f ? z * g.acc[1][fm][fn][r] : 0.f;
          h[(size_t)m * a.N + col] = f32_to_bf16(hv);
        }
      }
    }
}

__global__ __launch_bounds__(256) void gateup_f32(DenseArgs a) {
  using G = ValuGemm<2, 64, false, false>;
  __shared__ __attribute__((aligned(16))) float lds[G::LDS_BYTES / 4];
  const int nt = a.N / 64;
  const int m0 = (blockIdx.x / nt) * G::BM;
  const int n0 = (blockIdx.x % nt) * 64;
  const int mv = rows_valid(a);
  if (m0 >= mv) return;
  G g;
  const float* B[2] = {(const float*)a.b0, (const float*)a.b1};
  g.run(lds, (const float*)a.a, a.K, a.rowmap, m0, mv, B, a.K, n0, a.N, a.K);
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  float* h = (float*)a.out;
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j) {
      const int m = m0 + ty * G::TM + i;
      const int col = n0 + tx * G::TN + j;
      if (m < mv) {
        const float z = g.acc[0][i][j] + (a.bias ? a.bias[col] : 0.f);
        h[(size_t)m * a.N + col] = z > 0.f ? z * g.acc[1][i][j] : 0.f;
      }
    }
}

// --------------------------------------------------------------------- down
__global__ __launch_bounds__(256) void down_bf16(DenseArgs a) {
  using G = MfmaGemm<1, 128, false, true>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[G::LDS_BYTES / 2];
  const int nt = (a.N + 127) / 128;
  const int m0 = (blockIdx.x / nt) * G::BM;
  const int n0 = (blockIdx.x % nt) * 128;
  const int mv = rows_valid(a);
  if (m0 >= mv) return;
  G g;
  const uint16_t* B[1] = {(const uint16_t*)a.b0};
  g.init((const uint16_t*)a.a, a.K, nullptr, m0, mv, B, a.N, n0, a.N);
  g.run(lds, a.K);
  uint16_t* y = (uint16_t*)a.out;
  g.for_each([&](int, int row, int col, float v) {
    const int m = m0 + row, n = n0 + col;
    if (m < mv && n < a.N) {
      const int orow = a.rowmap ? a.rowmap[m] : m;
      y[(size_t)orow * a.N + n] = f32_to_bf16(v);
    }
  });
}

__global__ __launch_bounds__(256) void down_f32(DenseArgs a) {
  using G = ValuGemm<1, 128, true, false>;
  __shared__ __attribute__((aligned(16))) float lds[G::LDS_BYTES / 4];
  const int nt = (a.N + 127) / 128;
  const int m0 = (blockIdx.x / nt) * G::BM;
  const int n0 = (blockIdx.x % nt) * 128;
  const int mv = rows_valid(a);
  if (m0 >= mv) return;
  G g;
  const float* B[1] = {(const float*)a.b0};
  g.run(lds, (const float*)a.a, a.K, nullptr, m0, mv, B, a.N, n0, a.N, a.K);
  float* y = (float*)a.out;
  g.for_each([&](int, int row, int col, float v) {
    const int m = m0 + row, n = n0 + col;
    if (m < mv && n < a.N) {
      const int orow = a.rowmap ? a.rowmap[m] : m;
      y[(size_t)orow * a.N + n] = v;
    }
  });
}

// ------------------------------------------------ bf16, buffer-load main loop
// gate+up: 256 x 64 output tile of both z and u (2 x 2 waves of 128 x (32 + 32)),
// two workgroups per CU; or (DenseWide) 256 x 128 of both, eight waves as
// 4 x 2 of 64 x (64 + 64), one workgroup per CU: a quarter fewer LDS fragment
// bytes per MFMA, used when the tiles fill at least two rounds of the CUs,
// with each step's loads and fragment reads spread among its MFMAs.
using DenseNarrow = Gemm2<2, 64, false, 32, 2>;
using DenseWide = Gemm2<2, 128, false, 32, 2, false, 256, 4, 8, true>;

// Workgroups per CU that the LDS ring of a configuration allows (one or two).
template <class G>
constexpr int wg_per_cu() {
  return G::LDS_BYTES > 80 * 1024 ? 1 : 2;
}

template <class G>
__global__ __launch_bounds__(64 * G::NWAVES, wg_per_cu<G>()) void gateup_bf16_v2(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES];
  // each of the two B matrices (wg_t, wu_t) contributes BN / 2 columns of the tile
  static_assert(G::BN % 2 == 0, "two B matrices");
  constexpr int TW = G::BN / 2;
  const int nt = a.N / TW;
  const int mv = rows_valid(a);
  int mi, ni;
  tile_of((int)blockIdx.x, (a.M + G::BM - 1) / G::BM, nt, &mi, &ni);
  const int m0 = mi * G::BM, n0 = ni * TW;
  if (m0 >= mv) return;
  G g;
  const uint16_t* B[2] = {(const uint16_t*)a.b0, (const uint16_t*)a.b1};
  g.init((const uint16_t*)a.a, (size_t)a.M, a.rowmap, m0, mv, B, n0, a.N, a.K);
  g.run_pipe(lds, a.K);
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  const int wm = w % G::WAVES_M, wn = w / G::WAVES_M;
  uint16_t* h = (uint16_t*)a.out;
#pragma unroll
  for (int fn = 0; fn < G::FN; ++fn) {
    const int col = n0 + wn * G::WN + fn * 16 + (lane & 15);
    const float bb = a.bias ? a.bias[col] : 0.f;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * G::WM + fm * 16 + 4 * (lane >> 4) + r;
        if (m < mv) {
          const float z = g.acc[0][fm][fn][r] + bb;
          h[(size_t)m * a.N + col] = f32_to_bf16(z > 0.f ? z * g.acc[1][fm][fn][r] : 0.f);
        }
      }
  }
}

// down: wd [d_ff, d_model] staged K-major and read with transposing LDS
// reads.  DownNarrow: 128 x 128 output tiles, two workgroups per CU (the down
// GEMM has few N tiles); DownWide: 256 x 256 tiles, eight waves as 4 x 2 of
// 64 x 128, one workgroup per CU: a quarter fewer LDS fragment bytes per MFMA
// and half the staging per output, used when the tiles fill at least two
// rounds of the CUs (loads and fragment reads spread among the MFMAs).
using DownNarrow = Gemm2<1, 128, false, 32, 2, true, 128>;
using DownWide = Gemm2<1, 256, false, 32, 2, true, 256, 4, 8, true>;

template <class G>
__global__ __launch_bounds__(64 * G::NWAVES, wg_per_cu<G>()) void down_bf16_v2(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES];
  const int nt = (a.N + G::BN - 1) / G::BN;
  const int mv = rows_valid(a);
  int mi, ni;
  tile_of((int)blockIdx.x, (a.M + G::BM - 1) / G::BM, nt, &mi, &ni);
  const int m0 = mi * G::BM, n0 = ni * G::BN;
  if (m0 >= mv) return;
  G g;
  const uint16_t* B[1] = {(const uint16_t*)a.b0};
  g.init((const uint16_t*)a.a, (size_t)a.M, nullptr, m0, mv, B, n0, a.N, a.K);
  g.run_pipe(lds, a.K);
  uint16_t* y = (uint16_t*)a.out;
  g.for_each([&](int, int row, int col, float v) {
    const int m = m0 + row, n = n0 + col;
    if (m < mv && n < a.N) {
      const int orow = a.rowmap ? a.rowmap[m] : m;
      y[(size_t)orow * a.N + n] = f32_to_bf16(v);
    }
  });
}

// ------------------------------------------- routed rows (hybrid fallback)
// The number of routed rows is only known on the device, so these kernels run
// a fixed grid of workgroups that loop over the tiles (and K splits) of the
// actual row count, tile i -> tile_of(i): each XCD takes a contiguous run of
// tiles in which the row tiles of a column tile come together, so the weight
// rows of that column tile come into the XCD's L2 once (6-10% faster than
// spreading a column tile's row tiles over the XCDs).  128-row tiles and a deeper LDS
// pipeline than the full-size kernels: with few tiles there are few
// workgroups per CU to hide memory latency with.
constexpr int kRoutedStages = 5;     // LDS ring depth of the 128-row routed gate+up
constexpr int kRoutedGrid = 512;     // workgroups of the routed kernels
constexpr int kRoutedMaxSplit = 8;   // K splits of the routed down GEMM

// gate+up of the routed rows for one Gemm2 configuration: tiles
// blockIdx.x, blockIdx.x + gridDim.x, ... of the mt x nt tiles.
// ranks (mask mode): each tile's rows are written from the mask into the
// start of the pipeline LDS, read into the loaders' offsets, and released
// before the ring is filled.
template <typename G>
__device__ __forceinline__ void gateup_routed_tiles(const DenseArgs& a, int mv, uint8_t* lds,
                                                    const MaskRanks* ranks = nullptr) {
  constexpr int TW = G::BN / 2;  // columns of each of the two B matrices per tile
  static_assert(G::LDS_BYTES >= G::BM * 4, "a tile's row list fits the pipeline LDS");
  const int mt = (mv + G::BM - 1) / G::BM, nt = a.N / TW;
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  const int wm = w % G::WAVES_M, wn = w / G::WAVES_M;
  uint16_t* h = (uint16_t*)a.out;
  const uint16_t* B[2] = {(const uint16_t*)a.b0, (const uint16_t*)a.b1};
  G g;
  for (int tile = (int)blockIdx.x; tile < mt * nt; tile += (int)gridDim.x) {
    int mi, ni;  // the row tiles of one column tile on one XCD: its weight rows read once into that L2
    tile_of(tile, mt, nt, &mi, &ni);
    const int m0 = mi * G::BM, n0 = ni * TW;
    if (ranks) {
      int* rows_s = (int*)lds;
      __syncthreads();  // the previous tile's ring reads are done
      ranks->emit(a.route_mask, m0, min(mv, m0 + G::BM), rows_s);
      __syncthreads();
      g.init((const uint16_t*)a.a, (size_t)a.M, rows_s, 0, min(G::BM, mv - m0), B, n0, a.N, a.K);
      __syncthreads();  // every wave holds its row offsets
    } else {
      g.init((const uint16_t*)a.a, (size_t)a.M, a.rowmap, m0, mv, B, n0, a.N, a.K);
    }
    g.run_pipe(lds, a.K);
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn) {
      const int col = n0 + wn * G::WN + fn * 16 + (lane & 15);
      const float bb = a.bias ? a.bias[col] : 0.f;
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * G::WM + fm * 16 + 4 * (lane >> 4) + r;
          if (m < mv) {
            const float z = g.acc[0][fm][fn][r] + bb;
            h[(size_t)m * a.N + col] = f32_to_bf16(z > 0.f ? z * g.acc[1][fm][fn][r] : 0.f);
          }
        }
    }
  }
}

// Few routed rows: 128-row tiles with a deeper pipeline (few workgroups per CU
// to hide memory latency with); more than kRoutedBigRows: 256-row tiles.
// From kRoutedWideTokens tokens on, those many-row counts go to the eight-wave
// 256-row tiles of the full-size kernels (DenseWide, DownWide), one workgroup
// per CU, in kernels of their own (gateup_routed_wide, down_routed_wide) that
// the launcher adds; each kernel returns at once when the device-side row
// count is not its own.  Below that token count the extra launches (a few us
// each when they find nothing to do) would cost more than they can save.
constexpr int kRoutedBigRows = 1024;
constexpr int kRoutedWideTokens = 8192;
constexpr int kWideGrid = 256;  // workgroups of the eight-wave routed kernels
using RoutedSmall = Gemm2<2, 64, false, 32, 2, false, 128, kRoutedStages>;
using RoutedBig = Gemm2<2, 64, false, 32, 2>;
// With the fused route (at most kRouteBlock rows): one stage less, so that the
// row list fits beside the ring and two workgroups still share a CU.
using RoutedFused = Gemm2<2, 64, false, 32, 2, false, 128, kRoutedStages - 1>;

template <bool FUSED>
__global__ __launch_bounds__(256, 2) void gateup_routed(DenseArgs a) {
  constexpr size_t kLds = FUSED ? RoutedFused::LDS_BYTES
                          : RoutedSmall::LDS_BYTES > RoutedBig::LDS_BYTES ? RoutedSmall::LDS_BYTES
                                                                          : RoutedBig::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  if constexpr (FUSED) {
    static_assert(kLds >= kRouteBlock * 4, "route flags fit the pipeline LDS");
    static_assert(kRouteBlock <= kRoutedBigRows, "few rows");
    __shared__ int rows_s[kRouteBlock];
    __shared__ int wave_tot[kRouteBlock / kWave];
    // the route scan (flags in the pipeline LDS, which is free until the tiles start)
    const int mv = uniform(route_rows_lds(a.route_count, a.M, a.route_nt, a.route_cap, (int*)lds,
                                          rows_s, wave_tot));
    if (blockIdx.x == 0) {
      if ((int)threadIdx.x < mv) a.routed_out[threadIdx.x] = rows_s[threadIdx.x];
      if (threadIdx.x == 0) *a.n_routed_out = mv;
      for (int i = (int)threadIdx.x; i < a.tile_count_n; i += (int)blockDim.x) a.tile_count[i] = 0;
    }
    a.rowmap = rows_s;
    gateup_routed_tiles<RoutedFused>(a, mv, lds);
  } else if (a.route_mask) {
    // the routed list from the mask: this workgroup's share of it for the
    // kernels after this one, and its own tiles' rows (wave totals of the
    // scan in the pipeline LDS past the largest tile's row list)
    MaskRanks ranks;
    ranks.init(a.route_mask, a.route_groups, (int*)lds + 256);
    const int mv = uniform(ranks.total);
    const int share = (mv + (int)gridDim.x - 1) / (int)gridDim.x;
    const int lo = min(mv, (int)blockIdx.x * share);
    ranks.emit(a.route_mask, lo, min(mv, lo + share), a.routed_out + lo);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.n_routed_out = mv;
    if (mv <= kRoutedBigRows) gateup_routed_tiles<RoutedSmall>(a, mv, lds, &ranks);
    else if (!a.routed_wide) gateup_routed_tiles<RoutedBig>(a, mv, lds, &ranks);
  } else {
    const int mv = uniform(rows_valid(a));  // scalar: the tile loop and buffer descriptors stay uniform
    if (mv <= kRoutedBigRows) gateup_routed_tiles<RoutedSmall>(a, mv, lds);
    else if (!a.routed_wide) gateup_routed_tiles<RoutedBig>(a, mv, lds);
  }
}

// More than kRoutedBigRows routed rows: 256 x (128 + 128) tiles, eight waves.
__global__ __launch_bounds__(64 * DenseWide::NWAVES, 1) void gateup_routed_wide(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[DenseWide::LDS_BYTES];
  const int mv = uniform(rows_valid(a));
  if (mv > kRoutedBigRows) gateup_routed_tiles<DenseWide>(a, mv, lds);
}

// K splits of the routed down GEMM for mt x nt output tiles: the fewest splits
// whose work items fill at least 90% of the grid's last round (few tiles: enough
// items for the grid; just over a round: two or more shorter rounds instead of
// a nearly empty one), else the best filling; at most kRoutedMaxSplit, at least
// 8 K steps per split, and at most three rounds of items (which bounds the
// partials at 3 * kRoutedGrid tiles of 128 x 128 floats).
__host__ __device__ inline int routed_down_splits(int mt, int nt, int K, int grid) {
  const int tiles = max(1, mt * nt);
  const int s_max = max(1, min(kRoutedMaxSplit, K / 256));
  int best = 1;
  int best_num = 0, best_den = 1;  // best filling as a fraction
  for (int s = 1; s <= s_max; ++s) {
    const int items = tiles * s;
    if (s > 1 && items > 3 * grid) break;
    const int slots = ((items + grid - 1) / grid) * grid;
    if (10 * items >= 9 * slots) return s;
    if ((long)items * best_den > (long)best_num * slots) {
      best = s;
      best_num = items;
      best_den = slots;
    }
  }
  return best;
}

// The routed down GEMM for mv rows: square tiles of bm (128, or 256 on the
// eight-wave kernel above kRoutedBigRows rows when it runs), mt x nt of them,
// S K splits over that kernel's grid; partials [S][mt * bm][N] when S > 1.
struct DownPlan {
  bool wide;
  int bm, mt, nt, S;
};
__host__ __device__ inline DownPlan routed_down_plan(int mv, int N, int K, bool wide_ok) {
  DownPlan p;
  p.wide = wide_ok && mv > kRoutedBigRows;
  p.bm = p.wide ? 256 : 128;
  p.mt = (mv + p.bm - 1) / p.bm;
  p.nt = (N + p.bm - 1) / p.bm;
  p.S = routed_down_splits(p.mt, p.nt, K, p.wide ? kWideGrid : kRoutedGrid);
  return p;
}

// y rows of the routed list: with one split, written directly (rounded);
// with S > 1, float32 partials [S][mt * BM][N] that down_routed_reduce sums.
// FOLD (few tokens, a.tile_count set): the tile's last split sums the
// partials; a template flag so that the many-token instantiation keeps its
// registers (and occupancy) free of the summation.  G: square BM x BN tiles
// of the K-major down GEMM.
template <class G, bool FOLD>
__device__ __forceinline__ void down_routed_items(const DenseArgs& a, float* partial,
                                                  const DownPlan& p, int mv, uint8_t* lds) {
  static_assert(G::BM == G::BN, "square tiles");
  const int mt = p.mt, nt = p.nt, S = p.S;
  const int nks = a.K / 32;
  uint16_t* y = (uint16_t*)a.out;
  for (int item = (int)blockIdx.x; item < mt * nt * S; item += (int)gridDim.x) {
    int mi, np;  // the row tiles of one (column tile, split) on one XCD, as in the gate+up
    tile_of(item, mt, nt * S, &mi, &np);
    const int ni = np % nt, si = np / nt;
    const int m0 = mi * G::BM, n0 = ni * G::BN;
    const int k_lo = (int)(((long)si * nks) / S) * 32;
    const int k_hi = (int)(((long)(si + 1) * nks) / S) * 32;
    G g;
    const uint16_t* B[1] = {(const uint16_t*)a.b0 + (size_t)k_lo * a.N};
    g.init((const uint16_t*)a.a + k_lo, (size_t)a.M, nullptr, m0, mv, B, n0, a.N, k_hi - k_lo,
           a.K, k_lo);
    g.run_pipe(lds, k_hi - k_lo);
    if (S == 1) {
      g.for_each([&](int, int row, int col, float v) {
        const int m = m0 + row, n = n0 + col;
        if (m < mv && n < a.N) y[(size_t)a.rowmap[m] * a.N + n] = f32_to_bf16(v);
      });
    } else {
      float* part = partial + ((size_t)si * mt * G::BM) * a.N;
      g.for_each([&](int, int row, int col, float v) {
        const int m = m0 + row, n = n0 + col;
        if (m < mv && n < a.N) part[(size_t)m * a.N + n] = v;
      });
      if (FOLD) {
        // the tile's last split to finish sums the splits' partials in split
        // order and writes y (no reduction launch): agent-scope fences make the
        // partials visible across the XCDs' L2s; nothing waits.  The flag
        // lives in the pipeline LDS, free after run_pipe's closing barrier.
        int* last_s = (int*)lds;
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) *last_s = atomicAdd(&a.tile_count[mi + mt * ni], 1) == S - 1;
        __syncthreads();
        if (*last_s) {
          __threadfence();
          const size_t per = (size_t)mt * G::BM * a.N;
          constexpr int Q = G::BN / 4;  // float4 columns per tile row
          for (int q = (int)threadIdx.x; q < G::BM * Q; q += (int)blockDim.x) {
            const int m = m0 + q / Q, n = n0 + 4 * (q % Q);
            if (m >= mv || n >= a.N) continue;
            const size_t off = (size_t)m * a.N + n;
            f32x4_t v = *(const f32x4_t*)(partial + off);
            for (int s2 = 1; s2 < S; ++s2) v += *(const f32x4_t*)(partial + s2 * per + off);
            uint16_t* dst = y + (size_t)a.rowmap[m] * a.N + n;
            *(uint2*)dst = make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                                      (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
          }
        }
        __syncthreads();  // the flag's LDS is the next item's first stage
      }
    }
  }
}

using RoutedDown = Gemm2<1, 128, false, 32, 2, true, 128, kRoutedStages>;

template <bool FOLD>
__global__ __launch_bounds__(256, 2) void down_routed(DenseArgs a, float* partial) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[RoutedDown::LDS_BYTES];
  const int mv = uniform(rows_valid(a));
  const DownPlan p = routed_down_plan(mv, a.N, a.K, a.routed_wide != 0);
  if (!p.wide) down_routed_items<RoutedDown, FOLD>(a, partial, p, mv, lds);
}

// More than kRoutedBigRows routed rows: 256 x 256 tiles, eight waves.
__global__ __launch_bounds__(64 * DownWide::NWAVES, 1) void down_routed_wide(DenseArgs a,
                                                                             float* partial) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[DownWide::LDS_BYTES];
  const int mv = uniform(rows_valid(a));
  const DownPlan p = routed_down_plan(mv, a.N, a.K, a.routed_wide != 0);
  if (p.wide) down_routed_items<DownWide, false>(a, partial, p, mv, lds);
}

// y[rowmap[m], n] = sum over splits of the partials, in split order.
constexpr int kRedUnroll = 4;
__global__ __launch_bounds__(256) void down_routed_reduce(DenseArgs a, const float* partial) {
  const int mv = uniform(rows_valid(a));
  const DownPlan p = routed_down_plan(mv, a.N, a.K, a.routed_wide != 0);
  const int S = p.S;
  if (S == 1) return;
  const size_t per = (size_t)p.mt * p.bm * a.N;  // floats per split
  const size_t n4 = (size_t)mv * a.N / 4;     // N % 8 == 0
  uint16_t* y = (uint16_t*)a.out;
  // kRedUnroll float4 groups per thread at a time, all their loads in flight
  // together (the grid is small: one launch that finds nothing to do stays cheap)
  constexpr int U = kRedUnroll;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x; i0 < n4; i0 += U * stride) {
    f32x4_t v[U];
    int row[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = min(i0 + u * stride, n4 - 1);
      v[u] = *(const f32x4_t*)(partial + 4 * i);
      row[u] = a.rowmap[(int)(4 * i / a.N)];
    }
    for (int s = 1; s < S; ++s)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t i = min(i0 + u * stride, n4 - 1);
        v[u] += *(const f32x4_t*)(partial + s * per + 4 * i);
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = i0 + u * stride;
      if (i >= n4) break;
      const size_t e = 4 * i;
      const int m = (int)(e / a.N), n = (int)(e - (size_t)m * a.N);
      uint16_t* dst = y + (size_t)row[u] * a.N + n;
      const uint32_t lo = (uint32_t)f32_to_bf16(v[u][0]) | ((uint32_t)f32_to_bf16(v[u][1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(v[u][2]) | ((uint32_t)f32_to_bf16(v[u][3]) << 16);
      *(uint2*)dst = make_uint2(lo, hi);
    }
  }
}

}  // namespace

hipError_t launch_dense_gateup(int dtype, const void* x, const void* wg_t, const float* b_g,
                               const void* wu_t, void* h, int M, const int* rowmap,
                               const int* n_rows_dev, int K, int N, hipStream_t stream) {
  DenseArgs a{x, wg_t, wu_t, b_g, h, rowmap, n_rows_dev, M, K, N};
  if (dtype == 1 && K % 32 == 0) {
    const long wide_tiles = (long)((M + 255) / 256) * (N / 128);
    if (N % 128 == 0 && wide_tiles >= 2 * 256)
      hipLaunchKernelGGL(gateup_bf16_v2<DenseWide>, dim3((unsigned)wide_tiles),
                         dim3(64 * DenseWide::NWAVES), 0, stream, a);
    else
      hipLaunchKernelGGL(gateup_bf16_v2<DenseNarrow>, dim3((unsigned)(((M + 255) / 256) * (N / 64))),
                         dim3(64 * DenseNarrow::NWAVES), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(((M + 127) / 128) * (N / 64)));
  if (dtype == 1) hipLaunchKernelGGL(gateup_bf16, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(gateup_f32, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_down(int dtype, const void* h, const void* wd, void* y, int M,
                       const int* rowmap, const int* n_rows_dev, int K, int N,
                       hipStream_t stream) {
  DenseArgs a{h, wd, nullptr, nullptr, y, rowmap, n_rows_dev, M, K, N};
  if (dtype == 1 && K % 32 == 0) {
    const long wide_tiles = (long)((M + 255) / 256) * ((N + 255) / 256);
    if (wide_tiles >= 2 * 256)
      hipLaunchKernelGGL(down_bf16_v2<DownWide>, dim3((unsigned)wide_tiles),
                         dim3(64 * DownWide::NWAVES), 0, stream, a);
    else
      hipLaunchKernelGGL(down_bf16_v2<DownNarrow>,
                         dim3((unsigned)(((M + 127) / 128) * ((N + 127) / 128))),
                         dim3(64 * DownNarrow::NWAVES), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(((M + 127) / 128) * ((N + 127) / 128)));
  if (dtype == 1) hipLaunchKernelGGL(down_bf16, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(down_f32, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sffn

namespace sffn {

size_t routed_partial_core_bytes(int T, int N, int K) {
  const bool wide_ok = T >= kRoutedWideTokens;  // as launch_routed_ffn decides
  // the largest S * mt * bm of routed_down_plan over every possible row count
  // (S > 1 only: one split writes y directly); the plan depends on the row
  // count through mt (and the tile kind), so one count per (kind, mt) suffices
  size_t rows = 0;
  for (int bm = 128; bm <= 256; bm += 128) {
    for (int mt = 1; mt <= (T + bm - 1) / bm; ++mt) {
      const int mv = std::min(T, mt * bm);
      const DownPlan p = routed_down_plan(mv, N, K, wide_ok);
      if (p.bm != bm || p.mt != mt) continue;
      if (p.S > 1) rows = std::max(rows, (size_t)p.S * p.mt * p.bm);
    }
  }
  return (rows * (size_t)N * 4 + 255) & ~(size_t)255;
}

// the partials, then the fused route's per-tile split counters
size_t routed_partial_bytes(int T, int N, int K) {
  return routed_partial_core_bytes(T, N, K) +
         (size_t)((T + 127) / 128) * ((N + 127) / 128) * sizeof(int);
}

hipError_t launch_routed_ffn(const void* x, const void* wg_t, const float* b_g, const void* wu_t,
                             const void* wd, void* h, void* y, float* partial, int T,
                             int32_t* routed, int32_t* n_routed, const uint16_t* route_count,
                             const uint16_t* route_mask, int route_nt, int route_cap,
                             int d_model, int d_ff, hipStream_t stream) {
  // h [rows, d_ff] = gate+up of the routed rows of x
  DenseArgs g{x, wg_t, wu_t, b_g, h, routed, n_routed, T, d_model, d_ff};
  // fused route (few tokens): the down GEMM's splits are summed by the last
  // split of each tile, with counters after the partials in the workspace
  int* tile_count = nullptr;
  const int count_n = ((T + 127) / 128) * ((d_model + 127) / 128);
  if (route_count) {
    g.route_count = route_count;
    g.route_nt = route_nt;
    g.route_cap = route_cap;
    g.routed_out = routed;
    g.n_routed_out = n_routed;
    tile_count = (int*)((char*)partial + routed_partial_core_bytes(T, d_model, d_ff));
    g.tile_count = tile_count;
    g.tile_count_n = count_n;
  } else if (route_mask) {
    g.route_mask = route_mask;
    g.route_groups = route_mask_words(T);
    g.routed_out = routed;
    g.n_routed_out = n_routed;
  }
  // from kRoutedWideTokens tokens on, counts above kRoutedBigRows go to the
  // eight-wave kernels launched after the four-wave ones (which then return
  // at once for such counts; the eight-wave ones return for the others)
  const bool wide = route_count == nullptr && T >= kRoutedWideTokens;
  g.routed_wide = wide;
  const int tiles_max = ((T + 127) / 128) * (d_ff / 64);
  if (route_count)
    hipLaunchKernelGGL(gateup_routed<true>, dim3((unsigned)min(tiles_max, kRoutedGrid)), dim3(256),
                       0, stream, g);
  else
    hipLaunchKernelGGL(gateup_routed<false>, dim3((unsigned)min(tiles_max, kRoutedGrid)), dim3(256),
                       0, stream, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (wide) {
    const long wide_tiles = (long)((T + 255) / 256) * (d_ff / 128);
    hipLaunchKernelGGL(gateup_routed_wide, dim3((unsigned)std::min<long>(kWideGrid, wide_tiles)),
                       dim3(64 * DenseWide::NWAVES), 0, stream, g);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // y rows = h wd
  DenseArgs d{h, wd, nullptr, nullptr, y, routed, n_routed, T, d_ff, d_model};
  d.tile_count = tile_count;
  d.routed_wide = wide;
  // grids no larger than the most work the row count allows (few tokens: the
  // launches that find no routed row dispatch fewer workgroups)
  const long down_items = (long)((T + 127) / 128) * ((d_model + 127) / 128) * kRoutedMaxSplit;
  const long red_blocks = ((long)T * d_model / 4 + 255) / 256;
  if (tile_count)
    hipLaunchKernelGGL(down_routed<true>, dim3((unsigned)std::min<long>(kRoutedGrid, down_items)),
                       dim3(256), 0, stream, d, partial);
  else
    hipLaunchKernelGGL(down_routed<false>, dim3((unsigned)std::min<long>(kRoutedGrid, down_items)),
                       dim3(256), 0, stream, d, partial);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (wide) {
    hipLaunchKernelGGL(down_routed_wide, dim3((unsigned)kWideGrid), dim3(64 * DownWide::NWAVES), 0,
                       stream, d, partial);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (tile_count) return hipSuccess;  // the down GEMM summed its own splits
  hipLaunchKernelGGL(down_routed_reduce, dim3((unsigned)std::max<long>(1, std::min<long>(256, red_blocks))),
                     dim3(256), 0, stream, d, (const float*)partial);
  return hipGetLastError();
}

}  // namespace sffn
