// Backward of the routed rows on MFMA tiles (the dense fallback's rows of the
// hybrid routing; pwwt.cn article, sections 03-04: rows that overflow the
// compact format take the dense path, in training as in inference).
//
// A routed row is a heavy one: its complete activity list (the row-wise
// ELLPACK lists that the backward rebuilds from the recomputed gate, one
// entry per active column, the exact activity decision included) holds a
// large share of the columns, so its per-entry gradients are dense products
// of the routed rows' x and gy with the weights:
//   rd_prep   copies the routed rows of x and gy into contiguous matrices
//             (rows up to the next multiple of 32 zeroed) and spreads each
//             row's list into a dense array hR [r, j]: the bf16 h of an active
//             entry, -0 (sign bit alone) for an inactive one (an active h is
//             never negative, so the sign bit marks activity exactly);
//   rd_uga    per 256 x 128 tile, u = xR wu_t^T and ga = gyR wd^T (two K
//             loops over d_model, two accumulators), then per entry
//             gz = ga u + lambda/T, gu = ga h, a = h u on the active entries
//             (0 elsewhere), written as bf16 [r, j] (for gx) and transposed
//             [j, r] (for the weight gradients), and each tile's column sums
//             of gz;
//   rd_gx     gx_r = gz wg_t + gu wu_t (K over d_ff, both products in one
//             accumulator), written to the routed rows of gx;
//   rd_gw     gwg_t = gz^T xR, gwu_t = gu^T xR, gwd = a^T gyR (K over the
//             routed rows); the column walk of backward.hip then adds the
//             other rows' sums to these;
//   rd_gb     gb += the tiles' gz column sums, in tile order (after the
//             column walk, which writes gb).
// The GEMMs run eight waves per workgroup (two per SIMD).
// The per-entry gradients are rounded to bf16 before the three products (the
// rounding a dense bf16 backward applies too).  Every sum runs in a fixed
// order: deterministic.  The kernels run only when the routed count reaches
// kDenseRoutedRows (device-side count); below it the per-entry kernels of
// backward.hip take the routed rows, and these return at once.
#include "common.cuh"
#include "gemm_v2.cuh"
#include "launch.h"

namespace sffn {

namespace {

struct RdArgs {
  const uint16_t* x;     // [T, D]
  const uint16_t* gy;    // [T, D]
  const uint16_t* wg;    // [N, D]
  const uint16_t* wu;    // [N, D]
  const uint16_t* wd;    // [N, D]
  const int32_t* routed;  // ascending routed rows
  const int32_t* n_routed;
  const uint16_t* ecount;  // [R] complete list lengths
  const uint16_t* eidx;    // [R, N] complete lists (ascending columns)
  const uint16_t* eval;    // [R, N] bf16 h
  uint16_t* xR;            // [ldr, D]
  uint16_t* gyR;           // [ldr, D]
  uint16_t* hR;            // [R, N]
  uint16_t* gz;            // [ldr, N]
  uint16_t* gu;            // [ldr, N]
  uint16_t* gzT;           // [N, ldt]
  uint16_t* guT;           // [N, ldt]
  uint16_t* aT;            // [N, ldt]
  float* gbp;              // [ldr / 256, N]
  uint16_t* gx;            // [T, D]
  float* gwg;              // [N, D]
  float* gwu;
  float* gwd;
  float* gb;               // [N] or null
  int T, D, N, R, ldr;     // ldr: R rounded up to a multiple of 256
  int ldt;                 // row stride of the transposed arrays, see transposed_stride
  float l1g;
};

__device__ __forceinline__ int routed_rows(const RdArgs& a) {
  return uniform(min(*a.n_routed, a.R));
}

__device__ __forceinline__ bool dense_on(int nr) { return nr >= kDenseRoutedRows; }

// Workgroup r: row r of xR, gyR (zero from the routed count up to the next
// multiple of 32) and of hR.
__global__ __launch_bounds__(256) void rd_prep(RdArgs a) {
  const int nr = routed_rows(a);
  if (!dense_on(nr)) return;
  const int r = (int)blockIdx.x;
  const int kp = (nr + 31) & ~31;
  if (r >= kp) return;
  const int nch = a.D / 8;  // 16-byte chunks per row
  u32x4_t* xo = (u32x4_t*)(a.xR + (size_t)r * a.D);
  u32x4_t* go = (u32x4_t*)(a.gyR + (size_t)r * a.D);
  if (r >= nr) {
    for (int c = (int)threadIdx.x; c < nch; c += 256) {
      xo[c] = u32x4_t{0u, 0u, 0u, 0u};
      go[c] = u32x4_t{0u, 0u, 0u, 0u};
    }
    return;
  }
  const int t = min(max(a.routed[r], 0), a.T - 1);
  const u32x4_t* xi = (const u32x4_t*)(a.x + (size_t)t * a.D);
  const u32x4_t* gi = (const u32x4_t*)(a.gy + (size_t)t * a.D);
  for (int c = (int)threadIdx.x; c < nch; c += 256) {
    xo[c] = xi[c];
    go[c] = gi[c];
  }
  uint16_t* hrow = a.hR + (size_t)r * a.N;
  for (int c = (int)threadIdx.x; c < a.N / 8; c += 256)
    ((u32x4_t*)hrow)[c] = u32x4_t{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  __syncthreads();
  const int n = min((int)a.ecount[r], a.N);
  const uint16_t* li = a.eidx + (size_t)r * a.N;
  const uint16_t* lv = a.eval + (size_t)r * a.N;
  for (int i = (int)threadIdx.x; i < n; i += 256) {
    const int j = min((int)li[i], a.N - 1);
    hrow[j] = lv[i] & 0x7fffu;  // an active h is never negative
  }
}

// Tile (mi, ni) of workgroup blockIdx.x over the row tiles of the actual
// routed count (the grid is sized for the largest count; the workgroups past
// the actual tiles return), through the XCD-aware map.  Numbering the tiles
// by the actual count keeps the working ones first and spread over the XCDs:
// numbered by the largest count (a multiple of 8 row tiles when the buffers
// are sized for every token), every tile of a given row tile landed on one
// XCD (u/ga 0.90 -> 1.97 ms at 2799 routed rows of d_ff 14336).
__device__ __forceinline__ bool rd_tile(int nr, int nt, int* mi, int* ni) {
  const int mt = (nr + 255) / 256, b = (int)blockIdx.x;
  if (b >= mt * nt) return false;
  tile_of(b, mt, nt, mi, ni);
  return true;
}

// 256 x 256 tiles of eight waves as 4 x 2 of 64 x 128, B staged K-major (gx,
// the weight gradients).
using RdKN = Gemm2<1, 256, false, 32, 2, true, 256, 4, 8, true>;


// u and ga of one 256 x 128 tile, eight waves as 4 x 2 of 64 x 64, both
// accumulators in registers.
using RdUG = Gemm2<1, 128, false, 32, 2, false, 256, 4, 8, true>;

__global__ __launch_bounds__(64 * RdUG::NWAVES, 1) void rd_uga(RdArgs a) {
  using G = RdUG;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES];
  const int nr = routed_rows(a);
  if (!dense_on(nr)) return;
  int mi, ni;
  if (!rd_tile(nr, a.N / 128, &mi, &ni)) return;
  const int m0 = mi * 256, n0 = ni * 128;
  G gu_, gg_;
  {
    const uint16_t* B[1] = {a.wu};
    gu_.init(a.xR, (size_t)a.ldr, nullptr, m0, nr, B, n0, a.N, a.D);
    gu_.run_pipe(lds, a.D);
  }
  {
    const uint16_t* B[1] = {a.wd};
    gg_.init(a.gyR, (size_t)a.ldr, nullptr, m0, nr, B, n0, a.N, a.D);
    gg_.run_pipe(lds, a.D);
  }
  const uint16_t* __restrict__ hR = a.hR;
  uint16_t* __restrict__ gzo = a.gz;
  uint16_t* __restrict__ guo = a.gu;
  uint16_t* __restrict__ gzT = a.gzT;
  uint16_t* __restrict__ guT = a.guT;
  uint16_t* __restrict__ aT = a.aT;
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  const int wm = w % G::WAVES_M, wn = w / G::WAVES_M;
  const int jl = wn * G::WN + (lane & 15);  // the lane's first column in the tile
  float colsum[G::FN];
#pragma unroll
  for (int fn = 0; fn < G::FN; ++fn) colsum[fn] = 0.f;
#pragma unroll
  for (int fm = 0; fm < G::FM; ++fm) {
    const int rb = m0 + wm * G::WM + fm * 16 + 4 * (lane >> 4);  // rows rb .. rb + 3
    // the block's h values first, all loads in flight together
    uint16_t hb[G::FN][4];
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hb[fn][i] = rb + i < nr ? hR[(size_t)(rb + i) * a.N + n0 + jl + fn * 16] : (uint16_t)0x8000u;
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn) {
      const int j = n0 + jl + fn * 16;
      uint32_t pz[2], pu[2], pa[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float gz = 0.f, gu = 0.f, av = 0.f;
        if (!(hb[fn][i] & 0x8000u)) {
          const float h = bf16_to_f32(hb[fn][i]);
          const float u = gu_.acc[0][fm][fn][i], ga = gg_.acc[0][fm][fn][i];
          gz = ga * u + a.l1g;
          gu = ga * h;
          av = h * u;
        }
        colsum[fn] += gz;
        const uint16_t bz = f32_to_bf16(gz), bu = f32_to_bf16(gu), ba = f32_to_bf16(av);
        gzo[(size_t)(rb + i) * a.N + j] = bz;
        guo[(size_t)(rb + i) * a.N + j] = bu;
        if (i & 1) {
          pz[i >> 1] |= (uint32_t)bz << 16;
          pu[i >> 1] |= (uint32_t)bu << 16;
          pa[i >> 1] |= (uint32_t)ba << 16;
        } else {
          pz[i >> 1] = bz;
          pu[i >> 1] = bu;
          pa[i >> 1] = ba;
        }
      }
      // transposed: rows rb .. rb + 3 of column j are 8 contiguous bytes
      const size_t to = (size_t)j * a.ldt + rb;
      *(uint2*)(gzT + to) = make_uint2(pz[0], pz[1]);
      *(uint2*)(guT + to) = make_uint2(pu[0], pu[1]);
      *(uint2*)(aT + to) = make_uint2(pa[0], pa[1]);
    }
  }
  // the tile's column sums of gz: lanes 16 apart hold other rows of the same
  // column, then the four waves of a column half add in wave order (in the
  // pipeline's LDS, free after its closing barrier: one LDS object)
  float(*red)[128] = (float(*)[128])lds;
#pragma unroll
  for (int fn = 0; fn < G::FN; ++fn) {
    float s = colsum[fn];
    s += __shfl_xor(s, 16, kWave);
    s += __shfl_xor(s, 32, kWave);
    if (lane < 16) red[wm][wn * G::WN + fn * 16 + lane] = s;
  }
  __syncthreads();
  const int c = (int)threadIdx.x;
  if (c < 128)
    a.gbp[(size_t)mi * a.N + n0 + c] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// gx of the routed rows: gz wg_t + gu wu_t, the weights staged K-major
// (transposing LDS reads), both products in one accumulator.
__global__ __launch_bounds__(64 * RdKN::NWAVES, 1) void rd_gx(RdArgs a) {
  using G = RdKN;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES];
  const int nr = routed_rows(a);
  if (!dense_on(nr)) return;
  int mi, di;
  if (!rd_tile(nr, (a.D + 255) / 256, &mi, &di)) return;
  const int m0 = mi * 256, n0 = di * 256;
  G g;
  {
    const uint16_t* B[1] = {a.wg};
    g.init(a.gz, (size_t)a.ldr, nullptr, m0, nr, B, n0, a.D, a.N);
    g.run_pipe(lds, a.N);
  }
  {
    const uint16_t* B[1] = {a.wu};
    g.init(a.gu, (size_t)a.ldr, nullptr, m0, nr, B, n0, a.D, a.N, 0, 0, false);
    g.run_pipe(lds, a.N);
  }
  g.for_each([&](int, int row, int col, float v) {
    const int r = m0 + row, d = n0 + col;
    if (r < nr && d < a.D) a.gx[(size_t)a.routed[r] * a.D + d] = f32_to_bf16(v);
  });
}

// The weight gradients' routed part: out[j, :] = A[j, :] B, K over the
// routed rows (padded with zeros to a multiple of 32), B (xR or gyR,
// [rows, D]) staged K-major.  blockIdx.x: product (gwg_t, gwu_t, gwd)
// outermost, then column tiles, then row tiles.
__device__ __forceinline__ void gw_tile(const RdArgs& a, const uint16_t* A, const uint16_t* Bm,
                                        float* out, int m0, int n0, int kp, uint8_t* lds) {
  using G = RdKN;
  G g;
  const uint16_t* B[1] = {Bm};
  g.init(A, (size_t)a.N, nullptr, m0, a.N, B, n0, a.D, kp, a.ldt);
  g.run_pipe(lds, kp);
  g.for_each([&](int, int row, int col, float v) {
    const int j = m0 + row, d = n0 + col;
    if (j < a.N && d < a.D) out[(size_t)j * a.D + d] = v;
  });
}

__global__ __launch_bounds__(64 * RdKN::NWAVES, 1) void rd_gw(RdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[RdKN::LDS_BYTES];
  const int nr = routed_rows(a);
  if (!dense_on(nr)) return;
  const int kp = (nr + 31) & ~31;
  const int mt = (a.N + 255) / 256, dt = (a.D + 255) / 256;
  const int prod = (int)blockIdx.x / (mt * dt);
  int mi, di;
  tile_of((int)blockIdx.x % (mt * dt), mt, dt, &mi, &di);
  const int m0 = mi * 256, n0 = di * 256;
  // one call per product, each with its operands straight from the kernel
  // arguments, so that the buffer descriptors stay in scalar registers
  if (prod == 0) gw_tile(a, a.gzT, a.xR, a.gwg, m0, n0, kp, lds);
  else if (prod == 1) gw_tile(a, a.guT, a.xR, a.gwu, m0, n0, kp, lds);
  else gw_tile(a, a.aT, a.gyR, a.gwd, m0, n0, kp, lds);
}

// gb += the tiles' gz column sums, in tile order.
__global__ __launch_bounds__(256) void rd_gb(RdArgs a) {
  const int nr = routed_rows(a);
  if (!dense_on(nr) || a.gb == nullptr) return;
  const int j = (int)(blockIdx.x * 256 + threadIdx.x);
  if (j >= a.N) return;
  const int mt = (nr + 255) / 256;
  float s = 0.f;
  for (int mi = 0; mi < mt; ++mi) s += a.gbp[(size_t)mi * a.N + j];
  a.gb[j] += s;
}

size_t al256r(size_t v) { return (v + 255) & ~(size_t)255; }

// Row stride (elements) of gzT, guT and aT: ldr, or ldr + 256 when ldr / 256
// is even, so that the stride is an odd multiple of 512 bytes.  A stride of
// a large power of two (ldr = 16384 when the buffers are sized for every
// token) puts the 256 rows that a weight-gradient tile reads, and the
// columns that rd_uga stores, on the same few memory channels.
int transposed_stride(int ldr) { return (ldr / 256) % 2 == 0 ? ldr + 256 : ldr; }

}  // namespace

size_t routed_dense_workspace_bytes(int N, int D, int R) {
  const size_t ldr = ((size_t)R + 255) & ~(size_t)255;
  const size_t ldt = (size_t)transposed_stride((int)ldr);
  return 2 * al256r(ldr * D * 2) + al256r((size_t)R * N * 2) + 2 * al256r(ldr * N * 2) +
         3 * al256r((size_t)N * ldt * 2) + al256r(ldr / 256 * N * 4);
}

hipError_t launch_backward_routed_dense(const void* x, const void* gy, const void* wg_t,
                                        const void* wu_t, const void* wd, const int32_t* routed,
                                        const int32_t* n_routed, const uint16_t* ecount,
                                        const uint16_t* eidx, const void* eval, void* gx,
                                        float* gwg_t, float* gwu_t, float* gwd, float* gb,
                                        int T, int D, int N, int R, float l1g, void* ws,
                                        int stage, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const int ldr = (R + 255) & ~255, ldt = transposed_stride(ldr);
  char* p = (char*)ws;
  RdArgs a{};
  a.x = (const uint16_t*)x;
  a.gy = (const uint16_t*)gy;
  a.wg = (const uint16_t*)wg_t;
  a.wu = (const uint16_t*)wu_t;
  a.wd = (const uint16_t*)wd;
  a.routed = routed;
  a.n_routed = n_routed;
  a.ecount = ecount;
  a.eidx = eidx;
  a.eval = (const uint16_t*)eval;
  a.xR = (uint16_t*)p;
  p += al256r((size_t)ldr * D * 2);
  a.gyR = (uint16_t*)p;
  p += al256r((size_t)ldr * D * 2);
  a.hR = (uint16_t*)p;
  p += al256r((size_t)R * N * 2);
  a.gz = (uint16_t*)p;
  p += al256r((size_t)ldr * N * 2);
  a.gu = (uint16_t*)p;
  p += al256r((size_t)ldr * N * 2);
  a.gzT = (uint16_t*)p;
  p += al256r((size_t)N * ldt * 2);
  a.guT = (uint16_t*)p;
  p += al256r((size_t)N * ldt * 2);
  a.aT = (uint16_t*)p;
  p += al256r((size_t)N * ldt * 2);
  a.gbp = (float*)p;
  a.gx = (uint16_t*)gx;
  a.gwg = gwg_t;
  a.gwu = gwu_t;
  a.gwd = gwd;
  a.gb = gb;
  a.T = T;
  a.D = D;
  a.N = N;
  a.R = R;
  a.ldr = ldr;
  a.ldt = ldt;
  a.l1g = l1g;
  const unsigned mtw = (unsigned)(ldr / 256);
  if (stage == 0) {
    // the routed rows' products, before the column walk (which adds the
    // other rows' weight-gradient sums to rd_gw's)
    const dim3 blk(64 * RdKN::NWAVES);
    hipLaunchKernelGGL(rd_prep, dim3((unsigned)(((R + 31) / 32) * 32)), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(rd_uga, dim3(mtw * (unsigned)(N / 128)), blk, 0, stream, a);
    hipLaunchKernelGGL(rd_gx, dim3(mtw * (unsigned)((D + 255) / 256)), blk, 0, stream, a);
    hipLaunchKernelGGL(rd_gw, dim3((unsigned)(3 * ((N + 255) / 256) * ((D + 255) / 256))), blk, 0,
                       stream, a);
    return hipGetLastError();
  }
  // stage 1: gb, added to what the column walk wrote (after it)
  hipLaunchKernelGGL(rd_gb, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sffn
