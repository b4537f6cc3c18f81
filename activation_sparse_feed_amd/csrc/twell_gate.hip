// Gate projection with the TwELL epilogue.
//
// One workgroup computes a 128-token x 128-column tile of z = x wg_t^T + b_g,
// i.e. exactly one TwELL column tile for 128 rows, so every (row, tile) list
// is built inside one workgroup with no atomics and no second kernel (the
// format is produced in the GEMM epilogue: pwwt.cn article, section 02; 1D
// column tiles: same section, and the neo-ai.one article on TwELL).
//
// Epilogue, per row (one wavefront per row, two columns per lane):
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
  int T, K, N, cap;
  GuardBand gb;
};

// Rows [r0, r0 + nrows) of the tile are staged in zs (row stride zld, float32
// or bfloat16 bits); the four waves take every fourth row.
__device__ __forceinline__ float zget(const float* zs, int i) { return zs[i]; }
__device__ __forceinline__ float zget(const uint16_t* zs, int i) { return bf16_to_f32(zs[i]); }

template <typename T, typename ZT>
__device__ void twell_rows(const GateArgs& a, const ZT* zs, int zld, int nrows, float band_scale,
                           const float* rn_a, const float* rn_b, int r0, int m0, int n0) {
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int nt = a.N / kTile;
  const int kt = n0 / kTile;
  const float b0 = a.b ? a.b[n0 + lane] : 0.f;
  const float b1 = a.b ? a.b[n0 + 64 + lane] : 0.f;
  const float nw0 = rn_b[lane], nw1 = rn_b[64 + lane];
  const T* x = (const T*)a.x;
  const T* wg = (const T*)a.wg;
  for (int rr = w; rr < nrows; rr += 4) {
    const int r = r0 + rr;
    const int t = m0 + r;
    if (t >= a.T) break;
    float z0 = zget(zs, rr * zld + lane);
    float z1 = zget(zs, rr * zld + 64 + lane);
    const float nx = rn_a[r];
    const float d0 = band_scale * (a.gb.coef_xw * nx * nw0 + a.gb.coef_b * fabsf(b0));
    const float d1 = band_scale * (a.gb.coef_xw * nx * nw1 + a.gb.coef_b * fabsf(b1));
    bool act0 = z0 > 0.f, act1 = z1 > 0.f;
    uint64_t f0 = __ballot(!(fabsf(z0) > d0));
    uint64_t f1 = __ballot(!(fabsf(z1) > d1));
    while (f0 | f1) {
      int c;
      if (f0) { c = __builtin_ctzll(f0); f0 &= f0 - 1; }
      else    { c = 64 + __builtin_ctzll(f1); f1 &= f1 - 1; }
      const float bc = a.b ? a.b[n0 + c] : 0.f;
      const ExactResult e = exact_gate_value<T>(x + (size_t)t * a.K, wg + (size_t)(n0 + c) * a.K,
                                                bc, a.K);
      if (c < 64) {
        if (lane == c) { act0 = e.sign > 0; z0 = (float)e.value; }
      } else {
        if (lane == c - 64) { act1 = e.sign > 0; z1 = (float)e.value; }
      }
    }
    const uint64_t m0m = __ballot(act0);
    const uint64_t m1m = __ballot(act1);
    const int c0 = __popcll(m0m);
    const size_t base = ((size_t)t * nt + kt) * a.cap;
    if (act0) {
      const int s = lanes_below(m0m);
      if (s < a.cap) {
        a.idx[base + s] = (uint16_t)(n0 + lane);
        Elt<T>::store1(a.val, base + s, z0);
      }
    }
    if (act1) {
      const int s = c0 + lanes_below(m1m);
      if (s < a.cap) {
        a.idx[base + s] = (uint16_t)(n0 + 64 + lane);
        Elt<T>::store1(a.val, base + s, z1);
      }
    }
    if (lane == 0) a.count[(size_t)t * nt + kt] = (uint16_t)(c0 + __popcll(m1m));
  }
}

// bf16: the whole 128 x 128 z tile (bias added) is staged in LDS as bfloat16,
// which is the value TwELL stores anyway; the guard band is widened by 2^-7
// to cover that rounding.  The accumulators are dead after staging, which
// keeps the exact re-evaluation from competing with them for registers.
constexpr int kZld16 = kTile + 8;

__global__ __launch_bounds__(256) void gate_twell_bf16(GateArgs a) {
  using G = MfmaGemm<1, kTile, true>;
  static_assert(G::LDS_BYTES >= (size_t)(128 * kZld16 * 2 + 256 * 4), "epilogue staging fits");
  __shared__ __attribute__((aligned(16))) uint16_t lds[G::LDS_BYTES / 2];
  const int nt = a.N / kTile;
  const int m0 = (blockIdx.x / nt) * G::BM;
  const int n0 = (blockIdx.x % nt) * kTile;
  G g;
  const uint16_t* B[1] = {(const uint16_t*)a.wg};
  g.init((const uint16_t*)a.x, a.K, nullptr, m0, a.T, B, a.K, n0, a.N);
  g.run(lds, a.K);
  // stage-buffer space is free now: z tile (bf16), then the row norms
  uint16_t* zs = lds;
  float* rn_a = (float*)(lds + 128 * kZld16);
  float* rn_b = rn_a + 128;
  g.write_norms(rn_a, rn_b);
  g.for_each([&](int, int row, int col, float v) {
    const float bb = a.b ? a.b[n0 + col] : 0.f;
    zs[row * kZld16 + col] = f32_to_bf16(v + bb);
  });
  __syncthreads();
  twell_rows<uint16_t>(a, zs, kZld16, 128, 1.0f + 0x1p-7f, rn_a, rn_b, 0, m0, n0);
}

__global__ __launch_bounds__(256) void gate_twell_f32(GateArgs a) {
  using G = ValuGemm<1, kTile, false, true>;
  constexpr size_t kZBytes = (64 * kZld + 256) * 4;
  constexpr size_t kBytes = G::LDS_BYTES > kZBytes ? G::LDS_BYTES : kZBytes;
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
  g.write_norms(rn_a, rn_b);
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
    g.for_each([&](int, int row, int col, float v) {
      if ((row >> 6) == half) {
        const float bb = a.b ? a.b[n0 + col] : 0.f;
        zs[(row - half * 64) * kZld + col] = v + bb;
      }
    });
    __syncthreads();
    twell_rows<float>(a, zs, kZld, 64, 1.0f, rn_a, rn_b, half * 64, m0, n0);
  }
}

}  // namespace

hipError_t launch_gate_twell(int dtype, const void* x, const void* wg_t, const float* b_g,
                             uint16_t* count, uint16_t* idx, void* val, int T, int K, int N,
                             int cap, GuardBand gb, hipStream_t stream) {
  GateArgs a{x, wg_t, b_g, count, idx, val, T, K, N, cap, gb};
  const int mt = (T + 127) / 128;
  const int nt = N / kTile;
  const dim3 grid((unsigned)(mt * nt));
  if (dtype == 1) {
    hipLaunchKernelGGL(gate_twell_bf16, grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(gate_twell_f32, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sffn
