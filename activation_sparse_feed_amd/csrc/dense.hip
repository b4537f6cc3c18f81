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
#include "common.cuh"
#include "gemm_core.cuh"
#include "gemm_v2.cuh"
#include "launch.h"

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
// gate+up: 256 x 64 output tile of both z and u (2 x 2 waves of 128 x (32 + 32)).
__global__ __launch_bounds__(256, 2) void gateup_bf16_v2(DenseArgs a) {
  using G = Gemm2<2, 64, false, 32, 2>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES];
  const int nt = a.N / 64;
  const int mv = rows_valid(a);
  int mi, ni;
  tile_of((int)blockIdx.x, (a.M + G::BM - 1) / G::BM, nt, &mi, &ni);
  const int m0 = mi * G::BM, n0 = ni * 64;
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

// down: 128 x 128 output tile (the down GEMM has few N tiles, so 128-row tiles
// keep two workgroups per CU busy), wd [d_ff, d_model] staged K-major and
// read with transposing LDS reads.
__global__ __launch_bounds__(256, 2) void down_bf16_v2(DenseArgs a) {
  using G = Gemm2<1, 128, false, 32, 2, true, 128>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES];
  const int nt = (a.N + 127) / 128;
  const int mv = rows_valid(a);
  int mi, ni;
  tile_of((int)blockIdx.x, (a.M + G::BM - 1) / G::BM, nt, &mi, &ni);
  const int m0 = mi * G::BM, n0 = ni * 128;
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

}  // namespace

hipError_t launch_dense_gateup(int dtype, const void* x, const void* wg_t, const float* b_g,
                               const void* wu_t, void* h, int M, const int* rowmap,
                               const int* n_rows_dev, int K, int N, hipStream_t stream) {
  DenseArgs a{x, wg_t, wu_t, b_g, h, rowmap, n_rows_dev, M, K, N};
  if (dtype == 1 && K % 32 == 0) {
    hipLaunchKernelGGL(gateup_bf16_v2, dim3((unsigned)(((M + 255) / 256) * (N / 64))), dim3(256), 0,
                       stream, a);
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
    hipLaunchKernelGGL(down_bf16_v2, dim3((unsigned)(((M + 127) / 128) * ((N + 127) / 128))),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(((M + 127) / 128) * ((N + 127) / 128)));
  if (dtype == 1) hipLaunchKernelGGL(down_bf16, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(down_f32, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sffn
