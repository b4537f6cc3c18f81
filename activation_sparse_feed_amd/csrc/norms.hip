// Euclidean norms of matrix rows (float32), used by the guard band of the
// TwELL activity decision: |z32 - z| <= c * ||x_t|| * ||w_j|| bounds the
// float32 accumulation error of z = x_t . w_j (Cauchy-Schwarz on sum |x_k w_k|).
//
// One wavefront per row, 16-byte loads, float32 sum of squares, uniform DPP
// reduction.  Two matrices can be handled by one launch (rows of the first,
// then rows of the second).
#include "common.cuh"
#include "launch.h"

namespace sffn {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void row_norms_kernel(const T* __restrict__ a, int rows_a,
                                                        float* __restrict__ out_a,
                                                        const T* __restrict__ b, int rows_b,
                                                        float* __restrict__ out_b, int K) {
  constexpr int E = Elt<T>::kPerChunk;
  const int row = uniform((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (row >= rows_a + rows_b) return;
  const bool first = row < rows_a;
  const T* src = first ? a + (size_t)row * K : b + (size_t)(row - rows_a) * K;
  const int lane = lane_id();
  const int nch = K / E;
  float s = 0.f;
  constexpr int U = 4;
  for (int base = 0; base < nch; base += kWave * U) {
    u32x4_t c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = base + lane + kWave * u;
      c[u] = ch < nch ? ldg16(src + (size_t)ch * E) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[E];
      Elt<T>::unpack(c[u], f);
#pragma unroll
      for (int e = 0; e < E; ++e) s = fmaf(f[e], f[e], s);
    }
  }
  const float tot = wave_sum_uniform(s);
  if (lane == 0) {
    if (first) out_a[row] = sqrtf(tot);
    else out_b[row - rows_a] = sqrtf(tot);
  }
}

}  // namespace

hipError_t launch_row_norms(int dtype, const void* a, int rows_a, float* out_a, const void* b,
                            int rows_b, float* out_b, int K, hipStream_t stream) {
  const int rows = rows_a + rows_b;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (dtype == 1) {
    hipLaunchKernelGGL(row_norms_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       (const uint16_t*)a, rows_a, out_a, (const uint16_t*)b, rows_b, out_b, K);
  } else {
    hipLaunchKernelGGL(row_norms_kernel<float>, grid, dim3(256), 0, stream, (const float*)a,
                       rows_a, out_a, (const float*)b, rows_b, out_b, K);
  }
  return hipGetLastError();
}

}  // namespace sffn
