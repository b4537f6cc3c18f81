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

// L1 regulariser reduction: block b sums its contiguous slice of the
// per-(row, tile) sums in float64 (each thread a fixed stride, then a fixed
// butterfly and wave order); the final launch sums the block results the same
// way.  Deterministic.
constexpr int kL1Blocks = 256;

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum(v);
  const int w = (int)(threadIdx.x >> 6);
  if (lane_id() == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  return t;
}

__global__ __launch_bounds__(256) void l1_partial_sums(const float* __restrict__ part, size_t n,
                                                       double* __restrict__ blk) {
  __shared__ double red[4];
  const size_t chunk = (n + kL1Blocks - 1) / kL1Blocks;
  const size_t lo = (size_t)blockIdx.x * chunk, hi = min(n, lo + chunk);
  double s = 0.0;
  for (size_t i = lo + threadIdx.x; i < hi; i += blockDim.x) s += (double)part[i];
  const double t = block_sum_f64(s, red);
  if (threadIdx.x == 0) blk[blockIdx.x] = t;
}

// One workgroup for up to kL1Single sums: each thread a fixed stride, then the
// same fixed butterfly and wave order.
constexpr size_t kL1Single = 65536;

__global__ __launch_bounds__(1024) void l1_single(const float* __restrict__ part, size_t n,
                                                  double scale, float* __restrict__ out) {
  __shared__ double red[16];
  double s = 0.0;
  for (size_t i = threadIdx.x; i < n; i += blockDim.x) s += (double)part[i];
  const double t = block_sum_f64(s, red);
  if (threadIdx.x == 0) *out = (float)(t * scale);
}

__global__ __launch_bounds__(256) void l1_final(const double* __restrict__ blk, double scale,
                                                float* __restrict__ out) {
  __shared__ double red[4];
  const double t = block_sum_f64(threadIdx.x < kL1Blocks ? blk[threadIdx.x] : 0.0, red);
  if (threadIdx.x == 0) *out = (float)(t * scale);
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

size_t l1_ws_bytes() { return (size_t)kL1Blocks * sizeof(double); }

namespace {
__global__ void l1_set_zero(float* out) { *out = 0.f; }
}  // namespace

hipError_t launch_l1_zero(float* out, hipStream_t stream) {
  hipLaunchKernelGGL(l1_set_zero, dim3(1), dim3(1), 0, stream, out);
  return hipGetLastError();
}

hipError_t launch_l1_reduce(const float* part, size_t n, double scale, void* ws, float* out,
                            hipStream_t stream) {
  if (n <= kL1Single) {
    hipLaunchKernelGGL(l1_single, dim3(1), dim3(1024), 0, stream, part, n, scale, out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(l1_partial_sums, dim3(kL1Blocks), dim3(256), 0, stream, part, n, (double*)ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(l1_final, dim3(1), dim3(256), 0, stream, (const double*)ws, scale, out);
  return hipGetLastError();
}

}  // namespace sffn
