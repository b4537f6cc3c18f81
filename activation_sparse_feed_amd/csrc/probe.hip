// Peak probes: the achievable HBM bandwidth and bf16 MFMA rate of the GPU the
// library runs on, measured with kernels of the same kind as the hot path's,
// so that every roofline fraction can also be stated against a measured
// denominator beside AMD's published one.
//
//   probe_stream  a grid-stride pass over a buffer much larger than the
//                 256 MB Infinity Cache: 16-byte loads, four chunks in flight
//                 per lane, either copied to a second buffer (read + write) or
//                 only read (folded into a register the compiler must keep).
//   probe_mfma    every wave runs 16 independent chains of
//                 v_mfma_f32_16x16x32_bf16 on operands of ones, with enough
//                 workgroups for several waves per SIMD: one wave alone (any
//                 chain count) leaves the matrix core idle about a third of
//                 the time, two or more keep it busy.  Each lane's sum of its
//                 accumulators is stored (2048 * iters, exact in float32 for
//                 iters < 8192), which also checks that every MFMA ran.
//   probe_cached  every workgroup reads the same small window (resident in
//                 each XCD's L2 after the first pass) many times with 16-byte
//                 loads, eight in flight per lane (four reach only about 60%
//                 of the rate): the rate at which the
//                 vector-memory path brings cached data into the CUs, the
//                 ceiling of any kernel that gathers rows it re-reads from L2.
//   probe_gather  one wave per listed row reads that row of two matrices
//                 (16-byte loads, the whole row in flight): the rate of a
//                 row gather like the sparse kernel's, without arithmetic.
//   probe_mfma_step
//                 one v_mfma_f32_16x16x32_bf16 per wave on caller-given
//                 operand registers, so a test can compare the instruction's
//                 result with the exact C + A.B: the error model that the
//                 TwELL epilogue's guard band assumes (one rounding of the
//                 result per instruction) is checked on the hardware itself.
#include <algorithm>

#include "common.cuh"
#include "sffn.h"

namespace sffn {

namespace {

constexpr int kProbeChains = 16;
constexpr int kProbeBlock = 256;

__global__ __launch_bounds__(kProbeBlock) void probe_stream(const u32x4_t* __restrict__ src,
                                                            u32x4_t* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4_t v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride],
                  v3 = src[i + 3 * stride];
    if (dst) {
      dst[i] = v0;
      dst[i + stride] = v1;
      dst[i + 2 * stride] = v2;
      dst[i + 3 * stride] = v3;
    } else {
      acc ^= (v0.x ^ v1.y) ^ (v2.z ^ v3.w);
    }
  }
  for (; i < n; i += stride) {
    const u32x4_t v = src[i];
    if (dst) dst[i] = v;
    else acc ^= v.x;
  }
  asm volatile("" ::"v"(acc));  // the read-only pass keeps its loads
}

__global__ __launch_bounds__(kProbeBlock) void probe_mfma(float* __restrict__ out, int iters,
                                                          uint32_t one_a, uint32_t one_b) {
  // two registers of the same value: the compiler then keeps every chain in
  // place instead of rotating accumulators through shared registers
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, u32x4_t{one_a, one_a, one_a, one_a});
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, u32x4_t{one_b, one_b, one_b, one_b});
  f32x4_t acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kCachedInflight = 8;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kProbeBlock) void probe_cached(const u32x4_t* __restrict__ src,
                                                            size_t n16, int reps) {
  uint32_t acc = 0;
  for (int r = 0; r < reps; ++r) {
    size_t i = threadIdx.x;
    for (; i + (kCachedInflight - 1) * kProbeBlock < n16; i += kCachedInflight * kProbeBlock) {
      u32x4_t v[kCachedInflight];
#pragma unroll
      for (int q = 0; q < kCachedInflight; ++q) v[q] = src[i + q * kProbeBlock];
#pragma unroll
      for (int q = 0; q < kCachedInflight; ++q) acc ^= v[q].x ^ v[q].w;
    }
    for (; i < n16; i += kProbeBlock) acc ^= src[i].x;
  }
  asm volatile("" ::"v"(acc));  // keeps the loads
}

template <int CH>  // 16-byte chunks per lane per row
__global__ __launch_bounds__(kProbeBlock) void probe_gather(const u32x4_t* __restrict__ a,
                                                            const u32x4_t* __restrict__ b,
                                                            const int* __restrict__ rows,
                                                            int nrows) {
  const int item = (int)blockIdx.x * (kProbeBlock / 64) + (int)(threadIdx.x >> 6);
  if (item >= nrows) return;
  const size_t base = (size_t)rows[item] * (CH * 64) + (threadIdx.x & 63);
  u32x4_t va[CH], vb[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    va[c] = a[base + 64 * c];
    vb[c] = b[base + 64 * c];
  }
  uint32_t acc = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) acc ^= va[c].x ^ vb[c].w;
  asm volatile("" ::"v"(acc));
}

// Wave w, lane l: A and B operand registers a/b[(w * 64 + l) * 8 .. + 8]
// (bf16 bits), accumulator c[(w * 64 + l) * 4 .. + 4]; d receives the MFMA's
// four accumulator registers at the same place.
__global__ __launch_bounds__(64) void probe_mfma_step(const u32x4_t* __restrict__ a,
                                                      const u32x4_t* __restrict__ b,
                                                      const f32x4_t* __restrict__ c,
                                                      f32x4_t* __restrict__ d) {
  const size_t i = (size_t)blockIdx.x * 64 + threadIdx.x;
  const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a[i]);
  const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b[i]);
  d[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c[i], 0, 0, 0);
}

// out[i] = the library's float32 -> bfloat16 rounding of in[i].
__global__ __launch_bounds__(kProbeBlock) void probe_bf16_round(const float* __restrict__ in,
                                                                uint16_t* __restrict__ out,
                                                                size_t n) {
  for (size_t i = (size_t)blockIdx.x * kProbeBlock + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kProbeBlock)
    out[i] = f32_to_bf16(in[i]);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

}  // namespace sffn

extern "C" int32_t sffn_probe_hbm(const void* src, void* dst, size_t bytes, int32_t workgroups,
                                  void* stream) {
  using namespace sffn;
  if (!src || !aligned16(src) || (dst && !aligned16(dst)) || bytes % 16 != 0 || workgroups <= 0)
    return SFFN_ERR_ARG;
  if (bytes == 0) return SFFN_OK;
  hipLaunchKernelGGL(probe_stream, dim3((unsigned)workgroups), dim3(kProbeBlock), 0,
                     (hipStream_t)stream, (const u32x4_t*)src, (u32x4_t*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}

extern "C" int32_t sffn_probe_mfma(float* out, int32_t workgroups, int32_t iters, void* stream) {
  using namespace sffn;
  if (!out || workgroups <= 0 || iters <= 0 || iters >= 8192) return SFFN_ERR_ARG;
  hipLaunchKernelGGL(probe_mfma, dim3((unsigned)workgroups), dim3(kProbeBlock), 0,
                     (hipStream_t)stream, out, (int)iters, 0x3F803F80u, 0x3F803F80u);
  return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}

extern "C" int32_t sffn_probe_mfma_step(const void* a, const void* b, const float* c, float* d,
                                        int32_t waves, void* stream) {
  using namespace sffn;
  if (!a || !b || !c || !d || !aligned16(a) || !aligned16(b) || !aligned16(c) || !aligned16(d) ||
      waves <= 0)
    return SFFN_ERR_ARG;
  hipLaunchKernelGGL(probe_mfma_step, dim3((unsigned)waves), dim3(64), 0, (hipStream_t)stream,
                     (const u32x4_t*)a, (const u32x4_t*)b, (const f32x4_t*)c, (f32x4_t*)d);
  return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}

extern "C" int32_t sffn_probe_cached(const void* src, size_t window_bytes, int32_t reps,
                                     int32_t workgroups, void* stream) {
  using namespace sffn;
  if (!src || !aligned16(src) || window_bytes % 16 != 0 || window_bytes == 0 || reps <= 0 ||
      workgroups <= 0)
    return SFFN_ERR_ARG;
  hipLaunchKernelGGL(probe_cached, dim3((unsigned)workgroups), dim3(kProbeBlock), 0,
                     (hipStream_t)stream, (const u32x4_t*)src, window_bytes / 16, (int)reps);
  return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}

extern "C" int32_t sffn_probe_gather(const void* a, const void* b, const int32_t* rows,
                                     int32_t nrows, int32_t row_bytes, void* stream) {
  using namespace sffn;
  if (!a || !b || !rows || !aligned16(a) || !aligned16(b) || nrows < 0) return SFFN_ERR_ARG;
  if (nrows == 0) return SFFN_OK;
  const dim3 grid((unsigned)((nrows + 3) / 4)), blk(kProbeBlock);
  hipStream_t s = (hipStream_t)stream;
  switch (row_bytes) {
    case 1024: hipLaunchKernelGGL(probe_gather<1>, grid, blk, 0, s, (const u32x4_t*)a, (const u32x4_t*)b, rows, nrows); break;
    case 2048: hipLaunchKernelGGL(probe_gather<2>, grid, blk, 0, s, (const u32x4_t*)a, (const u32x4_t*)b, rows, nrows); break;
    case 4096: hipLaunchKernelGGL(probe_gather<4>, grid, blk, 0, s, (const u32x4_t*)a, (const u32x4_t*)b, rows, nrows); break;
    case 8192: hipLaunchKernelGGL(probe_gather<8>, grid, blk, 0, s, (const u32x4_t*)a, (const u32x4_t*)b, rows, nrows); break;
    case 16384: hipLaunchKernelGGL(probe_gather<16>, grid, blk, 0, s, (const u32x4_t*)a, (const u32x4_t*)b, rows, nrows); break;
    default: return SFFN_ERR_ARG;
  }
  return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}

extern "C" int32_t sffn_probe_bf16_round(const float* in, uint16_t* out, size_t n, void* stream) {
  using namespace sffn;
  if (!in || !out) return SFFN_ERR_ARG;
  if (n == 0) return SFFN_OK;
  const size_t blocks = std::min<size_t>((n + kProbeBlock - 1) / kProbeBlock, 4096);
  hipLaunchKernelGGL(probe_bf16_round, dim3((unsigned)blocks), dim3(kProbeBlock), 0,
                     (hipStream_t)stream, in, out, n);
  return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}
