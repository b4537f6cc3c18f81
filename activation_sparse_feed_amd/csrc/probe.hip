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
