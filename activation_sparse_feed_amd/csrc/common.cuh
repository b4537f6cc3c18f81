// Device helpers shared by the sffn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sffn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round-to-nearest-even float -> bfloat16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // v_cvt_pk_bf16_f32
}

// Storage traits: elements per 16-byte chunk and conversion of one chunk.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int kPerChunk = 4;
  __device__ static __forceinline__ void unpack(const u32x4_t& c, float* o) {
    o[0] = __uint_as_float(c.x); o[1] = __uint_as_float(c.y);
    o[2] = __uint_as_float(c.z); o[3] = __uint_as_float(c.w);
  }
  __device__ static __forceinline__ float load1(const void* p, size_t i) {
    return ((const float*)p)[i];
  }
  __device__ static __forceinline__ void store1(void* p, size_t i, float v) {
    ((float*)p)[i] = v;
  }
};
template <> struct Elt<uint16_t> {  // bfloat16 stored as its bit pattern
  static constexpr int kPerChunk = 8;
  __device__ static __forceinline__ void unpack(const u32x4_t& c, float* o) {
    o[0] = bf16lo(c.x); o[1] = bf16hi(c.x); o[2] = bf16lo(c.y); o[3] = bf16hi(c.y);
    o[4] = bf16lo(c.z); o[5] = bf16hi(c.z); o[6] = bf16lo(c.w); o[7] = bf16hi(c.w);
  }
  __device__ static __forceinline__ float load1(const void* p, size_t i) {
    return bf16_to_f32(((const uint16_t*)p)[i]);
  }
  __device__ static __forceinline__ void store1(void* p, size_t i, float v) {
    ((uint16_t*)p)[i] = f32_to_bf16(v);
  }
};

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Number of set bits of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// DPP move of a float (all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xf, 0xf, false));
}

// Sum over the 64 lanes, returned uniformly: butterfly within each 16-lane
// row (quad_perm [1,0,3,2], [2,3,0,1], row_ror 4, row_ror 8), then the four
// row sums read from lanes 0, 16, 32, 48.  Fixed order: deterministic.
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x124>(v);
  v += dpp_f32<0x128>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Dot of two packed bfloat16 pairs accumulated in float32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return (T)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ u32x4_t ldg16(const void* p) {
  return *(const u32x4_t*)p;
}

}  // namespace sffn
