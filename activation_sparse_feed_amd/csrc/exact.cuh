// Exact sign (and accurate value) of a gate pre-activation z = b + sum_k x_k w_k.
//
// The TwELL epilogue decides activity (z > 0) on the exact value of z.  The
// float32 GEMM result is trusted only outside a guard band around zero; the
// few entries inside it are re-evaluated here by a whole wavefront:
//
//   stage 1  float64 sum of the products, which are exact in float64 for
//            float32 and bfloat16 inputs (at most 24 + 24 significand bits),
//            together with sum |p|.  With n terms per lane and a 6-level
//            butterfly, |error| <= gamma_{n+7} (sum|p| + |b|); the sign is
//            taken when |s| exceeds twice that bound.
//   stage 2  otherwise, exact fixed-point accumulation: a 640-bit two's
//            complement integer whose bit 0 weighs 2^-352 holds every product
//            of finite float32 values (>= 2^-298, < 2^256) and the sum of up
//            to 2^16 of them without rounding or overflow.
#pragma once

#include "common.cuh"

namespace sffn {

constexpr int kAccLimbs = 20;      // 20 x 32 bits
constexpr int kAccLsbShift = 352;  // bit 0 weighs 2^-352

struct ExactAcc {
  uint32_t l[kAccLimbs];
};

__device__ __forceinline__ void acc_zero(ExactAcc& a) {
#pragma unroll
  for (int i = 0; i < kAccLimbs; ++i) a.l[i] = 0u;
}

// a += p, exactly.  p must be 0 or have magnitude in [2^-350, 2^270).
__device__ __forceinline__ void acc_add(ExactAcc& a, double p) {
  const uint64_t bits = (uint64_t)__double_as_longlong(p);
  if ((bits << 1) == 0) return;
  const int E = (int)((bits >> 52) & 0x7ff);
  const uint64_t m = (bits & 0xFFFFFFFFFFFFFull) | (E ? (1ull << 52) : 0ull);
  const int pos = (E ? E : 1) - 1075 + kAccLsbShift;  // bit index of m's LSB
  const int q = pos >> 5, sh = pos & 31;
  // m << sh as three 32-bit pieces at limbs q, q+1, q+2
  const uint32_t w0 = (uint32_t)(m << sh);
  const uint32_t w1 = sh ? (uint32_t)(m >> (32 - sh)) : (uint32_t)(m >> 32);
  const uint32_t w2 = sh ? (uint32_t)(m >> (64 - sh)) : 0u;
  const bool neg = (bits >> 63) != 0;
  int64_t carry = 0;
#pragma unroll
  for (int i = 0; i < kAccLimbs; ++i) {
    const uint32_t piece = (i == q) ? w0 : (i == q + 1) ? w1 : (i == q + 2) ? w2 : 0u;
    int64_t t = (int64_t)a.l[i] + (neg ? -(int64_t)piece : (int64_t)piece) + carry;
    a.l[i] = (uint32_t)t;
    carry = t >> 32;  // arithmetic shift: -1, 0 or 1
  }
}

// a += b (two's complement, exact).
__device__ __forceinline__ void acc_merge(ExactAcc& a, const ExactAcc& b) {
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < kAccLimbs; ++i) {
    uint64_t t = (uint64_t)a.l[i] + (uint64_t)b.l[i] + carry;
    a.l[i] = (uint32_t)t;
    carry = t >> 32;
  }
}

__device__ __forceinline__ int acc_sign(const ExactAcc& a) {
  if ((int32_t)a.l[kAccLimbs - 1] < 0) return -1;
  uint32_t any = 0;
#pragma unroll
  for (int i = 0; i < kAccLimbs; ++i) any |= a.l[i];
  return any ? 1 : 0;
}

// Value of the accumulator as a double (relative error below 2^-52).
__device__ __forceinline__ double acc_value(const ExactAcc& a) {
  ExactAcc m = a;
  const int s = acc_sign(a);
  if (s == 0) return 0.0;
  if (s < 0) {
    uint64_t carry = 1;
#pragma unroll
    for (int i = 0; i < kAccLimbs; ++i) {
      uint64_t t = (uint64_t)(~m.l[i]) + carry;
      m.l[i] = (uint32_t)t;
      carry = t >> 32;
    }
  }
  double v = 0.0;
  int found = 0;
#pragma unroll
  for (int i = kAccLimbs - 1; i >= 0; --i) {
    // take the top nonzero limb and the two below it
    if (m.l[i] != 0u && found == 0) found = 3;
    if (found > 0) {
      v += ldexp((double)m.l[i], 32 * i - kAccLsbShift);
      --found;
    }
  }
  return s < 0 ? -v : v;
}

struct ExactResult {
  int sign;      // -1, 0, +1: sign of the exact z
  double value;  // z to float64 accuracy
};

// Whole-wave exact evaluation of z = b + sum_k x[k] * w[k] for rows of K
// elements (K a multiple of the 16-byte chunk width).  Every lane of the wave
// must call it with the same arguments; every lane gets the same result.
template <typename T>
__device__ ExactResult exact_gate_value(const T* __restrict__ xrow, const T* __restrict__ wrow,
                                        float b, int K) {
  constexpr int E = Elt<T>::kPerChunk;
  const int lane = lane_id();
  const int nch = K / E;
  double s = 0.0, a = 0.0;
  for (int c = lane; c < nch; c += kWave) {
    float xf[E], wf[E];
    Elt<T>::unpack(ldg16(xrow + (size_t)c * E), xf);
    Elt<T>::unpack(ldg16(wrow + (size_t)c * E), wf);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double p = (double)xf[e] * (double)wf[e];
      s += p;
      a += fabs(p);
    }
  }
  s = wave_sum(s);
  a = wave_sum(a);
  s += (double)b;
  a += fabs((double)b);
  const int n_lane = ((nch + kWave - 1) / kWave) * E;
  const double bound = 2.0 * (double)(n_lane + 8) * 0x1p-53 * a;
  if (fabs(s) > bound) return ExactResult{s > 0.0 ? 1 : -1, s};

  // stage 2: exact fixed-point accumulation
  ExactAcc acc;
  acc_zero(acc);
  for (int c = lane; c < nch; c += kWave) {
    float xf[E], wf[E];
    Elt<T>::unpack(ldg16(xrow + (size_t)c * E), xf);
    Elt<T>::unpack(ldg16(wrow + (size_t)c * E), wf);
#pragma unroll
    for (int e = 0; e < E; ++e) acc_add(acc, (double)xf[e] * (double)wf[e]);
  }
  if (lane == 0) acc_add(acc, (double)b);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    ExactAcc other;
#pragma unroll
    for (int i = 0; i < kAccLimbs; ++i) other.l[i] = (uint32_t)__shfl_xor((int)acc.l[i], o, kWave);
    acc_merge(acc, other);
  }
  return ExactResult{acc_sign(acc), acc_value(acc)};
}

}  // namespace sffn
