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
//            to 2^16 of them without rounding or overflow.  One such integer
//            per lane lives in LDS (the stage is rare; keeping it out of
//            registers leaves the caller's register budget alone), and the
//            lanes' integers are summed by a tree over the wave.
#pragma once

#include "common.cuh"

namespace sffn {

constexpr int kAccLimbs = 20;      // 20 x 32 bits
constexpr int kAccLsbShift = 352;  // bit 0 weighs 2^-352
// LDS words the exact stage needs per wave: one 640-bit accumulator per lane,
// limb i of lane l at word i * 64 + l.
constexpr int kExactLdsWords = kAccLimbs * 64;

// acc += p exactly (acc: this lane's limbs in LDS, stride 64 words).
// p must be 0 or have magnitude in [2^-350, 2^270).
__device__ __forceinline__ void acc_add(uint32_t* acc, double p) {
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
  for (int i = 0; i < kAccLimbs; ++i) {
    const uint32_t piece = (i == q) ? w0 : (i == q + 1) ? w1 : (i == q + 2) ? w2 : 0u;
    const int64_t t = (int64_t)acc[i * 64] + (neg ? -(int64_t)piece : (int64_t)piece) + carry;
    acc[i * 64] = (uint32_t)t;
    carry = t >> 32;  // arithmetic shift: -1, 0 or 1
  }
}

// dst += src (two's complement, exact).
__device__ __forceinline__ void acc_merge(uint32_t* dst, const uint32_t* src) {
  uint64_t carry = 0;
  for (int i = 0; i < kAccLimbs; ++i) {
    const uint64_t t = (uint64_t)dst[i * 64] + (uint64_t)src[i * 64] + carry;
    dst[i * 64] = (uint32_t)t;
    carry = t >> 32;
  }
}

__device__ __forceinline__ int acc_sign(const uint32_t* acc) {
  if ((int32_t)acc[(kAccLimbs - 1) * 64] < 0) return -1;
  uint32_t any = 0;
  for (int i = 0; i < kAccLimbs; ++i) any |= acc[i * 64];
  return any ? 1 : 0;
}

// Value of an accumulator as a double (relative error below 2^-52).
__device__ __forceinline__ double acc_value(const uint32_t* acc) {
  const int s = acc_sign(acc);
  if (s == 0) return 0.0;
  // magnitude limbs, most significant first; the top three nonzero ones suffice
  uint32_t borrow_chain = s < 0 ? 1u : 0u;  // two's complement negation: ~a + 1
  uint32_t mag[kAccLimbs];
  uint64_t carry = borrow_chain;
  for (int i = 0; i < kAccLimbs; ++i) {
    const uint32_t w = s < 0 ? ~acc[i * 64] : acc[i * 64];
    const uint64_t t = (uint64_t)w + carry;
    mag[i] = (uint32_t)t;
    carry = s < 0 ? (t >> 32) : 0u;
  }
  double v = 0.0;
  int found = 0;
  for (int i = kAccLimbs - 1; i >= 0; --i) {
    if (mag[i] != 0u && found == 0) found = 3;
    if (found > 0) {
      v += ldexp((double)mag[i], 32 * i - kAccLsbShift);
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
// must call it with the same arguments and gets the same result.  lds_acc:
// kExactLdsWords words of LDS owned by this wave (used by stage 2 only).
// U: 16-byte chunks per lane whose loads are issued together (more U, fewer
// round trips to memory, more registers).
template <typename T, int U = 2>
__device__ ExactResult exact_gate_value(const T* __restrict__ xrow, const T* __restrict__ wrow,
                                        float b, int K, uint32_t* lds_acc) {
  constexpr int E = Elt<T>::kPerChunk;
  const int lane = lane_id();
  const int nch = K / E;
  double s = 0.0, a = 0.0;
  for (int base = 0; base < nch; base += kWave * U) {
    u32x4_t xc[U], wc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + lane + kWave * u;
      const bool ok = c < nch;
      xc[u] = ok ? ldg16(xrow + (size_t)c * E) : u32x4_t{0u, 0u, 0u, 0u};
      wc[u] = ok ? ldg16(wrow + (size_t)c * E) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xf[E], wf[E];
      Elt<T>::unpack(xc[u], xf);
      Elt<T>::unpack(wc[u], wf);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const double p = (double)xf[e] * (double)wf[e];  // exact, zero for padding
        s += p;
        a += fabs(p);
      }
    }
  }
  s = wave_sum(s);
  a = wave_sum(a);
  s += (double)b;
  a += fabs((double)b);
  const int n_lane = ((nch + kWave * U - 1) / (kWave * U)) * U * E;  // terms per lane, padding included
  const double bound = 2.0 * (double)(n_lane + 8) * 0x1p-53 * a;
  if (fabs(s) > bound) return ExactResult{s > 0.0 ? 1 : -1, s};

  // stage 2: exact fixed-point accumulation in LDS, then a tree over lanes
  uint32_t* mine = lds_acc + lane;
  for (int i = 0; i < kAccLimbs; ++i) mine[i * 64] = 0u;
  for (int c = lane; c < nch; c += kWave) {
    float xf[E], wf[E];
    Elt<T>::unpack(ldg16(xrow + (size_t)c * E), xf);
    Elt<T>::unpack(ldg16(wrow + (size_t)c * E), wf);
    for (int e = 0; e < E; ++e) acc_add(mine, (double)xf[e] * (double)wf[e]);
  }
  if (lane == 0) acc_add(mine, (double)b);
  for (int o = 32; o >= 1; o >>= 1) {
    __builtin_amdgcn_wave_barrier();
    if (lane < o) acc_merge(mine, lds_acc + lane + o);
  }
  __builtin_amdgcn_wave_barrier();
  return ExactResult{acc_sign(lds_acc), acc_value(lds_acc)};
}

}  // namespace sffn
