// GEMM main loops of the gate, dense gate+up and down kernels (gfx950).
//
// bf16: 128 x (NB * BNW) workgroup tile, 4 waves in a 2 x 2 grid, BK = 64,
// operands staged through double-buffered LDS, v_mfma_f32_16x16x32_bf16 with
// float32 accumulators.  Rows are K-contiguous in LDS (16-byte chunks XOR-
// swizzled by row so that the 16-byte fragment reads are conflict free).
//
// float32: plain FMA tiles (used by the float32 workloads), BK = 16.
#pragma once

#include "common.cuh"

namespace sffn {

// ------------------------------------------------------------------ bf16 MFMA
// LDS offset (in bf16 elements) of 16-byte chunk q of row r in a K-contiguous
// tile with 8 chunks (64 elements) per row.
__device__ __forceinline__ int lds_off(int r, int q) { return r * 64 + ((q ^ (r & 7)) << 3); }

// MFMA 16x16x32 bf16 lane layout: lane l feeds row/column (l & 15) with the
// eight K values [8 * (l >> 4), 8 * (l >> 4) + 8); it receives output column
// (l & 15), rows 4 * (l >> 4) + {0, 1, 2, 3}.

// A operand: rows of a [M, K] matrix (optionally gathered through a row map).
// B operands, B_KN == false: NB matrices [N, K] (K-contiguous), BNW rows each.
//             B_KN == true : one matrix [K, N] (N-contiguous); the loader
//             transposes it into the same K-contiguous LDS layout.
template <int NB, int BNW, bool NORMS, bool B_KN = false>
struct MfmaGemm {
  static constexpr int BM = 128, BK = 64;
  static constexpr int A_ROWS = BM, ROWS = BM + NB * BNW;
  static constexpr int STAGE = ROWS * BK;            // bf16 elements per stage
  static constexpr int PER_THREAD = ROWS * 8 / 256;  // 16-byte chunks per thread
  static constexpr int A_PER_THREAD = A_ROWS * 8 / 256;
  static constexpr int B_PER_THREAD = PER_THREAD - A_PER_THREAD;
  static constexpr int WN = BNW / 2;                 // per-wave columns per B matrix
  static constexpr int FM = 4, FN = WN / 16;         // 16x16 blocks per wave
  static constexpr size_t LDS_BYTES = 2 * STAGE * 2;
  static_assert(ROWS * 8 % 256 == 0, "tile rows");
  static_assert((NB * BNW * 8) % 256 == 0, "B rows");
  static_assert(!B_KN || (NB == 1 && BNW == 128), "K-major B: one 128-wide matrix");

  f32x4_t acc[NB][FM][FN];
  // per-thread sums of squares of the A and B rows it loads (guard-band norms)
  float sqa[A_PER_THREAD], sqb[B_PER_THREAD];
  const uint16_t* src[PER_THREAD];  // row pointers (nullptr = zero row)
  int b_ld, b_nvalid;               // B_KN: leading dimension, columns valid in tile
  u32x4_t stage_regs[PER_THREAD];

  __device__ __forceinline__ void init(const uint16_t* A, int lda, const int* rowmap, int m0,
                                       int m_valid, const uint16_t* const* B, int ldb, int n0,
                                       int N) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i) {
      const int r = (tid + 256 * i) >> 3;
      const int m = m0 + r;
      src[i] = nullptr;
      if (m < m_valid) src[i] = A + (size_t)(rowmap ? rowmap[m] : m) * lda;
    }
    if (!B_KN) {
#pragma unroll
      for (int i = A_PER_THREAD; i < PER_THREAD; ++i) {
        const int rb = ((tid + 256 * i) >> 3) - A_ROWS;
        const int b = rb / BNW, n = rb % BNW;
        src[i] = B[b] + (size_t)(n0 + n) * ldb;
      }
    } else {
      // two (k-pair, 8-column chunk) combos per thread: kp = c & 31, nc = c >> 5
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;
        const int nc = c >> 5;
        src[A_PER_THREAD + 2 * i] = B[0] + n0 + nc * 8;
        src[A_PER_THREAD + 2 * i + 1] = B[0] + n0 + nc * 8;
      }
      b_ld = ldb;
      b_nvalid = N - n0;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[b][fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i) sqa[i] = 0.f;
#pragma unroll
    for (int i = 0; i < B_PER_THREAD; ++i) sqb[i] = 0.f;
  }

  __device__ __forceinline__ void load(int k0, int K) {
    const int q = threadIdx.x & 7;
    const int k = k0 + q * 8;
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i)
      stage_regs[i] = (src[i] != nullptr && k < K) ? ldg16(src[i] + k) : u32x4_t{0u, 0u, 0u, 0u};
    if (!B_KN) {
#pragma unroll
      for (int i = A_PER_THREAD; i < PER_THREAD; ++i)
        stage_regs[i] = (k < K) ? ldg16(src[i] + k) : u32x4_t{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int kp = c & 31, nc = c >> 5;
        const int kr = k0 + 2 * kp;
        const bool col_ok = nc * 8 < b_nvalid;
        stage_regs[A_PER_THREAD + 2 * i] =
            (col_ok && kr < K) ? ldg16(src[A_PER_THREAD + 2 * i] + (size_t)kr * b_ld)
                               : u32x4_t{0u, 0u, 0u, 0u};
        stage_regs[A_PER_THREAD + 2 * i + 1] =
            (col_ok && kr + 1 < K) ? ldg16(src[A_PER_THREAD + 2 * i + 1] + (size_t)(kr + 1) * b_ld)
                                   : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    if (NORMS) {
#pragma unroll
      for (int i = 0; i < PER_THREAD; ++i) {
        float v[8];
        Elt<uint16_t>::unpack(stage_regs[i], v);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(v[e], v[e], s);
        if (i < A_PER_THREAD) sqa[i] += s; else sqb[i - A_PER_THREAD] += s;
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds) {
    const int q = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i) {
      const int r = (threadIdx.x + 256 * i) >> 3;
      *(u32x4_t*)(lds + lds_off(r, q)) = stage_regs[i];
    }
    if (!B_KN) {
#pragma unroll
      for (int i = A_PER_THREAD; i < PER_THREAD; ++i) {
        const int r = (threadIdx.x + 256 * i) >> 3;
        *(u32x4_t*)(lds + lds_off(r, q)) = stage_regs[i];
      }
    } else {
      // transpose: element e of rows (k, k+1) goes to B row n = nc*8 + e as one u32
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int kp = c & 31, nc = c >> 5;
        const u32x4_t lo = stage_regs[A_PER_THREAD + 2 * i];
        const u32x4_t hi = stage_regs[A_PER_THREAD + 2 * i + 1];
        const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w};
        const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a = lw[e >> 1], b = hw[e >> 1];
          const uint32_t pk = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
          const int r = A_ROWS + nc * 8 + e;
          const int kk = 2 * kp;
          *(uint32_t*)(lds + lds_off(r, kk >> 3) + (kk & 7)) = pk;
        }
      }
    }
  }

  __device__ __forceinline__ void compute(const uint16_t* lds) {
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const int wm = w & 1, wn = w >> 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int q = ks * 4 + (lane >> 4);
      bf16x8_t af[FM], bfr[NB][FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = wm * 64 + fm * 16 + (lane & 15);
        af[fm] = *(const bf16x8_t*)(lds + lds_off(r, q));
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int r = A_ROWS + b * BNW + wn * WN + fn * 16 + (lane & 15);
          bfr[b][fn] = *(const bf16x8_t*)(lds + lds_off(r, q));
        }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[b][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[b][fn],
                                                                    acc[b][fm][fn], 0, 0, 0);
    }
  }

  // Full K loop.  lds must hold LDS_BYTES.
  __device__ __forceinline__ void run(uint16_t* lds, int K) {
    const int nk = (K + BK - 1) / BK;
    load(0, K);
    store(lds);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      uint16_t* cur = lds + (kt & 1) * STAGE;
      uint16_t* nxt = lds + ((kt + 1) & 1) * STAGE;
      if (kt + 1 < nk) load((kt + 1) * BK, K);
      compute(cur);
      if (kt + 1 < nk) store(nxt);
      __syncthreads();
    }
  }

  // Row norms: reduce the per-thread partial sums over the 8 threads that
  // share a row and write sqrt to rn_a[BM], rn_b[NB*BNW] (LDS).
  __device__ __forceinline__ void write_norms(float* rn_a, float* rn_b) {
    const int q = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      float s = (i < A_PER_THREAD) ? sqa[i] : sqb[i - A_PER_THREAD];
      s += __shfl_xor(s, 1, kWave);
      s += __shfl_xor(s, 2, kWave);
      s += __shfl_xor(s, 4, kWave);
      const int r = (threadIdx.x + 256 * i) >> 3;
      if (q == 0) {
        if (i < A_PER_THREAD) rn_a[r] = sqrtf(s); else rn_b[r - A_ROWS] = sqrtf(s);
      }
    }
  }

  // Visit every accumulator element: f(b, row_in_tile, col_in_Btile, value).
  template <typename F>
  __device__ __forceinline__ void for_each(F&& f) const {
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const int wm = w & 1, wn = w >> 1;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = wm * 64 + fm * 16 + 4 * (lane >> 4) + r;
            const int col = wn * WN + fn * 16 + (lane & 15);
            f(b, row, col, acc[b][fm][fn][r]);
          }
  }
};

// ------------------------------------------------------------- float32 VALU
// 128 x (NB * BNW) tile, 256 threads as 16 x 16, each 8 rows x (BNW/16) cols
// per B matrix.  A: [M, K] K-contiguous (optionally row-mapped).  B: either
// NB matrices [N, K] K-contiguous (B_KN == false) or one matrix [K, N]
// N-contiguous (B_KN == true, used by the down projection).
template <int NB, int BNW, bool B_KN, bool NORMS>
struct ValuGemm {
  static constexpr int BM = 128, BK = 16, TM = 8, TN = BNW / 16;
  static constexpr size_t LDS_BYTES = (size_t)(BK * BM + NB * BK * BNW) * 4;
  float acc[NB][TM][TN];
  float sqa[2], sqb[2];
  const float* asrc[2];

  __device__ __forceinline__ void run(float* lds, const float* A, int lda, const int* rowmap,
                                      int m0, int m_valid, const float* const* B, int ldb, int n0,
                                      int N, int K) {
    float* As = lds;             // [BK][BM]
    float* Bs = lds + BK * BM;   // [NB][BK][BNW]
    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[b][i][j] = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (tid + 256 * i) >> 2;
      const int m = m0 + r;
      asrc[i] = (m < m_valid) ? A + (size_t)(rowmap ? rowmap[m] : m) * lda : nullptr;
      sqa[i] = 0.f;
      sqb[i] = 0.f;
    }
    for (int k0 = 0; k0 < K; k0 += BK) {
      // A tile: 128 rows x 16 k, 2 float4 per thread, stored transposed
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;
        const int r = c >> 2, kq = (c & 3) * 4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (asrc[i] != nullptr && k0 + kq < K) v = *(const float4*)(asrc[i] + k0 + kq);
        if (NORMS) sqa[i] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        As[(kq + 0) * BM + r] = v.x;
        As[(kq + 1) * BM + r] = v.y;
        As[(kq + 2) * BM + r] = v.z;
        As[(kq + 3) * BM + r] = v.w;
      }
      if (!B_KN) {
        // NB*BNW rows x 16 k; NB*BNW == 128 here: 2 float4 per thread
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int c = tid + 256 * i;
          const int rr = c >> 2, kq = (c & 3) * 4;
          const int b = rr / BNW, n = rr % BNW;
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (k0 + kq < K) v = *(const float4*)(B[b] + (size_t)(n0 + n) * ldb + k0 + kq);
          if (NORMS) sqb[i] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          float* dst = Bs + b * BK * BNW;
          dst[(kq + 0) * BNW + n] = v.x;
          dst[(kq + 1) * BNW + n] = v.y;
          dst[(kq + 2) * BNW + n] = v.z;
          dst[(kq + 3) * BNW + n] = v.w;
        }
      } else {
        // one [K, N] matrix: 16 k rows x BNW cols
        for (int c = tid; c < BK * BNW / 4; c += 256) {
          const int kk = c / (BNW / 4), nq = (c % (BNW / 4)) * 4;
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (k0 + kk < K && n0 + nq < N) v = *(const float4*)(B[0] + (size_t)(k0 + kk) * ldb + n0 + nq);
          *(float4*)(Bs + kk * BNW + nq) = v;
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[TM], bv[NB][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = As[kk * BM + ty * TM + i];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < TN; ++j) bv[b][j] = Bs[b * BK * BNW + kk * BNW + tx * TN + j];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[b][i][j] = fmaf(a[i], bv[b][j], acc[b][i][j]);
      }
      __syncthreads();
    }
  }

  __device__ __forceinline__ void write_norms(float* rn_a, float* rn_b) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float s = sqa[i];
      s += __shfl_xor(s, 1, kWave);
      s += __shfl_xor(s, 2, kWave);
      float t = sqb[i];
      t += __shfl_xor(t, 1, kWave);
      t += __shfl_xor(t, 2, kWave);
      const int r = (threadIdx.x + 256 * i) >> 2;
      if ((threadIdx.x & 3) == 0) {
        rn_a[r] = sqrtf(s);
        rn_b[r] = sqrtf(t);
      }
    }
  }

  template <typename F>
  __device__ __forceinline__ void for_each(F&& f) const {
    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) f(b, ty * TM + i, tx * TN + j, acc[b][i][j]);
  }
};

}  // namespace sffn
