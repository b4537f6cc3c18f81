// Dense gated FFN for few tokens (M <= 32, e.g. decode): the speed-up
// reference at that shape is a stream of the three weight matrices, so each
// projection is split along K over many workgroups (like the few-token gate
// kernels) and the partial tiles are summed by a second kernel.
//
//   gate+up  skinny_gateup_partial: workgroup = (64-column tile, K split);
//            four waves take consecutive quarters of the split's K steps
//            and load their wg_t and wu_t fragments (and x) straight into
//            MFMA operand registers, all steps at once; the waves' tiles are
//            summed in LDS and written as a float32 partial.
//            skinny_gateup_epilogue sums the partials in split order and
//            writes h = ReLU(z + b) * u rounded to bf16.
//   down     skinny_down_partial: workgroup = (128-column tile, K split).
//            wd is [d_ff, d_model] (K-major for this product): each wave
//            streams its K rows of the tile through a private double buffer
//            in LDS (buffer loads straight into LDS, 256 contiguous bytes per
//            row) and reads the B fragments with the transposing LDS read;
//            h fragments come straight from global memory.
//            skinny_down_epilogue sums the partials and writes y (bf16).
// Deterministic: every sum is in a fixed order.
#include "common.cuh"
#include "gemm_v2.cuh"
#include "launch.h"

namespace sffn {

namespace {

constexpr int kSkMF = 2;      // row fragments: M <= 32
constexpr int kSkSteps = 4;   // gate+up: max K steps (of 32) per wave, all loads in flight
constexpr int kSkWgs = 512;   // target workgroups per projection

struct SkArgs {
  const uint16_t* a;   // [M, K]
  const uint16_t* b0;  // gate+up: wg_t [N, K]; down: wd [K, N]
  const uint16_t* b1;  // gate+up: wu_t [N, K]
  const float* bias;   // gate bias [N] or null
  uint16_t* out;       // h [M, N] or y [M, N]
  float* partial;
  int M, K, N, S;
};

// ---------------------------------------------------------------- gate + up
constexpr int kGuFN = 4;                          // 64 columns per B matrix
constexpr int kGuFrags = 2 * kSkMF * kGuFN;       // fragments per partial
constexpr int kGuPart = kGuFrags * 256;           // floats per partial

__global__ __launch_bounds__(256) void skinny_gateup_partial(SkArgs a) {
  constexpr int MF = kSkMF, FN = kGuFN, ST = kSkSteps;
  __shared__ f32x4_t red[2][kGuFrags][64];
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  const int kt = (int)blockIdx.x / a.S;
  const int s = (int)blockIdx.x - kt * a.S;
  const int n0 = kt * 64;
  const int nk = a.K / 32;
  const int sp = s * 4 + w, nsp = a.S * 4;
  const int k_lo = (int)(((long)sp * nk) / nsp);
  const int nst = (int)(((long)(sp + 1) * nk) / nsp) - k_lo;  // <= ST
  const int r = lane & 15, g = lane >> 4;
  const uint32_t ld = (uint32_t)a.K * 2u;
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(a.b0 + (size_t)n0 * a.K, 64u * ld);
  const __amdgpu_buffer_rsrc_t rb1 = make_rsrc(a.b1 + (size_t)n0 * a.K, 64u * ld);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.a, (uint32_t)a.M * ld);
  const uint32_t vb = (uint32_t)r * ld + (uint32_t)k_lo * 64u + 16u * g;
  uint32_t va[MF];
#pragma unroll
  for (int fm = 0; fm < MF; ++fm) {
    // rows past M read row 0: those output rows are never written
    const int row = 16 * fm + r;
    va[fm] = (uint32_t)(row < a.M ? row : 0) * ld + (uint32_t)k_lo * 64u + 16u * g;
  }
  u32x4_t bf[ST][2][FN], af[ST][MF];
#pragma unroll
  for (int i = 0; i < ST; ++i) {
    if (i < nst) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int so = (int)(fn * 16 * ld + (uint32_t)i * 64u);
        bf[i][0][fn] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb0, vb, so, 0));
        bf[i][1][fn] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb1, vb, so, 0));
      }
#pragma unroll
      for (int fm = 0; fm < MF; ++fm)
        af[i][fm] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, va[fm], i * 64, 0));
    }
  }
  f32x4_t acc[2][MF][FN];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[b][fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < ST; ++i)
    if (i < nst)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int fm = 0; fm < MF; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[b][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, af[i][fm]), __builtin_bit_cast(bf16x8_t, bf[i][b][fn]),
                acc[b][fm][fn], 0, 0, 0);
  // (w0 + w2) + (w1 + w3)
  if (w >= 2) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int fm = 0; fm < MF; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) red[w - 2][(b * MF + fm) * FN + fn][lane] = acc[b][fm][fn];
  }
  __syncthreads();
  if (w < 2) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int fm = 0; fm < MF; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[b][fm][fn] += red[w][(b * MF + fm) * FN + fn][lane];
  }
  __syncthreads();
  if (w == 1) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int fm = 0; fm < MF; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) red[0][(b * MF + fm) * FN + fn][lane] = acc[b][fm][fn];
  }
  __syncthreads();
  if (w != 0) return;
  float* mine = a.partial + ((size_t)kt * a.S + s) * kGuPart;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int f = (b * MF + fm) * FN + fn;
        *(f32x4_t*)(mine + (size_t)(f * 64 + lane) * 4) = acc[b][fm][fn] + red[0][f][lane];
      }
}

// Sum of the S partials of one float4 entry, in split order, eight splits'
// loads in flight at a time.
__device__ __forceinline__ f32x4_t sum_splits(const float* p, size_t stride, int S) {
  f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4_t ld[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) ld[u] = *(const f32x4_t*)(p + (size_t)(s0 + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) v += ld[u];
  }
  return v;
}

// Workgroup = (64-column tile, 256 of its (fm, fn, lane) entries); a thread
// sums its z and u entries over the splits.
__global__ __launch_bounds__(256) void skinny_gateup_epilogue(SkArgs a) {
  constexpr int MF = kSkMF, FN = kGuFN;
  constexpr int PER_TILE = MF * FN * 64 / 256;  // workgroups per tile
  const int kt = (int)blockIdx.x / PER_TILE;
  const int q = ((int)blockIdx.x - kt * PER_TILE) * 256 + (int)threadIdx.x;  // (fm * FN + fn) * 64 + lane
  const int n0 = kt * 64;
  const float* part0 = a.partial + (size_t)kt * a.S * kGuPart;
  const int fl = q & 63, ff = q >> 6;
  const int fm = ff / FN, fn = ff - fm * FN;
  const f32x4_t z = sum_splits(part0 + (size_t)((0 * MF * FN + ff) * 64 + fl) * 4, kGuPart, a.S);
  const f32x4_t u = sum_splits(part0 + (size_t)((1 * MF * FN + ff) * 64 + fl) * 4, kGuPart, a.S);
  const int col = n0 + 16 * fn + (fl & 15);
  const float bb = a.bias ? a.bias[col] : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * fm + 4 * (fl >> 4) + i;
    if (row < a.M) {
      const float zz = z[i] + bb;
      a.out[(size_t)row * a.N + col] = f32_to_bf16(zz > 0.f ? zz * u[i] : 0.f);
    }
  }
}

// ---------------------------------------------------------------- down
constexpr int kDnFN = 8;                       // 128 columns
constexpr int kDnFrags = kSkMF * kDnFN;
constexpr int kDnPart = kDnFrags * 256;
constexpr int kDnRowB = 256;                   // bytes per staged k row (128 columns)
constexpr int kDnStepB = 32 * kDnRowB;         // 8 KB per K step
// chunk swizzle of a staged row: no bank conflicts for the transposing reads
__device__ __forceinline__ int dn_slot(int k, int q) { return q ^ (2 * ((k & 3) | ((k >> 1) & 4))); }

__global__ __launch_bounds__(256) void skinny_down_partial(SkArgs a) {
  constexpr int MF = kSkMF, FN = kDnFN;
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * 2 * kDnStepB];  // 64 KB
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  const int kt = (int)blockIdx.x / a.S;
  const int s = (int)blockIdx.x - kt * a.S;
  const int n0 = kt * 128;
  const int nk = a.K / 32;
  const int sp = s * 4 + w, nsp = a.S * 4;
  const int k_lo = (int)(((long)sp * nk) / nsp);
  const int nst = (int)(((long)(sp + 1) * nk) / nsp) - k_lo;
  const int r = lane & 15, g = lane >> 4;
  uint8_t* buf = lds + w * 2 * kDnStepB;
  // B: rows k of wd, 128 columns from n0: 4 rows per 1 KB load block, lane l
  // fetches chunk dn_slot(k, l & 15) of row 4 blk + (l >> 4) into LDS chunk l & 15
  const uint32_t bld = (uint32_t)a.N * 2u;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.b0 + n0, (uint32_t)((size_t)a.K * a.N * 2 - (size_t)n0 * 2));
  uint32_t vbo[8];
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    const int kk = 4 * blk + (lane >> 4);
    vbo[blk] = (uint32_t)kk * bld + (uint32_t)dn_slot(kk, lane & 15) * 16u;
  }
  auto issue = [&](int st, uint8_t* dst) {  // K step st of this wave into dst
    const int soff = (k_lo + st) * 32 * (int)bld;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(dst + blk * 1024), 16, vbo[blk],
                                               soff, 0, 0);
  };
  const uint32_t ald = (uint32_t)a.K * 2u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.a, (uint32_t)a.M * ald);
  uint32_t va[MF];
#pragma unroll
  for (int fm = 0; fm < MF; ++fm) {
    const int row = 16 * fm + r;
    va[fm] = (uint32_t)(row < a.M ? row : 0) * ald + (uint32_t)k_lo * 64u + 16u * g;
  }
  f32x4_t acc[MF][FN];
#pragma unroll
  for (int fm = 0; fm < MF; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (nst > 0) issue(0, buf);
  for (int st = 0; st < nst; ++st) {
    u32x4_t af[MF];
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
      af[fm] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, va[fm], st * 64, 0));
    if (st + 1 < nst) {
      issue(st + 1, buf + ((st + 1) & 1) * kDnStepB);
      __builtin_amdgcn_s_waitcnt(Gemm2<1, 128, false>::vmcnt_imm<8 + MF>());  // step st landed
    } else {
      __builtin_amdgcn_s_waitcnt(Gemm2<1, 128, false>::vmcnt_imm<0>());
    }
    const uint8_t* bst = buf + (st & 1) * kDnStepB;
    u32x4_t bfr[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      // lane (g, i): 4 consecutive k of column 16 fn + 4 (i & 3) + j per read
      const int i = lane & 15;
      const int nl = fn * 16 + 4 * (i & 3);
      const int k1 = 8 * g + (i >> 2), k2 = k1 + 4;
      const uint8_t* p1 = bst + k1 * kDnRowB + dn_slot(k1, nl >> 3) * 16 + (nl & 7) * 2;
      const uint8_t* p2 = bst + k2 * kDnRowB + dn_slot(k2, nl >> 3) * 16 + (nl & 7) * 2;
      typedef short s16x4_t __attribute__((ext_vector_type(4)));
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(lds_void_t*)p1);
      const s16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(lds_void_t*)p2);
      bfr[fn] = u32x4_t{(uint32_t)(uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16),
                        (uint32_t)(uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16),
                        (uint32_t)(uint16_t)v2[0] | ((uint32_t)(uint16_t)v2[1] << 16),
                        (uint32_t)(uint16_t)v2[2] | ((uint32_t)(uint16_t)v2[3] << 16)};
    }
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, af[fm]), __builtin_bit_cast(bf16x8_t, bfr[fn]),
            acc[fm][fn], 0, 0, 0);
    // this wave's reads of the buffer are done before it is refilled
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  }
  // (w0 + w2) + (w1 + w3), through the (now free) LDS
  __syncthreads();
  f32x4_t* red = (f32x4_t*)lds;  // [2][kDnFrags][64]
  if (w >= 2) {
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) red[((w - 2) * kDnFrags + fm * FN + fn) * 64 + lane] = acc[fm][fn];
  }
  __syncthreads();
  if (w < 2) {
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] += red[(w * kDnFrags + fm * FN + fn) * 64 + lane];
  }
  __syncthreads();
  if (w == 1) {
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) red[(fm * FN + fn) * 64 + lane] = acc[fm][fn];
  }
  __syncthreads();
  if (w != 0) return;
  float* mine = a.partial + ((size_t)kt * a.S + s) * kDnPart;
#pragma unroll
  for (int fm = 0; fm < MF; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int f = fm * FN + fn;
      *(f32x4_t*)(mine + (size_t)(f * 64 + lane) * 4) = acc[fm][fn] + red[f * 64 + lane];
    }
}

// Workgroup = (128-column tile, 256 of its (fm, fn, lane) entries).
__global__ __launch_bounds__(256) void skinny_down_epilogue(SkArgs a) {
  constexpr int FN = kDnFN;
  constexpr int PER_TILE = kSkMF * FN * 64 / 256;
  const int kt = (int)blockIdx.x / PER_TILE;
  const int q = ((int)blockIdx.x - kt * PER_TILE) * 256 + (int)threadIdx.x;  // (fm * FN + fn) * 64 + lane
  const int n0 = kt * 128;
  const int fl = q & 63, ff = q >> 6;
  const int fm = ff / FN, fn = ff - fm * FN;
  const f32x4_t v = sum_splits(a.partial + (size_t)kt * a.S * kDnPart + (size_t)q * 4, kDnPart, a.S);
  const int col = n0 + 16 * fn + (fl & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * fm + 4 * (fl >> 4) + i;
    if (row < a.M) a.out[(size_t)row * a.N + col] = f32_to_bf16(v[i]);
  }
}

int gateup_splits(int K, int N) {
  const int nt = N / 64, nk = K / 32;
  const int s_min = (nk + 4 * kSkSteps - 1) / (4 * kSkSteps);
  int S = max(kSkWgs / nt, s_min);
  return max(1, min(S, max(1, nk / 4)));
}

int down_splits(int K, int N) {
  const int nt = N / 128, nk = K / 32;
  int S = kSkWgs / nt;
  return max(1, min(S, max(1, nk / 4)));
}

}  // namespace

bool dense_skinny_ok(int dtype, int M, int d_model, int d_ff) {
  return dtype == 1 && M >= 1 && M <= 16 * kSkMF && d_model % 128 == 0 && d_ff % 128 == 0;
}

size_t dense_skinny_partial_bytes(int d_model, int d_ff) {
  const size_t gu = (size_t)(d_ff / 64) * gateup_splits(d_model, d_ff) * kGuPart * 4;
  const size_t dn = (size_t)(d_model / 128) * down_splits(d_ff, d_model) * kDnPart * 4;
  return gu > dn ? gu : dn;
}

hipError_t launch_dense_skinny(const void* x, const void* wg_t, const float* b_g, const void* wu_t,
                               const void* wd, void* h, float* partial, void* y, int M,
                               int d_model, int d_ff, hipStream_t stream) {
  SkArgs g{(const uint16_t*)x, (const uint16_t*)wg_t, (const uint16_t*)wu_t, b_g, (uint16_t*)h,
           partial, M, d_model, d_ff, gateup_splits(d_model, d_ff)};
  hipLaunchKernelGGL(skinny_gateup_partial, dim3((unsigned)((d_ff / 64) * g.S)), dim3(256), 0,
                     stream, g);
  hipLaunchKernelGGL(skinny_gateup_epilogue, dim3((unsigned)((d_ff / 64) * (kSkMF * kGuFN * 64 / 256))),
                     dim3(256), 0, stream, g);
  SkArgs d{(const uint16_t*)h, (const uint16_t*)wd, nullptr, nullptr, (uint16_t*)y, partial, M,
           d_ff, d_model, down_splits(d_ff, d_model)};
  hipLaunchKernelGGL(skinny_down_partial, dim3((unsigned)((d_model / 128) * d.S)), dim3(256), 0,
                     stream, d);
  hipLaunchKernelGGL(skinny_down_epilogue, dim3((unsigned)((d_model / 128) * (kSkMF * kDnFN * 64 / 256))),
                     dim3(256), 0, stream, d);
  return hipGetLastError();
}

}  // namespace sffn
