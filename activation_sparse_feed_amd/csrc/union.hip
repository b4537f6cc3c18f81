// Fused up(.)gate -> down with the column union of a token block staged in
// LDS: the organisation of the pages' fused kernel (pwwt.cn article, section
// 02: the active columns that the tokens of a block share are fetched once per
// block and reused from shared memory), built beside the row walk of
// sparse.hip so that the two can be measured on the same TwELL.
//
// Workgroup = WAVES consecutive tokens, one wavefront per token holding x_t
// (bf16, 16-byte chunks) and the float32 y_t in registers, as in the row walk.
// The workgroup walks the column tiles in order; per tile k:
//   1. every wave lists its row's live entries of the tile (j, val) in LDS and
//      sets bit j - 128k of the tile's 128-bit union mask;
//   2. the union columns are numbered in ascending order (prefix popcounts of
//      the mask) and staged UC at a time: the wu_t row and the wd row of each
//      union column are read from global memory ONCE for the whole block, with
//      16-byte loads spread over all lanes of the workgroup, into LDS;
//   3. every wave computes, for its entries whose column is staged,
//        u = x_t . wu_t[j]          (packed bf16 dot2 on the LDS row, DPP sum)
//        y_t += (val * u) * wd[j]   (float32 FMA on the LDS row)
//      and the workgroup meets at a barrier before the next chunk is staged.
// The sums run in the same order as the row walk's per-entry order (ascending
// column within the tile, tiles in order) but with a float32 FMA for the down
// projection, so y agrees with sparse_ffn_fwd to rounding, not bit for bit.
// Rows with any count above cap are skipped (the hybrid route owns them); they
// take part in the barriers only.
#include "common.cuh"
#include "launch.h"

namespace sffn {

namespace {

constexpr int kUnionLdsBytes = 128 * 1024;  // staged wu_t and wd rows per chunk
constexpr int kUnionMaxCap = 32;             // entries a wave lists per tile

struct UnionArgs {
  const uint16_t* x;
  const uint16_t* wu;
  const uint16_t* wd;
  const uint16_t* count;
  const uint16_t* idx;
  const uint16_t* val;
  uint16_t* y;
  int T, nt, cap;
};

// Number of set bits of the 128-bit mask m[0..3] below bit c (0 <= c < 128).
__device__ __forceinline__ int bits_below(const uint32_t* m, int c) {
  const int w = c >> 5;
  int n = __popc(m[w] & ((1u << (c & 31)) - 1u));
  for (int i = 0; i < w; ++i) n += __popc(m[i]);
  return n;
}

template <int NCH, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void sparse_updown_union(UnionArgs a) {
  constexpr int E = 8;                    // bf16 per 16-byte chunk
  constexpr int K = NCH * 64 * E;         // d_model
  constexpr int RC = K / E;               // 16-byte chunks per row
  constexpr int UC = kUnionLdsBytes / (4 * K);  // union columns per staged chunk
  constexpr int NTHR = WAVES * 64;
  constexpr int PER = (UC * 2 * RC + NTHR - 1) / NTHR;  // staging loads per thread
  static_assert(UC >= 1 && UC <= 128, "staged chunk");
  __shared__ u32x4_t rows[UC * 2 * RC];  // [UC][wu_t row, wd row][RC]
  __shared__ uint16_t list_j[WAVES][kUnionMaxCap];
  __shared__ float list_h[WAVES][kUnionMaxCap];
  __shared__ uint32_t mask[2][4];
  __shared__ uint8_t ucol[128];

  const int tid = (int)threadIdx.x;
  const int lane = lane_id();
  const int w = tid >> 6;
  const int t = uniform((int)(blockIdx.x * WAVES + w));
  bool active = t < a.T;
  const uint16_t* cnt_row = a.count + (size_t)(active ? t : 0) * a.nt;
  if (active) {
    bool over = false;
    for (int k = lane; k < a.nt; k += kWave) over |= (int)cnt_row[k] > a.cap;
    active = __ballot(over) == 0ull;
  }
  u32x4_t xr[NCH];
  float yv[NCH][E];
  const uint16_t* xrow = a.x + (size_t)(active ? t : 0) * K;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    xr[c] = active ? ldg16(xrow + (size_t)(lane + kWave * c) * E) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < E; ++e) yv[c][e] = 0.f;
  }
  if (tid < 8) mask[tid >> 2][tid & 3] = 0u;
  __syncthreads();

  const int cap = a.cap;
  for (int k = 0; k < a.nt; ++k) {
    uint32_t* mk = mask[k & 1];
    // 1. this row's live entries of tile k, and the tile's union mask
    // (an index outside the tile, never written by twell_pack, is listed as
    // 0xffff and skipped)
    int n = 0;
    if (active) {
      n = min((int)cnt_row[k], cap);
      if (lane < n) {
        const size_t off = ((size_t)t * a.nt + k) * cap + lane;
        const int c = (int)a.idx[off] - 128 * k;
        const bool live = c >= 0 && c < 128;
        list_j[w][lane] = live ? (uint16_t)c : (uint16_t)0xffff;
        list_h[w][lane] = bf16_to_f32(a.val[off]);
        if (live) atomicOr(&mk[c >> 5], 1u << (c & 31));
      }
    }
    __syncthreads();
    // 2. union columns in ascending order; the other mask is cleared for tile k + 1
    uint32_t m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = mk[i];
    const int n_union = __popc(m[0]) + __popc(m[1]) + __popc(m[2]) + __popc(m[3]);
    if (tid < 128 && ((m[tid >> 5] >> (tid & 31)) & 1u)) ucol[bits_below(m, tid)] = (uint8_t)tid;
    if (tid >= 128 && tid < 132) mask[(k + 1) & 1][tid - 128] = 0u;
    __syncthreads();  // also ends the tile when nothing is staged
    if (n_union == 0) continue;  // uniform: nobody of the block is active in tile k
    for (int u0 = 0; u0 < n_union; u0 += UC) {
      const int nu = min(UC, n_union - u0);
      // stage the wu_t and wd rows of union columns u0 .. u0 + nu, all loads in flight
      u32x4_t st[PER];
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int q = tid + p * NTHR;
        const int s = q / (2 * RC);
        const int r = q - s * 2 * RC;
        if (s < nu) {
          const int j = 128 * k + (int)ucol[u0 + s];
          const uint16_t* src = (r < RC ? a.wu : a.wd) + (size_t)j * K;
          st[p] = ldg16(src + (size_t)(r < RC ? r : r - RC) * E);
        }
      }
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int q = tid + p * NTHR;
        if (q / (2 * RC) < nu) rows[q] = st[p];
      }
      __syncthreads();
      // 3. this wave's entries whose column is staged
      for (int e = 0; e < n; ++e) {
        const int c = (int)list_j[w][e];
        if (c >= 128) continue;
        const int s = bits_below(m, c) - u0;
        if (s < 0 || s >= nu) continue;  // uniform across the wave
        const u32x4_t* ru = rows + (size_t)s * 2 * RC;
        const u32x4_t* rd = ru + RC;
        float p = 0.f;
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
          const u32x4_t ur = ru[lane + kWave * cc];
          p = dot2_bf16(xr[cc].x, ur.x, p);
          p = dot2_bf16(xr[cc].y, ur.y, p);
          p = dot2_bf16(xr[cc].z, ur.z, p);
          p = dot2_bf16(xr[cc].w, ur.w, p);
        }
        const float g = list_h[w][e] * wave_sum_uniform(p);
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
          float f[E];
          Elt<uint16_t>::unpack(rd[lane + kWave * cc], f);
#pragma unroll
          for (int q = 0; q < E; ++q) yv[cc][q] = fmaf(g, f[q], yv[cc][q]);
        }
      }
      __syncthreads();
    }
  }
  if (!active) return;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    u32x4_t o;
    o.x = (uint32_t)f32_to_bf16(yv[c][0]) | ((uint32_t)f32_to_bf16(yv[c][1]) << 16);
    o.y = (uint32_t)f32_to_bf16(yv[c][2]) | ((uint32_t)f32_to_bf16(yv[c][3]) << 16);
    o.z = (uint32_t)f32_to_bf16(yv[c][4]) | ((uint32_t)f32_to_bf16(yv[c][5]) << 16);
    o.w = (uint32_t)f32_to_bf16(yv[c][6]) | ((uint32_t)f32_to_bf16(yv[c][7]) << 16);
    *(u32x4_t*)(a.y + (size_t)t * K + (size_t)(lane + kWave * c) * E) = o;
  }
}

template <int NCH, int WAVES>
hipError_t launch_union(const UnionArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.T + WAVES - 1) / WAVES)), block(WAVES * 64);
  hipLaunchKernelGGL((sparse_updown_union<NCH, WAVES>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool union_supported(int dtype, int d_model, int cap) {
  return dtype == 1 && cap <= kUnionMaxCap &&
         (d_model == 512 || d_model == 1024 || d_model == 2048 || d_model == 4096);
}

hipError_t launch_sparse_union(const void* x, const void* wu_t, const void* wd,
                               const uint16_t* count, const uint16_t* idx, const void* val,
                               void* y, int T, int K, int n_tiles, int cap, hipStream_t stream) {
  const UnionArgs a{(const uint16_t*)x, (const uint16_t*)wu_t, (const uint16_t*)wd, count, idx,
                    (const uint16_t*)val, (uint16_t*)y, T, n_tiles, cap};
  switch (K) {
    case 512: return launch_union<1, 16>(a, stream);
    case 1024: return launch_union<2, 16>(a, stream);
    case 2048: return launch_union<4, 16>(a, stream);
    case 4096: return launch_union<8, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sffn
