// Backward of the activation-sparse gated FFN through TwELL and the hybrid
// routing (training through the format: pwwt.cn article, sections 03-04).
//
// For an upstream gradient gy = dL/dy of y = (ReLU(x wg_t^T + b) * x wu_t^T) wd,
// only the active entries (t, j) carry gradient.  Per entry, with h its TwELL
// value:
//   u  = x_t . wu_t[j],  ga = gy_t . wd[j]
//   gz = ga u + l1g,  gu = ga h,  a = h u
//     (l1g = lambda / T: the gradient of the L1 activation regulariser
//     lambda / T sum ReLU(z) on an active entry; 0 when it is not trained)
//   gx_t     += gz wg_t[j] + gu wu_t[j]
//   gwg_t[j] += gz x_t,  gwu_t[j] += gu x_t,  gwd[j] += a gy_t,  gb[j] += gz
// Rows within capacity take their entries from the forward's TwELL lists;
// routed rows (a tile over capacity) from complete activity lists rebuilt here
// (their gate recomputed with the same GEMM and the same exact activity
// decision).
//
// Kernels, in stream order:
//   bwd_prep   one wave per row: tile-major copies of the counts and live
//              indices of rows within capacity (0 for routed rows), and the
//              start of every tile in a routed row's complete list;
//   bwd_rows   one wave per row within capacity: walks the row's entries in
//              order, computes the two dot products and gz, gu, a per entry
//              (stored for the weight gradients) and accumulates gx_t in
//              registers;
//   bwd_routed_items, bwd_routed, bwd_routed_gx
//              the same for the routed rows, whose long lists are cut into up
//              to eight parts (one wave each) whose partial gx are summed in
//              part order;
//   csc_count, csc_colscan, csc_ptr, csc_fill
//              the TwELL entries regrouped by column (row order within a
//              column), deterministic;
//   bwd_cols   one wave per (column, d chunk): the column's entries from its
//              list, then the routed rows' (binary search in their lists),
//              summed into the weight-gradient rows in registers; every column
//              is written (zero when inactive).
// With d_model <= 2048 and more than kSplitMaxT tokens the order is fused
// instead: no bwd_rows; the column lists carry each entry's TwELL position and
// h, bwd_cols_fused (one wave per column over the whole d_model) computes the
// per-entry gradients itself while summing the weight gradients, and bwd_gx
// then gathers the wg_t and wu_t rows for gx.
// Every sum runs in a fixed order, so the gradients are deterministic.
#include <algorithm>

#include "common.cuh"
#include "launch.h"

namespace sffn {

namespace {

constexpr int kBTile = 128;

struct BwdArgs {
  const uint16_t* x;
  const uint16_t* wg;
  const uint16_t* wu;
  const uint16_t* wd;
  const uint16_t* gy;
  const uint16_t* count;   // forward TwELL [T, nt] (uncapped)
  const uint16_t* idx;     // [T, nt, cap]
  const uint16_t* val;     // [T, nt, cap] bf16 h
  const int32_t* routed;   // ascending routed rows
  const int32_t* n_routed;
  const uint16_t* ecount;  // routed row r: complete list length
  const uint16_t* eidx;    // [T, N] complete lists of the routed rows (row r = routed[r])
  const uint16_t* eval;    // [T, N] bf16 h
  int32_t* eoff;           // [T, nt] start of tile k in routed row r's list
  uint16_t* count_t;       // [nt, T] counts of rows within capacity, 0 for routed rows
  uint16_t* idx_t;         // [nt, T, cap] their live indices
  f32x4_t* co;             // [T, nt, cap] (gz, gu, a, 0) of the TwELL entries
  f32x4_t* co_r;           // [T, N] (gz, gu, a, 0) of the routed rows' entries
  uint16_t* gx;            // [T, D] bf16
  float* gwg;              // [N, D]
  float* gwu;              // [N, D]
  float* gwd;              // [N, D]
  float* gb;               // [N] or null
  int T, D, N, nt, cap;
  float l1g;               // lambda / T, added to gz of every active entry
  int R;                   // routed rows the workspace holds (<= T)
  int routed_dense;        // the MFMA kernels of backward_routed.hip were launched too
};

// The routed rows go to the MFMA kernels (backward_routed.hip) instead of the
// per-entry ones below: launched, and enough routed rows on the device.
__device__ __forceinline__ bool routed_on_tiles(const BwdArgs& a, int nr) {
  return a.routed_dense && nr >= kDenseRoutedRows;
}

// Position of row t in the ascending routed list (binary search), or -1.
__device__ __forceinline__ int routed_index(const int32_t* routed, int n, int t) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (routed[mid] < t) lo = mid + 1;
    else hi = mid;
  }
  return (lo < n && routed[lo] == t) ? lo : -1;
}

// Eight float32 weight-gradient values of a lane: stored, or added to what is
// there (the routed rows' part, written before by the MFMA kernels).
__device__ __forceinline__ void store_w8(float* p, const float* v, bool add) {
  f32x4_t lo = f32x4_t{v[0], v[1], v[2], v[3]}, hi = f32x4_t{v[4], v[5], v[6], v[7]};
  if (add) {
    lo = *(const f32x4_t*)p + lo;
    hi = *(const f32x4_t*)(p + 4) + hi;
  }
  *(f32x4_t*)p = lo;
  *(f32x4_t*)(p + 4) = hi;
}

// A row is routed when some tile count exceeds the capacity.
__device__ __forceinline__ bool row_is_routed(const BwdArgs& a, int t) {
  bool over = false;
  for (int k = lane_id(); k < a.nt; k += kWave) over |= (int)a.count[(size_t)t * a.nt + k] > a.cap;
  return __ballot(over) != 0ull;
}

__global__ __launch_bounds__(256) void bwd_prep(BwdArgs a) {
  const int w = uniform((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int t = (int)blockIdx.x * 4 + w;
  if (t >= a.T) return;
  const bool routed = row_is_routed(a, t);
  if (!routed) {
    for (int k = lane; k < a.nt; k += kWave) {
      const int c = (int)a.count[(size_t)t * a.nt + k];
      a.count_t[(size_t)k * a.T + t] = (uint16_t)c;
      const uint16_t* src = a.idx + ((size_t)t * a.nt + k) * a.cap;
      uint16_t* dst = a.idx_t + ((size_t)k * a.T + t) * a.cap;
      for (int s = 0; s < c; ++s) dst[s] = src[s];
    }
    return;
  }
  for (int k = lane; k < a.nt; k += kWave) a.count_t[(size_t)k * a.T + t] = 0;
  const int r = uniform(routed_index(a.routed, min(*a.n_routed, a.R), t));
  if (r < 0) return;  // not in the routed list: the row keeps no entries
  int carry = 0;
  for (int k0 = 0; k0 < a.nt; k0 += kWave) {
    const int k = k0 + lane;
    const int c = k < a.nt ? (int)a.count[(size_t)t * a.nt + k] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    if (k < a.nt) a.eoff[(size_t)r * a.nt + k] = carry + incl - c;
    carry += __shfl(incl, kWave - 1, kWave);
  }
}

// gx_t (bf16) from this lane's float32 chunks.
template <int P>
__device__ __forceinline__ void store_gx(const BwdArgs& a, int t, float (*gxa)[8]) {
  const size_t xo = (size_t)t * a.D + (size_t)lane_id() * 8;
#pragma unroll
  for (int c = 0; c < P; ++c) {
    u32x4_t o;
    o.x = (uint32_t)f32_to_bf16(gxa[c][0]) | ((uint32_t)f32_to_bf16(gxa[c][1]) << 16);
    o.y = (uint32_t)f32_to_bf16(gxa[c][2]) | ((uint32_t)f32_to_bf16(gxa[c][3]) << 16);
    o.z = (uint32_t)f32_to_bf16(gxa[c][4]) | ((uint32_t)f32_to_bf16(gxa[c][5]) << 16);
    o.w = (uint32_t)f32_to_bf16(gxa[c][6]) | ((uint32_t)f32_to_bf16(gxa[c][7]) << 16);
    *(u32x4_t*)(a.gx + xo + c * 512) = o;
  }
}

// One entry of row t: the two dot products, the per-entry gradients (stored
// at *out by lane 0) and the gx accumulation.  xc / gyc: this lane's chunks of
// x_t and gy_t (8 bf16 each, at c * 512 + lane * 8), chunk c at xc[c * S]
// (S = 1: registers; S = kWave: a per-wave row copy in LDS).
template <int P, int S = 1>
__device__ __forceinline__ void bwd_entry(const BwdArgs& a, int j, float h, const u32x4_t* xc,
                                          const u32x4_t* gyc, float (*gxa)[8], f32x4_t* out) {
  const int lane = lane_id();
  const size_t rowo = (size_t)j * a.D + (size_t)lane * 8;
  u32x4_t uw[P], dw[P], gw[P];
#pragma unroll
  for (int c = 0; c < P; ++c) {
    uw[c] = ldg16(a.wu + rowo + c * 512);
    dw[c] = ldg16(a.wd + rowo + c * 512);
    gw[c] = ldg16(a.wg + rowo + c * 512);
  }
  // the dot products on the packed bf16 pairs (exact products, float32 sums):
  // no unpacked copies of the weight rows stay live across the reductions
  float su = 0.f, sg = 0.f;
#pragma unroll
  for (int c = 0; c < P; ++c) {
    const u32x4_t xv = xc[c * S], gv = gyc[c * S];
    su = dot2_bf16(xv.x, uw[c].x, su);
    su = dot2_bf16(xv.y, uw[c].y, su);
    su = dot2_bf16(xv.z, uw[c].z, su);
    su = dot2_bf16(xv.w, uw[c].w, su);
    sg = dot2_bf16(gv.x, dw[c].x, sg);
    sg = dot2_bf16(gv.y, dw[c].y, sg);
    sg = dot2_bf16(gv.z, dw[c].z, sg);
    sg = dot2_bf16(gv.w, dw[c].w, sg);
  }
  const float u = wave_sum_uniform(su);
  const float ga = wave_sum_uniform(sg);
  const float gz = ga * u + a.l1g, gu = ga * h;
#pragma unroll
  for (int c = 0; c < P; ++c) {
    float uf[8], wf[8];
    Elt<uint16_t>::unpack(uw[c], uf);
    Elt<uint16_t>::unpack(gw[c], wf);
#pragma unroll
    for (int e = 0; e < 8; ++e) gxa[c][e] = fmaf(gu, uf[e], fmaf(gz, wf[e], gxa[c][e]));
  }
  if (lane == 0) *out = f32x4_t{gz, gu, h * u, 0.f};
}

template <int P>
__device__ __forceinline__ void load_row(const uint16_t* base, int t, int D, u32x4_t* c8) {
  const size_t o = (size_t)t * D + (size_t)lane_id() * 8;
#pragma unroll
  for (int c = 0; c < P; ++c) c8[c] = ldg16(base + o + c * 512);
}

// Entries of one row staged per wave in LDS at a time (column | h << 16, slot
// k * cap + s in the row's TwELL arrays).
constexpr int kRowList = 256;

// Rows within capacity: one wave walks the row's TwELL entries in order and
// writes gx_t.  Routed rows are left to bwd_routed.  The entries are staged a
// group of tiles at a time into a per-wave list in LDS (one lane per tile, all
// the group's count, idx and val loads in flight together), so that the walk
// waits on one memory latency per entry (its weight rows), not on the list
// reads before them.  The row's x_t and gy_t live in LDS too (each lane reads
// back only the chunks it wrote), which keeps the wave within 256 registers:
// two waves per SIMD instead of one, twice the weight rows in flight.  Waves
// share no LDS: no barrier.
template <int P>
__global__ __launch_bounds__(256, 2) void bwd_rows(BwdArgs a) {
  __shared__ uint2 list_s[4][kRowList];
  __shared__ u32x4_t rows_s[4][2][P * kWave];
  const int w = uniform((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int t = (int)blockIdx.x * 4 + w;
  if (t >= a.T) return;
  if (row_is_routed(a, t)) return;
  u32x4_t* xs = rows_s[w][0] + lane;
  u32x4_t* gs = rows_s[w][1] + lane;
  {
    u32x4_t xc[P], gyc[P];
    load_row<P>(a.x, t, a.D, xc);
    load_row<P>(a.gy, t, a.D, gyc);
#pragma unroll
    for (int c = 0; c < P; ++c) {
      xs[c * kWave] = xc[c];
      gs[c * kWave] = gyc[c];
    }
  }
  float gxa[P][8];
#pragma unroll
  for (int c = 0; c < P; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) gxa[c][e] = 0.f;
  uint2* list = list_s[w];
  const int group = max(1, min(kWave, kRowList / max(a.cap, 1)));  // tiles per staging
  const size_t row0 = (size_t)t * a.nt * a.cap;
  for (int k0 = 0; k0 < a.nt; k0 += group) {
    const int k = k0 + lane;
    const int c = (lane < group && k < a.nt) ? min((int)a.count[(size_t)t * a.nt + k], a.cap) : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const int n = uniform(__shfl(incl, kWave - 1, kWave));
    const uint32_t slot0 = (uint32_t)k * (uint32_t)a.cap;
    for (int s = 0; s < c; ++s) {
      const size_t pos = row0 + slot0 + s;
      list[incl - c + s] = make_uint2((uint32_t)a.idx[pos] | ((uint32_t)a.val[pos] << 16),
                                      slot0 + (uint32_t)s);
    }
    // LDS operations of one wave complete in order: the reads below see the
    // writes above once the compiler keeps them in program order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int e = 0; e < n; ++e) {
      const uint2 v = list[e];
      const int j = uniform(min((int)(v.x & 0xffffu), a.N - 1));  // valid lists: j < N already
      const float h = bf16_to_f32((uint16_t)uniform((int)(v.x >> 16)));
      bwd_entry<P, kWave>(a, j, h, xs, gs, gxa, a.co + row0 + uniform((int)v.y));
    }
    __builtin_amdgcn_wave_barrier();
  }
  store_gx<P>(a, t, gxa);
}

// Few tokens (T <= kSplitMaxT): one wave per row would leave the GPU almost
// idle, so each row's tiles are cut into kRowParts equal ranges, one wave per
// range, each writing its partial gx (float32); bwd_rows_combine sums a row's
// ranges in order.  Routed rows are skipped (bwd_routed writes them).
constexpr int kSplitMaxT = 256;
constexpr int kRowParts = 16;

template <int P>
__global__ __launch_bounds__(256) void bwd_rows_split(BwdArgs a, float* rpart) {
  const int item = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int t = item / kRowParts, pi = item - t * kRowParts;
  if (t >= a.T || row_is_routed(a, t)) return;
  u32x4_t xc[P], gyc[P];
  load_row<P>(a.x, t, a.D, xc);
  load_row<P>(a.gy, t, a.D, gyc);
  float gxa[P][8];
#pragma unroll
  for (int c = 0; c < P; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) gxa[c][e] = 0.f;
  const int k0 = (int)((long)pi * a.nt / kRowParts), k1 = (int)((long)(pi + 1) * a.nt / kRowParts);
  for (int k = k0; k < k1; ++k) {
    const size_t tk = (size_t)t * a.nt + k;
    const int c = uniform(min((int)a.count[tk], a.cap));
    for (int s = 0; s < c; ++s) {
      const size_t pos = tk * a.cap + s;
      const int j = uniform(min((int)a.idx[pos], a.N - 1));  // valid lists: j < N already
      bwd_entry<P>(a, j, bf16_to_f32(a.val[pos]), xc, gyc, gxa, a.co + pos);
    }
  }
  float* dst = rpart + (size_t)item * a.D + (size_t)lane_id() * 8;
#pragma unroll
  for (int c = 0; c < P; ++c) {
    *(f32x4_t*)(dst + c * 512) = f32x4_t{gxa[c][0], gxa[c][1], gxa[c][2], gxa[c][3]};
    *(f32x4_t*)(dst + c * 512 + 4) = f32x4_t{gxa[c][4], gxa[c][5], gxa[c][6], gxa[c][7]};
  }
}

__global__ __launch_bounds__(256) void bwd_rows_combine(BwdArgs a, const float* rpart) {
  const int t = (int)blockIdx.y;
  // routed rows: written by bwd_routed_gx (their flag: some count over cap)
  __shared__ int routed_s;
  if (threadIdx.x < kWave) {
    const bool r = row_is_routed(a, t);
    if (threadIdx.x == 0) routed_s = r;
  }
  __syncthreads();
  if (routed_s) return;
  for (int d = ((int)blockIdx.x * 256 + (int)threadIdx.x) * 2; d < a.D; d += (int)gridDim.x * 512) {
    float v0 = 0.f, v1 = 0.f;
    for (int p = 0; p < kRowParts; ++p) {
      const float* src = rpart + ((size_t)t * kRowParts + p) * a.D + d;
      v0 += src[0];
      v1 += src[1];
    }
    *(uint32_t*)(a.gx + (size_t)t * a.D + d) =
        (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
  }
}

// Routed rows: their complete lists are long (a routed row is a heavy one),
// so the lists are cut into parts of `chunk` entries, one wave per part over a
// persistent grid; each part writes its partial gx (float32) and
// bwd_routed_gx sums a row's parts in order.  chunk = max(kRoutedChunk,
// ceil(E / (7 T))) for E routed entries in all, so there are at most 8 T
// parts (the partial buffer's size).  item_start[r]: first part of routed row
// r (exclusive prefix of the part counts, bwd_routed_items);
// item_start[n_routed]: all parts; item_start[n_routed + 1]: chunk.
constexpr int kRoutedChunk = 64;
constexpr int kRoutedSplit = 8;  // parts per row that the partial buffer holds
constexpr int kRoutedWaves = 4096;

__global__ __launch_bounds__(1024) void bwd_routed_items(BwdArgs a, int32_t* item_start) {
  __shared__ int wsum[16];
  const int nr = uniform(min(*a.n_routed, a.R));
  if (routed_on_tiles(a, nr)) return;
  const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
  // all routed entries, then the part size
  int e = 0;
  for (int r = (int)threadIdx.x; r < nr; r += 1024) e += min((int)a.ecount[r], a.N);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) e += __shfl_xor(e, o, kWave);
  if (lane == 0) wsum[w] = e;
  __syncthreads();
  int etot = 0;
  for (int i = 0; i < 16; ++i) etot += wsum[i];
  __syncthreads();
  const int budget = max(1, (kRoutedSplit - 1) * a.R);
  const int chunk = max(kRoutedChunk, (int)(((long)etot + budget - 1) / budget));
  int carry = 0;
  for (int r0 = 0; r0 < nr; r0 += 1024) {
    const int r = r0 + (int)threadIdx.x;
    const int c = r < nr ? (min((int)a.ecount[r], a.N) + chunk - 1) / chunk : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) wsum[w] = incl;
    __syncthreads();
    int before = carry, total = carry;
    for (int i = 0; i < 16; ++i) {
      before += i < w ? wsum[i] : 0;
      total += wsum[i];
    }
    if (r < nr) item_start[r] = before + incl - c;
    __syncthreads();
    carry = total;
  }
  if (threadIdx.x == 0) {
    item_start[nr] = carry;
    item_start[nr + 1] = chunk;
  }
}

template <int P>
__global__ __launch_bounds__(256) void bwd_routed(BwdArgs a, const int32_t* item_start,
                                                  float* part) {
  const int nr = uniform(min(*a.n_routed, a.R));
  if (routed_on_tiles(a, nr)) return;
  const int items = uniform(item_start[nr]);
  const int lane = lane_id();
  for (int it = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6); it < items; it += kRoutedWaves) {
    // routed row of this chunk: the last r with item_start[r] <= it
    int lo = 0, hi = nr - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (item_start[mid] <= it) lo = mid;
      else hi = mid - 1;
    }
    const int r = uniform(lo);
    const int t = uniform(min(max(a.routed[r], 0), a.T - 1));
    const int n = uniform(min((int)a.ecount[r], a.N));
    const int chunk = item_start[nr + 1], pi = it - item_start[r];
    const int s0 = min(pi * chunk, n), s1 = min(s0 + chunk, n);
    u32x4_t xc[P], gyc[P];
    load_row<P>(a.x, t, a.D, xc);
    load_row<P>(a.gy, t, a.D, gyc);
    float gxa[P][8];
#pragma unroll
    for (int c = 0; c < P; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) gxa[c][e] = 0.f;
    for (int s = s0; s < s1; ++s) {
      const size_t pos = (size_t)r * a.N + s;
      const int j = uniform(min((int)a.eidx[pos], a.N - 1));
      bwd_entry<P>(a, j, bf16_to_f32(a.eval[pos]), xc, gyc, gxa, a.co_r + pos);
    }
    float* dst = part + (size_t)it * a.D + (size_t)lane * 8;
#pragma unroll
    for (int c = 0; c < P; ++c) {
      *(f32x4_t*)(dst + c * 512) = f32x4_t{gxa[c][0], gxa[c][1], gxa[c][2], gxa[c][3]};
      *(f32x4_t*)(dst + c * 512 + 4) = f32x4_t{gxa[c][4], gxa[c][5], gxa[c][6], gxa[c][7]};
    }
  }
}

// gx of routed row r = the sum of its parts' partials, in part order (a
// routed row without entries gets zero).  Workgroups loop over the rows.
__global__ __launch_bounds__(256) void bwd_routed_gx(BwdArgs a, const int32_t* item_start,
                                                     const float* part) {
  const int nr = uniform(min(*a.n_routed, a.R));
  if (routed_on_tiles(a, nr)) return;
  for (int r = (int)blockIdx.y; r < nr; r += (int)gridDim.y) {
    const int t = min(max(a.routed[r], 0), a.T - 1);
    const int i0 = item_start[r], i1 = item_start[r + 1];
    for (int d = ((int)blockIdx.x * 256 + (int)threadIdx.x) * 2; d < a.D;
         d += (int)gridDim.x * 512) {
      float v0 = 0.f, v1 = 0.f;
      for (int it = i0; it < i1; ++it) {
        v0 += part[(size_t)it * a.D + d];
        v1 += part[(size_t)it * a.D + d + 1];
      }
      *(uint32_t*)(a.gx + (size_t)t * a.D + d) =
          (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
    }
  }
}

// Column lists of the TwELL entries (rows within capacity), built once so
// that each column's weight-gradient sums read its entries as one contiguous
// list in row order: csc_count counts the entries of every column per block
// of kCscRows rows, csc_colscan turns the counts into each block's start
// within its column and the column totals, csc_ptr scans the totals into
// col_ptr, and csc_fill places every entry (row, gz, gu, a).  Inside a 64-row
// chunk an entry's rank among its column's entries is the number of lower
// lanes (rows) that hold the column, read from a per-column lane mask in LDS,
// so the lists are in row order and the build is deterministic.
constexpr int kCscRows = 256;

__device__ __forceinline__ int tile_col(const BwdArgs& a, size_t g, int s, int k) {
  return min(max((int)a.idx_t[g * a.cap + s] - k * kBTile, 0), kBTile - 1);
}

__global__ __launch_bounds__(64) void csc_count(BwdArgs a, int* hist) {
  __shared__ int cnt[kBTile];
  const int lane = lane_id();
  const int k = (int)blockIdx.x % a.nt, rb = (int)blockIdx.x / a.nt;
  cnt[lane] = 0;
  cnt[lane + kWave] = 0;
  __syncthreads();
  const int r1 = min((rb + 1) * kCscRows, a.T);
  for (int t = rb * kCscRows + lane; t < r1; t += kWave) {
    const size_t g = (size_t)k * a.T + t;
    const int c = (int)a.count_t[g];
    for (int s = 0; s < c; ++s) atomicAdd(&cnt[tile_col(a, g, s, k)], 1);
  }
  __syncthreads();
  int* h = hist + (size_t)rb * a.N + k * kBTile;
  h[lane] = cnt[lane];
  h[lane + kWave] = cnt[lane + kWave];
}

__global__ __launch_bounds__(256) void csc_colscan(BwdArgs a, int* hist, int* total, int nblk) {
  const int j = (int)(blockIdx.x * 256 + threadIdx.x);
  if (j >= a.N) return;
  int run = 0;
  for (int b = 0; b < nblk; ++b) {
    const int v = hist[(size_t)b * a.N + j];
    hist[(size_t)b * a.N + j] = run;
    run += v;
  }
  total[j] = run;
}

__global__ __launch_bounds__(1024) void csc_ptr(const int* total, int N, int* col_ptr) {
  __shared__ int wsum[16];
  const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
  const int per = (N + 1023) / 1024;
  const int lo = min((int)threadIdx.x * per, N), hi = min(lo + per, N);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += total[i];
  int incl = sum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) wsum[w] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int i = 0; i < w; ++i) run += wsum[i];
  for (int i = lo; i < hi; ++i) {
    col_ptr[i] = run;
    run += total[i];
  }
  if (threadIdx.x == 1023) col_ptr[N] = run;
}

// Entries: (row, gz, gu, a) when the per-entry gradients exist already
// (with_grads), else (row, TwELL position, h) for bwd_cols_fused.
__global__ __launch_bounds__(64) void csc_fill(BwdArgs a, const int* hist, const int* col_ptr,
                                               f32x4_t* csc, int with_grads) {
  __shared__ int run[kBTile];
  __shared__ uint32_t mlo[kBTile], mhi[kBTile];
  const int lane = lane_id();
  const int k = (int)blockIdx.x % a.nt, rb = (int)blockIdx.x / a.nt;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int jl = lane + kWave * h;
    run[jl] = col_ptr[k * kBTile + jl] + hist[(size_t)rb * a.N + k * kBTile + jl];
  }
  const uint64_t below = (1ull << lane) - 1ull;
  const int r1 = min((rb + 1) * kCscRows, a.T);
  for (int t0 = rb * kCscRows; t0 < r1; t0 += kWave) {
    const int t = t0 + lane;
    const size_t g = (size_t)k * a.T + t;
    const int c = t < r1 ? (int)a.count_t[g] : 0;
    mlo[lane] = mlo[lane + kWave] = 0u;
    mhi[lane] = mhi[lane + kWave] = 0u;
    __syncthreads();
    for (int s = 0; s < c; ++s) {
      const int jl = tile_col(a, g, s, k);
      if (lane < 32) atomicOr(&mlo[jl], 1u << lane);
      else atomicOr(&mhi[jl], 1u << (lane - 32));
    }
    __syncthreads();
    for (int s = 0; s < c; ++s) {
      const int jl = tile_col(a, g, s, k);
      const uint64_t m = ((uint64_t)mhi[jl] << 32) | mlo[jl];
      const int pos = run[jl] + __popcll(m & below);
      const size_t tp = ((size_t)t * a.nt + k) * a.cap + s;
      if (with_grads) {
        const f32x4_t co = a.co[tp];
        csc[pos] = f32x4_t{__int_as_float(t), co[0], co[1], co[2]};
      } else {
        csc[pos] = f32x4_t{__int_as_float(t), __int_as_float((int)tp), bf16_to_f32(a.val[tp]), 0.f};
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int jl = lane + kWave * h;
      run[jl] += __popcll(((uint64_t)mhi[jl] << 32) | mlo[jl]);
    }
    __syncthreads();
  }
}

// Weight gradients: one wave per (column, chunk of PC * 512 model dimensions).
// The column's TwELL entries come from its list (row order), kColBatch
// entries' x and gy rows loaded together; then the routed rows' entries (one
// binary search per routed row in its complete list, ascending rows).  Every
// column is written (zero when inactive).

// acc += coef * (this lane's chunks of row t), for one matched entry.
template <int PC>
__device__ __forceinline__ void col_accumulate(const BwdArgs& a, int t, int d0, f32x4_t coef,
                                               float (*ag)[8], float (*au)[8], float (*ad)[8],
                                               float& gbs) {
  const size_t ro = (size_t)t * a.D + d0 + (size_t)lane_id() * 8;
  u32x4_t xc[PC], gc[PC];
#pragma unroll
  for (int c = 0; c < PC; ++c) {
    xc[c] = ldg16(a.x + ro + c * 512);
    gc[c] = ldg16(a.gy + ro + c * 512);
  }
#pragma unroll
  for (int c = 0; c < PC; ++c) {
    float xf[8], gf[8];
    Elt<uint16_t>::unpack(xc[c], xf);
    Elt<uint16_t>::unpack(gc[c], gf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ag[c][e] = fmaf(coef[0], xf[e], ag[c][e]);
      au[c][e] = fmaf(coef[1], xf[e], au[c][e]);
      ad[c][e] = fmaf(coef[2], gf[e], ad[c][e]);
    }
  }
  gbs += coef[0];
}

// The same for kColBatch entries (rows t[i], coefficients coef[i] = (gz, gu,
// a); entries past the list carry 0), their rows loaded together, summed in
// batch order.
constexpr int kColBatch = 4;

template <int PC>
__device__ __forceinline__ void col_accumulate_batch(const BwdArgs& a, const int* t, int d0,
                                                     const f32x4_t* coef, float (*ag)[8],
                                                     float (*au)[8], float (*ad)[8], float& gbs) {
  u32x4_t xc[kColBatch][PC], gc[kColBatch][PC];
#pragma unroll
  for (int i = 0; i < kColBatch; ++i) {
    const size_t ro = (size_t)t[i] * a.D + d0 + (size_t)lane_id() * 8;
#pragma unroll
    for (int c = 0; c < PC; ++c) {
      xc[i][c] = ldg16(a.x + ro + c * 512);
      gc[i][c] = ldg16(a.gy + ro + c * 512);
    }
  }
#pragma unroll
  for (int i = 0; i < kColBatch; ++i) {
#pragma unroll
    for (int c = 0; c < PC; ++c) {
      float xf[8], gf[8];
      Elt<uint16_t>::unpack(xc[i][c], xf);
      Elt<uint16_t>::unpack(gc[i][c], gf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ag[c][e] = fmaf(coef[i][0], xf[e], ag[c][e]);
        au[c][e] = fmaf(coef[i][1], xf[e], au[c][e]);
        ad[c][e] = fmaf(coef[i][2], gf[e], ad[c][e]);
      }
    }
    gbs += coef[i][0];
  }
}

template <int PC>
__global__ __launch_bounds__(256) void bwd_cols(BwdArgs a, const int* col_ptr, const f32x4_t* csc) {
  const int w = uniform((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int dchunks = a.D / (PC * 512);
  const int dc = (int)blockIdx.x % dchunks;
  const int j = ((int)blockIdx.x / dchunks) * 4 + w;
  const int d0 = dc * PC * 512;
  float ag[PC][8], au[PC][8], ad[PC][8];
#pragma unroll
  for (int c = 0; c < PC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) ag[c][e] = au[c][e] = ad[c][e] = 0.f;
  float gbs = 0.f;
  const int e0 = uniform(col_ptr[j]), e1 = uniform(col_ptr[j + 1]);
  for (int e = e0; e < e1; e += kColBatch) {
    int tb[kColBatch];
    f32x4_t cb[kColBatch];
#pragma unroll
    for (int i = 0; i < kColBatch; ++i) {
      const f32x4_t v = csc[min(e + i, e1 - 1)];
      tb[i] = min(max(__float_as_int(v[0]), 0), a.T - 1);
      cb[i] = e + i < e1 ? f32x4_t{v[1], v[2], v[3], 0.f} : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    col_accumulate_batch<PC>(a, tb, d0, cb, ag, au, ad, gbs);
  }
  // routed rows: their complete lists, one binary search per row (unless
  // their products run on MFMA tiles and are added afterwards)
  const int k = j / kBTile;
  const int nr0 = uniform(min(*a.n_routed, a.R));
  const int nr = routed_on_tiles(a, nr0) ? 0 : nr0;
  for (int r0 = 0; r0 < nr; r0 += kWave) {
    const int r = r0 + lane;
    int match = -1, tr = 0;
    if (r < nr) {
      tr = a.routed[r];
      // the tile's range of the row's list, kept inside the list's N slots
      const int beg = min(max(a.eoff[(size_t)r * a.nt + k], 0), a.N);
      const int end = min(beg + (int)a.count[(size_t)min(max(tr, 0), a.T - 1) * a.nt + k], a.N);
      const uint16_t* li = a.eidx + (size_t)r * a.N;
      int lo = beg, hi = end;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int)li[mid] < j) lo = mid + 1;
        else hi = mid;
      }
      if (lo < end && (int)li[lo] == j) match = lo;
    }
    uint64_t m = __ballot(match >= 0);
    while (m) {
      const int L = __builtin_ctzll(m);
      m &= m - 1;
      const int t = min(max(__shfl(tr, L, kWave), 0), a.T - 1);
      const int s = __shfl(match, L, kWave);
      const f32x4_t coef = a.co_r[(size_t)(r0 + L) * a.N + s];
      col_accumulate<PC>(a, t, d0, coef, ag, au, ad, gbs);
    }
  }
  const size_t wo = (size_t)j * a.D + d0 + (size_t)lane * 8;
  const bool add = routed_on_tiles(a, nr0);  // the routed rows' sums are there already
#pragma unroll
  for (int c = 0; c < PC; ++c) {
    store_w8(a.gwg + wo + c * 512, ag[c], add);
    store_w8(a.gwu + wo + c * 512, au[c], add);
    store_w8(a.gwd + wo + c * 512, ad[c], add);
  }
  if (a.gb && dc == 0 && lane == 0) a.gb[j] = gbs;
}

// Fused order for d_model <= 2048 and more than kSplitMaxT tokens.  The
// column pass already loads x_t and gy_t for every entry of a column, so with
// the column's wu_t and wd rows at hand (in LDS) it computes the entry's dot
// products itself (gz, gu, a, stored at the entry's TwELL position) and sums
// the weight gradients in the same step; the row pass (bwd_gx) then only
// gathers wg_t and wu_t rows per entry for gx, with no reduction in its chain.
// Four gathered rows per entry instead of five.
constexpr int kFusedBatch = 2;

template <int P>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_cols_fused(BwdArgs a, const int* col_ptr,
                                                      const f32x4_t* csc) {
  const int w = uniform((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int j = (int)blockIdx.x * 4 + w;
  // the column's wu_t and wd rows, each lane's 8-element pieces kept in LDS
  // (read back by the same lane only, so no barrier) to leave registers for
  // two waves per SIMD
  __shared__ u32x4_t wrow_s[4][2][P][kWave];
  {
    u32x4_t uw[P], dw[P];
    load_row<P>(a.wu, j, a.D, uw);
    load_row<P>(a.wd, j, a.D, dw);
#pragma unroll
    for (int c = 0; c < P; ++c) {
      wrow_s[w][0][c][lane] = uw[c];
      wrow_s[w][1][c][lane] = dw[c];
    }
  }
  float ag[P][8], au[P][8], ad[P][8];
#pragma unroll
  for (int c = 0; c < P; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) ag[c][e] = au[c][e] = ad[c][e] = 0.f;
  float gbs = 0.f;
  const int e0 = uniform(col_ptr[j]), e1 = uniform(col_ptr[j + 1]);
  for (int e = e0; e < e1; e += kFusedBatch) {
    u32x4_t xc[kFusedBatch][P], gc[kFusedBatch][P];
    int pos[kFusedBatch];
    float h[kFusedBatch];
#pragma unroll
    for (int i = 0; i < kFusedBatch; ++i) {
      const f32x4_t v = csc[min(e + i, e1 - 1)];
      const int t = min(max(__float_as_int(v[0]), 0), a.T - 1);
      pos[i] = __float_as_int(v[1]);
      h[i] = v[2];
      load_row<P>(a.x, t, a.D, xc[i]);
      load_row<P>(a.gy, t, a.D, gc[i]);
    }
    // an opaque zero offset: keeps the compiler from hoisting the LDS reads
    // (and the registers they would hold) out of the loop
    int lofs = 0;
    asm volatile("" : "+v"(lofs));
    const u32x4_t* wu_l = &wrow_s[w][0][0][lane + lofs];
    const u32x4_t* wd_l = &wrow_s[w][1][0][lane + lofs];
#pragma unroll
    for (int i = 0; i < kFusedBatch; ++i) {
      float su = 0.f, sg = 0.f;
#pragma unroll
      for (int c = 0; c < P; ++c) {
        float xf[8], uf[8], gf[8], df[8];
        Elt<uint16_t>::unpack(xc[i][c], xf);
        Elt<uint16_t>::unpack(wu_l[c * kWave], uf);
        Elt<uint16_t>::unpack(gc[i][c], gf);
        Elt<uint16_t>::unpack(wd_l[c * kWave], df);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          su = fmaf(xf[q], uf[q], su);
          sg = fmaf(gf[q], df[q], sg);
        }
      }
      const float u = wave_sum_uniform(su);
      const float ga = wave_sum_uniform(sg);
      const bool live = e + i < e1;
      const float gz = live ? ga * u + a.l1g : 0.f, gu = live ? ga * h[i] : 0.f;
      const float aa = live ? h[i] * u : 0.f;
      if (live && lane == 0) a.co[pos[i]] = f32x4_t{gz, gu, aa, 0.f};
#pragma unroll
      for (int c = 0; c < P; ++c) {
        float xf[8], gf[8];
        Elt<uint16_t>::unpack(xc[i][c], xf);
        Elt<uint16_t>::unpack(gc[i][c], gf);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          ag[c][q] = fmaf(gz, xf[q], ag[c][q]);
          au[c][q] = fmaf(gu, xf[q], au[c][q]);
          ad[c][q] = fmaf(aa, gf[q], ad[c][q]);
        }
      }
      gbs += gz;
    }
  }
  // routed rows: their entries' gradients come from bwd_routed (unless their
  // products run on MFMA tiles and are added afterwards)
  const int k = j / kBTile;
  const int nr0 = uniform(min(*a.n_routed, a.R));
  const int nr = routed_on_tiles(a, nr0) ? 0 : nr0;
  for (int r0 = 0; r0 < nr; r0 += kWave) {
    const int r = r0 + lane;
    int match = -1, tr = 0;
    if (r < nr) {
      tr = a.routed[r];
      const int beg = min(max(a.eoff[(size_t)r * a.nt + k], 0), a.N);
      const int end = min(beg + (int)a.count[(size_t)min(max(tr, 0), a.T - 1) * a.nt + k], a.N);
      const uint16_t* li = a.eidx + (size_t)r * a.N;
      int lo = beg, hi = end;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int)li[mid] < j) lo = mid + 1;
        else hi = mid;
      }
      if (lo < end && (int)li[lo] == j) match = lo;
    }
    uint64_t m = __ballot(match >= 0);
    while (m) {
      const int L = __builtin_ctzll(m);
      m &= m - 1;
      const int t = min(max(__shfl(tr, L, kWave), 0), a.T - 1);
      const int s = __shfl(match, L, kWave);
      const f32x4_t coef = a.co_r[(size_t)(r0 + L) * a.N + s];
      col_accumulate<P>(a, t, 0, coef, ag, au, ad, gbs);
    }
  }
  const size_t wo = (size_t)j * a.D + (size_t)lane * 8;
  const bool add = routed_on_tiles(a, nr0);  // the routed rows' sums are there already
#pragma unroll
  for (int c = 0; c < P; ++c) {
    store_w8(a.gwg + wo + c * 512, ag[c], add);
    store_w8(a.gwu + wo + c * 512, au[c], add);
    store_w8(a.gwd + wo + c * 512, ad[c], add);
  }
  if (a.gb && lane == 0) a.gb[j] = gbs;
}

// gx of the rows within capacity from the stored per-entry gradients: the
// row's entries are gathered a group of tiles at a time into a per-wave list
// (TwELL positions, ascending) and taken kGxBatch at a time, their wg_t and
// wu_t rows loaded together.
constexpr int kGxList = 512;
constexpr int kGxBatch = 4;

template <int P>
__global__ __launch_bounds__(256) void bwd_gx(BwdArgs a) {
  __shared__ int list_s[4][kGxList];
  const int w = uniform((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int t = (int)blockIdx.x * 4 + w;
  if (t >= a.T || row_is_routed(a, t)) return;
  int* list = list_s[w];
  float gxa[P][8];
#pragma unroll
  for (int c = 0; c < P; ++c)
#pragma unroll
    for (int q = 0; q < 8; ++q) gxa[c][q] = 0.f;
  const int G = min(kWave, max(1, kGxList / max(a.cap, 1)));  // tiles per group
  for (int kb = 0; kb < a.nt; kb += G) {
    const int k = kb + lane;
    const int c = (lane < G && k < a.nt) ? min((int)a.count[(size_t)t * a.nt + k], a.cap) : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const int n = uniform(__shfl(incl, kWave - 1, kWave));
    for (int s = 0; s < c; ++s) list[incl - c + s] = (int)(((size_t)t * a.nt + k) * a.cap + s);
    __builtin_amdgcn_wave_barrier();
    for (int e0 = 0; e0 < n; e0 += kGxBatch) {
      u32x4_t gw[kGxBatch][P], uw[kGxBatch][P];
      f32x4_t co[kGxBatch];
#pragma unroll
      for (int i = 0; i < kGxBatch; ++i) {
        const int pos = uniform(list[min(e0 + i, n - 1)]);
        const int j = uniform(min((int)a.idx[pos], a.N - 1));  // valid lists: j < N already
        co[i] = e0 + i < n ? a.co[pos] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        load_row<P>(a.wg, j, a.D, gw[i]);
        load_row<P>(a.wu, j, a.D, uw[i]);
      }
#pragma unroll
      for (int i = 0; i < kGxBatch; ++i)
#pragma unroll
        for (int cc = 0; cc < P; ++cc) {
          float gf[8], uf[8];
          Elt<uint16_t>::unpack(gw[i][cc], gf);
          Elt<uint16_t>::unpack(uw[i][cc], uf);
#pragma unroll
          for (int q = 0; q < 8; ++q)
            gxa[cc][q] = fmaf(co[i][1], uf[q], fmaf(co[i][0], gf[q], gxa[cc][q]));
        }
    }
    __builtin_amdgcn_wave_barrier();  // the list is rewritten by the next group
  }
  store_gx<P>(a, t, gxa);
}

// ---------------------------------------------------------------------------
// The general path: float32 shapes (d_model up to 2048), and bf16 widths that
// are not a multiple of 512 (up to 4096): at most 8 16-byte chunks per lane.  The entries come from complete activity
// lists for every row: twell_pack's own kernels run again at the full capacity
// of 128 per tile (the same exact activity decision, so a row within the
// forward's capacity gets exactly its forward entries and a routed row its
// complete list), and no row is routed here.  One wave per row walks its
// entries for the per-entry gradients and gx (rows in 16-byte chunks per lane,
// the last chunk masked); the column lists of the bf16 path (bwd_prep, csc_*)
// are built on these arrays; one wave per column sums the weight gradients.
constexpr int kGenCap = 128;
constexpr int kGenMaxChunks = 8;  // 16-byte chunks per lane and row

struct GenArgs {
  const void* x;
  const void* wg;
  const void* wu;
  const void* wd;
  const void* gy;
  const uint16_t* count;  // [T, nt] complete lists (capacity kGenCap)
  const uint16_t* idx;    // [T, nt, kGenCap]
  const void* val;        // [T, nt, kGenCap] h (element type)
  f32x4_t* co;            // [T, nt, kGenCap] (gz, gu, a, 0)
  void* gx;               // [T, D] (element type)
  float* gwg;             // [N, D]
  float* gwu;
  float* gwd;
  float* gb;              // [N] or null
  int T, D, N, nt;
  float l1g;
};

// this lane's chunks c (E values at E (64 c + lane)) of a row of D values,
// unpacked to float32 (zero past D)
template <typename T, int NCH>
__device__ __forceinline__ void gen_row(const void* base, size_t row, int D,
                                        float (*v)[Elt<T>::kPerChunk]) {
  constexpr int E = Elt<T>::kPerChunk;
  const T* r = (const T*)base + row * D;
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e = E * (kWave * c + lane);
    const u32x4_t q = e < D ? ldg16(r + e) : u32x4_t{0u, 0u, 0u, 0u};
    Elt<T>::unpack(q, v[c]);
  }
}

template <typename T, int NCH>
__global__ __launch_bounds__(256) void gen_rows(GenArgs a) {
  constexpr int E = Elt<T>::kPerChunk;
  const int lane = lane_id();
  const int t = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (t >= a.T) return;
  float xc[NCH][E], gc[NCH][E], gxa[NCH][E];
  gen_row<T, NCH>(a.x, t, a.D, xc);
  gen_row<T, NCH>(a.gy, t, a.D, gc);
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int e = 0; e < E; ++e) gxa[c][e] = 0.f;
  for (int k = 0; k < a.nt; ++k) {
    const size_t tk = (size_t)t * a.nt + k;
    const int n = uniform(min((int)a.count[tk], kGenCap));
    for (int s = 0; s < n; ++s) {
      const size_t pos = tk * kGenCap + s;
      const int j = uniform(min((int)a.idx[pos], a.N - 1));  // valid lists: j < N already
      const float h = __int_as_float(uniform(__float_as_int(Elt<T>::load1(a.val, pos))));
      float uw[NCH][E], dw[NCH][E], gw[NCH][E];
      gen_row<T, NCH>(a.wu, j, a.D, uw);
      gen_row<T, NCH>(a.wd, j, a.D, dw);
      gen_row<T, NCH>(a.wg, j, a.D, gw);
      float su = 0.f, sg = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          su = fmaf(xc[c][e], uw[c][e], su);
          sg = fmaf(gc[c][e], dw[c][e], sg);
        }
      const float u = wave_sum_uniform(su), ga = wave_sum_uniform(sg);
      const float gz = ga * u + a.l1g, gu = ga * h;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) gxa[c][e] = fmaf(gu, uw[c][e], fmaf(gz, gw[c][e], gxa[c][e]));
      if (lane == 0) a.co[pos] = f32x4_t{gz, gu, h * u, 0.f};
    }
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e0 = E * (kWave * c + lane);
    if (e0 < a.D)
#pragma unroll
      for (int e = 0; e < E; ++e) Elt<T>::store1(a.gx, (size_t)t * a.D + e0 + e, gxa[c][e]);
  }
}

// One wave per column: its list's entries (row order) summed into the three
// weight-gradient rows and gb; every column is written (zero when inactive).
template <typename T, int NCH>
__global__ __launch_bounds__(256) void gen_cols(GenArgs a, const int* col_ptr, const f32x4_t* csc) {
  constexpr int E = Elt<T>::kPerChunk;
  const int lane = lane_id();
  const int j = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (j >= a.N) return;
  float ag[NCH][E], au[NCH][E], ad[NCH][E];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int e = 0; e < E; ++e) ag[c][e] = au[c][e] = ad[c][e] = 0.f;
  float gbs = 0.f;
  const int e0 = uniform(col_ptr[j]), e1 = uniform(col_ptr[j + 1]);
  for (int i = e0; i < e1; ++i) {
    const f32x4_t v = csc[i];
    const int t = min(max(__float_as_int(v[0]), 0), a.T - 1);
    float xc[NCH][E], gc[NCH][E];
    gen_row<T, NCH>(a.x, t, a.D, xc);
    gen_row<T, NCH>(a.gy, t, a.D, gc);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int q = 0; q < E; ++q) {
        ag[c][q] = fmaf(v[1], xc[c][q], ag[c][q]);
        au[c][q] = fmaf(v[2], xc[c][q], au[c][q]);
        ad[c][q] = fmaf(v[3], gc[c][q], ad[c][q]);
      }
    gbs += v[1];
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e = E * (kWave * c + lane);
    if (e < a.D) {
      const size_t o = (size_t)j * a.D + e;
#pragma unroll
      for (int q = 0; q < E; q += 4) {
        *(f32x4_t*)(a.gwg + o + q) = f32x4_t{ag[c][q], ag[c][q + 1], ag[c][q + 2], ag[c][q + 3]};
        *(f32x4_t*)(a.gwu + o + q) = f32x4_t{au[c][q], au[c][q + 1], au[c][q + 2], au[c][q + 3]};
        *(f32x4_t*)(a.gwd + o + q) = f32x4_t{ad[c][q], ad[c][q + 1], ad[c][q + 2], ad[c][q + 3]};
      }
    }
  }
  if (a.gb && lane == 0) a.gb[j] = gbs;
}

template <typename T>
void launch_gen_kernels(const GenArgs& a, const int* col_ptr, const f32x4_t* csc, bool rows,
                        hipStream_t stream) {
  constexpr int E = Elt<T>::kPerChunk;
  const int nch = (a.D / E + kWave - 1) / kWave;  // 16-byte chunks per lane
  const dim3 blk(256);
  if (rows) {
    const dim3 g((unsigned)((a.T + 3) / 4));
    if (nch <= 1) hipLaunchKernelGGL((gen_rows<T, 1>), g, blk, 0, stream, a);
    else if (nch <= 2) hipLaunchKernelGGL((gen_rows<T, 2>), g, blk, 0, stream, a);
    else if (nch <= 4) hipLaunchKernelGGL((gen_rows<T, 4>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((gen_rows<T, 8>), g, blk, 0, stream, a);
  } else {
    const dim3 g((unsigned)((a.N + 3) / 4));
    if (nch <= 1) hipLaunchKernelGGL((gen_cols<T, 1>), g, blk, 0, stream, a, col_ptr, csc);
    else if (nch <= 2) hipLaunchKernelGGL((gen_cols<T, 2>), g, blk, 0, stream, a, col_ptr, csc);
    else if (nch <= 4) hipLaunchKernelGGL((gen_cols<T, 4>), g, blk, 0, stream, a, col_ptr, csc);
    else hipLaunchKernelGGL((gen_cols<T, 8>), g, blk, 0, stream, a, col_ptr, csc);
  }
}

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

bool backward_supported(int dtype, int d_model) {
  return (dtype == 1 && d_model % 512 == 0 && d_model <= 4096) || backward_general(dtype, d_model);
}

bool backward_general(int dtype, int d_model) {
  const int per_chunk = dtype == 0 ? 4 : 8;  // values per 16 bytes
  return (dtype == 0 || d_model % 512 != 0) && d_model % 8 == 0 &&
         d_model <= kGenMaxChunks * kWave * per_chunk;
}

int backward_general_cap() { return kGenCap; }

// The general path: tile-major copies, per-entry gradients, column lists of
// the complete lists (capacity kGenCap).
size_t backward_general_workspace_bytes(int T, int N) {
  const size_t nt = (size_t)N / kBTile, cap = kGenCap;
  return al256(nt * T * 2) + al256(nt * T * cap * 2) + al256((size_t)T * nt * cap * 16) +
         al256((size_t)((T + kCscRows - 1) / kCscRows) * N * 4) + al256((size_t)N * 4) +
         al256(((size_t)N + 1) * 4) + al256((size_t)T * nt * cap * 16);
}

hipError_t launch_backward_general(int dtype, const void* x, const void* wg_t, const void* wu_t,
                                   const void* wd, const uint16_t* count, const uint16_t* idx,
                                   const void* val, const void* gy, void* gx, float* gwg_t,
                                   float* gwu_t, float* gwd, float* gb, int T, int D, int N,
                                   float l1g, void* ws, hipStream_t stream) {
  if (!backward_general(dtype, D)) return hipErrorInvalidValue;
  const int nt = N / kBTile;
  char* p = (char*)ws;
  uint16_t* count_t = (uint16_t*)p;
  p += al256((size_t)nt * T * 2);
  uint16_t* idx_t = (uint16_t*)p;
  p += al256((size_t)nt * T * kGenCap * 2);
  f32x4_t* co = (f32x4_t*)p;
  p += al256((size_t)T * nt * kGenCap * 16);
  const int nblk = (T + kCscRows - 1) / kCscRows;
  int* hist = (int*)p;
  p += al256((size_t)nblk * N * 4);
  int* total = (int*)p;
  p += al256((size_t)N * 4);
  int* col_ptr = (int*)p;
  p += al256(((size_t)N + 1) * 4);
  f32x4_t* csc = (f32x4_t*)p;
  // the tile-major copies and column lists of the bf16 path, on the complete
  // lists: no row exceeds the capacity, so none is treated as routed
  BwdArgs b{};
  b.count = count;
  b.idx = idx;
  b.count_t = count_t;
  b.idx_t = idx_t;
  b.co = co;
  b.T = T;
  b.D = D;
  b.N = N;
  b.nt = nt;
  b.cap = kGenCap;
  GenArgs a{x, wg_t, wu_t, wd, gy, count, idx, val, co, gx, gwg_t, gwu_t, gwd, gb, T, D, N, nt, l1g};
  const dim3 blk(256);
  hipLaunchKernelGGL(bwd_prep, dim3((unsigned)((T + 3) / 4)), blk, 0, stream, b);
  if (dtype == 0) launch_gen_kernels<float>(a, nullptr, nullptr, true, stream);
  else launch_gen_kernels<uint16_t>(a, nullptr, nullptr, true, stream);
  hipLaunchKernelGGL(csc_count, dim3((unsigned)(nblk * nt)), dim3(64), 0, stream, b, hist);
  hipLaunchKernelGGL(csc_colscan, dim3((unsigned)((N + 255) / 256)), blk, 0, stream, b, hist,
                     total, nblk);
  hipLaunchKernelGGL(csc_ptr, dim3(1), dim3(1024), 0, stream, (const int*)total, N, col_ptr);
  hipLaunchKernelGGL(csc_fill, dim3((unsigned)(nblk * nt)), dim3(64), 0, stream, b,
                     (const int*)hist, (const int*)col_ptr, csc, 1);
  if (dtype == 0) launch_gen_kernels<float>(a, col_ptr, csc, false, stream);
  else launch_gen_kernels<uint16_t>(a, col_ptr, csc, false, stream);
  return hipGetLastError();
}

// Workspace of the backward: the routed rows' z (later reused for their
// per-entry gradients), their complete lists and tile offsets, the tile-major
// copies and the per-entry gradients of the TwELL entries.
// Routed-row buffers are sized for R rows (the routed rows the caller allows
// for), the others for all T rows.
// The first region holds the routed rows' z, then their per-entry gradients,
// or (MFMA path) the dense buffers of backward_routed.hip.
size_t routed_region_bytes(int T, int N, int D, int R) {
  size_t n = al256((size_t)R * N * 16);
  if (routed_dense_launch(T, R)) n = std::max(n, routed_dense_workspace_bytes(N, D, R));
  return n;
}

size_t backward_workspace_bytes(int T, int N, int D, int cap, int R) {
  const size_t nt = (size_t)N / kBTile;
  return routed_region_bytes(T, N, D, R) + 2 * al256((size_t)R * N * 2) + al256((size_t)R * 2) +
         al256((size_t)R * nt * 4) + al256(nt * T * 2) + al256(nt * T * cap * 2) +
         al256((size_t)T * nt * cap * 16) + al256(((size_t)R + 2) * 4) +
         al256((size_t)R * kRoutedSplit * D * 4) +
         (T <= kSplitMaxT ? al256((size_t)T * kRowParts * D * 4) : 0) +
         al256((size_t)((T + kCscRows - 1) / kCscRows) * N * 4) + al256((size_t)N * 4) +
         al256(((size_t)N + 1) * 4) + al256((size_t)T * nt * cap * 16);
}

// More routed rows than the workspace holds (the forward routed more than the
// caller allowed for): the rows past R were not processed, so the result is
// made unusable in a way no training loop misses: gb (when given) and the
// first row of gx become NaN.
__global__ __launch_bounds__(256) void bwd_routed_overflow(BwdArgs a) {
  if (*a.n_routed <= a.R) return;
  if (a.gb)
    for (int j = (int)threadIdx.x; j < a.N; j += 256) a.gb[j] = __builtin_nanf("");
  for (int d = (int)threadIdx.x; d < a.D; d += 256) a.gx[d] = (uint16_t)0x7fc0u;
}

hipError_t launch_backward(const void* x, const void* wg_t, const float* b_g, const void* wu_t,
                           const void* wd, const float* xnorm, const float* wnorm,
                           const uint16_t* count, const uint16_t* idx, const void* val,
                           const int32_t* routed, const int32_t* n_routed, const void* gy,
                           void* gx, float* gwg_t, float* gwu_t, float* gwd, float* gb, int T,
                           int D, int N, int cap, float l1g, int R, GuardBand band, void* ws,
                           hipStream_t stream) {
  const int nt = N / kBTile;
  char* p = (char*)ws;
  float* z_r = (float*)p;          // routed rows' z, then (same bytes) their entry gradients
  f32x4_t* co_r = (f32x4_t*)p;
  void* dense_ws = p;              // or the MFMA path's buffers
  const bool dense = routed_dense_launch(T, R);
  p += routed_region_bytes(T, N, D, R);
  uint16_t* eidx = (uint16_t*)p;
  p += al256((size_t)R * N * 2);
  uint16_t* eval = (uint16_t*)p;
  p += al256((size_t)R * N * 2);
  uint16_t* ecount = (uint16_t*)p;
  p += al256((size_t)R * 2);
  int32_t* eoff = (int32_t*)p;
  p += al256((size_t)R * nt * 4);
  uint16_t* count_t = (uint16_t*)p;
  p += al256((size_t)nt * T * 2);
  uint16_t* idx_t = (uint16_t*)p;
  p += al256((size_t)nt * T * cap * 2);
  f32x4_t* co = (f32x4_t*)p;
  p += al256((size_t)T * nt * cap * 16);
  int32_t* item_start = (int32_t*)p;
  p += al256(((size_t)R + 2) * 4);
  float* part = (float*)p;
  p += al256((size_t)R * kRoutedSplit * D * 4);
  float* rpart = (float*)p;  // few tokens only
  p += T <= kSplitMaxT ? al256((size_t)T * kRowParts * D * 4) : 0;
  const int nblk = (T + kCscRows - 1) / kCscRows;
  int* hist = (int*)p;
  p += al256((size_t)nblk * N * 4);
  int* total = (int*)p;
  p += al256((size_t)N * 4);
  int* col_ptr = (int*)p;
  p += al256(((size_t)N + 1) * 4);
  f32x4_t* csc = (f32x4_t*)p;

  // routed rows: z with the gate GEMM, then complete activity lists
  hipError_t e = hipSuccess;
  if (R > 0) {
    e = launch_gate_preact(x, wg_t, b_g, z_r, T, D, N, routed, n_routed, stream, R);
    if (e != hipSuccess) return e;
    e = launch_ell_convert(z_r, x, wg_t, b_g, xnorm, wnorm, N, ecount, eidx, eval, T, D, N, band,
                           routed, n_routed, stream, R);
    if (e != hipSuccess) return e;
  }

  BwdArgs a{(const uint16_t*)x, (const uint16_t*)wg_t, (const uint16_t*)wu_t,
            (const uint16_t*)wd, (const uint16_t*)gy, count, idx, (const uint16_t*)val,
            routed, n_routed, ecount, eidx, eval, eoff, count_t, idx_t, co, co_r,
            (uint16_t*)gx, gwg_t, gwu_t, gwd, gb, T, D, N, nt, cap, l1g, R, dense ? 1 : 0};
  const dim3 rows_grid((unsigned)((T + 3) / 4));
  hipLaunchKernelGGL(bwd_prep, rows_grid, dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dense) {  // the routed rows' u, ga, per-entry gradients and gx on MFMA tiles
    e = launch_backward_routed_dense(x, gy, wg_t, wu_t, wd, routed, n_routed, ecount, eidx, eval,
                                     gx, gwg_t, gwu_t, gwd, gb, T, D, N, R, l1g, dense_ws, 0,
                                     stream);
    if (e != hipSuccess) return e;
  }
  // the fused order keeps TwELL positions in 31 bits and a row's group of
  // tiles inside bwd_gx's list
  const bool fused = D <= 2048 && T > kSplitMaxT && cap <= kGxList &&
                     (size_t)T * nt * (size_t)cap < ((size_t)1 << 31);
  const dim3 tiles_blocks((unsigned)(nt * nblk));
  switch (D / 512) {
#define SFFN_BWD_ROWS(P)                                                                        \
  case P:                                                                                        \
    if (!fused && T <= kSplitMaxT)                                                               \
      hipLaunchKernelGGL(bwd_rows_split<P>, dim3((unsigned)((T * kRowParts + 3) / 4)),           \
                         dim3(256), 0, stream, a, rpart);                                        \
    else if (!fused)                                                                             \
      hipLaunchKernelGGL(bwd_rows<P>, rows_grid, dim3(256), 0, stream, a);                       \
    hipLaunchKernelGGL(bwd_routed_items, dim3(1), dim3(1024), 0, stream, a, item_start);         \
    hipLaunchKernelGGL(bwd_routed<P>, dim3(kRoutedWaves / 4), dim3(256), 0, stream, a,           \
                       (const int32_t*)item_start, part);                                        \
    break;
    SFFN_BWD_ROWS(1) SFFN_BWD_ROWS(2) SFFN_BWD_ROWS(3) SFFN_BWD_ROWS(4)
    SFFN_BWD_ROWS(5) SFFN_BWD_ROWS(6) SFFN_BWD_ROWS(7) SFFN_BWD_ROWS(8)
#undef SFFN_BWD_ROWS
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_routed_gx, dim3((unsigned)((D + 511) / 512), 256), dim3(256), 0, stream,
                     a, (const int32_t*)item_start, (const float*)part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!fused && T <= kSplitMaxT) {
    hipLaunchKernelGGL(bwd_rows_combine, dim3((unsigned)((D + 511) / 512), (unsigned)T), dim3(256),
                       0, stream, a, (const float*)rpart);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the TwELL entries' column lists, then the weight gradients (and, fused,
  // the per-entry gradients, then gx)
  hipLaunchKernelGGL(csc_count, tiles_blocks, dim3(64), 0, stream, a, hist);
  hipLaunchKernelGGL(csc_colscan, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, a, hist,
                     total, nblk);
  hipLaunchKernelGGL(csc_ptr, dim3(1), dim3(1024), 0, stream, (const int*)total, N, col_ptr);
  hipLaunchKernelGGL(csc_fill, tiles_blocks, dim3(64), 0, stream, a, (const int*)hist,
                     (const int*)col_ptr, csc, fused ? 0 : 1);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (fused) {
    const dim3 cg((unsigned)(N / 4));
    switch (D / 512) {
      case 1: hipLaunchKernelGGL(bwd_cols_fused<1>, cg, dim3(256), 0, stream, a, (const int*)col_ptr, (const f32x4_t*)csc); hipLaunchKernelGGL(bwd_gx<1>, rows_grid, dim3(256), 0, stream, a); break;
      case 2: hipLaunchKernelGGL(bwd_cols_fused<2>, cg, dim3(256), 0, stream, a, (const int*)col_ptr, (const f32x4_t*)csc); hipLaunchKernelGGL(bwd_gx<2>, rows_grid, dim3(256), 0, stream, a); break;
      case 3: hipLaunchKernelGGL(bwd_cols_fused<3>, cg, dim3(256), 0, stream, a, (const int*)col_ptr, (const f32x4_t*)csc); hipLaunchKernelGGL(bwd_gx<3>, rows_grid, dim3(256), 0, stream, a); break;
      default: hipLaunchKernelGGL(bwd_cols_fused<4>, cg, dim3(256), 0, stream, a, (const int*)col_ptr, (const f32x4_t*)csc); hipLaunchKernelGGL(bwd_gx<4>, rows_grid, dim3(256), 0, stream, a); break;
    }
  } else {
    // one wave per (column, 512 model dimensions): at d_model 4096 this ran
    // the column pass in 1.39 ms against 1.78 ms with 1024 dimensions per
    // wave (twice the waves, each with fewer registers: more of them resident)
    hipLaunchKernelGGL(bwd_cols<1>, dim3((unsigned)(N / 4 * (D / 512))), dim3(256), 0, stream, a,
                       (const int*)col_ptr, (const f32x4_t*)csc);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dense) {  // the routed rows' weight gradients and gb, added to the sums above
    e = launch_backward_routed_dense(x, gy, wg_t, wu_t, wd, routed, n_routed, ecount, eidx, eval,
                                     gx, gwg_t, gwu_t, gwd, gb, T, D, N, R, l1g, dense_ws, 1,
                                     stream);
    if (e != hipSuccess) return e;
  }
  if (R < T) hipLaunchKernelGGL(bwd_routed_overflow, dim3(1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sffn
