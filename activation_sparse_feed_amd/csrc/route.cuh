// Routed-row scan of up to 256 rows inside one workgroup of 256 threads
// (pwwt.cn article, section 03: a row whose activity overflows the compact
// format in any tile goes to the dense path).
#pragma once

#include "common.cuh"

namespace sffn {

constexpr int kRouteBlock = 256;  // rows (and threads) of the one-workgroup scan

// Row t < T is routed when count[t, k] > cap for some tile k.  Every thread of
// the workgroup returns the number of routed rows n, and rows_s[0 .. n) holds
// them in ascending order.  flag_s: kRouteBlock ints of scratch LDS,
// wave_tot: kRouteBlock / 64 ints.  Deterministic, no atomics.
__device__ __forceinline__ int route_rows_lds(const uint16_t* __restrict__ count, int T, int nt,
                                              int cap, int* flag_s, int* rows_s, int* wave_tot) {
  const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
  constexpr int R = 16;
  // wave w takes rows w, w + 4, ...; the lanes read a row's tile counts side
  // by side, sixteen rows' loads in flight together
  for (int u0 = 0; u0 < kRouteBlock / 4 && u0 * 4 < T; u0 += R) {
    bool over[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int t = (u0 + u) * 4 + w;
      over[u] = false;
      if (t < T)
        for (int k = lane; k < nt; k += kWave) over[u] |= (int)count[(size_t)t * nt + k] > cap;
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int t = (u0 + u) * 4 + w;
      const int f = __ballot(over[u]) != 0ull;
      if (t < T && lane == 0) flag_s[t] = f;
    }
  }
  __syncthreads();
  const int t = (int)threadIdx.x;
  const int f = t < T ? flag_s[t] : 0;
  const uint64_t m = __ballot(f);
  if (lane == 0) wave_tot[w] = __popcll(m);
  __syncthreads();
  int off = 0, n = 0;
  for (int i = 0; i < kRouteBlock / kWave; ++i) {
    off += i < w ? wave_tot[i] : 0;
    n += wave_tot[i];
  }
  if (f) rows_s[off + lanes_below(m)] = t;
  __syncthreads();
  return n;
}

// Routed-row mask: bit i of word g is set when row 16 g + i is routed
// (route_flags writes it, one word per 16 rows).  MaskRanks turns it into the
// ascending routed list inside one 256-thread workgroup: init gives each
// thread a run of words and the number of routed rows before them (one block
// scan), after which emit writes any range of ranks with no further scan, so
// the consumers of the list can build the parts they need themselves.
struct MaskRanks {
  int g0, g1;   // this thread's words
  int before;   // routed rows in the words before g0
  int total;    // routed rows in all (the same in every thread)

  // wave_s: kRouteBlock / kWave ints of LDS; ends with a barrier.
  __device__ __forceinline__ void init(const uint16_t* __restrict__ mask, int groups,
                                       int* wave_s) {
    const int per = (groups + kRouteBlock - 1) / kRouteBlock;
    const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
    g0 = min(groups, (int)threadIdx.x * per);
    g1 = min(groups, g0 + per);
    int c = 0;
    for (int g = g0; g < g1; ++g) c += __popc((uint32_t)mask[g]);
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) wave_s[w] = incl;
    __syncthreads();
    before = incl - c;
    total = 0;
    for (int i = 0; i < kRouteBlock / kWave; ++i) {
      const int t = wave_s[i];
      before += i < w ? t : 0;
      total += t;
    }
    __syncthreads();
  }

  // out[r - lo] = the routed row of rank r, for lo <= r < hi.
  __device__ __forceinline__ void emit(const uint16_t* __restrict__ mask, int lo, int hi,
                                       int* out) const {
    int r = before;
    for (int g = g0; g < g1 && r < hi; ++g) {
      uint32_t m = mask[g];
      const int n = __popc(m);
      if (r + n <= lo) {
        r += n;
        continue;
      }
      while (m != 0u) {
        const int i = __ffs(m) - 1;
        m &= m - 1u;
        if (r >= lo && r < hi) out[r - lo] = 16 * g + i;
        ++r;
      }
    }
  }
};

}  // namespace sffn
