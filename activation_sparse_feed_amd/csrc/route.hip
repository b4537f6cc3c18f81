// Hybrid routing scan (pwwt.cn article, section 03: the rare high-activity
// tokens that do not fit the compact format are diverted to a dense path).
//
// A row is routed when any of its TwELL tiles holds more active columns than
// the capacity.  Small kernels, no atomics, deterministic:
//   route_flags    per row (lanes over the tiles): flag = OR_k (count[t, k] > cap),
//                  written as a mask of one 16-bit word per 16 rows
//   route_compact  each 256-row block counts the routed rows of the words
//                  before it, then writes its routed rows in ascending order;
//                  the last block writes n_routed.
// With at most 256 rows, one workgroup does both (route_small, route.cuh).
// The MFMA fallback needs only route_flags: its gate+up kernel builds the
// list from the mask itself (MaskRanks, route.cuh), one launch fewer.
#include "common.cuh"
#include "launch.h"
#include "route.cuh"

namespace sffn {

namespace {

constexpr int kBlock = 256;

constexpr int kFlagRows = 16;  // rows per workgroup of route_flags (4 per wave)

__global__ __launch_bounds__(kBlock) void route_flags(const uint16_t* __restrict__ count, int T,
                                                      int nt, int cap,
                                                      uint16_t* __restrict__ mask) {
  // wave w takes rows w, w + 4, ... of the workgroup's 16; for each row the
  // lanes read the tiles' counts side by side (coalesced), all four rows'
  // loads in flight together
  const int lane = lane_id(), w = threadIdx.x >> 6;
  constexpr int R = kFlagRows / 4;
  bool over[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int t = blockIdx.x * kFlagRows + u * 4 + w;
    over[u] = false;
    if (t < T)
      for (int k = lane; k < nt; k += kWave) over[u] |= (int)count[(size_t)t * nt + k] > cap;
  }
  __shared__ int wave_bits[kBlock / kWave];
  int bits = 0;
#pragma unroll
  for (int u = 0; u < R; ++u)
    if (__ballot(over[u]) != 0ull) bits |= 1 << (u * 4 + w);  // row u * 4 + w of the 16
  if (lane == 0) wave_bits[w] = bits;
  __syncthreads();
  if (threadIdx.x == 0)
    mask[blockIdx.x] = (uint16_t)((wave_bits[0] | wave_bits[1]) | (wave_bits[2] | wave_bits[3]));
}

__global__ __launch_bounds__(kBlock) void route_compact(const uint16_t* __restrict__ mask, int T,
                                                        int32_t* __restrict__ routed,
                                                        int32_t* __restrict__ n_routed) {
  __shared__ int wave_tot[kBlock / kWave];
  __shared__ int prefix_s;
  const int b = blockIdx.x;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  // routed rows before this block: the set bits of the words before it
  int acc = 0;
  for (int i = threadIdx.x; i < b * (kBlock / kFlagRows); i += kBlock)
    acc += __popc((uint32_t)mask[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if (lane == 0) wave_tot[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int p = 0;
    for (int i = 0; i < kBlock / kWave; ++i) p += wave_tot[i];
    prefix_s = p;
  }
  __syncthreads();
  const int prefix = prefix_s;
  __syncthreads();
  // in-block scan of the flags
  const int t = b * kBlock + threadIdx.x;
  const int f = (t < T) ? ((int)mask[t / kFlagRows] >> (t % kFlagRows)) & 1 : 0;
  const uint64_t m = __ballot(f);
  if (lane == 0) wave_tot[w] = __popcll(m);
  __syncthreads();
  int off = prefix;
  for (int i = 0; i < w; ++i) off += wave_tot[i];
  if (f) routed[off + lanes_below(m)] = t;
  if (b == (int)gridDim.x - 1 && threadIdx.x == kBlock - 1) {
    int tot = off;
    for (int i = w; i < kBlock / kWave; ++i) tot += wave_tot[i];
    *n_routed = tot;
  }
}

// T <= 256: one workgroup does both steps (one launch instead of two).
__global__ __launch_bounds__(kBlock) void route_small(const uint16_t* __restrict__ count, int T,
                                                      int nt, int cap, int32_t* __restrict__ routed,
                                                      int32_t* __restrict__ n_routed) {
  __shared__ int flag_s[kRouteBlock], rows_s[kRouteBlock], wave_tot[kRouteBlock / kWave];
  const int n = route_rows_lds(count, T, nt, cap, flag_s, rows_s, wave_tot);
  if ((int)threadIdx.x < n) routed[threadIdx.x] = rows_s[threadIdx.x];
  if (threadIdx.x == 0) *n_routed = n;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t route_workspace_bytes(int T) {
  return align256((size_t)route_mask_words(T) * 2);
}

int route_mask_words(int T) { return (T + kFlagRows - 1) / kFlagRows; }

hipError_t launch_route_mask(const uint16_t* count, int T, int n_tiles, int cap, uint16_t* mask,
                             hipStream_t stream) {
  hipLaunchKernelGGL(route_flags, dim3((unsigned)route_mask_words(T)), dim3(kBlock), 0, stream,
                     count, T, n_tiles, cap, mask);
  return hipGetLastError();
}

hipError_t launch_route(const uint16_t* count, int T, int n_tiles, int cap, int32_t* routed,
                        int32_t* n_routed, void* ws, hipStream_t stream) {
  if (T <= kBlock) {
    hipLaunchKernelGGL(route_small, dim3(1), dim3(kBlock), 0, stream, count, T, n_tiles, cap,
                       routed, n_routed);
    return hipGetLastError();
  }
  uint16_t* mask = (uint16_t*)ws;
  hipError_t e = launch_route_mask(count, T, n_tiles, cap, mask, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_compact, dim3((unsigned)((T + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                     stream, mask, T, routed, n_routed);
  return hipGetLastError();
}

}  // namespace sffn
