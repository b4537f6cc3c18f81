// Fused up(.)gate -> down over the TwELL nonzeros (pwwt.cn article, section
// 02: one pass computes the up projection only for the packed nonzeros,
// multiplies by the gate value and accumulates the down projection, so the
// intermediate h never goes to memory).
//
// Work item = (token t, column split s): one wavefront walks the live TwELL
// entries of tiles [s*nt/S, (s+1)*nt/S) of row t.  For each entry (j, h):
//   u  = x_t . wu_t[j]      16-byte loads of the wu_t row, lane-local dot,
//                           wave reduction
//   y += (h * u) * wd[j]    16-byte loads of the wd row, float32 FMA into the
//                           lane's slice of y_t held in registers
// With S == 1 the wave writes y_t once, rounded to dtype.  With S > 1 (few
// tokens) each split writes a float32 partial; the last split to finish a
// token (ticket counter) sums the partials in split order and writes y_t, so
// the result does not depend on timing.  The tickets are cleared by a small
// kernel at the start of every call: the workspace carries nothing from one
// call to the next.
// Rows with any tile over capacity are skipped (the hybrid route owns them).
#include "common.cuh"
#include "launch.h"

namespace sffn {

namespace {

struct SparseArgs {
  const void* x;
  const void* wu;
  const void* wd;
  const uint16_t* count;
  const uint16_t* idx;
  const void* val;
  void* y;
  int* tickets;    // [T], S > 1 only
  float* partial;  // [S, T, K], S > 1 only
  int T, K, nt, cap, S;
};

template <typename T, int NCH>
__global__ __launch_bounds__(256) void sparse_updown(SparseArgs a) {
  constexpr int E = Elt<T>::kPerChunk;
  const int lane = lane_id();
  const int item = uniform((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int t = item / a.S;
  const int s = item - t * a.S;
  if (t >= a.T) return;
  const uint16_t* cnt_row = a.count + (size_t)t * a.nt;

  // routed row?  (any tile over capacity)
  bool over = false;
  for (int k = lane; k < a.nt; k += kWave) over |= (int)cnt_row[k] > a.cap;
  if (__ballot(over) != 0ull) return;

  const int nch = a.K / E;  // 16-byte chunks per row
  const T* xrow = (const T*)a.x + (size_t)t * a.K;
  float xv[NCH][E];
  float yv[NCH][E];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + kWave * c;
    if (ch < nch) {
      Elt<T>::unpack(ldg16(xrow + (size_t)ch * E), xv[c]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) xv[c][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) yv[c][e] = 0.f;
  }

  const int k_lo = (int)(((long)s * a.nt) / a.S);
  const int k_hi = (int)(((long)(s + 1) * a.nt) / a.S);
  const T* wu = (const T*)a.wu;
  const T* wd = (const T*)a.wd;
  for (int k = k_lo; k < k_hi; ++k) {
    const int n = min((int)cnt_row[k], a.cap);
    const size_t base = ((size_t)t * a.nt + k) * a.cap;
    for (int e = 0; e < n; ++e) {
      const int j = uniform((int)a.idx[base + e]);
      if (j >= a.nt * 128) continue;  // never true for a TwELL written by twell_pack
      const float h = Elt<T>::load1(a.val, base + e);
      const T* urow = wu + (size_t)j * a.K;
      const T* drow = wd + (size_t)j * a.K;
      u32x4_t ur[NCH], dr[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int ch = lane + kWave * c;
        ur[c] = ch < nch ? ldg16(urow + (size_t)ch * E) : u32x4_t{0u, 0u, 0u, 0u};
        dr[c] = ch < nch ? ldg16(drow + (size_t)ch * E) : u32x4_t{0u, 0u, 0u, 0u};
      }
      float p = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float uf[E];
        Elt<T>::unpack(ur[c], uf);
#pragma unroll
        for (int q = 0; q < E; ++q) p = fmaf(xv[c][q], uf[q], p);
      }
      const float g = h * wave_sum(p);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float df[E];
        Elt<T>::unpack(dr[c], df);
#pragma unroll
        for (int q = 0; q < E; ++q) yv[c][q] = fmaf(g, df[q], yv[c][q]);
      }
    }
  }

  if (a.S == 1) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + kWave * c;
      if (ch < nch)
#pragma unroll
        for (int q = 0; q < E; ++q) Elt<T>::store1(a.y, (size_t)t * a.K + (size_t)ch * E + q, yv[c][q]);
    }
    return;
  }

  // split partial, then the last split of this token reduces in split order
  float* prow = a.partial + ((size_t)s * a.T + t) * a.K;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + kWave * c;
    if (ch < nch) {
#pragma unroll
      for (int q = 0; q < E; q += 4)
        *(float4*)(prow + (size_t)ch * E + q) = make_float4(yv[c][q], yv[c][q + 1], yv[c][q + 2], yv[c][q + 3]);
    }
  }
  __threadfence();
  int ticket = 0;
  if (lane == 0) ticket = atomicAdd(a.tickets + t, 1);
  ticket = __shfl(ticket, 0, kWave);
  if (ticket != a.S - 1) return;
  __threadfence();
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int q = 0; q < E; ++q) yv[c][q] = 0.f;
  for (int ss = 0; ss < a.S; ++ss) {
    const float* pr = a.partial + ((size_t)ss * a.T + t) * a.K;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + kWave * c;
      if (ch < nch) {
#pragma unroll
        for (int q = 0; q < E; q += 4) {
          const float4 v = *(const float4*)(pr + (size_t)ch * E + q);
          yv[c][q] += v.x; yv[c][q + 1] += v.y; yv[c][q + 2] += v.z; yv[c][q + 3] += v.w;
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + kWave * c;
    if (ch < nch)
#pragma unroll
      for (int q = 0; q < E; ++q) Elt<T>::store1(a.y, (size_t)t * a.K + (size_t)ch * E + q, yv[c][q]);
  }
}

__global__ void clear_tickets(int* tickets, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) tickets[i] = 0;
}

// Many tokens (prefill): one token per wave, WAVES tokens per workgroup.  The
// waves of a workgroup walk the column tiles in windows of kWinTiles tiles and
// meet at a barrier after each window, so the workgroups resident on one XCD
// sweep the weight rows in near lockstep and the rows they share are served
// from that XCD's L2 rather than from the last-level cache or HBM.  Per
// window, a wave first lists its live entries (lane-parallel, in LDS), then
// processes them two at a time so that four row loads are in flight:
//   u = x_t . wu_t[j] with packed bf16 dot2, uniform DPP reduction;
//   y_t += (h * u) * wd[j] in float32 registers.
constexpr int kWinTiles = 4;

template <int NCH, int WAVES, bool FULL>
__global__ __launch_bounds__(WAVES * 64) void sparse_updown_win(SparseArgs a) {
  constexpr int E = 8;  // bf16 per 16-byte chunk
  constexpr int LIST = kWinTiles * 128;  // upper bound of live entries per window (cap <= 128)
  __shared__ uint32_t list_j[WAVES][kWinTiles * 32];
  __shared__ float list_h[WAVES][kWinTiles * 32];
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int t = uniform((int)(blockIdx.x * WAVES + w));
  const int nch = a.K / E;
  bool active = t < a.T;
  const uint16_t* cnt_row = a.count + (size_t)(active ? t : 0) * a.nt;
  if (active) {
    bool over = false;
    for (int k = lane; k < a.nt; k += kWave) over |= (int)cnt_row[k] > a.cap;
    active = __ballot(over) == 0ull;
  }
  u32x4_t xr[NCH];
  float yv[NCH][E];
  const uint16_t* xrow = (const uint16_t*)a.x + (size_t)(active ? t : 0) * a.K;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + kWave * c;
    xr[c] = (active && (FULL || ch < nch)) ? ldg16(xrow + (size_t)ch * E) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < E; ++e) yv[c][e] = 0.f;
  }
  const uint16_t* wu = (const uint16_t*)a.wu;
  const uint16_t* wd = (const uint16_t*)a.wd;
  const int cap = a.cap;
  const int per_win = kWinTiles * cap;  // slots examined per window (<= LIST)
  (void)LIST;
  for (int k0 = 0; k0 < a.nt; k0 += kWinTiles) {
    if (active) {
      // lane-parallel listing of the window's live entries (ascending column)
      int n = 0;
      for (int base = 0; base < per_win; base += kWave) {
        const int slot = base + lane;
        const int k = k0 + slot / (cap > 0 ? cap : 1);
        const int ss = cap > 0 ? slot % cap : 0;
        bool live = false;
        uint32_t j = 0;
        float h = 0.f;
        if (cap > 0 && slot < per_win && k < a.nt) {
          const int c = min((int)cnt_row[k], cap);
          if (ss < c) {
            const size_t off = ((size_t)t * a.nt + k) * cap + ss;
            j = a.idx[off];
            h = bf16_to_f32(((const uint16_t*)a.val)[off]);
            live = j < (uint32_t)(a.nt * 128);
          }
        }
        const uint64_t m = __ballot(live);
        if (live) {
          const int pos = n + lanes_below(m);
          if (pos < kWinTiles * 32) { list_j[w][pos] = j; list_h[w][pos] = h; }
        }
        n += __popcll(m);
      }
      n = min(n, kWinTiles * 32);
      __builtin_amdgcn_wave_barrier();
      // Entries go in pairs: the down projection of a pair is one packed
      // dot2 per output element, y += (wd_j0, wd_j1) . (g0, g1), with g split
      // into a bf16 high part and a bf16 remainder (two dot2) so that the
      // pair costs as much as one float32 FMA pass while keeping about 16
      // significant bits of g.  The wu row of the next entry is in flight
      // while the current one is reduced.
      u32x4_t ur[NCH], dr0[NCH], dr1[NCH];
      auto load_row = [&](u32x4_t* dst, const uint16_t* row) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const int ch = lane + kWave * c;
          dst[c] = (FULL || ch < nch) ? ldg16(row + (size_t)ch * E) : u32x4_t{0u, 0u, 0u, 0u};
        }
      };
      auto dot_x = [&](const u32x4_t* r) {
        float p = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          p = dot2_bf16(xr[c].x, r[c].x, p);
          p = dot2_bf16(xr[c].y, r[c].y, p);
          p = dot2_bf16(xr[c].z, r[c].z, p);
          p = dot2_bf16(xr[c].w, r[c].w, p);
        }
        return p;
      };
      auto row_j = [&](int i) { return wu + (size_t)uniform((int)list_j[w][i]) * a.K; };
      auto drow_j = [&](int i) { return wd + (size_t)uniform((int)list_j[w][i]) * a.K; };
      if (n > 0) load_row(ur, row_j(0));
      int i = 0;
      for (; i + 1 < n; i += 2) {
        // the waves with the most entries left set the window's length (the
        // others wait at its barrier): they issue first
        {
          const int rem = n - i;
          if (rem >= 8) __builtin_amdgcn_s_setprio(3);
          else if (rem >= 5) __builtin_amdgcn_s_setprio(2);
          else if (rem >= 3) __builtin_amdgcn_s_setprio(1);
          else __builtin_amdgcn_s_setprio(0);
        }
        const float h0 = list_h[w][i], h1 = list_h[w][i + 1];
        load_row(dr0, drow_j(i));
        const float p0 = dot_x(ur);
        load_row(ur, row_j(i + 1));
        const float g0 = h0 * wave_sum_uniform(p0);
        load_row(dr1, drow_j(i + 1));
        const float p1 = dot_x(ur);
        if (i + 2 < n) load_row(ur, row_j(i + 2));
        const float g1 = h1 * wave_sum_uniform(p1);
        const uint32_t gh0 = f32_to_bf16(g0), gh1 = f32_to_bf16(g1);
        const uint32_t gl0 = f32_to_bf16(g0 - bf16_to_f32((uint16_t)gh0));
        const uint32_t gl1 = f32_to_bf16(g1 - bf16_to_f32((uint16_t)gh1));
        const uint32_t gh = gh0 | (gh1 << 16), gl = gl0 | (gl1 << 16);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint32_t a4[4] = {dr0[c].x, dr0[c].y, dr0[c].z, dr0[c].w};
          const uint32_t b4[4] = {dr1[c].x, dr1[c].y, dr1[c].z, dr1[c].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = __builtin_amdgcn_perm(b4[q], a4[q], 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(b4[q], a4[q], 0x07060302u);
            yv[c][2 * q] = dot2_bf16(lo, gl, dot2_bf16(lo, gh, yv[c][2 * q]));
            yv[c][2 * q + 1] = dot2_bf16(hi, gl, dot2_bf16(hi, gh, yv[c][2 * q + 1]));
          }
        }
      }
      if (i < n) {  // odd count: last entry alone, float32 FMA
        const float h = list_h[w][i];
        load_row(dr0, drow_j(i));
        const float g = h * wave_sum_uniform(dot_x(ur));
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          float f[E];
          Elt<uint16_t>::unpack(dr0[c], f);
#pragma unroll
          for (int e = 0; e < E; ++e) yv[c][e] = fmaf(g, f[e], yv[c][e]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
  }
  if (!active) return;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + kWave * c;
    if (ch < nch) {
      u32x4_t o;
      o.x = (uint32_t)f32_to_bf16(yv[c][0]) | ((uint32_t)f32_to_bf16(yv[c][1]) << 16);
      o.y = (uint32_t)f32_to_bf16(yv[c][2]) | ((uint32_t)f32_to_bf16(yv[c][3]) << 16);
      o.z = (uint32_t)f32_to_bf16(yv[c][4]) | ((uint32_t)f32_to_bf16(yv[c][5]) << 16);
      o.w = (uint32_t)f32_to_bf16(yv[c][6]) | ((uint32_t)f32_to_bf16(yv[c][7]) << 16);
      *(u32x4_t*)((uint16_t*)a.y + (size_t)t * a.K + (size_t)ch * E) = o;
    }
  }
}

// Few tokens (bf16): two passes, so that every pass has thousands of
// independent row loads in flight instead of one token's chain per wave.
// Both passes take a group of consecutive TwELL tiles per wavefront with one
// lane per slot (lane l: slot l % cap of tile k0 + l / cap), and load every
// slot's count, index and value speculatively in one round trip (slots past
// the count are in bounds and ignored), so a wave waits for memory twice: once
// for the slot metadata, once per batch of weight rows.
//
// Pass 1 (sparse_up_pass): for each live entry (t, k, s),
//   a[t, k, s] = val * (x_t . wu_t[j])   in float32, into the workspace.
// x_t stays in registers (16-byte chunks); up to kUpBatch wu_t rows are read
// at once, then reduced with packed bf16 dot2 and DPP.  Entries of routed rows
// are computed too (they are rare and pass 2 ignores them), which saves the
// row scan.
//
// Pass 2 (sparse_down_pass): y[t, c0 .. c0 + 512) = sum over the token's live
// entries of a * wd[j, c0 .. c0 + 512).  Workgroup = (token, 512-column
// chunk), its kDownWaves waves take every kDownWaves-th tile group; each lane
// owns 8 output columns (one 16-byte load per entry row, kDownInflight rows in
// flight), the partial chunks are summed in LDS in wave order and written
// once, rounded.  Rows with every count 0 get y = 0; routed rows are left
// alone.  No atomics: deterministic.
struct TwoPassArgs {
  const uint16_t* x;
  const uint16_t* wu;
  const uint16_t* wd;
  const uint16_t* count;
  const uint16_t* idx;
  const uint16_t* val;
  uint16_t* y;
  float* acts;  // [T, nt, cap]
  int T, K, nt, cap;
};

constexpr int kUpSlots = 16;  // slots per wave in pass 1 (<= 64)
constexpr int kUpBatch = 4;   // wu_t rows in flight per wave

// Tiles per group for a given number of lanes: whole tiles, at least one.
__host__ __device__ inline int tiles_per_group(int lanes, int cap) {
  return cap >= lanes ? 1 : lanes / cap;
}

// One lane per slot of tiles [k_first, k_first + G): live flag, column, slot offset.
struct SlotMeta {
  bool live;
  int j;
  size_t off;
};

__device__ __forceinline__ SlotMeta slot_meta(const TwoPassArgs& a, int t, int k_first, int G,
                                              int q) {
  SlotMeta m{false, 0, 0};
  const int cap = a.cap;
  const int k = k_first + q / cap;
  const int ss = q - (q / cap) * cap;
  if (q < G * cap && k < a.nt) {
    m.off = ((size_t)t * a.nt + k) * cap + ss;
    const int c = a.count[(size_t)t * a.nt + k];
    m.j = a.idx[m.off];
    m.live = ss < min(c, cap) && m.j < a.nt * 128;
  }
  return m;
}

template <int NCH>
__global__ __launch_bounds__(256) void sparse_up_pass(TwoPassArgs a, int groups) {
  constexpr int E = 8;
  const int lane = lane_id();
  const int item = uniform((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int t = item / groups;
  const int gi = item - t * groups;
  if (t >= a.T) return;
  const int cap = a.cap;
  const int G = tiles_per_group(kUpSlots, cap);
  const int nch = a.K / E;
  const uint16_t* xrow = a.x + (size_t)t * a.K;
  u32x4_t xr[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + kWave * c;
    xr[c] = ch < nch ? ldg16(xrow + (size_t)ch * E) : u32x4_t{0u, 0u, 0u, 0u};
  }
  for (int base = 0; base < G * cap; base += kUpSlots) {
    const int q = base + lane;
    const SlotMeta sm = lane < kUpSlots ? slot_meta(a, t, gi * G, G, q) : SlotMeta{false, 0, 0};
    // value loaded with the slot's count and index (one round trip), used if live
    const float hv = bf16_to_f32(a.val[sm.off]);
    const float h = sm.live ? hv : 0.f;
    uint64_t m = __ballot(sm.live);
    while (m) {
      int es[kUpBatch];
      u32x4_t r[kUpBatch][NCH];
#pragma unroll
      for (int u = 0; u < kUpBatch; ++u) {
        es[u] = -1;
        if (m) {
          es[u] = __builtin_ctzll(m);
          m &= m - 1;
          const uint16_t* row = a.wu + (size_t)__builtin_amdgcn_readlane(sm.j, es[u]) * a.K;
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            const int ch = lane + kWave * c;
            r[u][c] = ch < nch ? ldg16(row + (size_t)ch * E) : u32x4_t{0u, 0u, 0u, 0u};
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kUpBatch; ++u) {
        if (es[u] < 0) break;
        float p = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          p = dot2_bf16(xr[c].x, r[u][c].x, p);
          p = dot2_bf16(xr[c].y, r[u][c].y, p);
          p = dot2_bf16(xr[c].z, r[u][c].z, p);
          p = dot2_bf16(xr[c].w, r[u][c].w, p);
        }
        p = wave_sum_uniform(p);
        if (lane == es[u]) a.acts[sm.off] = h * p;
      }
    }
  }
}

constexpr int kDownCols = 512;  // output columns per workgroup of pass 2
constexpr int kDownWaves = 8;   // waves per workgroup of pass 2
constexpr int kDownInflight = 8;  // wd row loads in flight per wave

__global__ __launch_bounds__(kDownWaves * 64) void sparse_down_pass(TwoPassArgs a, int groups,
                                                                    int chunks) {
  __shared__ f32x4_t red[kDownWaves - 1][2][64];
  __shared__ int routed_flag;
  const int lane = lane_id();
  const int w = uniform((int)(threadIdx.x >> 6));
  const int t = (int)blockIdx.x / chunks;
  const int cc = (int)blockIdx.x - t * chunks;
  const int cap = a.cap;
  // routed row?  (wave 0 scans the counts while the others start their slots)
  if (w == 0) {
    bool over = false;
    for (int k = lane; k < a.nt; k += kWave) over |= (int)a.count[(size_t)t * a.nt + k] > cap;
    const bool any = __ballot(over) != 0ull;
    if (lane == 0) routed_flag = any;
  }
  const int col = cc * kDownCols + 8 * lane;
  const bool cok = col < a.K;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = 0.f;
  const int G = cap > 0 ? tiles_per_group(kWave, cap) : 1;
  for (int gi = w; gi < groups && cap > 0; gi += kDownWaves) {
    for (int base = 0; base < G * cap; base += kWave) {
      const SlotMeta sm = slot_meta(a, t, gi * G, G, base + lane);
      // activation loaded with the slot's count and index (one round trip);
      // slots that are not live hold stale workspace values and are masked
      const float gv = a.acts[sm.off];
      const float g = sm.live ? gv : 0.f;
      uint64_t m = __ballot(sm.live);
      while (m) {
        int es[kDownInflight];
        u32x4_t d[kDownInflight];
#pragma unroll
        for (int u = 0; u < kDownInflight; ++u) {
          es[u] = -1;
          if (m) {
            es[u] = __builtin_ctzll(m);
            m &= m - 1;
            const int jj = __builtin_amdgcn_readlane(sm.j, es[u]);
            d[u] = cok ? ldg16(a.wd + (size_t)jj * a.K + col) : u32x4_t{0u, 0u, 0u, 0u};
          }
        }
#pragma unroll
        for (int u = 0; u < kDownInflight; ++u) {
          if (es[u] < 0) break;
          const float gg = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g), es[u]));
          float f[8];
          Elt<uint16_t>::unpack(d[u], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = fmaf(gg, f[e], y[e]);
        }
      }
    }
  }
  if (w > 0) {
    red[w - 1][0][lane] = f32x4_t{y[0], y[1], y[2], y[3]};
    red[w - 1][1][lane] = f32x4_t{y[4], y[5], y[6], y[7]};
  }
  __syncthreads();
  if (w != 0 || !cok || routed_flag) return;
#pragma unroll
  for (int v = 0; v < kDownWaves - 1; ++v) {
    const f32x4_t lo = red[v][0][lane], hi = red[v][1][lane];
    y[0] += lo.x; y[1] += lo.y; y[2] += lo.z; y[3] += lo.w;
    y[4] += hi.x; y[5] += hi.y; y[6] += hi.z; y[7] += hi.w;
  }
  u32x4_t o;
  o.x = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(y[4]) | ((uint32_t)f32_to_bf16(y[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(y[6]) | ((uint32_t)f32_to_bf16(y[7]) << 16);
  *(u32x4_t*)(a.y + (size_t)t * a.K + col) = o;
}

hipError_t launch_two_pass(const SparseArgs& s, float* acts, hipStream_t stream) {
  TwoPassArgs a{(const uint16_t*)s.x, (const uint16_t*)s.wu, (const uint16_t*)s.wd, s.count,
                s.idx, (const uint16_t*)s.val, (uint16_t*)s.y, acts, s.T, s.K, s.nt, s.cap};
  if (s.cap > 0) {
    const int G = tiles_per_group(kUpSlots, s.cap);
    const int groups = (s.nt + G - 1) / G;
    const dim3 grid((unsigned)((s.T * groups + 3) / 4));
    const int nch = (s.K / 8 + 63) / 64;
    if (nch <= 1) hipLaunchKernelGGL(sparse_up_pass<1>, grid, dim3(256), 0, stream, a, groups);
    else if (nch <= 2) hipLaunchKernelGGL(sparse_up_pass<2>, grid, dim3(256), 0, stream, a, groups);
    else if (nch <= 4) hipLaunchKernelGGL(sparse_up_pass<4>, grid, dim3(256), 0, stream, a, groups);
    else if (nch <= 8) hipLaunchKernelGGL(sparse_up_pass<8>, grid, dim3(256), 0, stream, a, groups);
    else hipLaunchKernelGGL(sparse_up_pass<16>, grid, dim3(256), 0, stream, a, groups);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int G = s.cap > 0 ? tiles_per_group(kWave, s.cap) : 1;
  const int groups = (s.nt + G - 1) / G;
  const int chunks = (s.K + kDownCols - 1) / kDownCols;
  hipLaunchKernelGGL(sparse_down_pass, dim3((unsigned)(s.T * chunks)), dim3(kDownWaves * 64), 0,
                     stream, a, groups, chunks);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const SparseArgs& a, int nch_per_lane, hipStream_t stream) {
  const int items = a.T * a.S;
  const dim3 grid((unsigned)((items + 3) / 4));
  switch (nch_per_lane) {
    case 1: hipLaunchKernelGGL((sparse_updown<T, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((sparse_updown<T, 2>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((sparse_updown<T, 4>), grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((sparse_updown<T, 8>), grid, dim3(256), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((sparse_updown<T, 16>), grid, dim3(256), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((sparse_updown<T, 32>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NCH, int WAVES>
void launch_win(const SparseArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.T + WAVES - 1) / WAVES)), block(WAVES * 64);
  if (a.K == NCH * 64 * 8) hipLaunchKernelGGL((sparse_updown_win<NCH, WAVES, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((sparse_updown_win<NCH, WAVES, false>), grid, block, 0, stream, a);
}

hipError_t launch_window(const SparseArgs& a, int nch, hipStream_t stream) {
  switch (nch) {
    case 1: launch_win<1, 16>(a, stream); break;
    case 2: launch_win<2, 16>(a, stream); break;
    case 4: launch_win<4, 16>(a, stream); break;
    case 8: launch_win<8, 8>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace

// bf16 with few tokens takes the two-pass kernels.
static bool use_two_pass(int dtype, int T) { return dtype == 1 && T <= 256; }

int sparse_splits(int T, int n_tiles, int /*d_model*/) {
  // enough wavefronts to cover the chip (~2048) when there are few tokens
  if (T <= 0) return 1;
  int s = (2048 + T - 1) / T;
  if (s > n_tiles) s = n_tiles;
  if (s > 64) s = 64;
  return s < 1 ? 1 : s;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t sparse_workspace_bytes(int dtype, int T, int n_tiles, int d_model, int cap) {
  if (use_two_pass(dtype, T)) return align256((size_t)T * n_tiles * (size_t)cap * 4);
  const int S = sparse_splits(T, n_tiles, d_model);
  if (S <= 1) return 0;
  return align256((size_t)T * 4) + (size_t)S * T * d_model * 4;
}

hipError_t launch_sparse_updown(int dtype, const void* x, const void* wu_t, const void* wd,
                                const uint16_t* count, const uint16_t* idx, const void* val,
                                void* y, void* ws, int T, int K, int n_tiles, int cap,
                                hipStream_t stream) {
  if (use_two_pass(dtype, T)) {
    SparseArgs a{x, wu_t, wd, count, idx, val, y, nullptr, nullptr, T, K, n_tiles, cap, 1};
    return launch_two_pass(a, (float*)ws, stream);
  }
  const int S = sparse_splits(T, n_tiles, K);
  SparseArgs a{x, wu_t, wd, count, idx, val, y, nullptr, nullptr, T, K, n_tiles, cap, S};
  if (S > 1) {
    a.tickets = (int*)ws;
    a.partial = (float*)((char*)ws + align256((size_t)T * 4));
    hipLaunchKernelGGL(clear_tickets, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream,
                       a.tickets, T);
  }
  if (dtype == 1) {
    const int nch = pow2_at_least((K / 8 + 63) / 64);
    if (S == 1 && cap <= 32 && nch <= 8) return launch_window(a, nch, stream);
    return launch_typed<uint16_t>(a, nch, stream);
  }
  return launch_typed<float>(a, pow2_at_least((K / 4 + 63) / 64), stream);
}

}  // namespace sffn
