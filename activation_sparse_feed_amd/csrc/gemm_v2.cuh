// Second-generation bf16 GEMM main loop for gfx950 (K-contiguous A and B).
//
//   workgroup tile BM (128 or 256) x BN (NB B matrices of BNW columns; 128, or
//   256 for one B), NWAVES waves as WAVES_M x WAVES_N, each wave WM x WN per B
//   matrix; v_mfma_f32_16x16x32_bf16, float32 accumulators.
//   K step BK (32 or 64), STAGES LDS stages filled by buffer loads straight into
//   LDS (16 bytes per lane, no VGPR staging).  Each LDS row of BK bf16 holds its
//   16-byte chunks XOR-swizzled by row (slot): a load instruction writes 64
//   consecutive chunks, so lane l fetches the global chunk that lands in its
//   slot; fragment reads of consecutive rows then hit distinct bank groups.
//   Rows past the valid range read as zero through the buffer range check.
//   One barrier per K step: stage kt is consumed while the later stages are in
//   flight.
//
// NORMS: the waves also accumulate sum of squares of the A rows (waves with
// wn == 0) and B rows (waves with wm == 0) from the bf16 fragments they feed to
// the MFMA (packed dot2), for the guard band of the TwELL epilogue.
#pragma once

#include "common.cuh"

namespace sffn {

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}


// Workgroup barrier for the LDS pipeline: waits for this wave's LDS
// instructions, then s_barrier.  Unlike __syncthreads() it does not drain the
// vector-memory counter, so buffer loads into later LDS stages stay in flight;
// the caller waits for its own stage with s_waitcnt vmcnt first.
// Written with builtins (not inline asm) so that the compiler's own wait
// insertion sees the lgkmcnt(0) and does not add a second wait before the
// next MFMAs.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Byte offset of an LDS pointer (LDS addresses are 32-bit).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Tile of a linear workgroup id.  Workgroups are dispatched round-robin over
// the 8 XCDs (id % 8); each XCD is given a contiguous run of tile indices, and
// tile indices walk groups of 4 M-tiles with N fastest inside a group, so the
// workgroups resident on one XCD share A and B tiles in its L2.  Any mapping
// is correct; this one only affects cache reuse.
__device__ __forceinline__ void tile_of(int bid, int mt, int nt, int* m, int* n) {
  const int total = mt * nt;
  const int xcd = bid & 7, j = bid >> 3;
  const int per = total >> 3, extra = total & 7;
  const int t = xcd * per + min(xcd, extra) + j;  // contiguous run per XCD
  constexpr int GM = 4;
  const int group = t / (GM * nt);
  const int gm = min(GM, mt - group * GM);
  const int r = t - group * GM * nt;
  *m = group * GM + r % gm;
  *n = r / gm;
}

// WAVES_N: waves along N (2: 2 x 2 waves of 128 rows x BNW/2 columns; 1: 4 x 1
// waves of 64 rows x BNW columns, so that every row of a B matrix's tile lives
// in one wave).
// B_KN: the single B matrix is [K, N] (N-contiguous, e.g. the down projection
// weight).  Its K step is staged as BK rows of BNW columns (256 or 512 bytes),
// with 16-byte chunks XOR-swizzled by row (kn_slot); MFMA B fragments are read
// with the gfx950 transposing LDS read, which hands each lane four consecutive
// k of one column per 8-byte read.
template <int NB, int BNW, bool NORMS, int BK_ = 32, int WAVES_N = 2, bool B_KN = false,
          int BM_ = 256, int STAGES_ = 3, int NWAVES_ = 4, bool INTERLEAVE = false>
struct Gemm2 {
  static constexpr int BM = BM_, BK = BK_, STAGES = STAGES_, NWAVES = NWAVES_;
  static constexpr int BN = NB * BNW;
  static constexpr int ROWB = BK * 2;                  // bytes per LDS row
  static constexpr int CPR = BK / 8;                   // 16-byte chunks per row
  static constexpr int ROWS = BM + BN;                 // LDS rows per stage
  static constexpr int STAGE_BYTES = ROWS * ROWB;
  static constexpr int RPB = 64 / CPR;                 // rows per 1 KB load block
  static constexpr int BLOCKS = ROWS / RPB;            // 1 KB load blocks per stage
  static constexpr int LOADS = BLOCKS / NWAVES;        // load instructions per wave per stage
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(!NORMS || WAVES_N == 2, "norm split assumes 2 x 2 waves");
  static_assert(!B_KN || (NB == 1 && (BNW == 128 || BNW == 256) && BK == 32 && !NORMS),
                "K-major B layout");
  static constexpr int KN_ROWB = BNW * 2;   // bytes per staged k row of a [K, N] B
  static constexpr int KN_CPR = KN_ROWB / 16;  // 16-byte chunks per staged k row
  // 16-byte chunk q of staged k row k sits at chunk q ^ 2 c(k), c(k) = bits 0, 1 and 3 of k:
  // the rows one transposing read touches at a time (k = 8 g + 0..3, g = 0, 1,
  // or those + 4) land in 16 distinct chunks modulo 16, so no two lanes share a
  // bank (the row length is a multiple of the 256 bytes of the 64 banks).
  static __device__ __forceinline__ int kn_slot(int k, int q) {
    return q ^ (2 * ((k & 3) | ((k >> 1) & 4)));
  }
  static constexpr int WAVES_M = NWAVES / WAVES_N, WAVE_COLS = WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BNW / WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE_BYTES;
  static_assert(BN == 128 || BN == 256, "workgroup N tile");
  static_assert(BM == 256 || BM == 128 || BM == 64 || BM == 32, "workgroup M tile");
  static_assert(BLOCKS % NWAVES == 0, "load blocks per wave");
  static_assert(!NORMS || NWAVES == 4, "norm split assumes 4 waves");

  // Physical 16-byte slot of logical chunk q in row r: 8 consecutive rows
  // read at one logical chunk land in 8 distinct 16-byte bank groups.
  static __device__ __forceinline__ int slot(int r, int q) {
    return BK == 64 ? (q ^ (r & 7)) : (q ^ ((r >> 1) & 3));
  }

  f32x4_t acc[NB][FM][FN];
  float sqa[FM];
  float sqb[NB][FN];
  uint32_t voff[LOADS];     // per-lane byte offset of its chunk within the source matrix
  __amdgpu_buffer_rsrc_t ra;
  __amdgpu_buffer_rsrc_t rb[NB];
  int b_ld;  // B_KN: bytes per row of B
  __amdgpu_buffer_rsrc_t rw;  // WAVE_ALIGNED: the matrix this wave's load blocks come from
  int kstride;  // WAVE_ALIGNED and B_KN: bytes per K element in that matrix (2, or b_ld)

  // A: [*, K] bf16 rows; rows m0 .. m0+255 (gathered through rowmap when
  // given); rows >= m_valid read as zero.  B[b]: [N, K] bf16; rows n0 ..
  // K is the length of the K loop.  lda (0: K) is the row stride in elements
  // of A and of a K-contiguous B; a_skip is the number of elements of each A
  // row before A (a split of a longer K range starts inside the rows).
  // zero: clear the accumulators (false: a further K range adds to them).
  __device__ __forceinline__ void init(const uint16_t* A, size_t a_rows_total, const int* rowmap,
                                       int m0, int m_valid, const uint16_t* const* B, int n0,
                                       int N, int K, int lda = 0, int a_skip = 0,
                                       bool zero = true) {
    const int lane = lane_id();
    const int w = uniform((int)(threadIdx.x >> 6));
    const int ldk = lda > 0 ? lda : K;
    const uint32_t ld = (uint32_t)ldk * 2u;
    const uint16_t* abase = rowmap ? A : A + (size_t)m0 * ldk;
    const size_t a_rows = rowmap ? a_rows_total : (size_t)min(m_valid - m0, BM);
    ra = make_rsrc(abase, (uint32_t)(a_rows * ld - (size_t)a_skip * 2));
    if (B_KN) {
      b_ld = N * 2;
      rb[0] = make_rsrc(B[0] + n0, (uint32_t)((size_t)K * N * 2 - (size_t)n0 * 2));
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        // a 256-wide tile may hang over the end of B by 128 rows: those read as zero
        const int rows = BNW > 128 ? min(BNW, N - n0) : BNW;
        rb[b] = make_rsrc(B[b] + (size_t)n0 * ldk, (uint32_t)(rows * ld));
      }
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int blk = w * LOADS + i;
      const int row = blk * RPB + lane / CPR;
      const int q = slot(row, lane % CPR);  // slot is an involution: physical -> logical
      if (blk * RPB < BM) {
        const int m = m0 + row;
        uint32_t off = 0x80000000u;  // beyond any buffer: reads as zero
        if (m < m_valid) off = (uint32_t)((rowmap ? (uint32_t)rowmap[m] : (uint32_t)row) * ld);
        voff[i] = off + (uint32_t)q * 16u;
      } else if (!B_KN) {
        const int rb_ = row - BM;
        voff[i] = (uint32_t)(rb_ % BNW) * ld + (uint32_t)q * 16u;
      } else {
        // B block bb = blk - BM/RPB covers the 1024 / KN_ROWB k rows from
        // bb * 1024 / KN_ROWB on; lane l lands in physical chunk l % KN_CPR
        const int bb = blk - BM / RPB;
        const int kk = (1024 / KN_ROWB) * bb + lane / KN_CPR;
        const int qq = kn_slot(kk, lane % KN_CPR);
        voff[i] = (uint32_t)kk * (uint32_t)b_ld + (uint32_t)qq * 16u;
      }
    }
    if constexpr (WAVE_ALIGNED) {
      const int blk0 = w * LOADS;
      rw = blk0 * RPB < BM ? ra : ((NB == 1 || (blk0 * RPB - BM) < BNW) ? rb[0] : rb[NB - 1]);
      kstride = (B_KN && blk0 * RPB >= BM) ? b_ld : 2;
    }
    if (!zero) return;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[b][fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) sqa[fm] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) sqb[b][fn] = 0.f;
  }

  // Every load block of a wave comes from the same matrix (chosen once per
  // wave, a uniform branch around whole loops: no per-load descriptor select).
  static constexpr bool WAVE_ALIGNED =
      (BM / RPB) % LOADS == 0 && (BNW / RPB) % LOADS == 0 && (!B_KN || BM == 256);

  __device__ __forceinline__ void issue(uint8_t* stage, int k0) {
    const int w = uniform((int)(threadIdx.x >> 6));
    const int soff = (WAVE_ALIGNED && B_KN) ? k0 * kstride : k0 * 2;
    if constexpr (WAVE_ALIGNED) {
      // the wave's descriptor was chosen once in init: no branch here, so the
      // loads can be scheduled among the MFMAs of the step
      lds_void_t* dst0 = (lds_void_t*)(stage + w * LOADS * 1024);
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)((uint8_t*)dst0 + i * 1024), 16,
                                                 voff[i], soff, 0, 0);
      return;
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int blk = w * LOADS + i;  // wave-uniform
      lds_void_t* dst = (lds_void_t*)(stage + blk * 1024);
      if (blk * RPB < BM) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, voff[i], soff, 0, 0);
      } else if (B_KN) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb[0], dst, 16, voff[i], k0 * b_ld, 0, 0);
      } else if (NB == 1 || (blk * RPB - BM) < BNW) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb[0], dst, 16, voff[i], soff, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb[NB - 1], dst, 16, voff[i], soff, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void compute(const uint8_t* stage) {
    const int lane = lane_id();
    const int w = uniform((int)(threadIdx.x >> 6));
    const int wm = w % WAVES_M, wn = w / WAVES_M;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      // rows of every fragment start at a multiple of 16, so the swizzle only
      // depends on the lane's row within the fragment
      const int cq = slot(lane & 15, ks * 4 + (lane >> 4)) * 16;
      bf16x8_t af[FM], bfr[NB][FN];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int r = BM + b * BNW + wn * WN + fn * 16 + (lane & 15);
          bfr[b][fn] = *(const bf16x8_t*)(stage + r * ROWB + cq);
        }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = wm * WM + fm * 16 + (lane & 15);
        af[fm] = *(const bf16x8_t*)(stage + r * ROWB + cq);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[b][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[b][fn],
                                                                    acc[b][fm][fn], 0, 0, 0);
      if (NORMS) {
        // the two waves that load the same A rows (same wm) share their norm
        // work by fragment halves, and likewise for B rows (same wn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          if ((fm * 2) / FM == wn) {
            const u32x4_t v = __builtin_bit_cast(u32x4_t, af[fm]);
            sqa[fm] = dot2_bf16(v.x, v.x, dot2_bf16(v.y, v.y, dot2_bf16(v.z, v.z, dot2_bf16(v.w, v.w, sqa[fm]))));
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            if (((b * FN + fn) * 2) / (NB * FN) == wm) {
              const u32x4_t v = __builtin_bit_cast(u32x4_t, bfr[b][fn]);
              sqb[b][fn] = dot2_bf16(v.x, v.x, dot2_bf16(v.y, v.y, dot2_bf16(v.z, v.z, dot2_bf16(v.w, v.w, sqb[b][fn]))));
            }
          }
      }
    }
  }

  // ---- fragment-pipelined K loop: the MFMAs of step kt run on fragments
  // read during step kt-1, while the fragments of step kt+1 are read from LDS
  // and the buffer loads of later stages are in flight.  A step is one LDS
  // stage of BK columns (KS = BK / 32 MFMA K slices).
  static constexpr int KS = BK / 32;
  struct Frags {
    bf16x8_t a[KS][FM];
    bf16x8_t b[KS][NB][FN];
  };

  __device__ __forceinline__ void load_frags(Frags& f, const uint8_t* stage) const {
    const int lane = lane_id();
    const int w = uniform((int)(threadIdx.x >> 6));
    const int wm = w % WAVES_M, wn = w / WAVES_M;
    if (B_KN) {
      const uint8_t* bst = stage + BM * ROWB;
      const int g = lane >> 4, i = lane & 15;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int nl = wn * WN + fn * 16 + 4 * (i & 3);
        const int k1 = 8 * g + (i >> 2), k2 = k1 + 4;
        const uint8_t* p1 = bst + k1 * KN_ROWB + kn_slot(k1, nl >> 3) * 16 + (nl & 7) * 2;
        const uint8_t* p2 = bst + k2 * KN_ROWB + kn_slot(k2, nl >> 3) * 16 + (nl & 7) * 2;
        typedef short s16x4_t __attribute__((ext_vector_type(4)));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(lds_void_t*)p1);
        const s16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(lds_void_t*)p2);
        const u32x4_t u = {(uint32_t)(uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16),
                           (uint32_t)(uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16),
                           (uint32_t)(uint16_t)v2[0] | ((uint32_t)(uint16_t)v2[1] << 16),
                           (uint32_t)(uint16_t)v2[2] | ((uint32_t)(uint16_t)v2[3] << 16)};
        f.b[0][0][fn] = __builtin_bit_cast(bf16x8_t, u);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cq = slot(lane & 15, ks * 4 + (lane >> 4)) * 16;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int r = BM + b * BNW + wn * WN + fn * 16 + (lane & 15);
            f.b[ks][b][fn] = *(const bf16x8_t*)(stage + r * ROWB + cq);
          }
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cq = slot(lane & 15, ks * 4 + (lane >> 4)) * 16;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = wm * WM + fm * 16 + (lane & 15);
        f.a[ks][fm] = *(const bf16x8_t*)(stage + r * ROWB + cq);
      }
    }
  }

  __device__ __forceinline__ void mma(const Frags& f) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[b][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                f.a[ks][fm], f.b[ks][b][fn], acc[b][fm][fn], 0, 0, 0);
  }

  // Step kt: stage kt+1 must have landed (loads of stages kt+2 .. kt+S-2 may
  // still be in flight), then the loads of stage kt+S-1 are issued into the
  // buffer of stage kt-1, whose fragments were read during step kt-2.
  // The scheduling barriers keep the compiler from moving the MFMAs of one
  // step next to the fragment reads that feed them (which would make every
  // MFMA wait for an LDS read): the reads of step kt+1 are all issued before
  // the MFMAs of step kt.
  // Sums of squares of the A rows from the fragments of a step (lane l: row
  // l & 15 of fragment fm, one quarter of the step's K range), for the waves
  // that call it.
  __device__ __forceinline__ void sq_a(const Frags& f) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const u32x4_t v = __builtin_bit_cast(u32x4_t, f.a[ks][fm]);
        sqa[fm] = dot2_bf16(v.x, v.x, dot2_bf16(v.y, v.y, dot2_bf16(v.z, v.z, dot2_bf16(v.w, v.w, sqa[fm]))));
      }
  }

  // INTERLEAVE (steady steps): the buffer loads and fragment reads of the step
  // are spread among its MFMAs (one load or read, then a few MFMAs) instead
  // of all being issued ahead of them, so that a wave's MFMA issue is not held
  // up behind a burst of memory instructions.
  static constexpr int N_DS = KS * FM + (B_KN ? 2 * FN : KS * NB * FN);  // fragment reads per step
  static constexpr int N_MFMA = KS * FM * NB * FN;                      // MFMAs per step
  static __device__ __forceinline__ void interleave_schedule() {
    constexpr int per_load = 1;
    constexpr int left = N_MFMA - LOADS * per_load;
    constexpr int per_ds = left / N_DS > 0 ? left / N_DS : 1;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         // one buffer load
      __builtin_amdgcn_sched_group_barrier(0x008, per_load, 0);  // MFMAs
    }
#pragma unroll
    for (int i = 0; i < N_DS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, per_ds, 0);  // MFMAs
    }
    if constexpr (left - per_ds * N_DS > 0)
      __builtin_amdgcn_sched_group_barrier(0x008, left - per_ds * N_DS, 0);
  }

  // The buffer loads of a step write one LDS stage while its fragment reads
  // come from another: the restrict qualifiers tell the compiler so (the two
  // stages are distinct since STAGES >= 3).  Without that knowledge it makes
  // every transposing read wait for all buffer loads in flight, which would
  // expose the global-load latency once per step.
  __device__ __forceinline__ void issue_and_read(uint8_t* __restrict__ dst, int k0,
                                                 const uint8_t* __restrict__ src, Frags& nxt) {
    issue(dst, k0);
    load_frags(nxt, src);
  }

  template <bool STEADY, bool SQA = false>
  __device__ __forceinline__ void pipe_step(uint8_t* lds, int kt, int nk, Frags& cur, Frags& nxt) {
    if constexpr (INTERLEAVE && STEADY && !SQA) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<(STAGES - 3) * LOADS>());
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue_and_read(lds + ((kt + STAGES - 1) % STAGES) * STAGE_BYTES, (kt + STAGES - 1) * BK,
                     lds + ((kt + 1) % STAGES) * STAGE_BYTES, nxt);
      mma(cur);
      interleave_schedule();
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    if (STEADY || kt + 1 < nk) {
      if (STEADY) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<(STAGES - 3) * LOADS>());
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
      }
      lds_barrier();
      if (STEADY || kt + STAGES - 1 < nk)
        issue_and_read(lds + ((kt + STAGES - 1) % STAGES) * STAGE_BYTES, (kt + STAGES - 1) * BK,
                       lds + ((kt + 1) % STAGES) * STAGE_BYTES, nxt);
      else
        load_frags(nxt, lds + ((kt + 1) % STAGES) * STAGE_BYTES);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(cur);
    if (SQA && uniform((int)(threadIdx.x >> 6)) / WAVES_M == 0) sq_a(cur);
    __builtin_amdgcn_sched_barrier(0);
  }

  // SQA: the waves with wn == 0 also accumulate the sums of squares of the A
  // rows (sqa, per lane as in sq_a).  after_issue() runs once the first
  // stages' loads are in flight, before the wait for them: work whose own
  // memory latency can hide behind theirs (its LDS writes, outside the
  // pipeline's stages, are visible to the whole workgroup after the loop's
  // first barrier).
  template <bool SQA = false, typename F>
  __device__ __forceinline__ void run_pipe(uint8_t* lds, int K, F&& after_issue) {
    static_assert(STAGES >= 3, "stages");
    const int nk = K / BK;
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(lds + s * STAGE_BYTES, s * BK);
    after_issue();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
    lds_barrier();
    Frags f0, f1;
    load_frags(f0, lds);
    int kt = 0;
    // steady state (every stage it refers to exists): no conditions, so the
    // fragment reads of step kt+1 overlap the MFMAs of step kt
    for (; kt + STAGES < nk; kt += 2) {  // step kt+1 issues stage kt+STAGES
      pipe_step<true, SQA>(lds, kt, nk, f0, f1);
      pipe_step<true, SQA>(lds, kt + 1, nk, f1, f0);
    }
    for (; kt < nk; kt += 2) {
      pipe_step<false, SQA>(lds, kt, nk, f0, f1);
      if (kt + 1 < nk) pipe_step<false, SQA>(lds, kt + 1, nk, f1, f0);
    }
    __syncthreads();
  }

  template <bool SQA = false>
  __device__ __forceinline__ void run_pipe(uint8_t* lds, int K) {
    run_pipe<SQA>(lds, K, [] {});
  }

  // Full K loop; K must be a multiple of 64.  lds must hold LDS_BYTES.
  __device__ __forceinline__ void run(uint8_t* lds, int K) {
    const int nk = K / BK;
    issue(lds, 0);
    if (nk > 1) issue(lds + STAGE_BYTES, BK);
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<LOADS>());
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
      }
      lds_barrier();
      if (kt + 2 < nk) issue(lds + ((kt + 2) % STAGES) * STAGE_BYTES, (kt + 2) * BK);
      compute(lds + (kt % STAGES) * STAGE_BYTES);
    }
    __syncthreads();
  }

  // s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= N only.
  template <int N>
  static constexpr int vmcnt_imm() {
    return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  }

  // Guard-band norms: sqrt of the row sums of squares, A rows to rn_a[256]
  // and B rows to rn_b[NB * BNW] (LDS).
  __device__ __forceinline__ void write_norms(float* rn_a, float* rn_b) {
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const int wm = w % WAVES_M, wn = w / WAVES_M;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      float s = sqa[fm];
      s += __shfl_xor(s, 16, kWave);
      s += __shfl_xor(s, 32, kWave);
      if ((fm * 2) / FM == wn && lane < 16) rn_a[wm * WM + fm * 16 + lane] = sqrtf(s);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        float s = sqb[b][fn];
        s += __shfl_xor(s, 16, kWave);
        s += __shfl_xor(s, 32, kWave);
        if (((b * FN + fn) * 2) / (NB * FN) == wm && lane < 16)
          rn_b[b * BNW + wn * WN + fn * 16 + lane] = sqrtf(s);
      }
  }

  // f(b, row, col, value) over the accumulators (row in 0..255, col in 0..BNW-1).
  template <typename F>
  __device__ __forceinline__ void for_each(F&& f) const {
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const int wm = w % WAVES_M, wn = w / WAVES_M;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = wm * WM + fm * 16 + 4 * (lane >> 4) + r;
            const int col = wn * WN + fn * 16 + (lane & 15);
            f(b, row, col, acc[b][fm][fn][r]);
          }
  }
};

}  // namespace sffn
