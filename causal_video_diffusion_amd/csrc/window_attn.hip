// Chunk-causal attention over the limited temporal window (UnStep, abstract:
// the attention KV cache keeps only a limited window of latent frames; Table
// 3: chunks of three latent frames), with the query RoPE fused into the
// Q-tile load (abstract: RoPE applied from precomputed coefficients).
//
// Design (gfx950, wave64, bf16 MFMA 32x32x16 with fp32 accumulation):
//  * One workgroup of 8 waves per CU owns 256 queries of one head (32 per
//    wave), so every K/V tile brought into LDS feeds 256 queries.  Waves w
//    and w+4 share a SIMD.  The two groups (waves 0-3, 4-7) run a phase
//    apart ("ping-pong"): in every phase one group issues MFMAs (QK of the
//    current tile, then PV of the previous one, as one pipeline of LDS
//    fragment reads running ahead of the MFMAs) while the other computes the
//    softmax of its current tile, so on each SIMD one wave's VALU work runs
//    under the other wave's matrix work.  A workgroup barrier separates the
//    phases.
//  * The window's keys form one virtual sequence (frame after frame, each
//    frame's T keys read from its ring slot), walked in tiles of 64 keys;
//    only the last tile can be partial, and a tile may straddle frames.
//  * Scores are computed transposed, S^T = K Q^T: the MFMA output puts one
//    query per lane (column) and 16 keys per lane in registers, so the row
//    max and row sum are in-lane reductions plus one exchange between lanes
//    l and l^32.  The query rotation, the softmax scale and log2(e) are
//    folded into the bf16 query fragments once per workgroup.
//  * The score accumulators start at -m (the lane's running reference max),
//    so the MFMA yields s - m directly.  The reference is set from the exact
//    tile max on a segment's first tile; after that the tile max is not
//    taken at all unless the running sum leaves [0, 2^64] (a probability
//    large enough to risk overflow, an infinity or a NaN): then the raw
//    scores, still in registers, set a new reference (if they exceed the old
//    one by more than 2^8) and the tile is redone.  So almost every tile
//    costs its exponentials, sums and packs only; the final normalisation by
//    the running sum makes the result exact regardless of the reference.
//  * The A-operand rows of S^T are permuted (bits 2 and 3 of the key index
//    swapped) so that each lane's 8 score registers of one 16-key group hold
//    8 consecutive keys: those registers, rounded to bf16, are directly the
//    B operand of O^T = V^T P^T.  V^T comes from the transposed value cache,
//    so neither P nor V is transposed on chip.  The row sum uses plain fp32
//    adds: on gfx950 dot-product instructions share the matrix pipe and
//    would stall behind the partner wave's MFMAs.
//  * K and V^T tiles go straight from global memory to LDS
//    (global_load_lds_dwordx4, no register staging) through a 4-stage ring:
//    tile t+2 is requested while tile t is consumed, so each load has four
//    phases to land.  16-byte chunks are XOR-swizzled so that every 16-lane
//    group of an MFMA operand read touches 64 distinct banks.  The loop is
//    unrolled over the 4 stages so every LDS address is a register plus an
//    immediate.
//  * Workgroups are numbered so that each XCD (8 per chip, dispatched round
//    robin) gets a contiguous run of (head, query tile) work: the workgroups
//    streaming one head's K/V share an L2.
//  * Two schedules (attn_schedule.h).  Either each workgroup owns one (head,
//    query tile) over all key tiles, or, for G workgroups, whole (head,
//    query tile) units run G at a time and the key tiles of the remainder
//    are cut into G equal ranges, so the last round is not partly empty.  A
//    unit split between workgroups leaves each part's normalised output and
//    log-sum-exp in a workspace, and a second kernel merges them.

#include <type_traits>

#include "attn_schedule.h"
#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kWaves = 8;
constexpr int kStages = 4;     // LDS ring of K/V tiles
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr float kRescale = 8.0f;  // move the reference max when exceeded (log2 units)
constexpr float kSumBound = 0x1p64f;  // a lane's running sum above this triggers a rescale

// swap bits 2 and 3 of a row index within a 32-row MFMA block
__device__ __forceinline__ int perm_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// XOR key of a K-tile row's 16-byte chunks: distinct across any 16 rows that
// one 16-lane group reads (rows of 256 B for D=128, of 128 B for D=64)
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}
// XOR key of a V^T-tile row (128 B: 64 keys)
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

// Combine a value with the one held by lane l^32.  v_permlane32_swap with the
// same register as both operands leaves, in its two results, this lane's value
// and the partner's (one in each), so max and sum of the two results are the
// pair's max and sum whichever result holds which.
__device__ __forceinline__ float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// map blockIdx to work so each XCD gets a contiguous range
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb / 8, rem = nb % 8;
  const int x = b % 8, k = b / 8;
  return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + k;
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane
// (global_load_lds_dwordx4).  Issued from inline asm so that the compiler
// does not track the LDS write: it would otherwise wait for every such load
// before any later LDS read.  Ordering is explicit instead: each wave waits
// for its own loads (vmcnt) before the workgroup barrier that precedes the
// first read of the stage, and a stage is only rewritten after the barrier
// that follows its last read.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint16_t*)(p)));
}
__device__ __forceinline__ void load_lds16(const uint16_t* g, uint32_t m0) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0));
}
// sbase must be wave-uniform; it is passed through readfirstlane so that it
// sits in scalar registers whatever the compiler proves about it
__device__ __forceinline__ void load_lds16_s(const uint16_t* sbase, uint32_t voff_bytes, uint32_t m0) {
  // (readfirstlane returns int: widen through uint32_t, or a low word with
  // bit 31 set would sign-extend into the high half)
  const uint64_t p = reinterpret_cast<uint64_t>(sbase);
  const uint64_t su = (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(p >> 32)))) << 32) |
                      uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(p))));
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff_bytes), "s"(reinterpret_cast<const uint16_t*>(su)),
               "{m0}"(m0));
}

// s_waitcnt with vmcnt <= N and the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// workgroup barrier that neither waits for outstanding loads nor lets the
// compiler move memory accesses across it
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Order N (LDS read, MFMA) pairs as: kPre reads, then alternately one MFMA
// and one read, then the last kPre MFMAs, so every MFMA finds its operand
// read kPre MFMAs earlier.
constexpr int kPre = 4;
template <int N>
__device__ __forceinline__ void sched_pipeline() {
  constexpr int kMfma = 0x008, kDsRead = 0x100;
  __builtin_amdgcn_sched_group_barrier(kDsRead, kPre, 0);
#pragma unroll
  for (int i = 0; i < N - kPre; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, kPre, 0);
}

template <int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
window_attn_kernel(AttnArgs a) {
  constexpr int KS = D / 16;                          // k-steps of the score product
  constexpr int DB = D / 32;                          // 32-row blocks of O^T
  constexpr int KCPR = D / 8;                         // 16-byte chunks per key row
  constexpr int KRPI = 64 / KCPR;                     // key rows per 1 KB load
  constexpr int KINST = kBN * D * 2 / 1024 / kWaves;  // K loads per wave per tile
  constexpr int VINST = D * kBN * 2 / 1024 / kWaves;  // V^T loads per wave per tile
  constexpr int NLD = KINST + VINST;                  // loads per wave per tile
  // one array per ring; the stage offsets (multiples of 16 KB for D = 128)
  // are compile-time constants, so they fold into the LDS instructions'
  // immediate offsets (under 64 KB) and each lane needs one address register
  // per fragment position for all stages
  __shared__ __attribute__((aligned(1024))) uint16_t lk[kStages * kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lv[kStages * D * kBN];
  auto kstage = [&](auto tag) __attribute__((always_inline)) -> uint16_t* {
    return lk + decltype(tag)::value * (kBN * D);
  };
  auto vstage = [&](auto tag) __attribute__((always_inline)) -> uint16_t* {
    return lv + decltype(tag)::value * (D * kBN);
  };
  __shared__ uint32_t kbase[UST_MAX_WINDOW_FRAMES];
  __shared__ uint32_t vbase[UST_MAX_WINDOW_FRAMES];

  const int nqt = (a.NQ + kBM - 1) / kBM;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_a = wave < 4;   // waves w and w + 4 share a SIMD
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int T = a.T;
  const int TV = a.TV;
  const int nk = a.n_frames * T;
  const int ntiles = (nk + kBN - 1) / kBN;

  // ---- this workgroup's share of the work (attn_schedule.h) ----
  const AttnPlan plan = attn_plan(nqt * a.H, ntiles, a.n_wg);
  const int w = xcd_remap(blockIdx.x, plan.G);

  // ---- per-lane constants of the tile loads ----
  // K load i of wave w fills LDS bytes [(w*KINST + i) KB, +1 KB): key row
  // `row`, logical 16-byte chunk (stored at this lane's position).
  int koff[KINST], voff[VINST];
#pragma unroll
  for (int i = 0; i < KINST; ++i) {
    const int row = KRPI * (wave * KINST + i) + lane / KCPR;
    koff[i] = row * D + (((lane % KCPR) ^ kswz<D>(row)) * 8);
  }
#pragma unroll
  for (int i = 0; i < VINST; ++i) {
    const int d = 8 * (wave * VINST + i) + lane / 8;
    voff[i] = d * TV + (((lane % 8) ^ vswz(d)) * 8);
  }

  // Element offsets of this lane's MFMA operand fragments within a tile
  // buffer.  Key block kb adds 32 rows (kswz is the same for rows r and
  // r + 32) and O^T block b adds 32 dims (vswz likewise), so those and the
  // buffer index fold into the ds_read immediate offsets.
  int koffr[KS], voffr[4];
  {
    const int row = perm_row(l32);
#pragma unroll
    for (int s = 0; s < KS; ++s) koffr[s] = row * D + (((2 * s + half) ^ kswz<D>(row)) * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) voffr[q] = l32 * kBN + (((2 * q + half) ^ vswz(l32)) * 8);
  }

  // One pass per segment: a whole unit, or key tiles k0 .. k0+nseg-1 of one.
  AttnWalk walk = attn_walk(w, plan);
  AttnSegment sg;
  while (attn_next(walk, w, plan, sg)) {
    const int k0 = sg.k0;
    const int nseg = sg.n;
    const int slot = sg.slot;
    const int h = sg.unit / nqt;
    const int q0 = (sg.unit % nqt) * kBM;

    __syncthreads();  // the previous segment is done with kbase / vbase
    for (int i = tid; i < a.n_frames; i += 512) {
      kbase[i] = uint32_t((a.slots[i] * a.H + h) * T * D);
      vbase[i] = uint32_t((a.slots[i] * a.H + h) * D * TV);
    }

    // ---- query fragments: RoPE at the query's own position, scale, bf16 ----
    const int qn = q0 + wave * 32 + l32;
    const bool qvalid = qn < a.NQ;
    // a wave whose queries all lie past the chunk (in a head's last, ragged
    // query tile) only loads its share of the tiles and keeps the barriers
    const bool wave_busy = q0 + wave * 32 < a.NQ;
    bf16x8 qf[KS];
    {
      const uint16_t* qp = a.q + (int64_t(qn) * a.H + h) * D;
      const int64_t trow = (int64_t(a.tab_frame) * T + qn) * (D / 2);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int d0 = 16 * s + 8 * half;
        uint4 raw = make_uint4(0, 0, 0, 0);
        float4 cs = make_float4(0, 0, 0, 0), sn = make_float4(0, 0, 0, 0);
        if (qvalid) {
          raw = *reinterpret_cast<const uint4*>(qp + d0);
          cs = *reinterpret_cast<const float4*>(a.cos_tab + trow + d0 / 2);
          sn = *reinterpret_cast<const float4*>(a.sin_tab + trow + d0 / 2);
        }
        const uint32_t in[4] = {raw.x, raw.y, raw.z, raw.w};
        const float c4[4] = {cs.x, cs.y, cs.z, cs.w};
        const float s4[4] = {sn.x, sn.y, sn.z, sn.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf16_lo(in[e]), x1 = bf16_hi(in[e]);
          o[e] = pack_bf16x2((x0 * c4[e] - x1 * s4[e]) * a.qscale,
                             (x0 * s4[e] + x1 * c4[e]) * a.qscale);
        }
        qf[s] = as_bf16x8(make_uint4(o[0], o[1], o[2], o[3]));
      }
    }
    __syncthreads();  // kbase / vbase visible

    // Issue the global->LDS loads of key tile t (starting at frame lfi, token
    // lt0).  kfb / vfb: the frame's key and value slot bases (wave-uniform),
    // reloaded only when the load position moves to the next frame.
    int lfi = k0 * kBN / T;   // position of the next tile to load
    int lt0 = k0 * kBN - lfi * T;
    const uint16_t* kfb = a.k_cache + (int64_t(a.slots[lfi]) * a.H + h) * T * D;
    const uint16_t* vfb = a.v_cache + (int64_t(a.slots[lfi]) * a.H + h) * D * TV;
    auto next_frame = [&]() __attribute__((always_inline)) {
      ++lfi;
      if (lfi < a.n_frames) {
        kfb = a.k_cache + (int64_t(a.slots[lfi]) * a.H + h) * T * D;
        vfb = a.v_cache + (int64_t(a.slots[lfi]) * a.H + h) * D * TV;
      }
    };
    auto issue = [&](int t, auto buf_tag) __attribute__((always_inline)) {
      const uint32_t lk = __builtin_amdgcn_readfirstlane(lds_addr(kstage(buf_tag) + wave * KINST * 512));
      const uint32_t lv = __builtin_amdgcn_readfirstlane(lds_addr(vstage(buf_tag) + wave * VINST * 512));
      if (lt0 + kBN <= T && t * kBN + kBN <= nk) {
        // whole tile inside one frame: uniform base + lane constants
        const uint16_t* kb = kfb + lt0 * D;
        const uint16_t* vb = vfb + lt0;
#pragma unroll
        for (int i = 0; i < KINST; ++i) load_lds16_s(kb, uint32_t(koff[i]) * 2u, lk + i * 1024);
#pragma unroll
        for (int i = 0; i < VINST; ++i) load_lds16_s(vb, uint32_t(voff[i]) * 2u, lv + i * 1024);
      } else {
        // straddles frames or runs past the window: per-lane frame lookup;
        // keys past the window are pointed at the window's first key (finite
        // data whose probability is masked to zero)
#pragma unroll
        for (int i = 0; i < KINST; ++i) {
          const int row = KRPI * (wave * KINST + i) + lane / KCPR;
          int tt = lt0 + row, f = lfi;
          while (tt >= T) { tt -= T; ++f; }
          if (f >= a.n_frames) { f = 0; tt = 0; }
          load_lds16(a.k_cache + kbase[f] + uint32_t(tt * D) + (koff[i] - row * D), lk + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < VINST; ++i) {
          const int d = 8 * (wave * VINST + i) + lane / 8;
          const int kc = (lane % 8) ^ vswz(d);
          int tt = lt0 + 8 * kc, f = lfi;
          while (tt >= T) { tt -= T; ++f; }
          if (f >= a.n_frames) { f = 0; tt = 0; }
          load_lds16(a.v_cache + vbase[f] + uint32_t(tt) + uint32_t(d * TV), lv + i * 1024);
        }
      }
      lt0 += kBN;
      while (lt0 >= T) {
        lt0 -= T;
        next_frame();
      }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
    float mref = 0.f;   // reference max (log2 units) of this lane's query
    float lrow = 0.f;   // this lane's share of the running sum, relative to mref
    f32x16 sacc[2];     // S^T - mref of the tile being computed
    bf16x8 pf[2][2];    // bf16 probabilities of the tile awaiting PV

    // ---- S^T - mref = K Q^T + (-mref), two 32-key blocks ----
    // The fragment reads run kPre ahead of the MFMAs that consume them (the
    // scheduling-group barriers pin that order), so the MFMA pipe does not
    // wait on LDS latency.
    auto qk = [&](auto buf_tag) __attribute__((always_inline)) {
      const uint16_t* K = kstage(buf_tag);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = -mref;
      bf16x8 kf[2 * KS];
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i)
        kf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(K + koffr[i >> 1] + (i & 1) * 32 * D));
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) sacc[i & 1] = mfma32(kf[i], qf[i >> 1], sacc[i & 1]);
      sched_pipeline<2 * KS>();
    };

    // ---- O^T += V^T P^T ----
    auto pv = [&](auto buf_tag) __attribute__((always_inline)) {
      const uint16_t* V = vstage(buf_tag);
      // fragment i: key chunk 4 kb + 2 g + half of dim 32 b + l32, with
      // q = 2 kb + g = i / DB, b = i % DB
      bf16x8 vf[4 * DB];
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i)
        vf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(V + voffr[i / DB] + (i % DB) * 32 * kBN));
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i)
        oacc[i % DB] = mfma32(vf[i], pf[(i / DB) >> 1][(i / DB) & 1], oacc[i % DB]);
      sched_pipeline<4 * DB>();
    };

    // ---- both products in one read/MFMA pipeline, so the first value
    // fragments are read while the last score MFMAs run ----
    auto qkpv = [&](auto kbuf, auto vbuf) __attribute__((always_inline)) {
      const uint16_t* K = kstage(kbuf);
      const uint16_t* V = vstage(vbuf);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = -mref;
      bf16x8 kf[2 * KS], vf[4 * DB];
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i)
        kf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(K + koffr[i >> 1] + (i & 1) * 32 * D));
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i)
        vf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(V + voffr[i / DB] + (i % DB) * 32 * kBN));
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) sacc[i & 1] = mfma32(kf[i], qf[i >> 1], sacc[i & 1]);
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i)
        oacc[i % DB] = mfma32(vf[i], pf[(i / DB) >> 1][(i / DB) & 1], oacc[i % DB]);
      sched_pipeline<2 * KS + 4 * DB>();
    };

    // ---- online softmax of the segment's j-th tile (key tile t = k0 + j):
    // bf16 probabilities into pf ----
    auto softmax = [&](int j) __attribute__((always_inline)) {
      const int t = k0 + j;
      if (t == ntiles - 1 && ntiles * kBN > nk) {
        asm volatile("; last tile: keys past the window end");
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = t * kBN + 32 * kb + 16 * (r / 8) + 8 * half + (r % 8);
            if (key >= nk) sacc[kb][r] = -INFINITY;
          }
      }
      // The exact tile max (shared by lanes l and l^32) is taken on the
      // segment's first tile, where it sets the reference, and otherwise only
      // when the tile's sum leaves [0, kSumBound]: a probability so large it
      // could overflow, an infinity or a NaN.  The scores are kept until that
      // test, so the rare path rescales and redoes the tile.
      auto rescale = [&](auto first_tag) __attribute__((always_inline)) {
        constexpr bool first = decltype(first_tag)::value;
        float m4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int kb = c >> 1, r0 = 8 * (c & 1);
          m4[c] = fmaxf(fmaxf(fmaxf(sacc[kb][r0], sacc[kb][r0 + 1]), sacc[kb][r0 + 2]),
                        fmaxf(fmaxf(sacc[kb][r0 + 3], sacc[kb][r0 + 4]),
                              fmaxf(fmaxf(sacc[kb][r0 + 5], sacc[kb][r0 + 6]), sacc[kb][r0 + 7])));
        }
        const float tmax = pair_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
        const float shift = (first || tmax > kRescale) ? tmax : 0.f;
        mref += shift;
        if constexpr (!first) {
          // On a segment's first tile the running sum and the output are
          // still zero and are not scaled: alpha = 2^-tmax overflows to
          // infinity when the whole tile scores below -128 (log2 units), and
          // 0 * inf would be NaN.
          const float alpha = __builtin_amdgcn_exp2f(-shift);
          lrow *= alpha;
#pragma unroll
          for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] -= shift;
      };
      // probabilities (32 independent exp2) straight into bf16 pairs, the row
      // sum in fp32 in four independent partial sums (plain adds:
      // dot-product instructions would contend with the partner wave's MFMAs)
      auto probs = [&]() __attribute__((always_inline)) -> float {
        float ls[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * g + 2 * e;
              const float p0 = __builtin_amdgcn_exp2f(sacc[kb][r]);
              const float p1 = __builtin_amdgcn_exp2f(sacc[kb][r + 1]);
              const int c = (kb * 16 + r) & 3;   // 0 or 2
              if (kb == 0 && g == 0 && e < 2) {
                ls[c] = p0;
                ls[c + 1] = p1;
              } else {
                ls[c] += p0;
                ls[c + 1] += p1;
              }
              pk[e] = pack_bf16x2(p0, p1);
            }
            pf[kb][g] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
          }
        return (ls[0] + ls[1]) + (ls[2] + ls[3]);
      };
      if (j == 0) rescale(std::true_type{});
      float lnew = lrow + probs();
      if (__builtin_amdgcn_ballot_w64(!(lnew <= kSumBound))) {
        rescale(std::false_type{});
        lnew = lrow + probs();
      }
      lrow = lnew;
    };

    // ---- the phase schedule ----
    // Tiles are counted from the segment's first (j = 0 is key tile k0).
    // Every wave runs the same sequence; group B starts one barrier later, so
    // its phases are offset by one from group A's:
    //   MFMA phase j:    QK(j) and PV(j-1) in one pipeline; barrier
    //   softmax phase j: request own share of tile j+L; softmax(j); wait for own
    //                    share of tile j+L-1; barrier
    // with L = 2 for group A and L = 3 for group B, so every share of tile v is
    // in LDS before group A's MFMA phase v, and the loads and their waits sit in
    // softmax phases, under the partner wave's MFMA phase.  Tile v lives in LDS
    // stage v % 4 from its first request (group B's softmax phase v-3) until
    // group B's PV(v) (its MFMA phase v+1).
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    const int lead = group_a ? 2 : 3;
    // MODE 0: the first tile (QK only); 1: QK(j) and PV(j-1); 2: the last PV
    auto step = [&](auto mode, int j, auto cur, auto prev, auto st2, auto st3) __attribute__((always_inline)) {
      constexpr int MODE = decltype(mode)::value;
      __builtin_amdgcn_s_setprio(2);
      if (wave_busy) {   // QK first, so its scores are ready for softmax(j)
        if constexpr (MODE == 1) qkpv(cur, prev);
        else if constexpr (MODE == 0) qk(cur);
        else pv(prev);
      }
      __builtin_amdgcn_s_setprio(0);
      barrier();
      const int v = j + lead;      // tile this wave requests now
      if (v < nseg) {
        if (group_a) issue(k0 + v, st2);
        else issue(k0 + v, st3);
      }
      if (MODE != 2 && wave_busy) softmax(j);
      if (v < nseg) wait_vmcnt<NLD>();   // own share of tile v-1 landed
      else wait_vmcnt<0>();
      barrier();
    };

    issue(k0, S0{});
    if (nseg > 1) issue(k0 + 1, S1{});
    if (!group_a && nseg > 2) issue(k0 + 2, S2{});
    wait_vmcnt<0>();
    barrier();                        // tiles 0 .. lead-1 are in LDS
    if (!group_a) barrier();          // group B runs one phase behind
    // The first tile and the last PV are peeled off, so that the unrolled
    // loop holds one kind of MFMA phase and keeps its accumulators in place.
    using M0 = std::integral_constant<int, 0>;
    using M1 = std::integral_constant<int, 1>;
    using M2 = std::integral_constant<int, 2>;
    step(M0{}, 0, S0{}, S3{}, S2{}, S3{});
    for (int j = 1; j < nseg; j += 4) {
      step(M1{}, j, S1{}, S0{}, S3{}, S0{});
      if (j + 1 < nseg) step(M1{}, j + 1, S2{}, S1{}, S0{}, S1{});
      if (j + 2 < nseg) step(M1{}, j + 2, S3{}, S2{}, S1{}, S2{});
      if (j + 3 < nseg) step(M1{}, j + 3, S0{}, S3{}, S2{}, S3{});
    }
    switch ((nseg - 1) & 3) {   // PV of the last tile, from its stage
      case 0: step(M2{}, nseg, S0{}, S0{}, S0{}, S0{}); break;
      case 1: step(M2{}, nseg, S0{}, S1{}, S0{}, S0{}); break;
      case 2: step(M2{}, nseg, S0{}, S2{}, S0{}, S0{}); break;
      default: step(M2{}, nseg, S0{}, S3{}, S0{}, S0{}); break;
    }
    if (group_a) barrier();           // match group B's extra barrier

    // ---- epilogue: normalise, store bf16 O and the log-sum-exp, or the
    // partial result of a split unit ----
    const float ltot = pair_sum(lrow);
    const float inv = 1.f / ltot;
    const float lse_nat = (mref + __builtin_log2f(ltot)) * 0.6931471805599453f;
    if (slot >= 0) {
      if (qvalid) {
        const int row = wave * 32 + l32;
        float* po = a.work_o + (int64_t(slot) * kBM + row) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d = 32 * b + 8 * g + 4 * half;
            *reinterpret_cast<float4*>(po + d) =
                make_float4(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv,
                            oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
          }
        if (half == 0) a.work_l[int64_t(slot) * kBM + row] = lse_nat;
      }
    } else if (qvalid) {
      uint16_t* op = a.out + (int64_t(qn) * a.H + h) * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * b + 8 * g + 4 * half;
          uint2 v;
          v.x = pack_bf16x2(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv);
          v.y = pack_bf16x2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
          *reinterpret_cast<uint2*>(op + d) = v;
        }
      if (a.lse && half == 0) a.lse[int64_t(h) * a.NQ + qn] = lse_nat;
    }
  }  // segments
}

// Merge the partial results of units that the key-split schedule divided
// between workgroups.  With per-part normalised outputs O_i and log-sum-exps
// L_i: O = sum_i e^(L_i - M) O_i / sum_i e^(L_i - M), L = M + ln sum_i
// e^(L_i - M), M = max_i L_i, taken part by part with a running maximum.
// One block per ROWS query rows of a key-split unit; each thread owns 4 dims
// of PER rows.  PER = 8 for units of a few parts (all rows of a part in
// flight at once); PER = 1 for units of many parts, with UNR parts in flight.
// The block first lists its unit's part slots in LDS, kMergeParts at a time.
constexpr int kMergeParts = 256;
template <int D, int PER>
__global__ void __launch_bounds__(256) window_attn_combine_kernel(AttnArgs a) {
  constexpr int CPR = D / 4;                  // float4 chunks per row
  constexpr int RSTEP = 256 / CPR;            // rows apart of one thread's rows
  constexpr int ROWS = RSTEP * PER;           // rows per block
  constexpr int BPU = kBM / ROWS;             // blocks per unit
  constexpr int UNR = PER == 1 ? 8 : 1;       // parts loaded together
  __shared__ int part_slot[kMergeParts];
  const int nqt = (a.NQ + kBM - 1) / kBM;
  const int ntiles = (a.n_frames * a.T + kBN - 1) / kBN;
  const AttnPlan plan = attn_plan(nqt * a.H, ntiles, a.n_wg);
  const int u = plan.u0 + int(blockIdx.x) / BPU;   // only key-split units
  if (attn_unit_whole(u, plan)) return;   // written by its workgroup
  const int64_t ue = attn_unit_end(u, plan);
  const int h = u / nqt;
  const int c = threadIdx.x % CPR;
  const int row0 = (blockIdx.x % BPU) * ROWS + threadIdx.x / CPR;
  float m[PER], sum[PER];
  float4 acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    m[k] = -INFINITY;
    sum[k] = 0.f;
    acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int base = attn_unit_first_wg(u, plan);
       base < plan.G && wg_range_start(base, plan) < ue; base += kMergeParts) {
    __syncthreads();   // the previous pass is done with part_slot
    // workgroups base .. base+255 that start before the unit's end form a
    // prefix (starts increase); empty ranges inside it hold no part
    const int b = base + int(threadIdx.x);
    const bool in_unit = b < plan.G && wg_range_start(b, plan) < ue;
    part_slot[threadIdx.x] =
        in_unit && attn_wg_has_part(b, plan) ? attn_partial_slot(b, u, plan) : -1;
    const int n_listed = __syncthreads_count(in_unit);
    for (int i = 0; i < n_listed; i += UNR) {
      int sl[UNR];
      float l[UNR][PER];
      float4 o[UNR][PER];
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        sl[j] = i + j < n_listed ? part_slot[i + j] : -1;
        if (sl[j] < 0) continue;
        const float* lp = a.work_l + int64_t(sl[j]) * kBM;
        const float* op = a.work_o + int64_t(sl[j]) * kBM * D + 4 * c;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const int row = row0 + k * RSTEP;
          l[j][k] = lp[row];
          o[j][k] = *reinterpret_cast<const float4*>(op + int64_t(row) * D);
        }
      }
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        if (sl[j] < 0) continue;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const float mn = fmaxf(m[k], l[j][k]);
          const float sa = expf(m[k] - mn);   // 0 on the first part (m = -inf)
          const float e = expf(l[j][k] - mn);
          m[k] = mn;
          sum[k] = sum[k] * sa + e;
          acc[k].x = acc[k].x * sa + e * o[j][k].x;
          acc[k].y = acc[k].y * sa + e * o[j][k].y;
          acc[k].z = acc[k].z * sa + e * o[j][k].z;
          acc[k].w = acc[k].w * sa + e * o[j][k].w;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int qn = (u % nqt) * kBM + row0 + k * RSTEP;
    if (qn >= a.NQ) continue;   // rows past the chunk: no partial was written
    const float inv = 1.f / sum[k];
    uint2 v;
    v.x = pack_bf16x2(acc[k].x * inv, acc[k].y * inv);
    v.y = pack_bf16x2(acc[k].z * inv, acc[k].w * inv);
    *reinterpret_cast<uint2*>(a.out + (int64_t(qn) * a.H + h) * D + 4 * c) = v;
    if (a.lse && c == 0) a.lse[int64_t(h) * a.NQ + qn] = m[k] + logf(sum[k]);
  }
}

}  // namespace

size_t window_attn_work_bytes(int32_t head_dim, int32_t n_wg) {
  return size_t(2) * size_t(n_wg) * kBM * (size_t(head_dim) + 1) * sizeof(float);
}

hipError_t launch_window_attn(const AttnArgs& args, hipStream_t s) {
  AttnArgs a = args;
  const int nqt = (a.NQ + kBM - 1) / kBM;
  const int units = nqt * a.H;
  const int ntiles = (a.n_frames * a.T + kBN - 1) / kBN;
  // one workgroup per unit, or the plan for the requested count; the
  // workspace is laid out for the requested count (slots < 2 G <= 2 n_wg)
  if (a.work_o) a.work_l = a.work_o + size_t(2) * a.n_wg * kBM * a.D;
  else a.n_wg = units;
  const AttnPlan plan = attn_plan(units, ntiles, a.n_wg);
  if (a.D == 128)
    hipLaunchKernelGGL(window_attn_kernel<128>, dim3(plan.G), dim3(64 * kWaves), 0, s, a);
  else
    hipLaunchKernelGGL(window_attn_kernel<64>, dim3(plan.G), dim3(64 * kWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.work_o) return e;
  if (!attn_any_split(plan)) return hipSuccess;   // nothing to merge
  // Parts per split unit: about ntiles / (steps per range) + 2.  Few: one
  // block per 64 rows (8 per thread); many: one block per 256 / (D / 4) rows
  // with several parts in flight.
  const int split_units = units - plan.u0;
  const bool many = plan.steps / plan.G * 4 < ntiles;
  const int rows = (256 / (a.D / 4)) * (many ? 1 : 8);
  const dim3 grid(split_units * (kBM / rows));
  if (a.D == 128) {
    if (many) hipLaunchKernelGGL((window_attn_combine_kernel<128, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((window_attn_combine_kernel<128, 8>), grid, dim3(256), 0, s, a);
  } else {
    if (many) hipLaunchKernelGGL((window_attn_combine_kernel<64, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((window_attn_combine_kernel<64, 8>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ust
