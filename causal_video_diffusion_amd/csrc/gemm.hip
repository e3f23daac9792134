// bf16 GEMM Y[M][N] = X[M][K] W[N][K]^T (+ bias), fp32 accumulation, bf16
// out: the two products of the truncated-SVD projections (UnStep, abstract:
// truncated SVD of the attention value and output projections), and the
// dense projection when the factor is a full weight.
//
// Design (gfx950, MFMA 32x32x16 bf16):
//  * The product is formed transposed, Y^T = W X^T, so each lane ends with
//    one output row m and runs of 4 consecutive columns n: 8-byte stores.
//  * Tiles BM x 128 (BM = 128 or 64) with BK = 64, 4 waves in a 2 x 2 grid,
//    both operand tiles k-contiguous in LDS with an XOR swizzle on 16-byte
//    chunks (conflict-free MFMA operand reads), double-buffered.
//  * Ragged M, N and K are zero-filled at the tile loads; stores are masked.
//  * When K is a multiple of 64 a pipelined variant (below) streams tiles
//    straight into LDS instead of through registers.

#include <mutex>
#include <type_traits>

#include "append_keys.h"
#include "gemm_order.h"
#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kKeysPerWg = 4;   // key tiles per key-append workgroup of the pipelined GEMM

template <int MB>  // 32-row blocks of X per wave; BM = 64 * MB
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_nt_kernel(GemmArgs g) {
  constexpr int BM = 64 * MB;
  constexpr int NB = 2;                  // 32-row blocks of W per wave
  constexpr int XITEMS = BM * 8 / 256;   // 16-byte chunks of the X tile per thread
  constexpr int WITEMS = kBN * 8 / 256;
  __shared__ __attribute__((aligned(16))) uint16_t lx[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t lw[2][kBN * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave & 1;   // wave's position in the 2 x 2 grid
  const int wn = wave >> 1;
  const int nbn = (g.N + kBN - 1) / kBN;
  const int m0 = (blockIdx.x / nbn) * BM;
  const int n0 = (blockIdx.x % nbn) * kBN;
  const int nkt = (g.K + kBK - 1) / kBK;

  const int ch = tid & 7;    // chunk within a 64-wide k row
  const int r0 = tid >> 3;   // first row this thread loads; then +32 each item
  uint4 xr[XITEMS], wr[WITEMS];
  auto gload = [&](int kt) {
    const int k = kt * kBK + ch * 8;
#pragma unroll
    for (int it = 0; it < XITEMS; ++it) {
      const int m = m0 + r0 + 32 * it;
      xr[it] = make_uint4(0, 0, 0, 0);
      if (m < g.M && k < g.K) xr[it] = *reinterpret_cast<const uint4*>(g.x + int64_t(m) * g.K + k);
    }
#pragma unroll
    for (int it = 0; it < WITEMS; ++it) {
      const int n = n0 + r0 + 32 * it;
      wr[it] = make_uint4(0, 0, 0, 0);
      if (n < g.N && k < g.K) wr[it] = *reinterpret_cast<const uint4*>(g.w + int64_t(n) * g.K + k);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < XITEMS; ++it) {
      const int r = r0 + 32 * it;
      *reinterpret_cast<uint4*>(&lx[buf][r * kBK + ((ch ^ (r & 7)) * 8)]) = xr[it];
    }
#pragma unroll
    for (int it = 0; it < WITEMS; ++it) {
      const int r = r0 + 32 * it;
      *reinterpret_cast<uint4*>(&lw[buf][r * kBK + ((ch ^ (r & 7)) * 8)]) = wr[it];
    }
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(0);
  lstore(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    __syncthreads();
    const bool more = kt + 1 < nkt;
    if (more) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int c = 2 * s + half;
      bf16x8 wf[NB], xf[MB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int r = wn * 32 * NB + 32 * i + l32;
        wf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&lw[buf][r * kBK + ((c ^ (r & 7)) * 8)]));
      }
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int r = wm * 32 * MB + 32 * j + l32;
        xf[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&lx[buf][r * kBK + ((c ^ (r & 7)) * 8)]));
      }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = mfma32(wf[i], xf[j], acc[i][j]);
    }
    if (more) lstore(buf ^ 1);
  }

  // epilogue: lane holds row m = ... + l32 and columns n = 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int m = m0 + wm * 32 * MB + 32 * j + l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 32 * NB + 32 * i + 8 * q + 4 * half;
        if (n >= g.N) continue;   // N % 8 == 0, so n..n+3 are all in or all out
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][4 * q + e];
          if (g.bias) v[e] += bf16_lo(g.bias[n + e]);
        }
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(g.y + int64_t(m) * g.N + n) = o;
      }
  }
}


// ---------------------------------------------------------------------------
// Pipelined variant for K % 64 == 0.  Tiles go global -> LDS by
// global_load_lds_dwordx4 (issued from inline asm, so the compiler adds no
// waits for them) through a ring of STAGES k-slices; the loads of slice
// kt + STAGES - 1 are issued at step kt.  Each wave waits for its own loads
// of slice kt (vmcnt) and its own LDS reads of slice kt - 1 (lgkmcnt) before
// the barrier that opens step kt, so after that barrier slice kt is complete
// and the stage slice kt - 1 used is free to be refilled.  Rows past M or N
// load clamped (finite) rows whose results are never stored.
//
// Tiles are BM x BN over a WM x WN grid of waves.  With 8 waves (4 x 2), two
// share each SIMD and cover each other's load-issue stalls with MFMAs; the
// launcher uses 8-wave 256 x 128 tiles for wide outputs and 128 x 128 for the
// narrow rank-r ones, and 4-wave 192 x 64 tiles for the 64-wide heads of the
// fused projection.  The
// workgroup -> tile map is XCD-aware: workgroups are dealt to the 8 XCDs
// round-robin, and each XCD gets a contiguous run of tiles (row-major within
// one round of the chip, grouped by four row blocks beyond), so the tiles
// that share rows of X or columns of W run on one XCD and find them in its
// L2.

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint16_t*)(p)));
}
// sbase must be wave-uniform; it is passed through readfirstlane so that it
// sits in scalar registers whatever the compiler proves about it.  A vector
// instruction's write of a scalar register is not interlocked with a vector
// memory read of it (5 wait states are required) and the compiler inserts
// none before inline asm, so the asm starts with s_nop 4: the base is safe
// however the compiler schedules the readfirstlane.
__device__ __forceinline__ void load_lds16_s(const uint16_t* sbase, uint32_t voff_bytes, uint32_t m0) {
  // (readfirstlane returns int: widen through uint32_t, or a low word with
  // bit 31 set would sign-extend into the high half)
  const uint64_t p = reinterpret_cast<uint64_t>(sbase);
  const uint64_t su = (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(p >> 32)))) << 32) |
                      uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(p))));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff_bytes),
               "s"(reinterpret_cast<const uint16_t*>(su)), "{m0}"(m0));
}
// wait until at most N vector-memory ops of this wave are in flight and all
// of its LDS reads have returned (so the next barrier orders them too)
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }  // 128-byte rows

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// QKV: the fused Q/K/V projection epilogue (QkvEpilogue) instead of Y.
// WM x WN waves (4 or 8); with 8, two waves share each SIMD, so one wave's
// load-issue stalls are covered by the other's MFMAs.
// KEYD (64 or 128, the head size; 0: none): workgroups past the product's
// tiles rotate and append a chunk's keys (ka, append_keys.h), four key tiles
// each, on the compute units the product leaves idle.
template <int BM, int BN, int STAGES, bool QKV, int WM, int WN, int KEYD = 0>
__global__ void __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4)))
gemm_nt_dma_kernel(GemmArgs g, QkvEpilogue e, AppendArgs ka) {
  constexpr int NW = WM * WN;
  constexpr int NT = 64 * NW;
  constexpr int MB = BM / (32 * WM);       // 32-row blocks of X per wave
  constexpr int NB = BN / (32 * WN);       // 32-row blocks of W per wave
  static_assert(MB * 32 * WM == BM && NB * 32 * WN == BN, "tile splits over the wave grid");
  constexpr int FR = NB + MB;              // fragments per 16-wide k substep
  constexpr int NMMA = NB * MB;            // MFMAs per substep
  constexpr int XI = BM / 8, WI = BN / 8;  // 1 KB loads per slice for X and W
  constexpr int NLD = (XI + WI) / NW;      // loads per wave per slice
  static_assert((XI + WI) % NW == 0, "loads split evenly over the waves");
  constexpr int STAGE = (BM + BN) * 64;    // elements per stage: X rows, then W rows
  constexpr int LA = STAGES - 1;           // slices in flight beyond the current one
  static_assert(STAGES >= 2 && STAGES <= 4, "the vmcnt cases below cover 1 to 3 slices");
  constexpr int ES = BN + 8;               // epilogue staging row stride (elements)
  static_assert(BM * ES <= STAGES * STAGE, "epilogue tile fits in the ring");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave % WM, wn = wave / WM;
  const int nbn = (g.N + BN - 1) / BN;
  const int nbm = (g.M + BM - 1) / BM;
  if constexpr (KEYD != 0) {
    // the launch's workgroups past the product's tiles append keys; the
    // branch is uniform over the workgroup and comes before any barrier
    constexpr int TPT = NT / kKeysPerWg;     // threads per key tile
    const int ntile = nbm * nbn;
    if (int(blockIdx.x) >= ntile) {
      const int pos = xcd_range_pos(blockIdx.x, ntile, gridDim.x);
      const int w = pos * kKeysPerWg + tid / TPT;
      if (w < key_tiles(ka.T, ka.C, ka.H)) append_key_tile<KEYD, TPT>(ka, w, tid % TPT);
      return;
    }
  }
  // XCD-aware tile order, row-major or grouped (gemm_order.h)
  const GemmTile tl = gemm_tile(blockIdx.x, nbm, nbn, int64_t(g.N) * g.K * 2);
  const int m0 = tl.m_blk * BM;
  const int n0 = tl.n_blk * BN;
  const int nkt = g.K / 64;

  // per-lane byte offsets of this wave's loads; 8 lanes fill one 128-byte
  // stage row, with the row's 16-byte chunks XOR-swizzled
  uint32_t voff[NLD];
  bool isx[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int gi = wave * NLD + i;
    const int row = 8 * gi + lane / 8;
    const int c = (lane % 8) ^ swz(row);
    isx[i] = gi < XI;
    const int rr = isx[i] ? min(m0 + row, g.M - 1) : min(n0 + row - BM, g.N - 1);
    voff[i] = uint32_t(rr * g.K + c * 8) * 2u;
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds)) + wave * NLD * 1024;
  // load i (of NLD) of slice kt into stage st
  auto dma = [&](int kt, int st, int i) __attribute__((always_inline)) {
    load_lds16_s(isx[i] ? g.x + kt * 64 : g.w + kt * 64, voff[i],
                 lds0 + st * STAGE * 2 + i * 1024);
  };

  // fragment f of substep s: f < NB is W block f, else X block f - NB
  int offr[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = (2 * s + half) ^ swz(l32);
    offr[s][0] = (BM + wn * 32 * NB + l32) * 64 + c * 8;
    offr[s][1] = (wm * 32 * MB + l32) * 64 + c * 8;
  }
  bf16x8 fr[4][FR];
  auto rd = [&](const uint16_t* L, int s, int f) __attribute__((always_inline)) {
    const int o = f < NB ? offr[s][0] + f * 32 * 64 : offr[s][1] + (f - NB) * 32 * 64;
    fr[s][f] = as_bf16x8(*reinterpret_cast<const uint4*>(L + o));
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  auto mma = [&](int s, int idx) __attribute__((always_inline)) {
    const int i = idx / MB, j = idx % MB;
    acc[i][j] = mfma32(fr[s][i], fr[s][NB + j], acc[i][j]);
  };

  // One half-slice phase: the MFMAs of substeps s0, s0 + 1 of the current
  // slice, interleaved with the reads of substeps rs0, rs0 + 1 from stage
  // RL and, when do_dma, with loads [d0, d1) of slice du into stage dst.
  // The loads sit behind uniform branches that also pin the MFMA order; the
  // MFMAs themselves are on the one path every wave takes.
  auto phase = [&](int s0, const uint16_t* RL, int rs0, bool do_dma, int du, int dst, auto d0c,
                   auto d1c) __attribute__((always_inline)) {
    constexpr int d0 = decltype(d0c)::value, d1 = decltype(d1c)::value;
    constexpr int NM = 2 * NMMA, NR = 2 * FR, ND = d1 - d0;
    static_for<0, NM>([&](auto qc) {
      constexpr int qi = decltype(qc)::value;
      static_for<qi * NR / NM, (qi + 1) * NR / NM>([&](auto rc) {
        constexpr int ri = decltype(rc)::value;
        rd(RL, rs0 + ri / FR, ri % FR);
      });
      if constexpr ((qi + 1) * ND / NM > qi * ND / NM) {
        if (do_dma) {
          static_for<qi * ND / NM, (qi + 1) * ND / NM>([&](auto dc) {
            dma(du, dst, d0 + decltype(dc)::value);
          });
        }
      }
      mma(s0 + qi / NMMA, qi % NMMA);
    });
  };
  using Z = std::integral_constant<int, 0>;
  using H = std::integral_constant<int, NLD / 2>;
  using F = std::integral_constant<int, NLD>;

  // wait for slice j (with `ahead` later slices possibly in flight) and for
  // this wave's LDS reads, then the barrier that publishes slice j
  auto sync_slice = [&](int ahead) __attribute__((always_inline)) {
    if (ahead >= LA - 1) wait_vm_lds<(LA - 1) * NLD>();
    else if (LA >= 3 && ahead == 1) wait_vm_lds<NLD>();
    else wait_vm_lds<0>();
    barrier();
  };

  // prologue: slices 0 .. LA-1, then slice 0 published, first half of
  // slice LA requested and the first two substeps of slice 0 read
  static_for<0, LA>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if (i < nkt) static_for<0, NLD>([&](auto dc) { dma(i, i, decltype(dc)::value); });
  });
  sync_slice(nkt - 1);
  if (LA < nkt) static_for<0, NLD / 2>([&](auto dc) { dma(LA, LA % STAGES, decltype(dc)::value); });
#pragma unroll
  for (int f = 0; f < FR; ++f) rd(lds, 0, f);
#pragma unroll
  for (int f = 0; f < FR; ++f) rd(lds, 1, f);

  // slice kt lives in stage st = kt % STAGES; after the last slice the
  // phase-B reads fetch a stale stage whose fragments go unused
  int st = 0;
  for (int kt = 0; kt < nkt; ++kt) {
    const int stn = st + 1 == STAGES ? 0 : st + 1;
    const int stl = st == 0 ? STAGES - 1 : st - 1;  // stage of slice kt + LA
    // A: substeps 0, 1; read substeps 2, 3; second half of slice kt + LA
    phase(0, lds + st * STAGE, 2, kt + LA < nkt, kt + LA, stl, H{}, F{});
    if (kt + 1 < nkt) sync_slice(nkt - 2 - kt);
    // B: substeps 2, 3; read substeps 0, 1 of slice kt + 1; first half of
    // slice kt + 1 + LA into the stage slice kt has just left
    phase(2, lds + stn * STAGE, 0, kt + 1 + LA < nkt, kt + 1 + LA, st, Z{}, H{});
    st = stn;
  }

  // which output of the fused projection this tile is (0 Q, 1 K, 2 V) and
  // its head; a product of fewer parts starts at part e.part0
  int which = 0, h = 0;
  if constexpr (QKV) {
    const int HD = e.H * BN;
    which = n0 / HD;
    h = (n0 - which * HD) / BN;
    which += e.part0;
  }

  // epilogue: bias, bf16, staged through LDS so each row leaves in 16-byte
  // pieces that cover it contiguously.  V^T leaves by columns instead: its
  // staging rows have an odd number of dwords, so the column reads (8 tokens
  // of one dim per 16-byte piece) hit distinct banks.
  constexpr int ESV = BN + 2;
  static_assert(BM * ESV <= STAGES * STAGE, "V staging tile fits in the ring");
  const int es = QKV && which == 2 ? ESV : ES;
  // K tiles stage the fp32 product (rows of ESF floats: the 16-byte writes of
  // 16 consecutive rows start 4 banks apart); the rotation and the one bf16
  // rounding happen on the way out, where the table rows are read coalesced
  constexpr int ESF = BN + 4;
  static_assert(BM * ESF * 2 <= STAGES * STAGE, "fp32 K staging tile fits in the ring");
  float* const ldsf = reinterpret_cast<float*>(lds);
  const bool kf32 = QKV && which == 1;
  wait_vm_lds<0>();
  barrier();
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int col = wn * 32 * NB + 32 * i + 8 * qq + 4 * half;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (g.bias && n0 + col < g.N) {  // N % 8 == 0: all four columns exist
        const uint2 b4 = *reinterpret_cast<const uint2*>(g.bias + n0 + col);
        bv[0] = bf16_lo(b4.x); bv[1] = bf16_hi(b4.x);
        bv[2] = bf16_lo(b4.y); bv[3] = bf16_hi(b4.y);
      }
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int row = wm * 32 * MB + 32 * j + l32;
        const f32x16& a4 = acc[i][j];
        if (kf32) {
          *reinterpret_cast<float4*>(ldsf + row * ESF + col) =
              make_float4(a4[4 * qq], a4[4 * qq + 1], a4[4 * qq + 2], a4[4 * qq + 3]);
          continue;
        }
        const uint32_t lo = pack_bf16x2(a4[4 * qq] + bv[0], a4[4 * qq + 1] + bv[1]);
        const uint32_t hi = pack_bf16x2(a4[4 * qq + 2] + bv[2], a4[4 * qq + 3] + bv[3]);
        if (es == ES) {
          *reinterpret_cast<uint2*>(lds + row * ES + col) = make_uint2(lo, hi);
        } else {   // 4-byte aligned only
          *reinterpret_cast<uint32_t*>(lds + row * ESV + col) = lo;
          *reinterpret_cast<uint32_t*>(lds + row * ESV + col + 2) = hi;
        }
      }
    }
  __syncthreads();
  constexpr int CPR = BN / 8;  // 16-byte pieces per tile row
  static_assert(BM * CPR % NT == 0, "row pieces split evenly over the threads");
  if constexpr (!QKV) {
#pragma unroll
    for (int it = 0; it < BM * CPR / NT; ++it) {
      const int idx = tid + NT * it;
      const int rrow = idx / CPR, c = idx % CPR;
      const int m = m0 + rrow, n = n0 + c * 8;
      if (m < g.M && n < g.N)
        *reinterpret_cast<uint4*>(g.y + int64_t(m) * g.N + n) =
            *reinterpret_cast<const uint4*>(lds + rrow * ES + c * 8);
    }
  } else if (which == 0) {
    // Q rows to q_out
#pragma unroll
    for (int it = 0; it < BM * CPR / NT; ++it) {
      const int idx = tid + NT * it;
      const int rrow = idx / CPR, c = idx % CPR;
      const int m = m0 + rrow;
      if (m < g.M)
        *reinterpret_cast<uint4*>(e.q_out + (int64_t(m) * e.H + h) * BN + c * 8) =
            *reinterpret_cast<const uint4*>(lds + rrow * ES + c * 8);
    }
  } else if (which == 1) {
    // K rows: 8 dims (4 rotation pairs) per piece, rotated in fp32 with the
    // token's table row (consecutive lanes read consecutive 16 bytes of it),
    // rounded once, into the ring slot of the token's frame
#pragma unroll
    for (int it = 0; it < BM * CPR / NT; ++it) {
      const int idx = tid + NT * it;
      const int rrow = idx / CPR, c = idx % CPR;
      const int m = m0 + rrow;
      if (m < g.M) {
        const float4 xa = *reinterpret_cast<const float4*>(ldsf + rrow * ESF + c * 8);
        const float4 xb = *reinterpret_cast<const float4*>(ldsf + rrow * ESF + c * 8 + 4);
        const int64_t trow = (int64_t(e.tab_frame) * e.T + m) * (BN / 2) + c * 4;
        const float4 cs = *reinterpret_cast<const float4*>(e.cos_tab + trow);
        const float4 sn = *reinterpret_cast<const float4*>(e.sin_tab + trow);
        const float x[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        const float c4[4] = {cs.x, cs.y, cs.z, cs.w};
        const float s4[4] = {sn.x, sn.y, sn.z, sn.w};
        float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (g.bias) {
          const uint4 b8 = *reinterpret_cast<const uint4*>(g.bias + n0 + c * 8);
          const uint32_t bw[4] = {b8.x, b8.y, b8.z, b8.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            bv[2 * k] = bf16_lo(bw[k]);
            bv[2 * k + 1] = bf16_hi(bw[k]);
          }
        }
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = x[2 * k], x1 = x[2 * k + 1];
          const float r0 = x0 * c4[k] - x1 * s4[k];
          const float r1 = x0 * s4[k] + x1 * c4[k];
          o[k] = pack_bf16x2(r0 + bv[2 * k], r1 + bv[2 * k + 1]);
        }
        const int fi = m / e.T, t = m - fi * e.T;
        *reinterpret_cast<uint4*>(
            e.k_cache + ((int64_t(e.chunk_slot[fi]) * e.H + h) * e.T + t) * BN + c * 8) =
            make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  } else {
    // V^T: piece (dim d, 8 tokens from m); 8 consecutive lanes take 8
    // consecutive token groups of one dim, so they store 128 contiguous bytes.
    // The tokens of a piece share a frame (the tile starts at a multiple of
    // 8 and T is a multiple of 8).
    constexpr int TG = BM / 8;   // token groups per tile, a multiple of 8
    static_assert(TG % 8 == 0 && BN * TG % NT == 0, "token groups in blocks of 8");
#pragma unroll
    for (int it = 0; it < BN * TG / NT; ++it) {
      const int idx = tid + NT * it;
      const int tg = (idx / (8 * BN)) * 8 + idx % 8;
      const int d = (idx / 8) % BN;
      const int m = m0 + tg * 8;
      if (m < g.M) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo = lds[(tg * 8 + 2 * k) * ESV + d];
          const uint32_t hi = lds[(tg * 8 + 2 * k + 1) * ESV + d];
          w[k] = lo | (hi << 16);
        }
        const int fi = m / e.T, t = m - fi * e.T;
        *reinterpret_cast<uint4*>(
            e.v_cache + ((int64_t(e.chunk_slot[fi]) * e.H + h) * BN + d) * e.TV + t) =
            make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

}  // namespace

// Device scratch of ust_lowrank_proj_static: the rank-r intermediate T of one
// call, for callers that cannot allocate.  Each GPU holds its own copy for
// the life of the process; kernels get its address from lowrank_scratch(),
// never from this name (in host code it is a host-side stand-in).
static __device__ __align__(256) uint16_t scratch[kLowrankScratchElems];

hipError_t lowrank_scratch(uint16_t** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = static_cast<uint16_t*>(addr[dev]);
  return hipSuccess;
}

hipError_t launch_qkv_append(const GemmArgs& g, const QkvEpilogue& e, hipStream_t s) {
  // one head per output tile: the tile's feature width is the head size
  if (e.D == 128) {
    dim3 grid(((g.M + 255) / 256) * (g.N / 128));
    hipLaunchKernelGGL((gemm_nt_dma_kernel<256, 128, 3, true, 4, 2>), grid, dim3(512), 0, s, g, e,
                       AppendArgs{});
  } else {
    dim3 grid(((g.M + 191) / 192) * (g.N / 64));
    hipLaunchKernelGGL((gemm_nt_dma_kernel<192, 64, 4, true, 2, 2>), grid, dim3(256), 0, s, g, e,
                       AppendArgs{});
  }
  return hipGetLastError();
}

bool gemm_nt_pipelined(const GemmArgs& g) {
  return g.K % 64 == 0 && int64_t(g.M) * g.K < (int64_t(1) << 31) &&
         int64_t(g.N) * g.K < (int64_t(1) << 31);
}

namespace {

// the pipelined kernel for this shape, with key_wgs key-append workgroups
// after its tiles (KEYD = head size, 0 for none)
template <int KEYD>
void launch_pipelined(const GemmArgs& g, const AppendArgs& ka, int key_wgs, hipStream_t s) {
  // narrow outputs (the rank-r factor product) get 128 x 128 tiles (148
  // workgroups at 4680 x 512), wide ones 256 x 128 (228 at 4680 x 1536):
  // one round on 256 CUs, 8 waves each
  const QkvEpilogue none{};
  if (g.N <= 768) {
    dim3 grid(((g.M + 127) / 128) * ((g.N + 127) / 128) + key_wgs);
    hipLaunchKernelGGL((gemm_nt_dma_kernel<128, 128, 3, false, 4, 2, KEYD>), grid, dim3(512), 0, s,
                       g, none, ka);
  } else {
    dim3 grid(((g.M + 255) / 256) * ((g.N + 127) / 128) + key_wgs);
    hipLaunchKernelGGL((gemm_nt_dma_kernel<256, 128, 3, false, 4, 2, KEYD>), grid, dim3(512), 0, s,
                       g, none, ka);
  }
}

}  // namespace

hipError_t launch_gemm_nt_keys(const GemmArgs& g, const AppendArgs& ka, hipStream_t s) {
  if (!gemm_nt_pipelined(g)) return hipErrorInvalidValue;
  const int key_wgs = (key_tiles(ka.T, ka.C, ka.H) + kKeysPerWg - 1) / kKeysPerWg;
  if (ka.D == 128) launch_pipelined<128>(g, ka, key_wgs, s);
  else launch_pipelined<64>(g, ka, key_wgs, s);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const GemmArgs& g, hipStream_t s) {
  if (gemm_nt_pipelined(g)) {
    launch_pipelined<0>(g, AppendArgs{}, 0, s);
    return hipGetLastError();
  }
  const int nbn = (g.N + kBN - 1) / kBN;
  const int tiles128 = ((g.M + 127) / 128) * nbn;
  // enough workgroups to cover the 256 CUs twice, else halve the row tile
  if (tiles128 >= 512) {
    dim3 grid(tiles128);
    hipLaunchKernelGGL(gemm_nt_kernel<2>, grid, dim3(256), 0, s, g);
  } else {
    dim3 grid(((g.M + 63) / 64) * nbn);
    hipLaunchKernelGGL(gemm_nt_kernel<1>, grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace ust
