// Chunk-causal attention over the limited temporal window (UnStep, abstract:
// "limiting the temporal window retained in the attention KV cache"; chunks
// of three latent frames, Table 3), with the query RoPE fused into the Q-tile
// load (abstract: fused RoPE with cached coefficients).
//
// Design (gfx950, wave64, bf16 MFMA 32x32x16 with fp32 accumulation):
//  * A workgroup of 4 waves owns 128 queries of one head; each wave owns 32.
//    Two workgroups share a CU (2 waves per SIMD), so one wave's softmax
//    VALU work overlaps the other's MFMA work.
//  * The window's keys form one virtual sequence (frame after frame, each
//    frame's T keys read from its ring slot), walked in tiles of 64 keys;
//    only the last tile can be partial, and a tile may straddle frames.
//  * Scores are computed transposed, S^T = K Q^T: the MFMA output puts one
//    query per lane (column) and 16 keys per lane in registers, so the row
//    max and row sum are in-lane reductions plus one exchange between lanes
//    l and l^32.  The query rotation, the softmax scale and log2(e) are
//    folded into the bf16 query fragments once per workgroup.
//  * The score accumulators start at -m (the lane's running reference max),
//    so the MFMA yields s - m directly.  The reference only moves when a
//    tile's scores exceed it by more than 2^8 (and on the first tile), so the
//    O/l rescale is skipped on almost every tile; the final normalisation by
//    the running sum makes the result exact regardless of the reference.
//  * The A-operand rows of S^T are permuted (bits 2 and 3 of the key index
//    swapped) so that each lane's 8 score registers of one 16-key group hold
//    8 consecutive keys: those registers, rounded to bf16, are directly the
//    B operand of O^T = V^T P^T.  V^T comes from the transposed value cache,
//    so neither P nor V is transposed on chip.  The row sum is accumulated
//    from the same bf16 pairs with v_dot2_f32_bf16.
//  * K and V^T tiles go straight from global memory to LDS
//    (global_load_lds_dwordx4, no register staging), double-buffered, with
//    16-byte chunks XOR-swizzled so that every 16-lane group of an MFMA
//    operand read touches 64 distinct banks.  Tiles inside one frame use a
//    uniform base address plus per-lane constant offsets.
//  * Workgroups are numbered so that each XCD (8 per chip, dispatched round
//    robin) gets a contiguous run of (head, query tile) work: the workgroups
//    streaming one head's K/V share an L2.

#include <type_traits>

#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr float kRescale = 8.0f;  // move the reference max when exceeded (log2 units)

typedef __attribute__((address_space(3))) void lds_void;

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

__device__ __forceinline__ void load_lds16(const uint16_t* g, uint16_t* l) {
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(g), (lds_void*)(l), 16, 0, 0);
}

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
window_attn_kernel(AttnArgs a) {
  constexpr int KS = D / 16;                          // k-steps of the score product
  constexpr int DB = D / 32;                          // 32-row blocks of O^T
  constexpr int KCPR = D / 8;                         // 16-byte chunks per key row
  constexpr int KRPI = 64 / KCPR;                     // key rows per 1 KB load
  constexpr int KINST = kBN * D * 2 / 1024 / kWaves;  // K loads per wave per tile
  constexpr int VINST = D * kBN * 2 / 1024 / kWaves;  // V^T loads per wave per tile
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k[2][kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v[2][D * kBN];
  __shared__ uint32_t kbase[UST_MAX_WINDOW_FRAMES];
  __shared__ uint32_t vbase[UST_MAX_WINDOW_FRAMES];

  const int nqt = (a.NQ + kBM - 1) / kBM;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int h = w / nqt;
  const int q0 = (w % nqt) * kBM;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int T = a.T;
  const int TV = a.TV;
  const int nk = a.n_frames * T;
  const int ntiles = (nk + kBN - 1) / kBN;

  for (int i = tid; i < a.n_frames; i += 256) {
    kbase[i] = uint32_t((a.slots[i] * a.H + h) * T * D);
    vbase[i] = uint32_t((a.slots[i] * a.H + h) * D * TV);
  }

  // ---- query fragments: RoPE at the query's own position, scale, bf16 ----
  const int qn = q0 + wave * 32 + l32;
  const bool qvalid = qn < a.NQ;
  bf16x8 qf[KS];
  {
    const uint16_t* qp = a.q + (int64_t(qn) * a.H + h) * D;
    const int64_t trow = (int64_t(a.frame_start) * T + qn) * (D / 2);
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

  // ---- per-lane constants of the tile loads ----
  // K load i of this wave fills LDS bytes [(wave*KINST + i) KB, +1 KB): key row
  // krow[i], 16-byte chunk kdc[i] (logical; stored at the lane's position).
  int krow[KINST], koff[KINST];
#pragma unroll
  for (int i = 0; i < KINST; ++i) {
    const int row = KRPI * (wave * KINST + i) + lane / KCPR;
    const int dc = (lane % KCPR) ^ kswz<D>(row);
    krow[i] = row;
    koff[i] = row * D + dc * 8;
  }
  // V^T load i: dimension vd[i], 8-key chunk vkc[i]
  int vd[VINST], vkc[VINST], voff[VINST];
#pragma unroll
  for (int i = 0; i < VINST; ++i) {
    const int d = 8 * (wave * VINST + i) + lane / 8;
    const int kc = (lane % 8) ^ vswz(d);
    vd[i] = d;
    vkc[i] = kc;
    voff[i] = d * TV + kc * 8;
  }

  // Issue the global->LDS loads of tile (fi, t0) into buffer buf.
  auto issue = [&](int j, int fi, int t0, int buf) {
    uint16_t* lk = &lds_k[buf][wave * KINST * 512];
    uint16_t* lv = &lds_v[buf][wave * VINST * 512];
    if (t0 + kBN <= T && j * kBN + kBN <= nk) {
      // whole tile inside frame fi: uniform base + lane constants
      const uint16_t* kb = a.k_cache + kbase[fi] + uint32_t(t0 * D);
      const uint16_t* vb = a.v_cache + vbase[fi] + uint32_t(t0);
#pragma unroll
      for (int i = 0; i < KINST; ++i) load_lds16(kb + koff[i], lk + i * 512);
#pragma unroll
      for (int i = 0; i < VINST; ++i) load_lds16(vb + voff[i], lv + i * 512);
    } else {
      // straddles frames or runs past the window: per-lane frame lookup;
      // keys past the window are pointed at the window's first key (finite
      // data whose probability is masked to zero)
#pragma unroll
      for (int i = 0; i < KINST; ++i) {
        int tt = t0 + krow[i], f = fi;
        while (tt >= T) { tt -= T; ++f; }
        if (f >= a.n_frames) { f = 0; tt = 0; }
        load_lds16(a.k_cache + kbase[f] + uint32_t(tt * D) + (koff[i] - krow[i] * D), lk + i * 512);
      }
#pragma unroll
      for (int i = 0; i < VINST; ++i) {
        int tt = t0 + 8 * vkc[i], f = fi;
        while (tt >= T) { tt -= T; ++f; }
        if (f >= a.n_frames) { f = 0; tt = 0; }
        load_lds16(a.v_cache + vbase[f] + uint32_t(tt) + uint32_t(vd[i] * TV), lv + i * 512);
      }
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float mref = 0.f;   // reference max (log2 units) of this lane's query
  float lrow = 0.f;   // this lane's share of the running sum, relative to mref

  int fi = 0, t0 = 0;           // frame index and token of the next tile to load
  issue(0, fi, t0, 0);
  t0 += kBN;
  while (t0 >= T) { t0 -= T; ++fi; }

  // Element offsets of this lane's MFMA operand fragments within a tile
  // buffer (fixed across tiles).  Key block kb adds 32 rows (kswz is the same
  // for rows r and r + 32) and O^T block b adds 32 dims (vswz likewise), so
  // those and the buffer index fold into the ds_read immediate offsets.
  int koffr[KS], voffr[4];
  {
    const int row = perm_row(l32);
#pragma unroll
    for (int s = 0; s < KS; ++s) koffr[s] = row * D + (((2 * s + half) ^ kswz<D>(row)) * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) voffr[q] = l32 * kBN + (((2 * q + half) ^ vswz(l32)) * 8);
  }

  // One tile: scores, online softmax, PV.  MASKED is the last tile, whose
  // keys past the window end get probability zero.
  auto tile = [&](int j, auto masked_tag, auto buf_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int buf = decltype(buf_tag)::value;   // == j & 1
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile j are in LDS
    __syncthreads();                 // ... and every wave's; buf^1 is free
    if (!MASKED && j + 1 < ntiles) {
      issue(j + 1, fi, t0, buf ^ 1);
      t0 += kBN;
      while (t0 >= T) { t0 -= T; ++fi; }
    }
    const uint16_t* K = lds_k[buf];
    const uint16_t* V = lds_v[buf];

    // ---- S^T - mref = K Q^T + (-mref), two 32-key blocks ----
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = -mref;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf =
            as_bf16x8(*reinterpret_cast<const uint4*>(K + koffr[s] + kb * 32 * D));
        sacc[kb] = mfma32(kf, qf[s], sacc[kb]);
      }
    }

    if constexpr (MASKED) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * kBN + 32 * kb + 16 * (r / 8) + 8 * half + (r % 8);
          if (key >= nk) sacc[kb][r] = -INFINITY;
        }
    }

    // ---- tile max relative to the reference; move it if needed ----
    float tmax = sacc[0][0];
#pragma unroll
    for (int r = 1; r < 15; r += 2) tmax = fmaxf(fmaxf(tmax, sacc[0][r]), sacc[0][r + 1]);
    tmax = fmaxf(fmaxf(tmax, sacc[0][15]), sacc[1][0]);
#pragma unroll
    for (int r = 1; r < 15; r += 2) tmax = fmaxf(fmaxf(tmax, sacc[1][r]), sacc[1][r + 1]);
    tmax = fmaxf(tmax, sacc[1][15]);
    tmax = pair_max(tmax);
    const bool need = (j == 0) || (tmax > kRescale);
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float shift = need ? tmax : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      mref += shift;
      lrow *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] -= shift;
    }

    // ---- probabilities (bf16) and their sum ----
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16x2 pp;
          pp[0] = (__bf16)__builtin_amdgcn_exp2f(sacc[kb][8 * g + 2 * e]);
          pp[1] = (__bf16)__builtin_amdgcn_exp2f(sacc[kb][8 * g + 2 * e + 1]);
          lrow = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, lrow, false);
          pk[e] = __builtin_bit_cast(uint32_t, pp);
        }
        pf[kb][g] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
      }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          // key chunk 4 kb + 2 g + half of dim 32 b + l32
          const bf16x8 vf = as_bf16x8(
              *reinterpret_cast<const uint4*>(V + voffr[2 * kb + g] + b * 32 * kBN));
          oacc[b] = mfma32(vf, pf[kb][g], oacc[b]);
        }
      }
  };

  // unrolled by two so that the LDS buffer of each tile is a compile-time
  // constant (folded into the ds_read offsets)
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  const bool last_partial = ntiles * kBN > nk;
  const int nfull = last_partial ? ntiles - 1 : ntiles;
  int j = 0;
  for (; j + 1 < nfull; j += 2) {
    tile(j, std::false_type{}, B0{});
    tile(j + 1, std::false_type{}, B1{});
  }
  if (j < nfull) {
    tile(j, std::false_type{}, B0{});
    ++j;
  }
  if (last_partial) {
    if (j & 1) tile(j, std::true_type{}, B1{});
    else tile(j, std::true_type{}, B0{});
  }

  // ---- epilogue: normalise, store bf16 O and the log-sum-exp ----
  const float ltot = pair_sum(lrow);
  const float inv = 1.f / ltot;
  if (qvalid) {
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
    if (a.lse && half == 0)
      a.lse[int64_t(h) * a.NQ + qn] = (mref + __builtin_log2f(ltot)) * 0.6931471805599453f;
  }
}

}  // namespace

hipError_t launch_window_attn(const AttnArgs& a, hipStream_t s) {
  const int nqt = (a.NQ + kBM - 1) / kBM;
  dim3 grid(nqt * a.H);
  if (a.D == 128)
    hipLaunchKernelGGL(window_attn_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(window_attn_kernel<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ust
