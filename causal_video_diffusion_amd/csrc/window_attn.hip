// Chunk-causal attention over the limited temporal window (UnStep, abstract:
// "limiting the temporal window retained in the attention KV cache"; chunks
// of three latent frames, Table 3), with the query RoPE fused into the Q-tile
// load (abstract: fused RoPE with cached coefficients).
//
// Design (gfx950, wave64, bf16 MFMA 32x32x16 with fp32 accumulation):
//  * A workgroup of 4 waves owns 128 queries of one head; each wave owns 32.
//    The window's keys form one virtual sequence (frame after frame, each
//    frame's T keys read from its ring slot), walked in tiles of 64 keys;
//    only the last tile can be partial, so a tile may straddle frames.
//  * Scores are computed transposed, S^T = K Q^T: the MFMA output puts one
//    query per lane (column) and 16 keys per lane in registers, so the row
//    max and row sum of the online softmax are in-lane reductions plus one
//    swap between lane l and l^32.  The query rotation, the softmax scale and
//    log2(e) are folded into the bf16 query fragments once per workgroup.
//  * The A operand rows of S^T are permuted (bits 2 and 3 of the key index
//    swapped) so that each lane's 8 score registers of one 16-key group hold
//    8 consecutive keys.  Those registers, rounded to bf16, are directly the
//    B operand of O^T = V^T P^T; V^T comes from the transposed value cache,
//    so neither P nor V is transposed in LDS.
//  * K and V^T tiles are staged through LDS (XOR-swizzled 16-byte chunks,
//    bank-conflict-free for the MFMA operand reads), double-buffered with the
//    next tile's global loads in flight during the current tile's math.
//  * Workgroups are numbered so that each XCD (8 per chip, dispatched round
//    robin) gets a contiguous run of (head, query tile) work: the workgroups
//    sharing a head's K/V stream share one L2.

#include "ust_device.h"
#include "ust_internal.h"

namespace ust {
namespace {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per tile

// swap bits 2 and 3 of a row index within a 32-row MFMA block
__device__ __forceinline__ int perm_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}
// XOR key of a K-tile row's 16-byte chunks (bits 0, 1, 3 of the row)
__device__ __forceinline__ int kswz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }

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

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
window_attn_kernel(AttnArgs a) {
  constexpr int KS = D / 16;            // k-steps of the score product
  constexpr int DB = D / 32;            // 32-row blocks of O^T
  constexpr int KCH = D / 8;            // 16-byte chunks per key row
  constexpr int KITEMS = kBN * KCH / 256;   // K-tile chunks per thread
  constexpr int VITEMS = D * 8 / 256;       // V^T-tile chunks per thread
  constexpr int KTILE = kBN * D;        // elements per tile
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][KTILE];
  __shared__ int64_t kbase[UST_MAX_WINDOW_FRAMES];
  __shared__ int64_t vbase[UST_MAX_WINDOW_FRAMES];

  const int nqt = (a.NQ + kBM - 1) / kBM;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int h = w / nqt;
  const int q0 = (w % nqt) * kBM;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int T = a.T;
  const int nk = a.n_frames * T;
  const int ntiles = (nk + kBN - 1) / kBN;

  for (int i = tid; i < a.n_frames; i += 256) {
    kbase[i] = (int64_t(a.slots[i]) * a.H + h) * T * D;
    vbase[i] = (int64_t(a.slots[i]) * a.H + h) * D * a.TV;
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

  // ---- per-thread cursors of the tile chunks this thread loads ----
  // K items: key kl = tid / KCH + (256 / KCH) * it, chunk dc = tid % KCH
  // V items: dim d = tid / 8 + 32 * it, key chunk kc = tid % 8 (keys 8kc..8kc+7)
  const int k_dc = tid % KCH;
  const int k_kl0 = tid / KCH;
  const int v_kc = tid % 8;
  const int v_d0 = tid / 8;
  int kf[KITEMS], kt[KITEMS];          // (window frame, token) of each K item
#pragma unroll
  for (int it = 0; it < KITEMS; ++it) {
    const int m = k_kl0 + (256 / KCH) * it;
    kf[it] = m / T;
    kt[it] = m % T;
  }
  int vf = (8 * v_kc) / T, vt = (8 * v_kc) % T;

  uint4 kreg[KITEMS], vreg[VITEMS];
  auto gload = [&]() {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      kreg[it] = make_uint4(0, 0, 0, 0);
      if (kf[it] < a.n_frames)
        kreg[it] = *reinterpret_cast<const uint4*>(a.k_cache + kbase[kf[it]] + int64_t(kt[it]) * D + k_dc * 8);
    }
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      vreg[it] = make_uint4(0, 0, 0, 0);
      if (vf < a.n_frames)
        vreg[it] = *reinterpret_cast<const uint4*>(a.v_cache + vbase[vf] + int64_t(v_d0 + 32 * it) * a.TV + vt);
    }
  };
  auto advance = [&]() {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      kt[it] += kBN;
      while (kt[it] >= T) { kt[it] -= T; ++kf[it]; }
    }
    vt += kBN;
    while (vt >= T) { vt -= T; ++vf; }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int kl = k_kl0 + (256 / KCH) * it;
      *reinterpret_cast<uint4*>(&lds_k[buf][kl * D + ((k_dc ^ kswz(kl)) * 8)]) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int d = v_d0 + 32 * it;
      *reinterpret_cast<uint4*>(&lds_v[buf][d * kBN + ((v_kc ^ (d & 7)) * 8)]) = vreg[it];
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float mrow = -INFINITY;   // running max (log2 units) of this lane's query
  float lrow = 0.f;         // this lane's share of the running sum

  gload();
  advance();
  lstore(0);

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    __syncthreads();
    const bool more = j + 1 < ntiles;
    if (more) {
      gload();
      advance();
    }

    // ---- S^T = K Q^T for the tile's two 32-key blocks ----
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      const int kl = 32 * kb + perm_row(l32);
      const uint16_t* krow = &lds_k[buf][kl * D];
      const int sw = kswz(kl);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int dc = 2 * s + half;
        const bf16x8 kfrag = as_bf16x8(*reinterpret_cast<const uint4*>(krow + ((dc ^ sw) * 8)));
        sacc[kb] = mfma32(kfrag, qf[s], sacc[kb]);
      }
    }

    // ---- mask the keys past the window end (last tile only) ----
    if (j * kBN + kBN > nk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * kBN + 32 * kb + 16 * (r / 8) + 8 * half + (r % 8);
          if (key >= nk) sacc[kb][r] = -INFINITY;
        }
    }

    // ---- online softmax (base 2) ----
    float tmax = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[kb][r]);
    tmax = pair_max(tmax);
    const float mnew = fmaxf(mrow, tmax);
    const float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
    mrow = mnew;
    float psum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[kb][8 * g + 2 * e] - mnew);
          const float p1 = __builtin_amdgcn_exp2f(sacc[kb][8 * g + 2 * e + 1] - mnew);
          psum += p0 + p1;
          pk[e] = pack_bf16x2(p0, p1);
        }
        pf[kb][g] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
      }
    lrow = lrow * alpha + psum;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int kc = 4 * kb + 2 * g + half;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const int d = 32 * b + l32;
          const bf16x8 vfrag =
              as_bf16x8(*reinterpret_cast<const uint4*>(&lds_v[buf][d * kBN + ((kc ^ (d & 7)) * 8)]));
          oacc[b] = mfma32(vfrag, pf[kb][g], oacc[b]);
        }
      }

    if (more) lstore(buf ^ 1);
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
      a.lse[int64_t(h) * a.NQ + qn] = (mrow + __builtin_log2f(ltot)) * 0.6931471805599453f;
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
