// Internal interface between the C-ABI entry points (ust_host.cpp) and the
// kernel launchers (*.hip).  Arguments reaching a launcher are validated.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/ust.h"
#include "../../include/ust_calib.h"

namespace ust {

struct RopeTableArgs {
  float* cos_out;
  float* sin_out;
  int32_t first_frame;       // absolute frame of row 0
  int32_t n_frames, grid_h, grid_w;
  int32_t pairs_t, pairs_h, pairs_w;
  double theta;
};

struct AppendArgs {
  const uint16_t* k_new;     // [C*T][H][D]
  const uint16_t* v_new;     // [C*T][H][D]
  const float* cos_tab;      // [F][T][P], row f = frame tab_first + f
  const float* sin_tab;
  uint16_t* k_cache;         // [slots][H][T][D]
  uint16_t* v_cache;         // [slots][H][D][TV]
  int32_t T, TV, H, D, C;
  int32_t tab_frame;         // table row frame of the chunk's first token
  int32_t chunk_slot[8];     // slot of each chunk frame (C <= 8)
  int32_t with_v;            // 0: keys only (v_new unused)
};

struct AttnArgs {
  const uint16_t* q;         // [NQ][H][D] un-rotated
  const float* cos_tab;      // [F][T][P], row f = frame tab_first + f
  const float* sin_tab;
  const uint16_t* k_cache;   // [slots][H][T][D]
  const uint16_t* v_cache;   // [slots][H][D][TV]
  uint16_t* out;             // [NQ][H][D]
  float* lse;                // [H][NQ] or nullptr
  int32_t T, TV, H, D, NQ;
  int32_t tab_frame;         // table row frame of query token 0
  int32_t n_frames;          // frames in the window
  float qscale;              // scale * log2(e), folded into the rotated query
  // Schedule (attn_schedule.h).  work_o == nullptr: one workgroup per
  // (head, query tile).  Otherwise the plan for n_wg workgroups; a (head,
  // query tile) split between workgroups leaves normalised partial outputs
  // and their log-sum-exps here for the merge kernel.
  float* work_o;             // [2 n_wg][256][D] fp32
  float* work_l;             // [2 n_wg][256] fp32 (natural log), set by the launcher
  int32_t n_wg;              // requested workgroups (>= 1), set by the launcher when unsplit
  int32_t slots[UST_MAX_WINDOW_FRAMES];
};

struct GemmArgs {
  const uint16_t* x;         // [M][K]
  const uint16_t* w;         // [N][K]
  const uint16_t* bias;      // [N] or nullptr
  uint16_t* y;               // [M][N]
  int32_t M, N, K;
};

// Epilogue of the fused Q/K/V projection: output features [0, HD) are Q,
// [HD, 2HD) K, [2HD, 3HD) V, one head per tile (the tile's feature width is
// D).  Q goes to q_out [M][H][D]; K is rotated and V transposed into the
// chunk's ring slots, as ust_kv_append stores them.
struct QkvEpilogue {
  uint16_t* q_out;           // [M][H][D]
  uint16_t* k_cache;         // [slots][H][T][D]
  uint16_t* v_cache;         // [slots][H][D][TV]
  const float* cos_tab;      // [F][T][P], row f = frame tab_first + f
  const float* sin_tab;
  int32_t T, TV, H, D;
  int32_t tab_frame;         // table row frame of the chunk's first token
  int32_t chunk_slot[8];     // slot of each chunk frame
  int32_t part0;             // output part of the product's first head-wide tiles: 0 Q, 1 K, 2 V
};

// One sampler step: x0_hat = x - sigma v, x_next = keep x0_hat + sigma_next
// noise (keep = 1 - sigma_next, rounded to fp32 by the caller); noise NULL
// means sigma_next = 0 and x_next = x0_hat.  x0_out may be NULL.
struct FlowStepArgs {
  const float* x;            // [n]
  const uint16_t* v;         // [n] bf16
  const float* noise;        // [n] or nullptr
  float* x0_out;             // [n] or nullptr
  float* x_next;             // [n]
  int64_t n;
  float sigma, sigma_next, keep;
};

// Causal 3-D convolution (conv3d.hip); validated: Ci in {16, 32, 64, 128},
// Co a multiple of 128, 16-byte aligned pointers, T*H*W < 2^31
struct ConvArgs {
  const uint16_t* x;         // [T][H][W][Ci] bf16
  const uint16_t* w;         // [Co][3][3][3][Ci] bf16
  const float* bias;         // [Co] or nullptr
  uint16_t* y;               // [T][H][W][Co] bf16
  int32_t T, H, W, Ci, Co;
  int32_t hist;              // 1: x starts with two history frames ([T+2][H][W][Ci])
};

hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t s);
hipError_t launch_conv3d_causal(const ConvArgs& a, hipStream_t s);
hipError_t launch_flow_step(const FlowStepArgs& a, hipStream_t s);
// X [M][K] W [3HD][K]^T with the QKV epilogue; K % 64 == 0, D in {64, 128}
hipError_t launch_qkv_append(const GemmArgs& g, const QkvEpilogue& e, hipStream_t s);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_window_attn(const AttnArgs& a, hipStream_t s);
// workspace bytes of the key-split schedule over n_wg workgroups
size_t window_attn_work_bytes(int32_t head_dim, int32_t n_wg);
hipError_t launch_gemm_nt(const GemmArgs& a, hipStream_t s);
// Whether launch_gemm_nt runs the pipelined kernel for this shape.
bool gemm_nt_pipelined(const GemmArgs& a);
// launch_gemm_nt's pipelined product with the keys of ka (with_v 0) rotated
// and appended by extra workgroups of the same launch; for shapes where
// gemm_nt_pipelined holds (hipErrorInvalidValue otherwise, nothing launched).
hipError_t launch_gemm_nt_keys(const GemmArgs& a, const AppendArgs& ka, hipStream_t s);
// bf16 elements of the device scratch behind ust_lowrank_proj_static
constexpr size_t kLowrankScratchElems = size_t(UST_LOWRANK_STATIC_MAX_ELEMS);
// that scratch's address on the current device (looked up once per device)
hipError_t lowrank_scratch(uint16_t** ptr);
// measurement aid (calib.hip): MFMA-only kernel and its flop count
hipError_t launch_calib_mfma(int32_t n_wg, int32_t iters, float* out, hipStream_t s);
double calib_mfma_flops(int32_t n_wg, int32_t iters);

}  // namespace ust
