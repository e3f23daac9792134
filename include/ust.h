/*
 * ust.h - windowed chunk attention for causal video diffusion on MI355X.
 *
 * The per-chunk DiT self-attention path of UnStep (arXiv 2609.32518,
 * "UnStep: Training-Free Acceleration of Causal Video Diffusion with Fewer
 * Steps Than Distillation"), as a C ABI over hand-written gfx950 kernels:
 *
 *   ust_rope_table_build  cos/sin coefficients of the 3-D RoPE for a range of
 *                         frames, cached (abstract: RoPE from precomputed
 *                         coefficients); a chunk's own frames suffice
 *   ust_kv_append         RoPE the chunk's keys and store keys and values in
 *                         the frame slots of a KV ring (abstract: the KV
 *                         cache and its indexing)
 *   ust_window_attn       RoPE the chunk's queries and attend over the limited
 *                         temporal window: sink frames, recent frames, and
 *                         the chunk itself, bidirectional inside the window
 *                         (abstract: the attention KV cache keeps a limited
 *                         window of latent frames; Table 3: chunks of three
 *                         latent frames)
 *   ust_window_attn_split the same attention with the work divided evenly over
 *                         the workgroups (split key ranges merged afterwards)
 *   ust_qkv_append        the chunk's Q/K/V projections with the key RoPE and
 *                         the K/V append fused into the product's epilogue
 *   ust_lowrank_proj      Y = (X A_r) B_r, the truncated-SVD value and output
 *                         projections (abstract; Table 5 caption)
 *   ust_lowrank_proj_v_append  the value projection with the values stored
 *                         straight into the ring's slots, and the keys' RoPE
 *                         and append in the same call
 *   ust_lowrank_proj_static  the same with the intermediate in a fixed device
 *                         array, for callers that cannot allocate
 *   ust_flow_step         one step of the chunk sampler: denoised estimate and
 *                         renoising (Table 4; abstract)
 *   ust_sigma_schedule    the sampler's noise levels (host only; Table 4)
 *   ust_conv3d_causal     the decoder's causal 3-D convolution, channels last
 *                         (abstract: VAE decoding runtime stack; Table 3)
 *   ust_conv3d_causal_stream  the same for a clip decoded chunk by chunk, two
 *                         history frames in place of the zero padding
 *
 * Conventions (all entry points):
 *  - Device pointers are caller-owned.  The library never allocates, frees
 *    or keeps them past the call.  No entry point allocates device memory;
 *    ust_lowrank_proj_static uses a fixed device array of the library's
 *    own instead of a caller buffer.
 *  - Every call validates all of its arguments on the host before anything
 *    is launched; on an error nothing is launched, the status says which
 *    class of error, and ust_last_error() (thread-local) gives the detail.
 *  - Work is queued asynchronously on `stream` (0 = the null stream) and the
 *    call returns without synchronising.  Buffers must stay valid until the
 *    stream has passed the work.  A fault inside a kernel surfaces at the
 *    caller's next synchronisation, not here.
 *  - bf16 is bfloat16 (1-8-7) stored as 16-bit words; fp32 is IEEE binary32.
 *  - Every device pointer must be 16-byte aligned.
 *  - Apart from that array (and the per-device table of its addresses) the
 *    library holds no mutable global state and is safe to call from several
 *    host threads (each on its own stream).
 *  - No C++ exception crosses the ABI.
 *
 * Token order: a chunk has chunk_frames * T tokens, T = grid_h * grid_w.
 * Token n is latent frame frame_start + n / T at row y = (n % T) / grid_w,
 * column x = (n % T) % grid_w.  Per-token head vectors are stored
 * [chunk_frames * T][n_heads][head_dim] (the row-major output of a projection
 * to n_heads * head_dim columns).
 */
#ifndef UST_H
#define UST_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ust_status {
  UST_OK = 0,
  UST_E_NULL = 1,        /* a required pointer is NULL                         */
  UST_E_SHAPE = 2,       /* a size is non-positive or sizes disagree           */
  UST_E_RANGE = 3,       /* a frame lies outside the RoPE table, or a window
                            frame is no longer held by the ring                */
  UST_E_ALIGN = 4,       /* a device pointer is not 16-byte aligned            */
  UST_E_UNSUPPORTED = 5, /* well-formed but not supported (see each call)      */
  UST_E_HIP = 6          /* a HIP runtime call failed (e.g. the launch)        */
} ust_status;

/* Geometry of one DiT self-attention layer.
 * The head dimension is split into P = head_dim / 2 rotation pairs: the first
 * pairs_t rotate with the latent-frame index, the next pairs_h with the token
 * row, the last pairs_w with the token column; pair j of an axis with n pairs
 * turns by position * theta^(-j/n).  Pairs are adjacent elements (2p, 2p+1).
 * (The axis split is the 3-D RoPE of the Wan-family DiT the paper runs,
 * Table 1 caption.) */
typedef struct ust_geom {
  int32_t grid_h, grid_w;            /* tokens per latent frame T = grid_h*grid_w */
  int32_t n_heads, head_dim;         /* head_dim must be 64 or 128                */
  int32_t pairs_t, pairs_h, pairs_w; /* pairs_t + pairs_h + pairs_w == head_dim/2 */
  int32_t chunk_frames;              /* latent frames per causal chunk (3)        */
} ust_geom;

/* KV ring, caller-owned device memory.  One slot per latent frame.
 * Frame f lives in slot f if f < n_sink (sink frames are pinned), else in
 * slot n_sink + (f - n_sink) mod (n_slots - n_sink).
 *   k: bf16 [n_slots][n_heads][T][head_dim]        RoPE-rotated keys
 *   v: bf16 [n_slots][n_heads][head_dim][ust_v_row_len(T)]
 *      values stored transposed (dimension-major, token fastest); entries at
 *      token >= T are padding that no call reads or writes. */
typedef struct ust_kv {
  void* k;
  void* v;
  int32_t n_slots;
  int32_t n_sink;
} ust_kv;

/* Most frames one window may hold (sink + recent + chunk). */
#define UST_MAX_WINDOW_FRAMES 128

/* Tokens per row of the transposed value cache: T rounded up to a multiple
 * of 64.  Returns -1 if T <= 0. */
int32_t ust_v_row_len(int32_t tokens_per_frame);

/* Build the cached RoPE coefficients (abstract: RoPE is applied from
 * precomputed coefficients) for the frames first_frame .. first_frame +
 * n_frames - 1.  For every such frame f, row y, column x and pair p,
 * angle = pos * theta^(-j/n) with (pos, j, n) given by p's axis as in
 * ust_geom (pos = f, the absolute frame, on the temporal axis); computed in
 * fp64 and rounded to fp32.  The consumers read only the rows of the
 * chunk they process, so a table of one chunk's frames, built per chunk,
 * serves a stream of any length; a table from frame 0 serves every chunk
 * whose frames it covers.
 *   cos_out, sin_out: fp32 [n_frames][grid_h][grid_w][head_dim/2], written;
 *         row i holds frame first_frame + i.
 * Errors: NULL pointers; n_frames <= 0 or bad geometry (UST_E_SHAPE);
 * theta <= 0, first_frame < 0 or a frame past INT32_MAX (UST_E_RANGE);
 * head_dim not 64/128 (UST_E_UNSUPPORTED). */
ust_status ust_rope_table_build(const ust_geom* g, int32_t first_frame, int32_t n_frames,
                                double theta, float* cos_out, float* sin_out,
                                hipStream_t stream);

/* Append one chunk to the KV ring (abstract: the KV cache and its indexing).
 * For every token n of the chunk (frame f = frame_start + n / T at (y, x))
 * and head h:
 *   kv.k[slot(f)][h][n % T][:]  = bf16_rne(RoPE(f, y, x) k_new[n][h][:])
 *   kv.v[slot(f)][h][:][n % T]  = v_new[n][h][:]          (bit copy)
 * The rotation is done in fp32 with the table's coefficients.  Slots of
 * other frames are not touched.
 *   k_new, v_new: bf16 [chunk_frames*T][n_heads][head_dim], read.  v_new may
 *         be NULL: then only the keys are appended (the values reach the
 *         ring another way, e.g. ust_lowrank_proj_v_append).
 *   cos_tab, sin_tab: a table of ust_rope_table_build holding the frames
 *         tab_first_frame .. tab_first_frame + n_tab_frames - 1; only the
 *         chunk's own rows are read.
 * Errors: NULL k_new or table; frame_start < 0, tab_first_frame < 0 or the
 * chunk's frames not all in the table (UST_E_RANGE); n_slots - n_sink <
 * chunk_frames or n_sink < 0 (UST_E_RANGE); misaligned pointers; T not a
 * multiple of 8 or head_dim not 64/128 (UST_E_UNSUPPORTED). */
ust_status ust_kv_append(const ust_geom* g, const ust_kv* kv,
                         const void* k_new, const void* v_new,
                         const float* cos_tab, const float* sin_tab,
                         int32_t tab_first_frame, int32_t n_tab_frames,
                         int32_t frame_start, hipStream_t stream);

/* Chunk-causal attention over the limited window (abstract: limited temporal
 * window in the KV cache; Table 3: chunks of three latent frames).
 * Window W = the prior frames f < frame_start with f < n_sink or
 * f >= frame_start - n_recent (n_recent = -1: every prior frame), each once,
 * then the chunk's own frames; see ust_window_plan.  The chunk's keys and
 * values must already be appended.  For every query token n and head h:
 *   q' = RoPE(f, y, x) q[n][h]
 *   s_m = scale * <q', kv.k[m]> over every key m of every frame of W
 *   out[n][h] = sum_m softmax(s)_m kv.v[m]
 * There is no mask inside the window.  scale = 0 selects 1/sqrt(head_dim).
 * Arithmetic: bf16 MFMA products with fp32 accumulation and fp32 softmax;
 * the rotated, scaled query and the probabilities are rounded to bf16.
 *   q:   bf16 [chunk_frames*T][n_heads][head_dim], un-rotated, read.
 *   cos_tab, sin_tab, tab_first_frame, n_tab_frames: the table, as in
 *        ust_kv_append (the rows of the chunk's frames rotate the queries;
 *        the window's keys were rotated when they were appended).
 *   out: bf16, same layout, written.
 *   lse_opt: NULL, or fp32 [n_heads][chunk_frames*T]: ln sum_m exp(s_m).
 * Errors: as ust_kv_append, plus UST_E_RANGE when a window frame is no longer
 * held by the ring (its slot was reused by a later frame up to
 * frame_start + chunk_frames - 1) or the window exceeds
 * UST_MAX_WINDOW_FRAMES frames; n_recent < -1 (UST_E_RANGE). */
ust_status ust_window_attn(const ust_geom* g, const ust_kv* kv, const void* q,
                           const float* cos_tab, const float* sin_tab,
                           int32_t tab_first_frame, int32_t n_tab_frames, int32_t frame_start,
                           int32_t n_recent, float scale, void* out,
                           float* lse_opt, hipStream_t stream);

/* Bytes of device workspace that ust_window_attn_split needs when the work is
 * divided over n_workgroups workgroups (n_workgroups <= 0: one per compute
 * unit of the current device).  Depends only on head_dim and the workgroup
 * count: 2 * n_workgroups * 256 * (head_dim + 1) * 4.  Returns 0 if g is
 * invalid, n_workgroups exceeds 65536, or the device cannot be queried. */
size_t ust_window_attn_work_bytes(const ust_geom* g, int32_t n_workgroups);

/* The same attention as ust_window_attn, with the same arguments, result
 * definition and errors, scheduled for load balance.  ust_window_attn gives
 * each (head, 256-query tile) pair (a unit) to one workgroup, so a chunk
 * whose unit count is not a multiple of the device's compute units leaves
 * units idle in its last round.  Here, with G = n_workgroups: the first
 * floor(U / G) * G of the U units run whole, G at a time; the key tiles of
 * the other units, unit after unit, are cut into G equal contiguous ranges,
 * one per workgroup.  A unit whose keys fall in several ranges is finished
 * by a second kernel, which merges the ranges' normalised partial outputs by
 * their log-sum-exps (online softmax, merged exactly up to fp32 rounding;
 * the output is rounded to bf16 once, after the merge).  Each part rounds its
 * probabilities to bf16 against its own running maximum, so outputs can
 * differ from ust_window_attn's by that rounding; where no unit is split
 * they are identical.  It pays when U exceeds the compute-unit count and is
 * not a multiple of it (a last, partly empty round otherwise).
 *   work: device workspace, caller-owned, at least
 *         ust_window_attn_work_bytes(g, n_workgroups) bytes, 16-byte
 *         aligned.  Its contents are unspecified after the call.  Calls that
 *         share one workspace must be ordered (one stream).
 *   n_workgroups: workgroups to divide the work over, <= 65536; <= 0 selects
 *         one per compute unit of the current device.  Values above the
 *         number of key tiles in the whole chunk act as that number.
 * Errors: as ust_window_attn, plus work NULL (UST_E_NULL), misaligned
 * (UST_E_ALIGN), work_bytes too small or n_workgroups > 65536 (UST_E_SHAPE). */
ust_status ust_window_attn_split(const ust_geom* g, const ust_kv* kv, const void* q,
                                 const float* cos_tab, const float* sin_tab,
                                 int32_t tab_first_frame, int32_t n_tab_frames,
                                 int32_t frame_start,
                                 int32_t n_recent, float scale, void* out,
                                 float* lse_opt, void* work, size_t work_bytes,
                                 int32_t n_workgroups, hipStream_t stream);

/* The chunk's Q, K and V projections in one pass, with the key RoPE and
 * the append of ust_kv_append folded into the product's epilogue (abstract:
 * RoPE from precomputed coefficients, KV cache indexed by frame).  For
 * every token n of the chunk (frame f = frame_start + n / T) and head h:
 *   q_out[n][h][:]             = bf16_rne(x[n] W_q^T), un-rotated (the
 *                                attention rotates the queries itself)
 *   kv.k[slot(f)][h][n % T][:] = bf16_rne(RoPE(f, y, x) (x[n] W_k^T))
 *   kv.v[slot(f)][h][:][n % T] = bf16_rne(x[n] W_v^T)
 * with the rotation applied to the fp32 product before its one rounding.  A
 * truncated-SVD value projection whose rank r is above the break-even
 * hidden * H D / (hidden + H D) (768 at 1536 x 1536) enters as its
 * re-densified W_r = A_r B_r, which ust_lowrank_proj can form (x = B_r
 * stored output-major, a = A_r stored input-major, b = NULL).
 *   x:     bf16 [chunk_frames*T][hidden], read.
 *   w_qkv: bf16 [3 * n_heads * head_dim][hidden], output-major: rows of W_q,
 *          then of W_k, then of W_v (row j = output feature j).  Read.
 *   cos_tab, sin_tab, tab_first_frame, n_tab_frames: the table, as in
 *          ust_kv_append.
 *   q_out: bf16 [chunk_frames*T][n_heads][head_dim], written.
 * Arithmetic: bf16 MFMA with fp32 accumulation.
 * Errors: as ust_kv_append; hidden <= 0 (UST_E_SHAPE), not a multiple of 64
 * (UST_E_UNSUPPORTED); operands past 32-bit indexing (UST_E_SHAPE). */
ust_status ust_qkv_append(const ust_geom* g, const ust_kv* kv, const void* x,
                          const void* w_qkv, int32_t hidden, const float* cos_tab,
                          const float* sin_tab, int32_t tab_first_frame,
                          int32_t n_tab_frames, int32_t frame_start, void* q_out,
                          hipStream_t stream);

/* Low-rank projection Y = (X A_r) B_r (+ bias) (abstract: truncated SVD of
 * the attention value and output projections).
 *   x:    bf16 [M][K], read.
 *   a:    bf16 [r][K]: A_r stored output-major (row j = column j of A_r), as
 *         a linear layer stores its weight.  Read.
 *   b:    bf16 [N][r]: B_r stored output-major, or NULL for the dense
 *         projection Y = X A (then N must equal r and t_work may be NULL).
 *   bias: bf16 [N] or NULL.
 *   t_work: bf16 [M][r] scratch, caller-owned, required when b != NULL;
 *         receives T = X A_r rounded to bf16 (the contents are unspecified
 *         after the call).
 *   y:    bf16 [M][N], written.
 * Arithmetic: bf16 MFMA with fp32 accumulation; T is rounded to bf16 between
 * the two products.  Errors: NULL pointers; non-positive sizes (UST_E_SHAPE);
 * K, r or N not a multiple of 8, misaligned pointers (UST_E_ALIGN); b NULL
 * with N != r (UST_E_SHAPE). */
ust_status ust_lowrank_proj(const void* x, const void* a, const void* b,
                            const void* bias, void* t_work, void* y,
                            int32_t M, int32_t K, int32_t r, int32_t N,
                            hipStream_t stream);

/* The value projection of one chunk, V = (X A_r) B_r as ust_lowrank_proj
 * computes it (abstract: truncated SVD of the value projection), with the
 * values stored straight into the ring instead of a V buffer (abstract: the
 * KV cache indexed by latent frame): for every token n of the chunk (frame
 * f = frame_start + n / T) and head h,
 *   kv.v[slot(f)][h][:][n % T] = bf16_rne((x[n] A_r) B_r)[h][:]
 * with T rounded to bf16 between the two products, bit for bit the values
 * that ust_lowrank_proj followed by ust_kv_append would store.
 * With k_new given, the chunk's keys are rotated and appended too, bit for
 * bit as ust_kv_append with v_new NULL stores them; where the first
 * product's kernel allows (hidden a multiple of 64), extra workgroups of
 * its launch do it on the compute units the product leaves idle, otherwise
 * a launch of its own precedes it.  With k_new NULL the keys are not
 * touched (ust_kv_append with v_new NULL appends them).
 *   x:      bf16 [chunk_frames*T][hidden], read.
 *   a:      bf16 [rank][hidden], A_r output-major.  Read.
 *   b:      bf16 [n_heads*head_dim][rank], B_r output-major.  Read.
 *   t_work: bf16 [chunk_frames*T][rank] scratch, caller-owned (contents
 *           unspecified after the call).
 *   k_new:  NULL, or bf16 [chunk_frames*T][n_heads][head_dim], the chunk's
 *           un-rotated keys.  Read.
 *   cos_tab, sin_tab, tab_first_frame, n_tab_frames: the RoPE table, as in
 *           ust_kv_append; unused (may be NULL) when k_new is NULL.
 * Errors: NULL pointers (the table too when k_new is given); non-positive
 * hidden or rank (UST_E_SHAPE); hidden not a multiple of 8 or misaligned
 * pointers (UST_E_ALIGN); rank not a multiple of 64, T not a multiple of 8
 * or head_dim not 64/128 (UST_E_UNSUPPORTED); frame_start < 0, a ring that
 * cannot hold the chunk, or, with k_new, the chunk's frames outside the
 * table (UST_E_RANGE); operands past 32-bit indexing (UST_E_SHAPE). */
ust_status ust_lowrank_proj_v_append(const ust_geom* g, const ust_kv* kv, const void* x,
                                     const void* a, const void* b, void* t_work,
                                     int32_t hidden, int32_t rank, const void* k_new,
                                     const float* cos_tab, const float* sin_tab,
                                     int32_t tab_first_frame, int32_t n_tab_frames,
                                     int32_t frame_start, hipStream_t stream);

/* Largest M * r that ust_lowrank_proj_static accepts: the bf16 elements of
 * its device scratch (8 MiB). */
#define UST_LOWRANK_STATIC_MAX_ELEMS (4 * 1024 * 1024)

/* ust_lowrank_proj without the caller's t_work, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * hosts that forbid allocation): same arguments, result and errors as
 * ust_lowrank_proj, the same kernels, and T = X A_r kept in a device scratch
 * array that the library holds, one per GPU, for the life of the process.
 * The call allocates nothing (its first call on a device looks the array's
 * address up).  T is written in full before it is read, so nothing carries
 * over from an earlier call.
 *   Limit: M * r <= UST_LOWRANK_STATIC_MAX_ELEMS when b != NULL, else
 *   UST_E_RANGE (b == NULL needs no scratch).
 *   Calls that overlap on one GPU (different streams, or several host
 *   threads) share that array and race: order them on one stream. */
ust_status ust_lowrank_proj_static(const void* x, const void* a, const void* b,
                                   const void* bias, void* y, int32_t M, int32_t K,
                                   int32_t r, int32_t N, hipStream_t stream);

/* One step of the chunk sampler (Table 4: the noise levels of the denoising
 * steps and of the clean-cache forward; abstract: the generated frames are
 * renoised to a nearly clean level and the clean-cache forward refines
 * them).  With a latent at level sigma written (1 - sigma) x0 + sigma eps and
 * the DiT's output the velocity eps - x0 (flow matching, the parameterisation
 * of this model family), for every i < n:
 *   x0_hat[i] = x[i] - sigma v[i]                  (fp32, one fused multiply-add)
 *   x_next[i] = keep x0_hat[i] + sigma_next noise[i]  (keep = fp32(1 - sigma_next):
 *                                          the product rounded, then one fma)
 * and x_next = x0_hat exactly when sigma_next == 0 (noise is then not read).
 * A chunk's denoising steps run at the levels of ust_sigma_schedule, each
 * renoising to the next level with a fresh draw; the last one renoises to
 * the clean-cache level sigma* (0.02 for UnStep, 0 for Self Forcing); the
 * clean-cache forward's step (sigma = sigma*, sigma_next = 0) gives the chunk
 * kept.
 *   x:      fp32 [n] latent at level sigma, read.
 *   v:      bf16 [n] velocity from the DiT, read.
 *   noise:  fp32 [n] draw for the renoising, read; may be NULL when
 *           sigma_next == 0.  Random numbers are the caller's: the library
 *           draws none.
 *   x0_out: fp32 [n] or NULL: receives x0_hat.
 *   x_next: fp32 [n]: receives the renoised latent.
 *   Each output element depends only on the inputs at its own index, so an
 *   output may be the same buffer as an input (no partial overlap).
 * Errors: x, v or x_next NULL, or noise NULL with sigma_next != 0
 * (UST_E_NULL); n < 0 (UST_E_SHAPE); a level outside [0, 1] or NaN
 * (UST_E_RANGE); a pointer not 16-byte aligned (UST_E_ALIGN).  n == 0
 * launches nothing. */
ust_status ust_flow_step(const float* x, const void* v, const float* noise, float sigma,
                         float sigma_next, float* x0_out, float* x_next, int64_t n,
                         hipStream_t stream);

/* Causal 3-D convolution, the convolution kernel of the decoder runtime
 * stack (abstract: VAE decoding with an optimised memory layout, precision
 * and convolution kernels; Table 3: the decoder turns 21 latent frames of
 * 16 x 60 x 104 into 81 frames of 832 x 480).  The decoder's architecture is
 * not given; this is its 3x3x3 convolution, causal in time:
 *   y[t][r][c][o] = bias[o] + sum over dt, dr, dc in {0,1,2} and i of
 *                   w[o][dt][dr][dc][i] x[t+dt-2][r+dr-1][c+dc-1][i]
 * with x zero outside its frames, rows and columns (output frame t reads
 * input frames t-2 .. t; each frame keeps its size; stride 1).
 *   x:    bf16 [T][H][W][Ci] (channels last), read.
 *   w:    bf16 [Co][3][3][3][Ci], read.
 *   bias: fp32 [Co] or NULL.
 *   y:    bf16 [T][H][W][Co], written; must not overlap x.
 * Arithmetic: bf16 MFMA with fp32 accumulation, the output rounded to bf16
 * once (bias added in fp32).
 * Errors: NULL x, w or y (UST_E_NULL); a non-positive size, or x, y or w
 * of 2^30 elements or more (UST_E_SHAPE); Ci neither 16 nor a multiple of
 * 32, or Co not a multiple of 32 (UST_E_UNSUPPORTED); a pointer not 16-byte
 * aligned (UST_E_ALIGN). */
ust_status ust_conv3d_causal(const void* x, const void* w, const float* bias, void* y,
                             int32_t T, int32_t H, int32_t W, int32_t Ci, int32_t Co,
                             hipStream_t stream);

/* The same convolution for a clip decoded chunk by chunk (the pages'
 * generation is streamed in chunks of three latent frames, Table 3): x
 * holds two history frames, the last two input frames of the previous
 * chunk (zeros before a clip's first chunk), then the chunk's T frames, and
 * the history takes the place of the zero padding in front:
 *   y[t] = the convolution above at frame t + 2 of x, for t = 0 .. T-1.
 *   x:    bf16 [T + 2][H][W][Ci] (channels last), read.
 *   y:    bf16 [T][H][W][Co], written; must not overlap x.
 * The arithmetic is that of ust_conv3d_causal, so a clip decoded in chunks
 * equals the whole-clip call bit for bit.  Errors: as ust_conv3d_causal,
 * with (T + 2) H W Ci the size of x. */
ust_status ust_conv3d_causal_stream(const void* x, const void* w, const float* bias, void* y,
                                    int32_t T, int32_t H, int32_t W, int32_t Ci, int32_t Co,
                                    hipStream_t stream);

/* ---- host-only helpers (no GPU needed) ---- */

/* Noise levels of raw timesteps after the shift mapping (Table 4, shift 5,
 * n_train 1000: raw 1000, 750, 500, 250 give 1, 15/16, 5/6, 5/8):
 *   u = raw / n_train,  sigma = shift u / (1 + (shift - 1) u),  in fp64,
 * and the DiT's timestep label n_train sigma.  A Self Forcing chunk steps
 * through raw 1000, 750, 500, 250; an UnStep later chunk through two of
 * them (1000 and 500 in this library's workloads: the pages do not say
 * which two).
 *   raw_steps: [n] host array, each in [0, n_train].
 *   sigma_out: [n] host array, written.  label_out: [n] host array or NULL.
 * Errors: NULL raw_steps / sigma_out (UST_E_NULL); n < 0 (UST_E_SHAPE);
 * shift <= 0 or not finite, n_train <= 0, a raw step outside [0, n_train]
 * (UST_E_RANGE). */
ust_status ust_sigma_schedule(const int32_t* raw_steps, int32_t n, double shift,
                              int32_t n_train, double* sigma_out, double* label_out);

/* Ring slot of latent frame `frame`; -1 if frame < 0 or the ring is invalid
 * (n_sink < 0 or n_slots <= n_sink).  The KV cache is indexed by latent
 * frame (abstract: the runtime stack's faster KV indexing) and holds a
 * limited temporal window (abstract; Table 1 row C4), so it is a ring of
 * frame slots; the first n_sink frames stay pinned, after the attention
 * sinks of the streaming-attention work the paper builds on (its list of
 * cited work):
 *   slot(f) = f                                          if f < n_sink
 *   slot(f) = n_sink + (f - n_sink) mod (n_slots - n_sink)   otherwise. */
int32_t ust_slot_of_frame(const ust_kv* kv, int32_t frame);

/* The window of the chunk starting at frame_start, as ust_window_attn uses
 * it (abstract: the attention KV cache keeps a limited temporal window;
 * Table 1 row C4: the limited attention window; Table 3: chunks of three
 * latent frames): the prior frames f < n_sink or f >= frame_start -
 * n_recent, each once, then the chunk's own frames; n_recent = -1 keeps
 * every prior frame.  frames_out[i] ascending,
 * slots_out[i] = ust_slot_of_frame(frames[i]).
 * Writes at most cap entries and the count to *n_out.
 * Errors: NULL pointers; cap too small (UST_E_SHAPE); a window frame no
 * longer held by the ring, n_recent < -1, frame_start < 0, or more than
 * UST_MAX_WINDOW_FRAMES frames (UST_E_RANGE). */
ust_status ust_window_plan(const ust_geom* g, const ust_kv* kv, int32_t frame_start,
                           int32_t n_recent, int32_t* frames_out, int32_t* slots_out,
                           int32_t cap, int32_t* n_out);

/* Static text naming a status. */
const char* ust_status_str(ust_status s);

/* Detail of the last error on the calling thread ("" if none). */
const char* ust_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* UST_H */
