// C-ABI entry points: argument validation, the frame-slot ring and the
// window plan (host integer work), and dispatch to the kernel launchers.
//
// Every entry point validates everything before launching anything, records
// a thread-local error text, and never lets a C++ exception escape.

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "ust_internal.h"

extern "C" int32_t ust_v_row_len(int32_t T);

namespace {

thread_local std::string g_last_error;

ust_status fail(ust_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

ust_status ok() {
  g_last_error.clear();
  return UST_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ust_status check_geom(const ust_geom* g) {
  if (!g) return fail(UST_E_NULL, "geometry is NULL");
  if (g->grid_h <= 0 || g->grid_w <= 0 || g->n_heads <= 0 || g->head_dim <= 0 ||
      g->chunk_frames <= 0 || g->pairs_t < 0 || g->pairs_h < 0 || g->pairs_w < 0)
    return fail(UST_E_SHAPE, "geometry sizes must be positive");
  if (g->head_dim % 2 != 0 || g->pairs_t + g->pairs_h + g->pairs_w != g->head_dim / 2)
    return fail(UST_E_SHAPE, "pairs_t+pairs_h+pairs_w (%d) must equal head_dim/2 (%d)",
                g->pairs_t + g->pairs_h + g->pairs_w, g->head_dim / 2);
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(UST_E_UNSUPPORTED, "head_dim %d: only 64 and 128 are supported", g->head_dim);
  if (g->chunk_frames > 8)
    return fail(UST_E_UNSUPPORTED, "chunk_frames %d: at most 8 supported", g->chunk_frames);
  const int64_t T = int64_t(g->grid_h) * g->grid_w;
  const int64_t nq = T * g->chunk_frames;
  if (nq * g->n_heads * g->head_dim >= (int64_t(1) << 31))
    return fail(UST_E_SHAPE, "chunk tensor too large for 32-bit indexing");
  return UST_OK;
}

// Slot of a frame; -1 on invalid input.
int32_t slot_of(int32_t frame, int32_t n_slots, int32_t n_sink) {
  if (frame < 0 || n_sink < 0 || n_slots <= n_sink) return -1;
  if (frame < n_sink) return frame;
  return n_sink + (frame - n_sink) % (n_slots - n_sink);
}

ust_status check_kv(const ust_kv* kv) {
  if (!kv) return fail(UST_E_NULL, "kv is NULL");
  if (!kv->k || !kv->v) return fail(UST_E_NULL, "kv.k or kv.v is NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v))
    return fail(UST_E_ALIGN, "kv.k / kv.v must be 16-byte aligned");
  if (kv->n_sink < 0 || kv->n_slots <= kv->n_sink)
    return fail(UST_E_RANGE, "ring needs 0 <= n_sink < n_slots (got %d, %d)", kv->n_sink,
                kv->n_slots);
  return UST_OK;
}

// Element offsets into the ring are 32-bit in the kernels.
ust_status check_ring_size(const ust_geom* g, const ust_kv* kv) {
  const int64_t T = int64_t(g->grid_h) * g->grid_w;
  const int64_t per_slot = int64_t(g->n_heads) * g->head_dim * ust_v_row_len(int32_t(T));
  if (int64_t(kv->n_slots) * per_slot >= (int64_t(1) << 31))
    return fail(UST_E_SHAPE, "ring of %d slots too large for 32-bit indexing", kv->n_slots);
  return UST_OK;
}

// Slots of the chunk's own frames; they must be distinct and the frames must
// lie in the table, which holds frames tab_first .. tab_first + n_tab - 1.
ust_status chunk_slots(const ust_geom* g, const ust_kv* kv, int32_t tab_first, int32_t n_tab,
                       int32_t frame_start, int32_t* slots) {
  if (frame_start < 0) return fail(UST_E_RANGE, "frame_start %d < 0", frame_start);
  if (tab_first < 0) return fail(UST_E_RANGE, "tab_first_frame %d < 0", tab_first);
  if (frame_start < tab_first ||
      int64_t(frame_start) + g->chunk_frames > int64_t(tab_first) + n_tab)
    return fail(UST_E_RANGE, "frames %d..%lld outside the RoPE table of frames %d..%lld",
                frame_start, (long long)frame_start + g->chunk_frames - 1, tab_first,
                (long long)tab_first + n_tab - 1);
  for (int i = 0; i < g->chunk_frames; ++i) {
    slots[i] = slot_of(frame_start + i, kv->n_slots, kv->n_sink);
    for (int j = 0; j < i; ++j)
      if (slots[j] == slots[i])
        return fail(UST_E_RANGE, "ring of %d slots (%d sinks) cannot hold one chunk of %d frames",
                    kv->n_slots, kv->n_sink, g->chunk_frames);
  }
  return UST_OK;
}

// The window plan (see ust_window_plan in ust.h).  Only the frames that can
// be in the window are visited: the sinks before the chunk, then from the
// first recent frame (or the first non-sink frame) to the chunk's last frame.
ust_status plan(const ust_geom* g, const ust_kv* kv, int32_t frame_start, int32_t n_recent,
                int32_t* frames, int32_t* slots, int32_t cap, int32_t* n_out) {
  if (frame_start < 0) return fail(UST_E_RANGE, "frame_start %d < 0", frame_start);
  if (n_recent < -1) return fail(UST_E_RANGE, "n_recent %d < -1", n_recent);
  const int64_t last = int64_t(frame_start) + g->chunk_frames - 1;  // newest frame written
  if (last > INT32_MAX)
    return fail(UST_E_RANGE, "chunk at frame %d runs past frame %d", frame_start, INT32_MAX);
  const int64_t ring = int64_t(kv->n_slots) - kv->n_sink;
  int32_t n = 0;
  auto take = [&](int64_t f, bool sink) -> ust_status {
    // a ring frame f is overwritten once frame f + ring has been written
    if (!sink && f + ring <= last)
      return fail(UST_E_RANGE,
                  "window frame %lld is no longer in the ring (%d slots, %d sinks) after frame %lld",
                  static_cast<long long>(f), kv->n_slots, kv->n_sink, static_cast<long long>(last));
    if (n >= UST_MAX_WINDOW_FRAMES)
      return fail(UST_E_RANGE, "window exceeds %d frames", UST_MAX_WINDOW_FRAMES);
    if (n >= cap) return fail(UST_E_SHAPE, "plan capacity %d too small", cap);
    frames[n] = int32_t(f);
    slots[n] = slot_of(int32_t(f), kv->n_slots, kv->n_sink);
    ++n;
    return UST_OK;
  };
  // sink frames before the chunk (a sink inside the chunk counts as current)
  const int64_t sink_end = std::min<int64_t>(kv->n_sink, frame_start);
  for (int64_t f = 0; f < sink_end; ++f) {
    const ust_status s = take(f, true);
    if (s != UST_OK) return s;
  }
  // recent frames (every prior frame when n_recent = -1), then the chunk
  const int64_t recent0 = n_recent < 0 ? 0 : std::max<int64_t>(0, int64_t(frame_start) - n_recent);
  for (int64_t f = std::max(sink_end, recent0); f <= last; ++f) {
    const ust_status s = take(f, f < kv->n_sink);
    if (s != UST_OK) return s;
  }
  *n_out = n;
  return UST_OK;
}

ust_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(UST_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t ust_v_row_len(int32_t T) {
  if (T <= 0) return -1;
  return (T + 63) / 64 * 64;
}

const char* ust_status_str(ust_status s) {
  switch (s) {
    case UST_OK: return "UST_OK";
    case UST_E_NULL: return "UST_E_NULL";
    case UST_E_SHAPE: return "UST_E_SHAPE";
    case UST_E_RANGE: return "UST_E_RANGE";
    case UST_E_ALIGN: return "UST_E_ALIGN";
    case UST_E_UNSUPPORTED: return "UST_E_UNSUPPORTED";
    case UST_E_HIP: return "UST_E_HIP";
  }
  return "UST_E_UNKNOWN";
}

const char* ust_last_error(void) { return g_last_error.c_str(); }

int32_t ust_slot_of_frame(const ust_kv* kv, int32_t frame) {
  if (!kv) return -1;
  return slot_of(frame, kv->n_slots, kv->n_sink);
}

ust_status ust_window_plan(const ust_geom* g, const ust_kv* kv, int32_t frame_start,
                           int32_t n_recent, int32_t* frames_out, int32_t* slots_out,
                           int32_t cap, int32_t* n_out) {
  try {
    ust_status s = check_geom(g);
    if (s != UST_OK) return s;
    if (!kv) return fail(UST_E_NULL, "kv is NULL");
    if (kv->n_sink < 0 || kv->n_slots <= kv->n_sink)
      return fail(UST_E_RANGE, "ring needs 0 <= n_sink < n_slots");
    if (!frames_out || !slots_out || !n_out) return fail(UST_E_NULL, "output pointer is NULL");
    s = plan(g, kv, frame_start, n_recent, frames_out, slots_out, cap, n_out);
    if (s != UST_OK) return s;
    return ok();
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

ust_status ust_rope_table_build(const ust_geom* g, int32_t first_frame, int32_t n_frames,
                                double theta, float* cos_out, float* sin_out,
                                hipStream_t stream) {
  try {
    ust_status s = check_geom(g);
    if (s != UST_OK) return s;
    if (!cos_out || !sin_out) return fail(UST_E_NULL, "cos_out / sin_out is NULL");
    if (!aligned16(cos_out) || !aligned16(sin_out))
      return fail(UST_E_ALIGN, "table pointers must be 16-byte aligned");
    if (n_frames <= 0) return fail(UST_E_SHAPE, "n_frames %d <= 0", n_frames);
    if (!(theta > 0.0) || !std::isfinite(theta)) return fail(UST_E_RANGE, "theta must be > 0");
    if (first_frame < 0) return fail(UST_E_RANGE, "first_frame %d < 0", first_frame);
    if (int64_t(first_frame) + n_frames - 1 > INT32_MAX)
      return fail(UST_E_RANGE, "frames %d + %d pass INT32_MAX", first_frame, n_frames);
    if (int64_t(n_frames) * g->grid_h * g->grid_w * (g->head_dim / 2) >= (int64_t(1) << 31))
      return fail(UST_E_SHAPE, "table too large for 32-bit indexing");
    ust::RopeTableArgs a{cos_out, sin_out, first_frame, n_frames, g->grid_h, g->grid_w,
                         g->pairs_t, g->pairs_h, g->pairs_w, theta};
    return hip_status(ust::launch_rope_table(a, stream), "rope_table launch");
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

ust_status ust_kv_append(const ust_geom* g, const ust_kv* kv, const void* k_new,
                         const void* v_new, const float* cos_tab, const float* sin_tab,
                         int32_t tab_first_frame, int32_t n_tab_frames, int32_t frame_start,
                         hipStream_t stream) {
  try {
    ust_status s = check_geom(g);
    if (s != UST_OK) return s;
    s = check_kv(kv);
    if (s != UST_OK) return s;
    s = check_ring_size(g, kv);
    if (s != UST_OK) return s;
    if (!k_new || !cos_tab || !sin_tab)
      return fail(UST_E_NULL, "k_new or table pointer is NULL");
    if (!aligned16(k_new) || (v_new && !aligned16(v_new)) || !aligned16(cos_tab) ||
        !aligned16(sin_tab))
      return fail(UST_E_ALIGN, "pointers must be 16-byte aligned");
    const int32_t T = g->grid_h * g->grid_w;
    if (T % 8 != 0)
      return fail(UST_E_UNSUPPORTED, "tokens per frame %d: must be a multiple of 8", T);
    ust::AppendArgs a{};
    s = chunk_slots(g, kv, tab_first_frame, n_tab_frames, frame_start, a.chunk_slot);
    if (s != UST_OK) return s;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.cos_tab = cos_tab;
    a.sin_tab = sin_tab;
    a.k_cache = static_cast<uint16_t*>(kv->k);
    a.v_cache = static_cast<uint16_t*>(kv->v);
    a.T = T;
    a.TV = ust_v_row_len(T);
    a.H = g->n_heads;
    a.D = g->head_dim;
    a.C = g->chunk_frames;
    a.tab_frame = frame_start - tab_first_frame;
    a.with_v = v_new != nullptr;
    return hip_status(ust::launch_kv_append(a, stream), "kv_append launch");
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

}  // extern "C"

namespace {

// Compute units of the current device, or -1.
int32_t device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return n > 0 ? n : -1;
}

constexpr int32_t kMaxAttnWorkgroups = 1 << 16;

// ust_window_attn (work == nullptr) and ust_window_attn_split
ust_status window_attn(const ust_geom* g, const ust_kv* kv, const void* q,
                       const float* cos_tab, const float* sin_tab, int32_t tab_first_frame,
                       int32_t n_tab_frames, int32_t frame_start, int32_t n_recent,
                       float scale, void* out, float* lse_opt, bool split, void* work,
                       size_t work_bytes,
                       int32_t n_workgroups, hipStream_t stream) {
  try {
    ust_status s = check_geom(g);
    if (s != UST_OK) return s;
    s = check_kv(kv);
    if (s != UST_OK) return s;
    s = check_ring_size(g, kv);
    if (s != UST_OK) return s;
    if (!q || !cos_tab || !sin_tab || !out)
      return fail(UST_E_NULL, "q, table or out pointer is NULL");
    if (!aligned16(q) || !aligned16(cos_tab) || !aligned16(sin_tab) || !aligned16(out) ||
        (lse_opt && !aligned16(lse_opt)))
      return fail(UST_E_ALIGN, "pointers must be 16-byte aligned");
    const int32_t T = g->grid_h * g->grid_w;
    if (T % 8 != 0)
      return fail(UST_E_UNSUPPORTED, "tokens per frame %d: must be a multiple of 8", T);
    if (!std::isfinite(scale) || scale < 0.f) return fail(UST_E_RANGE, "scale must be >= 0");
    int32_t cslots[8];
    s = chunk_slots(g, kv, tab_first_frame, n_tab_frames, frame_start, cslots);
    if (s != UST_OK) return s;
    ust::AttnArgs a{};
    int32_t frames[UST_MAX_WINDOW_FRAMES];
    int32_t n = 0;
    s = plan(g, kv, frame_start, n_recent, frames, a.slots, UST_MAX_WINDOW_FRAMES, &n);
    if (s != UST_OK) return s;
    if (int64_t(n) * T >= (int64_t(1) << 30))
      return fail(UST_E_SHAPE, "window too large for 32-bit key indexing");
    const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(float(g->head_dim));
    a.q = static_cast<const uint16_t*>(q);
    a.cos_tab = cos_tab;
    a.sin_tab = sin_tab;
    a.k_cache = static_cast<const uint16_t*>(kv->k);
    a.v_cache = static_cast<const uint16_t*>(kv->v);
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse_opt;
    a.T = T;
    a.TV = ust_v_row_len(T);
    a.H = g->n_heads;
    a.D = g->head_dim;
    a.NQ = T * g->chunk_frames;
    a.tab_frame = frame_start - tab_first_frame;
    a.n_frames = n;
    a.qscale = sc * 1.4426950408889634f;  // log2(e): softmax runs in base 2
    if (split) {
      if (n_workgroups > kMaxAttnWorkgroups)
        return fail(UST_E_SHAPE, "n_workgroups %d exceeds %d", n_workgroups, kMaxAttnWorkgroups);
      const int32_t nwg = n_workgroups > 0 ? n_workgroups : device_cus();
      if (nwg <= 0) return fail(UST_E_HIP, "cannot query the device's compute units");
      const size_t need = ust::window_attn_work_bytes(g->head_dim, nwg);
      if (!work) return fail(UST_E_NULL, "work is NULL");
      if (!aligned16(work)) return fail(UST_E_ALIGN, "work must be 16-byte aligned");
      if (work_bytes < need)
        return fail(UST_E_SHAPE, "work holds %zu bytes, %zu needed for %d workgroups",
                    work_bytes, need, nwg);
      a.work_o = static_cast<float*>(work);
      a.n_wg = nwg;
    }
    return hip_status(ust::launch_window_attn(a, stream), "window_attn launch");
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

}  // namespace

extern "C" {

ust_status ust_window_attn(const ust_geom* g, const ust_kv* kv, const void* q,
                           const float* cos_tab, const float* sin_tab,
                           int32_t tab_first_frame, int32_t n_tab_frames, int32_t frame_start,
                           int32_t n_recent, float scale, void* out, float* lse_opt,
                           hipStream_t stream) {
  return window_attn(g, kv, q, cos_tab, sin_tab, tab_first_frame, n_tab_frames, frame_start,
                     n_recent, scale, out, lse_opt, false, nullptr, 0, 0, stream);
}

size_t ust_window_attn_work_bytes(const ust_geom* g, int32_t n_workgroups) {
  try {
    if (check_geom(g) != UST_OK || n_workgroups > kMaxAttnWorkgroups) return 0;
    const int32_t nwg = n_workgroups > 0 ? n_workgroups : device_cus();
    if (nwg <= 0) return 0;
    return ust::window_attn_work_bytes(g->head_dim, nwg);
  } catch (...) {
    return 0;
  }
}

ust_status ust_window_attn_split(const ust_geom* g, const ust_kv* kv, const void* q,
                                 const float* cos_tab, const float* sin_tab,
                                 int32_t tab_first_frame, int32_t n_tab_frames,
                                 int32_t frame_start, int32_t n_recent, float scale, void* out,
                                 float* lse_opt, void* work, size_t work_bytes,
                                 int32_t n_workgroups, hipStream_t stream) {
  return window_attn(g, kv, q, cos_tab, sin_tab, tab_first_frame, n_tab_frames, frame_start,
                     n_recent, scale, out, lse_opt, true, work, work_bytes, n_workgroups,
                     stream);
}

ust_status ust_qkv_append(const ust_geom* g, const ust_kv* kv, const void* x,
                          const void* w_qkv, int32_t hidden, const float* cos_tab,
                          const float* sin_tab, int32_t tab_first_frame,
                          int32_t n_tab_frames, int32_t frame_start, void* q_out,
                          hipStream_t stream) {
  try {
    ust_status s = check_geom(g);
    if (s != UST_OK) return s;
    s = check_kv(kv);
    if (s != UST_OK) return s;
    s = check_ring_size(g, kv);
    if (s != UST_OK) return s;
    if (!x || !w_qkv || !cos_tab || !sin_tab || !q_out)
      return fail(UST_E_NULL, "x, w_qkv, table or q_out pointer is NULL");
    if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(cos_tab) || !aligned16(sin_tab) ||
        !aligned16(q_out))
      return fail(UST_E_ALIGN, "pointers must be 16-byte aligned");
    if (hidden <= 0) return fail(UST_E_SHAPE, "hidden %d must be positive", hidden);
    if (hidden % 64 != 0)
      return fail(UST_E_UNSUPPORTED, "hidden %d: must be a multiple of 64", hidden);
    const int32_t T = g->grid_h * g->grid_w;
    if (T % 8 != 0)
      return fail(UST_E_UNSUPPORTED, "tokens per frame %d: must be a multiple of 8", T);
    const int32_t M = T * g->chunk_frames;
    const int32_t N = 3 * g->n_heads * g->head_dim;
    if (int64_t(M) * hidden >= (int64_t(1) << 31) || int64_t(N) * hidden >= (int64_t(1) << 31))
      return fail(UST_E_SHAPE, "operands too large for 32-bit indexing");
    ust::QkvEpilogue e{};
    s = chunk_slots(g, kv, tab_first_frame, n_tab_frames, frame_start, e.chunk_slot);
    if (s != UST_OK) return s;
    e.q_out = static_cast<uint16_t*>(q_out);
    e.k_cache = static_cast<uint16_t*>(kv->k);
    e.v_cache = static_cast<uint16_t*>(kv->v);
    e.cos_tab = cos_tab;
    e.sin_tab = sin_tab;
    e.T = T;
    e.TV = ust_v_row_len(T);
    e.H = g->n_heads;
    e.D = g->head_dim;
    e.tab_frame = frame_start - tab_first_frame;
    const ust::GemmArgs ga{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_qkv),
                           nullptr, nullptr, M, N, hidden};
    return hip_status(ust::launch_qkv_append(ga, e, stream), "qkv_append launch");
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

ust_status ust_lowrank_proj_v_append(const ust_geom* g, const ust_kv* kv, const void* x,
                                     const void* a, const void* b, void* t_work, int32_t hidden,
                                     int32_t rank, const void* k_new, const float* cos_tab,
                                     const float* sin_tab, int32_t tab_first_frame,
                                     int32_t n_tab_frames, int32_t frame_start,
                                     hipStream_t stream) {
  try {
    ust_status s = check_geom(g);
    if (s != UST_OK) return s;
    s = check_kv(kv);
    if (s != UST_OK) return s;
    s = check_ring_size(g, kv);
    if (s != UST_OK) return s;
    if (!x || !a || !b || !t_work) return fail(UST_E_NULL, "x, a, b or t_work is NULL");
    if (k_new && (!cos_tab || !sin_tab))
      return fail(UST_E_NULL, "k_new is given without the table");
    if (!aligned16(x) || !aligned16(a) || !aligned16(b) || !aligned16(t_work) ||
        (k_new && (!aligned16(k_new) || !aligned16(cos_tab) || !aligned16(sin_tab))))
      return fail(UST_E_ALIGN, "pointers must be 16-byte aligned");
    if (hidden <= 0 || rank <= 0)
      return fail(UST_E_SHAPE, "hidden %d and rank %d must be positive", hidden, rank);
    if (hidden % 8 != 0) return fail(UST_E_ALIGN, "hidden %d: must be a multiple of 8", hidden);
    if (rank % 64 != 0)
      return fail(UST_E_UNSUPPORTED, "rank %d: must be a multiple of 64", rank);
    const int32_t T = g->grid_h * g->grid_w;
    if (T % 8 != 0)
      return fail(UST_E_UNSUPPORTED, "tokens per frame %d: must be a multiple of 8", T);
    const int32_t M = T * g->chunk_frames;
    const int32_t N = g->n_heads * g->head_dim;
    if (int64_t(M) * std::max(hidden, rank) >= (int64_t(1) << 31) ||
        int64_t(rank) * hidden >= (int64_t(1) << 31) || int64_t(N) * rank >= (int64_t(1) << 31))
      return fail(UST_E_SHAPE, "operands too large for 32-bit indexing");
    ust::QkvEpilogue e{};
    // the values are not rotated: the table bounds the frames only when the
    // keys come along
    if (k_new) s = chunk_slots(g, kv, tab_first_frame, n_tab_frames, frame_start, e.chunk_slot);
    else s = chunk_slots(g, kv, 0, INT32_MAX, frame_start, e.chunk_slot);
    if (s != UST_OK) return s;
    e.v_cache = static_cast<uint16_t*>(kv->v);
    e.T = T;
    e.TV = ust_v_row_len(T);
    e.H = g->n_heads;
    e.D = g->head_dim;
    e.tab_frame = 0;
    e.part0 = 2;   // every tile of the second product is a head of V
    uint16_t* t = static_cast<uint16_t*>(t_work);
    const ust::GemmArgs g1{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(a),
                           nullptr, t, M, rank, hidden};
    hipError_t err;
    if (k_new) {
      // the keys' RoPE and append, as ust_kv_append with v_new NULL
      ust::AppendArgs ka{};
      for (int i = 0; i < g->chunk_frames; ++i) ka.chunk_slot[i] = e.chunk_slot[i];
      ka.k_new = static_cast<const uint16_t*>(k_new);
      ka.cos_tab = cos_tab;
      ka.sin_tab = sin_tab;
      ka.k_cache = static_cast<uint16_t*>(kv->k);
      ka.T = T;
      ka.TV = ust_v_row_len(T);
      ka.H = g->n_heads;
      ka.D = g->head_dim;
      ka.C = g->chunk_frames;
      ka.tab_frame = frame_start - tab_first_frame;
      ka.with_v = 0;
      // in the first product's launch where its kernel takes extra
      // workgroups, else as a launch of its own before it
      if (ust::gemm_nt_pipelined(g1)) {
        err = ust::launch_gemm_nt_keys(g1, ka, stream);
      } else {
        err = ust::launch_kv_append(ka, stream);
        if (err == hipSuccess) err = ust::launch_gemm_nt(g1, stream);
      }
    } else {
      err = ust::launch_gemm_nt(g1, stream);
    }
    if (err != hipSuccess) return hip_status(err, "lowrank_proj_v_append launch (X A)");
    const ust::GemmArgs g2{t, static_cast<const uint16_t*>(b), nullptr, nullptr, M, N, rank};
    return hip_status(ust::launch_qkv_append(g2, e, stream), "lowrank_proj_v_append launch (T B)");
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

}  // extern "C"

namespace {

// ust_lowrank_proj, and ust_lowrank_proj_static (t_work == nullptr with
// use_static: the library's device scratch)
ust_status lowrank_proj(const void* x, const void* a, const void* b, const void* bias,
                        void* t_work, bool use_static, void* y, int32_t M, int32_t K, int32_t r,
                        int32_t N, hipStream_t stream) {
  try {
    if (!x || !a || !y) return fail(UST_E_NULL, "x, a or y is NULL");
    if (b && !t_work && !use_static) return fail(UST_E_NULL, "t_work is required when b is given");
    if (M <= 0 || K <= 0 || r <= 0 || N <= 0)
      return fail(UST_E_SHAPE, "sizes must be positive (M=%d K=%d r=%d N=%d)", M, K, r, N);
    if (!b && N != r) return fail(UST_E_SHAPE, "dense mode (b NULL) needs N == r");
    if (K % 8 || r % 8 || N % 8)
      return fail(UST_E_ALIGN, "K, r and N must be multiples of 8 (K=%d r=%d N=%d)", K, r, N);
    if (!aligned16(x) || !aligned16(a) || !aligned16(y) || (b && !aligned16(b)) ||
        (t_work && !aligned16(t_work)) || (bias && !aligned16(bias)))
      return fail(UST_E_ALIGN, "pointers must be 16-byte aligned");
    if (int64_t(M) * std::max(std::max(K, r), N) >= (int64_t(1) << 31) ||
        int64_t(r) * K >= (int64_t(1) << 31) || int64_t(N) * r >= (int64_t(1) << 31))
      return fail(UST_E_SHAPE, "operands too large for 32-bit indexing");
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* ab = static_cast<const uint16_t*>(a);
    const uint16_t* bb = static_cast<const uint16_t*>(b);
    const uint16_t* biasb = static_cast<const uint16_t*>(bias);
    if (!b) {
      ust::GemmArgs g1{xb, ab, biasb, static_cast<uint16_t*>(y), M, r, K};
      return hip_status(ust::launch_gemm_nt(g1, stream), "lowrank_proj launch");
    }
    uint16_t* t = static_cast<uint16_t*>(t_work);
    if (use_static) {
      if (int64_t(M) * r > UST_LOWRANK_STATIC_MAX_ELEMS)
        return fail(UST_E_RANGE, "M * r = %lld exceeds the static scratch (%d elements)",
                    static_cast<long long>(int64_t(M) * r), UST_LOWRANK_STATIC_MAX_ELEMS);
      hipError_t e = ust::lowrank_scratch(&t);
      if (e != hipSuccess) return hip_status(e, "lowrank_proj_static scratch address");
    }
    ust::GemmArgs g1{xb, ab, nullptr, t, M, r, K};
    hipError_t e = ust::launch_gemm_nt(g1, stream);
    if (e != hipSuccess) return hip_status(e, "lowrank_proj launch (X A)");
    ust::GemmArgs g2{t, bb, biasb, static_cast<uint16_t*>(y), M, N, r};
    return hip_status(ust::launch_gemm_nt(g2, stream), "lowrank_proj launch (T B)");
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

// ust_conv3d_causal (hist false) and ust_conv3d_causal_stream (x starts
// with two history frames)
ust_status conv3d(const void* x, const void* w, const float* bias, void* y, int32_t T, int32_t H,
                  int32_t W, int32_t Ci, int32_t Co, bool hist, hipStream_t stream) {
  try {
    if (!x || !w || !y) return fail(UST_E_NULL, "x, w or y is NULL");
    if (T <= 0 || H <= 0 || W <= 0 || Ci <= 0 || Co <= 0)
      return fail(UST_E_SHAPE, "sizes must be positive (T=%d H=%d W=%d Ci=%d Co=%d)", T, H, W,
                  Ci, Co);
    const int64_t tx = int64_t(T) + (hist ? 2 : 0);   // frames of x
    if (tx * H * W >= (int64_t(1) << 31))
      return fail(UST_E_SHAPE, "%lld input positions: at most 2^31 - 1",
                  static_cast<long long>(tx * H * W));
    if (Ci != 16 && Ci % 32 != 0)
      return fail(UST_E_UNSUPPORTED, "Ci %d: 16 or a multiple of 32 supported", Ci);
    if (Co % 32 != 0) return fail(UST_E_UNSUPPORTED, "Co %d: a multiple of 32 supported", Co);
    if (tx * H * W * Ci >= (int64_t(1) << 30) || int64_t(T) * H * W * Co >= (int64_t(1) << 30) ||
        int64_t(Co) * 27 * Ci >= (int64_t(1) << 30))
      return fail(UST_E_SHAPE, "tensors too large for 32-bit byte offsets");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (bias && !aligned16(bias)))
      return fail(UST_E_ALIGN, "pointers must be 16-byte aligned");
    ust::ConvArgs a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), bias,
                    static_cast<uint16_t*>(y), T, H, W, Ci, Co, hist ? 1 : 0};
    return hip_status(ust::launch_conv3d_causal(a, stream), "conv3d_causal launch");
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

}  // namespace

extern "C" {

ust_status ust_lowrank_proj(const void* x, const void* a, const void* b, const void* bias,
                            void* t_work, void* y, int32_t M, int32_t K, int32_t r, int32_t N,
                            hipStream_t stream) {
  return lowrank_proj(x, a, b, bias, t_work, false, y, M, K, r, N, stream);
}

ust_status ust_lowrank_proj_static(const void* x, const void* a, const void* b, const void* bias,
                                   void* y, int32_t M, int32_t K, int32_t r, int32_t N,
                                   hipStream_t stream) {
  return lowrank_proj(x, a, b, bias, nullptr, true, y, M, K, r, N, stream);
}

ust_status ust_sigma_schedule(const int32_t* raw_steps, int32_t n, double shift,
                              int32_t n_train, double* sigma_out, double* label_out) {
  try {
    if (!raw_steps || !sigma_out) return fail(UST_E_NULL, "raw_steps / sigma_out is NULL");
    if (n < 0) return fail(UST_E_SHAPE, "n %d < 0", n);
    if (!(shift > 0.0) || !std::isfinite(shift)) return fail(UST_E_RANGE, "shift must be > 0");
    if (n_train <= 0) return fail(UST_E_RANGE, "n_train %d <= 0", n_train);
    for (int32_t i = 0; i < n; ++i)
      if (raw_steps[i] < 0 || raw_steps[i] > n_train)
        return fail(UST_E_RANGE, "raw step %d outside [0, %d]", raw_steps[i], n_train);
    for (int32_t i = 0; i < n; ++i) {
      const double u = double(raw_steps[i]) / double(n_train);
      const double sigma = shift * u / (1.0 + (shift - 1.0) * u);
      sigma_out[i] = sigma;
      if (label_out) label_out[i] = double(n_train) * sigma;
    }
    return ok();
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

ust_status ust_flow_step(const float* x, const void* v, const float* noise, float sigma,
                         float sigma_next, float* x0_out, float* x_next, int64_t n,
                         hipStream_t stream) {
  try {
    if (!x || !v || !x_next) return fail(UST_E_NULL, "x, v or x_next is NULL");
    if (sigma_next != 0.f && !noise)
      return fail(UST_E_NULL, "noise is NULL but sigma_next is %g, not 0", double(sigma_next));
    if (n < 0) return fail(UST_E_SHAPE, "n %lld < 0", static_cast<long long>(n));
    if (!(sigma >= 0.f && sigma <= 1.f) || !(sigma_next >= 0.f && sigma_next <= 1.f))
      return fail(UST_E_RANGE, "levels must lie in [0, 1] (got %g, %g)", double(sigma),
                  double(sigma_next));
    if (!aligned16(x) || !aligned16(v) || !aligned16(x_next) || (noise && !aligned16(noise)) ||
        (x0_out && !aligned16(x0_out)))
      return fail(UST_E_ALIGN, "pointers must be 16-byte aligned");
    if (n == 0) return ok();
    ust::FlowStepArgs a{x, static_cast<const uint16_t*>(v), sigma_next != 0.f ? noise : nullptr,
                        x0_out, x_next, n, sigma, sigma_next, 1.0f - sigma_next};
    return hip_status(ust::launch_flow_step(a, stream), "flow_step launch");
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

ust_status ust_calib_mfma_bf16(int32_t n_workgroups, int32_t iters, float* out,
                               double* flops_out, hipStream_t stream) {
  try {
    if (!out) return fail(UST_E_NULL, "out is NULL");
    if (n_workgroups <= 0 || n_workgroups > 65536 || iters <= 0)
      return fail(UST_E_SHAPE, "n_workgroups %d / iters %d out of range", n_workgroups, iters);
    if (!aligned16(out)) return fail(UST_E_ALIGN, "out must be 16-byte aligned");
    if (flops_out) *flops_out = ust::calib_mfma_flops(n_workgroups, iters);
    return hip_status(ust::launch_calib_mfma(n_workgroups, iters, out, stream), "calib launch");
  } catch (...) {
    return fail(UST_E_HIP, "internal error");
  }
}

ust_status ust_conv3d_causal(const void* x, const void* w, const float* bias, void* y,
                             int32_t T, int32_t H, int32_t W, int32_t Ci, int32_t Co,
                             hipStream_t stream) {
  return conv3d(x, w, bias, y, T, H, W, Ci, Co, false, stream);
}

ust_status ust_conv3d_causal_stream(const void* x, const void* w, const float* bias, void* y,
                                    int32_t T, int32_t H, int32_t W, int32_t Ci, int32_t Co,
                                    hipStream_t stream) {
  return conv3d(x, w, bias, y, T, H, W, Ci, Co, true, stream);
}

}  // extern "C"
