// Cached 3-D RoPE coefficients (UnStep, abstract: RoPE is applied from
// precomputed coefficients).  One thread per (frame, row, col, pair); angles in fp64,
// stored as fp32.  Row f of the table is the absolute frame first_frame + f.
// Runs once per geometry (or once per chunk for a table of the chunk's
// frames), so it is written for clarity.

#include "ust_internal.h"

namespace ust {
namespace {

__global__ void __launch_bounds__(256)
rope_table_kernel(RopeTableArgs a) {
  const int P = a.pairs_t + a.pairs_h + a.pairs_w;
  const int64_t total = int64_t(a.n_frames) * a.grid_h * a.grid_w * P;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int p = int(i % P);
  const int64_t tok = i / P;                 // ((f * grid_h) + y) * grid_w + x
  const int x = int(tok % a.grid_w);
  const int y = int((tok / a.grid_w) % a.grid_h);
  const int f = int(tok / (int64_t(a.grid_w) * a.grid_h));
  int pos, j, n;
  if (p < a.pairs_t) {
    pos = a.first_frame + f; j = p; n = a.pairs_t;
  } else if (p < a.pairs_t + a.pairs_h) {
    pos = y; j = p - a.pairs_t; n = a.pairs_h;
  } else {
    pos = x; j = p - a.pairs_t - a.pairs_h; n = a.pairs_w;
  }
  const double freq = pow(a.theta, -double(j) / double(n));
  const double ang = double(pos) * freq;
  a.cos_out[i] = float(cos(ang));
  a.sin_out[i] = float(sin(ang));
}

}  // namespace

hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t s) {
  const int P = a.pairs_t + a.pairs_h + a.pairs_w;
  const int64_t total = int64_t(a.n_frames) * a.grid_h * a.grid_w * P;
  const int blocks = int((total + 255) / 256);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ust
