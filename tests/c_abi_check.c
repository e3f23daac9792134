/*
 * Drives libust.so through its C ABI alone (C11, no Python, no C++), on the
 * GPU, with a small geometry: 2 heads x 64, 4 x 6 tokens per frame, chunks of
 * 3 frames, a 7-slot ring with 1 sink (it wraps), 3 recent frames.  Built by
 * the package's build step and run by test_gpu_parity.py.  It checks:
 *  - argument errors come back as statuses, with a message in ust_last_error;
 *  - with every value equal to 1 the attention returns 1 everywhere (each
 *    softmax row sums to 1), to the rounding of the bf16 probabilities;
 *  - on random inputs the key-split schedule (5 workgroups) agrees with the
 *    one-workgroup-per-tile schedule within the bf16 bar, and both are finite;
 *  - ust_window_attn_work_bytes matches its stated formula;
 *  - a RoPE table of the last chunk's own three frames gives the attention
 *    bit for bit as the table from frame 0, and ranges it does not hold are
 *    rejected;
 *  - ust_sigma_schedule gives the shift-5 levels 1 and 5/6 for raw 1000 and
 *    500, and ust_flow_step matches a double-precision loop within fp32
 *    rounding (2^-21 of the magnitudes involved: four roundings at most),
 *    for a size with a ragged tail, and rejects a NULL noise when it would
 *    be read.
 * Prints "ok" or the first failure and exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "../include/ust.h"

static uint16_t to_bf16(float f) {  /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t lcg_state = 12345u;
static float uniform_pm1(void) {  /* in [-1, 1) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)(lcg_state >> 8) * (2.0f / 16777216.0f) - 1.0f;
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      printf("FAIL %s: %s\n", #x, hipGetErrorString(e_));                      \
      return 1;                                                                \
    }                                                                          \
  } while (0)
#define UST_OK_(x)                                                             \
  do {                                                                         \
    ust_status s_ = (x);                                                       \
    if (s_ != UST_OK) {                                                        \
      printf("FAIL %s: %s %s\n", #x, ust_status_str(s_), ust_last_error());    \
      return 1;                                                                \
    }                                                                          \
  } while (0)
#define EXPECT(cond, ...)                                                      \
  do {                                                                         \
    if (!(cond)) {                                                             \
      printf("FAIL ");                                                         \
      printf(__VA_ARGS__);                                                     \
      printf("\n");                                                            \
      return 1;                                                                \
    }                                                                          \
  } while (0)

enum { GH = 4, GW = 6, T = GH * GW, H = 2, D = 64, CF = 3, NQ = T * CF, NF = 12 };
enum { N_SLOTS = 7, N_SINK = 1, N_RECENT = 3, N_CHUNKS = 4, N_WG = 5 };

int main(void) {
  const ust_geom g = {GH, GW, H, D, 12, 10, 10, CF};
  const int TV = ust_v_row_len(T);
  const size_t nk = (size_t)N_SLOTS * H * T * D, nv = (size_t)N_SLOTS * H * D * TV;
  const size_t nc = (size_t)NQ * H * D, nt = (size_t)NF * T * (D / 2);
  const size_t work_bytes = ust_window_attn_work_bytes(&g, N_WG);
  EXPECT(work_bytes == (size_t)2 * N_WG * 256 * (D + 1) * 4, "work bytes %zu", work_bytes);

  void *k, *v, *q, *kn, *vn, *o1, *o2, *work;
  float *cs, *sn;
  HIP_OK(hipMalloc(&k, nk * 2));
  HIP_OK(hipMalloc(&v, nv * 2));
  HIP_OK(hipMalloc(&q, nc * 2));
  HIP_OK(hipMalloc(&kn, nc * 2));
  HIP_OK(hipMalloc(&vn, nc * 2));
  HIP_OK(hipMalloc(&o1, nc * 2));
  HIP_OK(hipMalloc(&o2, nc * 2));
  HIP_OK(hipMalloc(&work, work_bytes));
  HIP_OK(hipMalloc((void**)&cs, nt * 4));
  HIP_OK(hipMalloc((void**)&sn, nt * 4));
  HIP_OK(hipMemset(k, 0, nk * 2));
  HIP_OK(hipMemset(v, 0, nv * 2));
  const ust_kv ring = {k, v, N_SLOTS, N_SINK};

  /* argument errors: nothing is launched, a status and a message come back */
  EXPECT(ust_window_attn(&g, &ring, NULL, cs, sn, 0, NF, 0, N_RECENT, 0.f, o1, NULL, 0) == UST_E_NULL &&
             strlen(ust_last_error()) > 0, "NULL q not rejected");
  EXPECT(ust_kv_append(&g, &ring, kn, vn, cs, sn, 0, NF, NF - 2, 0) == UST_E_RANGE,
         "chunk past the table not rejected");
  EXPECT(ust_window_attn_split(&g, &ring, q, cs, sn, 0, NF, 0, N_RECENT, 0.f, o1, NULL, work,
                               work_bytes - 4, N_WG, 0) == UST_E_SHAPE, "small workspace not rejected");

  UST_OK_(ust_rope_table_build(&g, 0, NF, 10000.0, cs, sn, 0));

  uint16_t* hq = malloc(nc * 2);
  uint16_t* hk = malloc(nc * 2);
  uint16_t* hv = malloc(nc * 2);
  uint16_t* h1 = malloc(nc * 2);
  uint16_t* h2 = malloc(nc * 2);
  if (!hq || !hk || !hv || !h1 || !h2) return 1;

  for (int pass = 0; pass < 2; ++pass) {   /* 0: V = 1; 1: random V */
    for (int c = 0; c < N_CHUNKS; ++c) {
      for (size_t i = 0; i < nc; ++i) {
        hq[i] = to_bf16(uniform_pm1());
        hk[i] = to_bf16(uniform_pm1());
        hv[i] = pass == 0 ? to_bf16(1.0f) : to_bf16(uniform_pm1());
      }
      HIP_OK(hipMemcpy(q, hq, nc * 2, hipMemcpyHostToDevice));
      HIP_OK(hipMemcpy(kn, hk, nc * 2, hipMemcpyHostToDevice));
      HIP_OK(hipMemcpy(vn, hv, nc * 2, hipMemcpyHostToDevice));
      UST_OK_(ust_kv_append(&g, &ring, kn, vn, cs, sn, 0, NF, CF * c, 0));
      UST_OK_(ust_window_attn(&g, &ring, q, cs, sn, 0, NF, CF * c, N_RECENT, 0.f, o1, NULL, 0));
      UST_OK_(ust_window_attn_split(&g, &ring, q, cs, sn, 0, NF, CF * c, N_RECENT, 0.f, o2, NULL,
                                    work, work_bytes, N_WG, 0));
      HIP_OK(hipDeviceSynchronize());
      HIP_OK(hipMemcpy(h1, o1, nc * 2, hipMemcpyDeviceToHost));
      HIP_OK(hipMemcpy(h2, o2, nc * 2, hipMemcpyDeviceToHost));
      double max_d = 0.0;
      for (size_t i = 0; i < nc; ++i) {
        const float a = from_bf16(h1[i]), b = from_bf16(h2[i]);
        EXPECT(isfinite(a) && isfinite(b), "non-finite output (pass %d chunk %d)", pass, c);
        if (pass == 0)   /* sum of bf16 probabilities over their fp32 sum */
          EXPECT(fabsf(a - 1.0f) <= 1.0f / 128 && fabsf(b - 1.0f) <= 1.0f / 128,
                 "V = 1 gave %g / %g (chunk %d)", a, b, c);
        if (fabs((double)a - b) > max_d) max_d = fabs((double)a - b);
      }
      EXPECT(max_d <= 2e-2, "split vs unsplit differ by %g (pass %d chunk %d)", max_d, pass, c);
    }
  }
  /* a table of the last chunk's own frames gives the same attention, bit for
     bit, as the table from frame 0 (h1 holds that chunk's output) */
  {
    const int f0 = CF * (N_CHUNKS - 1);
    float *cs3, *sn3;
    const size_t nt3 = (size_t)CF * T * (D / 2);
    HIP_OK(hipMalloc((void**)&cs3, nt3 * 4));
    HIP_OK(hipMalloc((void**)&sn3, nt3 * 4));
    EXPECT(ust_rope_table_build(&g, -1, CF, 10000.0, cs3, sn3, 0) == UST_E_RANGE,
           "negative first frame accepted");
    UST_OK_(ust_rope_table_build(&g, f0, CF, 10000.0, cs3, sn3, 0));
    EXPECT(ust_window_attn(&g, &ring, q, cs3, sn3, f0 + 1, CF, f0, N_RECENT, 0.f, o2, NULL, 0) ==
               UST_E_RANGE, "chunk before the table accepted");
    UST_OK_(ust_window_attn(&g, &ring, q, cs3, sn3, f0, CF, f0, N_RECENT, 0.f, o2, NULL, 0));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(h2, o2, nc * 2, hipMemcpyDeviceToHost));
    EXPECT(memcmp(h1, h2, nc * 2) == 0, "chunk table and full table differ");
    HIP_OK(hipFree(cs3));
    HIP_OK(hipFree(sn3));
  }
  /* the sampler step */
  {
    const int32_t raw[2] = {1000, 500};
    double sig[2], lab[2];
    UST_OK_(ust_sigma_schedule(raw, 2, 5.0, 1000, sig, lab));
    EXPECT(sig[0] == 1.0 && fabs(sig[1] - 5.0 / 6.0) < 1e-15 && fabs(lab[1] - 2500.0 / 3.0) < 1e-12,
           "sigma schedule %g %g", sig[0], sig[1]);
    enum { NS = 1001 };
    float hx[NS], he[NS], hn[NS];
    uint16_t hvb[NS];
    for (int i = 0; i < NS; ++i) {
      hx[i] = 2.0f * uniform_pm1();
      he[i] = uniform_pm1();
      hvb[i] = to_bf16(uniform_pm1());
    }
    float *dx, *de, *dn;
    void* dv;
    HIP_OK(hipMalloc((void**)&dx, sizeof(hx)));
    HIP_OK(hipMalloc((void**)&de, sizeof(he)));
    HIP_OK(hipMalloc((void**)&dn, sizeof(hn)));
    HIP_OK(hipMalloc(&dv, sizeof(hvb)));
    HIP_OK(hipMemcpy(dx, hx, sizeof(hx), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(de, he, sizeof(he), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, hvb, sizeof(hvb), hipMemcpyHostToDevice));
    const float s = (float)sig[1], sn = 0.02f;
    EXPECT(ust_flow_step(dx, dv, NULL, s, sn, NULL, dn, NS, 0) == UST_E_NULL, "NULL noise accepted");
    UST_OK_(ust_flow_step(dx, dv, de, s, sn, NULL, dn, NS, 0));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hn, dn, sizeof(hn), hipMemcpyDeviceToHost));
    for (int i = 0; i < NS; ++i) {
      const double v = from_bf16(hvb[i]);
      const double x0 = (double)hx[i] - (double)s * v;
      const double ref = (1.0 - (double)sn) * x0 + (double)sn * he[i];
      const double mag = fabs((double)hx[i]) + fabs((double)s * v) + fabs((double)sn * he[i]);
      EXPECT(fabs(hn[i] - ref) <= ldexp(mag, -21), "flow step %d: %g vs %g", i, hn[i], ref);
    }
  }
  printf("ok\n");
  return 0;
}
