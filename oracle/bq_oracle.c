/*
 * bq_oracle.c -- plain CPU reference for block-quantized integer GEMM/GEMV.
 *
 * TEST INFRASTRUCTURE ONLY (see bq_oracle.h).  Plain C11 loops, no intrinsics,
 * no fast-math; built with gcc -O3 -ffp-contract=off so every float operation
 * is the IEEE operation written.  Page citations are in bq_oracle.h.
 */
#include "bq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* fp16 conversions                                                          */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

static float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round the non-negative integer v right by s bits, to nearest, ties to even. */
static uint32_t shift_rne(uint32_t v, int s) {
  if (s <= 0) return v;
  if (s > 31) return 0; /* v < 2^32 <= half of 2^s: rounds to 0 */
  uint32_t kept = v >> s;
  uint32_t rem = v & ((1u << s) - 1u);
  uint32_t half = 1u << (s - 1);
  if (rem > half || (rem == half && (kept & 1u))) kept += 1u;
  return kept;
}

uint16_t orc_f32_to_f16(float x) {
  uint32_t u = f32_bits(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t ex = (u >> 23) & 0xffu;
  uint32_t man = u & 0x7fffffu;
  if (ex == 0xffu) {                   /* inf or NaN */
    if (man == 0) return sign | 0x7c00u;
    return sign | 0x7e00u | (uint16_t)(man >> 13); /* quiet NaN */
  }
  if (ex == 0) return sign; /* +-0 and fp32 subnormals (< 2^-126) round to 0 */
  /* value = sig * 2^(e - 23) with a 24-bit significand sig */
  int e = (int)ex - 127;
  uint32_t sig = man | 0x800000u;
  if (e >= -14) {
    /* fp16 normal range: keep 11 significant bits */
    uint32_t m11 = shift_rne(sig, 13); /* 0x400 .. 0x800 */
    /* a carry to 0x800 moves to the next binade; the sum below handles it */
    uint32_t h = ((uint32_t)(e + 15) << 10) + (m11 - 0x400u);
    if (h >= 0x7c00u) return sign | 0x7c00u; /* overflow -> inf */
    return sign | (uint16_t)h;
  }
  /* fp16 subnormal range: count units of 2^-24; value / 2^-24 = sig * 2^(e+1) */
  int s = -(e + 1); /* >= 14 */
  uint32_t units = shift_rne(sig, s); /* 0 .. 0x400 (0x400 = smallest normal) */
  return sign | (uint16_t)units;
}

float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  uint32_t ex = ((uint32_t)h >> 10) & 0x1fu;
  uint32_t man = (uint32_t)h & 0x3ffu;
  if (ex == 0x1fu) return bits_f32(sign | 0x7f800000u | (man << 13));
  if (ex == 0) {
    /* zero or subnormal: man * 2^-24, exact in fp32 */
    float v = (float)man * 0x1p-24f;
    return sign ? -v : v;
  }
  return bits_f32(sign | ((ex - 15u + 127u) << 23) | (man << 13));
}

void orc_f32_to_f16_array(const float *x, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_array(const uint16_t *h, int64_t n, float *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------ */
/* Q8_0 quantization                                                          */
/* ------------------------------------------------------------------------ */

/* One block of 32 fp32 values -> 32 codes and a scale (fp16 bits). */
static void quantize_block_q8_0(const float *x, int8_t *q, uint16_t *d_out) {
  float amax = 0.0f;
  for (int i = 0; i < ORC_QK; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float d32 = amax / 127.0f; /* IEEE fp32 division */
  uint16_t dh = orc_f32_to_f16(d32);
  float d = orc_f16_to_f32(dh);
  if (d == 0.0f) {
    for (int i = 0; i < ORC_QK; ++i) q[i] = 0;
    *d_out = 0; /* +0: covers all-zero, all -0, and underflow */
    return;
  }
  for (int i = 0; i < ORC_QK; ++i) {
    double t = round((double)x[i] / (double)d); /* half away from zero */
    if (t > 127.0) t = 127.0;
    if (t < -127.0) t = -127.0;
    q[i] = (int8_t)t;
  }
  *d_out = dh;
}

void orc_quantize_q8_0_f32(const float *x, int64_t rows, int64_t k,
                           int64_t ldx, int8_t *q, uint16_t *d) {
  int64_t nb = k / ORC_QK;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      quantize_block_q8_0(x + r * ldx + b * ORC_QK, q + r * k + b * ORC_QK,
                          d + r * nb + b);
}

void orc_quantize_q8_0_f16(const uint16_t *x, int64_t rows, int64_t k,
                           int64_t ldx, int8_t *q, uint16_t *d) {
  int64_t nb = k / ORC_QK;
  float tmp[ORC_QK];
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      for (int i = 0; i < ORC_QK; ++i)
        tmp[i] = orc_f16_to_f32(x[r * ldx + b * ORC_QK + i]);
      quantize_block_q8_0(tmp, q + r * k + b * ORC_QK, d + r * nb + b);
    }
}

/* ------------------------------------------------------------------------ */
/* 4-bit group quantization, packing                                          */
/* ------------------------------------------------------------------------ */

void orc_pack_w4(const uint8_t *codes, int64_t rows, int64_t k,
                 uint8_t *packed) {
  int64_t ng = k / ORC_QK;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < ng; ++g) {
      const uint8_t *c = codes + r * k + g * ORC_QK;
      uint8_t *p = packed + r * (k / 2) + g * (ORC_QK / 2);
      for (int j = 0; j < ORC_QK / 2; ++j)
        p[j] = (uint8_t)((c[j] & 0x0f) | ((c[j + ORC_QK / 2] & 0x0f) << 4));
    }
}

void orc_unpack_w4(const uint8_t *packed, int64_t rows, int64_t k,
                   uint8_t *codes) {
  int64_t ng = k / ORC_QK;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < ng; ++g) {
      const uint8_t *p = packed + r * (k / 2) + g * (ORC_QK / 2);
      uint8_t *c = codes + r * k + g * ORC_QK;
      for (int j = 0; j < ORC_QK / 2; ++j) {
        c[j] = p[j] & 0x0f;
        c[j + ORC_QK / 2] = (uint8_t)(p[j] >> 4);
      }
    }
}

void orc_quantize_w4(const float *w, int64_t rows, int64_t k, uint8_t *packed,
                     uint16_t *d) {
  int64_t ng = k / ORC_QK;
  uint8_t codes[ORC_QK];
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < ng; ++g) {
      const float *x = w + r * k + g * ORC_QK;
      float amax = 0.0f;
      for (int i = 0; i < ORC_QK; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
      }
      uint16_t dh = orc_f32_to_f16(amax / 7.0f);
      float dd = orc_f16_to_f32(dh);
      for (int i = 0; i < ORC_QK; ++i) {
        double t = 0.0;
        if (dd != 0.0f) {
          t = round((double)x[i] / (double)dd);
          if (t > 7.0) t = 7.0;
          if (t < -7.0) t = -7.0;
        }
        codes[i] = (uint8_t)((int)t + 8);
      }
      if (dd == 0.0f) dh = 0;
      d[r * ng + g] = dh;
      /* pack this group (same layout as orc_pack_w4) */
      uint8_t *p = packed + r * (k / 2) + g * (ORC_QK / 2);
      for (int j = 0; j < ORC_QK / 2; ++j)
        p[j] = (uint8_t)(codes[j] | (codes[j + ORC_QK / 2] << 4));
    }
}

/* ------------------------------------------------------------------------ */
/* Block dots and GEMMs                                                       */
/* ------------------------------------------------------------------------ */

static int32_t dot_block_i8(const int8_t *a, const int8_t *w) {
  int32_t s = 0;
  for (int i = 0; i < ORC_QK; ++i) s += (int32_t)a[i] * (int32_t)w[i];
  return s;
}

void orc_block_dots(const int8_t *aq, int64_t m, const int8_t *wq, int64_t n,
                    int64_t k, int32_t *P) {
  int64_t nb = k / ORC_QK;
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j)
      for (int64_t b = 0; b < nb; ++b)
        P[(i * n + j) * nb + b] =
            dot_block_i8(aq + i * k + b * ORC_QK, wq + j * k + b * ORC_QK);
}

/* One output of the Q8_0 GEMM: exact fp64 terms, summed in block order. */
static void q8_output(const int8_t *arow, const uint16_t *adrow,
                      const int8_t *wrow, const uint16_t *wdrow, int64_t k,
                      double *y, double *asum) {
  int64_t nb = k / ORC_QK;
  double acc = 0.0, aacc = 0.0;
  for (int64_t b = 0; b < nb; ++b) {
    int32_t p = dot_block_i8(arow + b * ORC_QK, wrow + b * ORC_QK);
    double term = (double)orc_f16_to_f32(wdrow[b]) *
                  (double)orc_f16_to_f32(adrow[b]) * (double)p;
    acc += term;
    aacc += fabs(term);
  }
  if (y) *y = acc;
  if (asum) *asum = aacc;
}

typedef struct {
  const int8_t *aq;
  const uint16_t *ad;
  const int8_t *wq;
  const uint16_t *wd;
  int64_t n, k, r0, r1;
  double *y, *asum;
} q8_job;

static void *q8_rows(void *arg) {
  q8_job *J = (q8_job *)arg;
  int64_t nb = J->k / ORC_QK;
  for (int64_t i = J->r0; i < J->r1; ++i)
    for (int64_t j = 0; j < J->n; ++j)
      q8_output(J->aq + i * J->k, J->ad + i * nb, J->wq + j * J->k,
                J->wd + j * nb, J->k, J->y ? J->y + i * J->n + j : NULL,
                J->asum ? J->asum + i * J->n + j : NULL);
  return NULL;
}

void orc_qgemm_q8_0(const int8_t *aq, const uint16_t *ad, int64_t m,
                    const int8_t *wq, const uint16_t *wd, int64_t n, int64_t k,
                    double *y, double *asum, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > m) nthreads = (int)(m > 0 ? m : 1);
  q8_job *jobs = (q8_job *)calloc((size_t)nthreads, sizeof(q8_job));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int t = 0; t < nthreads; ++t) {
    q8_job J = {aq, ad, wq, wd, n, k, m * t / nthreads, m * (t + 1) / nthreads,
                y, asum};
    jobs[t] = J;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, q8_rows, &jobs[t]);
  q8_rows(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(jobs);
  free(th);
}

void orc_qgemm_q8_0_at(const int8_t *aq, const uint16_t *ad, int64_t m,
                       const int8_t *wq, const uint16_t *wd, int64_t n,
                       int64_t k, const int64_t *mi, const int64_t *nj,
                       int64_t count, double *y, double *asum) {
  (void)m;
  (void)n;
  int64_t nb = k / ORC_QK;
  for (int64_t c = 0; c < count; ++c)
    q8_output(aq + mi[c] * k, ad + mi[c] * nb, wq + nj[c] * k, wd + nj[c] * nb,
              k, y ? y + c : NULL, asum ? asum + c : NULL);
}

int64_t orc_route_topk(const int32_t *ids, int64_t T, int64_t top_k, int64_t E,
                       int32_t *counts, int32_t *offsets, int32_t *rows) {
  int64_t R = T * top_k, invalid = 0;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t r = 0; r < R; ++r) {
    int32_t e = ids[r];
    if (e < 0 || e >= E)
      ++invalid;
    else
      ++counts[e];
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  /* stable placement: scan rows in increasing order */
  int32_t *fill = (int32_t *)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
  for (int64_t r = 0; r < R; ++r) {
    int32_t e = ids[r];
    if (e < 0 || e >= E) continue;
    rows[offsets[e] + fill[e]++] = (int32_t)r;
  }
  free(fill);
  return invalid;
}

/* One output of the grouped W4A8 GEMM for routed row r and column c. */
static void w4_output(const int8_t *aq, const uint16_t *ad, const int32_t *ids,
                      int64_t top_k, const uint8_t *wq4, const uint16_t *wd,
                      int64_t E, int64_t n, int64_t k, int64_t r, int64_t c,
                      double *y, double *asum) {
  int64_t nb = k / ORC_QK;
  int32_t e = ids[r];
  double acc = 0.0, aacc = 0.0;
  if (e >= 0 && e < E) {
    int64_t t = r / top_k;
    const int8_t *arow = aq + t * k;
    const uint16_t *adrow = ad + t * nb;
    const uint8_t *wrow = wq4 + ((int64_t)e * n + c) * (k / 2);
    const uint16_t *wdrow = wd + ((int64_t)e * n + c) * nb;
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t *p = wrow + b * (ORC_QK / 2);
      int32_t s = 0;
      for (int j = 0; j < ORC_QK / 2; ++j) {
        int32_t lo = (int32_t)(p[j] & 0x0f) - 8;
        int32_t hi = (int32_t)(p[j] >> 4) - 8;
        s += lo * (int32_t)arow[b * ORC_QK + j];
        s += hi * (int32_t)arow[b * ORC_QK + j + ORC_QK / 2];
      }
      double term = (double)orc_f16_to_f32(wdrow[b]) *
                    (double)orc_f16_to_f32(adrow[b]) * (double)s;
      acc += term;
      aacc += fabs(term);
    }
  }
  if (y) *y = acc;
  if (asum) *asum = aacc;
}

typedef struct {
  const int8_t *aq;
  const uint16_t *ad;
  const int32_t *ids;
  int64_t top_k;
  const uint8_t *wq4;
  const uint16_t *wd;
  int64_t E, n, k, r0, r1;
  double *y, *asum;
} w4_job;

static void *w4_rows(void *arg) {
  w4_job *J = (w4_job *)arg;
  for (int64_t r = J->r0; r < J->r1; ++r)
    for (int64_t c = 0; c < J->n; ++c)
      w4_output(J->aq, J->ad, J->ids, J->top_k, J->wq4, J->wd, J->E, J->n,
                J->k, r, c, J->y ? J->y + r * J->n + c : NULL,
                J->asum ? J->asum + r * J->n + c : NULL);
  return NULL;
}

void orc_qgemm_w4a8_grouped(const int8_t *aq, const uint16_t *ad, int64_t T,
                            const int32_t *ids, int64_t top_k,
                            const uint8_t *wq4, const uint16_t *wd, int64_t E,
                            int64_t n, int64_t k, double *y, double *asum,
                            int nthreads) {
  int64_t R = T * top_k;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > R) nthreads = (int)(R > 0 ? R : 1);
  w4_job *jobs = (w4_job *)calloc((size_t)nthreads, sizeof(w4_job));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int t = 0; t < nthreads; ++t) {
    w4_job J = {aq, ad, ids, top_k, wq4, wd, E, n, k,
                R * t / nthreads, R * (t + 1) / nthreads, y, asum};
    jobs[t] = J;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, w4_rows, &jobs[t]);
  w4_rows(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(jobs);
  free(th);
}

void orc_qgemm_w4a8_grouped_at(const int8_t *aq, const uint16_t *ad, int64_t T,
                               const int32_t *ids, int64_t top_k,
                               const uint8_t *wq4, const uint16_t *wd,
                               int64_t E, int64_t n, int64_t k,
                               const int64_t *ri, const int64_t *cj,
                               int64_t count, double *y, double *asum) {
  (void)T;
  for (int64_t c = 0; c < count; ++c)
    w4_output(aq, ad, ids, top_k, wq4, wd, E, n, k, ri[c], cj[c],
              y ? y + c : NULL, asum ? asum + c : NULL);
}

/* ---- MoE combine ---------------------------------------------------------------- */

void orc_moe_combine(const float *y, const float *p, int64_t T, int64_t top_k,
                     int64_t n, double *out, double *asum) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < n; ++c) {
      double s = 0.0, a = 0.0;
      for (int64_t j = 0; j < top_k; ++j) {
        /* product of two fp32 values: exact in fp64 (24 + 24 bits) */
        const double term = (double)p[t * top_k + j] * (double)y[(t * top_k + j) * n + c];
        s += term;
        a += fabs(term);
      }
      out[t * n + c] = s;
      if (asum) asum[t * n + c] = a;
    }
}

/* ---- GGUF block import ---------------------------------------------------------- */

static uint16_t le16(const uint8_t *b) { return (uint16_t)(b[0] | (b[1] << 8)); }

void orc_gguf_q8_0_to_planar(const uint8_t *blocks, int64_t rows, int64_t k,
                             int8_t *q, uint16_t *d) {
  const int64_t nb = k / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t *blk = blocks + (r * nb + b) * 34;
      d[r * nb + b] = le16(blk);
      for (int i = 0; i < 32; ++i) q[r * k + 32 * b + i] = (int8_t)blk[2 + i];
    }
}

void orc_gguf_q4_0_to_planar(const uint8_t *blocks, int64_t rows, int64_t k,
                             uint8_t *packed, uint16_t *d) {
  const int64_t nb = k / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t *blk = blocks + (r * nb + b) * 18;
      d[r * nb + b] = le16(blk);
      for (int i = 0; i < 16; ++i) packed[r * (k / 2) + 16 * b + i] = blk[2 + i];
    }
}
