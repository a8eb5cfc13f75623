/*
 * bq_oracle.h -- plain CPU reference ("oracle") for block-quantized integer
 * GEMM/GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may link,
 * load or call this code; it exists so that tests, the smoke check and the
 * CPU-baseline leg of the benchmark can check the HIP kernels against an
 * independent, obviously-correct implementation.  It shares no source, header,
 * table or constant generator with the HIP path.
 *
 * Sources for what is computed:
 *  - "Q8_0": named as the prefill GEMM's weight/activation format in
 *    "I wrote a custom CUDA inference engine to run Qwen3.5-27B on a $130
 *    mining card" (euno.news), section "Features" and section "Honest
 *    benchmark" ("same Q8_0 GGUFs"), and in the axbrief.com article on the
 *    same engine, section "DP4A kernels and 3-bit KV cache".  The pages name
 *    the format but do not define it; this library fixes it as: 32-element
 *    blocks along K, one fp16 scale per block equal to absmax/127 rounded to
 *    nearest-even, codes round-half-away-from-zero of x/d clamped to +-127.
 *  - W4A8: "group-wise symmetric 4-bit (Q4_0 family)" weights with 8-bit
 *    activations, "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB
 *    2011 GPU" (gist.science summary), Method 1 (hybrid prefill/decode) and
 *    Method 2 (memory and quantization); the grouped 4-bit GEMM for MoE
 *    routing is in Method 1.  Fixed here as 32-element groups, codes 0..15
 *    with offset 8, fp16 scale.
 *
 * Where the pages are silent the readings are stated next to each function.
 * All floating-point results that are not themselves quantities of the format
 * are computed in fp64 from exact per-block terms.
 */
#ifndef BQ_ORACLE_H
#define BQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_QK 32 /* elements per quantization block / group along K */

/* ---- fp16 (IEEE binary16) conversions, written out bit by bit ---------- */

/* fp32 -> fp16, round to nearest, ties to even; keeps subnormals; values
 * that round beyond 65504 become +-inf; NaN stays NaN (quiet). */
uint16_t orc_f32_to_f16(float x);
/* fp16 -> fp32, exact (every fp16 value is an fp32 value). */
float orc_f16_to_f32(uint16_t h);
/* Array forms of the two conversions (used by the exhaustive pins). */
void orc_f32_to_f16_array(const float *x, int64_t n, uint16_t *out);
void orc_f16_to_f32_array(const uint16_t *h, int64_t n, float *out);

/* ---- Q8_0 quantization ---------------------------------------------------
 * Per row r and block b (elements 32b..32b+31 of the row):
 *   amax = max |x|                       (fp32; fp16 input widened exactly)
 *   d    = fp16_rne(amax / 127)          (fp32 IEEE division, then RNE)
 *   q_i  = 0 if d == 0, else clamp(round_half_away(x_i / d), -127, 127)
 *          where x_i / d is the exact quotient with the *stored* fp16 d
 *          (evaluated in fp64, which decides the rounding exactly here).
 * x is [rows][ldx] (ldx >= k), q is [rows][k] int8, d is [rows][k/32] fp16
 * bits.  k must be a multiple of 32. */
void orc_quantize_q8_0_f32(const float *x, int64_t rows, int64_t k,
                           int64_t ldx, int8_t *q, uint16_t *d);
void orc_quantize_q8_0_f16(const uint16_t *x, int64_t rows, int64_t k,
                           int64_t ldx, int8_t *q, uint16_t *d);

/* ---- 4-bit group quantization (test data only) ----------------------------
 * Per 32-group: d = fp16_rne(amax / 7); q = clamp(round_half_away(x/d), -7, 7);
 * code c = q + 8 (so 1..15; the GEMM itself accepts all 16 codes).
 * Packing: a group's 32 codes occupy 16 bytes; byte j holds element j in its
 * low nibble and element j+16 in its high nibble.  packed is [rows][k/2],
 * d is [rows][k/32]. */
void orc_quantize_w4(const float *w, int64_t rows, int64_t k, uint8_t *packed,
                     uint16_t *d);
/* Packed nibbles -> one code (0..15) per element, [rows][k]. */
void orc_unpack_w4(const uint8_t *packed, int64_t rows, int64_t k,
                   uint8_t *codes);
/* One code per element (0..15) -> packed nibbles, inverse of the above. */
void orc_pack_w4(const uint8_t *codes, int64_t rows, int64_t k,
                 uint8_t *packed);

/* ---- per-block integer dot products ---------------------------------------
 * P[i][j][b] = sum_{t<32} aq[i][32b+t] * wq[j][32b+t]  (exact int32).
 * aq is [m][k], wq is [n][k], P is [m][n][k/32]. */
void orc_block_dots(const int8_t *aq, int64_t m, const int8_t *wq, int64_t n,
                    int64_t k, int32_t *P);

/* ---- Q8_0 x Q8_0 GEMM ---------------------------------------------------------
 * y[i][j] = sum_b  wd[j][b] * ad[i][b] * P[i][j][b]
 * Each term is formed exactly in fp64 (11 + 11 + 20 significant bits) and the
 * terms are summed in fp64 in block order.  asum[i][j] = sum_b |term_b| is the
 * scale of the acceptance bound for an fp32 result.  y and asum are [m][n]
 * (either may be NULL).  nthreads <= 1 runs on the calling thread; otherwise
 * output rows are split evenly over that many threads. */
void orc_qgemm_q8_0(const int8_t *aq, const uint16_t *ad, int64_t m,
                    const int8_t *wq, const uint16_t *wd, int64_t n, int64_t k,
                    double *y, double *asum, int nthreads);
/* The same quantity for `count` chosen outputs (mi[c], nj[c]). */
void orc_qgemm_q8_0_at(const int8_t *aq, const uint16_t *ad, int64_t m,
                       const int8_t *wq, const uint16_t *wd, int64_t n,
                       int64_t k, const int64_t *mi, const int64_t *nj,
                       int64_t count, double *y, double *asum);

/* ---- routing: top-k expert ids -> per-expert row groups -----------------------
 * ids is [T][top_k]; the routed row of (t, j) is r = t*top_k + j.
 * counts[e] = number of r with ids[r] == e; offsets[e] = sum_{e'<e} counts[e']
 * (offsets has E+1 entries); rows[offsets[e] .. offsets[e+1]) lists the r with
 * ids[r] == e in increasing r.  Ids outside [0, E) are left out.
 * Returns the number of left-out (invalid) entries. */
int64_t orc_route_topk(const int32_t *ids, int64_t T, int64_t top_k, int64_t E,
                       int32_t *counts, int32_t *offsets, int32_t *rows);

/* ---- grouped W4A8 GEMM ------------------------------------------------------------
 * For each routed row r = t*top_k + j with e = ids[r] in [0, E):
 *   y[r][c] = sum_b wd[e][c][b] * ad[t][b] * sum_{u<32} (code[e][c][32b+u] - 8) * aq[t][32b+u]
 * with the same exact fp64 terms and asum as the Q8_0 GEMM; rows with an
 * invalid id are 0 (asum 0).  wq4 is [E][n][k/2] packed as above,
 * wd is [E][n][k/32], y/asum are [T*top_k][n]. */
void orc_qgemm_w4a8_grouped(const int8_t *aq, const uint16_t *ad, int64_t T,
                            const int32_t *ids, int64_t top_k,
                            const uint8_t *wq4, const uint16_t *wd, int64_t E,
                            int64_t n, int64_t k, double *y, double *asum,
                            int nthreads);
/* The same for `count` chosen outputs (routed row ri[c], column cj[c]). */
void orc_qgemm_w4a8_grouped_at(const int8_t *aq, const uint16_t *ad, int64_t T,
                               const int32_t *ids, int64_t top_k,
                               const uint8_t *wq4, const uint16_t *wd,
                               int64_t E, int64_t n, int64_t k,
                               const int64_t *ri, const int64_t *cj,
                               int64_t count, double *y, double *asum);

/* ---- MoE combine (the step after the grouped GEMM) ---------------------------
 * "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU"
 * (gist.science summary), Method 1: the grouped 4-bit GEMM serves the MoE
 * routing; each token's expert outputs are then weighted by its router
 * probabilities and summed back in token order (Method 2 names the router
 * weighting).  For token t and column c:
 *   out[t][c] = sum_{j < top_k} p[t][j] * y[t][j][c]
 * Each product of two fp32 values is exact in fp64 and the sum is taken in
 * fp64 in slot order; asum[t][c] = sum_j |p[t][j] * y[t][j][c]| is the
 * tolerance scale.  y is [T][top_k][n] (fp32), p is [T][top_k]. */
void orc_moe_combine(const float *y, const float *p, int64_t T, int64_t top_k,
                     int64_t n, double *out, double *asum);

/* ---- GGUF block import ----------------------------------------------------------
 * "I wrote a custom CUDA inference engine to run Qwen3.5-27B on a $130 mining
 * card", Honest benchmark: the comparison runs on Q8_0 GGUF files.  On disk a
 * GGUF tensor of R rows x K columns (K % 32 == 0) is a contiguous array of
 * R*K/32 blocks, row-major, each block holding its fp16 scale (2 bytes,
 * little-endian) followed by its codes:
 *   Q8_0: 34 bytes = scale + 32 int8 codes;
 *   Q4_0: 18 bytes = scale + 16 bytes, byte j holding element j in its low
 *         nibble and element j+16 in its high nibble (value (nibble-8)*scale).
 * These split a block array into the planar layout of this library: codes
 * [R][K] (Q8_0) or packed [R][K/2] (Q4_0, the same nibble order), and scales
 * [R][K/32]. */
void orc_gguf_q8_0_to_planar(const uint8_t *blocks, int64_t rows, int64_t k,
                             int8_t *q, uint16_t *d);
void orc_gguf_q4_0_to_planar(const uint8_t *blocks, int64_t rows, int64_t k,
                             uint8_t *packed, uint16_t *d);

#ifdef __cplusplus
}
#endif
#endif /* BQ_ORACLE_H */
