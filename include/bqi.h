/*
 * bqi.h -- block-quantized integer GEMM/GEMV for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbqi.so.  Every entry point takes plain pointers and sizes, is
 * enqueued asynchronously on the caller's HIP stream, never allocates, frees
 * or synchronizes, and returns a status code.  All argument checks happen on
 * the host before any HIP call, so a rejected call launches nothing.
 *
 * Formats (the pages name them; the definitions below are this library's):
 *
 *  Q8_0  -- named as the format of the hand-written prefill GEMM in "I wrote a
 *    custom CUDA inference engine to run Qwen3.5-27B on a $130 mining card"
 *    (euno.news), section "Features", and of the benchmarked GGUF models in
 *    section "Honest benchmark"; the axbrief.com article on the same engine,
 *    section "DP4A kernels and 3-bit KV cache", describes the int8 DP4A GEMM.
 *    A Q8_0 matrix with R rows and K columns (K a multiple of 32) is stored
 *    planar: codes int8 [R][K] row-major, and scales as fp16 bit patterns
 *    uint16 [R][K/32] row-major; element (r, c) represents
 *    code[r][c] * scale[r][c/32].
 *
 *  W4 groups -- "group-wise symmetric 4-bit (Q4_0 family)" weights used with
 *    8-bit activations, "A 35B Hybrid-Attention Mixture-of-Experts Model on a
 *    6GB 2011 GPU: Hand-Written 4-bit CUDA Inference for Fermi" (gist.science
 *    summary), Method 2; the grouped 4-bit GEMM for MoE routing is in its
 *    Method 1.  A 4-bit matrix [R][K] is stored as packed codes uint8
 *    [R][K/2] and fp16 scales uint16 [R][K/32].  Within each 32-element
 *    group (16 bytes), byte j holds element j in its low nibble and element
 *    j+16 in its high nibble.  Element value = (code - 8) * scale.
 *
 * Below, "mining card" cites the euno.news article and "2011 GPU" the
 * gist.science summary, each with its section.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers, allocated and owned by the caller.
 *  - `stream` is a hipStream_t (NULL = the default stream).
 *  - Zero-sized problems return BQI_OK without launching anything.
 *  - Code arrays (int8 codes, packed nibbles) must be 16-byte aligned; scale
 *    arrays 2-byte aligned; fp32 outputs 4-byte aligned.
 *  - Results are deterministic: the same inputs give bit-identical outputs
 *    (no atomics in any floating-point reduction).
 *  - Calls are thread-safe, except overlapping calls of
 *    qgemm_w4a8_grouped_noalloc on one GPU (they share its workspace array).
 *    State kept between calls: that array, the worker threads of
 *    qgemm_w4a8_grouped_host, and kernel attributes (larger LDS limits) set
 *    once per device; none of it changes a result.
 */
#ifndef BQI_H
#define BQI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of this header are the only ones libbqi.so exports. */
#if defined(__GNUC__) || defined(__clang__)
#define BQI_API __attribute__((visibility("default")))
#else
#define BQI_API
#endif

/* status codes */
#define BQI_OK 0
#define BQI_EINVAL (-1) /* null pointer with nonzero size, bad dtype, workspace too small */
#define BQI_ESHAPE (-2) /* negative size, K not a multiple of 32, ldx < k, size too large */
#define BQI_EALIGN (-3) /* a pointer or leading dimension violates the alignment rules */
#define BQI_EHIP (-4)   /* the HIP runtime reported an error at launch */
#define BQI_ENOTSUP (-5) /* the host CPU lacks the instructions a host entry point needs */

/* activation dtypes for quantize_q8_0 */
#define BQI_F32 0
#define BQI_F16 1

/* Human-readable name of a status code (static string, never NULL). */
BQI_API const char *bqi_status_string(int status);

/* ABI version of this header (major * 100 + minor): 240.  Version 200 added
 * the k argument of qgemm_w4a8_grouped_workspace_size; 210 added
 * quantize_qgemm_q8_0; 220 added moe_combine_f32 and the GGUF import; 230
 * added qgemm_w4a8_grouped_host; 240 added qgemm_w4a8_grouped_noalloc. */
BQI_API int bqi_abi_version(void);

/*
 * quantize_q8_0 -- activations to Q8_0 (the quantizer of the pages' Q8_0
 * prefill path, "mining card", Features; and of the 8-bit activations of
 * W4A8, "2011 GPU", Method 2).
 *
 *   x      [rows][ldx] fp32 (x_dtype = BQI_F32) or fp16 (BQI_F16), row-major;
 *          only the first k columns of each row are read.
 *   q      [rows][k] int8 codes (output).
 *   d      [rows][k/32] fp16 scale bits (output).
 *
 * Per row and 32-element block:  amax = max|x| (fp16 input widened exactly),
 * d = fp16 round-to-nearest-even of (amax / 127) computed as an IEEE fp32
 * division, q = clamp(round-half-away-from-zero(x / d), -127, 127) with x / d
 * the exact quotient by the stored fp16 d; d == 0 gives q = 0 and scale bits
 * 0x0000.  Subnormal scales are kept.  NaN/Inf inputs are outside the contract.
 *
 * Requirements: k % 32 == 0, ldx >= k; x 16-byte aligned and
 * ldx * sizeof(element) a multiple of 16 (fp32) or 8 (fp16); q 16-byte aligned.
 */
BQI_API int quantize_q8_0(const void *x, int x_dtype, int64_t rows, int64_t k,
                  int64_t ldx, int8_t *q, uint16_t *d, void *stream);

/*
 * qgemm_q8_0 -- y = A * W^T with both operands Q8_0 (the prefill GEMM of
 * "mining card", Features, and the thin-M decode GEMM that "2011 GPU",
 * Results, names as the structural decode bottleneck).
 *
 *   aq [m][k] int8, ad [m][k/32] fp16 bits   -- activations A
 *   wq [n][k] int8, wd [n][k/32] fp16 bits   -- weights W (PyTorch Linear
 *                                               orientation: K contiguous)
 *   y  [m][n] fp32 row-major (output)
 *
 * y[i][j] = sum_b wd[j][b] * ad[i][b] * P[i][j][b], where
 * P[i][j][b] = sum_{t<32} aq[i][32b+t] * wq[j][32b+t] is the exact int32
 * block dot product (any int8 code, -128 included, is accepted).  Each term
 * is formed with at most one rounding and accumulated in fp32, each term
 * passing through at most nb = k/32 additions, so
 * |y - exact| <= (nb + 1) * 2^-24 * sum_b |term_b|  (below 1e-5 * sum|terms|
 * for k <= 5312).
 * m <= 16 runs the thin-M (decode) kernel, larger m the MFMA (prefill)
 * kernel, except that 16 < m <= 128 runs the thin-M MFMA kernel in chunks of
 * 16 rows where an estimate of both times (from m, n and k alone) favours
 * it; each chunk of at least 5 rows then comes out bit-identical to a call
 * on its rows alone.
 *
 * Requirements: k % 32 == 0; aq, wq 16-byte aligned; y 4-byte aligned.
 */
BQI_API int qgemm_q8_0(const int8_t *aq, const uint16_t *ad, int64_t m,
               const int8_t *wq, const uint16_t *wd, int64_t n, int64_t k,
               float *y, void *stream);

/*
 * quantize_qgemm_q8_0 -- quantize_q8_0 followed by qgemm_q8_0, the decode
 * step of the Q8_0 path (activation quantization, then the thin-M GEMM that
 * "2011 GPU", Results, names as the decode bottleneck).
 *
 *   x  [m][ldx] fp32 (x_dtype = BQI_F32) or fp16 (BQI_F16) activations
 *   wq [n][k] int8, wd [n][k/32] fp16 bits   -- Q8_0 weights
 *   y  [m][n] fp32 (output) = Q8_0(x) * W^T, bit-identical to qgemm_q8_0 on
 *      the codes below
 *   q  [m][k] int8, d [m][k/32] fp16 bits (output): the Q8_0 activations,
 *      bit-identical to quantize_q8_0(x)
 *
 * It is one launch for m == 1 with k <= 16384, and for 1 < m <= 16 with
 * m * k <= 4096 (16 KB of fp32) where the thin-M kernel of qgemm_q8_0 has a
 * quantizing form (the register kernel for m <= 4; the MFMA thin-M kernel
 * with k <= 1024 for m > 4): that kernel quantizes the activation rows itself
 * while its weight loads are in flight, which saves the quantizer's launch.
 * Other sizes (where repeating the quantization in every workgroup costs more
 * than the launch) run quantize_q8_0 and qgemm_q8_0 back to back on `stream`.
 * n == 0 only quantizes.  Requirements: those of quantize_q8_0 and
 * qgemm_q8_0.
 */
BQI_API int quantize_qgemm_q8_0(const void *x, int x_dtype, int64_t m, int64_t k,
                        int64_t ldx, const int8_t *wq, const uint16_t *wd,
                        int64_t n, float *y, int8_t *q, uint16_t *d,
                        void *stream);

/*
 * route_topk -- group routed rows by expert (the routing step of the grouped
 * 4-bit GEMM for MoE routing, "2011 GPU", Method 1).
 *
 *   topk_ids [n_tokens][top_k] int32 expert ids; routed row r = t*top_k + j.
 *   counts   [n_experts] int32 (output): rows routed to each expert.
 *   offsets  [n_experts + 1] int32 (output): exclusive prefix sum of counts.
 *   rows     [n_tokens*top_k] int32 (output): rows[offsets[e] .. offsets[e+1])
 *            are the r with topk_ids[r] == e, in increasing r.  Entries past
 *            offsets[n_experts] are left unwritten.
 *
 * Ids outside [0, n_experts) are skipped.  Deterministic (no atomics).
 * Requirements: n_tokens * top_k <= 2^30, n_experts <= 65536.
 */
BQI_API int route_topk(const int32_t *topk_ids, int64_t n_tokens, int64_t top_k,
               int64_t n_experts, int32_t *counts, int32_t *offsets,
               int32_t *rows, void *stream);

/* Bytes of device workspace qgemm_w4a8_grouped needs for these sizes (0 for
 * sizes it rejects).  The workspace holds the routing: counts, offsets and
 * the routed rows of each expert, about 4 * (n_tokens * top_k + 2 * n_experts)
 * bytes.  k is only validated (it must be a nonnegative multiple of 32): the
 * size no longer depends on it. */
BQI_API size_t qgemm_w4a8_grouped_workspace_size(int64_t n_tokens, int64_t top_k,
                                         int64_t n_experts, int64_t k);

/*
 * qgemm_w4a8_grouped -- expert-routed 4-bit-weight x Q8_0-activation GEMM
 * (the grouped 4-bit GEMM for MoE routing of "2011 GPU", Method 1, with the
 * W4A8 format of its Method 2).
 *
 *   aq [n_tokens][k] int8, ad [n_tokens][k/32] fp16 bits  -- Q8_0 activations
 *   topk_ids [n_tokens][top_k] int32                       -- expert per slot
 *   wq4 [n_experts][n][k/2] packed 4-bit codes, wd [n_experts][n][k/32] fp16
 *   y  [n_tokens][top_k][n] fp32 (output), token-major in slot order
 *   workspace: device memory of at least
 *              qgemm_w4a8_grouped_workspace_size(...) bytes, 256-byte aligned;
 *              its contents on entry do not matter and are overwritten.
 *
 * Up to 128 routed rows (n_tokens * top_k, the decode case) run a v_dot4
 * GEMV per routed row with no routing pass (the workspace is then unused);
 * larger problems route, then run the int8-MFMA kernel.  Both compute the
 * same function within the same bound.
 *
 * For routed row r = t*top_k + j with e = topk_ids[t][j]:
 *   y[t][j][c] = sum_b wd[e][c][b] * ad[t][b] * sum_{u<32} (code[e][c][32b+u] - 8) * aq[t][32b+u]
 * with the same per-term rounding and accumulation bound as qgemm_q8_0.
 * Rows whose id is outside [0, n_experts) are written as 0.0f; duplicate ids
 * within a token are legal and computed independently.
 *
 * Requirements: k % 32 == 0; aq and wq4 16-byte aligned; workspace 256-byte
 * aligned; n_tokens * top_k <= 2^30; n_experts <= 65536; n * k/2 and
 * n_tokens * k below 2^31 (one expert's packed weights and the activations
 * are addressed with 32-bit offsets).
 */
BQI_API int qgemm_w4a8_grouped(const int8_t *aq, const uint16_t *ad, int64_t n_tokens,
                       const int32_t *topk_ids, int64_t top_k,
                       const uint8_t *wq4, const uint16_t *wd,
                       int64_t n_experts, int64_t n, int64_t k, float *y,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Size of the device array that qgemm_w4a8_grouped_noalloc uses as its
 * workspace: 16 MiB per GPU the library runs on. */
#define BQI_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * qgemm_w4a8_grouped_noalloc -- qgemm_w4a8_grouped for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (without the workspace),
 * same kernels, same results.
 *
 * The workspace is a device array inside the library, BQI_NOALLOC_SCRATCH_BYTES
 * per GPU, created when the library is first used on that GPU and held until
 * the process ends; this call allocates nothing.  The caller still passes the
 * inputs and y.  Problems whose workspace
 * (qgemm_w4a8_grouped_workspace_size) exceeds the array return BQI_ESHAPE
 * before anything is launched (it holds about 4.19 million routed rows).  The array belongs to the current device: `stream` must be a stream
 * of that device.  Calls that overlap on one GPU (several host threads, or
 * several streams) share the array and race; serialize them.  Up to 128
 * routed rows need no workspace and never touch the array.
 */
BQI_API int qgemm_w4a8_grouped_noalloc(const int8_t *aq, const uint16_t *ad,
                               int64_t n_tokens, const int32_t *topk_ids,
                               int64_t top_k, const uint8_t *wq4,
                               const uint16_t *wd, int64_t n_experts,
                               int64_t n, int64_t k, float *y, void *stream);

/*
 * moe_combine_f32 -- the MoE combine after the grouped GEMM: each token's
 * top-k expert outputs weighted by its router probabilities and summed back
 * in token order ("2011 GPU": the grouped 4-bit GEMM serves the MoE routing,
 * Method 1; the experts are router-weighted, Method 2).
 *
 *   y   [n_tokens][top_k][n] fp32  -- e.g. the output of qgemm_w4a8_grouped
 *   p   [n_tokens][top_k] fp32     -- router probabilities of the slots
 *   out [n_tokens][n] fp32 (output) = sum_{j < top_k} p[t][j] * y[t][j][c]
 *
 * Slots are accumulated in order with one fma each (one rounding per
 * product-and-add): |out - exact| <= top_k * 2^-24 * sum_j |p y|;
 * deterministic.  top_k == 0 writes zeros.  Requirements: y, p, out 4-byte
 * aligned (16-byte alignment and n % 4 == 0 select wider loads).
 */
BQI_API int moe_combine_f32(const float *y, const float *p, int64_t n_tokens,
                    int64_t top_k, int64_t n, float *out, void *stream);

/*
 * gguf_q8_0_to_planar, gguf_q4_0_to_planar -- split a GGUF block array into
 * this library's planar layout, so that weights stored as GGUF (the format of
 * "mining card", Honest benchmark) can be consumed.
 *
 *   blocks: rows * k/32 contiguous blocks, row-major; each block is a
 *           little-endian fp16 scale followed by its codes:
 *           Q8_0: 32 int8 codes (34 bytes);
 *           Q4_0: 16 bytes, byte j = element j (low nibble) | element j+16
 *                 (high nibble), value (nibble - 8) * scale (18 bytes).
 *   q / wq4 (output): codes [rows][k] int8 (Q8_0) or packed [rows][k/2]
 *           uint8 (Q4_0, same nibble order: the wq4 layout of
 *           qgemm_w4a8_grouped);
 *   d / wd  (output): scale bits [rows][k/32].
 *
 * A byte shuffle; the output is exactly the blocks' fields.  Requirements:
 * k % 32 == 0; blocks and codes 16-byte aligned; scales 2-byte aligned.
 */
BQI_API int gguf_q8_0_to_planar(const void *blocks, int64_t rows, int64_t k,
                        int8_t *q, uint16_t *d, void *stream);
BQI_API int gguf_q4_0_to_planar(const void *blocks, int64_t rows, int64_t k,
                        uint8_t *wq4, uint16_t *wd, void *stream);

/*
 * qgemm_w4a8_grouped_host -- the grouped W4A8 GEMM on the host CPU, with
 * integer SIMD ("2011 GPU": the CPU decode path with a hand-written W4A8 kernel on
 * pmaddubsw, Method 1 and Contributions; here AVX2 vpmaddubsw).
 *
 * HOST pointers, same layouts and the same function as qgemm_w4a8_grouped
 * (ids outside [0, n_experts) give zero rows), within the same bound.  Runs
 * synchronously on `nthreads` threads (<= 0: all hardware threads); the
 * result does not depend on the thread count.  The calling thread takes a
 * share itself; the others are worker threads that the library starts on
 * first use and keeps for the rest of the process (calls from several host
 * threads at once take turns).  This is a separate entry point for data in
 * host memory, never a substitute for the GPU path.  Returns BQI_ENOTSUP on
 * a CPU without AVX2 and FMA.
 */
BQI_API int qgemm_w4a8_grouped_host(const int8_t *aq, const uint16_t *ad,
                            int64_t n_tokens, const int32_t *topk_ids,
                            int64_t top_k, const uint8_t *wq4,
                            const uint16_t *wd, int64_t n_experts, int64_t n,
                            int64_t k, float *y, int nthreads);

#ifdef __cplusplus
}
#endif
#endif /* BQI_H */
