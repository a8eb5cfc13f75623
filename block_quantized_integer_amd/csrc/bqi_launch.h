// bqi_launch.h -- host-side launchers of the gfx950 kernels (internal to
// libbqi; the public C ABI is include/bqi.h).  Each launcher assumes its
// arguments were already validated by the ABI layer and returns the HIP
// error state after enqueueing its kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bqi {

// Raises a kernel's dynamic-LDS limit (64 KB by default) to `bytes`, once per
// device: `done` is the calling launcher's own table, indexed by device.
// Concurrent first calls may both set the attribute, which is harmless.
inline hipError_t raise_dynamic_lds(const void *kernel, int bytes, bool (&done)[64]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < 64;
  if (cached && done[dev]) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && cached) done[dev] = true;
  return e;
}

hipError_t launch_quantize_q8_0(const void *x, bool f16, int64_t rows,
                                int64_t k, int64_t ldx, int8_t *q, uint16_t *d,
                                hipStream_t stream);

hipError_t launch_zero_f32(float *y, int64_t count, hipStream_t stream);

// thin-M Q8_0 GEMM/GEMV: m <= 16, or more rows in chunks of 16 where
// gemv_thin_chunks_ok (the MFMA thin-M kernel)
bool gemv_thin_chunks_ok(int64_t m, int64_t n, int64_t k, const uint16_t *wd);
hipError_t launch_gemv_thin(const int8_t *aq, const uint16_t *ad, int64_t m,
                            const int8_t *wq, const uint16_t *wd, int64_t n,
                            int64_t k, float *y, hipStream_t stream);

// fused quantize + thin-M GEMM (one launch, bit-identical to the quantizer
// and launch_gemv_thin) for the sizes it covers
bool gemv_fused_supported(int64_t m, int64_t n, int64_t k, const uint16_t *wd);
hipError_t launch_gemv_fused(const void *x, bool f16, int64_t ldx, int64_t m,
                             const int8_t *wq, const uint16_t *wd, int64_t n,
                             int64_t k, float *y, int8_t *q_out,
                             uint16_t *d_out, hipStream_t stream);

// large-M Q8_0 GEMM on int8 MFMA
hipError_t launch_gemm_mfma(const int8_t *aq, const uint16_t *ad, int64_t m,
                            const int8_t *wq, const uint16_t *wd, int64_t n,
                            int64_t k, float *y, hipStream_t stream);

// routing (counting sort by expert); y != nullptr also zeroes the output
// rows of invalid ids ([rows_total][n] floats)
hipError_t launch_route_topk(const int32_t *ids, int64_t rows_total,
                             int64_t n_experts, int64_t top_k, int32_t *counts,
                             int32_t *offsets, int32_t *rows, float *y, int64_t n,
                             hipStream_t stream);

// grouped W4A8 GEMM reading a routing produced by launch_route_topk (ad: the
// fp16 activation scales [n_tokens][k/32]); needs n * k/2 < 2^31
hipError_t launch_grouped_w4a8(const int8_t *aq, const uint16_t *ad,
                               int64_t top_k, const uint8_t *wq4,
                               const uint16_t *wd, int64_t n_experts, int64_t n,
                               int64_t k, int64_t rows_total, const int32_t *counts,
                               const int32_t *offsets, const int32_t *rows, float *y,
                               hipStream_t stream);

// grouped W4A8 for a few routed rows (decode): v_dot4 GEMV per routed row,
// no routing pass
bool grouped_gemv_supported(int64_t rows_total, int64_t k);
hipError_t launch_grouped_gemv(const int8_t *aq, const uint16_t *ad,
                               const int32_t *ids, int64_t rows_total,
                               int64_t top_k, const uint8_t *wq4,
                               const uint16_t *wd, int64_t n_experts, int64_t n,
                               int64_t k, float *y, hipStream_t stream);

// MoE combine: out[t][c] = sum_j p[t][j] * y[t][j][c]
hipError_t launch_moe_combine(const float *y, const float *p, int64_t T,
                              int64_t top_k, int64_t n, float *out,
                              hipStream_t stream);

// GGUF block arrays -> planar codes + scales (n_blocks = rows * k / 32)
hipError_t launch_gguf_q8_0(const void *src, int64_t n_blocks, int8_t *q,
                            uint16_t *d, hipStream_t stream);
hipError_t launch_gguf_q4_0(const void *src, int64_t n_blocks, uint8_t *wq4,
                            uint16_t *wd, hipStream_t stream);

}  // namespace bqi
