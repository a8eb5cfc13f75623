// moe_combine.hip -- the MoE combine that follows the grouped W4A8 GEMM: each
// token's top-k expert outputs, weighted by its router probabilities, summed
// back in token order.  "A 35B Hybrid-Attention Mixture-of-Experts Model on a
// 6GB 2011 GPU" (gist.science summary): the grouped 4-bit GEMM serves the MoE
// routing (Method 1) and the experts are router-weighted (Method 2).
//
//   out[t][c] = sum_{j < top_k} p[t][j] * y[t][j][c]
//
// An HBM stream: every y element is read once and every output written once.
// A thread owns 4 consecutive columns of one token (16-byte loads when the
// rows allow it) and accumulates the slots in order with one fma each, so
// every product-and-add is rounded once: |out - exact| <=
// top_k * 2^-24 * sum_j |p y|, and the result is deterministic.
#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

namespace {

constexpr int CT = 256;

template <bool VEC>
__global__ __launch_bounds__(CT) void k_moe_combine(const float *__restrict__ y,
                                                    const float *__restrict__ p,
                                                    int64_t T, int top_k, int64_t n,
                                                    float *__restrict__ out) {
  const int64_t cols4 = (n + 3) / 4;
  const int64_t total = T * cols4;
  for (int64_t idx = (int64_t)blockIdx.x * CT + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * CT) {
    const int64_t t = idx / cols4;
    const int64_t c = 4 * (idx - t * cols4);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const float *yt = y + t * top_k * n;
    for (int j = 0; j < top_k; ++j) {
      const float pj = p[t * top_k + j];
      if constexpr (VEC) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(yt + j * n + c));
        acc[0] = fmaf(pj, v.x, acc[0]);
        acc[1] = fmaf(pj, v.y, acc[1]);
        acc[2] = fmaf(pj, v.z, acc[2]);
        acc[3] = fmaf(pj, v.w, acc[3]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (c + u < n) acc[u] = fmaf(pj, yt[j * n + c + u], acc[u]);
      }
    }
    if constexpr (VEC) {
      *reinterpret_cast<f32x4 *>(out + t * n + c) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c + u < n) out[t * n + c + u] = acc[u];
    }
  }
}

}  // namespace

hipError_t launch_moe_combine(const float *y, const float *p, int64_t T,
                              int64_t top_k, int64_t n, float *out,
                              hipStream_t stream) {
  const int64_t work = T * ((n + 3) / 4);
  int64_t wgs = (work + CT - 1) / CT;
  if (wgs > 8192) wgs = 8192;
  const bool vec = n % 4 == 0 && ((uintptr_t)y & 15) == 0 && ((uintptr_t)out & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(k_moe_combine<true>, dim3((unsigned)wgs), dim3(CT), 0, stream,
                       y, p, T, (int)top_k, n, out);
  else
    hipLaunchKernelGGL(k_moe_combine<false>, dim3((unsigned)wgs), dim3(CT), 0, stream,
                       y, p, T, (int)top_k, n, out);
  return hipGetLastError();
}

}  // namespace bqi
