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
// rows allow it), issues the loads of all its slots at once (top_k <= 8) and
// accumulates the slots in order with one fma each, so every product-and-add
// is rounded once: |out - exact| <=
// top_k * 2^-24 * sum_j |p y|, and the result is deterministic.
#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

namespace {

constexpr int CT = 256;
constexpr int TK_UNROLL = 8;  // top_k up to this: all slot loads issued at once

// Idx: 32-bit when every index and offset fits, else 64-bit.  TK > 0: top_k
// <= TK, every load (probabilities and y slots) issued before the first fma;
// TK == 0: any top_k, one slot at a time.
template <bool VEC, int TK, typename Idx>
__global__ __launch_bounds__(CT) void k_moe_combine(const float *__restrict__ y,
                                                    const float *__restrict__ p,
                                                    Idx T, int top_k, Idx n,
                                                    float *__restrict__ out) {
  const Idx cols4 = (n + 3) / 4;
  const Idx total = T * cols4;
  for (Idx idx = (Idx)blockIdx.x * CT + threadIdx.x; idx < total;
       idx += (Idx)gridDim.x * CT) {
    const Idx t = idx / cols4;
    const Idx c = 4 * (idx - t * cols4);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const float *yt = y + (int64_t)t * top_k * n;
    const float *pt = p + (int64_t)t * top_k;
    if constexpr (TK > 0) {
      // slots past top_k re-read slot 0 and are skipped below (their product
      // is never formed, so no inf * 0 can enter the sum)
      float pj[TK];
      f32x4 v[TK];
      // a full row of TK probabilities, 16-byte aligned: TK / 4 loads
      const bool p4 = TK % 4 == 0 && top_k == TK && ((uintptr_t)pt & 15) == 0;
      if (p4) {
#pragma unroll
        for (int j = 0; j < TK; j += 4) {
          const f32x4 q = *reinterpret_cast<const f32x4 *>(pt + j);
          pj[j] = q.x; pj[j + 1] = q.y; pj[j + 2] = q.z; pj[j + 3] = q.w;
        }
      }
#pragma unroll
      for (int j = 0; j < TK; ++j) {
        const int jj = j < top_k ? j : 0;
        if (!p4) pj[j] = pt[jj];
        if constexpr (VEC) {
          v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(yt + (int64_t)jj * n + c));
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[j][u] = yt[(int64_t)jj * n + (c + u < n ? c + u : c)];
        }
      }
#pragma unroll
      for (int j = 0; j < TK; ++j) {
        if (j < top_k) {  // uniform
          acc[0] = fmaf(pj[j], v[j].x, acc[0]);
          acc[1] = fmaf(pj[j], v[j].y, acc[1]);
          acc[2] = fmaf(pj[j], v[j].z, acc[2]);
          acc[3] = fmaf(pj[j], v[j].w, acc[3]);
        }
      }
    } else {
      for (int j = 0; j < top_k; ++j) {
        const float pj = pt[j];
        if constexpr (VEC) {
          const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(yt + (int64_t)j * n + c));
          acc[0] = fmaf(pj, v.x, acc[0]);
          acc[1] = fmaf(pj, v.y, acc[1]);
          acc[2] = fmaf(pj, v.z, acc[2]);
          acc[3] = fmaf(pj, v.w, acc[3]);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (c + u < n) acc[u] = fmaf(pj, yt[(int64_t)j * n + c + u], acc[u]);
        }
      }
    }
    float *ot = out + (int64_t)t * n;
    if constexpr (VEC) {
      *reinterpret_cast<f32x4 *>(ot + c) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c + u < n) ot[c + u] = acc[u];
    }
  }
}

template <int TK, typename Idx>
void launch_combine_kernel(bool vec, unsigned wgs, const float *y, const float *p, int64_t T,
                           int64_t top_k, int64_t n, float *out, hipStream_t stream) {
  if (vec)
    hipLaunchKernelGGL((k_moe_combine<true, TK, Idx>), dim3(wgs), dim3(CT), 0, stream,
                       y, p, (Idx)T, (int)top_k, (Idx)n, out);
  else
    hipLaunchKernelGGL((k_moe_combine<false, TK, Idx>), dim3(wgs), dim3(CT), 0, stream,
                       y, p, (Idx)T, (int)top_k, (Idx)n, out);
}

}  // namespace

hipError_t launch_moe_combine(const float *y, const float *p, int64_t T,
                              int64_t top_k, int64_t n, float *out,
                              hipStream_t stream) {
  const int64_t work = T * ((n + 3) / 4);
  int64_t wgs = (work + CT - 1) / CT;
  if (wgs > 8192) wgs = 8192;
  const bool vec = n % 4 == 0 && ((uintptr_t)y & 15) == 0 && ((uintptr_t)out & 15) == 0;
  // 32-bit indices while the grid-stride index (work + one grid) fits
  const bool small = work + wgs * CT < ((int64_t)1 << 31) && n < ((int64_t)1 << 31);
  const unsigned g = (unsigned)wgs;
  if (top_k <= TK_UNROLL) {
    if (small) launch_combine_kernel<TK_UNROLL, uint32_t>(vec, g, y, p, T, top_k, n, out, stream);
    else launch_combine_kernel<TK_UNROLL, int64_t>(vec, g, y, p, T, top_k, n, out, stream);
  } else {
    if (small) launch_combine_kernel<0, uint32_t>(vec, g, y, p, T, top_k, n, out, stream);
    else launch_combine_kernel<0, int64_t>(vec, g, y, p, T, top_k, n, out, stream);
  }
  return hipGetLastError();
}

}  // namespace bqi
