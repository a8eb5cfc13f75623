// gemv_thin.hip -- thin-M Q8_0 x Q8_0 GEMM (m <= 16): the decode GEMV that
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU" names,
// under Results, as the structural ("thin-M GEMM") decode bottleneck; the
// integer dot product is the pages' DP4A step ("I wrote a custom CUDA
// inference engine...", Features; axbrief.com, "DP4A kernels and 3-bit KV
// cache"), here v_dot4_i32_i8 on gfx950.
//
// The weights are streamed from HBM exactly once.  A group of LPR lanes (LPR =
// 64 when k >= 4096) shares one weight row; each lane owns two consecutive
// 32-element blocks (64 bytes = four 16-byte loads) per pass, so one wave-wide
// load instruction covers 1 KB of a row and a row of 4 KB takes four.  Every
// wave keeps R rows in flight.  The m <= 16 activation rows of the current
// K chunk sit in LDS and are read once per R weight rows.
//
// Per (row, block) the lane forms P = sum of 32 int8 products exactly (eight
// dot4 ops), then acc = fma((float)P, da * dw, acc): the scale product of two
// fp16 values is exact in fp32, so each term is rounded once, inside the fma.
// Lanes reduce their fp32 partials with a fixed butterfly, so results are
// deterministic.
#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

namespace {

template <int MT>
struct ThinCfg {
  static constexpr int KC = (MT <= 8) ? 4096 : 2048;  // K elements per LDS chunk
  static constexpr int R = (MT <= 4) ? 4 : 2;         // weight rows per lane
};

template <int MT>
__global__ __launch_bounds__(256) void k_gemv_thin(
    const int8_t *__restrict__ aq, const uint16_t *__restrict__ ad, int m,
    const int8_t *__restrict__ wq, const uint16_t *__restrict__ wd, int n,
    int k, float *__restrict__ y, int lpr_log2) {
  constexpr int KC = ThinCfg<MT>::KC;
  constexpr int R = ThinCfg<MT>::R;
  __shared__ __attribute__((aligned(16))) int8_t sA[MT * KC];
  __shared__ uint16_t sAd[MT * (KC / QK)];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr = 1 << lpr_log2;
  const int sub = lane & (lpr - 1);   // lane within its row group
  const int rw = 64 >> lpr_log2;      // rows per wave pass
  const int nbk = k / QK;             // blocks per full row
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * (R * rw) + (lane >> lpr_log2);

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[r][i] = 0.0f;

  for (int c0 = 0; c0 < k; c0 += KC) {
    const int kc = min(KC, k - c0);
    const int nbc = kc / QK;
    // stage activations of this chunk: m rows x kc codes, 16 B per thread step
    __syncthreads();
    {
      const int per_row16 = kc / 16;
      for (int idx = threadIdx.x; idx < m * per_row16; idx += 256) {
        const int i = idx / per_row16, c = idx - i * per_row16;
        *reinterpret_cast<i32x4 *>(sA + i * KC + c * 16) =
            *reinterpret_cast<const i32x4 *>(aq + (int64_t)i * k + c0 + c * 16);
      }
      for (int idx = threadIdx.x; idx < m * nbc; idx += 256) {
        const int i = idx / nbc, b = idx - i * nbc;
        sAd[i * (KC / QK) + b] = ad[(int64_t)i * nbk + c0 / QK + b];
      }
    }
    __syncthreads();

    for (int b = 2 * sub; b < nbc; b += 2 * lpr) {
      const bool two = b + 1 < nbc;
      // weight rows: issue all loads first
      i32x4 w[R][4];
      float dw0[R], dw1[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + (int64_t)r * rw;
        const bool ok = row < n;
        const int8_t *src = wq + (ok ? row : 0) * (int64_t)k + c0 + b * QK;
        const i32x4 *s4 = reinterpret_cast<const i32x4 *>(src);
        // the second block's address stays inside the row even when absent
        const i32x4 *s4b = two ? s4 + 2 : s4;
        w[r][0] = ok ? __builtin_nontemporal_load(s4 + 0) : i32x4{0, 0, 0, 0};
        w[r][1] = ok ? __builtin_nontemporal_load(s4 + 1) : i32x4{0, 0, 0, 0};
        w[r][2] = (ok && two) ? __builtin_nontemporal_load(s4b + 0) : i32x4{0, 0, 0, 0};
        w[r][3] = (ok && two) ? __builtin_nontemporal_load(s4b + 1) : i32x4{0, 0, 0, 0};
        const uint16_t *ws = wd + (ok ? row : 0) * (int64_t)nbk + c0 / QK + b;
        dw0[r] = ok ? half_bits_to_float(ws[0]) : 0.0f;
        dw1[r] = (ok && two) ? half_bits_to_float(ws[two ? 1 : 0]) : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i < m) {
          const i32x4 *a4 = reinterpret_cast<const i32x4 *>(sA + i * KC + b * QK);
          const i32x4 a0 = a4[0], a1 = a4[1];
          const i32x4 *a4b = two ? a4 + 2 : a4;
          const i32x4 a2 = two ? a4b[0] : i32x4{0, 0, 0, 0};
          const i32x4 a3 = two ? a4b[1] : i32x4{0, 0, 0, 0};
          const float da0 = half_bits_to_float(sAd[i * (KC / QK) + b]);
          const float da1 = two ? half_bits_to_float(sAd[i * (KC / QK) + b + 1]) : 0.0f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            int32_t p0 = 0, p1 = 0;
            p0 = dot4_i8(a0.x, w[r][0].x, p0);
            p0 = dot4_i8(a0.y, w[r][0].y, p0);
            p0 = dot4_i8(a0.z, w[r][0].z, p0);
            p0 = dot4_i8(a0.w, w[r][0].w, p0);
            p0 = dot4_i8(a1.x, w[r][1].x, p0);
            p0 = dot4_i8(a1.y, w[r][1].y, p0);
            p0 = dot4_i8(a1.z, w[r][1].z, p0);
            p0 = dot4_i8(a1.w, w[r][1].w, p0);
            p1 = dot4_i8(a2.x, w[r][2].x, p1);
            p1 = dot4_i8(a2.y, w[r][2].y, p1);
            p1 = dot4_i8(a2.z, w[r][2].z, p1);
            p1 = dot4_i8(a2.w, w[r][2].w, p1);
            p1 = dot4_i8(a3.x, w[r][3].x, p1);
            p1 = dot4_i8(a3.y, w[r][3].y, p1);
            p1 = dot4_i8(a3.z, w[r][3].z, p1);
            p1 = dot4_i8(a3.w, w[r][3].w, p1);
            // each scale product da*dw is exact in fp32 (11 + 11 bits)
            acc[r][i] = fmaf((float)p0, da0 * dw0[r], acc[r][i]);
            acc[r][i] = fmaf((float)p1, da1 * dw1[r], acc[r][i]);
          }
        }
      }
    }
  }

  // fixed-order butterfly over the lpr lanes of each row group
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float v = acc[r][i];
      for (int off = lpr >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off);
      acc[r][i] = v;
    }
  if (sub == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + (int64_t)r * rw;
      if (row < n) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
          if (i < m) y[(int64_t)i * n + row] = acc[r][i];
      }
    }
  }
}

template <int MT>
hipError_t launch_mt(const int8_t *aq, const uint16_t *ad, int64_t m,
                     const int8_t *wq, const uint16_t *wd, int64_t n, int64_t k,
                     float *y, hipStream_t stream) {
  // lanes per row: enough lanes that each owns one pair of blocks per pass,
  // at most the whole wave
  const int64_t pairs = (k / QK + 1) / 2;
  int lpr_log2 = 0;
  while ((1 << lpr_log2) < pairs && lpr_log2 < 6) ++lpr_log2;
  const int64_t rows_per_wg = 4 * (int64_t)ThinCfg<MT>::R * (64 >> lpr_log2);
  const int64_t wgs = (n + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((k_gemv_thin<MT>), dim3((unsigned)wgs), dim3(256), 0,
                     stream, aq, ad, (int)m, wq, wd, (int)n, (int)k, y,
                     lpr_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_thin(const int8_t *aq, const uint16_t *ad, int64_t m,
                            const int8_t *wq, const uint16_t *wd, int64_t n,
                            int64_t k, float *y, hipStream_t stream) {
  if (m <= 1) return launch_mt<1>(aq, ad, m, wq, wd, n, k, y, stream);
  if (m <= 2) return launch_mt<2>(aq, ad, m, wq, wd, n, k, y, stream);
  if (m <= 4) return launch_mt<4>(aq, ad, m, wq, wd, n, k, y, stream);
  if (m <= 8) return launch_mt<8>(aq, ad, m, wq, wd, n, k, y, stream);
  return launch_mt<16>(aq, ad, m, wq, wd, n, k, y, stream);
}

}  // namespace bqi
