// gemv_thin.hip -- thin-M Q8_0 x Q8_0 GEMM (m <= 16): the decode GEMV that
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU" names,
// under Results, as the structural ("thin-M GEMM") decode bottleneck; the
// integer dot product is the pages' DP4A step ("I wrote a custom CUDA
// inference engine...", Features; axbrief.com, "DP4A kernels and 3-bit KV
// cache"), here v_dot4_i32_i8 on gfx950.
//
// The weights are streamed from HBM exactly once, and the kernel is shaped
// like a plain streaming read: every wave-wide load instruction fetches 1 KB
// of one weight row (lane l takes bytes 16l..16l+15 of each 1 KB chunk), all
// of a wave's weight loads are issued before any arithmetic, and nothing
// waits on LDS or a barrier first.
//
// k_gemv_reg (m <= 16, m * k <= 64 K codes, k <= 8 K for m > 1): each wave
// owns two weight rows; the activation rows are staged once per workgroup in
// LDS (dynamic, up to 68 KB) while the weight loads are in flight, and read
// with the weights' lane mapping; each activation row's sums are finished
// before the next row's, which keeps the register count low for m = 16.  A lane
// holds half of a 32-element block per chunk; it forms the half-block dot
// product with four dot4 ops, and one DPP lane swap adds the partner half,
// so every block's int32 P is exact before it is scaled.  Only even lanes
// carry the block's scale (odd lanes scale by zero),
// acc = fma((float)P, da * dw, acc) with the exact fp16 x fp16 product, and
// each half-wave reduces one of the two rows with DPP steps.
//
// k_gemv_mfma16 (4 < m <= 16 with k a multiple of 64 whose stages fit LDS):
// the same streaming loads, turned into int8 MFMA operands in registers; one
// MFMA per block replaces the m rows of dot4 work.  It also takes up to a few
// hundred rows as chunks of 16, one workgroup per (chunk, weight-row slot).
//
// k_gemv_lds (the rest of m <= 16: longer rows): the m activation rows of the
// current K chunk sit in LDS; a group of LPR lanes shares one weight row and each lane
// owns two consecutive blocks (64 bytes) per pass.
//
// Lanes reduce their fp32 partials with a fixed butterfly, so results are
// deterministic.
#include <algorithm>

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
__global__ __launch_bounds__(256) void k_gemv_lds(
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


// ---- m <= 16: coalesced 1 KB loads, two rows per wave ------------------------

constexpr int REG_RPW = 2;             // weight rows per wave
constexpr int REG_ACT_BYTES = 65536;   // m * k bytes of activation codes staged in LDS

// v + (v from lane ^ 1): the DPP quad permutation [1,0,3,2]
__device__ __forceinline__ int32_t add_partner_i32(int32_t v) {
  return v + __builtin_amdgcn_mov_dpp(v, 0xb1, 0xf, 0xf, false);
}

// Sum over the 32 lanes of each half-wave; the result is valid in lanes 0
// and 32.  Fixed order: four DPP steps inside rows of 16 lanes, then one
// cross-row shuffle.
__device__ __forceinline__ float half_wave_sum(float v) {
  v += bits_to_float(__builtin_amdgcn_mov_dpp(__builtin_bit_cast(int32_t, v), 0xb1, 0xf, 0xf, false));  // lane ^ 1
  v += bits_to_float(__builtin_amdgcn_mov_dpp(__builtin_bit_cast(int32_t, v), 0x4e, 0xf, 0xf, false));  // lane ^ 2
  v += bits_to_float(__builtin_amdgcn_mov_dpp(__builtin_bit_cast(int32_t, v), 0x141, 0xf, 0xf, false)); // half-row mirror
  v += bits_to_float(__builtin_amdgcn_mov_dpp(__builtin_bit_cast(int32_t, v), 0x140, 0xf, 0xf, false)); // row mirror
  // + lane ^ 16: the swap leaves each lane's own value in one result and its
  // partner's in the other
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), false, false);
  return bits_to_float((int32_t)r[0]) + bits_to_float((int32_t)r[1]);
}

// Activation source of the register kernel: Q8_0 codes and scales, or fp32 /
// fp16 values that every workgroup quantizes itself (the fused
// quantize-and-multiply decode path).
enum ActSrc { ACT_Q8 = 0, ACT_F32 = 1, ACT_F16 = 2 };

// Threads per workgroup: 4 waves for Q8_0 input of up to 4 rows; 8 waves when
// every workgroup quantizes the activations itself, or stages more than 4
// activation rows, which halves the number of workgroups repeating that work.
constexpr int reg_threads(int src, int mt) { return src == ACT_Q8 && mt <= 4 ? 256 : 512; }

// Dynamic LDS of the register kernel: the staged codes (MT * CH KB plus a
// spare 16-byte slot) and their scales (plus a spare slot).
constexpr int reg_lds_bytes(int mt, int ch) {
  return (mt * ch * 1024 + 16) + ((mt * ch * 32 + 1) * 2 + 14) / 16 * 16;
}

// (no __restrict__ on the inputs: with it the compiler may move the scale
// loads across the memory clobber below, behind the barrier)
template <int MT, int CH, int SRC>
__global__ __launch_bounds__(reg_threads(SRC, MT)) void k_gemv_reg(
    const int8_t *aq, const uint16_t *ad, const void *x, int ldx, int m,
    const int8_t *wq, const uint16_t *wd, int n, int k, float *y,
    int8_t *q_out, uint16_t *d_out) {
  static_assert(MT * CH * 1024 <= REG_ACT_BYTES, "activation stage too small");
  // one spare 16-byte slot (and scale slot) takes the stores of lanes with
  // nothing to stage, so the staging stores stay unconditional
  extern __shared__ __attribute__((aligned(16))) int8_t reg_lds[];
  int8_t *sA = reg_lds;                                                      // [MT*CH*1024 + 16]
  uint16_t *sAd = reinterpret_cast<uint16_t *>(reg_lds + MT * CH * 1024 + 16);  // [MT*CH*32 + 1]
  const int lane = threadIdx.x & 63;
  constexpr int NT = reg_threads(SRC, MT);
  const int row0 = ((int)blockIdx.x * (NT / 64) + (int)(threadIdx.x >> 6)) * REG_RPW;
  const int nbk = k / QK;
  const bool even = (lane & 1) == 0;

  // Load order matters: loads retire in order, so the activations (L2 hits)
  // are requested first, then all weight loads (HBM); staging the
  // activations in LDS then waits only for the former.  Every load is
  // unconditional (lanes past k re-read a valid address) so that none waits
  // on another; values are masked afterwards.
  constexpr int STAGE = MT * CH * 64 / NT;  // 16-byte activation chunks per thread
  static_assert(STAGE >= 1 || MT * CH * 64 < NT, "");
  constexpr int STAGE_N = STAGE > 0 ? STAGE : 1;
  constexpr int SD_N = MT * CH * 32 / NT > 0 ? MT * CH * 32 / NT : 1;
  // fused path: 8 lanes per 32-element block, 4 elements per lane
  // quantize tasks per thread (tasks past the staged blocks are masked)
  constexpr int QT = SRC == ACT_Q8 ? 1 : (MT * CH * 256 + NT - 1) / NT;
  i32x4 st[STAGE_N];
  uint16_t st_d[SD_N];
  float xv[QT][4];
  if constexpr (SRC == ACT_Q8) {
#pragma unroll
    for (int q = 0; q < STAGE_N; ++q) {
      const int c = (int)threadIdx.x + NT * q;
      const int i = c / (CH * 64), cc = c % (CH * 64);
      const bool ok = i < m && cc < k / 16;
      st[q] = *reinterpret_cast<const i32x4 *>(aq + (ok ? (int64_t)i * k + 16 * cc : 0));
    }
#pragma unroll
    for (int q = 0; q < SD_N; ++q) {
      const int c = (int)threadIdx.x + NT * q;
      const int i = c / (CH * 32), b = c % (CH * 32);
      const bool ok = i < m && b < nbk;
      st_d[q] = ad[ok ? (int64_t)i * nbk + b : 0];
    }
  } else {
    // task t = tid + NT u: block t/8 of the staged rows (row i, block b),
    // elements 4*(t%8) .. +3; tasks past m or k re-read element 0
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int t = (int)threadIdx.x + NT * u;
      const int blk = t >> 3, sub = t & 7;
      const int i = blk / (CH * 32), b = blk % (CH * 32);
      const bool ok = i < m && b < nbk;
      const int64_t off = ok ? (int64_t)i * ldx + QK * b + 4 * sub : 0;
      if constexpr (SRC == ACT_F32) {
        const f32x4 r = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(x) + off);
        xv[u][0] = r.x; xv[u][1] = r.y; xv[u][2] = r.z; xv[u][3] = r.w;
      } else {
        const uint2 r = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(x) + off);
        xv[u][0] = half_bits_to_float((uint16_t)(r.x & 0xffffu));
        xv[u][1] = half_bits_to_float((uint16_t)(r.x >> 16));
        xv[u][2] = half_bits_to_float((uint16_t)(r.y & 0xffffu));
        xv[u][3] = half_bits_to_float((uint16_t)(r.y >> 16));
      }
    }
  }
  // every activation load is issued before the first weight load: a later
  // one would make the quantize wait for the whole weight stream
  __asm__ volatile("" ::: "memory");

  i32x4 w[REG_RPW][CH];
  uint16_t dwh[REG_RPW][CH];
#pragma unroll
  for (int r = 0; r < REG_RPW; ++r) {
    const int row = min(row0 + r, n - 1);
    const i32x4 *src = reinterpret_cast<const i32x4 *>(wq + (int64_t)row * k);
    const uint16_t *ws = wd + (int64_t)row * nbk;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const bool ok = 1024 * j + 16 * lane < k;
      w[r][j] = __builtin_nontemporal_load(src + (ok ? 64 * j + lane : 0));
      dwh[r][j] = __builtin_nontemporal_load(ws + (ok ? 32 * j + (lane >> 1) : 0));
    }
  }
  // keep every weight load ahead of the LDS staging and the barrier (the
  // memory clobber stops the compiler from sinking them to their uses)
  __asm__ volatile("" ::: "memory");

  if constexpr (SRC == ACT_Q8) {
#pragma unroll
    for (int q = 0; q < STAGE_N; ++q) {
      const int c = (int)threadIdx.x + NT * q;
      const int i = c / (CH * 64), cc = c % (CH * 64);
      const bool ok = c < MT * CH * 64 && i < m && cc < k / 16;
      *reinterpret_cast<i32x4 *>(sA + (ok ? i * (CH * 1024) + 16 * cc : MT * CH * 1024)) = st[q];
    }
#pragma unroll
    for (int q = 0; q < SD_N; ++q) {
      const int c = (int)threadIdx.x + NT * q;
      const int i = c / (CH * 32), b = c % (CH * 32);
      const bool ok = c < MT * CH * 32 && i < m && b < nbk;
      sAd[ok ? i * (CH * 32) + b : MT * CH * 32] = st_d[q];
    }
  } else {
    // quantize while the weight loads are in flight (same device routine as
    // quantize_q8_0, so the codes are identical); workgroup 0 also writes the
    // Q8_0 activations out
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int t = (int)threadIdx.x + NT * u;
      const int blk = t >> 3, sub = t & 7;
      const int i = blk / (CH * 32), b = blk % (CH * 32);
      const bool ok = i < m && b < nbk;
      uint16_t dbits;
      const uint32_t packed = q8_0_quantize4(xv[u], dbits);
      *reinterpret_cast<uint32_t *>(sA + (ok ? i * (CH * 1024) + QK * b + 4 * sub : MT * CH * 1024)) = packed;
      if (sub == 0) sAd[ok ? i * (CH * 32) + b : MT * CH * 32] = dbits;
      if (ok && blockIdx.x == 0) {
        *reinterpret_cast<uint32_t *>(q_out + (int64_t)i * k + QK * b + 4 * sub) = packed;
        if (sub == 0) d_out[(int64_t)i * nbk + b] = dbits;
      }
    }
  }
  __syncthreads();

  float acc[REG_RPW][MT];
#pragma unroll
  for (int r = 0; r < REG_RPW; ++r)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[r][i] = 0.0f;

  // rows i >= m compute on whatever the stage holds and are never stored;
  // keeping the loop unconditional keeps the weight loads where they are
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    {
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const bool ok = 1024 * j + 16 * lane < k;
        // lanes past k read chunk 0 and scale by zero
        const i32x4 a = *reinterpret_cast<const i32x4 *>(sA + i * (CH * 1024) + (ok ? 1024 * j + 16 * lane : 0));
        const float das = half_bits_to_float(sAd[i * (CH * 32) + (ok ? 32 * j + (lane >> 1) : 0)]);
        // odd lanes hold the second half of a block: they scale by zero so
        // that each block is counted once
        const float da = (ok && even) ? das : 0.0f;
#pragma unroll
        for (int r = 0; r < REG_RPW; ++r) {
          int32_t ph = 0;
          ph = dot4_i8(a.x, w[r][j].x, ph);
          ph = dot4_i8(a.y, w[r][j].y, ph);
          ph = dot4_i8(a.z, w[r][j].z, ph);
          ph = dot4_i8(a.w, w[r][j].w, ph);
          // the partner lane (l ^ 1) holds the other half of the same block
          const int32_t p = add_partner_i32(ph);
          const float dw = ok ? half_bits_to_float(dwh[r][j]) : 0.0f;
          acc[r][i] = fmaf((float)p, da * dw, acc[r][i]);
        }
      }
    }
    // finish this row's sums here: otherwise the compiler sinks them into the
    // `i < m` store branches at the end and keeps every block's int32 dot
    // product of every row live until then
#pragma unroll
    for (int r = 0; r < REG_RPW; ++r) __asm__ volatile("" : "+v"(acc[r][i]));
  }

  // lanes 0..31 finish row 0, lanes 32..63 row 1
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    if (i < m) {
      // lane l < 32: acc0[l] + acc0[l + 32]; lane l >= 32: acc1[l - 32] + acc1[l]
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, acc[0][i]),
                                                       __builtin_bit_cast(uint32_t, acc[1][i]), false, false);
      const float v = half_wave_sum(bits_to_float((int32_t)sw[0]) + bits_to_float((int32_t)sw[1]));
      const int row = row0 + (lane >> 5);
      if ((lane & 31) == 0 && row < n) y[(int64_t)i * n + row] = v;
    }
  }
}

template <int MT, int CH, int SRC>
hipError_t launch_reg(const int8_t *aq, const uint16_t *ad, const void *x, int64_t ldx,
                      int64_t m, const int8_t *wq, const uint16_t *wd, int64_t n, int64_t k,
                      float *y, int8_t *q_out, uint16_t *d_out, hipStream_t stream) {
  constexpr int NT = reg_threads(SRC, MT);
  constexpr int LDS = reg_lds_bytes(MT, CH);
  if constexpr (LDS > 65536) {
    // above the default dynamic-LDS limit: raise it for this kernel
    static bool raised[64];
    const hipError_t e = raise_dynamic_lds((const void *)k_gemv_reg<MT, CH, SRC>, LDS, raised);
    if (e != hipSuccess) return e;
  }
  const int64_t rows_per_wg = (NT / 64) * REG_RPW;
  const int64_t wgs = (n + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((k_gemv_reg<MT, CH, SRC>), dim3((unsigned)wgs), dim3(NT), LDS,
                     stream, aq, ad, x, (int)ldx, (int)m, wq, wd, (int)n, (int)k, y,
                     q_out, d_out);
  return hipGetLastError();
}

// The register kernel covers MT * CH <= 64 (MT activation rows of CH KB of
// codes staged in LDS) with CH <= 8 weight chunks per lane (16 for a single
// row: more would leave no registers for anything else); the fused
// activation sources only MT * CH <= 16.
constexpr bool reg_fits(int mt, int ch, int src) {
  return ch <= (mt == 1 ? 16 : 8) && mt * ch <= (src == ACT_Q8 ? 64 : 16);
}

template <int MT, int SRC>
hipError_t launch_reg_ch(const int8_t *aq, const uint16_t *ad, const void *x, int64_t ldx,
                         int64_t m, const int8_t *wq, const uint16_t *wd, int64_t n,
                         int64_t k, float *y, int8_t *q_out, uint16_t *d_out,
                         hipStream_t stream) {
  const int64_t ch = (k + 1023) / 1024;
  if (ch <= 1) return launch_reg<MT, 1, SRC>(aq, ad, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream);
  if (ch <= 2) return launch_reg<MT, 2, SRC>(aq, ad, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream);
  if (ch <= 4) return launch_reg<MT, 4, SRC>(aq, ad, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream);
  if constexpr (reg_fits(MT, 8, SRC)) {
    if (ch <= 8) return launch_reg<MT, 8, SRC>(aq, ad, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream);
  }
  if constexpr (reg_fits(MT, 16, SRC)) {
    if (ch <= 16) return launch_reg<MT, 16, SRC>(aq, ad, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream);
  }
  return hipErrorInvalidValue;  // not reached: the dispatcher checks the size
}

// Smallest power of two >= v (v >= 1).
int64_t pow2_ceil(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
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
  hipLaunchKernelGGL((k_gemv_lds<MT>), dim3((unsigned)wgs), dim3(256), 0,
                     stream, aq, ad, (int)m, wq, wd, (int)n, (int)k, y,
                     lpr_log2);
  return hipGetLastError();
}


// ---- 4 < m <= 16: int8 MFMA on weights transposed in registers --------------
//
// One v_mfma_i32_16x16x32_i8 multiplies 16 activation rows by 16 weight rows
// over exactly one Q8_0 block: lane l supplies 8 codes of row l % 16 (K bytes
// 8 * (l / 16) .. +7 of the block) of each operand and receives the int32 dot
// products of activation rows 4 * (l / 16) + (0..3) with weight row l % 16.
// The accumulator seed and the two-fma scale epilogue are those of the
// large-M GEMM (one rounding per block term).
//
// Loading the weights straight into that fragment layout would make every
// load instruction touch 16 rows 32 bytes at a time, which streams at well
// under half the rate of whole cache lines.  A wave owns 16 weight rows and
// one K part of at most 1 KB (32 blocks, 8 chunks of 128 bytes); load pair p
// fetches chunk p of rows 0..7 and of rows 8..15, lane l = 16 q + 8 h + i
// taking bytes 32 q + 16 h .. +15 of row i (resp. 8 + i), so that every
// instruction reads eight whole 128-byte lines.  The pair is turned into four
// MFMA operands in registers:
//   1. two DPP moves per dword (rotation by 8 inside each 16-lane row, the
//      bank mask limiting each to the lanes that take the other row's half)
//      leave lane l = (row l % 16, q) holding all 32 bytes of block q of
//      the chunk;
//   2. a 4 x 4 transpose of 8-byte pieces between the four 16-lane rows q and
//      the four pieces of a block: v_permlane32_swap exchanges the upper
//      lane rows of pieces 0, 1 with the lower lane rows of pieces 2, 3, then
//      v_permlane16_swap the odd lane rows of pieces 0, 2 with the even lane
//      rows of pieces 1, 3.  Piece register e then holds, in lane row g,
//      bytes 8 g .. 8 g + 7 of block e: the MFMA operand of block 4 p + e.
// A workgroup has g groups of 16 weight rows and splits K over ks waves per
// group; the activation rows and their scales are staged once per workgroup
// in LDS (direct loads, then a barrier that does not wait for the weight
// stream), so each wave multiplies chunk p as soon as its pair has landed
// while the rest streams in.  The K parts are added in a fixed order through
// LDS at the end.  Activation rows past m read row m - 1 and are not stored.
constexpr int MF_WAVES = 12;                          // waves per workgroup at most
constexpr int MF_DEPTH = 3;                           // weight load pairs in flight per wave
constexpr int MF_DSTRIDE = 32 * 4 + 16;               // scale row stride in a wave's slot
constexpr int MF_SLOT = 16 * MF_DSTRIDE;              // LDS bytes per wave (weight scales)
constexpr int64_t MF_LDS_MAX = 160 * 1024;

// Activation stage row stride: whole 1 KB direct-load pieces plus 16 bytes,
// so that a fragment read of 16 rows touches every LDS bank once per half-wave.
constexpr int64_t mf_lda(int64_t k) { return (k + 1023) / 1024 * 1024 + 16; }
// The activation scale stage has 32 spare blocks (zeros) after the last, so
// that the last K part reads whole chunks without a bound check.
constexpr int64_t mf_lds_bytes(int64_t k, int64_t waves) {
  return 16 * mf_lda(k) + (k / QK + 32) * 16 * 4 + waves * MF_SLOT;
}

// 8-byte MFMA operand from two dwords (low dword first in K)
__device__ __forceinline__ long mf_pair(uint32_t lo, uint32_t hi) {
  return (long)(((uint64_t)hi << 32) | lo);
}

// RG groups of 16 weight rows per wave (the activation fragments and scales of
// a block serve RG MFMAs, and each wave's staging serves 16 RG rows); a
// workgroup has up to MF_WAVES waves (RG = 1: several row sets of ks waves;
// RG = 3: one row set, ks waves).

// (no __restrict__ on the inputs: with it the compiler may move loads across
// the compiler barriers that fix their issue order)
//
// SRC = ACT_F32 / ACT_F16 (quantize_qgemm_q8_0 on a few small rows, one K
// part: k <= 1 KB and m * k <= MF_FUSED_ELEMS): instead of loading Q8_0
// codes, the waves of a workgroup (MF_FUSED_GROUPS row groups) quantize the m
// activation rows between them (the quantizer's device routine, so the codes
// are those of quantize_q8_0) into the LDS stage, behind one barrier, and
// workgroup 0 writes the codes and scales out.  Each lane loads its elements
// before the weight stream and quantizes once the weight loads are issued.
constexpr int MF_FUSED_ELEMS = 4096;
constexpr int MF_FUSED_GROUPS = 4;

// CHUNKED: more than 16 rows of Q8_0 codes, taken in chunks (the weights load
// with the default cache policy, since the other chunks read them again;
// one chunk streams them past the caches)
template <int RG, int SRC, bool CHUNKED>
__global__ __launch_bounds__(64 * MF_WAVES) void k_gemv_mfma16(
    const int8_t *aq, const uint16_t *ad, const void *x, int ldx, int m,
    const int8_t *wq, const uint16_t *wd, int n, int k, int ks, float *y,
    int8_t *q_out, uint16_t *d_out, int chunks, int xcd_group) {
  // weight load pairs in flight per wave: MF_DEPTH for RG = 1 (12 waves per
  // CU); two whole chunks (six pairs) for RG = 3, one wave per SIMD
  // (measured: four pairs, which split a chunk, 14.1 us at m = 16; six 11.9;
  // nine 12.1; twelve 12.4)
  constexpr int DEPTH = RG == 1 ? MF_DEPTH : 2 * RG;
  constexpr int NPAIR = 8 * RG;  // pair q = chunk q / RG, row group q % RG
  extern __shared__ __attribute__((aligned(16))) int8_t mf_lds[];
  const int nbk = k / QK;
  const int lda = (int)mf_lda(k);
  // CHUNKED: chunks of 16 rows; each chunk is the m <= 16 computation of its
  // rows.  The chunks that read the same weight rows (one slot) are
  // dispatched side by side.  With xcd_group they also share an XCD (and
  // its L2): workgroups are dealt to the 8 XCDs in turn, so blockIdx b runs
  // on XCD b % 8 and takes chunk (b / 8) % chunks of slot
  // 8 (b / 8 / chunks) + b % 8 (the grid is padded to a multiple of 8 slots;
  // a padding slot's workgroups return at once).  Without it, blockIdx b
  // takes chunk b % chunks of slot b / chunks.
  int wg = (int)blockIdx.x;
  if constexpr (CHUNKED) {
    int chunk;
    if (xcd_group) {  // uniform
      const int idx = wg >> 3;
      chunk = idx % chunks;
      wg = (idx / chunks) * 8 + (wg & 7);
      if ((int64_t)wg * (((int)blockDim.x >> 6) / ks) * 16 * RG >= n) return;
    } else {
      chunk = wg % chunks;
      wg /= chunks;
    }
    aq += (int64_t)chunk * 16 * k;
    ad += (int64_t)chunk * 16 * nbk;
    y += (int64_t)chunk * 16 * n;
    m = min(16, m - 16 * chunk);
  }
  int8_t *sA = mf_lds;                                        // [16][lda], rows < m
  float *sD = reinterpret_cast<float *>(mf_lds + 16 * lda);   // [nbk + 32][16], rows < m
  const int nthreads = (int)blockDim.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nwaves = nthreads >> 6, groups = nwaves / ks;
  // the weight scales of the part as fp32, zero past the part
  int8_t *slotD = mf_lds + 16 * lda + (nbk + 32) * 64 + wave * (RG * MF_SLOT);  // [16 RG][MF_DSTRIDE]
  const int grp = wave / ks, part = wave - grp * ks;
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = (wg * groups + grp) * 16 * RG;
  const int pb0 = 32 * part;              // first block of this K part
  const int pb = min(32, nbk - pb0);      // blocks in it (even: k % 64 == 0)

  // Each wave stages the activation rows and scales of its own K part; the
  // waves of the other groups with the same part write the same bytes to the
  // same places, so no wave waits for another before it multiplies.  Issue
  // order matters (loads retire in order): the activation codes (L2, straight
  // to LDS, invisible to the compiler), their scales, the weight scales, then
  // the weight chunks in the order they are multiplied.
  // fused source: round u of the quantizer, lane l of wave w takes elements
  // 4 (l % 8) .. +3 of block c = 8 (u nwaves + w) + l / 8 of the part's
  // m x pb blocks (row c / pb, block c % pb; past them: element 0, not
  // stored); the launch gives the workgroup MF_FUSED_GROUPS waves, so QR
  // rounds cover m * k <= MF_FUSED_ELEMS
  constexpr int QR = SRC == ACT_Q8 ? 1 : MF_FUSED_ELEMS / 256 / MF_FUSED_GROUPS;
  // c / pb as (c * pb_inv) >> 16: exact for every c < 1024 and pb <= 32
  // (checked exhaustively); c stays below 8 QR MF_FUSED_GROUPS = 128
  static_assert(8 * QR * MF_FUSED_GROUPS <= 1024, "block index range of the reciprocal");
  const uint32_t pb_inv = (65536u + (uint32_t)pb - 1) / (uint32_t)pb;
  float xv[QR][4];
  uint16_t h[8];
  if constexpr (SRC == ACT_Q8) {
    // 1. activation codes: row r, bytes [1024 part + 16 lane, +16) (lanes
    //    past k re-read the row's last 16 bytes, never used)
    const int aoff = min(1024 * part + 16 * lane, k - 16);
    for (int r = 0; r < m; ++r) dma_lds16(aq + (int64_t)r * k + aoff, sA + r * lda + 1024 * part);
    // 2. activation scales of the part: value c = lane + 64 u is row c / 32,
    //    block c % 32 (past m or the part: re-read a valid one, not stored)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = lane + 64 * u, i = c >> 5, b = c & 31;
      h[u] = ad[(int64_t)min(i, m - 1) * nbk + pb0 + min(b, pb - 1)];
    }
  } else {
#pragma unroll
    for (int u = 0; u < QR; ++u) {
      const int c = 8 * (u * nwaves + wave) + (lane >> 3);
      const int i = (int)(((uint32_t)c * pb_inv) >> 16), b = c - i * pb;
      const int64_t off = i < m ? (int64_t)i * ldx + QK * (pb0 + b) + 4 * (lane & 7) : 0;
      if constexpr (SRC == ACT_F32) {
        const f32x4 r = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(x) + off);
        xv[u][0] = r.x; xv[u][1] = r.y; xv[u][2] = r.z; xv[u][3] = r.w;
      } else {
        const uint2 r = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(x) + off);
        xv[u][0] = half_bits_to_float((uint16_t)(r.x & 0xffffu));
        xv[u][1] = half_bits_to_float((uint16_t)(r.x >> 16));
        xv[u][2] = half_bits_to_float((uint16_t)(r.y & 0xffffu));
        xv[u][3] = half_bits_to_float((uint16_t)(r.y >> 16));
      }
    }
  }
  __asm__ volatile("" ::: "memory");
  // 3. weight scales of the part as dwords: instruction (j, i), lane l -> row
  //    16 j + 4 i + l / 16, blocks 2 (l % 16), 2 (l % 16) + 1 (past the part:
  //    its last pair; rows past n: row n - 1)
  uint32_t dw2[RG][4];
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = min(n0 + 16 * j + 4 * i + g, n - 1);
      const int b = pb0 + min(2 * l16, pb - 2);
      dw2[j][i] = *reinterpret_cast<const uint32_t *>(wd + (int64_t)row * nbk + b);
    }
  // 4. the weight chunks (HBM): pair q = (chunk p, group j) is rows
  //    n0 + 16 j + (l & 7) and n0 + 16 j + 8 + (l & 7), bytes 128 p + 16 (l >> 3)
  //    of the part (lanes past k: the row's last 16).  The first DEPTH pairs
  //    now, each later one once the pair DEPTH before it has been multiplied:
  //    a wave that issued all of its chunks at once would see its last one
  //    arrive only at the end of the whole stream (its lines sit at every
  //    depth of every channel's queue), and its multiplications would all
  //    fall after the stream.
  const int woff = QK * pb0 + 16 * (lane >> 3);
  const int8_t *wr[RG][2];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    wr[j][0] = wq + (int64_t)min(n0 + 16 * j + (lane & 7), n - 1) * k;
    wr[j][1] = wq + (int64_t)min(n0 + 16 * j + 8 + (lane & 7), n - 1) * k;
  }
  i32x4 w[NPAIR][2];
  auto load_pair = [&](int q) {
    const int p = q / RG, j = q % RG;
    const int off = min(woff + 128 * p, k - 16);
    if constexpr (CHUNKED) {
      w[q][0] = *reinterpret_cast<const i32x4 *>(wr[j][0] + off);
      w[q][1] = *reinterpret_cast<const i32x4 *>(wr[j][1] + off);
    } else {
      w[q][0] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(wr[j][0] + off));
      w[q][1] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(wr[j][1] + off));
    }
  };
#pragma unroll
  for (int q = 0; q < DEPTH; ++q) load_pair(q);
  __asm__ volatile("" ::: "memory");
  if constexpr (SRC == ACT_Q8) {
    // the loads above are the only ones issued after the scales (2.), so
    // this waits for the scales and the activation codes but not the weights
    wait_vmcnt<4 * RG + 2 * DEPTH>();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = lane + 64 * u, i = c >> 5, b = c & 31;
      // blocks past the part are zeros (the last part reads whole chunks)
      if (i < m) sD[(pb0 + b) * 16 + i] = b < pb ? half_bits_to_float(h[u]) : 0.0f;
    }
  } else {
    const bool out = blockIdx.x == 0;  // (fused sources come in one chunk)
#pragma unroll
    for (int u = 0; u < QR; ++u) {
      const int c = 8 * (u * nwaves + wave) + (lane >> 3), sub = lane & 7;
      const int i = (int)(((uint32_t)c * pb_inv) >> 16), b = c - i * pb;
      uint16_t dbits;
      const uint32_t packed = q8_0_quantize4(xv[u], dbits);  // every lane (DPP inside)
      if (i < m) {
        *reinterpret_cast<uint32_t *>(sA + i * lda + QK * (pb0 + b) + 4 * sub) = packed;
        if (sub == 0) sD[(pb0 + b) * 16 + i] = half_bits_to_float(dbits);
        if (out) {
          *reinterpret_cast<uint32_t *>(q_out + (int64_t)i * k + QK * (pb0 + b) + 4 * sub) = packed;
          if (sub == 0) d_out[(int64_t)i * nbk + pb0 + b] = dbits;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = lane + 64 * u, i = c >> 5, b = c & 31;
      if (i < m && b >= pb) sD[(pb0 + b) * 16 + i] = 0.0f;
    }
    __syncthreads();  // every wave's share of the stage
  }
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in_part = 2 * l16 < pb;
      float2 v;
      v.x = in_part ? half_bits_to_float((uint16_t)(dw2[j][i] & 0xffffu)) : 0.0f;
      v.y = in_part ? half_bits_to_float((uint16_t)(dw2[j][i] >> 16)) : 0.0f;
      *reinterpret_cast<float2 *>(slotD + (16 * j + 4 * i + g) * MF_DSTRIDE + 8 * l16) = v;
    }
  // the LDS operations of one wave complete in program order: the reads
  // below see this wave's stores and direct loads (other waves' stores of
  // the same values may land at any time)
  __asm__ volatile("" ::: "memory");

  const i32x4 seed = {MAGIC_BITS, MAGIC_BITS, MAGIC_BITS, MAGIC_BITS};
  const int8_t *arow = sA + min(l16, m - 1) * lda + QK * pb0 + 8 * g;
  const float *sDrow = sD + pb0 * 16 + 4 * g;
  float acc[RG][4];
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][r] = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if (4 * p < pb) {  // uniform
      long wf[RG][4];
#pragma unroll
      for (int j = 0; j < RG; ++j) {
        const int q = p * RG + j;
        // 1. lane (row l % 16, q'): block q' of chunk p, bytes 0..15 and
        //    16..31.  Lanes 8..15 of a row (DPP banks 2, 3) take bytes 0..15
        //    of their row from the second load of lane l ^ 8; lanes 0..7
        //    (banks 0, 1) take bytes 16..31 from the first load of lane l ^ 8.
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int a = w[q][0][d], b = w[q][1][d];
          lo[d] = (uint32_t)__builtin_amdgcn_update_dpp(a, b, 0x128, 0xf, 0xc, false);
          hi[d] = (uint32_t)__builtin_amdgcn_update_dpp(b, a, 0x128, 0xf, 0x3, false);
        }
        // 2. the 4 x 4 transpose of 8-byte pieces: pieces 0..3 are
        //    (lo0, lo1), (lo2, lo3), (hi0, hi1), (hi2, hi3)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const auto r = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
          lo[d] = r[0];
          hi[d] = r[1];
        }
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto r = __builtin_amdgcn_permlane16_swap(lo[d], lo[d + 2], false, false);
          lo[d] = r[0];
          lo[d + 2] = r[1];
          const auto s = __builtin_amdgcn_permlane16_swap(hi[d], hi[d + 2], false, false);
          hi[d] = s[0];
          hi[d + 2] = s[1];
        }
        wf[j][0] = mf_pair(lo[0], lo[1]);
        wf[j][1] = mf_pair(lo[2], lo[3]);
        wf[j][2] = mf_pair(hi[0], hi[1]);
        wf[j][3] = mf_pair(hi[2], hi[3]);
      }
      // the four blocks' weight scales of row 16 j + l % 16; blocks past the
      // part (its last chunk only) have a zero scale, which adds exactly
      // nothing, and their reads stay inside the stages
      f32x4 dsc[RG];
#pragma unroll
      for (int j = 0; j < RG; ++j)
        dsc[j] = *reinterpret_cast<const f32x4 *>(slotD + (16 * j + l16) * MF_DSTRIDE + 16 * p);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 4 * p + e;  // block within the part
        const long a = *reinterpret_cast<const long *>(arow + QK * b);
        const f32x4 da = *reinterpret_cast<const f32x4 *>(sDrow + b * 16);
#pragma unroll
        for (int j = 0; j < RG; ++j) {
          const i32x4 dd = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, wf[j][e], seed, 0, 0, 0);
          const float dw = dsc[j][e];
          const float ncd = -MAGIC_F * dw;  // exact
          acc[j][0] = fmaf(fmaf(bits_to_float(dd[0]), dw, ncd), da.x, acc[j][0]);
          acc[j][1] = fmaf(fmaf(bits_to_float(dd[1]), dw, ncd), da.y, acc[j][1]);
          acc[j][2] = fmaf(fmaf(bits_to_float(dd[2]), dw, ncd), da.z, acc[j][2]);
          acc[j][3] = fmaf(fmaf(bits_to_float(dd[3]), dw, ncd), da.w, acc[j][3]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const int q = p * RG + j + DEPTH;
      if (q < NPAIR) {
        __asm__ volatile("" ::: "memory");
        load_pair(q);
        __asm__ volatile("" ::: "memory");
      }
    }
  }

  // 5. the K parts of each group, added in order through LDS, then stored
  lds_barrier();  // every wave is done reading the stage
  float *red = reinterpret_cast<float *>(mf_lds);  // [group][part 1..][RG][4][64]
  if (part > 0) {
#pragma unroll
    for (int j = 0; j < RG; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[(((grp * (ks - 1) + part - 1) * RG + j) * 4 + r) * 64 + lane] = acc[j][r];
  }
  lds_barrier();
  if (part > 0) return;
  for (int pp = 1; pp < ks; ++pp)
#pragma unroll
    for (int j = 0; j < RG; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[j][r] += red[(((grp * (ks - 1) + pp - 1) * RG + j) * 4 + r) * 64 + lane];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    const int col = n0 + 16 * j + l16;
    if (col < n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        if (row < m) y[(int64_t)row * n + col] = acc[j][r];
      }
    }
  }
}

// Workgroup shape of the MFMA kernel: ks = ceil(k / 1 KB) waves per row set.
// When the 16-row groups fill at least 256 workgroups of three groups per
// wave (RG = 3, ks waves), that shape; otherwise RG = 1 with as many groups
// per workgroup as fit MF_WAVES waves and the LDS, but no more than keep one
// workgroup per CU.  Returns false when even one group does not fit (the
// caller then takes the register kernel).
struct MfShape {
  int ks, groups, rg;
};
bool mf_shape(int64_t n, int64_t k, MfShape *out) {
  const int64_t ks = (k + 1023) / 1024;
  if (k % 64 != 0 || ks > MF_WAVES) return false;
  const int64_t row_groups = (n + 15) / 16;
  if (row_groups >= 3 * 256 && mf_lds_bytes(k, ks * 3) <= MF_LDS_MAX) {
    *out = MfShape{(int)ks, 1, 3};
    return true;
  }
  int64_t groups = std::max<int64_t>(1, std::min<int64_t>(MF_WAVES / ks, row_groups / 256));
  while (groups > 1 && mf_lds_bytes(k, groups * ks) > MF_LDS_MAX) --groups;
  if (mf_lds_bytes(k, groups * ks) > MF_LDS_MAX) return false;
  *out = MfShape{(int)ks, (int)groups, 1};
  return true;
}

// weights of at least this many bytes: the chunks of one weight-row slot
// share an XCD, so that the later ones find the weights in that XCD's L2
// (measured: 8-20% faster from 8 MB of weights up, 0.1-0.2 us slower at
// 1.6 MB and below, where one slot's weights hardly fill the L2's queues)
constexpr int64_t MF_XCD_GROUP_BYTES = 4 << 20;

template <int RG, int SRC, bool CHUNKED>
hipError_t launch_mfma16_rg(const int8_t *aq, const uint16_t *ad, const void *x, int64_t ldx,
                            int64_t m, const int8_t *wq, const uint16_t *wd, int64_t n,
                            int64_t k, const MfShape &sh, float *y, int8_t *q_out,
                            uint16_t *d_out, hipStream_t stream) {
  // LDS: the stages plus one weight-scale slot per row group of every wave
  const int64_t lds = mf_lds_bytes(k, (int64_t)sh.ks * sh.groups * RG);
  static bool raised[64];
  if (lds > 65536) {
    const hipError_t e = raise_dynamic_lds((const void *)k_gemv_mfma16<RG, SRC, CHUNKED>, (int)MF_LDS_MAX, raised);
    if (e != hipSuccess) return e;
  }
  const int64_t rows_per_wg = 16 * RG * sh.groups;
  const int64_t wgs = (n + rows_per_wg - 1) / rows_per_wg;
  const int64_t chunks = (m + 15) / 16;
  const bool xcd_group = CHUNKED && n * k >= MF_XCD_GROUP_BYTES;
  const int64_t grid = xcd_group ? (wgs + 7) / 8 * 8 * chunks : wgs * chunks;
  hipLaunchKernelGGL((k_gemv_mfma16<RG, SRC, CHUNKED>), dim3((unsigned)grid),
                     dim3(64 * sh.ks * sh.groups), (unsigned)lds, stream, aq, ad, x, (int)ldx,
                     (int)m, wq, wd, (int)n, (int)k, sh.ks, y, q_out, d_out, (int)chunks,
                     (int)xcd_group);
  return hipGetLastError();
}

hipError_t launch_mfma16(const int8_t *aq, const uint16_t *ad, int64_t m,
                         const int8_t *wq, const uint16_t *wd, int64_t n, int64_t k,
                         const MfShape &sh, float *y, hipStream_t stream) {
  if (sh.rg == 3)
    return m > 16 ? launch_mfma16_rg<3, ACT_Q8, true>(aq, ad, nullptr, 0, m, wq, wd, n, k, sh, y, nullptr, nullptr, stream)
                  : launch_mfma16_rg<3, ACT_Q8, false>(aq, ad, nullptr, 0, m, wq, wd, n, k, sh, y, nullptr, nullptr, stream);
  return m > 16 ? launch_mfma16_rg<1, ACT_Q8, true>(aq, ad, nullptr, 0, m, wq, wd, n, k, sh, y, nullptr, nullptr, stream)
                : launch_mfma16_rg<1, ACT_Q8, false>(aq, ad, nullptr, 0, m, wq, wd, n, k, sh, y, nullptr, nullptr, stream);
}
}  // namespace

namespace {
// The kernel that the thin-M dispatch takes: more than 4 rows, int8 MFMA
// while its stages fit (k a multiple of 64 and wd 4-byte aligned: the weight
// scales load in aligned pairs); otherwise the register kernel while the m
// rows of codes fit its LDS stage; otherwise the LDS kernel.
enum class ThinPath { MFMA16, REG, LDS };

ThinPath thin_path(int64_t m, int64_t n, int64_t k, const uint16_t *wd, MfShape *sh) {
  if (m > 4 && ((uintptr_t)wd & 3) == 0 && mf_shape(n, k, sh)) return ThinPath::MFMA16;
  const int64_t ch = pow2_ceil((k + 1023) / 1024);
  if (pow2_ceil(m) <= 16 && reg_fits((int)pow2_ceil(m), (int)std::min<int64_t>(ch, 1 << 20), ACT_Q8))
    return ThinPath::REG;
  return ThinPath::LDS;
}
}  // namespace

bool gemv_thin_chunks_ok(int64_t m, int64_t n, int64_t k, const uint16_t *wd) {
  MfShape sh;
  return m > 16 && thin_path(m, n, k, wd, &sh) == ThinPath::MFMA16;
}

hipError_t launch_gemv_thin(const int8_t *aq, const uint16_t *ad, int64_t m,
                            const int8_t *wq, const uint16_t *wd, int64_t n,
                            int64_t k, float *y, hipStream_t stream) {
  MfShape sh;
  const ThinPath path = thin_path(m, n, k, wd, &sh);
  if (path == ThinPath::MFMA16) return launch_mfma16(aq, ad, m, wq, wd, n, k, sh, y, stream);
  if (m > 16) return hipErrorInvalidValue;  // only the MFMA kernel takes row chunks
  const int64_t mt = pow2_ceil(m);
  if (path == ThinPath::REG) {
    switch (mt) {
      case 1: return launch_reg_ch<1, ACT_Q8>(aq, ad, nullptr, 0, m, wq, wd, n, k, y, nullptr, nullptr, stream);
      case 2: return launch_reg_ch<2, ACT_Q8>(aq, ad, nullptr, 0, m, wq, wd, n, k, y, nullptr, nullptr, stream);
      case 4: return launch_reg_ch<4, ACT_Q8>(aq, ad, nullptr, 0, m, wq, wd, n, k, y, nullptr, nullptr, stream);
      case 8: return launch_reg_ch<8, ACT_Q8>(aq, ad, nullptr, 0, m, wq, wd, n, k, y, nullptr, nullptr, stream);
      default: return launch_reg_ch<16, ACT_Q8>(aq, ad, nullptr, 0, m, wq, wd, n, k, y, nullptr, nullptr, stream);
    }
  }
  if (m <= 1) return launch_mt<1>(aq, ad, m, wq, wd, n, k, y, stream);
  if (m <= 2) return launch_mt<2>(aq, ad, m, wq, wd, n, k, y, stream);
  if (m <= 4) return launch_mt<4>(aq, ad, m, wq, wd, n, k, y, stream);
  if (m <= 8) return launch_mt<8>(aq, ad, m, wq, wd, n, k, y, stream);
  return launch_mt<16>(aq, ad, m, wq, wd, n, k, y, stream);
}

// The fused launch runs the kernel that the two calls would run, with the
// quantizer inside, so its results are bit-identical to theirs.  Every
// workgroup (the MFMA kernel: every wave) quantizes the activation rows
// again, which pays off for one row at any k up to 16 K, and for a few rows
// while m * k <= MF_FUSED_ELEMS (16 KB of fp32).  Larger problems take the
// quantizer and then the GEMV (m = 4 on the decode shape: 19.9 us fused
// against 13.4 us for the two calls).
bool gemv_fused_supported(int64_t m, int64_t n, int64_t k, const uint16_t *wd) {
  MfShape sh;
  switch (thin_path(m, n, k, wd, &sh)) {
    case ThinPath::MFMA16:
      // (one row group per wave: the three-group shape would spill the
      // quantizer's registers)
      return sh.ks == 1 && sh.rg == 1 && m * k <= MF_FUSED_ELEMS;
    case ThinPath::REG:
      return m == 1 || (m <= 4 && m * k <= MF_FUSED_ELEMS);
    default:
      return false;
  }
}

hipError_t launch_gemv_fused(const void *x, bool f16, int64_t ldx, int64_t m,
                             const int8_t *wq, const uint16_t *wd, int64_t n,
                             int64_t k, float *y, int8_t *q_out,
                             uint16_t *d_out, hipStream_t stream) {
  MfShape sh;
  if (thin_path(m, n, k, wd, &sh) == ThinPath::MFMA16) {
    // one K part (k <= 1 KB) and one row group per wave, as the two-call
    // path runs it; MF_FUSED_GROUPS row groups per workgroup share the
    // quantization (the workgroup shape does not change any result)
    // (waves past the last row group compute clamped rows and store nothing)
    sh.groups = MF_FUSED_GROUPS;
    return f16 ? launch_mfma16_rg<1, ACT_F16, false>(nullptr, nullptr, x, ldx, m, wq, wd, n, k, sh, y, q_out, d_out, stream)
               : launch_mfma16_rg<1, ACT_F32, false>(nullptr, nullptr, x, ldx, m, wq, wd, n, k, sh, y, q_out, d_out, stream);
  }
  switch (pow2_ceil(m)) {
    case 1:
      return f16 ? launch_reg_ch<1, ACT_F16>(nullptr, nullptr, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream)
                 : launch_reg_ch<1, ACT_F32>(nullptr, nullptr, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream);
    case 2:
      return f16 ? launch_reg_ch<2, ACT_F16>(nullptr, nullptr, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream)
                 : launch_reg_ch<2, ACT_F32>(nullptr, nullptr, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream);
    default:
      return f16 ? launch_reg_ch<4, ACT_F16>(nullptr, nullptr, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream)
                 : launch_reg_ch<4, ACT_F32>(nullptr, nullptr, x, ldx, m, wq, wd, n, k, y, q_out, d_out, stream);
  }
}

}  // namespace bqi
