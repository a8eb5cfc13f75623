// grouped_w4a8.hip -- expert routing and the grouped 4-bit-weight x 8-bit-
// activation GEMM: the "grouped 4-bit GEMM for MoE routing" of "A 35B
// Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU" (gist.science
// summary, Method 1) with its group-wise symmetric 4-bit weights and 8-bit
// activations (Method 2).  The page's decode kernel widens 4-bit x 8-bit
// products with SSSE3 pmaddubsw; here the nibbles are unpacked in registers
// straight into int8 MFMA operands.
//
// Routing (k_route): one workgroup per expert reads all routed ids twice from
// L2 with coalesced loads: first to count the valid ids below the expert (its
// offset) and equal to it, then, staged in LDS, to place its rows: each
// thread owns a contiguous slice and one workgroup scan orders the matches,
// so rows come out in increasing row order.  No cross-workgroup pass and no
// atomics are needed, and the result is deterministic.
//
// GEMM (k_grouped_w4a8): one workgroup per (expert, 128-column tile); each of
// its 4 waves owns 32 output columns and loads those weight rows straight
// from HBM into registers (every weight byte is read once per token chunk of
// up to 96 routed rows).  The routed activation rows are gathered into LDS.
// Per 32-element group a lane unpacks 16 codes (low or high nibbles, by lane
// half) and maps c -> c - 8 bytewise with (c + 0x78) ^ 0x80, which gives the
// int8 value c - 8 without cross-byte carries.  The scale epilogue is the one
// of the Q8_0 MFMA GEMM (one rounding per term).
#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

namespace {

constexpr int ROUTE_THREADS = 256;

__device__ __forceinline__ int wg_exclusive_scan(int v, int *s_tmp, int &total) {
  // two-level scan: wave prefix via shuffles, then across the 4 waves in LDS
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int wave_base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < ROUTE_THREADS / 64; ++w) {
    const int x = s_tmp[w];
    if (w < wave) wave_base += x;
    sum += x;
  }
  __syncthreads();
  total = sum;
  return wave_base + incl - v;
}

constexpr int ROUTE_CHUNK = 8192;  // ids staged in LDS per pass (32 KB)

__global__ __launch_bounds__(ROUTE_THREADS) void k_route(
    const int32_t *__restrict__ ids, int rows_total, int n_experts,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ rows, float *__restrict__ y, int n) {
  __shared__ int s_ids[ROUTE_CHUNK];
  __shared__ int s_tmp[ROUTE_THREADS / 64];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;

  // pass 1: rows routed to experts below e (this expert's offset) and to e,
  // with coalesced loads
  int below = 0, eq = 0;
  for (int r = tid; r < rows_total; r += ROUTE_THREADS) {
    const int v = ids[r];
    below += (v >= 0 && v < e);
    eq += (v == e);
  }
  int n_below, n_eq;
  (void)wg_exclusive_scan(below, s_tmp, n_below);
  (void)wg_exclusive_scan(eq, s_tmp, n_eq);
  if (tid == 0) {
    counts[e] = n_eq;
    offsets[e] = n_below;
    if (e == n_experts - 1) offsets[n_experts] = n_below + n_eq;
  }

  // pass 2: stage ids chunk by chunk in LDS; each thread scans a contiguous
  // slice, one workgroup scan orders the matches, so rows come out in
  // increasing row index
  int base = n_below;
  for (int c0 = 0; c0 < rows_total; c0 += ROUTE_CHUNK) {
    const int len = min(ROUTE_CHUNK, rows_total - c0);
    for (int i = tid; i < len; i += ROUTE_THREADS) s_ids[i] = ids[c0 + i];
    __syncthreads();
    const int per = (len + ROUTE_THREADS - 1) / ROUTE_THREADS;
    const int r0 = min(len, tid * per), r1 = min(len, r0 + per);
    int mine = 0;
    for (int r = r0; r < r1; ++r) mine += (s_ids[r] == e);
    int total;
    int pos = base + wg_exclusive_scan(mine, s_tmp, total);
    for (int r = r0; r < r1 && mine > 0; ++r)
      if (s_ids[r] == e) {
        rows[pos++] = c0 + r;
        --mine;
      }
    base += total;
    __syncthreads();
  }

  // zero the output rows of invalid ids; workgroup e checks rows r = e (mod E)
  if (y != nullptr) {
    for (int r = e + tid * n_experts; r < rows_total; r += ROUTE_THREADS * n_experts) {
      const int v = ids[r];
      if (v < 0 || v >= n_experts)
        for (int c = 0; c < n; ++c) y[(int64_t)r * n + c] = 0.0f;
    }
  }
}

constexpr int GBN = 128;        // output columns per workgroup (4 waves x 32)
constexpr int GBK = 128;        // K elements per stage (4 groups)
constexpr int GNB = GBK / QK;   // groups per stage
constexpr int MT_MAX = 3;       // 32-row token tiles per chunk
constexpr int CHUNK = 32 * MT_MAX;

// Unpack the 16 codes this lane feeds to the MFMA (low nibbles for lanes
// 0..31 = elements 0..15 of the group, high nibbles for lanes 32..63 =
// elements 16..31) and map each code c to the int8 value c - 8.
__device__ __forceinline__ i32x4 unpack_w4(const i32x4 p, int shift) {
  i32x4 r;
  r.x = (int32_t)(((((uint32_t)p.x >> shift) & 0x0f0f0f0fu) + 0x78787878u) ^ 0x80808080u);
  r.y = (int32_t)(((((uint32_t)p.y >> shift) & 0x0f0f0f0fu) + 0x78787878u) ^ 0x80808080u);
  r.z = (int32_t)(((((uint32_t)p.z >> shift) & 0x0f0f0f0fu) + 0x78787878u) ^ 0x80808080u);
  r.w = (int32_t)(((((uint32_t)p.w >> shift) & 0x0f0f0f0fu) + 0x78787878u) ^ 0x80808080u);
  return r;
}

__global__ __launch_bounds__(256, 2) void k_grouped_w4a8(
    const int8_t *__restrict__ aq, const uint16_t *__restrict__ ad, int top_k,
    const uint8_t *__restrict__ wq4, const uint16_t *__restrict__ wd,
    int n_experts, int n, int k, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ rows,
    float *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) int8_t sA[2][CHUNK * GBK];  // [row][128 B], 16B chunks XOR-swizzled
  __shared__ __attribute__((aligned(16))) uint16_t sAd[2][GNB][CHUNK];
  __shared__ int s_tok[CHUNK];   // token index of each staged row
  __shared__ int s_row[CHUNK];   // routed row index (output row)

  // all column tiles of one expert share (blockIdx % n_experts), hence one XCD
  // when n_experts is a multiple of 8
  const int e = blockIdx.x % n_experts;
  const int tn = blockIdx.x / n_experts;
  const int cnt = counts[e];
  if (cnt == 0) return;
  const int off = offsets[e];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int nbk = k / QK;
  const int stages = (nbk + GNB - 1) / GNB;
  const int col = tn * GBN + wave * 32 + l32;           // this lane's output column
  const int wrow = min(col, n - 1);
  const uint8_t *wsrc = wq4 + ((int64_t)e * n + wrow) * (k / 2);
  const uint16_t *wdsrc = wd + ((int64_t)e * n + wrow) * nbk;

  i32x16 seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = MAGIC_BITS;

  for (int c0 = 0; c0 < cnt; c0 += CHUNK) {
    const int crows = min(CHUNK, cnt - c0);
    const int mtiles = (crows + 31) / 32;
    __syncthreads();
    if (tid < CHUNK) {
      const int rr = tid < crows ? rows[off + c0 + tid] : rows[off + c0];
      s_row[tid] = rr;
      s_tok[tid] = rr / top_k;
    }
    __syncthreads();

    // staging: activation rows (CHUNK x 128 B = 768 chunks of 16 B), scales
    // (CHUNK x 4 groups), and this lane's weight bytes (4 groups x 16 B)
    i32x4 a_st[3];
    uint16_t s_st[2];
    i32x4 w_st[GNB];
    uint16_t wd_st[GNB];
    auto load_stage = [&](int s) {
      const int k0 = s * GBK;
#pragma unroll
      for (int h = 0; h < 3; ++h) {
        const int c = tid + 256 * h;
        const int r = c >> 3, cc = c & 7;
        const bool ok = r < crows && k0 + cc * 16 < k;
        a_st[h] = ok ? *reinterpret_cast<const i32x4 *>(aq + (int64_t)s_tok[r] * k + k0 + cc * 16)
                     : i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = tid + 256 * h;  // CHUNK*GNB = 384 scale slots
        const int r = c >> 2, b = c & 3;
        const bool ok = c < CHUNK * GNB && r < crows && s * GNB + b < nbk;
        s_st[h] = ok ? ad[(int64_t)s_tok[r] * nbk + s * GNB + b] : (uint16_t)0;
      }
#pragma unroll
      for (int b = 0; b < GNB; ++b) {
        const bool ok = s * GNB + b < nbk;
        w_st[b] = ok ? __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(
                           wsrc + (int64_t)(s * GNB + b) * (QK / 2)))
                     : i32x4{0, 0, 0, 0};
        wd_st[b] = ok ? wdsrc[s * GNB + b] : (uint16_t)0;
      }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
      for (int h = 0; h < 3; ++h) {
        const int c = tid + 256 * h;
        const int r = c >> 3, cc = c & 7;
        *reinterpret_cast<i32x4 *>(&sA[buf][r * GBK + ((cc ^ (r & 7)) * 16)]) = a_st[h];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = tid + 256 * h;
        if (c < CHUNK * GNB) sAd[buf][c & 3][c >> 2] = s_st[h];
      }
    };

    float acc[MT_MAX][16];
#pragma unroll
    for (int t = 0; t < MT_MAX; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

    load_stage(0);
    store_stage(0);
    i32x4 w_cur[GNB];
    uint16_t wd_cur[GNB];
#pragma unroll
    for (int b = 0; b < GNB; ++b) {
      w_cur[b] = w_st[b];
      wd_cur[b] = wd_st[b];
    }
    __syncthreads();

    for (int s = 0; s < stages; ++s) {
      const int buf = s & 1;
      if (s + 1 < stages) load_stage(s + 1);
      const int nb_here = min(GNB, nbk - s * GNB);
#pragma unroll
      for (int b = 0; b < GNB; ++b) {
        if (b < nb_here) {
          const i32x4 wf = unpack_w4(w_cur[b], 4 * g);
          const float dw = half_bits_to_float(wd_cur[b]);
          const float ncd = -MAGIC_F * dw;
#pragma unroll
          for (int t = 0; t < MT_MAX; ++t) {
            if (t < mtiles) {
              const int r = t * 32 + l32;
              const i32x4 af = *reinterpret_cast<const i32x4 *>(
                  &sA[buf][r * GBK + (((2 * b + g) ^ (r & 7)) * 16)]);
              const i32x16 d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, wf, seed, 0, 0, 0);
              uint16_t dah[16];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint2 v = *reinterpret_cast<const uint2 *>(&sAd[buf][b][t * 32 + 8 * q + 4 * g]);
                dah[4 * q + 0] = (uint16_t)(v.x & 0xffffu);
                dah[4 * q + 1] = (uint16_t)(v.x >> 16);
                dah[4 * q + 2] = (uint16_t)(v.y & 0xffffu);
                dah[4 * q + 3] = (uint16_t)(v.y >> 16);
              }
#pragma unroll
              for (int r2 = 0; r2 < 16; ++r2) {
                const float tt = fmaf(bits_to_float(d[r2]), dw, ncd);
                acc[t][r2] = fmaf(tt, half_bits_to_float(dah[r2]), acc[t][r2]);
              }
            }
          }
        }
      }
      if (s + 1 < stages) {
        store_stage(buf ^ 1);
#pragma unroll
        for (int b = 0; b < GNB; ++b) {
          w_cur[b] = w_st[b];
          wd_cur[b] = wd_st[b];
        }
      }
      __syncthreads();
    }

    // store: lane's column `col`, rows t*32 + 8q + 4g + (0..3) of the chunk
    if (col < n) {
#pragma unroll
      for (int t = 0; t < MT_MAX; ++t) {
        if (t < mtiles) {
#pragma unroll
          for (int r2 = 0; r2 < 16; ++r2) {
            const int rr = t * 32 + 8 * (r2 >> 2) + 4 * g + (r2 & 3);
            if (rr < crows) y[(int64_t)s_row[rr] * n + col] = acc[t][r2];
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_route_topk(const int32_t *ids, int64_t rows_total,
                             int64_t n_experts, int32_t *counts,
                             int32_t *offsets, int32_t *rows, float *y,
                             int64_t n, hipStream_t stream) {
  hipLaunchKernelGGL(k_route, dim3((unsigned)n_experts), dim3(ROUTE_THREADS), 0,
                     stream, ids, (int)rows_total, (int)n_experts, counts,
                     offsets, rows, y, (int)n);
  return hipGetLastError();
}

hipError_t launch_grouped_w4a8(const int8_t *aq, const uint16_t *ad,
                               int64_t top_k, const uint8_t *wq4,
                               const uint16_t *wd, int64_t n_experts,
                               int64_t n, int64_t k, const int32_t *counts,
                               const int32_t *offsets, const int32_t *rows,
                               float *y, hipStream_t stream) {
  const int64_t tiles_n = (n + GBN - 1) / GBN;
  hipLaunchKernelGGL(k_grouped_w4a8, dim3((unsigned)(n_experts * tiles_n)),
                     dim3(256), 0, stream, aq, ad, (int)top_k, wq4, wd,
                     (int)n_experts, (int)n, (int)k, counts, offsets, rows, y);
  return hipGetLastError();
}

}  // namespace bqi
