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
constexpr int GNB = 4;          // 32-element groups per stage
constexpr int GBK = GNB * QK;   // activation bytes per row per stage (128)
constexpr int MT_MAX = 3;       // 32-row token tiles per chunk
constexpr int CHUNK = 32 * MT_MAX;
constexpr int NSTAGE = 2;       // LDS double buffer; loads run one stage ahead
constexpr int GTHREADS = 256;

// Physical slot of the 16-byte activation chunk c of staged row r (rows of
// 128 B; spreads a 16-lane fragment read over all 64 LDS banks).
__device__ __forceinline__ int aswz(int r, int c) { return c ^ ((r >> 1) & 7); }
// Physical slot of group b of weight column c (columns of 64 B = 4 groups).
__device__ __forceinline__ int wswz(int c, int b) { return b ^ ((c >> 2) & 3); }

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

struct GStage {
  int8_t a[CHUNK * GBK];      // gathered activation rows, swizzled 16-byte chunks
  uint8_t w[GBN * GNB * 16];  // packed 4-bit weights: [col][group] 16 B, swizzled
  float wd[GBN][GNB];         // weight scales, fp32, [col][group]
  float ad[GNB][CHUNK];       // activation scales, fp32, [group][row]
};

// The MFMA work of one stage, read from LDS.
__device__ __forceinline__ void grouped_stage_compute(
    const GStage *__restrict__ SB, int nb_here, int mtiles, int col_l, int l32,
    int g, const i32x16 &seed, float (&acc)[MT_MAX][16]) {
#pragma unroll
  for (int b = 0; b < GNB; ++b) {
    if (b >= nb_here) break;
    const int c = col_l;
    const i32x4 packed = *reinterpret_cast<const i32x4 *>(&SB->w[c * (GNB * 16) + 16 * wswz(c, b)]);
    const i32x4 wf = unpack_w4(packed, 4 * g);
    const float dw = SB->wd[c][b];
    const float ncd = -MAGIC_F * dw;
#pragma unroll
    for (int t = 0; t < MT_MAX; ++t) {
      if (t < mtiles) {
        const int r = t * 32 + l32;
        const i32x4 af = *reinterpret_cast<const i32x4 *>(&SB->a[r * GBK + 16 * aswz(r, 2 * b + g)]);
        const i32x16 d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, wf, seed, 0, 0, 0);
        float da[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = *reinterpret_cast<const f32x4 *>(&SB->ad[b][t * 32 + 8 * q + 4 * g]);
          da[4 * q + 0] = v.x;
          da[4 * q + 1] = v.y;
          da[4 * q + 2] = v.z;
          da[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) {
          const float tt = fmaf(bits_to_float(d[r2]), dw, ncd);
          acc[t][r2] = fmaf(tt, da[r2], acc[t][r2]);
        }
      }
    }
  }
}

__global__ __launch_bounds__(GTHREADS, 2) void k_grouped_w4a8(
    const int8_t *__restrict__ aq, const uint16_t *__restrict__ ad, int top_k,
    const uint8_t *__restrict__ wq4, const uint16_t *__restrict__ wd,
    int n_experts, int n, int k, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ rows,
    float *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) GStage S[NSTAGE];
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
  const int n0 = tn * GBN;
  const int col_l = wave * 32 + l32;  // this lane's output column within the tile
  const int64_t wrow0 = (int64_t)e * n;

  i32x16 seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = MAGIC_BITS;

  for (int c0 = 0; c0 < cnt; c0 += CHUNK) {
    const int crows = min(CHUNK, cnt - c0);
    const int mtiles = (crows + 31) / 32;
    __syncthreads();
    if (tid < CHUNK) {
      const int rr = rows[off + c0 + min(tid, crows - 1)];
      s_row[tid] = rr;
      s_tok[tid] = rr / top_k;
    }
    __syncthreads();

    // ---- stage loads ------------------------------------------------------
    // activations: 96 rows x 8 chunks = 12 wave loads (3 per wave); lane L of
    // load q fills row 8*(3*wave+q) + L/8, slot L%8 = chunk (L%8)^swizzle.
    // weights: 128 columns x 4 groups = 8 wave loads (2 per wave); lane L of
    // load q fills column 16*(2*wave+q) + L/4, slot L%4 = group (L%4)^swizzle.
    // scales (activation: 96 rows x 4 groups, weight: 128 columns x 4
    // groups) go through registers, 2 + 2 fp16 per thread, and are stored to
    // LDS as fp32.  Per stage each wave issues 4 scale loads into registers
    // (issue_scales) and 5 direct LDS loads (issue_direct).
    uint16_t sa_reg[2], sw_reg[2];
    auto issue_scales = [&](int s) {
      const int g0 = min(s, stages - 1) * GNB;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int idx = tid + GTHREADS * h;  // CHUNK*GNB = 384 entries
        const int r = min(idx / GNB, CHUNK - 1), b = idx % GNB;
        const int gb = g0 + b < nbk ? g0 + b : 0;
        sa_reg[h] = ad[(int64_t)s_tok[r] * nbk + gb];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int idx = tid + GTHREADS * h;  // GBN*GNB = 512 entries
        const int c = idx / GNB, b = idx % GNB;
        const int gb = g0 + b < nbk ? g0 + b : 0;
        sw_reg[h] = wd[(wrow0 + min(n0 + c, n - 1)) * nbk + gb];
      }
    };
    auto store_scales = [&](int slot) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int idx = tid + GTHREADS * h;
        if (idx < CHUNK * GNB) S[slot].ad[idx % GNB][idx / GNB] = half_bits_to_float(sa_reg[h]);
        S[slot].wd[idx / GNB][idx % GNB] = half_bits_to_float(sw_reg[h]);
      }
    };
    auto issue_direct = [&](int s, int slot) {
      const int g0 = min(s, stages - 1) * GNB;
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const int rt = 8 * (3 * wave + q);
        const int r = rt + lane / 8;
        const int c = (lane % 8) ^ ((r >> 1) & 7);
        const int kk = 32 * g0 + 16 * c < k ? 32 * g0 + 16 * c : 0;
        dma_lds16(aq + ((int64_t)s_tok[r] * k + kk), lds_addr(&S[slot].a[rt * GBK]));
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ct = 16 * (2 * wave + q);
        const int c = ct + lane / 4;
        const int b = (lane % 4) ^ ((c >> 2) & 3);
        const int gb = g0 + b < nbk ? g0 + b : 0;
        const int64_t wr = wrow0 + min(n0 + c, n - 1);
        dma_lds16(wq4 + (wr * (k / 2) + 16 * gb), lds_addr(&S[slot].w[ct * (GNB * 16)]));
      }
    };

    float acc[MT_MAX][16];
#pragma unroll
    for (int t = 0; t < MT_MAX; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

    // prologue: stage 0 in LDS
    issue_scales(0);
    issue_direct(0, 0);
    store_scales(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int s = 0; s < stages; ++s) {
      const int buf = s & 1;
      // stage s+1: scale loads first (loads retire in order, so storing the
      // scales waits only for them), then the direct loads, which run while
      // stage s computes
      // (Ordering rests on the explicit wait and barrier below: stage s reads
      // buffer buf, loaded and waited for one iteration earlier, while these
      // direct loads fill buf ^ 1.)
      const bool more = s + 1 < stages;
      if (more) {
        issue_scales(s + 1);
        issue_direct(s + 1, buf ^ 1);
      }
      grouped_stage_compute(&S[buf], min(GNB, nbk - s * GNB), mtiles, col_l, l32, g, seed, acc);
      if (more) store_scales(buf ^ 1);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of stage s+1 have landed
      __syncthreads();
    }
    // drain: no direct load may still target LDS when the next chunk (or the
    // next workgroup on this CU) reuses it
    __builtin_amdgcn_s_waitcnt(0);

    // store: lane's column, rows t*32 + 8q + 4g + (0..3) of the chunk
    const int col = n0 + col_l;
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
