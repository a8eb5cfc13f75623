// grouped_w4a8.hip -- expert routing and the grouped 4-bit-weight x 8-bit-
// activation GEMM: the "grouped 4-bit GEMM for MoE routing" of "A 35B
// Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU" (gist.science
// summary, Method 1) with its group-wise symmetric 4-bit weights and 8-bit
// activations (Method 2).  The page's decode kernel widens 4-bit x 8-bit
// products with SSSE3 pmaddubsw; here the nibbles are unpacked in registers
// straight into int8 MFMA operands.
//
// Routing (k_route): one workgroup of 1024 threads per expert.  Each thread
// owns a contiguous slice of 8 routed ids, counts the valid ids below the
// expert (its offset) and equal to it, and one workgroup scan orders the
// matches, so rows come out in increasing row order.  Up to 8192 routed rows
// this is a single pass over ids held in registers; beyond, a counting pass
// and a placing pass run chunk by chunk.  No atomics, deterministic.  For the grouped GEMM the same kernel also
// copies the activation scales of the routed rows, converted to fp32, into a
// block-major table in expert order (one 4-byte entry per routed row and
// block), which the GEMM then streams into LDS without conversion.
//
// GEMM (k_grouped_w4a8): one workgroup of 12 waves per (expert, 384-column
// tile); each wave owns 32 output columns.  K advances 4 groups (128
// elements) per stage through three LDS buffers, two stages in flight.  Every
// operand travels HBM/L2 -> LDS through gfx950's direct loads: the packed
// weights (64 bytes per column and stage), their fp16 scales, the routed
// activation rows (gathered by token, 128 bytes per row and stage) and the
// fp32 activation scales.  The products run on v_mfma_i32_32x32x32_i8 (one
// instruction = one 32x32 tile for exactly one group); on gfx950 it costs
// about as many cycles as the 16x16x32 form while doing four times the MACs,
// and MFMA and VALU time largely add up in this kernel.  Per group a lane
// unpacks its 16 codes (low or high nibbles by lane half) into the int8
// values 16*(c - 8) with a shift, a mask and an xor; the factor 16 is folded
// into the weight scale.  The scale epilogue is the one of the Q8_0
// MFMA GEMM (one rounding per term).  Routed rows are taken 96 at a time (six
// 16-row tiles), so an expert's weights are streamed once per 96 rows.
#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

namespace {

// ---------------------------------------------------------------- routing --
constexpr int RT = 1024;          // threads per routing workgroup
constexpr int RPT = 8;            // ids per thread per pass
constexpr int RCHUNK = RT * RPT;  // ids per pass

// Exclusive workgroup scan of one int per thread (RT threads); `total` gets
// the sum.  Contains two barriers.
__device__ __forceinline__ int route_scan(int v, int *s_tmp, int &total) {
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
  for (int w = 0; w < RT / 64; ++w) {
    const int x = s_tmp[w];
    if (w < wave) wave_base += x;
    sum += x;
  }
  __syncthreads();
  total = sum;
  return wave_base + incl - v;
}

// Copy the activation scales of this expert's `total` matched rows (routed
// rows s_match[0 .. total)) into the block-major fp32 table at positions
// base .. base+total-1.  Tiles of up to 96 rows x 64 groups go through LDS:
// each thread reads 8 consecutive scales of one row with one 16-byte load
// (4 two-byte loads for 64-row tiles where the scale rows are not 16-byte
// aligned), and each 16 threads write 16 consecutive positions of one table
// row, instead of scattering 2-byte reads over every matched token per table
// row.  An expert's rows rarely exceed 96, so its gather is one round trip.
constexpr int RC_ROWS = 96;            // routed rows per tile (16-byte path)
constexpr int RC_PITCH = RC_ROWS + 1;  // floats per group row of the tile

__device__ __forceinline__ void route_copy_scales(const int *s_match, int total, int base,
                                                  int top_k, const uint16_t *ad,
                                                  int nbk, float *__restrict__ ad32t, int rpad,
                                                  float *s_t) {
  const int tid = threadIdx.x;
  const bool vec = nbk % 8 == 0 && ((uintptr_t)ad & 15) == 0;
  const int tile_rows = vec ? RC_ROWS : 64;
  for (int i0 = 0; i0 < total; i0 += tile_rows) {
    for (int b0 = 0; b0 < nbk; b0 += 64) {
      if (vec) {
        // thread -> row i0 + tid/8, groups b0 + 8*(tid%8) .. +7
        const int r = tid >> 3, c = 8 * (tid & 7);
        const int i = i0 + r;
        if (r < RC_ROWS && i < total && b0 + c < nbk) {
          const uint4 v = *reinterpret_cast<const uint4 *>(ad + (int64_t)(s_match[i] / top_k) * nbk + b0 + c);
          const uint32_t h2[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            s_t[(c + 2 * u) * RC_PITCH + r] = half_bits_to_float((uint16_t)(h2[u] & 0xffffu));
            s_t[(c + 2 * u + 1) * RC_PITCH + r] = half_bits_to_float((uint16_t)(h2[u] >> 16));
          }
        }
      } else {
        // thread -> row i0 + tid/16, groups b0 + 4*(tid%16) .. +3
        const int r = tid >> 4, c = 4 * (tid & 15);
        const int i = i0 + r;
        if (i < total) {
          const uint16_t *src = ad + (int64_t)(s_match[i] / top_k) * nbk;
          // the four loads are unconditional (clamped to the row) so that
          // they are in flight together; the values are masked afterwards
          uint16_t h[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) h[u] = src[min(b0 + c + u, nbk - 1)];
          __asm__ volatile("" ::: "memory");
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (b0 + c + u < nbk) s_t[(c + u) * RC_PITCH + r] = half_bits_to_float(h[u]);
        }
      }
      __syncthreads();
      {
        // thread -> table row b0 + tid/16, positions i0 + (tid%16) + 16*u
        const int c = tid >> 4, r = tid & 15;
        if (b0 + c < nbk) {
          float *dst = ad32t + (int64_t)(b0 + c) * rpad + base + i0;
#pragma unroll
          for (int u = 0; u < RC_ROWS / 16; ++u)
            if (16 * u < tile_rows && i0 + r + 16 * u < total)
              dst[r + 16 * u] = s_t[c * RC_PITCH + r + 16 * u];
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(RT) void k_route(
    const int32_t *__restrict__ ids, int rows_total, int n_experts, int top_k,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ rows, const uint16_t *ad, int nbk,
    float *__restrict__ ad32t, int rpad, float *__restrict__ y, int n) {
  __shared__ int s_tmp[RT / 64];
  __shared__ int s_match[RCHUNK];  // (position - chunk base) -> routed row
  __shared__ float s_t[64 * RC_PITCH];  // transpose tile of the scale copy
  const int e = blockIdx.x;
  const int tid = threadIdx.x;

  if (rows_total <= RCHUNK) {
    // one pass: each thread keeps its 8 ids in registers; one workgroup scan
    // of (below << 16 | eq) gives both this expert's offset (the total of the
    // high halves) and each thread's first position (the prefix of the low
    // halves; at most 8192, so no carry reaches the high half)
    const int r0 = tid * RPT;
    int v[RPT];
    int below = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      v[j] = r0 + j < rows_total ? ids[r0 + j] : -1;
      below += (v[j] >= 0 && v[j] < e);
      eq += (v[j] == e);
    }
    int total;
    const int excl = route_scan((below << 16) | eq, s_tmp, total);
    const int n_below = total >> 16, n_eq = total & 0xffff;
    if (tid == 0) {
      counts[e] = n_eq;
      offsets[e] = n_below;
      if (e == n_experts - 1) offsets[n_experts] = n_below + n_eq;
    }
    int pos = excl & 0xffff;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      if (v[j] == e) {
        rows[n_below + pos] = r0 + j;
        s_match[pos] = r0 + j;
        ++pos;
      }
      // invalid ids: workgroup (row mod E) zeroes the output row
      const int r = r0 + j;
      if (y != nullptr && r < rows_total && (v[j] < 0 || v[j] >= n_experts) &&
          r % n_experts == e)
        for (int c = 0; c < n; ++c) y[(int64_t)r * n + c] = 0.0f;
    }
    if (ad32t != nullptr && n_eq > 0) {
      __syncthreads();
      route_copy_scales(s_match, n_eq, n_below, top_k, ad, nbk, ad32t, rpad, s_t);
    }
    return;
  }

  // general case, several chunks of ids
  // pass 1: valid ids below this expert (its offset) and equal to it
  int below = 0, eq = 0;
  for (int c0 = 0; c0 < rows_total; c0 += RCHUNK) {
    const int r0 = c0 + tid * RPT;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = r0 + j;
      const int v = r < rows_total ? ids[r] : -1;
      below += (v >= 0 && v < e);
      eq += (v == e);
    }
  }
  int n_below, n_eq;
  (void)route_scan(below, s_tmp, n_below);
  (void)route_scan(eq, s_tmp, n_eq);
  if (tid == 0) {
    counts[e] = n_eq;
    offsets[e] = n_below;
    if (e == n_experts - 1) offsets[n_experts] = n_below + n_eq;
  }

  // pass 2: place the matches in increasing row order; with ad32t, also copy
  // their activation scales (fp16 -> fp32) into the block-major table
  int base = n_below;
  for (int c0 = 0; c0 < rows_total && base < n_below + n_eq; c0 += RCHUNK) {
    const int r0 = c0 + tid * RPT;
    int v[RPT];
    int mine = 0;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      v[j] = r0 + j < rows_total ? ids[r0 + j] : -1;
      mine += (v[j] == e);
    }
    int total;
    int pos = route_scan(mine, s_tmp, total);
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      if (v[j] == e) {
        rows[base + pos] = r0 + j;
        s_match[pos] = r0 + j;
        ++pos;
      }
    if (ad32t != nullptr) {
      __syncthreads();
      route_copy_scales(s_match, total, base, top_k, ad, nbk, ad32t, rpad, s_t);
      __syncthreads();
    }
    base += total;
  }

  // zero the output rows of invalid ids; workgroup e checks rows r = e (mod E)
  if (y != nullptr) {
    for (int r = e + tid * n_experts; r < rows_total; r += RT * n_experts) {
      const int v = ids[r];
      if (v < 0 || v >= n_experts)
        for (int c = 0; c < n; ++c) y[(int64_t)r * n + c] = 0.0f;
    }
  }
}

// ------------------------------------------------------------ grouped GEMM --
constexpr int GW = 12;             // waves per workgroup
constexpr int GT = GW * 64;        // threads per workgroup
constexpr int GBN = GW * 32;       // output columns per workgroup (32 per wave)
constexpr int GNB = 4;             // 32-element groups per stage
constexpr int GBK = GNB * QK;      // activation bytes per row per stage
constexpr int GRT = 3;             // 32-row MFMA tiles per chunk
constexpr int GCH = 32 * GRT;      // routed rows per chunk
constexpr int GNS = 3;             // LDS stage buffers (two stages in flight)
constexpr int G_AD_WAVES = GNB * GCH / 64;  // waves issuing activation-scale loads

static_assert(GNB * GCH % 64 == 0 && G_AD_WAVES <= GW, "scale loads map to whole waves");
static_assert(GBN * GNB == 2 * GT, "two weight-scale loads per wave and stage");
static_assert(GCH == 8 * GW, "one activation-row load per wave and stage");

struct GBuf {
  uint8_t w[GBN * GNB * 16];  // packed weights: [column][4 groups x 16 B], swizzled
  int8_t a[GCH * GBK];        // gathered activation rows: [row][8 x 16 B], swizzled
  float ad[GNB][GCH];         // activation scales, fp32, [group][row]
  uint32_t wd[GBN][GNB];      // weight scales, fp16 bits zero-extended, [column][group]
};

// Physical slot of the 16-byte activation chunk c of staged row r (rows of
// 128 B; spreads a 16-lane fragment read over all 64 LDS banks).
__device__ __forceinline__ int aswz(int r, int c) { return c ^ ((r >> 1) & 7); }
// Physical slot of group b of weight column c (columns of 64 B = 4 groups).
__device__ __forceinline__ int wswz(int c, int b) { return b ^ ((c >> 2) & 3); }

// v_mfma_i32_32x32x32_i8 takes, in lane L, the 16 consecutive K elements
// 16*(L/32) .. +15 of row (A) or column (B) L%32.  For one 32-element group
// of 4-bit codes (16 bytes: byte i holds element i in its low nibble and
// element i+16 in its high nibble) that is the low nibbles of all 16 bytes
// for lanes 0..31 and the high nibbles for lanes 32..63.  Each code c becomes
// the int8 16*(c - 8): (nibble << 4) ^ 0x80 is the byte (c ^ 8) * 16, which
// read as a signed byte is 16 * (c - 8).  The factor 16 is folded into the
// weight scale (exact); |16 * P| <= 16 * 32 * 8 * 128 < 2^22 keeps the
// accumulator-seed conversion exact.
__device__ __forceinline__ i32x4 unpack_w4x16(i32x4 p, int shl) {
  i32x4 r;
  r.x = (int32_t)((((uint32_t)p.x << shl) & 0xf0f0f0f0u) ^ 0x80808080u);
  r.y = (int32_t)((((uint32_t)p.y << shl) & 0xf0f0f0f0u) ^ 0x80808080u);
  r.z = (int32_t)((((uint32_t)p.z << shl) & 0xf0f0f0f0u) ^ 0x80808080u);
  r.w = (int32_t)((((uint32_t)p.w << shl) & 0xf0f0f0f0u) ^ 0x80808080u);
  return r;
}

// The MFMA work of one stage for one wave: 32 columns x R 32-row tiles,
// groups 0 .. nb_here-1 of the stage, read from LDS.  The group loop is
// rolled and R is a compile-time constant, so the code per group is
// straight-line: the group's fragment reads first, then all R MFMAs, then the
// R epilogues, so that the matrix core works while the epilogues run.
// Output register r of tile t in lane L is row 32t + 8(r/4) + 4(L/32) + r%4,
// column L%32 of the wave's tile.
template <int R>
__device__ __forceinline__ void grouped_stage_compute(
    const GBuf &B, int nb_here, int wave, int lane, const i32x16 &seed,
    float (&acc)[R][16]) {
  const int l32 = lane & 31, g = lane >> 5;
  const int shl = g ? 0 : 4;
  const int cl = wave * 32 + l32;
#pragma unroll 1
  for (int b = 0; b < nb_here; ++b) {
    const i32x4 p = *reinterpret_cast<const i32x4 *>(&B.w[cl * (GNB * 16) + 16 * wswz(cl, b)]);
    const uint32_t sw = B.wd[cl][b];
    i32x4 af[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int r = 32 * t + l32;
      af[t] = *reinterpret_cast<const i32x4 *>(&B.a[r * GBK + 16 * aswz(r, 2 * b + g)]);
    }
    // keep the reads above ahead of the math (the scheduler would otherwise
    // sink each next to its first use and expose the LDS latency per tile)
    __builtin_amdgcn_sched_barrier(0);
    const i32x4 wf = unpack_w4x16(p, shl);
    const float dw16 = half_bits_to_float((uint16_t)sw) * 0.0625f;  // exact
    const float ncd = -MAGIC_F * dw16;                              // exact
    i32x16 d[R];
#pragma unroll
    for (int t = 0; t < R; ++t) d[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[t], wf, seed, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < R; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(&B.ad[b][32 * t + 8 * q + 4 * g]);
        const float da[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r2 = 4 * q + j;
          const float tt = fmaf(bits_to_float(d[t][r2]), dw16, ncd);
          acc[t][r2] = fmaf(tt, da[j], acc[t][r2]);
        }
      }
    }
  }
}

struct GArgs {
  const int8_t *aq;
  const float *ad32t;
  int rpad, top_k;
  const uint8_t *wq4;
  const uint16_t *wd;
  int n, k;
  float *y;
};

// One chunk of up to 16*R routed rows of expert e against the workgroup's
// column tile: the whole K pipeline, then the stores.
template <int R>
__device__ __forceinline__ void grouped_chunk(const GArgs &A, GBuf (&S)[GNS],
                                              const int *s_tok, const int *s_row,
                                              int64_t wrow0, int n0, int off,
                                              int c0, int crows) {
  const int n = A.n, k = A.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbk = k / QK;
  const int stages = (nbk + GNB - 1) / GNB;
  const bool wave_active = n0 + wave * 32 < n;
  const int64_t kh = k / 2;  // packed bytes per weight row

  i32x16 seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = MAGIC_BITS;

  // Issue the direct loads of stage s into buffer s % GNS (5 per wave, plus
  // one activation-scale load in waves 0 .. G_AD_WAVES-1).  They go through
  // inline asm, invisible to the compiler's wait counting (see dma_lds16);
  // the waits below are explicit.  Group indices past the last group of k
  // re-read the last group (never used); columns past n re-read column n-1;
  // rows past the chunk re-read its last row.  Addresses are rebuilt per
  // stage from the thread index, laundered through an empty asm, so that the
  // compiler does not hoist a dozen 64-bit addresses out of the stage loop
  // and hold them in registers across it.
  auto issue = [&](int s) {
    int tl = tid;
    asm volatile("" : "+v"(tl));
    const int ln = tl & 63, wv = tl >> 6;
    const int g0 = s * GNB;
    GBuf &D = S[s % GNS];
    // weights: wave load h (two per wave) fills columns ct .. ct+15,
    // ct = 16 * (2w + h); lane L lands in column ct + L/4, slot L%4, which
    // holds group (L%4) ^ swizzle(column)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cl = 16 * (2 * wv + h) + (ln >> 2);
      const int lg = (ln & 3) ^ ((cl >> 2) & 3);
      const int c = min(n0 + cl, n - 1);
      dma_lds16(A.wq4 + (wrow0 + c) * kh + 16 * min(g0 + lg, nbk - 1),
                &D.w[16 * (2 * wave + h) * (GNB * 16)]);
    }
    // weight scales: wave load h fills table entries e = 64 (2w + h) + L,
    // column e / 4, group e % 4 (one fp16, zero-extended, per 4-byte slot)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 64 * (2 * wv + h) + ln;
      const int c = min(n0 + (e >> 2), n - 1);
      dma_lds_u16(A.wd + (wrow0 + c) * nbk + min(g0 + (e & 3), nbk - 1),
                  &D.wd[0][0] + 64 * (2 * wave + h));
    }
    // activation rows: wave w fills staged rows 8w .. 8w+7; lane L lands in
    // row 8w + L/8, physical chunk L%8, which holds logical chunk
    // (L%8) ^ swizzle(row)
    {
      const int ra = 8 * wv + (ln >> 3);
      const int lc = (ln & 7) ^ ((ra >> 1) & 7);
      const int kb = min(g0 + (lc >> 1), nbk - 1);
      dma_lds16(A.aq + (int64_t)s_tok[ra] * k + 32 * kb + 16 * (lc & 1), &D.a[8 * wave * GBK]);
    }
    // activation scales (waves 0 .. G_AD_WAVES-1): flat entry f = 64w + L of
    // the stage's [group][row] table
    if (wave < G_AD_WAVES) {
      const int f = 64 * wv + ln;
      dma_lds4(A.ad32t + (int64_t)min(g0 + f / GCH, nbk - 1) * A.rpad + (off + c0 + f % GCH),
               &D.ad[0][0] + 64 * wave);
    }
  };

  float acc[R][16];
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;

  issue(0);
  if (stages > 1) issue(1);
  for (int s = 0; s < stages; ++s) {
    // this wave's loads of stage s have landed (only stage s+1's, issued
    // after them, may still be in flight)
    if (s + 1 < stages) {
      if (wave < G_AD_WAVES) wait_vmcnt<6>();
      else wait_vmcnt<5>();
    } else {
      wait_vmcnt<0>();
    }
    // every wave's loads of stage s have landed, and every wave is done with
    // stage s-1, whose buffer the loads below refill
    lds_barrier();
    if (s + 2 < stages) issue(s + 2);
    if (wave_active)
      grouped_stage_compute<R>(S[s % GNS], min(GNB, nbk - s * GNB), wave, lane, seed, acc);
  }

  // store: lane's column L%32, rows 32t + 8(r/4) + 4(L/32) + r%4 of the chunk
  const int col = n0 + wave * 32 + (lane & 31);
  if (wave_active && col < n) {
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) {
        const int rr = 32 * t + 8 * (r2 >> 2) + 4 * (lane >> 5) + (r2 & 3);
        if (rr < crows) A.y[(int64_t)s_row[rr] * n + col] = acc[t][r2];
      }
  }
}

__global__ __launch_bounds__(GT, 1) void k_grouped_w4a8(
    const int8_t *__restrict__ aq, const float *__restrict__ ad32t, int rpad,
    int top_k, const uint8_t *__restrict__ wq4, const uint16_t *__restrict__ wd,
    int n_experts, int n, int k, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ rows,
    float *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) GBuf S[GNS];
  __shared__ int s_tok[GCH];  // token of each staged row
  __shared__ int s_row[GCH];  // routed row (output row) of each staged row

  // both column tiles of one expert share (blockIdx % n_experts), hence one
  // XCD when n_experts is a multiple of 8, and so the expert's activation rows
  // in that XCD's L2
  const int e = blockIdx.x % n_experts;
  const int tn = blockIdx.x / n_experts;
  const int cnt = counts[e];
  if (cnt == 0) return;
  const int off = offsets[e];
  const GArgs A{aq, ad32t, rpad, top_k, wq4, wd, n, k, y};
  const int tid = threadIdx.x;
  const int n0 = tn * GBN;
  const int64_t wrow0 = (int64_t)e * n;

  for (int c0 = 0; c0 < cnt; c0 += GCH) {
    const int crows = min(GCH, cnt - c0);
    // the previous chunk is done with s_tok, s_row and S (and its direct
    // loads have all landed: each chunk ends with vmcnt(0))
    __syncthreads();
    if (tid < GCH) {
      const int rr = rows[off + c0 + min(tid, crows - 1)];
      s_row[tid] = rr;
      s_tok[tid] = rr / top_k;
    }
    __syncthreads();
    switch ((crows + 31) / 32) {
      case 1: grouped_chunk<1>(A, S, s_tok, s_row, wrow0, n0, off, c0, crows); break;
      case 2: grouped_chunk<2>(A, S, s_tok, s_row, wrow0, n0, off, c0, crows); break;
      default: grouped_chunk<3>(A, S, s_tok, s_row, wrow0, n0, off, c0, crows); break;
    }
  }
}

}  // namespace

int64_t grouped_ad32_rows(int64_t rows_total) { return rows_total + GCH; }

hipError_t launch_route_topk(const int32_t *ids, int64_t rows_total,
                             int64_t n_experts, int64_t top_k, int32_t *counts,
                             int32_t *offsets, int32_t *rows,
                             const uint16_t *ad, int64_t k, float *ad32t,
                             float *y, int64_t n, hipStream_t stream) {
  hipLaunchKernelGGL(k_route, dim3((unsigned)n_experts), dim3(RT), 0, stream,
                     ids, (int)rows_total, (int)n_experts, (int)top_k, counts,
                     offsets, rows, ad, (int)(k / QK), ad32t,
                     (int)grouped_ad32_rows(rows_total), y, (int)n);
  return hipGetLastError();
}

hipError_t launch_grouped_w4a8(const int8_t *aq, const float *ad32t,
                               int64_t rows_total, int64_t top_k,
                               const uint8_t *wq4, const uint16_t *wd,
                               int64_t n_experts, int64_t n, int64_t k,
                               const int32_t *counts, const int32_t *offsets,
                               const int32_t *rows, float *y,
                               hipStream_t stream) {
  const int64_t tiles_n = (n + GBN - 1) / GBN;
  hipLaunchKernelGGL(k_grouped_w4a8, dim3((unsigned)(n_experts * tiles_n)),
                     dim3(GT), 0, stream, aq, ad32t,
                     (int)grouped_ad32_rows(rows_total), (int)top_k, wq4, wd,
                     (int)n_experts, (int)n, (int)k, counts, offsets, rows, y);
  return hipGetLastError();
}


// ------------------------------------------------------- grouped decode GEMV --
// The decode case of the grouped W4A8 GEMM (a few tokens): the pages run it on
// the host CPU ("A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB
// 2011 GPU", Method 1: CPU decode from RAM with 4-bit weights); here it stays
// on the GPU, shaped like the thin-M Q8_0 GEMV: HBM-bound, v_dot4 instead of
// MFMA, and no routing pass.
//
// One workgroup of 4 waves per (routed row, 32-column tile).  The workgroup
// of row r reads every routed expert id (at most 128) and ranks r among the
// rows routed to the same expert: the workgroup of each even-ranked row
// computes that row and the next one of the same expert, and the others exit
// at once.  An expert's weights thus leave HBM once per pair of its rows
// (repeat reads mostly hit the MALL), and no workgroup does more than two
// rows.  Every lane issues all of its loads at once: for lane l, group l (then
// l + 64, ...) of each row's Q8_0 activation row (32 bytes + scale, from L2),
// the fp16 scales, and the same group of each of the wave's 8 weight columns
// (16 packed bytes = the group's 32 codes; one coalesced 1 KB wave load per
// column and 64 groups).  The lane unpacks the codes to int8 (c - 8), forms
// the exact int32 block dot (8 v_dot4) and accumulates P * (da * dw) with one
// fma (the fp16 x fp16 product is exact in fp32); each column is then reduced
// over the wave in a fixed order.  Rows with an invalid expert id are written
// as zeros by their own workgroup.
namespace {

constexpr int GV_CPW = 8;     // weight columns per wave (the column reduction assumes 8)
constexpr int GV_WAVES = 4;
constexpr int GV_COLS = GV_CPW * GV_WAVES;  // columns per workgroup
constexpr int GV_ROWS = 2;    // routed rows per pass over the weights
constexpr int GV_MAX_ROWS = 128;

// (c + 0x78) ^ 0x80 maps each nibble code c (0..15, in a byte) to the int8
// value c - 8 with no carry between bytes.
__device__ __forceinline__ int32_t w4_lo(uint32_t p) {
  return (int32_t)(((p & 0x0f0f0f0fu) + 0x78787878u) ^ 0x80808080u);
}
__device__ __forceinline__ int32_t w4_hi(uint32_t p) {
  return (int32_t)((((p >> 4) & 0x0f0f0f0fu) + 0x78787878u) ^ 0x80808080u);
}

// Reduces eight per-lane partial sums v[0..7] (one per column) over the 64
// lanes in a fixed order.  Three exchange steps halve the columns each lane
// carries (lanes l and l ^ 32 split columns 0..3 / 4..7, then l ^ 16 and l ^ 8
// split again), so that lane l ends with column (l >> 3) summed over 8 lanes;
// three DPP steps then sum the lanes that differ in bits 0..2.  The result is
// valid in the lanes with (l & 7) == 0.
__device__ __forceinline__ float reduce_columns8(const float (&v)[8], int lane) {
  const bool u32 = (lane & 32) != 0, u16 = (lane & 16) != 0, u8 = (lane & 8) != 0;
  float v4[4], v2[2];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float keep = u32 ? v[q + 4] : v[q];
    const float send = u32 ? v[q] : v[q + 4];
    v4[q] = keep + __shfl_xor(send, 32);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float keep = u16 ? v4[q + 2] : v4[q];
    const float send = u16 ? v4[q] : v4[q + 2];
    v2[q] = keep + __shfl_xor(send, 16);
  }
  float s;
  {
    const float keep = u8 ? v2[1] : v2[0];
    const float send = u8 ? v2[0] : v2[1];
    s = keep + __shfl_xor(send, 8);
  }
  s += bits_to_float(__builtin_amdgcn_mov_dpp(__builtin_bit_cast(int32_t, s), 0xb1, 0xf, 0xf, false));   // lane ^ 1
  s += bits_to_float(__builtin_amdgcn_mov_dpp(__builtin_bit_cast(int32_t, s), 0x4e, 0xf, 0xf, false));   // lane ^ 2
  s += bits_to_float(__builtin_amdgcn_mov_dpp(__builtin_bit_cast(int32_t, s), 0x141, 0xf, 0xf, false));  // half-row mirror
  return s;
}

// Takes the lowest set row of the 128-row mask (m0: rows 0..63, m1: 64..127)
// out of it; -1 when the mask is empty.
__device__ __forceinline__ int pop_row(uint64_t &m0, uint64_t &m1) {
  if (m0) {
    const int r = __builtin_ctzll(m0);
    m0 &= m0 - 1;
    return r;
  }
  if (m1) {
    const int r = 64 + __builtin_ctzll(m1);
    m1 &= m1 - 1;
    return r;
  }
  return -1;
}

// (no __restrict__ on the inputs: with it the compiler may move loads across
// the memory clobbers that fix their issue order)
__global__ __launch_bounds__(64 * GV_WAVES) void k_grouped_gemv(
    const int8_t *aq, const uint16_t *ad, const int32_t *ids, int rows_total,
    int top_k, const uint8_t *wq4, const uint16_t *wd, int n_experts, int n,
    int k, float *y) {
  const int tiles = (n + GV_COLS - 1) / GV_COLS;
  const int r = blockIdx.x / tiles;           // routed row t * top_k + j
  const int tn = blockIdx.x - r * tiles;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform
  const int c0 = tn * GV_COLS + wave * GV_CPW;
  const int e = ids[r];
  const int id0 = lane < rows_total ? ids[lane] : -1;
  const int id1 = lane + 64 < rows_total ? ids[lane + 64] : -1;
  if (e < 0 || e >= n_experts) {
    if (lane < GV_CPW && c0 + lane < n) y[(int64_t)r * n + c0 + lane] = 0.0f;
    return;
  }
  uint64_t m0 = __ballot(id0 == e), m1 = __ballot(id1 == e);
  // rank of row r among the rows routed to expert e; the workgroup of every
  // GV_ROWS-th of them computes it and the next GV_ROWS - 1, the others exit
  const uint64_t below0 = r < 64 ? m0 & ((1ull << r) - 1) : m0;
  const uint64_t below1 = r < 64 ? 0ull : m1 & ((1ull << (r - 64)) - 1);
  const int rank = __builtin_popcountll(below0) + __builtin_popcountll(below1);
  if (rank % GV_ROWS != 0) return;
  m0 &= ~below0;  // row r is now the lowest row left
  m1 &= ~below1;
  const int nbk = k / QK;
  const int64_t wrow0 = (int64_t)e * n;

  {
    int rr[GV_ROWS];
#pragma unroll
    for (int j = 0; j < GV_ROWS; ++j) rr[j] = pop_row(m0, m1);
    float acc[GV_ROWS][GV_CPW];
#pragma unroll
    for (int j = 0; j < GV_ROWS; ++j)
#pragma unroll
      for (int q = 0; q < GV_CPW; ++q) acc[j][q] = 0.0f;

    for (int g0 = 0; g0 < nbk; g0 += 64) {
      const int b = g0 + lane;
      const bool ok = b < nbk;
      const int bb = ok ? b : 0;  // lanes past k re-read group 0 and add zero
      // every load is issued before any is waited on: first the activation
      // groups and all scales (L2), then the weight groups (HBM)
      const uint32_t gofs = (uint32_t)bb;
      i32x4 a0[GV_ROWS], a1[GV_ROWS];
      uint16_t dah[GV_ROWS];
#pragma unroll
      for (int j = 0; j < GV_ROWS; ++j) {
        // an absent second row re-reads the first row's token
        const int t = (rr[j] >= 0 ? rr[j] : rr[0]) / top_k;
        const int8_t *arow = aq + (int64_t)t * k;
        a0[j] = *reinterpret_cast<const i32x4 *>(arow + 32u * gofs);
        a1[j] = *reinterpret_cast<const i32x4 *>(arow + 32u * gofs + 16u);
        dah[j] = ad[(int64_t)t * nbk + gofs];
      }
      uint16_t dwh[GV_CPW];
#pragma unroll
      for (int q = 0; q < GV_CPW; ++q) dwh[q] = wd[(wrow0 + min(c0 + q, n - 1)) * nbk + gofs];
      __asm__ volatile("" ::: "memory");  // (keeps this issue order)
      i32x4 w[GV_CPW];
#pragma unroll
      for (int q = 0; q < GV_CPW; ++q) {
        const int64_t col = wrow0 + min(c0 + q, n - 1);
        w[q] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(wq4 + col * (k / 2) + 16u * gofs));
      }
      // all of this pass's loads are in flight before any of them is waited on
      __asm__ volatile("" ::: "memory");
      float da[GV_ROWS];
#pragma unroll
      for (int j = 0; j < GV_ROWS; ++j) da[j] = ok ? half_bits_to_float(dah[j]) : 0.0f;
      const bool more = rr[1] >= 0;  // wave-uniform
#pragma unroll
      for (int q = 0; q < GV_CPW; ++q) {
        // elements 0..15 of the group pair with the low nibbles, 16..31 with
        // the high nibbles; each column is unpacked once for both rows
        const int32_t l0 = w4_lo((uint32_t)w[q].x), l1 = w4_lo((uint32_t)w[q].y);
        const int32_t l2 = w4_lo((uint32_t)w[q].z), l3 = w4_lo((uint32_t)w[q].w);
        const int32_t h0 = w4_hi((uint32_t)w[q].x), h1 = w4_hi((uint32_t)w[q].y);
        const int32_t h2 = w4_hi((uint32_t)w[q].z), h3 = w4_hi((uint32_t)w[q].w);
        const float dw = half_bits_to_float(dwh[q]);
#pragma unroll
        for (int j = 0; j < GV_ROWS; ++j) {
          if (j == 0 || more) {
            int32_t p = 0;
            p = dot4_i8(a0[j].x, l0, p);
            p = dot4_i8(a0[j].y, l1, p);
            p = dot4_i8(a0[j].z, l2, p);
            p = dot4_i8(a0[j].w, l3, p);
            p = dot4_i8(a1[j].x, h0, p);
            p = dot4_i8(a1[j].y, h1, p);
            p = dot4_i8(a1[j].z, h2, p);
            p = dot4_i8(a1[j].w, h3, p);
            acc[j][q] = fmaf((float)p, da[j] * dw, acc[j][q]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < GV_ROWS; ++j) {
      if (rr[j] < 0) break;  // wave-uniform
      const float v = reduce_columns8(acc[j], lane);
      const int c = c0 + (lane >> 3);
      if ((lane & 7) == 0 && c < n) y[(int64_t)rr[j] * n + c] = v;
    }
  }
}

}  // namespace

bool grouped_gemv_supported(int64_t rows_total, int64_t k) {
  // a few routed rows (decode): each workgroup checks every routed id
  (void)k;
  return rows_total <= GV_MAX_ROWS;
}

hipError_t launch_grouped_gemv(const int8_t *aq, const uint16_t *ad,
                               const int32_t *ids, int64_t rows_total,
                               int64_t top_k, const uint8_t *wq4,
                               const uint16_t *wd, int64_t n_experts, int64_t n,
                               int64_t k, float *y, hipStream_t stream) {
  const int64_t tiles = (n + GV_COLS - 1) / GV_COLS;
  hipLaunchKernelGGL(k_grouped_gemv, dim3((unsigned)(rows_total * tiles)), dim3(64 * GV_WAVES),
                     0, stream, aq, ad, ids, (int)rows_total, (int)top_k, wq4, wd,
                     (int)n_experts, (int)n, (int)k, y);
  return hipGetLastError();
}

}  // namespace bqi
