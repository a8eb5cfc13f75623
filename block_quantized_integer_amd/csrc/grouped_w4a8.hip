// grouped_w4a8.hip -- expert routing and the grouped 4-bit-weight x 8-bit-
// activation GEMM: the "grouped 4-bit GEMM for MoE routing" of "A 35B
// Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU" (gist.science
// summary, Method 1) with its group-wise symmetric 4-bit weights and 8-bit
// activations (Method 2).  The page's decode kernel widens 4-bit x 8-bit
// products with SSSE3 pmaddubsw; here the nibbles are unpacked in registers
// straight into int8 MFMA operands.
//
// Routing (k_route): one workgroup of 1024 threads per expert.  Each thread
// owns a contiguous slice of 8 routed ids (two 16-byte loads), counts the
// valid ids below the expert (its offset) and equal to it, and one workgroup
// scan (DPP within each wave, then the 16 wave totals through LDS) orders the
// matches, so rows come out in increasing row order.  Up to 8192 routed rows
// this is a single pass over ids held in registers; beyond, a counting pass
// and a placing pass run chunk by chunk.  Deterministic.  The same pass
// writes zeros to the output rows of invalid ids.
//
// GEMM (k_grouped_w4a8): one workgroup of 4 waves per (expert, 128-column
// tile), three per CU, for an expert's first 64 routed rows; its further rows
// (up to 256 experts) go in 16-row pieces to more workgroups, which split K
// over their waves.  The weights are the MFMA's A operand and the gathered
// activation rows its B operand (details below).
// The products run on v_mfma_i32_32x32x32_i8 (one instruction = one 32x32
// tile for exactly one group).  Per group a lane unpacks its 16 codes (low or
// high nibbles by lane half) into the int8 values 16*(c - 8) with a shift, a
// mask and an xor; the factor 16 is folded into the weight scale.  The scale
// epilogue is the one of the Q8_0 MFMA GEMM (one rounding per term).
#include <algorithm>

#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

namespace {

// ---------------------------------------------------------------- routing --
constexpr int RT = 1024;          // threads per routing workgroup
constexpr int RPT = 8;            // ids per thread per pass
constexpr int RCHUNK = RT * RPT;  // ids per pass

// Inclusive sum over the 64 lanes of a wave, with DPP: within each 16-lane
// row (shifts of 1, 2, 4, 8; lanes shifted in from outside the row add 0),
// then the end of row 0 / 2 into rows 1 / 3 and the end of row 1 into rows 2
// and 3.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive workgroup scan of one int per thread (RT threads); `total` gets
// the sum.  Contains two barriers.
__device__ __forceinline__ int route_scan(int v, int *s_tmp, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_scan_incl(v);
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

// Rows of an expert that its own GEMM workgroups take; the rest go to the
// split pieces of SPLIT_ROWS rows (see the grouped GEMM below).
constexpr int SPLIT_FIRST = 64;
constexpr int SPLIT_ROWS = 16;
constexpr int SPLIT_MAX_EXPERTS = 256;  // up to 4 experts per lane of one wave

__device__ __forceinline__ int split_pieces(int cnt) {
  return cnt > SPLIT_FIRST ? (cnt - SPLIT_FIRST + SPLIT_ROWS - 1) / SPLIT_ROWS : 0;
}

__global__ __launch_bounds__(RT) void k_route(
    const int32_t *__restrict__ ids, int rows_total, int n_experts, int top_k,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ rows, float *__restrict__ y, int n) {
  __shared__ int s_tmp[RT / 64];
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
    if (r0 + RPT <= rows_total && ((uintptr_t)ids & 15) == 0) {
#pragma unroll
      for (int j = 0; j < RPT; j += 4) {
        const i32x4 q = *reinterpret_cast<const i32x4 *>(ids + r0 + j);
        v[j] = q.x; v[j + 1] = q.y; v[j + 2] = q.z; v[j + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < RPT; ++j) v[j] = r0 + j < rows_total ? ids[r0 + j] : -1;
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
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
        ++pos;
      }
      // invalid ids: workgroup (row mod E) zeroes the output row
      const int r = r0 + j;
      if (y != nullptr && r < rows_total && (v[j] < 0 || v[j] >= n_experts) &&
          r % n_experts == e)
        for (int c = 0; c < n; ++c) y[(int64_t)r * n + c] = 0.0f;
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

  // pass 2: place the matches in increasing row order
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
        ++pos;
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
// One workgroup of GW = 4 waves per (expert, 128-column tile).  The MFMA runs with the weights as the A operand (lane = output
// column, K half) and the gathered activation rows as the B operand (lane =
// routed row), so in the output a lane holds one routed row and its registers
// hold 16 columns: the activation scale is lane-uniform (one per row tile and
// group) and the weight scales, one per register, are shared by every row
// tile of the wave.  Routed rows are taken 64 at a time (two 32-row tiles).
//
// Three workgroups share a CU (12 waves, 168 VGPRs each), so the MoE
// workload's 768 (expert, column tile) units run in one round.  Workgroup
// blockIdx takes expert blockIdx / column_tiles and, up to 256 experts, only
// its first 64 routed rows.  The rows past them form pieces of 16 rows; each
// 32-column strip of a piece is an item for the workgroups launched after
// the (expert, column tile) ones, which start as those finish.  An item's
// four waves take one quarter of K each over the same 16 rows and 32 columns
// and add their partial sums through LDS in wave order, so a heavy expert's
// extra rows are spread over many CUs instead of running after its first 64
// on the same workgroups.  (Ordering the experts by routed-row count made no
// difference once no workgroup takes more than 64 rows.)  Past 256 experts a
// workgroup takes all its expert's rows, 64 at a time; an expert with more
// rows streams its weights again for the next 64 (mostly from the Infinity
// Cache).
//
// Stages of GNB = 4 groups (128 K elements) go through two LDS buffers: the
// loads of stage s+1 are issued before the compute of stage s.  Per stage
// and thread: two 16-byte direct loads of packed weights and R of gathered
// activation rows (the chunk's 32R rows), and 2-byte direct loads of
// activation scales (ceil(R/2)) and weight scales (two), zero-extended into
// 4-byte slots.  All of them go through inline asm (the compiler does not
// count them) and are waited for explicitly; none of them writes a register.  After
// the stage barrier each wave converts, in place, the 128 weight scales that
// it alone reads (its 32 columns x 4 groups) to fp32 times 1/16 (the unpack
// factor), 0 for groups past k; LDS operations of one wave complete in order,
// so its later reads see the converted values without another barrier.
//
// When k is a multiple of 1024 and both scale arrays are 16-byte aligned
// (PAIRED), the scales instead arrive two stages at a time: each weight
// column's and activation row's 8 fp16 scales (16 bytes) with one direct load
// per lane, three wave loads per workgroup every other stage in place of
// twelve 2-byte loads every stage, into two pair buffers; the weight scales
// are converted from there into the same fp32 slots, and the activation
// scales are read from there.  A CU takes a 64-lane load instruction only
// every ~32-38 cycles whatever its width, so this is ~10% of the MoE call.
constexpr int GW = 4;              // waves per workgroup
constexpr int GT = GW * 64;        // threads per workgroup
constexpr int GBN = GW * 32;       // output columns per workgroup (32 per wave)
constexpr int GNB = 4;             // 32-element groups per stage
constexpr int GBK = GNB * QK;      // activation bytes per row per stage
constexpr int GRT = 2;             // 32-row tiles per chunk
constexpr int GCH = 32 * GRT;      // routed rows per chunk
constexpr int GNS = 2;             // LDS stage buffers (the next stage in flight)
constexpr int G_W_LOADS = GBN * GNB / GT;          // weight chunks per thread and stage (2)
// A chunk of R row tiles loads only its 32R rows: R activation chunks and
// ceil(R/2) activation-scale slots per thread and stage.
template <int R> constexpr int g_a_loads() { return 32 * R * (GBK / 16) / GT; }
template <int R> constexpr int g_as_loads() { return (32 * R * GNB + GT - 1) / GT; }
constexpr int G_AS_ROWS = 64;                      // rows of activation-scale slots (>= the most loaded)
constexpr int G_WS_LOADS = GBN * GNB / 64 / GW;    // weight-scale slots per thread and stage (2)

static_assert(G_W_LOADS == 2 && G_WS_LOADS == 2, "load mapping");
static_assert(g_a_loads<GRT>() == GRT && g_as_loads<GRT>() * GT / GNB <= G_AS_ROWS, "load mapping");
static_assert(G_AS_ROWS >= GCH, "activation-scale slots cover the chunk");
static_assert(SPLIT_FIRST == GCH && 4 * SPLIT_ROWS == GCH,
              "an expert's own workgroups take one chunk; a split piece stages four quarters of 16 rows");

struct GBuf {
  uint8_t w[GBN * GNB * 16];    // packed weights: [column][slot], slot = group ^ wswz(column)
  int8_t a[GCH * GBK];          // activation rows: [row][slot], slot = chunk ^ aswz(row)
  uint32_t as[G_AS_ROWS * GNB]; // activation scales, fp16 bits zero-extended: [row][group]
  uint32_t ws[GNB][GBN];        // weight scales: fp16 bits zero-extended as loaded, then
                                // converted in place to fp32 / 16 (0 past k): [group][column]
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

// The MFMA work of one stage for one wave: its 32 columns x R 32-row tiles
// over the stage's GNB groups.  Steps u = g * R + t run as a pipeline of
// depth one (tile u's MFMA is issued before tile u-1's epilogue, into the
// other of two result sets), each step pinned in place by empty asm
// statements as in the Q8_0 GEMM.  Output register r of tile t in lane L is
// column 8(r/4) + 4(L/32) + r%4 of the wave's columns, routed row 32t + L%32
// of the chunk.  Per term: t_r = fma(F_r, da, -1.5*2^23*da) = round(da * 16P)
// with da the lane's activation scale, then acc = fma(t_r, dw_r / 16, acc).
template <int R, bool PAIRED>
__device__ __forceinline__ void grouped_stage(const GBuf &B, const uint16_t *ra, int wave, int lane_in,
                                              const i32x16 &seed, f32x16 (&acc)[R]) {
  // the lane index is laundered so that the LDS addresses below are rebuilt
  // each stage instead of being hoisted out of the stage loop into registers
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, h = lane >> 5;
  const int shl = h ? 0 : 4;
  const int col = wave * 32 + l32;
  // activation scales of this stage's groups for the lane's row of each tile
  float da[R][GNB];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    if constexpr (PAIRED) {
      const uint2 v = *reinterpret_cast<const uint2 *>(ra + 2 * GNB * (32 * t + l32));
      da[t][0] = half_bits_to_float((uint16_t)(v.x & 0xffffu));
      da[t][1] = half_bits_to_float((uint16_t)(v.x >> 16));
      da[t][2] = half_bits_to_float((uint16_t)(v.y & 0xffffu));
      da[t][3] = half_bits_to_float((uint16_t)(v.y >> 16));
    } else {
      const i32x4 v = *reinterpret_cast<const i32x4 *>(&B.as[(32 * t + l32) * GNB]);
      da[t][0] = half_bits_to_float((uint16_t)v.x);
      da[t][1] = half_bits_to_float((uint16_t)v.y);
      da[t][2] = half_bits_to_float((uint16_t)v.z);
      da[t][3] = half_bits_to_float((uint16_t)v.w);
    }
    // converted once here: left to itself the compiler folds the conversion
    // into each epilogue fma as v_fma_mix_f32, which issues at a lower rate
    asm volatile("" : "+v"(da[t][0]), "+v"(da[t][1]), "+v"(da[t][2]), "+v"(da[t][3]));
  }
  auto read_w = [&](int g) {
    return *reinterpret_cast<const i32x4 *>(&B.w[col * (GNB * 16) + 16 * wswz(col, g)]);
  };
  // the swizzle of row 32t + l32 does not depend on t, so one lane offset per
  // group serves every tile (the tile adds 32 * GBK bytes)
  const int aswz_l = (l32 >> 1) & 7;
  auto read_b = [&](int g, int t) {
    return *reinterpret_cast<const i32x4 *>(
        &B.a[32 * GBK * t + l32 * GBK + 16 * ((2 * g + h) ^ aswz_l)]);
  };
  auto read_dw = [&](int g, float (&dst)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(&B.ws[g][wave * 32 + 8 * q + 4 * h]);
      dst[4 * q + 0] = v.x;
      dst[4 * q + 1] = v.y;
      dst[4 * q + 2] = v.z;
      dst[4 * q + 3] = v.w;
    }
  };

  i32x4 wf = unpack_w4x16(read_w(0), shl);
  i32x4 bf[R];
#pragma unroll
  for (int t = 0; t < R; ++t) bf[t] = read_b(0, t);
  i32x4 wraw_n;
  float dwc[16];  // weight scales of the epilogue's group
  read_dw(0, dwc);
  i32x16 dres[2];
  auto epilogue = [&](const i32x16 &d, int u) {
    const int g = u / R, t = u % R;
    const float s = da[t][g], ncd = -MAGIC_F * s;  // exact
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float tt = fmaf(bits_to_float(d[r]), s, ncd);
      acc[t][r] = fmaf(tt, dwc[r], acc[t][r]);
    }
  };
  // Step u = (g, t): the MFMA of (g, t), the epilogue of step u-1, then tile
  // t's activation fragment of group g+1 is read into the register the MFMA
  // has just consumed, and (at t == 0) the next group's weight fragment and
  // this group's weight scales; at t == R-1 the next group's weight fragment
  // is unpacked.
#pragma unroll
  for (int u = 0; u < GNB * R; ++u) {
    const int g = u / R, t = u % R;
    asm volatile("" : "+v"(wf), "+v"(bf[t]));
    dres[u & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf, bf[t], seed, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (u > 0) {
      epilogue(dres[(u - 1) & 1], u - 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
      asm volatile("" : "+v"(acc[(u - 1) % R]), "+v"(dres[u & 1]));
    } else {
      asm volatile("" : "+v"(dres[u & 1]));
    }
    // the epilogue just run was the last of group g-1: group g's weight
    // scales replace its (first used at the next step)
    if (t == 0 && g > 0) read_dw(g, dwc);
    if (g + 1 < GNB) {
      bf[t] = read_b(g + 1, t);
      if (t == 0) wraw_n = read_w(g + 1);
      if (t == R - 1) wf = unpack_w4x16(wraw_n, shl);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  epilogue(dres[(GNB * R - 1) & 1], GNB * R - 1);
}

// A chunk of at most 16 rows (the last rows of an expert): the same work on
// 16-row tiles, as two v_mfma_i32_16x16x32_i8 per group (one per 16 of the
// wave's 32 columns), which halves the epilogue against a padded 32-row
// tile.  In lane L the A fragment is weight column 16 ct + L%16 and the B
// fragment routed row L%16, both over K elements 8 (L/16) .. +7 of the group
// (bytes 8 ((L/16) % 2) .. +7 of the packed group, low nibbles for L < 32);
// output register r of lane L is column 16 ct + 4 (L/16) + r, row L%16.  The
// int32 block dots and the epilogue per output are those of the 32-row
// tile, so the results are bit-identical to it.
__device__ __forceinline__ int64_t unpack_w4x8(int64_t p, int shl) {
  const uint32_t lo = (((uint32_t)p << shl) & 0xf0f0f0f0u) ^ 0x80808080u;
  const uint32_t hi = (((uint32_t)((uint64_t)p >> 32) << shl) & 0xf0f0f0f0u) ^ 0x80808080u;
  return (int64_t)((uint64_t)lo | ((uint64_t)hi << 32));
}

// arow0 (a multiple of 16): the first of the 16 staged rows that the wave
// reads.
template <bool PAIRED>
__device__ __forceinline__ void grouped_stage_half(const GBuf &B, const uint16_t *ra, int wave, int lane_in,
                                                   int arow0, const i32x4 &seed4, f32x4 (&acc)[2]) {
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int l16 = lane & 15, kg = lane >> 4;
  const int shl = (kg >> 1) ? 0 : 4;
  const int aswz_l = (l16 >> 1) & 7;  // aswz of row arow0 + l16
  const int arow = arow0 + l16;
  float da[GNB];
  if constexpr (PAIRED) {
    const uint2 v = *reinterpret_cast<const uint2 *>(ra + 2 * GNB * arow);
    da[0] = half_bits_to_float((uint16_t)(v.x & 0xffffu));
    da[1] = half_bits_to_float((uint16_t)(v.x >> 16));
    da[2] = half_bits_to_float((uint16_t)(v.y & 0xffffu));
    da[3] = half_bits_to_float((uint16_t)(v.y >> 16));
    asm volatile("" : "+v"(da[0]), "+v"(da[1]), "+v"(da[2]), "+v"(da[3]));
  } else {
    const i32x4 v = *reinterpret_cast<const i32x4 *>(&B.as[arow * GNB]);
    da[0] = half_bits_to_float((uint16_t)v.x);
    da[1] = half_bits_to_float((uint16_t)v.y);
    da[2] = half_bits_to_float((uint16_t)v.z);
    da[3] = half_bits_to_float((uint16_t)v.w);
    asm volatile("" : "+v"(da[0]), "+v"(da[1]), "+v"(da[2]), "+v"(da[3]));
  }
  auto read_w = [&](int g, int ct) {
    const int col = wave * 32 + 16 * ct + l16;
    return *reinterpret_cast<const int64_t *>(&B.w[col * (GNB * 16) + 16 * wswz(col, g) + 8 * (kg & 1)]);
  };
  auto read_b = [&](int g) {
    return *reinterpret_cast<const int64_t *>(
        &B.a[arow * GBK + 16 * ((2 * g + (kg >> 1)) ^ aswz_l) + 8 * (kg & 1)]);
  };
#pragma unroll
  for (int g = 0; g < GNB; ++g) {
    const int64_t b = read_b(g);
    const i32x4 d0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(unpack_w4x8(read_w(g, 0), shl), b, seed4, 0, 0, 0);
    const i32x4 d1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(unpack_w4x8(read_w(g, 1), shl), b, seed4, 0, 0, 0);
    const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&B.ws[g][wave * 32 + 4 * kg]);
    const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&B.ws[g][wave * 32 + 16 + 4 * kg]);
    const float sa = da[g], ncd = -MAGIC_F * sa;  // exact
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      acc[0][r] = fmaf(fmaf(bits_to_float(d0[r]), sa, ncd), w0[r], acc[0][r]);
      acc[1][r] = fmaf(fmaf(bits_to_float(d1[r]), sa, ncd), w1[r], acc[1][r]);
    }
  }
}

struct GArgs {
  const int8_t *aq;
  const uint16_t *ad;
  int top_k;
  const uint8_t *wq4;
  const uint16_t *wd;
  int n, k;
  float *y;
};

// The work shapes of grouped_chunk.
enum GMode {
  G_FULL = 0,   // up to 32 R rows x the workgroup's 128 columns, 32-row tiles
  G_HALF = 1,   // up to 16 rows x 128 columns, 16-row tiles (R == 1)
  G_SPLIT = 2,  // up to 16 rows x 32 columns, K split four ways over the waves
};

// One chunk of routed rows of expert e from column n0 on: the whole K
// pipeline, then the stores.
//
// G_SPLIT: every wave computes the same 32 columns and 16 rows over its own
// quarter of K (qg groups, a multiple of GNB, from group qg * wave on) on
// 16-row tiles.  The stage buffers keep their layout: wave w's 32 columns
// (columns 32w .. 32w+31 of the buffer) and staged rows 16w .. 16w+15 hold
// the workgroup's columns and rows over quarter w, so each wave loads exactly
// what it reads.  The four partial sums are added through LDS in wave order.
template <int R, int MODE, bool PAIRED>
__device__ __forceinline__ void grouped_chunk(const GArgs &A, GBuf (&S)[GNS], uint16_t *raw,
                                              const int *s_tok, const int *s_row, int e, int n0,
                                              int crows) {
  constexpr bool HALF = MODE != G_FULL;   // 16-row tiles
  constexpr bool SPLIT = MODE == G_SPLIT;
  static_assert(MODE == G_FULL || (MODE == G_HALF && R == 1) || (SPLIT && R == 2),
                "16-row tiles stage one 32-row tile's loads, split chunks four 16-row quarters");
  const int n = A.n, k = A.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nbk = k / QK;
  const int qg = SPLIT ? GNB * ((nbk + 4 * GNB - 1) / (4 * GNB)) : 0;
  const int gq0 = qg * wave_u;  // first group of the wave's loads and reads
  const int stages = SPLIT ? qg / GNB : (nbk + GNB - 1) / GNB;
  const int kh = k / 2;

  i32x16 seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = MAGIC_BITS;
  asm volatile("" : "+v"(seed));  // kept resident, not rebuilt per stage
  i32x4 seed4 = {MAGIC_BITS, MAGIC_BITS, MAGIC_BITS, MAGIC_BITS};
  asm volatile("" : "+v"(seed4));

  // per-lane load coordinates, fixed for the chunk
  // weights: chunk e = 64 (2w + q) + L -> column e/4, slot e%4 (group slot ^ wswz)
  // (split: the wave's buffer columns 32w.. are the workgroup's columns over
  // its quarter of K)
  int w_off[G_W_LOADS], w_g[G_W_LOADS];
#pragma unroll
  for (int q = 0; q < G_W_LOADS; ++q) {
    const int ce = 64 * (G_W_LOADS * wave + q) + lane;
    const int c = ce >> 2;
    w_g[q] = (ce & 3) ^ ((c >> 2) & 3);
    w_off[q] = min(n0 + (SPLIT ? (c & 31) : c), n - 1) * kh + 16 * gq0;
  }
  // activations: chunk e = 64 (3w + q) + L -> row e/8, slot e%8 (chunk slot
  // ^ aswz); 32-bit offsets from the activation base (the ABI layer
  // guarantees n_tokens * k < 2^31)
  constexpr int NA = g_a_loads<R>(), NAS = g_as_loads<R>();
  int a_row[NA], a_c[NA];
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    const int ce = 64 * (NA * wave + q) + lane;
    const int r = ce >> 3;
    a_c[q] = 16 * ((ce & 7) ^ ((r >> 1) & 7)) + 32 * gq0;  // split: rows 16w.. of quarter w
    a_row[q] = s_tok[r] * k;
  }
  // activation scales: slot e = 64 (2w + q) + L -> row e/4 (clamped to the
  // chunk's rows), group e%4; element offsets from the scale base
  int as_row[NAS];
#pragma unroll
  for (int q = 0; q < NAS; ++q) {
    const int ce = 64 * (NAS * wave + q) + lane;
    as_row[q] = s_tok[min(ce >> 2, GCH - 1)] * nbk + (ce & 3) + gq0;
  }
  // weight scales: slot e = 64 (2w + q) + L -> group e/128 (= w), column
  // e%128; element offsets from the expert's scale base (split: buffer column
  // c is column c%32 over quarter c/32, which differs between lanes)
  int ws_off[G_WS_LOADS], ws_q0[G_WS_LOADS];
#pragma unroll
  for (int q = 0; q < G_WS_LOADS; ++q) {
    const int ce = 64 * (G_WS_LOADS * wave + q) + lane;
    const int c = ce & (GBN - 1);
    ws_q0[q] = SPLIT ? qg * (c >> 5) : 0;
    ws_off[q] = min(n0 + (SPLIT ? (c & 31) : c), n - 1) * nbk + (ce >> 7) + ws_q0[q];
  }
  const uint8_t *wq_e = A.wq4 + (int64_t)e * n * kh;
  const uint16_t *wd_e = A.wd + (int64_t)e * n * nbk;

  // Issue stage s into buffer s % GNS.  Groups past the last one re-read the
  // last group (their scales become 0).
  auto issue = [&](int s) {
    const int g0 = s * GNB;
    const bool full = gq0 + g0 + GNB <= nbk;  // uniform in the wave
    GBuf &D = S[s % GNS];
    const uint8_t *wbase = wq_e + 16 * g0;
#pragma unroll
    for (int q = 0; q < G_W_LOADS; ++q) {
      const int off = w_off[q] + 16 * (full ? w_g[q] : min(w_g[q], nbk - 1 - g0 - gq0));
      const uint32_t lds = lds_addr(&D.w[1024 * (G_W_LOADS * wave_u + q)]);
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(off), "s"(wbase), "{m0}"(lds) : "memory");
    }
    const int8_t *abase = A.aq + 32 * g0;
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const int off = a_row[q] + (full ? a_c[q] : min(a_c[q], k - 16 - 32 * g0));
      const uint32_t lds = lds_addr(&D.a[1024 * (NA * wave_u + q)]);
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(off), "s"(abase), "{m0}"(lds) : "memory");
    }
    if constexpr (PAIRED) return;
    const uint16_t *asbase = A.ad + g0;
#pragma unroll
    for (int q = 0; q < NAS; ++q) {
      const int ce = 64 * (NAS * wave + q) + lane;
      const int off = as_row[q] + (full ? 0 : min(0, nbk - 1 - g0 - (ce & 3) - gq0));
      const uint32_t lds = lds_addr(&D.as[64 * (NAS * wave_u + q)]);
      asm volatile("s_nop 0\n\tglobal_load_lds_ushort %0, %1" :: "v"(2 * off), "s"(asbase), "{m0}"(lds) : "memory");
    }
    const uint16_t *wsbase = wd_e + g0;
#pragma unroll
    for (int q = 0; q < G_WS_LOADS; ++q) {
      const int gq = wave_u;  // group of this wave's slots
      const int off = ws_off[q] + (full && !SPLIT ? 0 : min(0, nbk - 1 - g0 - gq - ws_q0[q]));
      const uint32_t lds = lds_addr(&D.ws[0][0] + 64 * (G_WS_LOADS * wave_u + q));
      asm volatile("s_nop 0\n\tglobal_load_lds_ushort %0, %1" :: "v"(2 * off), "s"(wsbase), "{m0}"(lds) : "memory");
    }
  };
  // PAIRED: the fp16 scales of a pair of stages (2 GNB groups, 16 bytes per
  // row or column) arrive with one direct load per lane into raw[pair % 2]:
  // waves 0 and 1 load the weight scales of buffer columns 64 w .. +63,
  // wave 2 those of the 64 staged activation rows (split: buffer column c and
  // staged row r belong to quarter c / 32 and r / 16).  Pair p is loaded in
  // stage 2p - 1, when every wave is past stage 2p - 2, the last reader of
  // the buffer it overwrites; its stages read it after their stage barrier.
  constexpr int RAW_A = GCH * 2 * GNB;          // halves per pair buffer of activation scales
  constexpr int RAW_W = GBN * 2 * GNB;          // halves per pair buffer of weight scales
  int raw_off = 0;
  if constexpr (PAIRED) {
    if (wave_u < 2) {
      const int c = 64 * wave_u + lane;
      raw_off = 2 * (min(n0 + (SPLIT ? (c & 31) : c), n - 1) * nbk + (SPLIT ? qg * (c >> 5) : 0));
    } else if (wave_u == 2) {
      raw_off = 2 * (s_tok[lane] * nbk + (SPLIT ? qg * (lane >> 4) : 0));
    }
  }
  auto issue_raw = [&](int pair) {
    if (wave_u < 2) {
      const uint32_t lds = lds_addr(raw + 2 * RAW_A + RAW_W * (pair & 1) + 2 * GNB * 64 * wave_u);
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(raw_off + 4 * GNB * pair), "s"(wd_e), "{m0}"(lds) : "memory");
    } else if (wave_u == 2) {
      const uint32_t lds = lds_addr(raw + RAW_A * (pair & 1));
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(raw_off + 4 * GNB * pair), "s"(A.ad), "{m0}"(lds) : "memory");
    }
  };
  // The weight scales this wave reads in stage s (its 32 columns, all
  // groups), converted in place: lane L takes column 32 w + L%32, groups
  // 2 (L/32) and 2 (L/32) + 1.
  auto convert_ws = [&](int s) {
    GBuf &D = S[s % GNS];
    const int c = wave * 32 + (lane & 31);
    if constexpr (PAIRED) {
      const uint32_t two = *reinterpret_cast<const uint32_t *>(
          raw + 2 * RAW_A + RAW_W * ((s >> 1) & 1) + 2 * GNB * c + GNB * (s & 1) + 2 * (lane >> 5));
      const int g = 2 * (lane >> 5);
      D.ws[g][c] = __builtin_bit_cast(uint32_t, half_bits_to_float((uint16_t)(two & 0xffffu)) * 0.0625f);
      D.ws[g + 1][c] = __builtin_bit_cast(uint32_t, half_bits_to_float((uint16_t)(two >> 16)) * 0.0625f);
      return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = 2 * (lane >> 5) + i;
      const uint32_t bits = D.ws[g][c];
      const float v = gq0 + s * GNB + g < nbk ? half_bits_to_float((uint16_t)bits) * 0.0625f : 0.0f;  // exact
      D.ws[g][c] = __builtin_bit_cast(uint32_t, v);
    }
  };

  f32x16 acc[R];
  f32x4 acc16[2];
  if constexpr (HALF) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc16[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  } else {
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;
  }

  // Stage s waits for its own loads (issued before stage s-1's compute); the
  // barrier then makes every wave's loads of stage s visible and frees the
  // buffer of stage s-1, which takes stage s+1's loads during this compute.
  if constexpr (PAIRED) issue_raw(0);
  issue(0);
  for (int s = 0; s < stages; ++s) {
    wait_vmcnt<0>();
    lds_barrier();
    if (s + 1 < stages) issue(s + 1);
    if constexpr (PAIRED) {
      if ((s & 1) && s + 1 < stages) issue_raw((s + 1) >> 1);
    }
    convert_ws(s);
    const uint16_t *ra = raw + RAW_A * ((s >> 1) & 1) + GNB * (s & 1);
    if constexpr (HALF)
      grouped_stage_half<PAIRED>(S[s % GNS], ra, wave, lane, SPLIT ? 16 * wave : 0, seed4, acc16);
    else
      grouped_stage<R, PAIRED>(S[s % GNS], ra, wave, lane, seed, acc);
  }

  if constexpr (SPLIT) {
    // the four quarters' partial sums, added in wave order: wave w finishes
    // outputs 2w, 2w+1 of the lane's eight (columns 16 (w/2) + 4 (L/16) +
    // 2 (w%2) + 0..1, row L%16)
    __syncthreads();  // every wave is done with the stage buffers
    f32x4 *red = reinterpret_cast<f32x4 *>(&S[0]);  // [wave][lane][2]
    red[(wave * 64 + lane) * 2 + 0] = acc16[0];
    red[(wave * 64 + lane) * 2 + 1] = acc16[1];
    __syncthreads();
    const float *redf = reinterpret_cast<const float *>(&S[0]);
    const int i0 = 2 * wave;
    float v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float sum = redf[lane * 8 + i0 + i];
#pragma unroll
      for (int w = 1; w < GW; ++w) sum += redf[(w * 64 + lane) * 8 + i0 + i];
      v[i] = sum;
    }
    const int rr = lane & 15;
    if (rr < crows) {
      float *yrow = A.y + (int64_t)s_row[rr] * n;
      const int c = n0 + 16 * (wave >> 1) + 4 * (lane >> 4) + 2 * (wave & 1);
      if (c < n) yrow[c] = v[0];
      if (c + 1 < n) yrow[c + 1] = v[1];
    }
    return;
  }
  const bool vec = (n & 3) == 0 && ((uintptr_t)A.y & 15) == 0;
  if constexpr (HALF) {
    // store: lane's routed row L%16, columns n0 + 32 wave + 16 ct + 4 (L/16) + (0..3)
    const int rr = lane & 15;
    if (rr < crows) {
      float *yrow = A.y + (int64_t)s_row[rr] * n;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int c = n0 + wave * 32 + 16 * ct + 4 * (lane >> 4);
        if (vec && c + 3 < n) {
          *reinterpret_cast<f32x4 *>(yrow + c) = acc16[ct];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (c + i < n) yrow[c + i] = acc16[ct][i];
        }
      }
    }
    return;
  }
  // store: lane's routed row 32t + L%32 of the chunk, columns
  // n0 + 32 wave + 8q + 4(L/32) + (0..3) in registers 4q .. 4q+3
  const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int rr = 32 * t + l32;
    if (rr < crows) {
      float *yrow = A.y + (int64_t)s_row[rr] * n;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = n0 + wave * 32 + 8 * q + 4 * h;
        if (vec && c + 3 < n) {
          f32x4 v;
          v.x = acc[t][4 * q + 0];
          v.y = acc[t][4 * q + 1];
          v.z = acc[t][4 * q + 2];
          v.w = acc[t][4 * q + 3];
          *reinterpret_cast<f32x4 *>(yrow + c) = v;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (c + i < n) yrow[c + i] = acc[t][4 * q + i];
        }
      }
    }
  }
}

template <bool PAIRED>
__global__ __launch_bounds__(GT, 3) void k_grouped_w4a8(
    const int8_t *__restrict__ aq, const uint16_t *__restrict__ ad, int top_k,
    const uint8_t *__restrict__ wq4, const uint16_t *__restrict__ wd,
    int n_experts, int n, int k, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ rows,
    float *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) GBuf S[GNS];
  // PAIRED: raw fp16 scales of a pair of stages, two pair buffers of the
  // activation scales [GCH][2 GNB], then two of the weight scales [GBN][2 GNB]
  __shared__ __attribute__((aligned(16))) uint16_t raw[PAIRED ? 2 * (GCH + GBN) * 2 * GNB : 8];
  __shared__ int s_tok[GCH];  // token of each staged row
  __shared__ int s_row[GCH];  // routed row (output row) of each staged row

  const int tiles_n = (n + GBN - 1) / GBN;
  const int main_wgs = n_experts * tiles_n;
  const int tid = threadIdx.x;
  const GArgs A{aq, ad, top_k, wq4, wd, n, k, y};
  const bool split = n_experts <= SPLIT_MAX_EXPERTS;

  if ((int)blockIdx.x >= main_wgs) {
    // The split pieces, numbered expert by expert: expert e's pieces follow
    // those of the experts below it.  Every wave finds them from the routed-row
    // counts alone: lane l holds experts 4l .. 4l+3, and two wave sums give,
    // per lane, the pieces and the rows of the experts up to its own.  Item t
    // is 32-column strip t % strips of piece t / strips; the workgroups past
    // the (expert, column tile) ones take items blockIdx - main_wgs, then
    // every gridDim - main_wgs further.
    const int lane = tid & 63;
    int c4[4], rsum = 0, psum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ex = 4 * lane + j;
      c4[j] = ex < n_experts ? counts[ex] : 0;
      rsum += c4[j];
      psum += split_pieces(c4[j]);
    }
    const int rinc = wave_scan_incl(rsum), pinc = wave_scan_incl(psum);
    const int strips = (n + 31) / 32;
    const int step = (int)gridDim.x - main_wgs;
    const int64_t items = (int64_t)__builtin_amdgcn_readlane(pinc, 63) * strips;
    for (int64_t t = (int)blockIdx.x - main_wgs; t < items; t += step) {
      const int piece = (int)(t / strips);
      const int strip = (int)(t - (int64_t)piece * strips);
      // the lane holding the piece's expert: the first whose running piece
      // count passes it (one exists, as piece < the wave's total)
      const int src = __builtin_ctzll(__ballot(pinc > piece));
      int pbase = __builtin_amdgcn_readlane(pinc - psum, src);
      int rbase = __builtin_amdgcn_readlane(rinc - rsum, src);
      int e = 4 * src, c = 0, i = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cj = __builtin_amdgcn_readlane(c4[j], src);
        const int pj = split_pieces(cj);
        if (c == 0 && piece < pbase + pj) {
          e = 4 * src + j;
          c = cj;
          i = piece - pbase;
        } else if (c == 0) {
          pbase += pj;
          rbase += cj;
        }
      }
      // rows of expert e start at rbase (the routed rows of the experts below
      // it); the piece is rows c0 .. c0 + crows - 1 of the expert
      const int c0 = SPLIT_FIRST + SPLIT_ROWS * i;
      const int crows = min(SPLIT_ROWS, c - c0);
      const int r0 = rbase + c0;
      // the previous item is done with s_tok, s_row and S
      __syncthreads();
      if (tid < GCH) {
        // staged row r is row r % 16 of the piece (for K quarter r / 16)
        const int rr = rows[r0 + min(tid & (SPLIT_ROWS - 1), crows - 1)];
        s_row[tid] = rr;
        s_tok[tid] = rr / top_k;
      }
      __syncthreads();
      grouped_chunk<2, G_SPLIT, PAIRED>(A, S, raw, s_tok, s_row, e, 32 * strip, crows);
    }
    return;
  }

  // With a multiple of 8 experts, the column tiles of an expert run on one
  // XCD (workgroup b runs on XCD b % 8), so its gathered activation rows
  // meet in one L2: 1% per call on the MoE workload
  int e, tn;
  if ((n_experts & 7) == 0) {
    const int b = blockIdx.x, x = b & 7, j = b >> 3;
    const int q = j / tiles_n;
    e = 8 * q + x;
    tn = j - q * tiles_n;
  } else {
    e = blockIdx.x / tiles_n;
    tn = blockIdx.x - e * tiles_n;
  }
  const int cnt = counts[e];
  if (cnt == 0) return;
  const int off = offsets[e];
  const int n0 = tn * GBN;
  // with the split pieces, rows past the first SPLIT_FIRST go to the split
  // workgroups
  const int own = split ? min(cnt, SPLIT_FIRST) : cnt;

  for (int c0 = 0; c0 < own; c0 += GCH) {
    const int crows = min(GCH, own - c0);
    // the previous chunk is done with s_tok, s_row and S (each chunk ends
    // with every load landed)
    __syncthreads();
    if (tid < GCH) {
      const int rr = rows[off + c0 + min(tid, crows - 1)];
      s_row[tid] = rr;
      s_tok[tid] = rr / top_k;
    }
    __syncthreads();
    if (crows <= 16)
      grouped_chunk<1, G_HALF, PAIRED>(A, S, raw, s_tok, s_row, e, n0, crows);
    else if (crows <= 32)
      grouped_chunk<1, G_FULL, PAIRED>(A, S, raw, s_tok, s_row, e, n0, crows);
    else
      grouped_chunk<2, G_FULL, PAIRED>(A, S, raw, s_tok, s_row, e, n0, crows);
  }
}

}  // namespace

hipError_t launch_route_topk(const int32_t *ids, int64_t rows_total,
                             int64_t n_experts, int64_t top_k, int32_t *counts,
                             int32_t *offsets, int32_t *rows, float *y, int64_t n,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_route, dim3((unsigned)n_experts), dim3(RT), 0, stream,
                     ids, (int)rows_total, (int)n_experts, (int)top_k, counts,
                     offsets, rows, y, (int)n);
  return hipGetLastError();
}

// Workgroups for the split pieces: one per item while the items fit in
// G_SPLIT_WGS (those without an item exit at once), else a loop over items.
constexpr int64_t G_SPLIT_WGS = 1536;

hipError_t launch_grouped_w4a8(const int8_t *aq, const uint16_t *ad,
                               int64_t top_k, const uint8_t *wq4,
                               const uint16_t *wd, int64_t n_experts, int64_t n,
                               int64_t k, int64_t rows_total, const int32_t *counts,
                               const int32_t *offsets, const int32_t *rows, float *y,
                               hipStream_t stream) {
  const int64_t tiles_n = (n + GBN - 1) / GBN;
  // at most rows_total / 16 pieces (each covers 16 rows past an expert's
  // first 64), each of (n + 31) / 32 strips
  const int64_t most = n_experts <= SPLIT_MAX_EXPERTS && rows_total > SPLIT_FIRST
                           ? rows_total / SPLIT_ROWS * ((n + 31) / 32)
                           : 0;
  const int64_t split_wgs = std::min(most, G_SPLIT_WGS);
  const bool paired = (k / QK) % (8 * GNB) == 0 && ((uintptr_t)ad & 15) == 0 && ((uintptr_t)wd & 15) == 0;
  if (paired)
    hipLaunchKernelGGL(k_grouped_w4a8<true>, dim3((unsigned)(n_experts * tiles_n + split_wgs)),
                       dim3(GT), 0, stream, aq, ad, (int)top_k, wq4, wd,
                       (int)n_experts, (int)n, (int)k, counts, offsets, rows, y);
  else
    hipLaunchKernelGGL(k_grouped_w4a8<false>, dim3((unsigned)(n_experts * tiles_n + split_wgs)),
                       dim3(GT), 0, stream, aq, ad, (int)top_k, wq4, wd,
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
  const bool u8 = (lane & 8) != 0;
  float v4[4], v2[2];
  // lane ^ 32 and lane ^ 16 with gfx950's half swaps: swapping the upper 32
  // lanes of a (the odd 16-lane rows of a) with the lower 32 lanes of b (the
  // even rows of b) leaves, in every lane, the value it keeps in one result
  // and its partner's in the other
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v[q]),
                                                    __builtin_bit_cast(uint32_t, v[q + 4]), false, false);
    v4[q] = bits_to_float((int32_t)r[0]) + bits_to_float((int32_t)r[1]);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v4[q]),
                                                    __builtin_bit_cast(uint32_t, v4[q + 2]), false, false);
    v2[q] = bits_to_float((int32_t)r[0]) + bits_to_float((int32_t)r[1]);
  }
  float s;
  {
    const float keep = u8 ? v2[1] : v2[0];
    const float send = u8 ? v2[0] : v2[1];
    s = keep + bits_to_float(__builtin_amdgcn_mov_dpp(__builtin_bit_cast(int32_t, send), 0x128, 0xf, 0xf, false));  // lane ^ 8
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
