// gemm_mfma.hip -- large-M Q8_0 x Q8_0 GEMM on CDNA4 int8 MFMA: the prefill
// GEMM that "I wrote a custom CUDA inference engine to run Qwen3.5-27B on a
// $130 mining card" (Features) builds from DP4A tiles because that card's
// tensor cores are throttled (Throttle, Workaround).  On gfx950 the same
// per-block integer dot product is one v_mfma_i32_32x32x32_i8: a 32x32 output
// tile for exactly one 32-element Q8_0 block.
//
// Tiling: a workgroup of 4 waves owns a 128x128 output tile; each wave a 64x64
// quarter as 2x2 MFMA tiles.  K advances NBS = 4 blocks per stage through two
// LDS buffers.  The operand tiles travel HBM -> LDS with gfx950's direct
// loads (global_load_lds_dwordx4: each wave instruction fills 1 KB of LDS, 16
// bytes per lane), so they occupy no registers and need no LDS stores; lane L
// fetches the global chunk that the XOR swizzle assigns to LDS slot L.  The
// fp16 scales are converted to fp32 once, on their way into the stage's LDS
// scale arrays.  When k is a multiple of 256 and both scale arrays are 16-byte
// aligned (PAIRED), each row's scales for two stages (16 bytes) arrive in LDS
// with one direct load per lane, four such wave loads per workgroup every
// other stage, and the lane that loaded a row converts it; otherwise every
// thread loads 2-byte scales into registers each stage.  Both give the same
// LDS contents.  The load instructions, not their bytes, are what a CU takes
// slowly (one 64-lane load per ~32-38 cycles), so the paired path's 2 scale
// loads per stage instead of 16 make the GEMM ~4% faster (k_gemm_mfma_w8
// below takes the same paired path, ~6% faster).
// The loads of stage s+1 are in flight while stage s computes.
//
// Scale epilogue (per 32x32 tile and block), two fp32 FMAs per output:
//   the MFMA accumulator is seeded with the bit pattern of 1.5*2^23, so its
//   int32 result reads as the fp32 value F = 1.5*2^23 + P exactly;
//   t   = fma(F, dw, -1.5*2^23*dw)  = round(dw * P)   (dw: the lane's column,
//                                                       one for all its outputs)
//   acc = fma(t, da, acc)                               (da: per register row)
// -1.5*2^23*dw is exact in fp32, so every term carries one rounding before
// it joins the fp32 sum, and the result stays within
// (nb + 1) * 2^-24 * sum|terms| of the exact value (nb = k/32).  Both FMAs
// are plain v_fma_f32 (the fp16-reading v_fma_mix_f32 issues at about half
// the rate on gfx950).  The epilogue, not the MFMA, bounds this kernel: two
// VALU ops per output and block against one MFMA per 32 MACs.
//
// Workgroup -> tile order: consecutive workgroup ids go to different XCDs, so
// the ids are first remapped so each XCD walks a contiguous range of tiles,
// and tiles are ordered in groups of 8 row-tiles so that workgroups running
// together on an XCD share A and W tiles through that XCD's L2.
//
// Grids of at most one tile per CU (short prompts: m up to ~128 rows for
// wide weights) run k_gemm_mfma_w8 instead: the same tile, operand layout and
// epilogue, with 8 waves per workgroup (a 32x64 part each) and one workgroup
// per CU, so every SIMD still holds two waves where the 4-wave kernel would
// leave one.  With the CU to itself it keeps three stage buffers in (dynamic)
// LDS and issues the loads two stages ahead.  Larger grids stay on the 4-wave
// kernel, whose two workgroups per CU cover each other's stalls.
#include <type_traits>

#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

namespace {

constexpr int BM = 128, BN = 128;  // output tile
constexpr int NBS = 4;             // Q8_0 blocks per stage
constexpr int BK = NBS * QK;       // K bytes per tile row per stage (128)
constexpr int CPR = BK / 16;       // 16-byte chunks per tile row per stage (8)
constexpr int GROUP_M = 8;
constexpr int NUM_XCD = 8;
constexpr int THREADS = 256;
constexpr int ROWS_PER_LOAD = 64 / CPR;                      // rows filled by one wave load (8)
constexpr int LOADS_PER_WAVE = BM / ROWS_PER_LOAD / 4;       // per operand tile (4)
constexpr int SCALES_PER_THREAD = BM * NBS / THREADS;        // per operand (2)

static_assert(CPR == 8, "the swizzle assumes 8 chunks per row");

// Physical 16-byte chunk of logical chunk c in tile row r.  Rows are 128 B
// (32 of the 64 LDS banks); a fragment read has 16 lanes on 16 consecutive
// rows at one logical chunk, and this swizzle spreads them over all banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

struct Tiles {
  int8_t a[BM * BK];
  int8_t w[BN * BK];
  float ad[NBS][BM];  // [block][row]
  float wd[BN][NBS];  // [col][block]
};

// Origin (m0, n0) of this workgroup's tile: XCD-contiguous ranges of tile
// ids, grouped by GROUP_M row tiles.
__device__ __forceinline__ void tile_origin(int tiles_m, int tiles_n, int &m0, int &n0) {
  const int tiles = tiles_m * tiles_n;
  int tile;
  {
    const int i = blockIdx.x;
    const int xcd = i % NUM_XCD, local = i / NUM_XCD;
    const int base = tiles / NUM_XCD, rem = tiles % NUM_XCD;
    tile = xcd * base + min(xcd, rem) + local;
  }
  const int per_group = GROUP_M * tiles_n;
  const int group = tile / per_group;
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = tile - group * per_group;
  m0 = (first_m + in_group % gm) * BM;
  n0 = (in_group / gm) * BN;
}

template <bool PAIRED>
__global__ __launch_bounds__(THREADS, 2) void k_gemm_mfma(
    const int8_t *__restrict__ aq, const uint16_t *__restrict__ ad, int m,
    const int8_t *__restrict__ wq, const uint16_t *__restrict__ wd, int n,
    int k, float *__restrict__ y, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) Tiles T[2];
  // PAIRED: the fp16 scales of a pair of stages (2 NBS blocks per row) as
  // loaded: [operand][row][block], the A tile's rows, then the W tile's
  __shared__ __attribute__((aligned(16))) uint16_t raw[PAIRED ? 2 * BM * 2 * NBS : 8];

  int m0, n0;
  tile_origin(tiles_m, tiles_n, m0, n0);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave's 64x64 quarter
  const int l32 = lane & 31, g = lane >> 5;
  const int nbk = k / QK;
  const int stages = (nbk + NBS - 1) / NBS;

  // ---- stage loads -----------------------------------------------------------
  // Wave load q fills tile rows rt .. rt+7 (rt = 8*(4*wave + q)); lane L lands
  // in LDS slot L: row rt + L/8, physical chunk L%8, which holds logical chunk
  // (L%8) ^ swizzle(row).  Rows past m (n) re-read the last row, so every
  // load stays in bounds.  The loads take a wave-uniform 64-bit base in
  // SGPRs (the operand pointer advanced to the stage's first byte) and a
  // loop-invariant 32-bit lane offset (the ABI layer guarantees m*k, n*k <
  // 2^31), so a full stage issues its loads with no per-lane address
  // arithmetic.  In a short last stage, chunks past k re-read the row's last
  // chunk instead (their blocks get scale 0 below), which keeps every offset
  // non-negative and inside the row.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  int aoff[LOADS_PER_WAVE], woff[LOADS_PER_WAVE], c16[LOADS_PER_WAVE];
#pragma unroll
  for (int q = 0; q < LOADS_PER_WAVE; ++q) {
    const int r = ROWS_PER_LOAD * (LOADS_PER_WAVE * wave + q) + lane / CPR;
    c16[q] = 16 * ((lane % CPR) ^ ((r >> 1) & 7));
    aoff[q] = min(m0 + r, m - 1) * k + c16[q];
    woff[q] = min(n0 + r, n - 1) * k + c16[q];
  }
  // scales: thread -> (row, block) pairs tid + THREADS*h; a short last stage
  // clamps the block to the row's last one (its scale is replaced by 0)
  int sa_off[SCALES_PER_THREAD], sw_off[SCALES_PER_THREAD];
#pragma unroll
  for (int h = 0; h < SCALES_PER_THREAD; ++h) {
    const int c = tid + THREADS * h;
    const int row = c / NBS, blk = c % NBS;
    sa_off[h] = min(m0 + row, m - 1) * nbk + blk;
    sw_off[h] = min(n0 + row, n - 1) * nbk + blk;
  }
  uint16_t sa_reg[SCALES_PER_THREAD], sw_reg[SCALES_PER_THREAD];
  // full: stage s lies inside k (a compile-time flag, so that a full stage
  // issues its loads with the loop-invariant offsets and no clamping)
  auto issue_stage = [&](int s, int buf, auto full_c) {
    constexpr bool full = decltype(full_c)::value;
    const int k0 = s * BK;
    const int8_t *abase = aq + k0, *wbase = wq + k0;
#pragma unroll
    for (int q = 0; q < LOADS_PER_WAVE; ++q) {
      int ao = aoff[q], wo = woff[q];
      if constexpr (!full) {
        const int fix = min(c16[q], k - 16 - k0) - c16[q];
        ao += fix;
        wo += fix;
      }
      const uint32_t lds_a = lds_addr(&T[buf].a[ROWS_PER_LOAD * (LOADS_PER_WAVE * wave_u + q) * BK]);
      const uint32_t lds_w = lds_addr(&T[buf].w[ROWS_PER_LOAD * (LOADS_PER_WAVE * wave_u + q) * BK]);
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(ao), "s"(abase), "{m0}"(lds_a) : "memory");
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(wo), "s"(wbase), "{m0}"(lds_w) : "memory");
    }
    const uint16_t *sabase = ad + s * NBS, *swbase = wd + s * NBS;
#pragma unroll
    for (int h = 0; h < SCALES_PER_THREAD; ++h) {
      int ao = sa_off[h], wo = sw_off[h];
      if constexpr (!full) {
        const int blk = (tid + THREADS * h) % NBS;
        const int fix = min(blk, nbk - 1 - s * NBS) - blk;
        ao += fix;
        wo += fix;
      }
      if constexpr (!PAIRED) {
        sa_reg[h] = sabase[(uint32_t)ao];
        sw_reg[h] = swbase[(uint32_t)wo];
      }
    }
  };
  // PAIRED: wave w < 2 loads the scales of A tile rows 64 w .. +63, wave
  // w >= 2 those of W tile rows 64 (w - 2) .. +63 (rows past m or n re-read
  // the last one), 16 bytes (a pair of stages) per lane; the lane converts
  // its row's four scales of each stage itself, after its own wait, so no
  // other barrier is needed.  Pair p is loaded at the start of stage 2p - 1,
  // after the end of stage 2p - 2 read the previous pair for the last time.
  const bool sc_a = wave_u < 2;
  const int sc_row = 64 * (wave_u & 1) + lane;
  const int sc_goff = 2 * ((sc_a ? min(m0 + sc_row, m - 1) : min(n0 + sc_row, n - 1)) * nbk);
  const uint16_t *sc_base = sc_a ? ad : wd;
  uint16_t *sc_raw = &raw[PAIRED ? (sc_a ? 0 : BM * 2 * NBS) : 0];
  auto issue_raw = [&](int pair) {
    const uint32_t lds = lds_addr(sc_raw + 2 * NBS * 64 * (wave_u & 1));
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(sc_goff + 4 * NBS * pair), "s"(sc_base), "{m0}"(lds) : "memory");
  };
  auto convert_raw = [&](int s, int buf) {
    const uint2 v = *reinterpret_cast<const uint2 *>(sc_raw + 2 * NBS * sc_row + NBS * (s & 1));
    const float f0 = half_bits_to_float((uint16_t)(v.x & 0xffffu)), f1 = half_bits_to_float((uint16_t)(v.x >> 16));
    const float f2 = half_bits_to_float((uint16_t)(v.y & 0xffffu)), f3 = half_bits_to_float((uint16_t)(v.y >> 16));
    if (sc_a) {
      T[buf].ad[0][sc_row] = f0;
      T[buf].ad[1][sc_row] = f1;
      T[buf].ad[2][sc_row] = f2;
      T[buf].ad[3][sc_row] = f3;
    } else {
      *reinterpret_cast<f32x4 *>(&T[buf].wd[sc_row][0]) = f32x4{f0, f1, f2, f3};
    }
  };
  // Blocks past k (a short last stage) get activation scale 0: the stage
  // loop always runs all NBS blocks, and such a block's term
  // fma(t, 0, acc) leaves acc unchanged (t is finite, and acc, which starts
  // at +0 and only ever gains round-to-nearest sums, is never -0).
  auto store_scales = [&](int s, int buf) {
#pragma unroll
    for (int h = 0; h < SCALES_PER_THREAD; ++h) {
      const int c = tid + THREADS * h;
      const int row = c / NBS, blk = c % NBS;
      const bool valid = s * NBS + blk < nbk;
      T[buf].ad[blk][row] = valid ? half_bits_to_float(sa_reg[h]) : 0.0f;
      T[buf].wd[row][blk] = half_bits_to_float(sw_reg[h]);
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  i32x16 seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = MAGIC_BITS;

  // stage s is full while (s + 1) * BK <= k (the branch is uniform)
  auto issue = [&](int s, int buf) {
    if ((s + 1) * BK <= k)
      issue_stage(s, buf, std::true_type{});
    else
      issue_stage(s, buf, std::false_type{});
  };
  if constexpr (PAIRED) issue_raw(0);
  issue(0, 0);
  if constexpr (!PAIRED) store_scales(0, 0);
  wait_vmcnt<0>();  // direct loads of stage 0 have landed
  if constexpr (PAIRED) convert_raw(0, 0);
  __syncthreads();

  for (int s = 0; s < stages; ++s) {
    const int buf = s & 1;
    const Tiles &TB = T[buf];
    if (s + 1 < stages) issue(s + 1, buf ^ 1);
    if constexpr (PAIRED) {
      if ((s & 1) && s + 1 < stages) issue_raw((s + 1) >> 1);
    }

    // The stage's 16 MFMAs (4 blocks x 2x2 tiles) run as a pipeline of depth
    // one: tile u's MFMA is issued before tile u-1's epilogue, into the other
    // of two result register sets, so the matrix core works on tile u while
    // the VALU scales tile u-1.  The block loop is unrolled, so every scale
    // sits in a register named at compile time.
    float dwf[2][NBS], ncd[2][NBS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 four = *reinterpret_cast<const f32x4 *>(&TB.wd[wn * 64 + j * 32 + l32][0]);
      dwf[j][0] = four.x;
      dwf[j][1] = four.y;
      dwf[j][2] = four.z;
      dwf[j][3] = four.w;
#pragma unroll
      for (int b = 0; b < NBS; ++b) ncd[j][b] = -MAGIC_F * dwf[j][b];  // exact
    }

    // Operands are read from LDS one step ahead of their use: at step u the
    // wave reads the fragments of tile u+1 that it does not hold yet and the
    // activation scales that the next epilogues need, so about one tile of
    // operands is in flight beside the accumulators.
    //
    // Each step is pinned in place with empty asm statements (the compiler
    // otherwise places the pure MFMA and FMA operations anywhere in the
    // unrolled stage: it issued a dozen MFMAs into separate registers and
    // spilled).  A step starts with a statement that takes the MFMA's
    // fragments (so the MFMA cannot move above it) and ends with one that
    // takes the epilogue's accumulators and the new MFMA result (so neither
    // can move below it); by then 32 VALU instructions separate the MFMA from
    // that statement, so reading its result costs no wait.
    i32x4 af[2], wf[2];        // [row tile], [column tile] of the current block
    i32x4 af_n, wf_n[2];       // the next block's first row fragment and column fragments
    float da[2][16];           // activation scales of the block's two row tiles
    auto read_a = [&](int b, int i) {
      const int r = wm * 64 + i * 32 + l32;
      return *reinterpret_cast<const i32x4 *>(&TB.a[r * BK + swz(r, 2 * b + g) * 16]);
    };
    auto read_w = [&](int b, int j) {
      const int c = wn * 64 + j * 32 + l32;
      return *reinterpret_cast<const i32x4 *>(&TB.w[c * BK + swz(c, 2 * b + g) * 16]);
    };
    auto read_da = [&](int b, int i, float (&dst)[16]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(&TB.ad[b][wm * 64 + i * 32 + 8 * q + 4 * g]);
        dst[4 * q + 0] = v.x;
        dst[4 * q + 1] = v.y;
        dst[4 * q + 2] = v.z;
        dst[4 * q + 3] = v.w;
      }
    };
    auto epilogue = [&](const i32x16 &d, int u) {
      const int b = u >> 2, i = (u >> 1) & 1, j = u & 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float t = fmaf(bits_to_float(d[r]), dwf[j][b], ncd[j][b]);
        acc[i][j][r] = fmaf(t, da[i][r], acc[i][j][r]);
      }
    };

    // tiles of a block in the order (0,0) (0,1) (1,0) (1,1)
    af[0] = read_a(0, 0);
    wf[0] = read_w(0, 0);
    wf[1] = read_w(0, 1);
    read_da(0, 0, da[0]);
    i32x16 dres[2];
#pragma unroll
    for (int u = 0; u < 4 * NBS; ++u) {
      const int b = u >> 2, t = u & 3, i = t >> 1, j = t & 1;
      if (t == 0) af[1] = read_a(b, 1);
      if (t == 1) read_da(b, 1, da[1]);
      if (t == 2 && b + 1 < NBS) { af_n = read_a(b + 1, 0); wf_n[0] = read_w(b + 1, 0); }
      if (t == 3 && b + 1 < NBS) wf_n[1] = read_w(b + 1, 1);
      asm volatile("" : "+v"(af[i]), "+v"(wf[j]));
      dres[u & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], wf[j], seed, 0, 0, 0);
      // within the step: the MFMA first, then the previous tile's epilogue
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (u > 0) {
        epilogue(dres[(u - 1) & 1], u - 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
        const int pi = ((u - 1) >> 1) & 1, pj = (u - 1) & 1;
        asm volatile("" : "+v"(acc[pi][pj]), "+v"(dres[u & 1]));
      } else {
        asm volatile("" : "+v"(dres[u & 1]));
      }
      if (t == 3 && b + 1 < NBS) {
        // the next block's fragments become current; its row tile 0 scales
        // replace this block's (their last use was the epilogue above)
        af[0] = af_n;
        wf[0] = wf_n[0];
        wf[1] = wf_n[1];
        read_da(b + 1, 0, da[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    epilogue(dres[(4 * NBS - 1) & 1], 4 * NBS - 1);

    if constexpr (!PAIRED) {
      if (s + 1 < stages) store_scales(s + 1, buf ^ 1);
    }
    wait_vmcnt<0>();  // this wave's direct loads have landed
    if constexpr (PAIRED) {
      if (s + 1 < stages) convert_raw(s + 1, buf ^ 1);
    }
    __syncthreads();
  }

  // ---- store: lane holds column n0+wn*64+j*32+l32, rows 8q+4g+(0..3) ------
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + wn * 64 + j * 32 + l32;
    if (col < n) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (row < m) y[(int64_t)row * n + col] = acc[i][j][r];
        }
    }
  }
}

// ---- small grids: 8 waves per tile, three stage buffers -------------------
constexpr int W8_WAVES = 8;
constexpr int W8_THREADS = 64 * W8_WAVES;
constexpr int W8_NBUF = 3;                                          // stage buffers
constexpr int W8_LOADS_PER_WAVE = BM / ROWS_PER_LOAD / W8_WAVES;    // per operand tile (2)
constexpr int W8_LDS = W8_NBUF * (int)sizeof(Tiles);
static_assert(BM * NBS == W8_THREADS, "one scale of each operand per thread and stage");

// Wave w owns row tile w/2 and column tiles 2(w%2), 2(w%2)+1 of the 128x128
// tile.  Stage s issues the scales of stage s+1 and the tiles of stage s+2
// (three buffers), and ends by waiting for those scales: loads complete in
// issue order, so that wait also covers the tiles of stage s+1, and leaves
// only the tiles of stage s+2 in flight.  All of these loads go through
// inline asm (dma_lds16 and the scale loads below), which the compiler
// neither counts nor waits for, because its own count of direct loads ends in
// a full drain (vmcnt(0)) at every stage.
template <bool PAIRED>
__global__ __launch_bounds__(W8_THREADS, 1) void k_gemm_mfma_w8(
    const int8_t *__restrict__ aq, const uint16_t *__restrict__ ad, int m,
    const int8_t *__restrict__ wq, const uint16_t *__restrict__ wd, int n,
    int k, float *__restrict__ y, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) int8_t gemm_lds[];
  Tiles *T = reinterpret_cast<Tiles *>(gemm_lds);  // [W8_NBUF]
  int m0, n0;
  tile_origin(tiles_m, tiles_n, m0, n0);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave's 32x64 part: row tile wm, column tiles 2wn, 2wn+1
  const int l32 = lane & 31, g = lane >> 5;
  const int nbk = k / QK;
  const int stages = (nbk + NBS - 1) / NBS;

  auto issue_direct = [&](int s, int buf) {
    const int k0 = s * BK;
#pragma unroll
    for (int q = 0; q < W8_LOADS_PER_WAVE; ++q) {
      const int rt = ROWS_PER_LOAD * (W8_LOADS_PER_WAVE * wave + q);  // wave-uniform
      const int r = rt + lane / CPR;
      const int c = (lane % CPR) ^ ((r >> 1) & 7);
      const int kk = k0 + 16 * c < k ? k0 + 16 * c : 0;
      dma_lds16(aq + (min(m0 + r, m - 1) * k + kk), &T[buf].a[rt * BK]);
      dma_lds16(wq + (min(n0 + r, n - 1) * k + kk), &T[buf].w[rt * BK]);
    }
  };
  // The explicit waits take the two scale registers as operands, so that
  // nothing reads them before their loads have landed.
  uint32_t sa_reg, sw_reg;
  auto issue_scales = [&](int s) {
    const int row = tid / NBS, blk = tid % NBS;
    const int kb = s * NBS + blk < nbk ? s * NBS + blk : 0;
    const uint16_t *pa = ad + min(m0 + row, m - 1) * nbk + kb;
    const uint16_t *pw = wd + min(n0 + row, n - 1) * nbk + kb;
    asm volatile("global_load_ushort %0, %1, off" : "=v"(sa_reg) : "v"(pa) : "memory");
    asm volatile("global_load_ushort %0, %1, off" : "=v"(sw_reg) : "v"(pw) : "memory");
  };
  auto store_scales = [&](int buf) {
    const int row = tid / NBS, blk = tid % NBS;
    T[buf].ad[blk][row] = half_bits_to_float((uint16_t)sa_reg);
    T[buf].wd[row][blk] = half_bits_to_float((uint16_t)sw_reg);
  };
  // PAIRED: as in the 4-wave kernel, waves 0 and 1 load the scales of A tile
  // rows 64 w .. +63 for two stages (16 bytes per lane), waves 2 and 3 those
  // of W tile rows 64 (w - 2) .. +63, into the raw area after the stage
  // buffers, and each lane converts its own row
  uint16_t *raw = reinterpret_cast<uint16_t *>(gemm_lds + W8_LDS);  // [2][BM][2 NBS]
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool sc_a = wave_u < 2;
  const int sc_row = 64 * (wave_u & 1) + lane;
  const int sc_goff = 2 * ((sc_a ? min(m0 + sc_row, m - 1) : min(n0 + sc_row, n - 1)) * nbk);
  const uint16_t *sc_base = sc_a ? ad : wd;
  uint16_t *sc_raw = raw + (sc_a ? 0 : BM * 2 * NBS);
  auto issue_raw = [&](int pair) {
    if (wave_u < 4) {
      const uint32_t lds = lds_addr(sc_raw + 2 * NBS * 64 * (wave_u & 1));
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(sc_goff + 4 * NBS * pair), "s"(sc_base), "{m0}"(lds) : "memory");
    }
  };
  auto convert_raw = [&](int s, int buf) {
    if (wave_u < 4) {
      const uint2 v = *reinterpret_cast<const uint2 *>(sc_raw + 2 * NBS * sc_row + NBS * (s & 1));
      const float f0 = half_bits_to_float((uint16_t)(v.x & 0xffffu)), f1 = half_bits_to_float((uint16_t)(v.x >> 16));
      const float f2 = half_bits_to_float((uint16_t)(v.y & 0xffffu)), f3 = half_bits_to_float((uint16_t)(v.y >> 16));
      if (sc_a) {
        T[buf].ad[0][sc_row] = f0;
        T[buf].ad[1][sc_row] = f1;
        T[buf].ad[2][sc_row] = f2;
        T[buf].ad[3][sc_row] = f3;
      } else {
        *reinterpret_cast<f32x4 *>(&T[buf].wd[sc_row][0]) = f32x4{f0, f1, f2, f3};
      }
    }
  };

  float acc[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  i32x16 seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = MAGIC_BITS;

  // stage 0 landed and its scales stored; stage 1's tiles in flight
  if constexpr (PAIRED) {
    issue_raw(0);
    issue_direct(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    convert_raw(0, 0);
  } else {
    issue_scales(0);
    issue_direct(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" : "+v"(sa_reg), "+v"(sw_reg) :: "memory");
    store_scales(0);
  }
  if (stages > 1) issue_direct(1, 1);
  __syncthreads();

  for (int s = 0; s < stages; ++s) {
    const int buf = s % W8_NBUF;
    const Tiles &TB = T[buf];
    // The tile loads are unconditional, so that every stage issues the same
    // loads and the wait count below is exact: past the last stage they
    // re-read it into the buffer that no stage reads any more.  The scale
    // register loads are issued only for a stage that follows: the last stage
    // leaves none in flight, so no register load outlives the waits that name
    // its destination.
    if constexpr (PAIRED) {
      if ((s & 1) && s + 1 < stages) issue_raw((s + 1) >> 1);
    } else {
      if (s + 1 < stages) issue_scales(s + 1);
    }
    issue_direct(min(s + 2, stages - 1), (s + 2) % W8_NBUF);

    float dwf[2][NBS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 four = *reinterpret_cast<const f32x4 *>(&TB.wd[wn * 64 + j * 32 + l32][0]);
      dwf[j][0] = four.x;
      dwf[j][1] = four.y;
      dwf[j][2] = four.z;
      dwf[j][3] = four.w;
    }
    const int nb_here = min(NBS, nbk - s * NBS);

    for (int b = 0; b < nb_here; ++b) {
      const int r = wm * 32 + l32;
      const i32x4 af = *reinterpret_cast<const i32x4 *>(&TB.a[r * BK + swz(r, 2 * b + g) * 16]);
      float da[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(&TB.ad[b][wm * 32 + 8 * q + 4 * g]);
        da[4 * q + 0] = v.x;
        da[4 * q + 1] = v.y;
        da[4 * q + 2] = v.z;
        da[4 * q + 3] = v.w;
      }
      i32x4 wf[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = wn * 64 + j * 32 + l32;
        wf[j] = *reinterpret_cast<const i32x4 *>(&TB.w[c * BK + swz(c, 2 * b + g) * 16]);
      }
      float dwb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        dwb[j] = dwf[j][0];
#pragma unroll
        for (int bb = 1; bb < NBS; ++bb)
          if (b == bb) dwb[j] = dwf[j][bb];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const i32x16 d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, wf[j], seed, 0, 0, 0);
        const float dw = dwb[j];
        const float ncd = -MAGIC_F * dw;  // exact
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const float t = fmaf(bits_to_float(d[rr]), dw, ncd);
          acc[j][rr] = fmaf(t, da[rr], acc[j][rr]);
        }
      }
    }

    if (s + 1 < stages) {
      // everything but stage s+2's 2 * W8_LOADS_PER_WAVE tile loads has landed
      if constexpr (PAIRED) {
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * W8_LOADS_PER_WAVE) : "memory");
        convert_raw(s + 1, (s + 1) % W8_NBUF);
      } else {
        asm volatile("s_waitcnt vmcnt(%2)" : "+v"(sa_reg), "+v"(sw_reg) : "n"(2 * W8_LOADS_PER_WAVE) : "memory");
        store_scales((s + 1) % W8_NBUF);
      }
      __syncthreads();
    }
  }

  // no direct load may land after the workgroup ends; the scale registers
  // are named so that this wait also orders them (none is in flight here)
  if constexpr (PAIRED)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" : "+v"(sa_reg), "+v"(sw_reg) :: "memory");
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + wn * 64 + j * 32 + l32;
    if (col < n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < m) y[(int64_t)row * n + col] = acc[j][r];
      }
    }
  }
}

}  // namespace

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

hipError_t launch_gemm_mfma(const int8_t *aq, const uint16_t *ad, int64_t m,
                            const int8_t *wq, const uint16_t *wd, int64_t n,
                            int64_t k, float *y, hipStream_t stream) {
  const int tiles_m = (int)((m + BM - 1) / BM);
  const int tiles_n = (int)((n + BN - 1) / BN);
  const int tiles = tiles_m * tiles_n;
  if (tiles <= device_cus()) {
    // at most one tile per CU: the 8-wave, three-stage kernel
    const bool paired = (k / QK) % (2 * NBS) == 0 && ((uintptr_t)ad & 15) == 0 && ((uintptr_t)wd & 15) == 0;
    constexpr int RAW = 2 * BM * 2 * NBS * 2;  // bytes of the PAIRED raw scale area
    if (paired) {
      static bool raised[64];
      const hipError_t e = raise_dynamic_lds((const void *)k_gemm_mfma_w8<true>, W8_LDS + RAW, raised);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_gemm_mfma_w8<true>, dim3((unsigned)tiles), dim3(W8_THREADS), W8_LDS + RAW, stream,
                         aq, ad, (int)m, wq, wd, (int)n, (int)k, y, tiles_m, tiles_n);
    } else {
      static bool raised[64];
      const hipError_t e = raise_dynamic_lds((const void *)k_gemm_mfma_w8<false>, W8_LDS, raised);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_gemm_mfma_w8<false>, dim3((unsigned)tiles), dim3(W8_THREADS), W8_LDS, stream,
                         aq, ad, (int)m, wq, wd, (int)n, (int)k, y, tiles_m, tiles_n);
    }
    return hipGetLastError();
  }
  const bool paired = (k / QK) % (2 * NBS) == 0 && ((uintptr_t)ad & 15) == 0 && ((uintptr_t)wd & 15) == 0;
  if (paired)
    hipLaunchKernelGGL(k_gemm_mfma<true>, dim3((unsigned)tiles), dim3(THREADS),
                       0, stream, aq, ad, (int)m, wq, wd, (int)n, (int)k, y,
                       tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(k_gemm_mfma<false>, dim3((unsigned)tiles), dim3(THREADS),
                       0, stream, aq, ad, (int)m, wq, wd, (int)n, (int)k, y,
                       tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace bqi
