// gemm_mfma.hip -- large-M Q8_0 x Q8_0 GEMM on CDNA4 int8 MFMA: the prefill
// GEMM that "I wrote a custom CUDA inference engine to run Qwen3.5-27B on a
// $130 mining card" (Features) builds from DP4A tiles because that card's
// tensor cores are throttled (Throttle, Workaround).  On gfx950 the same
// per-block integer dot product is one v_mfma_i32_32x32x32_i8: a 32x32 output
// tile for exactly one 32-element Q8_0 block.
//
// Tiling: a workgroup of 4 waves owns a 128x128 output tile; each wave a 64x64
// quarter as 2x2 MFMA tiles.  K advances 64 elements (two Q8_0 blocks) per
// stage; both operand tiles and their scales go through double-buffered,
// XOR-swizzled LDS, with the next stage's global loads in flight while the
// current stage computes.
//
// Scale epilogue (per 32x32 tile and block), two fp32 VALU ops per output:
//   the MFMA accumulator is seeded with the bit pattern of 1.5*2^23, so its
//   int32 result reads as the fp32 value F = 1.5*2^23 + P exactly;
//   t   = fma(F, dw, -1.5*2^23*dw)  = round(dw * P)   (dw is lane-uniform)
//   acc = fma(t, da, acc)                               (da per register)
// -1.5*2^23*dw is exact in fp32, so every term carries one rounding before
// it joins the fp32 sum, and the result stays within
// (nb + 1) * 2^-24 * sum|terms| of the exact value (nb = k/32).
//
// Workgroup -> tile order: consecutive workgroup ids go to different XCDs, so
// the ids are first remapped so each XCD walks a contiguous range of tiles,
// and tiles are ordered in groups of 8 row-tiles so that workgroups running
// together on an XCD share A and W tiles through that XCD's L2.
#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

namespace {

constexpr int BM = 128, BN = 128;  // output tile
constexpr int BK = 64;             // K elements per stage (two blocks)
constexpr int NBS = BK / QK;       // blocks per stage
constexpr int GROUP_M = 8;
constexpr int NUM_XCD = 8;

struct Stage {
  i32x4 a[2];       // two 16-byte chunks of the A tile
  i32x4 w[2];       // two 16-byte chunks of the W tile
  uint16_t sa, sw; // one scale each
};

__global__ __launch_bounds__(256, 2) void k_gemm_mfma(
    const int8_t *__restrict__ aq, const uint16_t *__restrict__ ad, int m,
    const int8_t *__restrict__ wq, const uint16_t *__restrict__ wd, int n,
    int k, float *__restrict__ y, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) int8_t sW[2][BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sAd[2][NBS][BM];  // [block][row]
  __shared__ __attribute__((aligned(16))) uint16_t sWd[2][BN][NBS];  // [col][block]

  // ---- tile selection: XCD-contiguous ranges, grouped along M -------------
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
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave's 64x64 quarter
  const int l32 = lane & 31, g = lane >> 5;
  const int nbk = k / QK;
  const int stages = (nbk + NBS - 1) / NBS;

  // ---- global -> register staging assignment ------------------------------
  // A/W tiles: 128 rows x 64 B = 512 chunks of 16 B; thread t takes chunks t
  // and t+256 (row = c/4, column chunk = c%4).  Scales: 128 rows x 2 blocks
  // = 256 values; thread t takes row t/2, block t%2.
  const int8_t *a_src[2], *w_src[2];
  int chunk_row[2], chunk_col[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid + 256 * h;
    chunk_row[h] = c >> 2;
    chunk_col[h] = c & 3;
    const int ar = min(m0 + chunk_row[h], m - 1);
    const int wr = min(n0 + chunk_row[h], n - 1);
    a_src[h] = aq + (int64_t)ar * k + chunk_col[h] * 16;
    w_src[h] = wq + (int64_t)wr * k + chunk_col[h] * 16;
  }
  const int s_row = tid >> 1, s_blk = tid & 1;
  const uint16_t *ad_src = ad + (int64_t)min(m0 + s_row, m - 1) * nbk + s_blk;
  const uint16_t *wd_src = wd + (int64_t)min(n0 + s_row, n - 1) * nbk + s_blk;

  auto load_stage = [&](int s, Stage &st) {
    const int k0 = s * BK;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool ok = k0 + chunk_col[h] * 16 < k;
      st.a[h] = ok ? *reinterpret_cast<const i32x4 *>(a_src[h] + k0) : i32x4{0, 0, 0, 0};
      st.w[h] = ok ? *reinterpret_cast<const i32x4 *>(w_src[h] + k0) : i32x4{0, 0, 0, 0};
    }
    const bool sok = s * NBS + s_blk < nbk;
    st.sa = sok ? ad_src[s * NBS] : (uint16_t)0;
    st.sw = sok ? wd_src[s * NBS] : (uint16_t)0;
  };
  auto store_stage = [&](int buf, const Stage &st) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = chunk_row[h];
      const int pc = swz64(r, chunk_col[h]);
      *reinterpret_cast<i32x4 *>(&sA[buf][r * BK + pc * 16]) = st.a[h];
      *reinterpret_cast<i32x4 *>(&sW[buf][r * BK + pc * 16]) = st.w[h];
    }
    sAd[buf][s_blk][s_row] = st.sa;
    sWd[buf][s_row][s_blk] = st.sw;
  };

  float acc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  i32x16 seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = MAGIC_BITS;

  Stage st;
  load_stage(0, st);
  store_stage(0, st);
  __syncthreads();

  for (int s = 0; s < stages; ++s) {
    const int buf = s & 1;
    if (s + 1 < stages) load_stage(s + 1, st);

    // scales for this stage: lane-uniform dw of the lane's two columns
    float dwf[2][NBS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wn * 64 + j * 32 + l32;
      const uint32_t two = *reinterpret_cast<const uint32_t *>(&sWd[buf][col][0]);
      dwf[j][0] = half_bits_to_float((uint16_t)(two & 0xffffu));
      dwf[j][1] = half_bits_to_float((uint16_t)(two >> 16));
    }
    const int nb_here = min(NBS, nbk - s * NBS);
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      if (b < nb_here) {
        i32x4 af[2], wf[2];
        uint16_t dah[2][16];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wm * 64 + i * 32 + l32;
          af[i] = *reinterpret_cast<const i32x4 *>(&sA[buf][r * BK + swz64(r, 2 * b + g) * 16]);
          // rows of this lane's 16 outputs: 8*q + 4*g + (0..3), q = 0..3
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint2 v = *reinterpret_cast<const uint2 *>(
                &sAd[buf][b][wm * 64 + i * 32 + 8 * q + 4 * g]);
            dah[i][4 * q + 0] = (uint16_t)(v.x & 0xffffu);
            dah[i][4 * q + 1] = (uint16_t)(v.x >> 16);
            dah[i][4 * q + 2] = (uint16_t)(v.y & 0xffffu);
            dah[i][4 * q + 3] = (uint16_t)(v.y >> 16);
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int c = wn * 64 + j * 32 + l32;
          wf[j] = *reinterpret_cast<const i32x4 *>(&sW[buf][c * BK + swz64(c, 2 * b + g) * 16]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const i32x16 d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], wf[j], seed, 0, 0, 0);
            const float dw = dwf[j][b];
            const float ncd = -MAGIC_F * dw;  // exact
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float t = fmaf(bits_to_float(d[r]), dw, ncd);
              acc[i][j][r] = fmaf(t, half_bits_to_float(dah[i][r]), acc[i][j][r]);
            }
          }
      }
    }
    if (s + 1 < stages) {
      store_stage(buf ^ 1, st);
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

}  // namespace

hipError_t launch_gemm_mfma(const int8_t *aq, const uint16_t *ad, int64_t m,
                            const int8_t *wq, const uint16_t *wd, int64_t n,
                            int64_t k, float *y, hipStream_t stream) {
  const int tiles_m = (int)((m + BM - 1) / BM);
  const int tiles_n = (int)((n + BN - 1) / BN);
  hipLaunchKernelGGL(k_gemm_mfma, dim3((unsigned)(tiles_m * tiles_n)), dim3(256),
                     0, stream, aq, ad, (int)m, wq, wd, (int)n, (int)k, y,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace bqi
