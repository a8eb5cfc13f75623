// quantize.hip -- fp32/fp16 activations -> Q8_0 (32-element blocks, fp16
// scale), the activation quantizer of the Q8_0 prefill path ("I wrote a custom
// CUDA inference engine to run Qwen3.5-27B on a $130 mining card", section
// Features) and the 8-bit activations of W4A8 ("A 35B Hybrid-Attention
// Mixture-of-Experts Model on a 6GB 2011 GPU", Method 2).
//
// HBM-bound streaming kernel: 8 lanes own one 32-element block (each lane a
// 16-byte fp32 / 8-byte fp16 vector), the block's absmax is reduced across
// the 8 lanes, and each lane stores its 4 codes as one 32-bit word, so a wave
// reads 1 KB (fp32) and writes 256 B of codes, all coalesced.
//
// Exactness: d = fp16_rne(amax / 127) uses HIP's correctly rounded fp32
// division followed by the RNE conversion (equal to rounding the exact
// quotient, because a correctly rounded fp32 quotient can never land on an
// fp16 rounding midpoint it did not start on).  Codes round the exact
// quotient |x| / d half away from zero without dividing: a candidate from an
// approximate reciprocal is corrected by the exact signs of
// |x| - (k -/+ 1/2) d (the product is exact in fp32 and the fma rounds the
// difference once).  The 8-lane absmax reduction runs on DPP moves.  This
// file must not be compiled with fast-math.
#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

// CONTIG: rows are contiguous (ldx == k), so block blk starts at element
// 32 * blk and no row / column split is needed.
template <bool F16, bool CONTIG, typename Idx>
__global__ __launch_bounds__(256) void k_quantize_q8_0(
    const void *__restrict__ x, Idx ldx, Idx blocks_per_row, Idx total_blocks,
    int8_t *__restrict__ q, uint16_t *__restrict__ d) {
  const int sub = threadIdx.x & 7;  // this lane's 4-element slice of the block
  const Idx stride = (Idx)((gridDim.x * (uint32_t)blockDim.x) >> 3);
  for (Idx blk = (Idx)((blockIdx.x * (uint32_t)blockDim.x + threadIdx.x) >> 3);
       blk < total_blocks; blk += stride) {
    Idx off;
    if constexpr (CONTIG) {
      off = blk * QK + sub * 4;
    } else {
      const Idx row = blk / blocks_per_row;
      const Idx b = blk - row * blocks_per_row;
      off = row * ldx + b * QK + sub * 4;
    }
    float v[4];
    if constexpr (F16) {
      const uint2 raw = *reinterpret_cast<const uint2 *>(
          reinterpret_cast<const uint16_t *>(x) + off);
      v[0] = half_bits_to_float((uint16_t)(raw.x & 0xffffu));
      v[1] = half_bits_to_float((uint16_t)(raw.x >> 16));
      v[2] = half_bits_to_float((uint16_t)(raw.y & 0xffffu));
      v[3] = half_bits_to_float((uint16_t)(raw.y >> 16));
    } else {
      const f32x4 raw =
          __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(
              reinterpret_cast<const float *>(x) + off));
      v[0] = raw.x;
      v[1] = raw.y;
      v[2] = raw.z;
      v[3] = raw.w;
    }
    uint16_t dbits;
    const uint32_t packed = q8_0_quantize4(v, dbits);
    *reinterpret_cast<uint32_t *>(q + (size_t)blk * QK + sub * 4) = packed;
    if (sub == 0) d[blk] = dbits;
  }
}

hipError_t launch_quantize_q8_0(const void *x, bool f16, int64_t rows,
                                int64_t k, int64_t ldx, int8_t *q, uint16_t *d,
                                hipStream_t stream) {
  const int64_t bpr = k / QK;
  const int64_t total = rows * bpr;
  // 8 lanes per block; enough workgroups to cover the chip several times
  // over, then grid-stride.
  int64_t wgs = (total * 8 + 255) / 256;
  const int64_t cap = 256 * 16;
  if (wgs > cap) wgs = cap;
  const dim3 grid((unsigned)wgs), block(256);
  const bool small = rows * ldx < ((int64_t)1 << 31) && total < ((int64_t)1 << 28);
  const bool contig = ldx == k;
#define BQI_QUANT_LAUNCH(F16_, CONTIG_, IDX_)                                        \
  hipLaunchKernelGGL((k_quantize_q8_0<F16_, CONTIG_, IDX_>), grid, block, 0, stream, x, \
                     (IDX_)ldx, (IDX_)bpr, (IDX_)total, q, d)
  if (f16) {
    if (small) {
      if (contig) BQI_QUANT_LAUNCH(true, true, uint32_t);
      else BQI_QUANT_LAUNCH(true, false, uint32_t);
    } else {
      if (contig) BQI_QUANT_LAUNCH(true, true, int64_t);
      else BQI_QUANT_LAUNCH(true, false, int64_t);
    }
  } else {
    if (small) {
      if (contig) BQI_QUANT_LAUNCH(false, true, uint32_t);
      else BQI_QUANT_LAUNCH(false, false, uint32_t);
    } else {
      if (contig) BQI_QUANT_LAUNCH(false, true, int64_t);
      else BQI_QUANT_LAUNCH(false, false, int64_t);
    }
  }
#undef BQI_QUANT_LAUNCH
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero_f32(float *__restrict__ y, int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    y[i] = 0.0f;
}

// Zero-fill by a kernel rather than hipMemsetAsync, so that a caller may
// capture the call in a HIP graph.
hipError_t launch_zero_f32(float *y, int64_t count, hipStream_t stream) {
  int64_t wgs = (count + 255) / 256;
  if (wgs > 4096) wgs = 4096;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)wgs), dim3(256), 0, stream, y, count);
  return hipGetLastError();
}

}  // namespace bqi
