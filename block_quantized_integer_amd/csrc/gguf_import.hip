// gguf_import.hip -- split GGUF Q8_0 and Q4_0 block arrays into the planar
// layout of this library (codes, then scales, each as its own array), so that
// weights stored as GGUF can be consumed: the pages compare against llama.cpp
// on "Q8_0 GGUF" files ("I wrote a custom CUDA inference engine to run
// Qwen3.5-27B on a $130 mining card", Honest benchmark) and use Q4_0-family
// weights ("A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011
// GPU", Method 2).
//
// A GGUF tensor of R x K (K % 32 == 0) is R*K/32 contiguous blocks: a
// little-endian fp16 scale followed by 32 int8 codes (Q8_0, 34 bytes) or by 16
// bytes of nibbles (Q4_0, 18 bytes; byte j = element j low, element j+16
// high, the nibble order the library's 4-bit layout already uses).  Block i
// of the array becomes codes [32i, 32i+32) (Q8_0) or packed bytes [16i, 16i+16)
// (Q4_0) and scale i, so the split is a byte shuffle.
//
// An HBM stream: a workgroup copies 256 consecutive blocks into LDS with
// 16-byte loads (256 * 34 and 256 * 18 bytes are multiples of 16, so every
// workgroup's span stays 16-byte aligned), then each thread writes one block's
// codes with 16-byte stores and its scale.
#include "bqi_device.h"
#include "bqi_launch.h"

namespace bqi {

namespace {

constexpr int GT_ = 256;  // blocks per workgroup (one per thread)

template <int BLOCK_BYTES, int CODE_BYTES>
// (no __restrict__ on src: with it the compiler sinks the chunk loads past the
// barrier into the stores that use them)
__global__ __launch_bounds__(GT_) void k_gguf_split(const uint8_t *src,
                                                    int64_t n_blocks,
                                                    uint8_t *__restrict__ codes,
                                                    uint16_t *__restrict__ scales) {
  static_assert(BLOCK_BYTES == 2 + CODE_BYTES, "block = scale + codes");
  static_assert(GT_ * BLOCK_BYTES % 16 == 0, "workgroup spans stay 16-byte aligned");
  constexpr int SPAN = GT_ * BLOCK_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t s[SPAN];
  for (int64_t b0 = (int64_t)blockIdx.x * GT_; b0 < n_blocks; b0 += (int64_t)gridDim.x * GT_) {
    const int nb = (int)min((int64_t)GT_, n_blocks - b0);
    const int bytes = nb * BLOCK_BYTES;
    const uint8_t *g = src + b0 * BLOCK_BYTES;
    // full 16-byte chunks, all of a thread's loads issued before any LDS
    // store (chunks past the span re-read chunk 0, which a span of at least
    // one block always holds), then the tail byte by byte (last span only)
    constexpr int CHUNKS = (SPAN / 16 + GT_ - 1) / GT_;
    i32x4 r[CHUNKS];
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int o = 16 * ((int)threadIdx.x + GT_ * i);
      r[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(g + (o + 16 <= bytes ? o : 0)));
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int o = 16 * ((int)threadIdx.x + GT_ * i);
      if (o + 16 <= bytes) *reinterpret_cast<i32x4 *>(s + o) = r[i];
    }
    for (int o = (bytes & ~15) + threadIdx.x; o < bytes; o += GT_) s[o] = g[o];
    __syncthreads();
    const int t = threadIdx.x;
    if (t < nb) {
      const uint8_t *blk = s + t * BLOCK_BYTES;
      scales[b0 + t] = (uint16_t)(blk[0] | (blk[1] << 8));
      // the codes start at an even LDS offset: gather them as 16-bit halves
      uint32_t w[CODE_BYTES / 4];
#pragma unroll
      for (int i = 0; i < CODE_BYTES / 4; ++i) {
        const uint16_t lo = *reinterpret_cast<const uint16_t *>(blk + 2 + 4 * i);
        const uint16_t hi = *reinterpret_cast<const uint16_t *>(blk + 4 + 4 * i);
        w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
      i32x4 *dst = reinterpret_cast<i32x4 *>(codes + (b0 + t) * CODE_BYTES);
#pragma unroll
      for (int i = 0; i < CODE_BYTES / 16; ++i)
        dst[i] = i32x4{(int32_t)w[4 * i], (int32_t)w[4 * i + 1], (int32_t)w[4 * i + 2], (int32_t)w[4 * i + 3]};
    }
  }
}

template <int BLOCK_BYTES, int CODE_BYTES>
hipError_t launch_split(const void *src, int64_t n_blocks, void *codes,
                        uint16_t *scales, hipStream_t stream) {
  int64_t wgs = (n_blocks + GT_ - 1) / GT_;
  if (wgs > 16384) wgs = 16384;
  hipLaunchKernelGGL((k_gguf_split<BLOCK_BYTES, CODE_BYTES>), dim3((unsigned)wgs), dim3(GT_),
                     0, stream, static_cast<const uint8_t *>(src), n_blocks,
                     static_cast<uint8_t *>(codes), scales);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gguf_q8_0(const void *src, int64_t n_blocks, int8_t *q,
                            uint16_t *d, hipStream_t stream) {
  return launch_split<34, 32>(src, n_blocks, q, d, stream);
}

hipError_t launch_gguf_q4_0(const void *src, int64_t n_blocks, uint8_t *wq4,
                            uint16_t *wd, hipStream_t stream) {
  return launch_split<18, 16>(src, n_blocks, wq4, wd, stream);
}

}  // namespace bqi
