// bqi_device.h -- device-side helpers shared by the gfx950 kernels of libbqi.
//
// Nothing here is shared with the CPU oracle (oracle/); the two sides are
// written independently.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bqi {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int QK = 32;  // elements per Q8_0 block / W4 group along K

// fp16 bit pattern -> fp32 (exact; subnormals kept).
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Reinterpret int32 bits as fp32.  Always pass a scalar: on this compiler,
// __builtin_bit_cast applied directly to an ext_vector element (v[r]) is
// miscompiled to read element 0 for every r.
__device__ __forceinline__ float bits_to_float(int32_t v) {
  return __builtin_bit_cast(float, v);
}

// int8x4 . int8x4 + c with int32 accumulation (v_dot4_i32_i8).
__device__ __forceinline__ int32_t dot4_i8(int32_t a, int32_t b, int32_t c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// max(v, v of the lane that the DPP control CTRL selects), unsigned
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
  return v > o ? v : o;
}

// Q8_0 quantization of one 32-element block by the 8 consecutive lanes that
// own it (lane sub = lane % 8 holds elements 4*sub .. 4*sub+3 in v): the
// block's absmax is reduced across the 8 lanes, d = fp16_rne(amax / 127)
// with a correctly rounded fp32 division, and each code is
// clamp(round-half-away(x / d), -127, 127) for the exact quotient by the
// stored d (d == 0 gives codes 0 and scale bits 0).  Returns
// this lane's 4 codes packed (element 4*sub + i in byte i) and sets the
// block's scale bits.  Every quantizer in the library goes through this
// function, so all of them produce identical codes.  Finite inputs only (NaN
// and Inf are outside the quantizer's contract).  Never compile with
// fast-math.
__device__ __forceinline__ uint32_t q8_0_quantize4(const float (&v)[4], uint16_t &d_bits) {
  // |x| as its bit pattern: for finite values the unsigned order of the
  // magnitude bits is the order of the magnitudes
  uint32_t am = __builtin_bit_cast(uint32_t, v[0]) & 0x7fffffffu;
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v[i]) & 0x7fffffffu;
    am = am > b ? am : b;
  }
  // reduce over the 8 lanes of this block (lanes differ in bits 0..2) with
  // DPP moves, no LDS round trip: lane ^ 1 and lane ^ 2 (quad permutations),
  // then the mirror inside each 8-lane half-row, which pairs every lane of
  // one quad with a lane of the other
  am = dpp_max_u32<0xb1>(am);   // quad_perm [1, 0, 3, 2]
  am = dpp_max_u32<0x4e>(am);   // quad_perm [2, 3, 0, 1]
  am = dpp_max_u32<0x141>(am);  // row_half_mirror
  const float amax = __builtin_bit_cast(float, am);
  const _Float16 dh = (_Float16)(amax / 127.0f);  // IEEE div, then RNE
  const float dd = (float)dh;
  uint32_t packed = 0;
  if (dd != 0.0f) {
    // The code is round-half-away(|x| / d) with the sign of x.  First from
    // an approximate reciprocal: u = |x| * r + 1/2 (one fma) is within
    // 5e-5 of the exact |x| / d + 1/2 (r within 1 ulp of 1/d, |x| / d <
    // 256, one rounding of a value below 257), so floor(u) is the exact
    // code unless u lies within 2^-12 of an integer.  Such near-ties, rare,
    // are decided exactly instead: the candidate k is corrected with the
    // signs of |x| - (k -/+ 1/2) d, where (k +/- 1/2) d has at most 9 + 11
    // significant bits, so it is exact in fp32, and the fma rounds the
    // difference once, which keeps its sign; |x| = (k + 1/2) d exactly (a
    // tie) rounds up.
    const float r = __builtin_amdgcn_rcpf(dd);
    float kf[4];
    bool near = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = fmaf(fabsf(v[i]), r, 0.5f);
      kf[i] = floorf(u);
      const float fr = u - kf[i];  // exact: in [0, 1)
      near |= fabsf(fr - 0.5f) > 0.5f - 0x1p-12f;
    }
    if (near) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ax = fabsf(v[i]);
        float k = kf[i];
        if (fmaf(-(k - 0.5f), dd, ax) < 0.0f) k -= 1.0f;
        if (fmaf(-(k + 0.5f), dd, ax) >= 0.0f) k += 1.0f;
        kf[i] = k;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t q = (int32_t)fminf(kf[i], 127.0f);
      packed |= ((uint32_t)(v[i] < 0.0f ? -q : q) & 0xffu) << (8 * i);
    }
  }
  d_bits = dd != 0.0f ? __builtin_bit_cast(uint16_t, dh) : (uint16_t)0;
  return packed;
}

// 1.5 * 2^23: an fp32 whose ulp is exactly 1.  An int32 P with |P| < 2^22
// added to its bit pattern gives the bit pattern of the fp32 value
// 1.5 * 2^23 + P, exactly.  The MFMA kernels use it as the int32 accumulator
// seed so that the block dot product comes out already converted.
constexpr int32_t MAGIC_BITS = 0x4B400000;
constexpr float MAGIC_F = 12582912.0f;

// Direct global -> LDS loads (gfx950 LDS DMA), issued through inline asm:
// lane L's 16 bytes land at lds_wave_base + 16 * L; lds_wave_base must be
// wave-uniform (it travels in M0).  The compiler neither counts these loads
// in vmcnt nor sees their LDS writes.  A kernel whose loop keeps several
// stages of such loads in flight uses them instead of the compiler's
// direct-load builtin, because the compiler, seeing a builtin direct load,
// conservatively waits for all of them (vmcnt(0)) before the next LDS read,
// which would drain the pipeline every stage.  Every kernel that uses them
// waits for them explicitly (wait_vmcnt, and a barrier when another wave
// reads the destination).
// M0 carries the LDS base; the leading s_nop is the wait state GFX9 requires
// between an SALU write of M0 and an LDS DMA that reads it (the compiler
// places that write just before the asm and cannot see the DMA inside it).
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_addr(const void *generic_lds_ptr) {
  return (uint32_t)(uintptr_t)(const lds_char *)generic_lds_ptr;
}

__device__ __forceinline__ void dma_lds16(const void *gsrc, void *lds_wave_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base)))
               : "memory");
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima), in the
// GFX9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that orders LDS only: waits for this wave's own LDS
// operations (lgkmcnt(0)), then s_barrier.  Unlike __syncthreads() it does
// not wait for outstanding global loads, so direct-to-LDS loads of later
// stages stay in flight across it; kernels wait for the ones they need with
// wait_vmcnt first.  The memory clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace bqi
