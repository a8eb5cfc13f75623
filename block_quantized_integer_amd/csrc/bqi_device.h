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

// 1.5 * 2^23: an fp32 whose ulp is exactly 1.  An int32 P with |P| < 2^22
// added to its bit pattern gives the bit pattern of the fp32 value
// 1.5 * 2^23 + P, exactly.  The MFMA kernels use it as the int32 accumulator
// seed so that the block dot product comes out already converted.
constexpr int32_t MAGIC_BITS = 0x4B400000;
constexpr float MAGIC_F = 12582912.0f;

// Index of the LDS 16-byte chunk holding logical chunk c (0..3) of row r in
// a tile stored as rows of 64 bytes: an XOR swizzle that makes the MFMA
// fragment reads (32 rows, same logical chunk) hit 8 distinct bank groups
// per 8 lanes.
__device__ __forceinline__ int swz64(int r, int c) { return c ^ ((r >> 1) & 3); }

// Direct global -> LDS load (gfx950 LDS DMA, 16 bytes per lane).  Lane L's
// 16 bytes land at lds_wave_base + 16 * L
// (lds_wave_base must be wave-uniform).  Issued through inline asm so that the
// compiler does not track them: every kernel that uses them waits for them
// explicitly (s_waitcnt vmcnt(0) and a barrier) before any wave reads the
// destination.  Compiler-visible loads issued around them may then be waited
// on more than necessary, never less.  M0 carries the LDS base; the leading
// s_nop is the one wait state GFX9 requires between an SALU write of M0 and
// an LDS DMA that reads it (the compiler places that write just before the
// asm and cannot see the DMA inside it).
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_addr(const void *generic_lds_ptr) {
  return (uint32_t)(uintptr_t)(const lds_char *)generic_lds_ptr;
}

__device__ __forceinline__ void dma_lds16(const void *gsrc, uint32_t lds_wave_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_wave_base))
               : "memory");
}


}  // namespace bqi
