// Device-side helpers shared by the HIP kernels of the NVFP4 W4A4 layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Quotient and remainder by a fixed divisor with one multiply-high
// (round-up method; exact for every n < 2^31 and d < 2^31).
struct FastDiv {
  uint32_t d;
  uint32_t mul;
  uint32_t shift;
};

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  uint64_t t = ((uint64_t)__umulhi(n, f.mul) + n) >> f.shift;
  return (uint32_t)t;
}

// Maximum of the BF16 magnitudes packed in a 32-bit word pair list.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  uint32_t lo = max(a & 0xFFFFu, b & 0xFFFFu);
  uint32_t hi = max(a >> 16, b >> 16);
  return lo | (hi << 16);
}

// Maximum of v over the 64 lanes of a wave, the same value on every lane:
// DPP steps in a fixed order (pairs, quads, half rows, rows of 16, then rows
// 0+1 and 0+1+2+3 by row broadcasts 15 and 31; lane 63 ends with it), all in
// the VALU with no LDS round trip, then lane 63's value to every lane.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  // lanes of rows outside kRowMask take max(v, 0) = v
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<0xB1, 0xF>(v);     // quad_perm [1,0,3,2]
  v = dpp_max_u32<0x4E, 0xF>(v);     // quad_perm [2,3,0,1]
  v = dpp_max_u32<0x141, 0xF>(v);    // row_half_mirror
  v = dpp_max_u32<0x140, 0xF>(v);    // row_mirror
  v = dpp_max_u32<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
  v = dpp_max_u32<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Round-to-nearest-even float32 -> BF16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

}  // namespace nvfp4
