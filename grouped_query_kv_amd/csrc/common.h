// Small device helpers shared by the HIP kernels of libgqa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ u32x4 zero_u32x4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// 16-byte global load (the address must be 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *static_cast<const u32x4*>(p); }

// 16-byte streaming load for data read exactly once (non-temporal hint:
// the line is not kept in the caches for reuse).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Round-to-nearest-even fp32 -> bf16, two values packed low|high (one
// v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// 2^x on the hardware exponential unit; exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The int8 cache rule for a row with maximum magnitude amax > 0: code of x
// is clamp(rint(x * (127 / amax)), -127, 127) and the row's scale is
// amax / 127, all in IEEE fp32 with correctly rounded division (a row of
// zeros has codes 0 and scale 0).  Shared by every kernel that quantises.
__device__ __forceinline__ float int8_inv(float amax) { return __fdiv_rn(127.f, amax); }
__device__ __forceinline__ int int8_code(float x, float inv) {
  const float c = rintf(__fmul_rn(x, inv));
  return (int)fminf(fmaxf(c, -127.f), 127.f);
}
__device__ __forceinline__ float int8_scale(float amax) { return __fdiv_rn(amax, 127.f); }


}  // namespace gqa
