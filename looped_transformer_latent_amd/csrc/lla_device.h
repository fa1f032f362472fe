// Device-side helpers shared by the LLA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lla {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16 bit pattern, round to nearest even, through the compiler's
// float -> __bf16 conversion (one v_cvt_pk_bf16_f32 on gfx950).  For every
// non-NaN input the result equals the integer rounding (u + 0x7FFF + bit 16 of
// u) >> 16 of the fp32 bit pattern u, denormals included (all 2^32 patterns
// were compared on the device); a NaN gives a NaN.  Scalar conversions on
// purpose: the two-lane vector conversion has been seen to lose one lane under
// optimisation, and a hand-written instruction would bypass the compiler's
// wait-state insertion (e.g. after a transcendental op).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 2^x on the hardware exp unit.  Used for softmax weights, whose arguments are
// <= 0; results below the fp32 normal range may flush to zero, which only drops
// weights smaller than 2^-126 of the largest one.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations within 16-lane rows.
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror (lane i <-> 7 - i within 8)
constexpr int kDppMirror = 0x140;     // row_mirror (lane i <-> 15 - i within 16)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max over the 16 lanes of each row; every lane of the row gets the result.
// One fused DPP max per step (the compiler's fmaxf would add a move and a NaN
// canonicalisation per step).  Each step first waits the 2 wait states a DPP
// read of a just-written VGPR requires.  Inputs are finite or -inf.
__device__ __forceinline__ float max_in_row(float x) {
  asm volatile(
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf"
      : "+v"(x));
  return x;
}
__device__ __forceinline__ float sum_in_row(float x) {
  x += dpp<kDppQuadSwap1>(x);
  x += dpp<kDppQuadSwap2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return x;
}

// Sum over the four 16-lane rows (lanes l, l^16, l^32, l^48) with the gfx950
// row-swap permutes: after the 32-lane swap each lane holds rows {0+2, 1+3},
// after the 16-lane swap all four.
__device__ __forceinline__ float sum_across_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const uint32_t v = __float_as_uint(y);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ __forceinline__ float max_in_wave(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

}  // namespace lla
