// common.h — device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bit pattern -> fp32 (exact: bf16 is the top half of a binary32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (nearest, ties to even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// fp64 -> bf16 bits, nearest with ties to even, in one rounding: round the
// binary64 significand to 8 bits (drop 45 of its 52 stored bits), after which
// the value is exactly representable in binary32 and in bf16.  Finite values
// in the normal bf16 range only (rotated attention inputs are).
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  uint64_t u = __double_as_longlong(x);
  const uint64_t lsb = (u >> 45) & 1ull;
  u += 0x00000FFFFFFFFFFFull + lsb;  // 2^44 - 1 + lsb
  u &= ~0x00001FFFFFFFFFFFull;       // clear the 45 dropped bits
  return __float_as_uint((float)__longlong_as_double(u)) >> 16;
}

// Rotate one interleaved pair by the angle whose (cos, sin) is cs, in fp64.
__device__ __forceinline__ void rotate_pair(double x0, double x1, double2 cs, double& r0,
                                            double& r1) {
  r0 = x0 * cs.x - x1 * cs.y;
  r1 = x0 * cs.y + x1 * cs.x;
}

// Sum over groups of N consecutive lanes (N in 2,4,8,16) with DPP moves.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  // quad_perm [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  if (N >= 4)  // quad_perm [2,3,0,1]
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if (N >= 8)  // row_half_mirror: lane i <- lane 7-i within each 8
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  if (N >= 16)  // row_mirror: lane i <- lane 15-i within each 16
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

}  // namespace xattn
