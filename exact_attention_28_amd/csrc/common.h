// common.h — device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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

// IEEE binary16 bit patterns -> fp32 (exact: every binary16 value, subnormals
// included, is a binary32 value; v_cvt_f32_f16).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// Two fp32 -> packed binary16 pair (nearest, ties to even; v_cvt_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 r;
  r[0] = (_Float16)lo;
  r[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// fp64 -> binary16 bits, nearest with ties to even, in one rounding.  At or
// above 2^-14 (binary16's normal range) the binary64 significand is rounded to
// 11 bits (42 of its 52 stored bits dropped); below, the value is rounded to a
// multiple of 2^-24, the subnormal spacing.  Either way the result is exact in
// binary32 and, up to 65504, in binary16; a value that rounded to 65536 or more
// converts to an infinity, as in binary16's own rounding.
__host__ __device__ __forceinline__ uint32_t f64_to_f16_bits(double x) {
  double y;
  if (__builtin_fabs(x) < 0x1p-14) {
    y = __builtin_rint(x * 0x1p24) * 0x1p-24;
  } else {
    uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint64_t lsb = (u >> 42) & 1ull;
    u += 0x000001FFFFFFFFFFull + lsb;  // 2^41 - 1 + lsb
    u &= ~0x000003FFFFFFFFFFull;       // clear the 42 dropped bits
    y = __builtin_bit_cast(double, u);
  }
  return __builtin_bit_cast(unsigned short, (_Float16)(float)y);
}

// The two 16-bit input formats of the MFMA kernels: how a stored pair widens,
// how an fp64 value and a pair of fp32 values round to it, and the matching
// 32x32x16 matrix instruction (fp32 accumulation).
template <typename T>
struct Fmt16;
template <>
struct Fmt16<__bf16> {
  typedef bf16x8 v8;
  static __device__ __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
  static __device__ __forceinline__ uint32_t from_f64(double x) { return f64_to_bf16_bits(x); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16(a, b); }
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Fmt16<_Float16> {
  typedef f16x8 v8;
  static __device__ __forceinline__ float lo(uint32_t w) { return f16_lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return f16_hi(w); }
  static __device__ __forceinline__ uint32_t from_f64(double x) { return f64_to_f16_bits(x); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16(a, b); }
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Rotate one interleaved pair by the angle whose (cos, sin) is cs, in fp64.
__device__ __forceinline__ void rotate_pair(double x0, double x1, double2 cs, double& r0,
                                            double& r1) {
  r0 = x0 * cs.x - x1 * cs.y;
  r1 = x0 * cs.y + x1 * cs.x;
}

// fp64 -> bf16 through fp32 (v_cvt_f32_f64, then the packing instruction, both
// nearest with ties to even) rounds twice.  That equals the single rounding of
// f64_to_bf16_bits except when the fp32 value is itself a bf16 midpoint: every
// bf16 midpoint is an fp32 value, so the fp32 value nearest to x lies on the
// same side of each midpoint as x unless it is one.  bf16_mid_key(f) is 0
// exactly for a midpoint (low 16 bits 0x8000); callers take the minimum over
// their values, convert through fp32, and redo with f64_to_bf16_bits when it
// is 0.
__device__ __forceinline__ uint32_t bf16_mid_key(float f) {
  return (__float_as_uint(f) ^ 0x8000u) & 0xffffu;
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
