// lds.h — buffer resources, direct HBM->LDS loads and LDS transpose reads on
// gfx950, shared by the MFMA attention kernels.
#pragma once

#include "common.h"

namespace xattn {

// Word 3 of a gfx9 buffer resource for raw (unformatted, stride 0) 32-bit access.
constexpr int kBufferWord3 = 0x00020000;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i mod 4) of the 8-byte chunks addressed by lanes i/4 + 4e, e = 0..3.  When
// lane L of a group addresses row r0 + L/4, columns c0 + 4(L mod 4) .. +3 of a
// row-major bf16 tile, lane i receives rows r0 .. r0+3 of column c0 + i.
__device__ __forceinline__ s16x4 lds_read_tr16(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) char*)(p));
}

// s_waitcnt with vmcnt(0) and the other counters unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;
// s_waitcnt with lgkmcnt(0) (LDS and scalar loads) and the others unconstrained.
constexpr int kWaitLgkm0 = 0xC07F;

__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(u16* p) {
  return (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) char*)(p));
}

// Direct HBM->LDS loads: instruction i writes lane l's 16 bytes (buffer offset
// off[i] + t0) to dst + 1 KiB * i + 16 l.  (A plain device function: the
// gfx950 LDS-load builtin cannot sit in a lambda, which is also compiled for
// the host.)
template <int LD>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t rsrc, u16* dst, const uint32_t* off,
                                         uint32_t t0) {
#pragma unroll
  for (int i = 0; i < LD; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_ptr(dst + i * 64 * 8), 16, off[i] + t0, 0, 0, 0);
}

// Chunk swizzles (16-byte chunks, XORed with a function of the row).  LDS has
// 64 four-byte banks, i.e. 16 groups of one chunk.  K fragments are read 16 rows
// at a time at one logical chunk: the 16 (row, chunk) must fall in 16 distinct
// groups.  V fragments are read by transpose reads covering 4 consecutive rows
// (a multiple of 4 first) x 2 adjacent chunks (an even first): 8 distinct groups.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return (D == 64) ? ((row >> 1) & 7) : (row & 15);  // group = (row*KCH + chunk) mod 16
}
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return (D == 64) ? (2 * ((row >> 1) & 3)) : (2 * (row & 3));
}

// Direct HBM->LDS loads of one wave's share of a K and a V tile: instruction i
// fills the 64 consecutive 16-byte slots starting at kdst/vdst + 1 KiB * i.
// (A plain device function: the gfx950 LDS-load builtin cannot sit in a lambda,
// which is also compiled for the host.)
template <int LD>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                         u16* kdst, u16* vdst, const uint32_t* koff,
                                         const uint32_t* voff, uint32_t t0) {
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, lds_ptr(kdst + i * 64 * 8), 16, koff[i] + t0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, lds_ptr(vdst + i * 64 * 8), 16, voff[i] + t0, 0, 0, 0);
  }
}

}  // namespace xattn
