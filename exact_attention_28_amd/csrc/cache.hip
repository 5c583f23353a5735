// cache.hip — appending a chunk of keys and values to a token-major KV cache
// (the [B, rows, Hkv, D] layout of the decode caches), keys rotated at their
// positions.  Positions continue the cached sequence: row t of the chunk is
// position L_b + t, the position_offset of scirs2-neural 0.4.4
// src/layers/grouped_query_attention.rs (RotaryPositionEmbedding::apply, and
// forward_with_cache appending to its cache).

#include "common.h"
#include "kernels.h"

namespace xattn {

// One 16-byte chunk (8 bf16) of K and of V per thread and step.
__global__ __launch_bounds__(256) void cache_append_kernel(
    const u16* __restrict__ k_new, const u16* __restrict__ v_new, u16* __restrict__ kcache,
    u16* __restrict__ vcache, const int* __restrict__ lens, long long nchunks, int Sq, int Hkv,
    int D, int rows, const double2* __restrict__ tab) {
  const int cpr = D / 8;
  for (long long c = blockIdx.x * (long long)blockDim.x + threadIdx.x; c < nchunks;
       c += (long long)gridDim.x * blockDim.x) {
    const long long row = c / cpr;  // (b, t, h) of the chunk tensors
    const int part = (int)(c % cpr);
    const int h = (int)(row % Hkv);
    const long long bt = row / Hkv;
    const int t = (int)(bt % Sq);
    const int b = (int)(bt / Sq);
    const int L = min(max(lens[b], 0), rows - Sq);
    const long long dst = ((((long long)b * rows + L + t) * Hkv + h) * D) + part * 8;
    u32x4 kw = *reinterpret_cast<const u32x4*>(k_new + c * 8);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(v_new + c * 8);
    if (tab != nullptr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double2 cs = tab[(long long)(L + t) * (D / 2) + part * 4 + e];
        double r0, r1;
        rotate_pair((double)bf16_lo(kw[e]), (double)bf16_hi(kw[e]), cs, r0, r1);
        kw[e] = f64_to_bf16_bits(r0) | (f64_to_bf16_bits(r1) << 16);
      }
    }
    *reinterpret_cast<u32x4*>(kcache + dst) = kw;
    *reinterpret_cast<u32x4*>(vcache + dst) = vw;
  }
}

hipError_t launch_cache_append(const void* k_new, const void* v_new, void* kcache, void* vcache,
                               const int* lens, int B, int Sq, int Hkv, int D, int rows,
                               const double2* tab, hipStream_t stream) {
  if (D % 8 != 0 || Sq > rows) return hipErrorInvalidValue;
  const long long n = (long long)B * Sq * Hkv * (D / 8);
  const int threads = 256;
  long long blocks = (n + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  cache_append_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
      static_cast<const u16*>(k_new), static_cast<const u16*>(v_new), static_cast<u16*>(kcache),
      static_cast<u16*>(vcache), lens, n, Sq, Hkv, D, rows, tab);
  return hipGetLastError();
}

}  // namespace xattn
