// rope.hip — rotary position embedding for gfx950.
//
// Interleaved pair rotation of scirs2-neural 0.4.4 (src/layers/
// grouped_query_attention.rs, RotaryPositionEmbedding::apply): pair (2i, 2i+1)
// of a token at position p turns by theta = p / base^(2i/D); the page evaluates
// theta, cos and sin in f64.  Here the (cos, sin) table is built once in fp64 on
// the device and the rotation itself is done in fp64, then rounded once to the
// storage format (nearest, ties to even).
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace xattn {

// Row t of the table holds (cos, sin) of theta = (pos0 + t) / base^(2i/D), i < D/2.
__global__ void rope_table_kernel(double2* __restrict__ tab, int pos0, int npos, int half, int D,
                                  double base) {
  const long long n = (long long)npos * half;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const int t = (int)(idx / half), i = (int)(idx % half);
    const double theta = (double)(pos0 + t) / pow(base, (2.0 * i) / (double)D);
    double s, c;
    sincos(theta, &s, &c);
    tab[idx] = make_double2(c, s);
  }
}

hipError_t launch_rope_table(double2* tab, int pos0, int npos, int D, double base,
                             hipStream_t stream) {
  const int half = D / 2;
  const long long n = (long long)npos * half;
  const int threads = 256;
  long long blocks = (n + threads - 1) / threads;
  if (blocks > 65535) blocks = 65535;
  if (blocks < 1) blocks = 1;
  rope_table_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(tab, pos0, npos, half, D,
                                                                         base);
  return hipGetLastError();
}

// 16-bit formats (T = __bf16 or _Float16), 4 pairs (16 bytes) per thread;
// needs D % 8 == 0.
template <typename T>
__global__ void rope_rotate_16x8(const u16* x, u16* y,
                                   long long nchunks, int S, int H, int D,
                                   const double2* __restrict__ tab) {
  const int cpr = D / 8;  // 16-byte chunks per head row
  const int half = D / 2;
  for (long long c = blockIdx.x * (long long)blockDim.x + threadIdx.x; c < nchunks;
       c += (long long)gridDim.x * blockDim.x) {
    const long long row = c / cpr;  // (b, t, h) flattened
    const int part = (int)(c % cpr);
    const int t = (int)((row / H) % S);
    const u32x4 w = *reinterpret_cast<const u32x4*>(x + c * 8);
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double2 cs = tab[(long long)t * half + part * 4 + e];
      double r0, r1;
      rotate_pair((double)Fmt16<T>::lo(w[e]), (double)Fmt16<T>::hi(w[e]), cs, r0, r1);
      r[e] = Fmt16<T>::from_f64(r0) | (Fmt16<T>::from_f64(r1) << 16);
    }
    *reinterpret_cast<u32x4*>(y + c * 8) = r;
  }
}

// Any even D: one pair per thread, a 16-bit format (T = __bf16 or _Float16: a
// uint32 holds the pair) or fp32 (T = float).  x and y may alias (in-place
// rotation): each thread reads, then writes, only its own pair.
template <typename T>
__global__ void rope_rotate_pair(const void* xv, void* yv,
                                 long long npairs, int S, int H, int D,
                                 const double2* __restrict__ tab) {
  const int half = D / 2;
  for (long long pidx = blockIdx.x * (long long)blockDim.x + threadIdx.x; pidx < npairs;
       pidx += (long long)gridDim.x * blockDim.x) {
    const long long row = pidx / half;
    const int i = (int)(pidx % half);
    const int t = (int)((row / H) % S);
    const double2 cs = tab[(long long)t * half + i];
    double r0, r1;
    if constexpr (sizeof(T) == 2) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(xv)[pidx];
      rotate_pair((double)Fmt16<T>::lo(w), (double)Fmt16<T>::hi(w), cs, r0, r1);
      reinterpret_cast<uint32_t*>(yv)[pidx] =
          Fmt16<T>::from_f64(r0) | (Fmt16<T>::from_f64(r1) << 16);
    } else {
      const float2 w = reinterpret_cast<const float2*>(xv)[pidx];
      rotate_pair((double)w.x, (double)w.y, cs, r0, r1);
      reinterpret_cast<float2*>(yv)[pidx] = make_float2((float)r0, (float)r1);
    }
  }
}

// Queries and keys of an attention call in one launch (16-bit formats,
// D % 8 == 0): block (t, b) rotates, when q is given, query row t of batch b
// (Hq heads) at position Skv - Sq + t (bottom-right alignment) and, when k is
// given, key row t (Hkv heads) at position t.  A row is D / 8 chunks of 16
// bytes, one per thread; the token index comes from the grid, so no thread
// divides a 64-bit index.
template <typename T>
__global__ void rope_rotate_qk16(const u16* __restrict__ q, u16* __restrict__ qo, int Sq, int Hq,
                                 const u16* __restrict__ k, u16* __restrict__ ko, int Skv,
                                 int Hkv, int D, const double2* __restrict__ tab) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int cpr = D / 8, half = D / 2;
  auto rotate_row = [&](const u16* x, u16* y, int nchunks, const double2* trow) {
    for (int c = threadIdx.x; c < nchunks; c += blockDim.x) {
      const int part = c % cpr;
      const u32x4 w = *reinterpret_cast<const u32x4*>(x + (long long)c * 8);
      u32x4 r;
      // bf16: through fp32 (bf16_mid_key), the rare chunk with a value on a
      // bf16 midpoint redone with the single rounding
      constexpr bool VIA32 = std::is_same<T, __bf16>::value;
      double r0[4], r1[4];
      uint32_t mid = 1;  // 0 once a value lands on a bf16 midpoint
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rotate_pair((double)Fmt16<T>::lo(w[e]), (double)Fmt16<T>::hi(w[e]), trow[part * 4 + e],
                    r0[e], r1[e]);
        if constexpr (VIA32) {
          float f0 = (float)r0[e], f1 = (float)r1[e];
          // (opaque: the compiler would fuse the two conversions into its own
          // single-rounding sequence, which costs more)
          asm("" : "+v"(f0), "+v"(f1));
          mid = min(mid, min(bf16_mid_key(f0), bf16_mid_key(f1)));
          r[e] = Fmt16<T>::pack(f0, f1);
        } else {
          r[e] = Fmt16<T>::from_f64(r0[e]) | (Fmt16<T>::from_f64(r1[e]) << 16);
        }
      }
      if (VIA32 && mid == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r[e] = Fmt16<T>::from_f64(r0[e]) | (Fmt16<T>::from_f64(r1[e]) << 16);
      }
      *reinterpret_cast<u32x4*>(y + (long long)c * 8) = r;
    }
  };
  if (q != nullptr && t < Sq) {
    const long long row = ((long long)b * Sq + t) * Hq * D;
    rotate_row(q + row, qo + row, Hq * cpr, tab + (long long)(Skv - Sq + t) * half);
  }
  if (k != nullptr && t < Skv) {
    const long long row = ((long long)b * Skv + t) * Hkv * D;
    rotate_row(k + row, ko + row, Hkv * cpr, tab + (long long)t * half);
  }
}

hipError_t launch_rope_rotate_qk(const void* q, void* qo, int B, int Sq, int Hq, const void* k,
                                 void* ko, int Skv, int Hkv, int D, const double2* tab, int dtype,
                                 hipStream_t stream) {
  if ((dtype != 1 && dtype != 2) || D % 8 != 0 || B > 65535 || (q && Sq > Skv))
    return hipErrorInvalidValue;
  const int rows = max(q ? Sq : 0, k ? Skv : 0);
  const int most = max(q ? Hq : 0, k ? Hkv : 0) * (D / 8);  // chunks of the widest row
  if (rows == 0) return hipSuccess;
  const int threads = min(256, (most + 63) / 64 * 64);
  const dim3 grid((unsigned)rows, (unsigned)B);
  if (dtype == 1)
    rope_rotate_qk16<__bf16><<<grid, dim3(threads), 0, stream>>>(
        static_cast<const u16*>(q), static_cast<u16*>(qo), Sq, Hq, static_cast<const u16*>(k),
        static_cast<u16*>(ko), Skv, Hkv, D, tab);
  else
    rope_rotate_qk16<_Float16><<<grid, dim3(threads), 0, stream>>>(
        static_cast<const u16*>(q), static_cast<u16*>(qo), Sq, Hq, static_cast<const u16*>(k),
        static_cast<u16*>(ko), Skv, Hkv, D, tab);
  return hipGetLastError();
}

hipError_t launch_rope_rotate(const void* x, void* y, int B, int S, int H, int D,
                              const double2* tab, int dtype, hipStream_t stream) {
  const long long rows = (long long)B * S * H;
  const int threads = 256;
  const long long max_blocks = 256LL * 8 * 4;  // a few resident waves per SIMD, grid-stride
  if (dtype != 0 && dtype != 1 && dtype != 2) return hipErrorInvalidValue;
  if (dtype != 0 && D % 8 == 0) {
    const long long n = rows * (D / 8);
    long long blocks = (n + threads - 1) / threads;
    if (blocks > max_blocks) blocks = max_blocks;
    if (dtype == 1)
      rope_rotate_16x8<__bf16><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
          static_cast<const u16*>(x), static_cast<u16*>(y), n, S, H, D, tab);
    else
      rope_rotate_16x8<_Float16><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
          static_cast<const u16*>(x), static_cast<u16*>(y), n, S, H, D, tab);
  } else {
    const long long n = rows * (D / 2);
    long long blocks = (n + threads - 1) / threads;
    if (blocks > max_blocks) blocks = max_blocks;
    if (dtype == 1)
      rope_rotate_pair<__bf16><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
          x, y, n, S, H, D, tab);
    else if (dtype == 2)
      rope_rotate_pair<_Float16><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
          x, y, n, S, H, D, tab);
    else
      rope_rotate_pair<float><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
          x, y, n, S, H, D, tab);
  }
  return hipGetLastError();
}

}  // namespace xattn
