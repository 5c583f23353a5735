// pad.hip — head dims other than the kernels' 64 and 128: the inputs are
// copied into a zero-padded head dim (64 when D <= 64, else 128), with Q and K
// rotated on the way for RoPE (angles of the true D), the attention kernel
// runs at the padded width, and O's first D columns are copied back.  Zero
// columns add nothing to the scores and V's zero columns give zero output
// columns, so this is exact attention at the true D.  (whisper-apr 0.3.1
// src/model/lfm2/gqa.rs pads Moonshine's 36 to 40 the same way, with a Q
// correction for SDPA's 1/sqrt(padded) scale that the explicit scale here
// makes unnecessary.)

#include "common.h"
#include "kernels.h"

namespace xattn {

// y [rows, Dp] from x [rows, D] (rows = (b, t, h) of a [B, S, H, D] tensor):
// columns >= D are zero; with tab, pair i < D/2 of token t is rotated by table
// row pos0 + t (fp64, rounded once to the element type T: __bf16, _Float16 or
// float).
template <typename T>
__global__ __launch_bounds__(256) void pack_heads_kernel(const void* __restrict__ xv,
                                                         void* __restrict__ yv, long long n, int S,
                                                         int H, int D, int Dp,
                                                         const double2* __restrict__ tab,
                                                         int pos0) {
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / Dp;
    const int d = (int)(e % Dp);
    double val = 0.0;
    auto ld = [&](int c) -> double {
      const long long i = row * D + c;
      if constexpr (sizeof(T) == 2)
        return (double)Fmt16<T>::lo(static_cast<const u16*>(xv)[i]);
      else
        return (double)static_cast<const float*>(xv)[i];
    };
    if (d < D) {
      if (tab != nullptr) {
        const int t = (int)((row / H) % S);
        const double2 cs = tab[(long long)(pos0 + t) * (D / 2) + d / 2];
        double r0, r1;
        rotate_pair(ld(d & ~1), ld(d | 1), cs, r0, r1);
        val = (d & 1) ? r1 : r0;
      } else {
        val = ld(d);
      }
    }
    if constexpr (sizeof(T) == 2)
      static_cast<u16*>(yv)[e] = (u16)Fmt16<T>::from_f64(val);
    else
      static_cast<float*>(yv)[e] = (float)val;
  }
}

// o [rows, D] = first D columns of op [rows, Dp]
template <typename T>
__global__ __launch_bounds__(256) void unpack_heads_kernel(const T* __restrict__ op,
                                                           T* __restrict__ o, long long n, int D,
                                                           int Dp) {
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x)
    o[e] = op[(e / D) * Dp + e % D];
}

namespace {
unsigned grid_for(long long n) {
  long long b = (n + 255) / 256;
  return (unsigned)(b > 65536 ? 65536 : (b < 1 ? 1 : b));
}
}  // namespace

hipError_t launch_pack_heads(const void* x, void* y, int B, int S, int H, int D, int Dp,
                             const double2* tab, int pos0, int dtype, hipStream_t stream) {
  const long long n = (long long)B * S * H * Dp;
  if (dtype == 1)
    pack_heads_kernel<__bf16><<<grid_for(n), 256, 0, stream>>>(x, y, n, S, H, D, Dp, tab, pos0);
  else if (dtype == 2)
    pack_heads_kernel<_Float16><<<grid_for(n), 256, 0, stream>>>(x, y, n, S, H, D, Dp, tab, pos0);
  else
    pack_heads_kernel<float><<<grid_for(n), 256, 0, stream>>>(x, y, n, S, H, D, Dp, tab, pos0);
  return hipGetLastError();
}

hipError_t launch_unpack_heads(const void* op, void* o, long long rows, int D, int Dp, int dtype,
                               hipStream_t stream) {
  const long long n = rows * D;
  if (dtype == 1 || dtype == 2)
    unpack_heads_kernel<u16><<<grid_for(n), 256, 0, stream>>>(static_cast<const u16*>(op),
                                                              static_cast<u16*>(o), n, D, Dp);
  else
    unpack_heads_kernel<float><<<grid_for(n), 256, 0, stream>>>(static_cast<const float*>(op),
                                                                static_cast<float*>(o), n, D, Dp);
  return hipGetLastError();
}

}  // namespace xattn
