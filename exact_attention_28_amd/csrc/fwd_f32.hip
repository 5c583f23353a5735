// fwd_f32.hip — fp32 exact attention forward for gfx950 (fp32 inputs end to end).
//
// The loop structure is the tiled forward of scirs2-neural 0.4.3
// (src/layers/flash_attention.rs, fn flash_attention_forward): one workgroup per
// block of 64 query rows, key/value blocks inside, a running row max m and row
// sum l updated by fn online_softmax_update, the causal skip of key blocks that
// lie wholly after the block's last query, and the final division by l.
// Each query row is owned by LPR lanes (each holds D / LPR of its columns;
// the dot products are summed across them by DPP moves), so the row
// statistics stay in registers; K/V tiles are staged in LDS and read as
// broadcasts.  LPR = 2 (64 rows per workgroup) in general; LPR = 8 (16 rows)
// or 16 (8 rows) when that grid would leave most CUs idle, which cuts each
// lane's serial work per key several times for small problems.  fp32 has no dense MFMA advantage worth the fragment plumbing at
// these sizes, so this path is plain VALU fp32.
#include "common.h"
#include "kernels.h"

namespace xattn {

template <int D, bool CAUSAL, bool ROPE, int LPR>
__global__ __launch_bounds__(128) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Sq, int Skv,
    float scale_log2, const double2* __restrict__ tab, MaskView mask) {
  constexpr int BQ = 128 / LPR;
  constexpr int BK = (D == 64) ? 64 : 32;
  constexpr int HD = D / LPR;  // columns per lane
  __shared__ float Ks[BK][D];
  __shared__ float Vs[BK][D];

  const int t = threadIdx.x;
  const int r = t / LPR, half = t % LPR;  // row of the block, part of the row
  const int q0 = blockIdx.x * BQ;
  const int i = q0 + r;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int off = Skv - Sq;  // bottom-right causal alignment

  float q[HD], o[HD];
  {
    const long long base = (((long long)b * Sq + (i < Sq ? i : 0)) * Hq + h) * D + half * HD;
#pragma unroll
    for (int d = 0; d < HD; ++d) q[d] = (i < Sq) ? Q[base + d] : 0.f;
    if (ROPE && i < Sq) {
      const int pos = off + i;
#pragma unroll
      for (int d = 0; d < HD; d += 2) {
        double r0, r1;
        rotate_pair((double)q[d], (double)q[d + 1], tab[(long long)pos * (D / 2) + (half * HD + d) / 2],
                    r0, r1);
        q[d] = (float)r0;
        q[d + 1] = (float)r1;
      }
    }
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  // this row's additive mask (the [WH] compute_block_scores mask term), or null
  const float* mrow =
      mask.p ? mask.p + b * mask.bs + h * mask.hs + (long long)(i < Sq ? i : 0) * mask.rs : nullptr;

  int kv_end = Skv;
  if (CAUSAL) {
    const int last_q = min(q0 + BQ, Sq) - 1;
    kv_end = min(Skv, last_q + off + 1);
  }
  for (int k0 = 0; k0 < kv_end; k0 += BK) {
    __syncthreads();
    // stage the key/value block (rows past Skv are zero)
    for (int e = t; e < BK * D / 2; e += 128) {
      const int jj = e / (D / 2), pr = e % (D / 2);
      const int j = k0 + jj;
      float2 kv = make_float2(0.f, 0.f), vv = make_float2(0.f, 0.f);
      if (j < Skv) {
        const long long src = (((long long)b * Skv + j) * Hkv + g) * D + 2 * pr;
        kv = *reinterpret_cast<const float2*>(K + src);
        vv = *reinterpret_cast<const float2*>(V + src);
        if (ROPE) {
          double r0, r1;
          rotate_pair((double)kv.x, (double)kv.y, tab[(long long)j * (D / 2) + pr], r0, r1);
          kv = make_float2((float)r0, (float)r1);
        }
      }
      Ks[jj][2 * pr] = kv.x;
      Ks[jj][2 * pr + 1] = kv.y;
      Vs[jj][2 * pr] = vv.x;
      Vs[jj][2 * pr + 1] = vv.y;
    }
    __syncthreads();

    float s[BK];
    float bmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < BK; ++jj) {
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) part = fmaf(q[d], Ks[jj][half * HD + d], part);
      const int j = k0 + jj;
      // the row's lanes all get the same sum (DPP butterfly, same operand
      // order on every lane), so their softmax statistics agree bit for bit
      const float dot = group_sum<LPR>(part);
      float x = dot * scale_log2;
      if (mrow != nullptr && j < Skv) x = fmaf(dot, scale_log2, mrow[j] * kLog2e);
      if (j >= Skv || (CAUSAL && j > i + off)) x = -INFINITY;
      s[jj] = x;
      bmax = fmaxf(bmax, x);
    }
    const float m_new = fmaxf(m, bmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float corr = exp2f(m - m_use);  // 0 while m is -inf
    l *= corr;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] *= corr;
#pragma unroll
    for (int jj = 0; jj < BK; ++jj) {
      const float p = exp2f(s[jj] - m_use);
      l += p;
#pragma unroll
      for (int d = 0; d < HD; ++d) o[d] = fmaf(p, Vs[jj][half * HD + d], o[d]);
    }
    m = m_new;
  }

  if (i < Sq) {
    const long long base = (((long long)b * Sq + i) * Hq + h) * D + half * HD;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) O[base + d] = o[d] * inv;
    if (LSE != nullptr && half == 0)
      LSE[((long long)b * Hq + h) * Sq + i] = (l > 0.f) ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool ROPE, int LPR>
static hipError_t go_f32_lpr(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int Hq, int Hkv, int Sq, int Skv, float scale,
                             const double2* tab, MaskView mask, hipStream_t stream) {
  constexpr int BQ = 128 / LPR;
  dim3 grid((Sq + BQ - 1) / BQ, Hq, B);
  fwd_f32_kernel<D, CAUSAL, ROPE, LPR><<<grid, dim3(128), 0, stream>>>(
      static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      static_cast<float*>(o), lse, Hq, Hkv, Sq, Skv, scale * kLog2e, tab, mask);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool ROPE>
static hipError_t go_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int Hq, int Hkv, int Sq, int Skv, float scale, const double2* tab,
                         MaskView mask, hipStream_t stream) {
  // fewer 64-row workgroups than CUs: 8 lanes per row (16 rows per
  // workgroup), or 16 (8 rows) when there are fewer than a quarter as many
  const long long wg = (long long)((Sq + 63) / 64) * Hq * B;
  if (wg < 64)
    return go_f32_lpr<D, CAUSAL, ROPE, 16>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, mask,
                                           stream);
  if (wg < 256)
    return go_f32_lpr<D, CAUSAL, ROPE, 8>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, mask,
                                          stream);
  return go_f32_lpr<D, CAUSAL, ROPE, 2>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, mask,
                                        stream);
}

hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                          const double2* rope_tab, hipStream_t stream, MaskView mask) {
  const bool rope = rope_tab != nullptr;
#define XATTN_F32_CASE(DD, C, R)                                                           \
  if (D == DD && (causal != 0) == C && rope == R)                                        \
    return go_f32<DD, C, R>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, rope_tab, mask, stream);
  XATTN_F32_CASE(64, false, false)
  XATTN_F32_CASE(64, true, false)
  XATTN_F32_CASE(64, false, true)
  XATTN_F32_CASE(64, true, true)
  XATTN_F32_CASE(128, false, false)
  XATTN_F32_CASE(128, true, false)
  XATTN_F32_CASE(128, false, true)
  XATTN_F32_CASE(128, true, true)
#undef XATTN_F32_CASE
  return hipErrorInvalidValue;
}

}  // namespace xattn
