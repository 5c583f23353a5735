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
// broadcasts.  LPR = 4 (32 rows per workgroup) in general; LPR = 8 (16 rows)
// or 16 (8 rows) when a grid of 64-row blocks would leave most CUs idle, which
// cuts each lane's serial work per key several times for small problems.  fp32 has no
// dense MFMA advantage worth the fragment plumbing at these sizes, so this
// path is plain VALU fp32.
#include "common.h"
#include "kernels.h"

namespace xattn {

// LDS of one workgroup: a key and a value block, and with a mask its tile
// (rows padded by one entry so that the rows one wave reads sit in different
// banks).  The unmasked kernels carry no mask tile (32 KiB of LDS).
template <int BQ, int BK, int D, bool MASK>
struct alignas(16) F32Tiles {
  float k[BK][D];
  float v[BK][D];
  float m[BQ][BK + 1];
};
template <int BQ, int BK, int D>
struct alignas(16) F32Tiles<BQ, BK, D, false> {
  float k[BK][D];
  float v[BK][D];
};

template <int D, bool CAUSAL, bool ROPE, int LPR, bool MASK>
__global__ __launch_bounds__(128) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Sq, int Skv,
    float scale_log2, const double2* __restrict__ tab, MaskView mask) {
  constexpr int BQ = 128 / LPR;
  constexpr int BK = (D == 64) ? 64 : 32;
  constexpr int HD = D / LPR;        // columns per lane
  constexpr int CPR = D / 4;         // 16-byte chunks per key row
  constexpr int NCH = BK * CPR / 128;  // chunks of K (and of V) per thread and block
  constexpr int MPT = BQ * BK / 128;   // mask entries per thread and block
  static_assert(NCH * 128 == BK * CPR && MPT * 128 == BQ * BK, "block shape");
  __shared__ F32Tiles<BQ, BK, D, MASK> sm;
  auto& Ks = sm.k;
  auto& Vs = sm.v;

  const int t = threadIdx.x;
  const int r = t / LPR, half = t % LPR;  // row of the block, part of the row
  const int q0 = blockIdx.x * BQ;
  const int i = q0 + r;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int off = Skv - Sq;  // bottom-right causal alignment

  // Key/value blocks (and mask tiles) pass through registers into LDS, every
  // load of a block issued before the first wait.  With 8 or 16 lanes per row
  // (grids too small to hide latency by occupancy) the next block is fetched
  // while the current one is used; with 4 the loads of a block are issued
  // before the barrier that precedes its staging, so that the registers are
  // free during the arithmetic.  Rows past Skv are zero (mask entries 0).
  constexpr bool kAhead = LPR >= 8;
  float4 kr[NCH], vr[NCH];
  float mr[MASK ? MPT : 1];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = t + 128 * c;
      const int j = k0 + e / CPR;
      const long long src = (((long long)b * Skv + min(j, Skv - 1)) * Hkv + g) * D + 4 * (e % CPR);
      kr[c] = *reinterpret_cast<const float4*>(K + src);
      vr[c] = *reinterpret_cast<const float4*>(V + src);
    }
    if constexpr (MASK) {
#pragma unroll
      for (int c = 0; c < MPT; ++c) {
        const int e = t + 128 * c;
        const int mi = min(q0 + e / BK, Sq - 1), j = k0 + e % BK;
        mr[c] = (j < Skv) ? mask.p[b * mask.bs + h * mask.hs + (long long)mi * mask.rs + j] : 0.f;
      }
    }
  };
  auto stage = [&](int k0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = t + 128 * c;
      const int jj = e / CPR, cc = e % CPR;
      const int j = k0 + jj;
      float4 kv = kr[c], vv = vr[c];
      if (ROPE) {
        // table rows read unconditionally (clamped), so that every load of
        // the block is issued before the first rotation waits
        const double2* trow = tab + (long long)min(j, Skv - 1) * (D / 2) + 2 * cc;
        const double2 cs0 = trow[0], cs1 = trow[1];
        double r0, r1;
        rotate_pair((double)kv.x, (double)kv.y, cs0, r0, r1);
        kv.x = (float)r0;
        kv.y = (float)r1;
        rotate_pair((double)kv.z, (double)kv.w, cs1, r0, r1);
        kv.z = (float)r0;
        kv.w = (float)r1;
      }
      if (j >= Skv) {
        kv = make_float4(0.f, 0.f, 0.f, 0.f);
        vv = kv;
      }
      *reinterpret_cast<float4*>(&Ks[jj][4 * cc]) = kv;
      *reinterpret_cast<float4*>(&Vs[jj][4 * cc]) = vv;
    }
    if constexpr (MASK) {
#pragma unroll
      for (int c = 0; c < MPT; ++c) {
        const int e = t + 128 * c;
        sm.m[e / BK][e % BK] = mr[c];
      }
    }
  };

  float q[HD], o[HD];
  {
    const long long base = (((long long)b * Sq + min(i, Sq - 1)) * Hq + h) * D + half * HD;
#pragma unroll
    for (int d = 0; d < HD; d += 4) {
      const float4 x = *reinterpret_cast<const float4*>(Q + base + d);
      q[d] = x.x;
      q[d + 1] = x.y;
      q[d + 2] = x.z;
      q[d + 3] = x.w;
    }
    if (ROPE) {
      const double2* trow = tab + (long long)(off + min(i, Sq - 1)) * (D / 2) + half * HD / 2;
#pragma unroll
      for (int d = 0; d < HD; d += 2) {
        double r0, r1;
        rotate_pair((double)q[d], (double)q[d + 1], trow[d / 2], r0, r1);
        q[d] = (float)r0;
        q[d + 1] = (float)r1;
      }
    }
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int kv_end = Skv;
  if (CAUSAL) {
    const int last_q = min(q0 + BQ, Sq) - 1;
    kv_end = min(Skv, last_q + off + 1);
  }
  if (kAhead && kv_end > 0) fetch(0);
  for (int k0 = 0; k0 < kv_end; k0 += BK) {
    if (!kAhead) fetch(k0);
    __syncthreads();  // every wave is done with the previous block
    stage(k0);
    __syncthreads();
    if (kAhead && k0 + BK < kv_end) fetch(k0 + BK);

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
      // the row's additive mask (the [WH] compute_block_scores mask term)
      if constexpr (MASK) {
        if (j < Skv) x = fmaf(dot, scale_log2, sm.m[r][jj] * kLog2e);
      }
      if (j >= Skv || (CAUSAL && j > i + off)) x = -INFINITY;
      s[jj] = x;
      bmax = fmaxf(bmax, x);
      // key-major order: with 32 or more columns per lane the compiler may
      // otherwise turn the loop inside out (four columns of every key at a
      // time) and then wait for each LDS read before the next
      if constexpr (HD >= 32) asm volatile("" ::: "memory");
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
      if constexpr (HD >= 32) asm volatile("" ::: "memory");  // key-major, as above
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
  const float* qf = static_cast<const float*>(q);
  const float* kf = static_cast<const float*>(k);
  const float* vf = static_cast<const float*>(v);
  if (mask.p != nullptr)
    launch_kernel(fwd_f32_kernel<D, CAUSAL, ROPE, LPR, true>, grid, dim3(128), stream, qf, kf, vf,
                  static_cast<float*>(o), lse, Hq, Hkv, Sq, Skv, scale * kLog2e, tab, mask);
  else
    launch_kernel(fwd_f32_kernel<D, CAUSAL, ROPE, LPR, false>, grid, dim3(128), stream, qf, kf, vf,
                  static_cast<float*>(o), lse, Hq, Hkv, Sq, Skv, scale * kLog2e, tab, mask);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool ROPE>
static hipError_t go_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int Hq, int Hkv, int Sq, int Skv, float scale, const double2* tab,
                         MaskView mask, hipStream_t stream) {
  // counted in 64-row blocks: fewer than there are CUs, 8 lanes per row (16
  // rows per workgroup), or 16 (8 rows) below a quarter of that; else 4 (32)
  const long long wg = (long long)((Sq + 63) / 64) * Hq * B;
  if (wg < 64)
    return go_f32_lpr<D, CAUSAL, ROPE, 16>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, mask,
                                           stream);
  if (wg < 256)
    return go_f32_lpr<D, CAUSAL, ROPE, 8>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, mask,
                                          stream);
  return go_f32_lpr<D, CAUSAL, ROPE, 4>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, mask,
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
