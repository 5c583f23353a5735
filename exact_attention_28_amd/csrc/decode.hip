// decode.hip — split-KV flash-decoding for gfx950.
//
// What is computed follows oxibonsai-model 0.1.4 (src/layers/flash_decode.rs):
// the key/value positions of a sequence are cut into tiles (splits); each tile
// yields its own normalised output and log-sum-exp (fn flash_decode_tile), and
// a second pass merges the tiles, weighting each by exp(lse_i - lse), with
// tiles of non-finite lse dropped (fn combine_tile_outputs).  The cache is the
// token-major [B, Smax, Hkv, D] layout of that page's fn
// flash_decode_multi_head and of whisper-apr 0.3.1 src/model/lfm2/gqa.rs
// (KvCache); query head h reads kv head h / (Hq / Hkv) (fn attention_cached).
//
// How it runs on CDNA4: one workgroup per (split, group of GW query heads
// sharing one kv head, batch).  The pass is HBM-bound (each cached K/V byte is
// read once and feeds GW heads), so the kernel is built for bytes in flight:
// D/8 lanes cover one 16-byte slice each of a token's K and V rows, a wave
// takes 64/(D/8) tokens per sub-step and kDecUnroll sub-steps per step, and
// the loads of the next step are in flight while a step is consumed.  Dot
// products are fp32 FMAs reduced across the D/8 lanes with DPP; the online softmax keeps a reference
// maximum per lane and rescales only when a score exceeds it by more than 2^8
// in the exp2 domain (the final O / l and m + log2 l are the same for any
// reference, so this is exact).  Partial states of the lanes and waves of a
// workgroup are merged in registers and LDS before one write per split.
#include "common.h"
#include "kernels.h"

namespace xattn {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecUnroll = 4;
constexpr int kMaxSplits = 64;

// workspace: partial O [B][Hq][ns][D] fp32, then lse [B][Hq][ns] fp32
size_t decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
  const size_t n = (size_t)B * Hq * num_splits * (D + 1) * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float m2, float l2,
                                            const float* acc2) {
  const float M = fmaxf(m, m2);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  const float a = __builtin_amdgcn_exp2f(m - Mu), b = __builtin_amdgcn_exp2f(m2 - Mu);
  l = l * a + l2 * b;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a + acc2[e] * b;
  m = M;
}

template <int D, int GW>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const u16* __restrict__ Qg, const u16* __restrict__ Kc, const u16* __restrict__ Vc,
    const int* __restrict__ seqlens, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    int Hq, int Hkv, int Smax, int ns, float scale_log2) {
  constexpr int LPT = D / 8;        // lanes per token
  constexpr int TPW = 64 / LPT;     // tokens per wave step
  constexpr int TOK_IT = kDecWaves * kDecUnroll * TPW;  // tokens per workgroup iteration

  const int split = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int h0 = hg * GW;
  const int kvh = h0 / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane % LPT, slot = lane / LPT;

  int L = seqlens[b];
  L = L < 0 ? 0 : (L > Smax ? Smax : L);
  // balanced chunks rounded up to 16 tokens; later splits may be empty
  int chunk = (L + ns - 1) / ns;
  chunk = (chunk + 15) & ~15;
  const int start = min(L, split * chunk);
  const int end = min(L, start + chunk);

  // query slice (scale * log2 e folded in; stays fp32)
  float qv[GW][8];
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    const u32x4 wq = *reinterpret_cast<const u32x4*>(Qg + ((long long)b * Hq + h0 + hh) * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[hh][2 * e] = bf16_lo(wq[e]) * scale_log2;
      qv[hh][2 * e + 1] = bf16_hi(wq[e]) * scale_log2;
    }
  }

  float m[GW], l[GW], acc[GW][8];
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  }

  const long long tok_stride = (long long)Hkv * D;
  const u16* kb = Kc + (long long)b * Smax * tok_stride + (long long)kvh * D + sub * 8;
  const u16* vb = Vc + (long long)b * Smax * tok_stride + (long long)kvh * D + sub * 8;

  // Loads are never predicated: a token past `end` reads the last valid row
  // (finite data) and gets probability 0, so no NaN beyond the length is read.
  auto load_step = [&](int base, u32x4* kr, u32x4* vr) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int t = min(base + (w * kDecUnroll + u) * TPW + slot, end - 1);
      kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + t * tok_stride));
      vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + t * tok_stride));
    }
  };
  auto consume = [&](int base, const u32x4* kr, const u32x4* vr) __attribute__((always_inline)) {
    float sc[kDecUnroll][GW];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const bool live = base + (w * kDecUnroll + u) * TPW + slot < end;
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = bf16_lo(kr[u][e]);
        kf[2 * e + 1] = bf16_hi(kr[u][e]);
      }
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(qv[hh][e], kf[e], part);
        const float sv = group_sum<LPT>(part);
        sc[u][hh] = live ? sv : -INFINITY;
      }
    }
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      float mx = sc[0][hh];
#pragma unroll
      for (int u = 1; u < kDecUnroll; ++u) mx = fmaxf(mx, sc[u][hh]);
      if (mx > m[hh] + 8.f) {  // new reference maximum (always taken at the first token)
        const float a = __builtin_amdgcn_exp2f(m[hh] - mx);
        l[hh] *= a;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] *= a;
        m[hh] = mx;
      }
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_lo(vr[u][e]);
        vf[2 * e + 1] = bf16_hi(vr[u][e]);
      }
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) {
        const float mu = (m[hh] == -INFINITY) ? 0.f : m[hh];  // no token seen yet
        const float p = __builtin_amdgcn_exp2f(sc[u][hh] - mu);  // 0 for masked (-inf)
        l[hh] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(p, vf[e], acc[hh][e]);
      }
    }
  };

  // two register sets: the loads of step i+1 are in flight while step i is used
  u32x4 ka[kDecUnroll], va[kDecUnroll], kb2[kDecUnroll], vb2[kDecUnroll];
  if (start < end) load_step(start, ka, va);
  for (int base = start; base < end; base += 2 * TOK_IT) {
    if (base + TOK_IT < end) load_step(base + TOK_IT, kb2, vb2);
    consume(base, ka, va);
    if (base + TOK_IT >= end) break;
    if (base + 2 * TOK_IT < end) load_step(base + 2 * TOK_IT, ka, va);
    consume(base + TOK_IT, kb2, vb2);
  }

  // merge the token slots of the wave (lanes sub + LPT*slot, same sub)
#pragma unroll
  for (int x = LPT; x < 64; x <<= 1) {
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      const float m2 = __shfl_xor(m[hh], x), l2 = __shfl_xor(l[hh], x);
      float a2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a2[e] = __shfl_xor(acc[hh][e], x);
      merge_state(m[hh], l[hh], acc[hh], m2, l2, a2);
    }
  }

  // merge the waves through LDS
  __shared__ float sm[kDecWaves][GW], sl[kDecWaves][GW], sacc[kDecWaves][GW][D];
  if (slot == 0) {
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      if (sub == 0) {
        sm[w][hh] = m[hh];
        sl[w][hh] = l[hh];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sacc[w][hh][sub * 8 + e] = acc[hh][e];
    }
  }
  __syncthreads();
  const long long ws_head = (long long)b * Hq + h0;
  for (int idx = tid; idx < GW * D; idx += kDecThreads) {
    const int hh = idx / D, d = idx % D;
    float M = sm[0][hh];
#pragma unroll
    for (int ww = 1; ww < kDecWaves; ++ww) M = fmaxf(M, sm[ww][hh]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float f = __builtin_amdgcn_exp2f(sm[ww][hh] - Mu);
      lt += sl[ww][hh] * f;
      ot += sacc[ww][hh][d] * f;
    }
    const long long slotidx = (ws_head + hh) * ns + split;
    ws_o[slotidx * D + d] = (lt > 0.f) ? ot / lt : 0.f;
    if (d == 0) ws_lse[slotidx] = (lt > 0.f) ? (M + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

// One wave per (batch, query head): merge the splits by log-sum-exp.  Lane i
// holds split i's lse and weight exp(lse_i - L); each lane then accumulates
// its D/64 output elements over the splits.  The partial outputs of the
// first kPre splits are loaded together with the lse values, before the
// weights are known, so the merge waits on one round trip to memory
// instead of three.
constexpr int kPre = 16;

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws_o,
                                                            const float* __restrict__ ws_lse,
                                                            u16* __restrict__ O,
                                                            float* __restrict__ LSE, int ns) {
  constexpr int PER = D / 64;
  const long long bh = blockIdx.x;
  const int lane = threadIdx.x;
  const float* op = ws_o + bh * ns * D + lane * PER;
  float pre[kPre][PER];
#pragma unroll
  for (int i = 0; i < kPre; ++i)
#pragma unroll
    for (int e = 0; e < PER; ++e) pre[i][e] = (i < ns) ? op[(long long)i * D + e] : 0.f;
  const float li = (lane < ns) ? ws_lse[bh * ns + lane] : -INFINITY;
  const bool fin = li > -INFINITY && li < INFINITY;  // empty splits carry -inf
  float M = fin ? li : -INFINITY;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
  float se = fin ? __expf(li - M) : 0.f;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) se += __shfl_xor(se, x);
  const bool any = M > -INFINITY;
  const float Lg = any ? M + __logf(se) : -INFINITY;
  const float wl = fin ? __expf(li - Lg) : 0.f;

  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    // splits past ns have weight 0 (lanes >= ns carry -inf) and loaded 0
    const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = fmaf(wi, pre[i][e], o[e]);
  }
#pragma unroll 8
  for (int i = kPre; i < ns; ++i) {
    const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = fmaf(wi, op[(long long)i * D + e], o[e]);
  }
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(O + bh * D + lane * 2) = pack_bf16(o[0], o[1]);
  } else {
    bf16x2 r;
    r[0] = (__bf16)o[0];
    O[bh * D + lane] = __builtin_bit_cast(u16, r[0]);
  }
  if (LSE != nullptr && lane == 0) LSE[bh] = Lg;
}

template <int D, int GW>
static void go_split(const void* q, const void* kc, const void* vc, const int* seqlens, float* wso,
                     float* wsl, int B, int Hq, int Hkv, int Smax, int ns, float scale,
                     hipStream_t stream) {
  dim3 grid(ns, Hq / GW, B);
  decode_split_kernel<D, GW><<<grid, dim3(kDecThreads), 0, stream>>>(
      static_cast<const u16*>(q), static_cast<const u16*>(kc), static_cast<const u16*>(vc),
      seqlens, wso, wsl, Hq, Hkv, Smax, ns, scale * kLog2e);
}

template <int D>
static void pick_gw(const void* q, const void* kc, const void* vc, const int* seqlens, float* wso,
                    float* wsl, int B, int Hq, int Hkv, int Smax, int ns, float scale,
                    hipStream_t stream) {
  const int G = Hq / Hkv;
  // the largest head count <= 8 that divides the group
  if (G % 8 == 0) return go_split<D, 8>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, Smax, ns, scale, stream);
  if (G % 7 == 0) return go_split<D, 7>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, Smax, ns, scale, stream);
  if (G % 6 == 0) return go_split<D, 6>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, Smax, ns, scale, stream);
  if (G % 5 == 0) return go_split<D, 5>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, Smax, ns, scale, stream);
  if (G % 4 == 0) return go_split<D, 4>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, Smax, ns, scale, stream);
  if (G % 3 == 0) return go_split<D, 3>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, Smax, ns, scale, stream);
  if (G % 2 == 0) return go_split<D, 2>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, Smax, ns, scale, stream);
  return go_split<D, 1>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, Smax, ns, scale, stream);
}

hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int* seqlens, void* o,
                         float* lse, int B, int Hq, int Hkv, int D, int num_splits, float scale,
                         int max_seqlen, void* workspace, hipStream_t stream) {
  float* wso = static_cast<float*>(workspace);
  float* wsl = wso + (size_t)B * Hq * num_splits * D;
  if (D == 64)
    pick_gw<64>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, max_seqlen, num_splits, scale, stream);
  else if (D == 128)
    pick_gw<128>(q, kc, vc, seqlens, wso, wsl, B, Hq, Hkv, max_seqlen, num_splits, scale, stream);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D == 64)
    decode_combine_kernel<64><<<dim3(B * Hq), dim3(64), 0, stream>>>(wso, wsl, static_cast<u16*>(o), lse, num_splits);
  else
    decode_combine_kernel<128><<<dim3(B * Hq), dim3(64), 0, stream>>>(wso, wsl, static_cast<u16*>(o), lse, num_splits);
  return hipGetLastError();
}

}  // namespace xattn
