// fwd_bf16.hip — bf16 exact attention forward on gfx950 matrix cores.
//
// What is computed is the tiled forward with online softmax of scirs2-neural
// 0.4.3 (src/layers/flash_attention.rs): fn flash_attention_forward (query
// blocks outside, key/value blocks inside, causal skip of key blocks after the
// block's last query, final O /= l where l > 0), fn compute_block_scores
// (S = Q K^T * scale), fn apply_causal_mask, fn online_softmax_update (running
// max m, correction exp(m_old - m_new) that is 0 while m_old = -inf, running
// sum l, O rescaled then accumulated).  The per-row LSE m + ln l is stored, as
// the log-sum-exp of oxibonsai-model 0.1.4 (src/layers/flash_decode.rs,
// fn flash_decode_tile).  Query heads map to kv head h / (Hq / Hkv)
// (scirs2-neural 0.4.4 src/layers/grouped_query_attention.rs forward loop;
// whisper-apr 0.3.1 src/model/lfm2/gqa.rs fn attention_scalar).
//
// How it runs on CDNA4:
//  * A workgroup of 4 waves owns 128 query columns: HPW query heads that share
//    one kv head x (128 / HPW) positions, so every K/V tile fetched from HBM is
//    reused by the whole head group.  Wave w owns columns [32w, 32w + 32).
//  * Scores are produced transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand, the wave's
//    query fragment (kept in registers for the whole loop) the B operand.
//    In the 32x32 accumulator a lane holds one query column and 16 key rows,
//    so the row max / row sum are 15 in-lane ops plus one exchange with the
//    lane 32 away, and the probabilities are already laid out as the B
//    operand of the second contraction O^T += V^T P^T (no LDS round trip).
//  * K tiles are stored row-major in LDS, V tiles transposed (d-major) so the
//    A operand of O^T += V^T P^T is two 8-byte LDS reads per lane.  Both are
//    double buffered: the next tile is loaded from HBM into registers with
//    16-byte loads while the current one is consumed, then written to the
//    other buffer; one barrier per tile.
//  * Softmax runs in the base-2 domain: scale * log2(e) is applied by one FMA
//    per score together with the max subtraction, exp2 is v_exp_f32.
//  * RoPE on queries is applied while the query fragment is loaded (fp64
//    rotation from the fp64 table, one rounding to bf16).  Keys are rotated
//    once per call by the RoPE kernel before this one (each K tile is read by
//    every query tile, so rotating it here would repeat the work Sq/128 times).
//  * Workgroups are issued heaviest-first under the causal mask, and the
//    (batch, head group) index is the fastest-varying part of the block index
//    so that the workgroups of one head group land on one XCD (block i runs on
//    XCD i mod 8) and share its L2.
#include "common.h"
#include "kernels.h"

namespace xattn {

// Word 3 of a gfx9 buffer resource for raw (unformatted, stride 0) 32-bit access.
constexpr int kBufferWord3 = 0x00020000;

template <int D, int HPW, bool CAUSAL, bool ROPE>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    u16* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Sq, int Skv,
    float scale_log2, const double2* __restrict__ tab, int n_qt, int n_bh) {
  constexpr int BM = 128, BN = 64, NP = BM / HPW;
  constexpr int KST = D + 8;                 // K row stride in LDS (elements)
  constexpr int VST = BN + 8;                // V^T row stride in LDS (elements)
  constexpr int KCH = D / 8;                 // 16-byte chunks per row
  constexpr int K_LD = BN * KCH / 256;       // K chunks per thread per tile
  constexpr int V_LD = (BN / 2) * KCH / 256; // V (row pair, chunk) items per thread
  constexpr int NDB = D / 32;                // 32-row blocks of O^T
  constexpr int NKS = D / 16;                // k-steps of the QK^T contraction
  static_assert(K_LD >= 1 && V_LD >= 1, "tile loads");

  __shared__ __attribute__((aligned(16))) u16 Ks[2][BN * KST];
  __shared__ __attribute__((aligned(16))) u16 Vt[2][D * VST];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;

  const int bid = blockIdx.x;
  const int qt = CAUSAL ? (n_qt - 1 - bid / n_bh) : (bid / n_bh);
  const int bh = bid % n_bh;
  const int HG = Hq / HPW;
  const int b = bh / HG;
  const int h0 = (bh % HG) * HPW;
  const int kvh = h0 / (Hq / Hkv);
  const int p0 = qt * NP;
  const int off = Skv - Sq;

  const int gc = w * 32 + c;
  const int hh = h0 + gc / NP;
  const int pos = p0 + gc % NP;
  const bool qvalid = pos < Sq;

  // ---- query fragment: lane holds q[pos, hh, 16ks + 8g .. +7] for every ks
  bf16x8 qf[NKS];
  {
    const u16* qp = Q + (((long long)b * Sq + (qvalid ? pos : 0)) * Hq + hh) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 wv = {0u, 0u, 0u, 0u};
      if (qvalid) wv = *reinterpret_cast<const u32x4*>(qp + ks * 16);
      if (ROPE && qvalid) {
        const double2* tp = tab + (long long)(off + pos) * (D / 2) + ks * 8 + g * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          double r0, r1;
          rotate_pair((double)bf16_lo(wv[e]), (double)bf16_hi(wv[e]), tp[e], r0, r1);
          wv[e] = f64_to_bf16_bits(r0) | (f64_to_bf16_bits(r1) << 16);
        }
      }
      qf[ks] = __builtin_bit_cast(bf16x8, wv);
    }
  }

  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, min(p0 + NP, Sq) - 1 + off + 1);
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int first_q = p0 + off;  // smallest query position of the workgroup

  // K and V of this (batch, kv head) through range-checked buffer resources:
  // rows at or past Skv read as zero, offsets are 32-bit.
  const long long head_base = (long long)b * Skv * Hkv * D + (long long)kvh * D;
  const uint32_t nbytes = (uint32_t)(((long long)Skv * Hkv * D - (long long)kvh * D) * 2);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + head_base), (short)0, nbytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + head_base), (short)0, nbytes, kBufferWord3);
  const uint32_t row_bytes = (uint32_t)Hkv * D * 2;

  uint32_t koff[K_LD], voff[V_LD];
#pragma unroll
  for (int i = 0; i < K_LD; ++i) {
    const int cid = tid + 256 * i;
    koff[i] = (uint32_t)(cid / KCH) * row_bytes + (uint32_t)(cid % KCH) * 16u;
  }
#pragma unroll
  for (int i = 0; i < V_LD; ++i) {
    const int cid = tid + 256 * i;
    voff[i] = (uint32_t)(2 * (cid / KCH)) * row_bytes + (uint32_t)(cid % KCH) * 16u;
  }

  u32x4 kreg[K_LD], vreg[2 * V_LD];
  auto gload = [&](int k0) {
    const uint32_t t0 = (uint32_t)k0 * row_bytes;
#pragma unroll
    for (int i = 0; i < K_LD; ++i)
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[i] + t0, 0, 0);
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      vreg[2 * i] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i] + t0, 0, 0);
      vreg[2 * i + 1] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i] + t0 + row_bytes, 0, 0);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int cid = tid + 256 * i, row = cid / KCH, ch = cid % KCH;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * KST + ch * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int cid = tid + 256 * i, pr = cid / KCH, ch = cid % KCH;
      const u32x4 a = vreg[2 * i], bb = vreg[2 * i + 1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // element e of row 2pr (low half) and of row 2pr+1 (high half)
        const uint32_t word = __builtin_amdgcn_perm(bb[e >> 1], a[e >> 1],
                                                    (e & 1) ? 0x07060302u : 0x05040100u);
        *reinterpret_cast<uint32_t*>(&Vt[buf][(ch * 8 + e) * VST + 2 * pr]) = word;
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  // m_run is a reference maximum (log2 domain): the true running maximum never
  // exceeds it by more than 8, so every probability stays <= 2^8; it is moved
  // (and O, l rescaled) only when a score would break that bound.  O / l and
  // m_run + log2(l) do not depend on which reference is used.
  float m_run = -INFINITY, l_run = 0.f;

  if (ntiles > 0) {
    gload(0);
    swrite(0);
  }
  // Everything the prologue loaded (the query fragment included) has landed:
  // without this the loop head inherits a pending query load from the path
  // with no tile and waits for every in-flight prefetch at each iteration.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int k0 = t * BN;
    if (t + 1 < ntiles) gload(k0 + BN);

    // S^T (64 keys x 32 queries) = K_tile Q^T
    f32x16 s[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[0][r] = s[1][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&Ks[buf][(blk * 32 + c) * KST + ks * 16 + g * 8]);
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[blk], 0, 0, 0);
      }
    }

    // mask: key rows past Skv, and keys after the query under the causal rule
    const bool need_mask = (k0 + BN > Skv) || (CAUSAL && k0 + BN - 1 > first_q);
    if (need_mask) {
      const int qlim = CAUSAL ? min(pos + off, Skv - 1) : Skv - 1;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + blk * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (j > qlim) s[blk][r] = -INFINITY;
        }
    }

    // online softmax for this lane's query column
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float mxs = mx * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mxs > m_run + 8.f)) {  // wave-uniform
      const float m_new = fmaxf(m_run, mxs);
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float ls = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[blk][r], scale_log2, -m_use));
        s[blk][r] = p;
        ls += p;
      }
    l_run += ls;  // per half-wave partial; the halves are added after the loop

    // probabilities as bf16 B operands: chunk kc covers keys 16kc .. 16kc+15
    bf16x8 pf[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[kc][e] = (__bf16)s[kc >> 1][(kc & 1) * 8 + e];

    // O^T (D x 32) += V^T (D x 64) P^T (64 x 32)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u16* vrow = &Vt[buf][(db * 32 + c) * VST + 4 * g];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + kc * 16);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + kc * 16 + 8);
        const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[kc],
                                                           oacc[db], 0, 0, 0);
      }
    }

    if (t + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }

  if (qvalid) {
    const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
    u16* op = O + (((long long)b * Sq + pos) * Hq + hh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = db * 32 + 8 * a + 4 * g;
        u32x2 pk;
        pk[0] = pack_bf16(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv);
        pk[1] = pack_bf16(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d) = pk;
      }
    if (LSE != nullptr && g == 0)
      LSE[((long long)b * Hq + hh) * Sq + pos] =
          (l_run > 0.f) ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  }
}

template <int D, int HPW, bool CAUSAL, bool ROPE>
static hipError_t go_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int Hq, int Hkv, int Sq, int Skv, float scale, const double2* tab,
                          hipStream_t stream) {
  constexpr int NP = 128 / HPW;
  const int n_qt = (Sq + NP - 1) / NP;
  const int n_bh = B * (Hq / HPW);
  const long long nblocks = (long long)n_qt * n_bh;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  fwd_bf16_kernel<D, HPW, CAUSAL, ROPE><<<dim3((unsigned)nblocks), dim3(256), 0, stream>>>(
      static_cast<const u16*>(q), static_cast<const u16*>(k), static_cast<const u16*>(v),
      static_cast<u16*>(o), lse, Hq, Hkv, Sq, Skv, scale * kLog2e, tab, n_qt, n_bh);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool ROPE>
static hipError_t pick_hpw(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int Sq, int Skv, float scale,
                           const double2* tab, hipStream_t stream) {
  const int G = Hq / Hkv;
  if (G % 8 == 0)
    return go_bf16<D, 8, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, stream);
  if (G % 4 == 0)
    return go_bf16<D, 4, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, stream);
  if (G % 2 == 0)
    return go_bf16<D, 2, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, stream);
  return go_bf16<D, 1, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, tab, stream);
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                           float scale, const double2* rope_tab, hipStream_t stream) {
  const bool rope = rope_tab != nullptr;
#define XATTN_BF16_CASE(DD, C, R)                                                          \
  if (D == DD && (causal != 0) == C && rope == R)                                        \
    return pick_hpw<DD, C, R>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, scale, rope_tab, stream);
  XATTN_BF16_CASE(64, false, false)
  XATTN_BF16_CASE(64, true, false)
  XATTN_BF16_CASE(64, false, true)
  XATTN_BF16_CASE(64, true, true)
  XATTN_BF16_CASE(128, false, false)
  XATTN_BF16_CASE(128, true, false)
  XATTN_BF16_CASE(128, false, true)
  XATTN_BF16_CASE(128, true, true)
#undef XATTN_BF16_CASE
  return hipErrorInvalidValue;
}

}  // namespace xattn
