// fwd16p_kernel.h — the unmasked 16-bit forward (bf16 or fp16 inputs, fp32
// accumulation) with a software-pipelined key loop.
//
// What is computed is the tiled forward with online softmax of scirs2-neural
// 0.4.3 (src/layers/flash_attention.rs): fn flash_attention_forward (query
// blocks outside, key/value blocks inside, causal skip of key blocks after the
// block's last query, final O /= l where l > 0), fn compute_block_scores,
// fn apply_causal_mask and fn online_softmax_update (running max, rescale of
// O and l when it moves); the per-row LSE m + ln l is stored as the
// log-sum-exp of oxibonsai-model 0.1.4 (src/layers/flash_decode.rs,
// fn flash_decode_tile).  Query head h reads kv head h / (Hq / Hkv)
// (scirs2-neural 0.4.4 src/layers/grouped_query_attention.rs forward loop).
//
// Layout and tiling are those of fwd16_kernel (fwd16_kernel.h): a workgroup of 4
// waves owns 128 * NQB query columns (HPW heads of one kv head x positions;
// under-filled launches add key groups, see KS below),
// S^T = K Q^T and O^T += V^T P^T on the 32x32x16 matrix instructions, K and V
// tiles of 64 keys in XOR-swizzled LDS filled by direct HBM->LDS loads.  What
// differs is the order of work inside a wave.  Keys are consumed in halves of
// 32; step h of a wave issues
//   * the QK^T products of half h+1 (into the second score buffer),
//   * the PV products of half h-1 (its probabilities packed in step h-1),
//   * the softmax of half h (scores produced in step h-1),
// as one block, so the matrix unit runs the products while the vector unit
// runs the exponentials of the same wave: on gfx950 a wave can issue several
// independent vector instructions while one of its matrix instructions
// executes, and the softmax (one FMA, one exp, one add per score, one
// conversion per pair) costs more issue cycles than the products it feeds.
//
// The softmax keeps a reference maximum per query column (log2 units) and
// does not look for a new maximum in every half: the probabilities of a half
// are 2^(s * scale * log2(e) - m_ref) right away, and only when a lane's sum
// over the half exceeds 2^8 (a score may be more than 8 above the
// reference), or a column has no reference yet, does the wave take the slow
// path: the half's true column maximum, m_ref moved to it, O and l rescaled
// by 2^(m_old - m_new) (0 when there was no reference), the half's
// probabilities recomputed from the scores, which are kept until then.
// O / l and m_ref + log2(l) do not depend on which reference is used, so the
// result is that of the page's update with the exact running maximum, up to
// rounding.  A reference that is a maximum of earlier scores keeps l >= 1, so
// later probabilities far below it only lose what is negligible against l.
// The window of 8 bounds the probabilities by 2^8 and keeps the key that
// set the reference at exactly 1: the probabilities enter the PV product
// rounded to 16 bits, and a dominant one rounded loses up to 2^-8 of the
// output (a wider window, 2^64, measured up to 0.7 % on rows dominated by one
// key).
//
// LDS: two buffers each for K and V.  Step h reads K of half h+1 and V of
// half h-1, so the steps of one tile-step pair (halves 2u+1, 2u+2) read the
// K tile u+1 and the V tile u; the loads of K tile u+2 and V tile u+1 are
// issued when that pair starts, into the buffers the previous pair finished,
// and one barrier per pair (64 keys) orders them.
//
// ONEBUF instances are a check of that ordering, not a fast path: one buffer
// each for K and V, filled only between pairs (a barrier after the last read
// of the buffer, the loads, a wait for them, a barrier), so no load is ever
// in flight while a wave reads LDS.  The arithmetic and its order are the
// same, so their results must equal the double-buffered ones bit for bit.

#pragma once

#include "common.h"
#include "kernels.h"
#include "lds.h"

#include <cstdlib>
#include <type_traits>

namespace xattn {

// A lane's sum of probabilities over a half above which the reference moves.
constexpr float kRefWindow = 0x1p8f;

// Query waves per key group: 4, or 2 in the four-group instances (KS = 4).
template <int KS>
constexpr int fwdp_query_waves() { return KS == 4 ? 2 : 4; }

template <typename T, int D, int HPW, bool CAUSAL, bool ROPE, int NQB, int KS, bool ONEBUF>
__global__ __launch_bounds__(64 * fwdp_query_waves<KS>() * KS)
__attribute__((amdgpu_waves_per_eu(2))) void fwdp_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    u16* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Sq, int Skv_all,
    const int* __restrict__ kv_lens, int kv_rows, float scale_log2,
    const double2* __restrict__ tab, int n_qt, int n_bh) {
  constexpr int QW = fwdp_query_waves<KS>();  // waves of a key group
  constexpr int BM = 32 * QW * NQB, BN = 64, NP = BM / HPW;
  constexpr int KCH = D / 8;                // 16-byte chunks per row
  constexpr int LD = BN * KCH / (64 * QW);  // 16-byte chunks per thread per tile (K and V each)
  constexpr int NDB = D / 32;         // 32-row blocks of O^T
  constexpr int NKS = D / 16;         // k-steps of the QK^T contraction
  static_assert(LD >= 1, "tile loads");
  typedef Fmt16<T> F;
  typedef typename F::v8 v8;

  // K and V double buffers of each key group (KS groups of QW waves; see below)
  __shared__ __attribute__((aligned(16))) u16 Ks0g[KS][BN * D];
  __shared__ __attribute__((aligned(16))) u16 Vs0g[KS][BN * D];
  __shared__ __attribute__((aligned(16))) u16 Ks1g[KS][BN * D];
  __shared__ __attribute__((aligned(16))) u16 Vs1g[KS][BN * D];
  // RoPE (cos, sin) rows of the workgroup's NP positions, loaded once and
  // read by every wave (the HPW heads of a position share its row) when the
  // workgroup's LDS stays within 80 KiB (two workgroups per CU); otherwise
  // each lane reads its rows from the table
  constexpr bool TAB_LDS = ROPE && HPW > 1 && 4 * BN * D * 2 + NP * D * 8 <= 81920 &&
                           (NP * D / 2) % 256 == 0;
  __shared__ __attribute__((aligned(16))) double2 Ts[TAB_LDS ? NP * (D / 2) : 1];

  // KS = 2 or 4 (launches with fewer workgroups than CUs): KS groups of QW
  // waves take KS consecutive ranges of the workgroup's key tiles for the
  // same query columns, with their own K/V buffers, and merge (m, l, O)
  // through LDS at the end.  Every group runs the same number of pairs (the
  // last groups' last tiles may lie past the keys: range-checked loads read
  // zeros there and the mask drops them), so they meet at every barrier.
  const int tid = threadIdx.x, lane = tid & 63, w = (tid >> 6) % QW;
  const int grp = KS > 1 ? (tid >> 6) / QW : 0;
  const int c = lane & 31, g = lane >> 5;
  u16* const Ks0 = Ks0g[grp];
  u16* const Vs0 = Vs0g[grp];
  u16* const Ks1 = Ks1g[grp];
  u16* const Vs1 = Vs1g[grp];

  // block -> (query tile, batch-head group).  Consecutive blocks go to the 8
  // XCDs in turn.  Causal: the group varies fastest (each XCD keeps a fixed
  // set of groups), query tiles heaviest first.  Non-causal, when the groups
  // divide among the XCDs: XCD x takes the groups x, x + 8, ... one after
  // the other, all query tiles of a group before the next, so its L2 holds
  // the K and V of fewer groups at a time (the Whisper shape 1-4 % faster in
  // three A/B runs; the causal LFM2 launch was 10 % slower that way).
  const int bid = blockIdx.x;
  int bh, qi;
  if (!CAUSAL && n_bh % 8 == 0) {
    const int j = bid >> 3;
    bh = (bid & 7) + 8 * (j / n_qt);
    qi = j % n_qt;
  } else {
    bh = bid % n_bh;
    qi = bid / n_bh;
  }
  const int qt = CAUSAL ? (n_qt - 1 - qi) : qi;
  const int HG = Hq / HPW;
  const int b = bh / HG;
  const int h0 = (bh % HG) * HPW;
  const int kvh = h0 / (Hq / Hkv);
  const int p0 = qt * NP;
  const int Skv = kv_lens ? min(max(kv_lens[b], 0), kv_rows - Sq) + Sq : Skv_all;
  const int off = Skv - Sq;

  int hh[NQB], pos[NQB];
  bool qvalid[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int gc = (w * NQB + qb) * 32 + c;
    hh[qb] = h0 + gc / NP;
    pos[qb] = p0 + gc % NP;
    qvalid[qb] = pos[qb] < Sq;
  }

  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, min(p0 + NP, Sq) - 1 + off + 1);
  const int nt_all = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;  // 64-key tiles
  const int nt = (nt_all + KS - 1) / KS;  // tiles of this wave's key group
  const int t0 = grp * nt;                // its first tile
  const int first_q = p0 + off;

  const long long head_base = (long long)b * kv_rows * Hkv * D + (long long)kvh * D;
  const uint32_t nbytes = (uint32_t)(((long long)Skv * Hkv * D - (long long)kvh * D) * 2);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + head_base), (short)0, nbytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + head_base), (short)0, nbytes, kBufferWord3);
  const uint32_t row_bytes = (uint32_t)Hkv * D * 2;

  uint32_t koff[LD], voff[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int sl = (w * LD + i) * 64 + lane, row = sl / KCH, phys = sl % KCH;
    koff[i] = (uint32_t)row * row_bytes + (uint32_t)(phys ^ kswz<D>(row)) * 16u;
    voff[i] = (uint32_t)row * row_bytes + (uint32_t)(phys ^ vswz<D>(row)) * 16u;
  }
  // direct loads of key tile u into kb / value tile u into vb (this wave's share)
  // (u counts the group's tiles)
  auto load_k = [&](int u, u16* kb) {
    dma_rows<LD>(rk, kb + w * LD * 64 * 8, koff, (uint32_t)((t0 + u) * BN) * row_bytes);
  };
  auto load_v = [&](int u, u16* vb) {
    dma_rows<LD>(rv, vb + w * LD * 64 * 8, voff, (uint32_t)((t0 + u) * BN) * row_bytes);
  };
  // K fragment of half hb, k-step ks: row 32 hb + c, logical chunk 2 ks + g.
  // The swizzle of row 32 hb + c does not depend on hb, so a half's
  // fragments are those of half 0 plus 32 rows (an immediate offset).
  int ka_off[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) ka_off[ks] = c * D + ((2 * ks + g) ^ kswz<D>(c)) * 8;
  // V^T fragments by transpose reads: chunk kc of 16 keys, block db of 32
  // rows of V^T.  Lane (tq, tl) reads row 16 kc + 8 r + 4 (tq >> 1) + tl / 4,
  // whose swizzle does not depend on kc or r: those are immediate offsets.
  const int tq = lane >> 4, tl = lane & 15;
  int va_base[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int row = 4 * (tq >> 1) + (tl >> 2);
    const int col = 32 * db + 16 * (tq & 1) + 4 * (tl & 3);
    va_base[db] = row * D + (((col >> 3) ^ vswz<D>(row)) << 3) + (col & 7);
  }

  f32x16 oacc[NQB][NDB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  float m_run[NQB], l_run[NQB], nm[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
    nm[qb] = 0.f;
  }
  // scale * log2(e) in a vector register: an FMA that reads an SGPR issues at
  // about half the rate of one whose operands are all VGPRs when two waves
  // share a SIMD (measured on gfx950)
  float slv;
  asm("v_mov_b32 %0, %1" : "=v"(slv) : "s"(scale_log2));

  // ---- query fragments (as fwd16_kernel): lane holds q[pos, hh, 16ks + 8g .. +7]
  v8 qf[NQB][NKS];
  {
    if constexpr (TAB_LDS) {
      // rows p0 .. p0+NP-1 of the query positions (table rows off + p), the
      // pairs of row r stored at slot j ^ (r & 15): a wave's read of one
      // pair for 16 consecutive rows then touches 16 distinct bank groups.
      // Rows past the table's end (positions >= Sq) read as zero.
      constexpr int TCH = NP * (D / 2) / 256;  // 16-byte slots per thread
      const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(tab + (long long)(off + p0) * (D / 2)), (short)0,
          (uint32_t)(Sq - p0) * (uint32_t)(D / 2) * 16u, kBufferWord3);
      uint32_t toff[TCH];
#pragma unroll
      for (int i = 0; i < TCH; ++i) {
        const int sl = (w * TCH + i) * 64 + lane, r = sl / (D / 2), pj = sl % (D / 2);
        toff[i] = (uint32_t)(r * (D / 2) + (pj ^ (r & 15))) * 16u;
      }
      dma_rows<TCH>(rt, reinterpret_cast<u16*>(Ts) + w * TCH * 64 * 8, toff, 0u);
    }
    u32x4 qw[NQB][NKS];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const u16* qp =
          Q + (((long long)b * Sq + (qvalid[qb] ? pos[qb] : 0)) * Hq + hh[qb]) * D + g * 8;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qw[qb][ks] = *reinterpret_cast<const u32x4*>(qp + ks * 16);
    }
    double2 cs[NQB][NKS][4];
    if constexpr (ROPE && !TAB_LDS) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const double2* tp =
            tab + (long long)(off + (qvalid[qb] ? pos[qb] : 0)) * (D / 2) + g * 4;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int e = 0; e < 4; ++e) cs[qb][ks][e] = tp[ks * 8 + e];
      }
    }
    if constexpr (TAB_LDS) {
      // the first K and V tiles go out behind the table and Q (a second K
      // tile past the keys reads zeros into a buffer no step then reads);
      // loads complete in issue order, so waiting until only those 3 LD are
      // outstanding covers this wave's table slots, and the barrier every
      // wave's
      static_assert(3 * LD <= 15, "vmcnt immediate");
      load_k(0, Ks0);
      load_v(0, Vs0);
      if (!ONEBUF) load_k(1, Ks1);
      // (a bare barrier: __syncthreads would add a release fence that waits
      // for every outstanding load, the K and V tiles included)
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | ((ONEBUF ? 2 : 3) * LD));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else if (nt > 0) {
      load_k(0, Ks0);
      load_v(0, Vs0);
      if (nt > 1 && !ONEBUF) load_k(1, Ks1);
    }
    if constexpr (TAB_LDS) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int r = pos[qb] - p0;  // < NP
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            cs[qb][ks][e] = Ts[r * (D / 2) + ((ks * 8 + g * 4 + e) ^ (r & 15))];
      }
    }
    if constexpr (ROPE) {
      // bf16: the rotated values go to bf16 through fp32 (bf16_mid_key); the
      // rare group of 8 values with one on a bf16 midpoint is redone with the
      // single rounding by the whole wave, so the result is that rounding's
      constexpr bool VIA32 = std::is_same<T, __bf16>::value;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const u32x4 raw = qw[qb][ks];
          double r0[4], r1[4];
          uint32_t mid = 1;  // 0 once a value lands on a bf16 midpoint
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            rotate_pair((double)F::lo(raw[e]), (double)F::hi(raw[e]), cs[qb][ks][e], r0[e], r1[e]);
            if constexpr (VIA32) {
              float f0 = (float)r0[e], f1 = (float)r1[e];
              // (opaque: the compiler would fuse the two conversions into its own
              // single-rounding sequence, which costs more)
              asm("" : "+v"(f0), "+v"(f1));
              mid = min(mid, min(bf16_mid_key(f0), bf16_mid_key(f1)));
              qw[qb][ks][e] = F::pack(f0, f1);
            } else {
              qw[qb][ks][e] = F::from_f64(r0[e]) | (F::from_f64(r1[e]) << 16);
            }
          }
          if (VIA32 && __builtin_amdgcn_ballot_w64(mid == 0)) {  // wave-uniform, rare
#pragma unroll
            for (int e = 0; e < 4; ++e)
              qw[qb][ks][e] = F::from_f64(r0[e]) | (F::from_f64(r1[e]) << 16);
          }
        }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 wv = qw[qb][ks];
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] = qvalid[qb] ? wv[e] : 0u;
        asm volatile("" : "+v"(wv));
        qf[qb][ks] = __builtin_bit_cast(v8, wv);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- pieces of a step
  // S^T of half hb of the tile in kb (32 keys x 32 queries per query block)
  auto qk = [&](const u16* kb, int hb, f32x16(&s)[NQB]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[qb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const v8 ka = *reinterpret_cast<const v8*>(&kb[hb * 32 * D + ka_off[ks]]);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s[qb] = F::mfma(ka, qf[qb][ks], s[qb]);
    }
  };
  // O^T += V^T P^T for half hb of the tile in vb (its two chunks of 16 keys)
  auto pv = [&](const u16* vb, int hb, const u32x4(&p)[NQB][2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int kc = 2 * hb + j;
        const s16x4 lo = lds_read_tr16(&vb[va_base[db] + 16 * kc * D]);
        const s16x4 hi = lds_read_tr16(&vb[va_base[db] + (16 * kc + 8) * D]);
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 vv = {lo2[0], lo2[1], hi2[0], hi2[1]};
        const v8 va = __builtin_bit_cast(v8, vv);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          oacc[qb][db] = F::mfma(va, __builtin_bit_cast(v8, p[qb][j]), oacc[qb][db]);
      }
  };
  // keys past Skv and (causal) after the query: scores to -inf.  Key of
  // accumulator row r of the half starting at k0: k0 + 8 (r >> 2) + 4 g + (r & 3).
  auto mask_half = [&](f32x16(&s)[NQB], int k0) {
    if ((k0 + 32 > Skv) || (CAUSAL && k0 + 31 > first_q)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qlim = CAUSAL ? min(pos[qb] + off, Skv - 1) : Skv - 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (j > qlim) s[qb][r] = -INFINITY;
        }
      }
    }
  };
  // probabilities of a half against the current reference, packed to the
  // 16-bit B operand (chunk j holds accumulator rows 8j .. 8j+7), and this
  // lane's sum over them; the scores are left as they are
  auto sm_fast = [&](const f32x16(&s)[NQB], u32x4(&p)[NQB][2], float(&ls)[NQB]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      ls[qb] = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = __builtin_amdgcn_exp2f(fmaf(s[qb][8 * j + 2 * e], slv, nm[qb]));
          const float bb = __builtin_amdgcn_exp2f(fmaf(s[qb][8 * j + 2 * e + 1], slv, nm[qb]));
          ls[qb] += a;
          ls[qb] += bb;
          p[qb][j][e] = F::pack(a, bb);
        }
    }
  };
  // the slow path: true column maximum of the half, reference moved to it
  // (O and l rescaled), probabilities recomputed.  The fast path's results
  // (in p and ls on entry) are merged into the new ones with an opaque zero
  // mask: without a use on this path the compiler would move the fast path
  // below the branch and split the block whose interleave sched_step orders.
  int zmask;
  asm("v_mov_b32 %0, 0" : "=v"(zmask));
  auto sm_slow = [&](const f32x16(&s)[NQB], u32x4(&p)[NQB][2], float(&ls)[NQB]) {
    u32x4 pf[NQB][2];
    float lf[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      lf[qb] = ls[qb];
      pf[qb][0] = p[qb][0];
      pf[qb][1] = p[qb][1];
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = fmaxf(s[qb][0], s[qb][1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[qb][r]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float m_new = fmaxf(m_run[qb], mx * scale_log2);
      const float alpha =
          __builtin_amdgcn_exp2f(m_run[qb] - (m_new == -INFINITY ? 0.f : m_new));
      l_run[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
      m_run[qb] = m_new;
      nm[qb] = (m_new == -INFINITY) ? 0.f : -m_new;
    }
    sm_fast(s, p, ls);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      ls[qb] = __int_as_float(__float_as_int(ls[qb]) | (__float_as_int(lf[qb]) & zmask));
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[qb][j][e] |= pf[qb][j][e] & (uint32_t)zmask;
    }
  };
  bool have_ref = false;  // wave-uniform: every column of the wave has a reference
  // step: softmax of the half in s_sm (first key k0) into p_out; optionally
  // the QK^T of another half into s_qk and the PV of the packed half p_in.
  // The block is written as slots in issue order: slot i issues one matrix
  // product (the QK^T products first, whose results the next step needs,
  // then the PV products) and its share of the softmax's vector
  // instructions; a scheduling barrier after each slot keeps that order
  // (the scheduler would otherwise issue the products back to back).
  auto step = [&](auto do_mask, f32x16(&s_sm)[NQB], int k0, u32x4(&p_out)[NQB][2], auto do_qk,
                  f32x16(&s_qk)[NQB], const u16* kb, int khb, auto do_pv,
                  const u32x4(&p_in)[NQB][2], const u16* vb, int vhb)
                  __attribute__((always_inline)) {
    constexpr bool DQ = decltype(do_qk)::value, DP = decltype(do_pv)::value;
    constexpr int NQK = DQ ? NKS * NQB : 0, NPV = DP ? 2 * NDB * NQB : 0, NM = NQK + NPV;
    constexpr int NE = NQB * 16;  // scores per lane in the half
    if constexpr (decltype(do_mask)::value) mask_half(s_sm, k0);
    float ls[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) ls[qb] = 0.f;
    // fragments are read from LDS a few slots ahead of their first product
    // (K fragment ks is first used in slot ks * NQB, V fragment (j, db) in
    // slot NQK + (j * NDB + db) * NQB), so that few of them are live at once
    constexpr int LEAD_K = 2, LEAD_V = 3;
    v8 kf[NKS];
    v8 vf[2][NDB];
    auto read_k = [&](int ks) __attribute__((always_inline)) {
      kf[ks] = *reinterpret_cast<const v8*>(&kb[khb * 32 * D + ka_off[ks]]);
    };
    auto read_v = [&](int j, int db) __attribute__((always_inline)) {
      const int kc = 2 * vhb + j;
      const s16x4 lo = lds_read_tr16(&vb[va_base[db] + 16 * kc * D]);
      const s16x4 hi = lds_read_tr16(&vb[va_base[db] + (16 * kc + 8) * D]);
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 vv = {lo2[0], lo2[1], hi2[0], hi2[1]};
      vf[j][db] = __builtin_bit_cast(v8, vv);
    };
    // score e of the lane (query block e / 16, accumulator row e % 16) in
    // three stages a slot apart: the FMA (scale and reference), the exp, then
    // the row sum and, at odd e, the packing of the pair; a slot issues the
    // FMAs of the next slot's scores, the exps of its own and the sums of the
    // previous slot's, so no vector instruction waits on the one before it
    float xs[NE], ps[NE];
    auto st_fma = [&](int e) __attribute__((always_inline)) {
      xs[e] = fmaf(s_sm[e / 16][e % 16], slv, nm[e / 16]);
    };
    auto st_exp = [&](int e) __attribute__((always_inline)) { ps[e] = __builtin_amdgcn_exp2f(xs[e]); };
    auto st_acc = [&](int e) __attribute__((always_inline)) {
      const int qb = e / 16, r = e % 16;
      ls[qb] += ps[e];
      if (r & 1) p_out[qb][r / 8][(r % 8) / 2] = F::pack(ps[e - 1], ps[e]);
    };
    constexpr int NMM = NM > 0 ? NM : 1;
    constexpr int PERS = NE / NMM;  // scores per slot
#pragma unroll
    for (int e = 0; e < PERS; ++e) st_fma(e);
#pragma unroll
    for (int m = 0; m < NMM + 1; ++m) {
      if (NM > 0 && m < NM) {
        if constexpr (DQ) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            if (m == (ks * NQB > LEAD_K ? ks * NQB - LEAD_K : 0)) read_k(ks);
        }
        if constexpr (DP) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const int first = NQK + (j * NDB + db) * NQB;
              if (m == (first > LEAD_V ? first - LEAD_V : 0)) read_v(j, db);
            }
        }
        if (m < NQK) {
          const int ks = m / NQB, qb = m % NQB;
          if (ks == 0)
            s_qk[qb] = F::mfma(kf[0], qf[qb][0], f32x16{});
          else
            s_qk[qb] = F::mfma(kf[ks], qf[qb][ks], s_qk[qb]);
        } else {
          const int pm = m - NQK, j = pm / (NDB * NQB), db = (pm / NQB) % NDB, qb = pm % NQB;
          oacc[qb][db] = F::mfma(vf[j][db], __builtin_bit_cast(v8, p_in[qb][j]), oacc[qb][db]);
        }
      }
      if (m + 1 < NMM) {
#pragma unroll
        for (int e = (m + 1) * PERS; e < (m + 2) * PERS; ++e) st_fma(e);
      }
      if (m < NMM) {
#pragma unroll
        for (int e = m * PERS; e < (m + 1) * PERS; ++e) st_exp(e);
      }
      if (m >= 1) {
#pragma unroll
        for (int e = (m - 1) * PERS; e < m * PERS; ++e) st_acc(e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) over = over || (ls[qb] > kRefWindow);
    if (!have_ref || __builtin_amdgcn_ballot_w64(over)) {  // wave-uniform
      sm_slow(s_sm, p_out, ls);
      bool none = false;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) none = none || (m_run[qb] == -INFINITY);
      have_ref = __builtin_amdgcn_ballot_w64(none) == 0;
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) l_run[qb] += ls[qb];
  };

  if (nt > 0) {
    const std::true_type Y;
    const std::false_type N;
    f32x16 sA[NQB], sB[NQB];
    u32x4 pA[NQB][2], pB[NQB][2];
    const int kbase = t0 * BN;  // first key of the group's range
    // prologue: S of half 0, then its softmax with the products of half 1
    qk(Ks0, 0, sA);
    step(Y, sA, kbase, pA, Y, sB, Ks0, 1, N, pB, Vs0, 0);
    __syncthreads();  // every wave has read K tile 0 (its buffer takes tile 2)
    // the second buffers (the first ones again in ONEBUF instances)
    u16* const Kb1 = ONEBUF ? Ks0 : Ks1;
    u16* const Vb1 = ONEBUF ? Vs0 : Vs1;
    if (ONEBUF && nt > 1) {
      load_k(1, Kb1);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    }
    // tile-step pairs: halves 2u+1 and 2u+2 read K tile u+1 and V tile u
    auto pair = [&](auto do_mask, int u, u16* kcur, u16* knext, u16* vcur, u16* vnext)
                    __attribute__((always_inline)) {
      // (issuing these one instruction per slot instead, to keep the
      // address unit busy evenly, measured no faster)
      if (!ONEBUF) {
        if (u + 2 < nt) load_k(u + 2, knext);  // into the buffer K tile u used
        load_v(u + 1, vnext);                  // into the buffer V tile u-1 used
      }
      const int k1 = kbase + u * BN + 32;
      step(do_mask, sB, k1, pB, Y, sA, kcur, 0, Y, pA, vcur, 0);
      step(do_mask, sA, k1 + 32, pA, Y, sB, kcur, 1, Y, pB, vcur, 1);
      if (ONEBUF) {
        __syncthreads();  // every wave is done with K tile u+1 and V tile u
        if (u + 2 < nt) load_k(u + 2, knext);
        load_v(u + 1, vnext);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    };
    // Halves 0 .. h_open-1 (first key 32 h) need no mask: every key of
    // them is below Skv and (causal) at or before the workgroup's first
    // query.  Masking is monotone in the key, so the pairs run first
    // without the mask test while both of a double pair's halves are below
    // h_open, then with it.
    const int kmax = CAUSAL ? min(first_q, Skv - 1) : Skv - 1;  // last key every column sees
    const int h_open = kmax >= 31 ? (kmax + 1) / 32 : 0;
    // pair u reads K tile u+1 from buffer (u+1) & 1 and V tile u from u & 1
    int u = 0;
    for (; u + 2 < nt && 2 * (t0 + u) + 5 <= h_open; u += 2) {
      pair(N, u, Kb1, Ks0, Vs0, Vb1);
      pair(N, u + 1, Ks0, Kb1, Vb1, Vs0);
    }
    for (; u + 1 < nt; u += 2) {
      pair(Y, u, Kb1, Ks0, Vs0, Vb1);
      if (u + 2 < nt) pair(Y, u + 1, Ks0, Kb1, Vb1, Vs0);
    }
    // epilogue: softmax of the last half with the PV of the one before, then
    // the PV of the last half (V tile nt-1 in buffer (nt-1) & 1)
    const u16* vlast = ((nt - 1) & 1) ? Vb1 : Vs0;
    // (the last half's softmax and PV products are left out when it lies
    // wholly past the keys every query of the workgroup sees: Skv mod 64 in
    // 1..32; their probabilities would all be 0)
    if (KS == 1 && nt >= 2 && (t0 + nt - 1) * BN + 32 >= kv_end) {
      pv(vlast, 0, pA);
    } else {
      step(Y, sB, kbase + (nt - 1) * BN + 32, pB, N, sA, Ks0, 0, Y, pA, vlast, 0);
      pv(vlast, 1, pB);
    }
  }

  if constexpr (KS == 2) {
    // the second key group's (m, l, O) into the first's: lane (w, lane) of
    // both groups holds the same query column.  The exchange reuses the K/V
    // buffers once every wave's last reads of them are done: O block db of
    // the group's 4 waves (16 KiB) at float (16 (db mod NDB/2) + r) * 256 +
    // 64 w + lane of Ks0g (db < NDB/2) or Vs0g, m and l in Ks1g.
    static_assert(KS == 2 && NQB == 1 && !ROPE && NDB % 2 == 0, "key groups");
    static_assert(16 * 256 * 4 * (NDB / 2) <= (int)sizeof(Ks0g), "exchange space");
    float* const xo0 = reinterpret_cast<float*>(&Ks0g[0][0]);
    float* const xo1 = reinterpret_cast<float*>(&Vs0g[0][0]);
    float* const xml = reinterpret_cast<float*>(&Ks1g[0][0]);
    const int xl = w * 64 + lane;
    __syncthreads();
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          (db < NDB / 2 ? xo0 : xo1)[(16 * (db % (NDB / 2)) + r) * 256 + xl] = oacc[0][db][r];
      xml[xl] = m_run[0];
      xml[256 + xl] = l_run[0];
    }
    __syncthreads();
    if (grp == 0) {
      const float m1 = xml[xl], l1 = xml[256 + xl];
      const float mn = fmaxf(m_run[0], m1);
      const float a0 = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[0] - mn);
      const float a1 = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - mn);
      l_run[0] = l_run[0] * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[0][db][r] = oacc[0][db][r] * a0 +
                           (db < NDB / 2 ? xo0 : xo1)[(16 * (db % (NDB / 2)) + r) * 256 + xl] * a1;
      m_run[0] = mn;
    }
  }
  if constexpr (KS == 4) {
    // groups 1..3 store (m, l, O) in the K/V buffers once every wave's last
    // reads of them are done (group i in Ks0g, Vs0g, Ks1g: O block db of
    // the group's QW waves at float (16 db + r) * 64 QW + 64 w + lane, then m
    // and l), and group 0 merges the four with one common maximum.
    static_assert(NQB == 1 && !ROPE, "key groups");
    constexpr int XW = 64 * QW;  // lanes of a group
    static_assert((NDB * 16 + 2) * XW * 4 <= (int)sizeof(Ks0g), "exchange space");
    auto xg = [&](int i) -> float* {  // exchange area of group i + 1
      return reinterpret_cast<float*>(i == 0 ? &Ks0g[0][0] : (i == 1 ? &Vs0g[0][0] : &Ks1g[0][0]));
    };
    const int xl = w * 64 + lane;
    __syncthreads();
    if (grp > 0) {
      float* const x = xg(grp - 1);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[(16 * db + r) * XW + xl] = oacc[0][db][r];
      x[NDB * 16 * XW + xl] = m_run[0];
      x[(NDB * 16 + 1) * XW + xl] = l_run[0];
    }
    __syncthreads();
    if (grp == 0) {
      float mi[4], li[4];
      mi[0] = m_run[0];
      li[0] = l_run[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        mi[i] = xg(i - 1)[NDB * 16 * XW + xl];
        li[i] = xg(i - 1)[(NDB * 16 + 1) * XW + xl];
      }
      const float mn = fmaxf(fmaxf(mi[0], mi[1]), fmaxf(mi[2], mi[3]));
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mi[i] - mn);
      l_run[0] = li[0] * a[0] + li[1] * a[1] + li[2] * a[2] + li[3] * a[3];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = oacc[0][db][r] * a[0];
#pragma unroll
          for (int i = 1; i < 4; ++i) acc += xg(i - 1)[(16 * db + r) * XW + xl] * a[i];
          oacc[0][db][r] = acc;
        }
      m_run[0] = mn;
    }
  }
  if (KS > 1 && grp != 0) return;

#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[qb]),
                                                     __float_as_uint(l_run[qb]), false, false);
    const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (qvalid[qb]) {
      const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
      u16* op = O + (((long long)b * Sq + pos[qb]) * Hq + hh[qb]) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = db * 32 + 8 * a + 4 * g;
          u32x2 pk;
          pk[0] = F::pack(oacc[qb][db][4 * a] * inv, oacc[qb][db][4 * a + 1] * inv);
          pk[1] = F::pack(oacc[qb][db][4 * a + 2] * inv, oacc[qb][db][4 * a + 3] * inv);
          *reinterpret_cast<u32x2*>(op + d) = pk;
        }
      if (LSE != nullptr && g == 0)
        LSE[((long long)b * Hq + hh[qb]) * Sq + pos[qb]] =
            (l_tot > 0.f) ? (m_run[qb] + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <bool ONEBUF, typename T, int D, int HPW, bool CAUSAL, bool ROPE, int NQB, int KS>
static hipError_t gop(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int Hq, int Hkv, int Sq, int Skv, const int* kv_lens, int kv_rows,
                      float scale, const double2* tab, hipStream_t stream) {
  constexpr int NP = 32 * fwdp_query_waves<KS>() * NQB / HPW;
  const int n_qt = (Sq + NP - 1) / NP;
  const int n_bh = B * (Hq / HPW);
  const long long nblocks = (long long)n_qt * n_bh;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_kernel(fwdp_kernel<T, D, HPW, CAUSAL, ROPE, NQB, KS, ONEBUF>, dim3((unsigned)nblocks),
                dim3(64 * fwdp_query_waves<KS>() * KS),
                stream, static_cast<const u16*>(q), static_cast<const u16*>(k),
                static_cast<const u16*>(v), static_cast<u16*>(o), lse, Hq, Hkv, Sq, Skv, kv_lens,
                kv_rows, scale * kLog2e, tab, n_qt, n_bh);
  return hipGetLastError();
}

template <bool ONEBUF, typename T, int D, int HPW, bool CAUSAL, bool ROPE>
static hipError_t gop_nqb(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Skv, const int* kv_lens,
                          int kv_rows, float scale, const double2* tab, hipStream_t stream) {
  // two query blocks per wave at D = 64 when the grid still has two
  // workgroups per CU (each K and V fragment read from LDS feeds two
  // products), else one
  if constexpr (D == 64) {
    const long long wg2 = (long long)((Sq + 256 / HPW - 1) / (256 / HPW)) * B * (Hq / HPW);
    if (wg2 >= 2 * 256)
      return gop<ONEBUF, T, D, HPW, CAUSAL, ROPE, 2, 1>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens,
                                             kv_rows, scale, tab, stream);
  }
  // fewer one-block workgroups than CUs and 16 or more key tiles: two key
  // groups per workgroup (without RoPE).  With fewer tiles the merge and the
  // second group's prologue cost more than the halved loop saves (1024 query
  // rows, 8 heads: 512 keys 12.5 -> 13.1 us, 1024 keys 17.3 -> 14.5 us)
  if constexpr (!ROPE) {
    // one head per workgroup at D = 64 with at most one 64-query workgroup
    // per CU: four key groups of two waves (64 query rows), so the launch
    // covers up to every CU rather than half of them
    if constexpr (D == 64 && HPW == 1) {
      const long long wg64 = (long long)((Sq + 63) / 64) * B * Hq;
      if (wg64 <= 256 && Skv >= 16 * 64)
        return gop<ONEBUF, T, D, HPW, CAUSAL, ROPE, 1, 4>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv,
                                                          kv_lens, kv_rows, scale, tab, stream);
    }
    const long long wg1 = (long long)((Sq + 128 / HPW - 1) / (128 / HPW)) * B * (Hq / HPW);
    if (wg1 < 256 && Skv >= 16 * 64)
      return gop<ONEBUF, T, D, HPW, CAUSAL, ROPE, 1, 2>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens,
                                                kv_rows, scale, tab, stream);
  }
  return gop<ONEBUF, T, D, HPW, CAUSAL, ROPE, 1, 1>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows,
                                         scale, tab, stream);
}

template <bool ONEBUF, typename T, int D, bool CAUSAL, bool ROPE>
static hipError_t gop_hpw(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Skv, const int* kv_lens,
                          int kv_rows, float scale, const double2* tab, hipStream_t stream) {
  const int G = Hq / Hkv;
  if (G % 8 == 0)
    return gop_nqb<ONEBUF, T, D, 8, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows,
                                          scale, tab, stream);
  if (G % 4 == 0)
    return gop_nqb<ONEBUF, T, D, 4, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows,
                                          scale, tab, stream);
  if (G % 2 == 0)
    return gop_nqb<ONEBUF, T, D, 2, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows,
                                          scale, tab, stream);
  return gop_nqb<ONEBUF, T, D, 1, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows,
                                        scale, tab, stream);
}

template <bool ONEBUF, typename T>
static hipError_t gop_fmt(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                          float scale, const double2* tab, hipStream_t stream,
                          const int* kv_lens, int kv_rows) {
  const bool rope = tab != nullptr;
#define XATTN_FWDP_CASE(DD, C, R)                                                            \
  if (D == DD && (causal != 0) == C && rope == R)                                            \
    return gop_hpw<ONEBUF, T, DD, C, R>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows, scale, \
                                tab, stream);
  XATTN_FWDP_CASE(64, false, false)
  XATTN_FWDP_CASE(64, true, false)
  XATTN_FWDP_CASE(64, false, true)
  XATTN_FWDP_CASE(64, true, true)
  XATTN_FWDP_CASE(128, false, false)
  XATTN_FWDP_CASE(128, true, false)
  XATTN_FWDP_CASE(128, false, true)
  XATTN_FWDP_CASE(128, true, true)
#undef XATTN_FWDP_CASE
  return hipErrorInvalidValue;
}

// launch_fwd16_pipelined (ONEBUF = false) or its single-buffer check
// (ONEBUF = true): arguments as there
template <bool ONEBUF>
static hipError_t launch_fwdp(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                              float scale, const double2* rope_tab, int dtype, hipStream_t stream,
                              const int* kv_lens, int kv_rows) {
  if (kv_lens == nullptr) kv_rows = Skv;
  if (dtype == 1)
    return gop_fmt<ONEBUF, __bf16>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                                   rope_tab, stream, kv_lens, kv_rows);
  if (dtype == 2)
    return gop_fmt<ONEBUF, _Float16>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                                     rope_tab, stream, kv_lens, kv_rows);
  return hipErrorInvalidValue;
}

}  // namespace xattn
