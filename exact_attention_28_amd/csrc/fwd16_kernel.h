// fwd16_kernel.h — exact attention forward on gfx950 matrix cores for 16-bit
// inputs (bf16, or IEEE binary16 / fp16: the same kernel with the fp16 MFMA
// and conversions; fp32 accumulation either way).
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
//    v_mfma_f32_32x32x16_bf16 (_f16): K (from LDS) is the A operand, the wave's
//    query fragment (kept in registers for the whole loop) the B operand.
//    In the 32x32 accumulator a lane holds one query column and 16 key rows,
//    so the row max / row sum are 15 in-lane ops plus one exchange with the
//    lane 32 away, and the probabilities are already laid out as the B
//    operand of the second contraction O^T += V^T P^T (no LDS round trip).
//  * K and V tiles are stored row-major in LDS (16-byte chunks XOR-swizzled
//    per row) by direct HBM->LDS buffer loads, double buffered: the next
//    tile's loads are in flight while the current one is consumed, with one
//    barrier per tile.  The A operand of O^T += V^T P^T comes from the V tile
//    by LDS transpose reads (ds_read_b64_tr_b16), two per lane per 16 keys.
//  * Softmax runs in the base-2 domain: scale * log2(e) is applied by one FMA
//    per score together with the max subtraction, exp2 is v_exp_f32.
//  * RoPE on queries is applied while the query fragment is loaded (fp64
//    rotation from the fp64 table, one rounding to the input format).  Keys
//    are rotated once per call by the RoPE kernel before this one (each K tile
//    is read by every query tile, so rotating it here would repeat the work
//    Sq/128 times).
//  * An additive mask enters the scores as fma(s, scale, mask), and the
//    softmax then scales by log2(e) in its exp2 argument.  A lane needs, per
//    tile, its query row's mask at its 32 keys, which come in runs of 4
//    (accumulator rows 4a..4a+3).  MASK = 3 (D = 64, 16-byte aligned mask
//    shared by all heads, two or more heads per workgroup): the workgroup's
//    NP query rows x 64 keys go to LDS by direct loads that cover 4 rows of
//    256 bytes per instruction (chunks XOR-swizzled per row), double
//    buffered and issued with the K/V tile one tile ahead; every wave reads
//    its runs of 4 without bank conflicts.  MASK = 2 (the same, per-head
//    masks or one head per workgroup): each wave stages its own 32 rows in a
//    single buffer, refilled in the middle of a tile once its reads are done.
//    MASK = 1 (any other mask, D = 128): each lane loads its runs of 4
//    itself, 8 loads per tile that each touch 32 rows.
//  * Workgroups are issued heaviest-first under the causal mask, and the
//    (batch, head group) index is the fastest-varying part of the block index
//    so that the workgroups of one head group land on one XCD (block i runs on
//    XCD i mod 8) and share its L2.
//  * Key splits (SPLIT instantiations, unmasked): when a launch would leave
//    most CUs idle and each query tile has many key tiles, the keys of a query
//    tile are split into runs handled by separate workgroups, each writing its
//    partial O (normalised) and LSE; fwd16_combine_kernel merges them by
//    log-sum-exp, as split-KV decoding merges its chunks (oxibonsai-model 0.1.4
//    src/layers/flash_decode.rs, fn combine_tile_outputs).
//  * ONEBUF instances check the double buffering: one K/V buffer (and one
//    shared-mask buffer), refilled after a barrier that follows the tile's
//    last read of it, so no load is in flight while LDS is read; same
//    arithmetic in the same order, so the results must equal bit for bit.

#pragma once

#include "common.h"
#include "kernels.h"
#include "lds.h"

#include <algorithm>
#include <cstdlib>
#include <type_traits>

namespace xattn {

// The shared-mask variant with 4 or 8 heads per workgroup needs 40-48 KiB of
// LDS, so three workgroups fit a CU if the registers allow three waves per
// SIMD (<= 168 VGPRs, reached without spills; measured 6 % faster).
template <typename T, int D, int HPW, bool CAUSAL, bool ROPE, int NQB, int MASK, bool SPLIT,
          bool ONEBUF>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(MASK == 3 && HPW >= 4 ? 3 : 1))) void fwd16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    u16* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Sq, int Skv_all,
    const int* __restrict__ kv_lens, int kv_rows, float scale_log2,
    const double2* __restrict__ tab, int n_qt, int n_bh, MaskView mask, float scale,
    KeySplit ks_) {
  constexpr int BM = 128 * NQB, BN = 64, NP = BM / HPW;
  constexpr int KCH = D / 8;                 // 16-byte chunks per row
  constexpr int LD = BN * KCH / 256;         // 16-byte chunks per thread per tile (K and V each)
  constexpr int NDB = D / 32;                // 32-row blocks of O^T
  constexpr int NKS = D / 16;                // k-steps of the QK^T contraction
  static_assert(LD >= 1, "tile loads");
  typedef Fmt16<T> F;
  typedef typename F::v8 v8;

  // K and V tiles live in LDS unpadded (row = D 16-bit values), written by direct
  // HBM->LDS loads; 16-byte chunks are XOR-swizzled per row so the fragment
  // reads hit distinct banks (see kswz / vswz).
  // two buffers as separate arrays: with the loop unrolled by two, every LDS
  // read and every direct load names its buffer statically, so the compiler
  // can see that the tile being read is not the one being loaded (otherwise it
  // waits for the in-flight load before each read)
  __shared__ __attribute__((aligned(16))) u16 Ks0[BN * D];
  __shared__ __attribute__((aligned(16))) u16 Vs0[BN * D];
  __shared__ __attribute__((aligned(16))) u16 Ks1[BN * D];
  __shared__ __attribute__((aligned(16))) u16 Vs1[BN * D];
  // MASK = 2: per wave 32 query rows x 64 keys of fp32 mask (8 KiB);
  // MASK = 3: the workgroup's NP rows x 64 keys, two buffers
  __shared__ __attribute__((aligned(16))) float Ms[MASK == 2 ? 4 * 32 * BN : 1];
  __shared__ __attribute__((aligned(16))) float Mx0[MASK == 3 ? NP * BN : 1];
  __shared__ __attribute__((aligned(16))) float Mx1[MASK == 3 ? NP * BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;

  // block -> (query tile, key split, batch-head group); the group varies
  // fastest (one XCD per group), query tiles heaviest first under causal
  const int bid = blockIdx.x;
  const int bh = bid % n_bh;
  static_assert(!SPLIT || MASK == 0, "key splits are for unmasked launches");
  const int nsplit = SPLIT ? ks_.n : 1;
  const int split = (bid / n_bh) % nsplit;
  const int qi = bid / n_bh / nsplit;
  const int qt = CAUSAL ? (n_qt - 1 - qi) : qi;
  const int HG = Hq / HPW;
  const int b = bh / HG;
  const int h0 = (bh % HG) * HPW;
  const int kvh = h0 / (Hq / Hkv);
  const int p0 = qt * NP;
  // Keys of this batch: Skv_all, or with a cache (kv_lens non-null) the
  // batch's cached rows (clamped to the capacity) plus the Sq new ones.  K and
  // V hold kv_rows rows per batch.
  const int Skv = kv_lens ? min(max(kv_lens[b], 0), kv_rows - Sq) + Sq : Skv_all;
  const int off = Skv - Sq;

  // this lane's query columns: qb-th block of 32 columns of wave w
  int hh[NQB], pos[NQB];
  bool qvalid[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int gc = (w * NQB + qb) * 32 + c;
    hh[qb] = h0 + gc / NP;
    pos[qb] = p0 + gc % NP;
    qvalid[qb] = pos[qb] < Sq;
  }

  // with a mask, the scores are scaled (and the mask added) right after the
  // contraction, so the softmax below only converts to base 2
  const float sl = MASK ? kLog2e : scale_log2;
  const float* mrow[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
    mrow[qb] = MASK == 1 ? mask.p + b * mask.bs + hh[qb] * mask.hs +
                               (long long)(qvalid[qb] ? pos[qb] : 0) * mask.rs
                         : nullptr;

  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, min(p0 + NP, Sq) - 1 + off + 1);
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int first_q = p0 + off;  // smallest query position of the workgroup
  // key tiles of this workgroup: all, or with nsplit > 1 the split-th of
  // nsplit runs of ceil(ntiles / nsplit) tiles (possibly empty)
  int t_lo = 0, t_hi = ntiles;
  if constexpr (SPLIT) {
    const int per = (ntiles + nsplit - 1) / nsplit;
    t_lo = min(ntiles, split * per);
    t_hi = min(ntiles, t_lo + per);
  }

  // K and V of this (batch, kv head) through range-checked buffer resources:
  // rows at or past Skv read as zero, offsets are 32-bit.
  const long long head_base = (long long)b * kv_rows * Hkv * D + (long long)kvh * D;
  const uint32_t nbytes = (uint32_t)(((long long)Skv * Hkv * D - (long long)kvh * D) * 2);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + head_base), (short)0, nbytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + head_base), (short)0, nbytes, kBufferWord3);
  const uint32_t row_bytes = (uint32_t)Hkv * D * 2;

  // A direct load writes lane l's 16 bytes to LDS base + 16 l, so slot
  // s = (w*LD + i)*64 + lane of a tile is filled by this lane: it fetches the
  // logical chunk that the swizzle places at (row s / KCH, chunk s % KCH).
  uint32_t koff[LD], voff[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int sl = (w * LD + i) * 64 + lane, row = sl / KCH, phys = sl % KCH;
    koff[i] = (uint32_t)row * row_bytes + (uint32_t)(phys ^ kswz<D>(row)) * 16u;
    voff[i] = (uint32_t)row * row_bytes + (uint32_t)(phys ^ vswz<D>(row)) * 16u;
  }
  // MASK = 2: this wave's mask rows r = 0..31 (its query columns) through a
  // buffer resource based at the wave's first head; direct-load instruction i
  // fills LDS rows 4i .. 4i+3, lane l the physical chunk l % 16 of row
  // 4i + l / 16, which holds the row's logical chunk (l % 16) ^ (row % 16).
  // The host takes this path only when every offset fits in 31 bits and Skv is
  // a multiple of 4, so the resource's range ends on a chunk boundary: past the
  // last valid element whole chunks read zeros.
  // MASK = 3: rows r = 0..NP-1 are positions p0 + r; wave w issues
  // instructions i < NI of the NP / 4 that fill them (LDS rows 4(w NI + i) ..
  // +3), and lane (c, g) reads row (32 w + c) mod NP, its own position.
  constexpr int NI = MASK == 3 ? NP / 16 : 8;
  __amdgpu_buffer_rsrc_t rm;
  uint32_t moff[NI];
  int mrd[2][4];  // LDS float offset of this lane's run (blk, a)
  float* Mw = Ms + w * 32 * BN;
  if constexpr (MASK == 3) {
    const long long last = (long long)(Sq - 1) * mask.rs + Skv;
    const uint32_t mbytes = (uint32_t)min(last * 4, 0xFFFFFFFFLL);
    rm = __builtin_amdgcn_make_buffer_rsrc((void*)(mask.p + b * mask.bs), (short)0, mbytes,
                                           kBufferWord3);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = 4 * (w * NI + i) + (lane >> 4);
      int pr = p0 + r;
      pr = pr < Sq ? pr : 0;
      const int lc = (lane & 15) ^ (r & 15);
      moff[i] = (uint32_t)(((long long)pr * mask.rs + 4 * lc) * 4);
    }
    const int r = (w * 32 + c) % NP;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int a = 0; a < 4; ++a) mrd[blk][a] = r * BN + (((8 * blk + 2 * a + g) ^ (r & 15)) << 2);
  }
  if constexpr (MASK == 2) {
    const int hw = h0 + (w * 32) / NP;
    const long long last = (long long)(Hq - 1 - hw) * mask.hs + (long long)(Sq - 1) * mask.rs + Skv;
    const uint32_t mbytes = (uint32_t)min(last * 4, 0xFFFFFFFFLL);
    rm = __builtin_amdgcn_make_buffer_rsrc((void*)(mask.p + b * mask.bs + hw * mask.hs), (short)0,
                                           mbytes, kBufferWord3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4), gc = w * 32 + r;
      const int hr = h0 + gc / NP;
      int pr = p0 + gc % NP;
      pr = pr < Sq ? pr : 0;
      const int lc = (lane & 15) ^ (r & 15);
      moff[i] = (uint32_t)(((long long)(hr - hw) * mask.hs + (long long)pr * mask.rs + 4 * lc) * 4);
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int a = 0; a < 4; ++a) mrd[blk][a] = c * BN + (((8 * blk + 2 * a + g) ^ (c & 15)) << 2);
  }
  auto dma = [&](int k0, u16* kb, u16* vb) {
    dma_tile<LD>(rk, rv, kb + w * LD * 64 * 8, vb + w * LD * 64 * 8, koff, voff,
                 (uint32_t)k0 * row_bytes);
  };

  // fragment addressing (elements within a tile buffer)
  int ka_off[2][NKS];  // K fragment of key block blk, k-step ks: row blk*32 + c, chunk 2ks + g
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int row = blk * 32 + c;
      ka_off[blk][ks] = row * D + ((2 * ks + g) ^ kswz<D>(row)) * 8;
    }
  // V^T fragments by transpose reads: lane (group tq, index tl) addresses row
  // 16kc + 8r + 4g + tl/4 and logical column 32db + 16(tq&1) + 4(tl&3)
  const int tq = lane >> 4, tl = lane & 15;
  int va_off[NDB][4][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = 16 * kc + 8 * r + 4 * (tq >> 1) + (tl >> 2);
        const int col = 32 * db + 16 * (tq & 1) + 4 * (tl & 3);
        va_off[db][kc][r] = row * D + (((col >> 3) ^ vswz<D>(row)) << 3) + (col & 7);
      }

  f32x16 oacc[NQB][NDB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  // m_run is a reference maximum (log2 domain): the true running maximum never
  // exceeds it by more than 8, so every probability stays <= 2^8; it is moved
  // (and O, l rescaled) only when a score would break that bound.  O / l and
  // m_run + log2(l) do not depend on which reference is used.
  float m_run[NQB], l_run[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  // ---- query fragments: lane holds q[pos, hh, 16ks + 8g .. +7] for every ks.
  // Columns past Sq read row 0 (and its table row) and are zeroed afterwards:
  // with no per-lane branch every load of the prologue (fragments, table
  // entries, the first tile) is in flight at once, and the rotation waits for
  // its own operands only, while the tile's direct loads land.
  v8 qf[NQB][NKS];
  {
    u32x4 qw[NQB][NKS];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const u16* qp =
          Q + (((long long)b * Sq + (qvalid[qb] ? pos[qb] : 0)) * Hq + hh[qb]) * D + g * 8;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qw[qb][ks] = *reinterpret_cast<const u32x4*>(qp + ks * 16);
    }
    double2 cs[NQB][NKS][4];
    if constexpr (ROPE) {
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
    if (t_hi > t_lo) {
      dma(t_lo * BN, Ks0, Vs0);
      if constexpr (MASK == 2) dma_rows<8>(rm, reinterpret_cast<u16*>(Mw), moff, 0u);
      if constexpr (MASK == 3)
        dma_rows<NI>(rm, reinterpret_cast<u16*>(Mx0 + w * NI * 256), moff, 0u);
    }
    if constexpr (ROPE) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            double r0, r1;
            rotate_pair((double)F::lo(qw[qb][ks][e]), (double)F::hi(qw[qb][ks][e]),
                        cs[qb][ks][e], r0, r1);
            qw[qb][ks][e] = F::from_f64(r0) | (F::from_f64(r1) << 16);
          }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 wv = qw[qb][ks];
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] = qvalid[qb] ? wv[e] : 0u;
        // an empty register constraint keeps the fragment (and so its loads)
        // ahead of the barrier below, which the compiler would otherwise let
        // read-only loads sink past
        asm volatile("" : "+v"(wv));
        qf[qb][ks] = __builtin_bit_cast(v8, wv);
      }
  }

  // everything the prologue loaded (query fragments, first tile) has landed
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // one key/value tile: its K and V are in (kc_, vc_); the next tile is loaded
  // into (kn_, vn_), last read in the previous step, which every wave has left
  // (likewise the shared mask rows, MASK = 3, in mc_ and mn_)
  auto tile = [&](int t, const u16* kc_, const u16* vc_, u16* kn_, u16* vn_, const float* mc_,
                  float* mn_) {
    const int k0 = t * BN;
    // mask values of this lane's 32 (query, key) pairs: keys
    // k0 + 32 blk + 8a + 4g + e at accumulator row 4a + e; 0 past Skv.
    // D = 64 issues them before the contraction (their latency hides behind
    // it); D = 128 after it, where holding them across it would cost the
    // registers of a second wave per SIMD.
    float mv[NQB][2][16];
    auto load_mask = [&]() {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int j0 = k0 + blk * 32 + 8 * a + 4 * g;
            const float* mp = mrow[qb] + j0;
            if (mask.vec && j0 + 4 <= Skv) {
              const float4 x = *reinterpret_cast<const float4*>(mp);
              mv[qb][blk][4 * a] = x.x;
              mv[qb][blk][4 * a + 1] = x.y;
              mv[qb][blk][4 * a + 2] = x.z;
              mv[qb][blk][4 * a + 3] = x.w;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) mv[qb][blk][4 * a + e] = j0 + e < Skv ? mp[e] : 0.f;
            }
          }
    };
    if constexpr (MASK == 1 && D == 64) load_mask();
    if (!ONEBUF && t + 1 < t_hi) {
      dma(k0 + BN, kn_, vn_);
      if constexpr (MASK == 3)
        dma_rows<NI>(rm, reinterpret_cast<u16*>(mn_ + w * NI * 256), moff, (uint32_t)(k0 + BN) * 4u);
    }

    // S^T (64 keys x 32 queries per block) = K_tile Q^T
    f32x16 s[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[qb][0][r] = s[qb][1][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const v8 ka = *reinterpret_cast<const v8*>(&kc_[ka_off[blk][ks]]);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) s[qb][blk] = F::mfma(ka, qf[qb][ks], s[qb][blk]);
      }
    }

    if constexpr (MASK == 3) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(mc_ + mrd[blk][a]);
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[0][blk][4 * a + e] = x[e];
        }
    }
    if constexpr (MASK == 2) {
      // this tile's rows landed with the previous end-of-tile wait
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(Mw + mrd[blk][a]);
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[0][blk][4 * a + e] = x[e];
        }
      // the reads are done before the next tile's rows overwrite the area
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < t_hi)
        dma_rows<8>(rm, reinterpret_cast<u16*>(Mw), moff, (uint32_t)(k0 + BN) * 4u);
    }
    if constexpr (MASK != 0) {
      if constexpr (MASK == 1 && D != 64) load_mask();
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[qb][blk][r] = fmaf(s[qb][blk][r], scale, mv[qb][blk][r]);
    }

    // mask: key rows past Skv, and keys after the query under the causal rule
    const bool need_mask = (k0 + BN > Skv) || (CAUSAL && k0 + BN - 1 > first_q);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qlim = CAUSAL ? min(pos[qb] + off, Skv - 1) : Skv - 1;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = k0 + blk * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (j > qlim) s[qb][blk][r] = -INFINITY;
          }
      }
    }

    // online softmax for this lane's query columns
    v8 pf[NQB][4];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = fmaxf(s[qb][0][0], s[qb][0][1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[qb][0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][1][r]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float mxs = mx * sl;
      if (__builtin_amdgcn_ballot_w64(mxs > m_run[qb] + 8.f)) {  // wave-uniform
        const float m_new = fmaxf(m_run[qb], mxs);
        const float alpha =
            __builtin_amdgcn_exp2f(m_run[qb] - (m_new == -INFINITY ? 0.f : m_new));
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
        m_run[qb] = m_new;
      }
      const float m_use = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
      float ls = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[qb][blk][r], sl, -m_use));
          s[qb][blk][r] = p;
          ls += p;
        }
      l_run[qb] += ls;  // per half-wave partial; the halves are added after the loop
      // probabilities as 16-bit B operands: chunk kc covers keys 16kc .. 16kc+15
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[qb][kc][e] = (T)s[qb][kc >> 1][(kc & 1) * 8 + e];
    }

    // O^T (D x 32) += V^T (D x 64) P^T (64 x 32); V^T fragments by transpose reads
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const s16x4 lo = lds_read_tr16(&vc_[va_off[db][kc][0]]);
        const s16x4 hi = lds_read_tr16(&vc_[va_off[db][kc][1]]);
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 vv = {lo2[0], lo2[1], hi2[0], hi2[1]};
        const v8 va = __builtin_bit_cast(v8, vv);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) oacc[qb][db] = F::mfma(va, pf[qb][kc], oacc[qb][db]);
      }
    }

    if (ONEBUF) {
      __syncthreads();  // every wave is done with this tile's buffers
      if (t + 1 < t_hi) {
        dma(k0 + BN, kn_, vn_);
        if constexpr (MASK == 3)
          dma_rows<NI>(rm, reinterpret_cast<u16*>(mn_ + w * NI * 256), moff,
                       (uint32_t)(k0 + BN) * 4u);
      }
    }
    // the next tile's direct loads have landed and every wave is done with this one
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };
  // the second buffers (the first ones again in ONEBUF instances)
  u16* const Kb1 = ONEBUF ? Ks0 : Ks1;
  u16* const Vb1 = ONEBUF ? Vs0 : Vs1;
  float* const Mb1 = ONEBUF ? Mx0 : Mx1;
  for (int t = t_lo; t < t_hi; t += 2) {
    tile(t, Ks0, Vs0, Kb1, Vb1, Mx0, Mb1);
    if (t + 1 < t_hi) tile(t + 1, Kb1, Vb1, Ks0, Vs0, Mb1, Mx0);
  }

  if constexpr (SPLIT) {
    // partial result over this run of keys: O normalised by its own sum and
    // its natural-log LSE (-inf when no key of the run is visible), at
    // [row][split] with row = (b*Sq + pos)*Hq + h (O's row order), so one
    // row's runs are contiguous for the combine kernel
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[qb]),
                                                       __float_as_uint(l_run[qb]), false, false);
      const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if (qvalid[qb]) {
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        const long long slot = (((long long)b * Sq + pos[qb]) * Hq + hh[qb]) * nsplit + split;
        float* op = ks_.o + slot * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 x = {oacc[qb][db][4 * a] * inv, oacc[qb][db][4 * a + 1] * inv,
                             oacc[qb][db][4 * a + 2] * inv, oacc[qb][db][4 * a + 3] * inv};
            *reinterpret_cast<f32x4*>(op + db * 32 + 8 * a + 4 * g) = x;
          }
        if (g == 0)
          ks_.l[slot] = (l_tot > 0.f) ? (m_run[qb] + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
    }
    return;
  }

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

template <bool ONEBUF, typename T, int D, int HPW, bool CAUSAL, bool ROPE, int NQB, int MASK,
          bool SPLIT>
static hipError_t go16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int Hq, int Hkv, int Sq, int Skv, const int* kv_lens, int kv_rows,
                          float scale, const double2* tab, MaskView mask, KeySplit ks,
                          hipStream_t stream) {
  constexpr int NP = 128 * NQB / HPW;
  const int n_qt = (Sq + NP - 1) / NP;
  const int n_bh = B * (Hq / HPW);
  const int nsplit = SPLIT ? ks.n : 1;
  const long long nblocks = (long long)n_qt * n_bh * nsplit;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_kernel(fwd16_kernel<T, D, HPW, CAUSAL, ROPE, NQB, MASK, SPLIT, ONEBUF>,
                dim3((unsigned)nblocks), dim3(256), stream, static_cast<const u16*>(q),
                static_cast<const u16*>(k), static_cast<const u16*>(v), static_cast<u16*>(o), lse,
                Hq, Hkv, Sq, Skv, kv_lens, kv_rows, scale * kLog2e, tab, n_qt, n_bh, mask, scale,
                ks);
  if constexpr (SPLIT) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_fwd16_merge(ks.o, ks.l, o, lse, (long long)B * Sq * Hq, Sq, Hq, nsplit, D,
                              std::is_same<T, __bf16>::value ? 1 : 2, stream);
  }
  return hipGetLastError();
}

// Two query blocks per wave halve the LDS traffic per MFMA (D = 64, where the
// registers allow it); one block keeps small problems spread over more
// workgroups (at least two per CU).  Masked runs use one block (the mask
// values take the registers a second block would need).
template <bool ONEBUF, typename T, int D, int HPW, bool CAUSAL, bool ROPE>
static hipError_t go16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int Hq, int Hkv, int Sq, int Skv, const int* kv_lens, int kv_rows,
                          float scale, const double2* tab, MaskView mask, KeySplit ks,
                          hipStream_t stream) {
  // an under-filled unmasked launch: one query block per wave, key splits
  if (mask.p == nullptr && ks.n > 1)
    return go16<ONEBUF, T, D, HPW, CAUSAL, ROPE, 1, 0, true>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv,
                                                     kv_lens, kv_rows, scale, tab, mask, ks, stream);
  if (mask.p != nullptr) {
    // staged mask rows for D = 64 when the loads can be 16-byte, the end of
    // the valid data (Skv keys into the last row) falls on a 16-byte boundary
    // (a load that straddles the buffer's range end may read zeros as a whole),
    // and every per-lane offset (a head step, a query row, a tile past the
    // keys) fits in 31 bits
    if constexpr (D == 64) {
      const long long reach = (mask.hs + (long long)Sq * mask.rs + Skv + 2 * 64) * 4;
      if (mask.vec && Skv % 4 == 0 && reach < (1LL << 31)) {
        // rows shared by the workgroup's heads when the mask is the same for all
        if constexpr (HPW >= 2)
          if (mask.hs == 0)
            return go16<ONEBUF, T, D, HPW, CAUSAL, ROPE, 1, 3, false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv,
                                                       kv_lens, kv_rows, scale, tab, mask, ks, stream);
        return go16<ONEBUF, T, D, HPW, CAUSAL, ROPE, 1, 2, false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens,
                                                   kv_rows, scale, tab, mask, ks, stream);
      }
    }
    return go16<ONEBUF, T, D, HPW, CAUSAL, ROPE, 1, 1, false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens,
                                               kv_rows, scale, tab, mask, ks, stream);
  }
  if constexpr (D == 64) {
    const long long wg2 = (long long)((Sq + 256 / HPW - 1) / (256 / HPW)) * B * (Hq / HPW);
    if (wg2 >= 2 * 256)
      return go16<ONEBUF, T, D, HPW, CAUSAL, ROPE, 2, 0, false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv,
                                                     kv_lens, kv_rows, scale, tab, mask, ks, stream);
  }
  return go16<ONEBUF, T, D, HPW, CAUSAL, ROPE, 1, 0, false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens,
                                                 kv_rows, scale, tab, mask, ks, stream);
}

template <bool ONEBUF, typename T, int D, bool CAUSAL, bool ROPE>
static hipError_t pick_hpw(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int Sq, int Skv, const int* kv_lens,
                           int kv_rows, float scale, const double2* tab, MaskView mask,
                           KeySplit ks, hipStream_t stream) {
  const int G = Hq / Hkv;
  if (G % 8 == 0)
    return go16<ONEBUF, T, D, 8, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows,
                                       scale, tab, mask, ks, stream);
  if (G % 4 == 0)
    return go16<ONEBUF, T, D, 4, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows,
                                       scale, tab, mask, ks, stream);
  if (G % 2 == 0)
    return go16<ONEBUF, T, D, 2, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows,
                                       scale, tab, mask, ks, stream);
  return go16<ONEBUF, T, D, 1, CAUSAL, ROPE>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows,
                                     scale, tab, mask, ks, stream);
}

template <bool ONEBUF, typename T>
static hipError_t launch_fmt(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                             float scale, const double2* rope_tab, hipStream_t stream,
                             const int* kv_lens, int kv_rows, MaskView mask, KeySplit ks) {
  const bool rope = rope_tab != nullptr;
#define XATTN_FWD16_CASE(DD, C, R)                                                         \
  if (D == DD && (causal != 0) == C && rope == R)                                          \
    return pick_hpw<ONEBUF, T, DD, C, R>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, kv_lens, kv_rows, scale, \
                                 rope_tab, mask, ks, stream);
  XATTN_FWD16_CASE(64, false, false)
  XATTN_FWD16_CASE(64, true, false)
  XATTN_FWD16_CASE(64, false, true)
  XATTN_FWD16_CASE(64, true, true)
  XATTN_FWD16_CASE(128, false, false)
  XATTN_FWD16_CASE(128, true, false)
  XATTN_FWD16_CASE(128, false, true)
  XATTN_FWD16_CASE(128, true, true)
#undef XATTN_FWD16_CASE
  return hipErrorInvalidValue;
}

// launch_fwd16's masked / key-split forward (ONEBUF = false) or its
// single-buffer check (ONEBUF = true): arguments as there, kv_rows set
template <bool ONEBUF>
static hipError_t launch_fwd16_kernel(const void* q, const void* k, const void* v, void* o,
                                      float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D,
                                      int causal, float scale, const double2* rope_tab, int dtype,
                                      hipStream_t stream, const int* kv_lens, int kv_rows,
                                      MaskView mask, KeySplit ks) {
  if (dtype == 1)
    return launch_fmt<ONEBUF, __bf16>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                                      rope_tab, stream, kv_lens, kv_rows, mask, ks);
  if (dtype == 2)
    return launch_fmt<ONEBUF, _Float16>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                                        rope_tab, stream, kv_lens, kv_rows, mask, ks);
  return hipErrorInvalidValue;
}

}  // namespace xattn
