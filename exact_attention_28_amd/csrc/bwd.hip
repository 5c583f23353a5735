// bwd.hip — attention backward on gfx950 for 16-bit inputs (bf16, or IEEE
// binary16 / fp16 through the same kernels with that format's MFMA and
// conversions) with D = 64.
//
// The gradient of O = softmax(scale * Q~ K~^T) V for an upstream gradient dO,
// as in the FA-2 backward per head of scirs2-neural 0.4.3
// src/layers/flash_attention.rs (fn flash_backward_head), with the sums over
// the query heads of a group and the inverse rotation of scirs2-neural 0.4.4
// src/layers/grouped_query_attention.rs (backward through grouped attention):
//   P_ij  = exp(s_ij - lse_i)              (lse saved by the forward)
//   D_i   = sum_d dO_i[d] O_i[d]
//   dV_j  = sum over the group's heads h and rows i of P_ij dO_i
//   dS_ij = P_ij (<dO_i, v_j> - D_i)
//   dQ~_i = scale sum_j dS_ij k~_j,   dK~_j = scale sum_{h,i} dS_ij q~_i
//   dq = R^T dQ~, dk = R^T dK~        (RoPE: rotation by the negated angle)
//
// Three kernels, deterministic (no atomics):
//  * bwd_prep_kernel: -D_i in fp32 (the dK/dV kernel starts its dP
//    accumulators from it, so the MFMAs produce dP - D), and lse in log2 units
//    with +inf for a row without visible keys (so that its P is 0).
//  * bwd_dkdv_kernel: one workgroup per (key tile of 128, batch, kv head).  The
//    tile's K and V stay in registers (MFMA B operands) while the Q and dO
//    tiles of every query head of the group stream through LDS; per 64-query
//    tile a wave computes S = Q K^T and dP = dO V^T (32 queries x 32 keys per
//    block), P and dS in registers, then dV^T += dO^T P and dK^T += Q^T dS
//    with dO^T and Q^T read by LDS transpose reads.  dK and dV accumulate in
//    registers over the whole group.
//  * bwd_dq_kernel: one workgroup per (query tile, batch, head group), shaped
//    like the forward kernel: Q and dO in registers, K and V tiles stream
//    through LDS; S^T and dP^T are recomputed here rather than passed through
//    memory, and dQ^T += K^T dS^T.
// Q and K arrive already rotated (the caller stages them); the epilogues of
// dK and dQ apply the inverse rotation in fp64.
// Both streaming kernels double-buffer their LDS tiles; ONEBUF instances (a
// check of that ordering) use one buffer, refilled after a barrier behind its
// last read, with the same arithmetic in the same order: bit-identical
// gradients.

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lds.h"

namespace xattn {

namespace {

constexpr int kD = 64;   // head dim of these kernels
constexpr int kKCH = 8;  // 16-byte chunks per row

// Chunk swizzle for tiles that are read both by rows (16 rows at one logical
// chunk: 16 distinct bank groups) and by transpose reads (4 rows x 2 adjacent
// chunks: 8 distinct groups).  With x = (row >> 1) & 7 the XOR value is x with
// its bits rotated right by one: within each row parity it runs over all 8
// values (row reads), and rows 4m and 4m+2 get values that differ above bit 0
// (transpose reads).  Group of (row, chunk) = (8 row + chunk) mod 16.
__device__ __forceinline__ int bswz(int row) {
  const int x = (row >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}

// element offset of (row, logical column) in a swizzled 64-wide 16-bit tile
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * kD + (((col >> 3) ^ bswz(row)) << 3) + (col & 7);
}

// MFMA A operand from a swizzled tile by rows: lane (r = lane mod 32, g)
// receives row row0 + r, columns 16 ks + 8 g .. +7.
template <typename T>
__device__ __forceinline__ typename Fmt16<T>::v8 rows_frag(const u16* t, int row0, int c, int g,
                                                           int ks) {
  return *reinterpret_cast<const typename Fmt16<T>::v8*>(&t[tile_off(row0 + c, 16 * ks + 8 * g)]);
}

// MFMA A operand of the transposed tile (columns become rows): lane (i, g)
// receives column 32 db + i at tile rows 16 kc + 8 (e / 4) + 4 g + (e mod 4),
// e = 0..7 — the order of the k slots in a 32x32 accumulator's lane.
template <typename T>
__device__ __forceinline__ typename Fmt16<T>::v8 trans_frag(const u16* t, int lane, int db,
                                                            int kc) {
  const int tq = lane >> 4, tl = lane & 15;
  const int col = 32 * db + 16 * (tq & 1) + 4 * (tl & 3);
  const int row = 16 * kc + 4 * (tq >> 1) + (tl >> 2);
  const s16x4 lo = lds_read_tr16(&t[tile_off(row, col)]);
  const s16x4 hi = lds_read_tr16(&t[tile_off(row + 8, col)]);
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  const u32x4 vv = {lo2[0], lo2[1], hi2[0], hi2[1]};
  return __builtin_bit_cast(typename Fmt16<T>::v8, vv);
}

// Stores a 32-column block of a transposed accumulator pair acc[db] (rows d,
// columns = this lane's row of the output) in the format T: lane (c, g) holds
// d = 32 db + 8 a + 4 g + e for a, e < 4.  With tab non-null the pairs
// (d, d+1) are rotated back (R^T at the table row given) in fp64.
template <typename T>
__device__ __forceinline__ void store_row(u16* out, const f32x16* acc, float mul, int g,
                                          const double2* tabrow) {
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d = db * 32 + 8 * a + 4 * g;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * a + e] * mul;
      u32x2 pk;
      if (tabrow != nullptr) {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const double2 cs = tabrow[d / 2 + pr];
          const double x0 = x[2 * pr], x1 = x[2 * pr + 1];
          const double r0 = x0 * cs.x + x1 * cs.y;
          const double r1 = -x0 * cs.y + x1 * cs.x;
          pk[pr] = Fmt16<T>::from_f64(r0) | (Fmt16<T>::from_f64(r1) << 16);
        }
      } else {
        pk[0] = Fmt16<T>::pack(x[0], x[1]);
        pk[1] = Fmt16<T>::pack(x[2], x[3]);
      }
      *reinterpret_cast<u32x2*>(out + d) = pk;
    }
}

}  // namespace

// ---------------------------------------------------------------- prep --

template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const u16* __restrict__ O,
                                                       const u16* __restrict__ dO,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ ndelta,
                                                       float* __restrict__ lse2, int B, int Sq,
                                                       int Hq) {
  // 8 lanes per (b, i, h) row of 64 16-bit values, rows in [B, Sq, Hq] order
  const long long row = (long long)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  const long long nrows = (long long)B * Sq * Hq;
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * kD + part * 8);
    const u32x4 c = *reinterpret_cast<const u32x4*>(dO + row * kD + part * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(Fmt16<T>::lo(a[e]), Fmt16<T>::lo(c[e]), acc);
      acc = fmaf(Fmt16<T>::hi(a[e]), Fmt16<T>::hi(c[e]), acc);
    }
  }
  acc = group_sum<8>(acc);
  if (row < nrows && part == 0) {
    const int h = (int)(row % Hq);
    const long long bi = row / Hq;
    const int i = (int)(bi % Sq);
    const int b = (int)(bi / Sq);
    const long long o = ((long long)b * Hq + h) * Sq + i;
    ndelta[o] = -acc;
    const float l = lse[o];
    lse2[o] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------- dK, dV --

template <typename T, bool CAUSAL, bool ROPE, bool ONEBUF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    const u16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ ndelta,
    u16* __restrict__ dK, u16* __restrict__ dV, int Hq, int Hkv, int Sq, int Skv, float scale,
    float scale_log2, const double2* __restrict__ tab, int n_bh) {
  constexpr int D = kD, BQ = 64, BK = 128, NKS = D / 16;
  constexpr int LD = BQ * kKCH / 256;  // direct loads per thread per tile and tensor
  static_assert(LD == 2, "layout assumed below");
  typedef Fmt16<T> F;
  typedef typename F::v8 v8;

  __shared__ __attribute__((aligned(16))) u16 Qs0[BQ * D];
  __shared__ __attribute__((aligned(16))) u16 Os0[BQ * D];  // dO
  __shared__ __attribute__((aligned(16))) u16 Qs1[BQ * D];
  __shared__ __attribute__((aligned(16))) u16 Os1[BQ * D];
  __shared__ __attribute__((aligned(16))) float Ls0[BQ];  // lse (log2), per tile row
  __shared__ __attribute__((aligned(16))) float Ds0[BQ];  // -D_i
  __shared__ __attribute__((aligned(16))) float Ls1[BQ];
  __shared__ __attribute__((aligned(16))) float Ds1[BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int kt = blockIdx.x / n_bh, bh = blockIdx.x % n_bh;  // heavy (early) key tiles first
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int G = Hq / Hkv, h0 = kvh * G;
  const int off = Skv - Sq;
  const int k0 = kt * BK;          // first key of the workgroup
  const int kw0 = k0 + 32 * w;     // first key of this wave
  const int key = kw0 + c;         // this lane's key (accumulator column)

  // K and V of the wave's 32 keys as B operands: lane (c, g), k-step ks holds
  // columns 16 ks + 8 g .. +7 of key `key`; keys past Skv are zero.
  v8 kf[NKS], vf[NKS];
  {
    const bool ok = key < Skv;
    const long long base = (((long long)b * Skv + (ok ? key : 0)) * Hkv + kvh) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, v = {0u, 0u, 0u, 0u};
      if (ok) {
        a = *reinterpret_cast<const u32x4*>(K + base + 16 * ks);
        v = *reinterpret_cast<const u32x4*>(V + base + 16 * ks);
      }
      kf[ks] = __builtin_bit_cast(v8, a);
      vf[ks] = __builtin_bit_cast(v8, v);
    }
  }

  // query tiles: every head of the group, positions from the first that sees
  // a key of this workgroup (causal) to Sq
  const int n_qt = (Sq + BQ - 1) / BQ;
  int qt0 = 0;
  if (CAUSAL) qt0 = max(0, k0 - off) / BQ;
  const int nq = max(0, n_qt - qt0);
  const int n_it = G * nq;

  // Q and dO rows of head h0 + hg through range-checked buffer resources based
  // at (b, row 0, h0): rows at or past Sq read as zero.
  const long long qbase = (long long)b * Sq * Hq * D + (long long)h0 * D;
  const uint32_t nbytes = (uint32_t)(((long long)Sq * Hq * D - (long long)h0 * D) * 2);
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Q + qbase), (short)0, nbytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc((void*)(dO + qbase), (short)0, nbytes, kBufferWord3);
  const uint32_t row_bytes = (uint32_t)Hq * D * 2;
  uint32_t soff[LD];  // this lane's slots: logical chunk of (row, physical chunk)
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int sl = (w * LD + i) * 64 + lane, row = sl / kKCH, phys = sl % kKCH;
    soff[i] = (uint32_t)row * row_bytes + (uint32_t)(phys ^ bswz(row)) * 16u;
  }
  // lse / D of a tile: threads 0..63 load lse rows, 64..127 load D rows
  auto stat_load = [&](int it) __attribute__((always_inline)) {
    float x = 0.f;
    if (tid < 2 * BQ && it < n_it) {
      const int hg = it / nq, qt = qt0 + it % nq;
      const int p = qt * BQ + (tid & (BQ - 1));
      const long long o = ((long long)b * Hq + h0 + hg) * Sq + p;
      if (tid < BQ)
        x = (p < Sq) ? lse2[o] : INFINITY;
      else
        x = (p < Sq) ? ndelta[o] : 0.f;
    }
    return x;
  };
  auto stat_store = [&](float x, float* ls, float* ds) __attribute__((always_inline)) {
    if (tid < BQ)
      ls[tid] = x;
    else if (tid < 2 * BQ)
      ds[tid - BQ] = x;
  };
  auto dma = [&](int it, u16* qd, u16* od) __attribute__((always_inline)) {
    const int hg = it / nq, qt = qt0 + it % nq;
    const uint32_t t0 = (uint32_t)(qt * BQ) * row_bytes + (uint32_t)(hg * D * 2);
    dma_rows<LD>(rq, qd + w * LD * 64 * 8, soff, t0);
    dma_rows<LD>(ro, od + w * LD * 64 * 8, soff, t0);
  };

  f32x16 dvacc[2], dkacc[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dvacc[db][r] = dkacc[db][r] = 0.f;

  auto tile = [&](int it, const u16* qs, const u16* os, const float* ls, const float* ds)
                  __attribute__((always_inline)) {
    const int qt = qt0 + it % nq;
    const int p0 = qt * BQ;
    // whole tile above the diagonal for this wave: every P is 0
    if (CAUSAL && kw0 > p0 + BQ - 1 + off) return;

    // S = Q K^T and dP - D = dO V^T - D: blocks of 32 queries (rows) x 32 keys,
    // the dP accumulators starting from the tile rows' -D_i
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&ds[32 * qb + 8 * a + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[qb][4 * a + e] = 0.f;
          dp[qb][4 * a + e] = d4[e];
        }
      }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[qb] = F::mfma(rows_frag<T>(qs, 32 * qb, c, g, ks), kf[ks], s[qb]);
        dp[qb] = F::mfma(rows_frag<T>(os, 32 * qb, c, g, ks), vf[ks], dp[qb]);
      }

    // P = exp2(c s - lse2) in place of S; lane holds tile rows
    // 32 qb + 8 a + 4 g + e (a, e < 4) of column `key`
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&ls[32 * qb + 8 * a + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[qb][4 * a + e] = __builtin_amdgcn_exp2f(fmaf(s[qb][4 * a + e], scale_log2, -l4[e]));
      }
    // causal: zero P above the diagonal on the tiles the diagonal crosses, in a
    // wave-uniform branch (a mask test inside the loop above would become
    // selects executed on every tile)
    if (CAUSAL && kw0 + 31 > p0 + off) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key > p0 + 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3) + off) s[qb][r] = 0.f;
    }
    // dS = P (dP - D); P and dS as 16-bit B operands
    v8 pf[4], sf[4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // k slot r of query block qb: chunk 2 qb + r / 8, element r mod 8
        pf[2 * qb + r / 8][r % 8] = (T)s[qb][r];
        sf[2 * qb + r / 8][r % 8] = (T)(s[qb][r] * dp[qb][r]);
      }

    // dV^T += dO^T P and dK^T += Q^T dS (rows d, columns keys)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        dvacc[db] = F::mfma(trans_frag<T>(os, lane, db, kc), pf[kc], dvacc[db]);
        dkacc[db] = F::mfma(trans_frag<T>(qs, lane, db, kc), sf[kc], dkacc[db]);
      }
  };

  if (n_it > 0) {
    dma(0, Qs0, Os0);
    stat_store(stat_load(0), Ls0, Ds0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // the second buffers (the first ones again in ONEBUF instances, refilled
  // once every wave is done with them)
  u16* const Qb1 = ONEBUF ? Qs0 : Qs1;
  u16* const Ob1 = ONEBUF ? Os0 : Os1;
  float* const Lb1 = ONEBUF ? Ls0 : Ls1;
  float* const Db1 = ONEBUF ? Ds0 : Ds1;
  for (int it = 0; it < n_it; it += 2) {
    // the next tile goes into the other buffers, last read in the previous step
    float x = stat_load(it + 1);
    if (!ONEBUF && it + 1 < n_it) dma(it + 1, Qb1, Ob1);
    tile(it, Qs0, Os0, Ls0, Ds0);
    if (ONEBUF) {
      __syncthreads();
      if (it + 1 < n_it) dma(it + 1, Qb1, Ob1);
    }
    stat_store(x, Lb1, Db1);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (it + 1 >= n_it) break;
    x = stat_load(it + 2);
    if (!ONEBUF && it + 2 < n_it) dma(it + 2, Qs0, Os0);
    tile(it + 1, Qb1, Ob1, Lb1, Db1);
    if (ONEBUF) {
      __syncthreads();
      if (it + 2 < n_it) dma(it + 2, Qs0, Os0);
    }
    stat_store(x, Ls0, Ds0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }

  if (key < Skv) {
    const long long orow = (((long long)b * Skv + key) * Hkv + kvh) * D;
    store_row<T>(dV + orow, dvacc, 1.f, g, nullptr);
    store_row<T>(dK + orow, dkacc, scale, g, ROPE ? tab + (long long)key * (D / 2) : nullptr);
  }
}

// ---------------------------------------------------------------- dQ --

template <typename T, int HPW, bool CAUSAL, bool ROPE, bool ONEBUF>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    const u16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ ndelta,
    u16* __restrict__ dQ, int Hq, int Hkv, int Sq, int Skv, float scale, float scale_log2,
    const double2* __restrict__ tab, int n_qt, int n_bh) {
  constexpr int D = kD, BM = 128, BN = 64, NP = BM / HPW, NKS = D / 16;
  constexpr int LD = BN * kKCH / 256;
  static_assert(LD == 2, "layout assumed below");
  typedef Fmt16<T> F;
  typedef typename F::v8 v8;

  __shared__ __attribute__((aligned(16))) u16 Ks0[BN * D];
  __shared__ __attribute__((aligned(16))) u16 Vs0[BN * D];
  __shared__ __attribute__((aligned(16))) u16 Ks1[BN * D];
  __shared__ __attribute__((aligned(16))) u16 Vs1[BN * D];

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

  // this lane's query column: head hh, position pos
  const int gc = w * 32 + c;
  const int hh = h0 + gc / NP, pos = p0 + gc % NP;
  const bool qvalid = pos < Sq;
  const int qlim = CAUSAL ? min(pos + off, Skv - 1) : Skv - 1;

  v8 qf[NKS], of[NKS];
  float l2 = INFINITY, ndl = 0.f;
  {
    const long long base = (((long long)b * Sq + (qvalid ? pos : 0)) * Hq + hh) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, o = {0u, 0u, 0u, 0u};
      if (qvalid) {
        a = *reinterpret_cast<const u32x4*>(Q + base + 16 * ks);
        o = *reinterpret_cast<const u32x4*>(dO + base + 16 * ks);
      }
      qf[ks] = __builtin_bit_cast(v8, a);
      of[ks] = __builtin_bit_cast(v8, o);
    }
    if (qvalid) {
      const long long st = ((long long)b * Hq + hh) * Sq + pos;
      l2 = lse2[st];
      ndl = ndelta[st];
    }
  }

  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, min(p0 + NP, Sq) - 1 + off + 1);
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int first_q = p0 + off;

  const long long head_base = (long long)b * Skv * Hkv * D + (long long)kvh * D;
  const uint32_t nbytes = (uint32_t)(((long long)Skv * Hkv * D - (long long)kvh * D) * 2);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + head_base), (short)0, nbytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + head_base), (short)0, nbytes, kBufferWord3);
  const uint32_t row_bytes = (uint32_t)Hkv * D * 2;
  uint32_t soff[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int sl = (w * LD + i) * 64 + lane, row = sl / kKCH, phys = sl % kKCH;
    soff[i] = (uint32_t)row * row_bytes + (uint32_t)(phys ^ bswz(row)) * 16u;
  }
  auto dma = [&](int t, u16* kd, u16* vd) __attribute__((always_inline)) {
    const uint32_t t0 = (uint32_t)(t * BN) * row_bytes;
    dma_rows<LD>(rk, kd + w * LD * 64 * 8, soff, t0);
    dma_rows<LD>(rv, vd + w * LD * 64 * 8, soff, t0);
  };

  f32x16 dqacc[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  auto tile = [&](int t, const u16* ks_, const u16* vs_) __attribute__((always_inline)) {
    const int k0 = t * BN;
    // S^T = K Q^T and dP^T = V dO^T: blocks of 32 keys (rows) x 32 queries
    // (dP^T accumulators start from this lane's query's -D_i: the MFMAs yield dP - D)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = 0.f;
        dp[kb][r] = ndl;
      }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = F::mfma(rows_frag<T>(ks_, 32 * kb, c, g, ks), qf[ks], s[kb]);
        dp[kb] = F::mfma(rows_frag<T>(vs_, 32 * kb, c, g, ks), of[ks], dp[kb]);
      }
    // P^T in place of S^T; lane holds keys k0 + 32 kb + 8 a + 4 g + e of its
    // query.  Keys at or past Skv need no mask here: their K rows read as
    // zero, so their dS contributes nothing to dQ = K^T dS.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale_log2, -l2));
    // causal: zero P above the diagonal on the tiles the diagonal crosses (a
    // wave-uniform branch)
    if (CAUSAL && k0 + BN - 1 > first_q) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3) > qlim) s[kb][r] = 0.f;
    }
    // dS^T = P^T (dP^T - D) as 16-bit B operands
    v8 sf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sf[2 * kb + r / 8][r % 8] = (T)(s[kb][r] * dp[kb][r]);
    // dQ^T += K^T dS^T (rows d, columns queries)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int db = 0; db < 2; ++db)
        dqacc[db] = F::mfma(trans_frag<T>(ks_, lane, db, kc), sf[kc], dqacc[db]);
  };

  if (ntiles > 0) dma(0, Ks0, Vs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // the second buffers (the first ones again in ONEBUF instances, refilled
  // once every wave is done with them)
  u16* const Kb1 = ONEBUF ? Ks0 : Ks1;
  u16* const Vb1 = ONEBUF ? Vs0 : Vs1;
  for (int t = 0; t < ntiles; t += 2) {
    if (!ONEBUF && t + 1 < ntiles) dma(t + 1, Kb1, Vb1);
    tile(t, Ks0, Vs0);
    if (ONEBUF) {
      __syncthreads();
      if (t + 1 < ntiles) dma(t + 1, Kb1, Vb1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 1 >= ntiles) break;
    if (!ONEBUF && t + 2 < ntiles) dma(t + 2, Ks0, Vs0);
    tile(t + 1, Kb1, Vb1);
    if (ONEBUF) {
      __syncthreads();
      if (t + 2 < ntiles) dma(t + 2, Ks0, Vs0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }

  if (qvalid)
    store_row<T>(dQ + (((long long)b * Sq + pos) * Hq + hh) * D, dqacc, scale, g,
              ROPE ? tab + (long long)(off + pos) * (D / 2) : nullptr);
}

// ---------------------------------------------------------------- host --

namespace {

template <typename T, bool C, bool R, bool ONEBUF>
hipError_t go_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
                  int Skv, float scale, const double2* tab, float* ndelta, float* lse2,
                  hipStream_t stream) {
  const u16* Q = static_cast<const u16*>(q);
  const u16* Kp = static_cast<const u16*>(k);
  const u16* Vp = static_cast<const u16*>(v);
  const u16* dO = static_cast<const u16*>(dout);
  const float sl2 = scale * kLog2e;

  const long long nrows = (long long)B * Sq * Hq;
  const long long nprep = (nrows + 31) / 32;
  if (nprep > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  bwd_prep_kernel<T><<<dim3((unsigned)nprep), dim3(256), 0, stream>>>(
      static_cast<const u16*>(o), dO, lse, ndelta, lse2, B, Sq, Hq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_bh_kv = B * Hkv;
  const long long nkv = (long long)((Skv + 127) / 128) * n_bh_kv;
  if (nkv > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  bwd_dkdv_kernel<T, C, R, ONEBUF><<<dim3((unsigned)nkv), dim3(256), 0, stream>>>(
      Q, Kp, Vp, dO, lse2, ndelta, static_cast<u16*>(dk), static_cast<u16*>(dv), Hq, Hkv, Sq, Skv,
      scale, sl2, tab, n_bh_kv);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const int G = Hq / Hkv;
  auto dq_launch = [&](auto hpw_c) {
    constexpr int HPW = decltype(hpw_c)::value;
    constexpr int NP = 128 / HPW;
    const int n_qt = (Sq + NP - 1) / NP;
    const int n_bh = B * (Hq / HPW);
    const long long nb = (long long)n_qt * n_bh;
    if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    bwd_dq_kernel<T, HPW, C, R, ONEBUF><<<dim3((unsigned)nb), dim3(256), 0, stream>>>(
        Q, Kp, Vp, dO, lse2, ndelta, static_cast<u16*>(dq), Hq, Hkv, Sq, Skv, scale, sl2, tab,
        n_qt, n_bh);
    return hipGetLastError();
  };
  if (G % 4 == 0) return dq_launch(std::integral_constant<int, 4>{});
  if (G % 2 == 0) return dq_launch(std::integral_constant<int, 2>{});
  return dq_launch(std::integral_constant<int, 1>{});
}

}  // namespace

size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D, bool rope) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t n = 2 * up((size_t)B * Hq * Sq * sizeof(float));
  if (rope) n += up((size_t)B * Sq * Hq * D * 2) + up((size_t)B * Skv * Hkv * D * 2);
  return n;
}

hipError_t launch_bwd16(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                        const double2* rope_tab, int dtype, void* workspace, hipStream_t stream) {
  if (D != kD || (dtype != 1 && dtype != 2)) return hipErrorInvalidValue;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* ws = static_cast<char*>(workspace);
  float* ndelta = reinterpret_cast<float*>(ws);
  float* lse2 = reinterpret_cast<float*>(ws + up((size_t)B * Hq * Sq * sizeof(float)));
  const bool rope = rope_tab != nullptr;
  const void* qin = q;
  const void* kin = k;
  if (rope) {
    char* qs = ws + 2 * up((size_t)B * Hq * Sq * sizeof(float));
    char* ks = qs + up((size_t)B * Sq * Hq * D * 2);
    // one pass: queries at positions Skv - Sq + i, keys at j
    hipError_t e =
        launch_rope_rotate_qk(q, qs, B, Sq, Hq, k, ks, Skv, Hkv, D, rope_tab, dtype, stream);
    if (e != hipSuccess) return e;
    qin = qs;
    kin = ks;
  }
  const bool onebuf = lds_single_buffer_enabled();
#define XATTN_BWD_CASE(TT, C, R)                                                                 \
  if ((causal != 0) == C && rope == R)                                                           \
    return (onebuf ? go_bwd<TT, C, R, true> : go_bwd<TT, C, R, false>)(                          \
        qin, kin, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, scale, rope_tab, ndelta, lse2, \
        stream);
  if (dtype == 1) {
    XATTN_BWD_CASE(__bf16, false, false)
    XATTN_BWD_CASE(__bf16, true, false)
    XATTN_BWD_CASE(__bf16, false, true)
    XATTN_BWD_CASE(__bf16, true, true)
  } else {
    XATTN_BWD_CASE(_Float16, false, false)
    XATTN_BWD_CASE(_Float16, true, false)
    XATTN_BWD_CASE(_Float16, false, true)
    XATTN_BWD_CASE(_Float16, true, true)
  }
#undef XATTN_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace xattn
