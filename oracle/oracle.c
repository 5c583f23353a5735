/*
 * oracle.c — plain, slow fp64 CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file or the library built from it: only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library (no headers, helpers, tables or constants) and includes nothing from it.
 *
 * Sources (docs.rs source pages; each function names the item it follows):
 *   [FA]  scirs2-neural 0.4.3, src/layers/flash_attention.rs
 *   [GQA] scirs2-neural 0.4.4, src/layers/grouped_query_attention.rs
 *   [WH]  whisper-apr 0.3.1, src/model/attention_generated.rs
 *   [FD]  oxibonsai-model 0.1.4, src/layers/flash_decode.rs
 *   [LF]  whisper-apr 0.3.1, src/model/lfm2/gqa.rs
 *
 * Everything is computed in fp64.  Inputs may be given as fp64, fp32, bf16 or
 * IEEE binary16 (fp16) bit patterns; they are widened exactly to fp64 on access.  The score matrix of
 * every (batch, query head) is materialised in full before the softmax, as in the
 * naive path of [WH] (fn scaled_dot_product_attention of MultiHeadAttention) and
 * the scalar path of [LF] (fn attention_scalar).
 *
 * Readings of points the pages leave open (all listed in the design notes too):
 *  - causal masking is bottom-right aligned: key j is hidden from query row i iff
 *    j > i + (Skv - Sq).  For Sq == Skv this is the k_pos > q_pos rule of
 *    [FA] fn apply_causal_mask; the offset is the cached-generation rule of
 *    [GQA] fn forward_with_cache and [WH] fn forward_streaming.
 *  - a row with no visible key returns O = 0 and LSE = -inf ([FA] final
 *    rescale only when the row sum is positive; [FD] fn flash_decode_tile
 *    returns zeros and -inf for an all -inf tile).
 *  - LSE is the natural log-sum-exp of the scaled scores ([FD] fn flash_decode_tile).
 *  - query head h reads kv head h / (Hq / Hkv) ([GQA] forward loop, [LF] fn
 *    attention_scalar: kv_head = q_head / gqa_ratio).
 *  - RoPE is the interleaved pair rotation of [GQA] RotaryPositionEmbedding::apply
 *    with the angle pos / base^(2i/D) in fp64; queries sit at Skv - Sq + i, keys
 *    at j.  When the attention inputs are 16- or 32-bit, the rotated values are
 *    rounded to that format (nearest, ties to even) before the contraction,
 *    because that is the precision in which they enter the dot products.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F64 0
#define ORC_F32 1
#define ORC_BF16 2
#define ORC_F16 3

#ifdef ORACLE_MUTATION
/* Planted mistakes, compiled only by the mutation test: each one is a plausible
 * slip that at least one pin must catch. */
#define MUT ORACLE_MUTATION
#else
#define MUT 0
#endif

/* ---------------------------------------------------------------- inputs -- */

/* the input formats widen() reads; any other code is rejected by the entry points */
static int known_dtype(int dtype) {
  return dtype == ORC_F64 || dtype == ORC_F32 || dtype == ORC_BF16 || dtype == ORC_F16;
}

static double widen(const void* p, int dtype, size_t idx) {
  if (dtype == ORC_F64) return ((const double*)p)[idx];
  if (dtype == ORC_F32) return (double)((const float*)p)[idx];
  if (dtype == ORC_F16) {
    /* IEEE 754 binary16: sign, 5 exponent bits (bias 15), 10 fraction bits;
     * exponent 0 holds zero and the subnormals (fraction * 2^-24), exponent 31
     * infinities and NaNs */
    const uint16_t h = ((const uint16_t*)p)[idx];
    const int sgn = h >> 15, ex = (h >> 10) & 31, fr = h & 1023;
    double v;
    if (ex == 0)
      v = ldexp((double)fr, -24);
    else if (ex == 31)
      v = fr ? NAN : INFINITY;
    else
#if MUT == 13
      v = ldexp((double)(1024 + fr), ex - 24); /* planted: exponent bias 14 */
#else
      v = ldexp((double)(1024 + fr), ex - 25);
#endif
    return sgn ? -v : v;
  }
  /* bf16: the 16 stored bits are the top half of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t*)p)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Nearest value with `sig` significant bits, ties to even (sig = 8 for bf16,
 * 24 for binary32; 0 = keep fp64).  For bf16 and binary32 the exponent-range
 * limits are ignored: the values here are far from overflow and from their
 * subnormals.  sig = 11 is IEEE binary16, whose range is narrow enough to
 * matter: below 2^-14 (the subnormals) the spacing is fixed at 2^-24, and a
 * value that rounds to 2^16 or more (|x| >= 65520) becomes an infinity. */
double oracle_round_sig(double x, int sig) {
  if (sig <= 0 || x == 0.0 || !isfinite(x)) return x;
#if MUT != 14
  if (sig == 11 && fabs(x) < ldexp(1.0, -14))
    return ldexp(nearbyint(ldexp(x, 24)), -24);
#endif
  int e;
  double m = frexp(x, &e);            /* x = m * 2^e, 0.5 <= |m| < 1 */
  double r = nearbyint(ldexp(m, sig)); /* default rounding: nearest, ties even */
  double y = ldexp(r, e - sig);
  if (sig == 11 && fabs(y) > 65504.0) return x > 0 ? INFINITY : -INFINITY;
  return y;
}

/* ------------------------------------------------------------------ RoPE -- */

/* [GQA] RotaryPositionEmbedding::apply: for pair i, theta = pos / base^(2i/D);
 * x'_{2i} = x_{2i} cos - x_{2i+1} sin, x'_{2i+1} = x_{2i} sin + x_{2i+1} cos. */
static void rope_rotate(double* x, int D, double pos, double base) {
  for (int i = 0; i < D / 2; ++i) {
    double theta = pos / pow(base, 2.0 * i / (double)D);
#if MUT == 3
    theta = -theta; /* planted: rotation in the wrong direction */
#endif
    double c = cos(theta), s = sin(theta);
    double x0 = x[2 * i], x1 = x[2 * i + 1];
    x[2 * i] = x0 * c - x1 * s;
    x[2 * i + 1] = x0 * s + x1 * c;
  }
}

/* Standalone rotation of a [B,S,H,D] tensor at positions pos_offset + t
 * ([GQA] RotaryPositionEmbedding::apply with its position_offset argument). */
int oracle_rope(const void* x, int dtype, double* out, int B, int S, int H, int D,
                int pos_offset, double base, int round_bits) {
  if (D % 2 != 0) return -1; /* [GQA] RoPE head_dim must be even */
  if (!known_dtype(dtype)) return -1;
  double* row = (double*)malloc(sizeof(double) * (size_t)D);
  if (!row) return -2;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < S; ++t)
      for (int h = 0; h < H; ++h) {
        size_t base_idx = (((size_t)b * S + t) * H + h) * D;
        for (int d = 0; d < D; ++d) row[d] = widen(x, dtype, base_idx + d);
        rope_rotate(row, D, (double)(pos_offset + t), base);
        for (int d = 0; d < D; ++d) out[base_idx + d] = oracle_round_sig(row[d], round_bits);
      }
  free(row);
  return 0;
}

/* ------------------------------------------------------------- prefill -- */

typedef struct {
  const void *q, *k, *v;
  int dtype;
  int B, Hq, Hkv, Sq, Skv, D, causal;
  double scale, rope_base;
  int round_bits;
  const int* rows; /* query rows to evaluate (NULL: all) */
  int nrows;
  const int* units; /* b*Hq + h to evaluate (NULL: all) */
  int nunits;
  double *o, *lse; /* [nunits][nrows][D], [nunits][nrows] */
  const double* mask; /* additive, row (b, h, i) at b*mbs + h*mhs + i*Skv (NULL: none) */
  long long mbs, mhs;
  int nthreads, tid;
  int status;
} fwd_job;

/* One (batch, query head): the definition, written out.
 *   s_ij = scale * <q~_i, k~_j> + mask_ij,  s_ij = -inf where causally hidden,
 * (the additive mask of [WH] compute_block_scores / scaled_dot_product_attention,
 * added to the scaled score; 0 without a mask)
 *   m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i),
 *   O_i = sum_j exp(s_ij - m_i) v_j / l_i,  LSE_i = m_i + ln l_i. */
static int fwd_unit(const fwd_job* J, int u_slot, int unit) {
  const int D = J->D, Skv = J->Skv, Sq = J->Sq;
  const int b = unit / J->Hq, h = unit % J->Hq;
  const int group = J->Hq / J->Hkv;
#if MUT == 1
  const int g = h % J->Hkv; /* planted: interleaved instead of contiguous groups */
#else
  const int g = h / group;
#endif
  const int nrows = J->rows ? J->nrows : Sq;
  const int use_rope = J->rope_base > 0.0;

  double* kt = (double*)malloc(sizeof(double) * (size_t)Skv * D);
  double* vt = (double*)malloc(sizeof(double) * (size_t)Skv * D);
  double* qt = (double*)malloc(sizeof(double) * (size_t)D);
  double* S = (double*)malloc(sizeof(double) * (size_t)nrows * (Skv > 0 ? Skv : 1));
  if (!kt || !vt || !qt || !S) {
    free(kt); free(vt); free(qt); free(S);
    return -2;
  }
  for (int j = 0; j < Skv; ++j) {
    size_t base_idx = (((size_t)b * Skv + j) * J->Hkv + g) * D;
    for (int d = 0; d < D; ++d) {
      kt[(size_t)j * D + d] = widen(J->k, J->dtype, base_idx + d);
      vt[(size_t)j * D + d] = widen(J->v, J->dtype, base_idx + d);
    }
    if (use_rope) {
      rope_rotate(kt + (size_t)j * D, D, (double)j, J->rope_base);
      for (int d = 0; d < D; ++d)
        kt[(size_t)j * D + d] = oracle_round_sig(kt[(size_t)j * D + d], J->round_bits);
    }
  }
  /* full score matrix for the requested rows */
  for (int r = 0; r < nrows; ++r) {
    const int i = J->rows ? J->rows[r] : r;
    size_t qbase = (((size_t)b * Sq + i) * J->Hq + h) * D;
    for (int d = 0; d < D; ++d) qt[d] = widen(J->q, J->dtype, qbase + d);
    if (use_rope) {
      rope_rotate(qt, D, (double)(Skv - Sq + i), J->rope_base);
      for (int d = 0; d < D; ++d) qt[d] = oracle_round_sig(qt[d], J->round_bits);
    }
    for (int j = 0; j < Skv; ++j) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += qt[d] * kt[(size_t)j * D + d];
#if MUT == 5
      double s = dot; /* planted: scale dropped */
#else
      double s = J->scale * dot;
#endif
#if MUT == 11
      if (J->mask) s += J->scale * J->mask[(size_t)b * J->mbs + (size_t)h * J->mhs + (size_t)i * Skv + j];
#elif MUT == 12
      if (J->mask) s += J->mask[(size_t)b * J->mbs + (size_t)h * J->mhs + (size_t)j * Sq + i];
#else
      if (J->mask) s += J->mask[(size_t)b * J->mbs + (size_t)h * J->mhs + (size_t)i * Skv + j];
#endif
#if MUT == 2
      int hidden = J->causal && j > i; /* planted: top-left alignment */
#else
      int hidden = J->causal && j > i + (Skv - Sq);
#endif
      S[(size_t)r * Skv + j] = hidden ? -INFINITY : s;
    }
  }
  /* row softmax and weighted sum of V */
  for (int r = 0; r < nrows; ++r) {
    const double* srow = S + (size_t)r * Skv;
    double* orow = J->o + ((size_t)u_slot * nrows + r) * D;
    double m = -INFINITY;
    for (int j = 0; j < Skv; ++j)
      if (srow[j] > m) m = srow[j];
    if (m == -INFINITY) { /* no visible key */
      for (int d = 0; d < D; ++d) orow[d] = 0.0;
      J->lse[(size_t)u_slot * nrows + r] = -INFINITY;
      continue;
    }
    double l = 0.0;
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    for (int j = 0; j < Skv; ++j) {
      if (srow[j] == -INFINITY) continue;
      double p = exp(srow[j] - m);
      l += p;
#if MUT == 4
      const double* vj = kt + (size_t)j * D; /* planted: K used in place of V */
#else
      const double* vj = vt + (size_t)j * D;
#endif
      for (int d = 0; d < D; ++d) orow[d] += p * vj[d];
    }
    for (int d = 0; d < D; ++d) orow[d] /= l;
#if MUT == 6
    J->lse[(size_t)u_slot * nrows + r] = m + log2(l); /* planted: base-2 log */
#else
    J->lse[(size_t)u_slot * nrows + r] = m + log(l);
#endif
  }
  free(kt); free(vt); free(qt); free(S);
  return 0;
}

static void* fwd_worker(void* arg) {
  fwd_job* J = (fwd_job*)arg;
  const int nunits = J->units ? J->nunits : J->B * J->Hq;
  for (int s = J->tid; s < nunits; s += J->nthreads) {
    int unit = J->units ? J->units[s] : s;
    int st = fwd_unit(J, s, unit);
    if (st) { J->status = st; break; }
  }
  return NULL;
}

/* Attention over [B,Sq,Hq,D] queries and [B,Skv,Hkv,D] keys/values.  Outputs are
 * ordered by unit then row: o[u][r][d], lse[u][r].  `units` lists b*Hq + h and
 * `rows` lists query rows; NULL means all of them.  `mask` (NULL: none) is an
 * fp64 additive mask whose row for (b, h, i) starts at
 * b*mask_bstride + h*mask_hstride + i*Skv (a zero stride broadcasts).  Units are
 * spread over `nthreads` threads; each unit is computed by exactly one thread. */
int oracle_attn_fwd(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                    int Hkv, int Sq, int Skv, int D, int causal, double scale,
                    double rope_base, int round_bits, const int* rows, int nrows,
                    const int* units, int nunits, double* o, double* lse, const double* mask,
                    long long mask_bstride, long long mask_hstride, int nthreads) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1) return -1;
  if (Hq % Hkv != 0) return -1;
  if (rope_base > 0.0 && D % 2 != 0) return -1;
  if (!known_dtype(dtype)) return -1;
  if (nthreads < 1) nthreads = 1;
  fwd_job* jobs = (fwd_job*)calloc((size_t)nthreads, sizeof(fwd_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) { free(jobs); free(th); return -2; }
  for (int t = 0; t < nthreads; ++t) {
    fwd_job j = {q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, causal, scale, rope_base,
                 round_bits, rows, nrows, units, nunits, o, lse, mask, mask_bstride,
                 mask_hstride, nthreads, t, 0};
    jobs[t] = j;
  }
  int status = 0;
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fwd_worker, &jobs[t]);
  fwd_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status) status = jobs[t].status;
  free(jobs); free(th);
  return status;
}

/* -------------------------------------------------------------- decode -- */

typedef struct {
  const void *q, *kc, *vc;
  int dtype;
  const int* seqlens;
  int B, Hq, Hkv, D, Smax;
  double scale;
  const int* units;
  int nunits;
  double *o, *lse;
  int nthreads, tid;
} dec_job;

/* One query token per (batch, query head) against the first L_b cached
 * positions of a token-major [B,Smax,Hkv,D] cache, with no mask
 * ([LF] fn attention_cached; cache layout of [LF] KvCache and [FD]
 * fn flash_decode_multi_head).  Same definition as the prefill unit. */
static void dec_unit(const dec_job* J, int slot, int unit) {
  const int D = J->D, b = unit / J->Hq, h = unit % J->Hq;
  const int g = h / (J->Hq / J->Hkv);
  const int L = J->seqlens[b];
  double* orow = J->o + (size_t)slot * D;
  for (int d = 0; d < D; ++d) orow[d] = 0.0;
  if (L <= 0) {
    J->lse[slot] = -INFINITY;
    return;
  }
  double* s = (double*)malloc(sizeof(double) * (size_t)L);
  double m = -INFINITY;
  for (int j = 0; j < L; ++j) {
    size_t kb = (((size_t)b * J->Smax + j) * J->Hkv + g) * D;
    size_t qb = ((size_t)b * J->Hq + h) * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += widen(J->q, J->dtype, qb + d) * widen(J->kc, J->dtype, kb + d);
    s[j] = J->scale * dot;
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int j = 0; j < L; ++j) {
    size_t vb = (((size_t)b * J->Smax + j) * J->Hkv + g) * D;
    double p = exp(s[j] - m);
    l += p;
    for (int d = 0; d < D; ++d) orow[d] += p * widen(J->vc, J->dtype, vb + d);
  }
  for (int d = 0; d < D; ++d) orow[d] /= l;
  J->lse[slot] = m + log(l);
  free(s);
}

static void* dec_worker(void* arg) {
  dec_job* J = (dec_job*)arg;
  const int nunits = J->units ? J->nunits : J->B * J->Hq;
  for (int s = J->tid; s < nunits; s += J->nthreads) dec_unit(J, s, J->units ? J->units[s] : s);
  return NULL;
}

int oracle_decode(const void* q, const void* kc, const void* vc, int dtype, const int* seqlens,
                  int B, int Hq, int Hkv, int D, int Smax, double scale, const int* units,
                  int nunits, double* o, double* lse, int nthreads) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || Smax < 1 || Hq % Hkv != 0) return -1;
  if (!known_dtype(dtype)) return -1;
  for (int b = 0; b < B; ++b)
    if (seqlens[b] < 0 || seqlens[b] > Smax) return -1;
  if (nthreads < 1) nthreads = 1;
  dec_job* jobs = (dec_job*)calloc((size_t)nthreads, sizeof(dec_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) { free(jobs); free(th); return -2; }
  for (int t = 0; t < nthreads; ++t) {
    dec_job j = {q, kc, vc, dtype, seqlens, B, Hq, Hkv, D, Smax, scale, units, nunits,
                 o, lse, nthreads, t};
    jobs[t] = j;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, dec_worker, &jobs[t]);
  dec_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(jobs); free(th);
  return 0;
}

/* ------------------------------------------------------------ backward -- */

/* Rotation by the negated angle, R(pos)^T: the gradient of the pre-rotation
 * input from the gradient of the rotated one ([GQA] backward through grouped
 * attention: un-rotate by applying RoPE with the sine negated). */
static void rope_rotate_back(double* x, int D, double pos, double base) {
  for (int i = 0; i < D / 2; ++i) {
    const double theta = pos / pow(base, (2.0 * i) / (double)D);
    const double c = cos(theta), sn = sin(theta);
    const double x0 = x[2 * i], x1 = x[2 * i + 1];
    x[2 * i] = x0 * c + x1 * sn;
    x[2 * i + 1] = -x0 * sn + x1 * c;
  }
}

typedef struct {
  const void *q, *k, *v, *dout;
  int dtype;
  int B, Hq, Hkv, Sq, Skv, D, causal;
  double scale, rope_base;
  int round_bits;
  const int* units; /* b*Hkv + g to evaluate (NULL: all) */
  int nunits;
  double *dq, *dk, *dv; /* [B,Sq,Hq,D], [B,Skv,Hkv,D], [B,Skv,Hkv,D] */
  int nthreads, tid;
  int status;
} bwd_job;

/* One (batch, kv head g) with all the query heads of its group: the gradient of
 * O = softmax(S) V, S = scale Q~ K~^T (masked), written out from the full
 * matrices ([FA] fn flash_backward_head gives the same quantities per block;
 * [GQA] sums dK, dV over the query heads of a group):
 *   P = softmax(S) by rows,  dV_g += P^T dO,  dP = dO V^T,
 *   D_i = sum_j P_ij dP_ij  (= rowsum(dO o O) since O = P V),
 *   dS = P o (dP - D),  dQ~ = scale dS K~,  dK~_g += scale dS^T Q~,
 * then dQ = R^T dQ~ and dK = R^T dK~ when RoPE is on (R at the same positions
 * as in the forward).  A row with no visible key has P = 0 and contributes
 * nothing. */
static int bwd_unit(const bwd_job* J, int unit) {
  const int D = J->D, Skv = J->Skv, Sq = J->Sq, Hq = J->Hq, Hkv = J->Hkv;
  const int b = unit / Hkv, g = unit % Hkv;
  const int group = Hq / Hkv;
  const int use_rope = J->rope_base > 0.0;
  double* kt = (double*)malloc(sizeof(double) * (size_t)Skv * D);
  double* vt = (double*)malloc(sizeof(double) * (size_t)Skv * D);
  double* qt = (double*)malloc(sizeof(double) * (size_t)Sq * D);
  double* dot_ = (double*)malloc(sizeof(double) * (size_t)Sq * D);
  double* P = (double*)malloc(sizeof(double) * (size_t)Sq * Skv);
  double* dP = (double*)malloc(sizeof(double) * (size_t)Sq * Skv);
  double* dkt = (double*)calloc((size_t)Skv * D, sizeof(double));
  double* dvt = (double*)calloc((size_t)Skv * D, sizeof(double));
  double* dqt = (double*)malloc(sizeof(double) * (size_t)D);
  if (!kt || !vt || !qt || !dot_ || !P || !dP || !dkt || !dvt || !dqt) {
    free(kt); free(vt); free(qt); free(dot_); free(P); free(dP); free(dkt); free(dvt); free(dqt);
    return -2;
  }
  for (int j = 0; j < Skv; ++j) {
    const size_t base_idx = (((size_t)b * Skv + j) * Hkv + g) * D;
    for (int d = 0; d < D; ++d) {
      kt[(size_t)j * D + d] = widen(J->k, J->dtype, base_idx + d);
      vt[(size_t)j * D + d] = widen(J->v, J->dtype, base_idx + d);
    }
    if (use_rope) {
      rope_rotate(kt + (size_t)j * D, D, (double)j, J->rope_base);
      for (int d = 0; d < D; ++d)
        kt[(size_t)j * D + d] = oracle_round_sig(kt[(size_t)j * D + d], J->round_bits);
    }
  }
#if MUT == 10
  const int h_end = g * group + 1; /* planted: only the first query head of a group */
#else
  const int h_end = (g + 1) * group;
#endif
  for (int h = g * group; h < h_end; ++h) {
    for (int i = 0; i < Sq; ++i) {
      const size_t qbase = (((size_t)b * Sq + i) * Hq + h) * D;
      for (int d = 0; d < D; ++d) {
        qt[(size_t)i * D + d] = widen(J->q, J->dtype, qbase + d);
        dot_[(size_t)i * D + d] = widen(J->dout, J->dtype, qbase + d);
      }
      if (use_rope) {
        rope_rotate(qt + (size_t)i * D, D, (double)(Skv - Sq + i), J->rope_base);
        for (int d = 0; d < D; ++d)
          qt[(size_t)i * D + d] = oracle_round_sig(qt[(size_t)i * D + d], J->round_bits);
      }
    }
    /* P by rows (masked entries exactly 0), and dP = dO V^T */
    for (int i = 0; i < Sq; ++i) {
      double* prow = P + (size_t)i * Skv;
      double m = -INFINITY;
      for (int j = 0; j < Skv; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qt[(size_t)i * D + d] * kt[(size_t)j * D + d];
        const int hidden = J->causal && j > i + (Skv - Sq);
        prow[j] = hidden ? -INFINITY : J->scale * dot;
        if (prow[j] > m) m = prow[j];
      }
      double l = 0.0;
      for (int j = 0; j < Skv; ++j) {
        prow[j] = (m == -INFINITY || prow[j] == -INFINITY) ? 0.0 : exp(prow[j] - m);
        l += prow[j];
      }
      for (int j = 0; j < Skv; ++j) prow[j] = (l > 0.0) ? prow[j] / l : 0.0;
      for (int j = 0; j < Skv; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += dot_[(size_t)i * D + d] * vt[(size_t)j * D + d];
        dP[(size_t)i * Skv + j] = dot;
      }
    }
    /* dV += P^T dO */
    for (int j = 0; j < Skv; ++j)
      for (int i = 0; i < Sq; ++i) {
        const double pij = P[(size_t)i * Skv + j];
        if (pij == 0.0) continue;
        for (int d = 0; d < D; ++d) dvt[(size_t)j * D + d] += pij * dot_[(size_t)i * D + d];
      }
    /* dS = P o (dP - D) in place of dP; dQ~ = scale dS K~; dK~ += scale dS^T Q~ */
    for (int i = 0; i < Sq; ++i) {
      double Di = 0.0;
      for (int j = 0; j < Skv; ++j) Di += P[(size_t)i * Skv + j] * dP[(size_t)i * Skv + j];
      for (int j = 0; j < Skv; ++j) {
#if MUT == 7
        dP[(size_t)i * Skv + j] = P[(size_t)i * Skv + j] * dP[(size_t)i * Skv + j]; /* planted: D dropped */
#else
        dP[(size_t)i * Skv + j] = P[(size_t)i * Skv + j] * (dP[(size_t)i * Skv + j] - Di);
#endif
      }
      for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int j = 0; j < Skv; ++j) acc += dP[(size_t)i * Skv + j] * kt[(size_t)j * D + d];
        dqt[d] = J->scale * acc;
      }
#if MUT != 9
      if (use_rope) rope_rotate_back(dqt, D, (double)(Skv - Sq + i), J->rope_base);
#endif
      const size_t qbase = (((size_t)b * Sq + i) * Hq + h) * D;
      for (int d = 0; d < D; ++d) J->dq[qbase + d] = dqt[d];
    }
    for (int j = 0; j < Skv; ++j)
      for (int i = 0; i < Sq; ++i) {
        const double ds = dP[(size_t)i * Skv + j];
        if (ds == 0.0) continue;
#if MUT == 8
        const double sc = 1.0; /* planted: scale dropped from dK */
#else
        const double sc = J->scale;
#endif
        for (int d = 0; d < D; ++d) dkt[(size_t)j * D + d] += sc * ds * qt[(size_t)i * D + d];
      }
  }
  for (int j = 0; j < Skv; ++j) {
#if MUT != 9
    if (use_rope) rope_rotate_back(dkt + (size_t)j * D, D, (double)j, J->rope_base);
#endif
    const size_t base_idx = (((size_t)b * Skv + j) * Hkv + g) * D;
    for (int d = 0; d < D; ++d) {
      J->dk[base_idx + d] = dkt[(size_t)j * D + d];
      J->dv[base_idx + d] = dvt[(size_t)j * D + d];
    }
  }
  free(kt); free(vt); free(qt); free(dot_); free(P); free(dP); free(dkt); free(dvt); free(dqt);
  return 0;
}

static void* bwd_worker(void* arg) {
  bwd_job* J = (bwd_job*)arg;
  const int nunits = J->units ? J->nunits : J->B * J->Hkv;
  for (int s = J->tid; s < nunits; s += J->nthreads) {
    int st = bwd_unit(J, J->units ? J->units[s] : s);
    if (st) { J->status = st; break; }
  }
  return NULL;
}

/* Gradients of the attention of oracle_attn_fwd with respect to q, k and v for
 * an upstream gradient dout [B,Sq,Hq,D] (same dtype as q).  dq [B,Sq,Hq,D],
 * dk and dv [B,Skv,Hkv,D] are fp64 arrays owned by the caller; the slices of
 * the listed units (b*Hkv + g: a kv head with its query heads) are written,
 * the rest is left untouched.  Units are spread over `nthreads` threads. */
int oracle_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                    int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal, double scale,
                    double rope_base, int round_bits, const int* units, int nunits,
                    double* dq, double* dk, double* dv, int nthreads) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1) return -1;
  if (Hq % Hkv != 0) return -1;
  if (rope_base > 0.0 && D % 2 != 0) return -1;
  if (!known_dtype(dtype)) return -1;
  if (nthreads < 1) nthreads = 1;
  bwd_job* jobs = (bwd_job*)calloc((size_t)nthreads, sizeof(bwd_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) { free(jobs); free(th); return -2; }
  for (int t = 0; t < nthreads; ++t) {
    bwd_job j = {q, k, v, dout, dtype, B, Hq, Hkv, Sq, Skv, D, causal, scale, rope_base,
                 round_bits, units, nunits, dq, dk, dv, nthreads, t, 0};
    jobs[t] = j;
  }
  int status = 0;
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, bwd_worker, &jobs[t]);
  bwd_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status) status = jobs[t].status;
  free(jobs); free(th);
  return status;
}

/* ------------------------------------------- algorithms of the pages -- */

/* [FD] fn combine_tile_outputs: drop parts whose lse is not finite; none left
 * gives zeros (and lse -inf); one left is returned as is; otherwise
 * L = M + ln sum exp(lse_i - M) with M = max lse_i and O = sum exp(lse_i - L) O_i.
 * The page returns only O; the merged lse L is returned here as well. */
void oracle_lse_merge(const double* o_parts, const double* lse_parts, int n, int D, double* o,
                      double* lse) {
  int nvalid = 0, last = -1;
  double M = -INFINITY;
  for (int i = 0; i < n; ++i)
    if (isfinite(lse_parts[i])) {
      ++nvalid;
      last = i;
      if (lse_parts[i] > M) M = lse_parts[i];
    }
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (nvalid == 0) {
    *lse = -INFINITY;
    return;
  }
  if (nvalid == 1) {
    for (int d = 0; d < D; ++d) o[d] = o_parts[(size_t)last * D + d];
    *lse = lse_parts[last];
    return;
  }
  double sum = 0.0;
  for (int i = 0; i < n; ++i)
    if (isfinite(lse_parts[i])) sum += exp(lse_parts[i] - M);
  double L = M + log(sum);
  for (int i = 0; i < n; ++i) {
    if (!isfinite(lse_parts[i])) continue;
    double w = exp(lse_parts[i] - L);
    for (int d = 0; d < D; ++d) o[d] += w * o_parts[(size_t)i * D + d];
  }
  *lse = L;
}

/* [FD] fn flash_decode_tile: scores, m = max; an all -inf tile gives zeros and
 * -inf; w = exp(s - m), sum, lse = m + ln(sum), output = sum w v / sum. */
static void decode_tile(const double* q, const double* k, const double* v, int len, int D,
                        double scale, double* out, double* lse) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
  double m = -INFINITY;
  for (int t = 0; t < len; ++t) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q[d] * k[(size_t)t * D + d];
    s[t] = dot * scale;
    if (s[t] > m) m = s[t];
  }
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (!isfinite(m)) {
    *lse = -INFINITY;
    free(s);
    return;
  }
  double sum = 0.0;
  for (int t = 0; t < len; ++t) {
    s[t] = exp(s[t] - m);
    sum += s[t];
  }
  for (int t = 0; t < len; ++t)
    for (int d = 0; d < D; ++d) out[d] += s[t] * v[(size_t)t * D + d];
  if (sum > 0.0)
    for (int d = 0; d < D; ++d) out[d] /= sum;
  *lse = m + log(sum);
  free(s);
}

/* [FD] fn flash_decode_single_head: num_tiles clamped to [1, S]; tile length
 * floor(S / n) plus one for the first S mod n tiles; tile outputs merged by
 * fn combine_tile_outputs.  q [D], k and v [S][D]. */
int oracle_flash_decode_head(const double* q, const double* k, const double* v, int S, int D,
                             int num_tiles, double scale, double* o, double* lse) {
  if (S <= 0) return -4; /* [FD] FlashDecodeError::EmptyKv */
  int n = num_tiles < S ? num_tiles : S;
  if (n < 1) n = 1;
  double* parts = (double*)malloc(sizeof(double) * (size_t)n * D);
  double* lses = (double*)malloc(sizeof(double) * (size_t)n);
  int base = S / n, rem = S % n, off = 0, used = 0;
  for (int t = 0; t < n; ++t) {
    int len = base + (t < rem ? 1 : 0);
    if (len == 0) break;
    decode_tile(q, k + (size_t)off * D, v + (size_t)off * D, len, D, scale,
                parts + (size_t)used * D, &lses[used]);
    ++used;
    off += len;
  }
  oracle_lse_merge(parts, lses, used, D, o, lse);
  free(parts); free(lses);
  return 0;
}

/* [FA] fn flash_attention_forward with fn compute_block_scores,
 * fn apply_causal_mask and fn online_softmax_update, for one head in fp64:
 * query blocks outside, key/value blocks inside (block sizes clamped to
 * [1, S]); a key block wholly after the last query of the block is skipped
 * under the causal mask; per row the running max m and sum l are updated with
 * the correction exp(m_old - m_new) (zero while m_old is -inf); scores of -inf
 * are skipped; finally O /= l where l > 0.  Mask offset Skv - Sq as in the
 * definition above.  Also returns LSE = m + ln l (-inf where l = 0). */
int oracle_attn_tiled_head(const double* q, const double* k, const double* v, int Sq, int Skv,
                           int D, int causal, double scale, int block_q, int block_kv,
                           double* o, double* lse) {
  if (Sq < 1 || Skv < 1 || D < 1) return -1;
  int bq = block_q < Sq ? block_q : Sq;
  if (bq < 1) bq = 1;
  int bk = block_kv < Skv ? block_kv : Skv;
  if (bk < 1) bk = 1;
  const int off = Skv - Sq;
  double* m = (double*)malloc(sizeof(double) * (size_t)Sq);
  double* l = (double*)malloc(sizeof(double) * (size_t)Sq);
  double* sc = (double*)malloc(sizeof(double) * (size_t)bq * bk);
  for (int i = 0; i < Sq; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.0;
    for (int d = 0; d < D; ++d) o[(size_t)i * D + d] = 0.0;
  }
  for (int q0 = 0; q0 < Sq; q0 += bq) {
    int q1 = q0 + bq < Sq ? q0 + bq : Sq;
    for (int k0 = 0; k0 < Skv; k0 += bk) {
      int k1 = k0 + bk < Skv ? k0 + bk : Skv;
      if (causal && k0 > q1 - 1 + off) continue;
      for (int i = q0; i < q1; ++i)
        for (int j = k0; j < k1; ++j) {
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += q[(size_t)i * D + d] * k[(size_t)j * D + d];
          double s = dot * scale;
          if (causal && j > i + off) s = -INFINITY;
          sc[(size_t)(i - q0) * bk + (j - k0)] = s;
        }
      for (int i = q0; i < q1; ++i) {
        const double* row = sc + (size_t)(i - q0) * bk;
        double bmax = -INFINITY;
        for (int j = 0; j < k1 - k0; ++j)
          if (row[j] > bmax) bmax = row[j];
        double mnew = m[i] > bmax ? m[i] : bmax;
        double corr = (m[i] == -INFINITY) ? 0.0 : exp(m[i] - mnew);
        for (int d = 0; d < D; ++d) o[(size_t)i * D + d] *= corr;
        l[i] *= corr;
        for (int j = 0; j < k1 - k0; ++j) {
          if (row[j] == -INFINITY) continue;
          double p = exp(row[j] - mnew);
          l[i] += p;
          for (int d = 0; d < D; ++d) o[(size_t)i * D + d] += p * v[(size_t)(k0 + j) * D + d];
        }
        m[i] = mnew;
      }
    }
  }
  for (int i = 0; i < Sq; ++i) {
    if (l[i] > 0.0) {
      for (int d = 0; d < D; ++d) o[(size_t)i * D + d] /= l[i];
      lse[i] = m[i] + log(l[i]);
    } else {
      lse[i] = -INFINITY;
    }
  }
  free(m); free(l); free(sc);
  return 0;
}
