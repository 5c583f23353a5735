/*
 * oracle_check.c — driver for the AddressSanitizer / UndefinedBehaviorSanitizer
 * build of the fp64 oracle (test infrastructure).  It calls every exported
 * oracle function on small inputs in each input format, with and without
 * causal masking, RoPE, a mask, row and unit subsets and several threads, plus
 * rejected arguments, and checks only that results are finite where they must
 * be: the numbers themselves are pinned by the Python tests; this run is for
 * out-of-bounds accesses, leaks and undefined behaviour in the C code.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_round_sig(double x, int sig);
int oracle_rope(const void* x, int dtype, double* out, int B, int S, int H, int D, int pos_offset,
                double base, int round_bits);
int oracle_attn_fwd(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv,
                    int Sq, int Skv, int D, int causal, double scale, double rope_base,
                    int round_bits, const int* rows, int nrows, const int* units, int nunits,
                    double* o, double* lse, const double* mask, long long mask_bstride,
                    long long mask_hstride, int nthreads);
int oracle_decode(const void* q, const void* kc, const void* vc, int dtype, const int* seqlens,
                  int B, int Hq, int Hkv, int D, int Smax, double scale, const int* units,
                  int nunits, double* o, double* lse, int nthreads);
int oracle_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                    int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal, double scale,
                    double rope_base, int round_bits, const int* units, int nunits, double* dq,
                    double* dk, double* dv, int nthreads);
void oracle_lse_merge(const double* o_parts, const double* lse_parts, int n, int D, double* o,
                      double* lse);
int oracle_flash_decode_head(const double* q, const double* k, const double* v, int S, int D,
                             int num_tiles, double scale, double* o, double* lse);
int oracle_attn_tiled_head(const double* q, const double* k, const double* v, int Sq, int Skv,
                           int D, int causal, double scale, int block_q, int block_kv, double* o,
                           double* lse);

static int bad = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c);    \
      ++bad;                                                  \
    }                                                         \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

/* n values in format dt (0 fp64, 1 fp32, 2 bf16 bits, 3 fp16 bits), exact
 * small dyadic values so every format holds them */
static void* fill(int dt, size_t n) {
  size_t es = dt == 0 ? 8 : dt == 1 ? 4 : 2;
  void* p = malloc(n * es);
  for (size_t i = 0; i < n; ++i) {
    double x = floor(urand() * 64.0) / 32.0; /* multiples of 1/32 in [-2, 2) */
    if (dt == 0) ((double*)p)[i] = x;
    else if (dt == 1) ((float*)p)[i] = (float)x;
    else if (dt == 2) {
      float f = (float)x;
      uint32_t u;
      memcpy(&u, &f, 4);
      ((uint16_t*)p)[i] = (uint16_t)(u >> 16);
    } else {
      /* binary16 of a multiple of 1/32 with |x| < 2: sign, exponent, 10-bit fraction */
      uint16_t h = 0;
      double a = fabs(x);
      if (a > 0) {
        int e;
        double m = frexp(a, &e); /* a = m 2^e, m in [0.5, 1) */
        h = (uint16_t)(((e - 1 + 15) << 10) | ((uint16_t)((m * 2.0 - 1.0) * 1024.0) & 0x3ff));
      }
      if (x < 0) h |= 0x8000;
      ((uint16_t*)p)[i] = h;
    }
  }
  return p;
}

static int all_finite(const double* x, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

int main(void) {
  const int rb[4] = {0, 24, 8, 11};
  for (int dt = 0; dt < 4; ++dt) {
    const int B = 2, Hq = 4, Hkv = 2, Sq = 5, Skv = 7, D = 6;
    void* q = fill(dt, (size_t)B * Sq * Hq * D);
    void* k = fill(dt, (size_t)B * Skv * Hkv * D);
    void* v = fill(dt, (size_t)B * Skv * Hkv * D);
    void* dout = fill(dt, (size_t)B * Sq * Hq * D);
    double* o = malloc(sizeof(double) * B * Hq * Sq * D);
    double* lse = malloc(sizeof(double) * B * Hq * Sq);
    for (int causal = 0; causal < 2; ++causal)
      for (int rope = 0; rope < 2; ++rope)
        for (int th = 1; th <= 3; th += 2) {
          CHECK(oracle_attn_fwd(q, k, v, dt, B, Hq, Hkv, Sq, Skv, D, causal, 0.4,
                                rope ? 10000.0 : 0.0, rb[dt], NULL, 0, NULL, 0, o, lse, NULL, 0, 0,
                                th) == 0);
          CHECK(all_finite(o, (size_t)B * Hq * Sq * D) && all_finite(lse, (size_t)B * Hq * Sq));
        }
    /* row and unit subsets, an additive mask per (batch, head) */
    const int rows[3] = {0, 2, 4}, units[2] = {1, 6};
    double* mask = malloc(sizeof(double) * B * Hq * Sq * Skv);
    for (int i = 0; i < B * Hq * Sq * Skv; ++i) mask[i] = (i % 5 == 0) ? -INFINITY : urand();
    CHECK(oracle_attn_fwd(q, k, v, dt, B, Hq, Hkv, Sq, Skv, D, 1, 0.4, 500.0, rb[dt], rows, 3,
                          units, 2, o, lse, mask, (long long)Hq * Sq * Skv,
                          (long long)Sq * Skv, 2) == 0);
    /* Sq > Skv, causal: leading rows see no key (O = 0, LSE = -inf) */
    CHECK(oracle_attn_fwd(q, k, v, dt, 1, Hq, Hkv, Sq, 3, D, 1, 0.4, 0.0, rb[dt], NULL, 0, NULL, 0,
                          o, lse, NULL, 0, 0, 1) == 0);
    CHECK(isinf(lse[0]) && lse[0] < 0 && o[0] == 0.0);
    /* rejected arguments return nonzero without touching memory */
    CHECK(oracle_attn_fwd(q, k, v, dt, B, 3, 2, Sq, Skv, D, 0, 0.4, 0.0, rb[dt], NULL, 0, NULL, 0, o,
                          lse, NULL, 0, 0, 1) != 0);
    CHECK(oracle_attn_fwd(q, k, v, 9, B, Hq, Hkv, Sq, Skv, D, 0, 0.4, 0.0, rb[dt], NULL, 0, NULL,
                          0, o, lse, NULL, 0, 0, 1) != 0);
    /* gradients, all units and a subset */
    double* dq = malloc(sizeof(double) * B * Sq * Hq * D);
    double* dk = malloc(sizeof(double) * B * Skv * Hkv * D);
    double* dv = malloc(sizeof(double) * B * Skv * Hkv * D);
    for (int rope = 0; rope < 2; ++rope) {
      CHECK(oracle_attn_bwd(q, k, v, dout, dt, B, Hq, Hkv, Sq, Skv, D, 1, 0.4,
                            rope ? 10000.0 : 0.0, rb[dt], NULL, 0, dq, dk, dv, 3) == 0);
      CHECK(all_finite(dq, (size_t)B * Sq * Hq * D) && all_finite(dk, (size_t)B * Skv * Hkv * D));
    }
    const int bunit[1] = {3};
    CHECK(oracle_attn_bwd(q, k, v, dout, dt, B, Hq, Hkv, Sq, Skv, D, 0, 0.4, 0.0, rb[dt], bunit, 1,
                          dq, dk, dv, 1) == 0);
    /* rotary embedding at an offset */
    double* r = malloc(sizeof(double) * B * Sq * Hq * D);
    CHECK(oracle_rope(q, dt, r, B, Sq, Hq, D, 17, 10000.0, rb[dt]) == 0);
    CHECK(all_finite(r, (size_t)B * Sq * Hq * D));
    CHECK(oracle_rope(q, dt, r, B, Sq, Hq, 5, 0, 10000.0, rb[dt]) != 0); /* odd head dim */
    CHECK(oracle_rope(q, 7, r, B, Sq, Hq, D, 0, 10000.0, rb[dt]) != 0);  /* unknown format */
    /* decode against a cache of capacity 9 with lengths 0, 4 and 9 */
    {
      const int Bd = 3, Smax = 9;
      void* qd = fill(dt, (size_t)Bd * Hq * D);
      void* kc = fill(dt, (size_t)Bd * Smax * Hkv * D);
      void* vc = fill(dt, (size_t)Bd * Smax * Hkv * D);
      const int lens[3] = {0, 4, 9}, dunits[2] = {0, 11};
      double* od = malloc(sizeof(double) * Bd * Hq * D);
      double* ld = malloc(sizeof(double) * Bd * Hq);
      CHECK(oracle_decode(qd, kc, vc, dt, lens, Bd, Hq, Hkv, D, Smax, 0.4, NULL, 0, od, ld, 2) == 0);
      CHECK(isinf(ld[0]) && all_finite(od, (size_t)Bd * Hq * D));
      CHECK(oracle_decode(qd, kc, vc, dt, lens, Bd, Hq, Hkv, D, Smax, 0.4, dunits, 2, od, ld, 1) ==
            0);
      free(qd), free(kc), free(vc), free(od), free(ld);
    }
    free(q), free(k), free(v), free(dout), free(o), free(lse), free(mask), free(dq), free(dk),
        free(dv), free(r);
  }
  /* fp64-only helpers: tiled forward, flash-decode head, LSE merge */
  {
    const int S = 9, D = 4;
    double *q = fill(0, (size_t)S * D), *k = fill(0, (size_t)S * D), *v = fill(0, (size_t)S * D);
    double o[9 * 4], lse[9];
    for (int bs = 1; bs <= S + 1; ++bs) {
      CHECK(oracle_attn_tiled_head(q, k, v, S, S, D, bs & 1, 0.5, bs, S + 1 - bs, o, lse) == 0);
      CHECK(all_finite(o, (size_t)S * D));
    }
    for (int nt = 1; nt <= S + 2; ++nt) {
      CHECK(oracle_flash_decode_head(q, k, v, S, D, nt, 0.5, o, lse) == 0);
      CHECK(all_finite(o, (size_t)D));
    }
    double parts[3 * 4], lparts[3] = {0.5, -INFINITY, 1.5};
    for (int i = 0; i < 12; ++i) parts[i] = urand();
    oracle_lse_merge(parts, lparts, 3, D, o, lse);
    CHECK(all_finite(o, (size_t)D) && isfinite(lse[0]));
    free(q), free(k), free(v);
  }
  for (int i = 0; i < 1000; ++i) {
    double x = ldexp(urand(), (i % 80) - 40);
    CHECK(isfinite(oracle_round_sig(x, 8)) && isfinite(oracle_round_sig(x, 24)));
    /* binary16 overflows to an infinity from 65520 on */
    CHECK(isfinite(oracle_round_sig(x, 11)) == (fabs(x) < 65520.0));
  }
  printf("oracle sanitizer driver: %s\n", bad ? "FAILED" : "ok");
  return bad != 0;
}
