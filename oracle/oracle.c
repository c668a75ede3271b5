/*
 * oracle.c — plain fp64 CPU oracle for the output-perturbation eviction score.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library. The product (libkvscore) never links,
 * loads or calls it, and this file includes nothing from the product.
 *
 * What it computes, following the pages:
 *   - DropKV page, "Methodology in Plain English" and Key Contribution 1: deleting
 *     token j from a softmax attention row moves the output a by
 *     p_j/(1-p_j) * (a - v_j) (the softmax renormalises over the survivors), and the
 *     per-token eviction score is p_j/(1-p_j) * ||a - v_j||_2, computed from the
 *     full (unevicted) cache.
 *   - Same section: in practice the per-token terms of the final w query rows are
 *     summed into one score per token. Its "squared" variant is offered as mode SQ:
 *     sum_i (p_ij/(1-p_ij))^2 * ||a_i - v_j||^2; mode L2 (the default) is
 *     sum_i p_ij/(1-p_ij) * ||a_i - v_j||_2.
 *   - Query heads that share a KV head (grouped-query attention) are summed into
 *     that KV head's score, as the PyramidKV page's aggregated window score sums
 *     over heads (its "Observation Window and Aggregated Attention Eviction").
 *   - Mode 2 is that aggregated window score itself: S_j = sum over the window rows
 *     and the group's heads of the attention weight p_ij (the SnapKV/PyramidKV
 *     ranking). Its isolated argmax term is the pair's weight p*.
 *
 * Everything is fp64. Inputs are bf16 bit patterns, converted exactly. Nothing is
 * blocked, fused or reordered beyond the definition: for one (sequence, layer,
 * KV head) unit the logits of every window row are materialised as a matrix, each
 * row's softmax statistics and output a_i are formed from it, and then every
 * score is a plain sum over rows of the per-pair term with the distance taken by
 * direct difference. The one exception is each row's argmax pair: there 1 - p can
 * round to 0 in fp64, so its term is taken from the definition itself (the output
 * recomputed without j*, over the survivors at their own scale) and not from the
 * closed form, which would divide by that rounded difference.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Problem description private to the oracle. Layouts (element strides):
 *   q : [L][S][Hq][W][d]                      contiguous
 *   k : k[l*ksl + g*ksh + t*kst + c]           t = global token index cu[s] + j
 *   v : v[l*vsl + g*vsh + t*vst + c]
 *   score : [L][Hkv][N]                        N = cu[S]
 *   a     : [L][S][Hq][W][d]
 *   lse, jstar, dom : [L][S][Hq][W]
 */
typedef struct {
  int32_t S, L, Hq, Hkv, d, W;
  const int64_t *cu; /* [S+1] */
  int64_t ksl, ksh, kst, vsl, vsh, vst;
  double scale; /* multiplies q.k */
  int32_t mode; /* 0 = L2, 1 = SQ, 2 = attention sum */
} oracle_shape;

static double bf16_to_double(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * One (s, l, g) unit. Rows r = hl*W + i (hl = head within the group, i = window
 * row). Row r is query head h = g*G + hl at position t_i = n - W + i, causal, so
 * it sees keys j = 0..t_i (the full cache up to itself).
 *
 * Outputs (any may be NULL): score_unit[n] (+=), a_rows[R][d], lse_rows[R],
 * jstar_rows[R], dom_rows[R] (the term of each row's argmax pair), pmax (max p).
 */
static int unit_eval(const oracle_shape *sh, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int s, int l, int g, double *score_unit, double *a_rows, double *lse_rows,
                     int32_t *jstar_rows, double *dom_rows, double *pmax_out) {
  const int d = sh->d, W = sh->W, G = sh->Hq / sh->Hkv, R = G * W;
  const int64_t n = sh->cu[s + 1] - sh->cu[s];
  const int64_t t0 = sh->cu[s];
  if (n <= W) return -1;

  /* fp64 copies of this unit's keys and values */
  double *K = (double *)malloc(sizeof(double) * (size_t)n * d);
  double *V = (double *)malloc(sizeof(double) * (size_t)n * d);
  double *Q = (double *)malloc(sizeof(double) * (size_t)R * d);
  double *S = (double *)malloc(sizeof(double) * (size_t)R * n); /* logits, materialised */
  double *A = (double *)malloc(sizeof(double) * (size_t)R * d);
  double *LSE = (double *)malloc(sizeof(double) * (size_t)R);
  double *TERM = (double *)malloc(sizeof(double) * (size_t)R);     /* each row's argmax-pair term */
  double *AM = (double *)malloc(sizeof(double) * (size_t)R * d);   /* a^(-j*) of each row */
  int32_t *JS = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);    /* each row's argmax j* */
  if (!K || !V || !Q || !S || !A || !LSE || !TERM || !AM || !JS) {
    free(K); free(V); free(Q); free(S); free(A); free(LSE); free(TERM); free(AM); free(JS);
    return -2;
  }
  for (int64_t j = 0; j < n; ++j) {
    const uint16_t *kr = k + l * sh->ksl + g * sh->ksh + (t0 + j) * sh->kst;
    const uint16_t *vr = v + l * sh->vsl + g * sh->vsh + (t0 + j) * sh->vst;
    for (int c = 0; c < d; ++c) {
      K[j * d + c] = bf16_to_double(kr[c]);
      V[j * d + c] = bf16_to_double(vr[c]);
    }
  }
  for (int hl = 0; hl < G; ++hl) {
    const int h = g * G + hl;
    const uint16_t *qb = q + ((((int64_t)l * sh->S + s) * sh->Hq + h) * W) * d;
    for (int i = 0; i < W; ++i)
      for (int c = 0; c < d; ++c) Q[(int64_t)(hl * W + i) * d + c] = bf16_to_double(qb[(int64_t)i * d + c]);
  }

  double pmax = 0.0;
  /* Row statistics: logits, max, softmax normaliser, output a. */
#pragma omp parallel for schedule(dynamic, 1) reduction(max : pmax)
  for (int r = 0; r < R; ++r) {
    const int i = r % W;
    const int64_t t = n - W + i; /* last visible key */
    double *srow = S + (int64_t)r * n;
    const double *qr = Q + (int64_t)r * d;
    double m = -INFINITY;
    int64_t jm = 0;
    for (int64_t j = 0; j <= t; ++j) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += qr[c] * K[j * d + c];
      srow[j] = acc * sh->scale;
      if (srow[j] > m) { m = srow[j]; jm = j; } /* strict: lowest index wins ties */
    }
    double lsum = 0.0;
    for (int64_t j = 0; j <= t; ++j) lsum += exp(srow[j] - m);
    const double lse = m + log(lsum);
    double *ar = A + (int64_t)r * d;
    for (int c = 0; c < d; ++c) ar[c] = 0.0;
    for (int64_t j = 0; j <= t; ++j) {
      const double p = exp(srow[j] - lse);
      for (int c = 0; c < d; ++c) ar[c] += p * V[j * d + c];
    }
    LSE[r] = lse;
    const double pm = exp(m - lse);
    if (pm > pmax) pmax = pm;
    JS[r] = (int32_t)jm;
  }

  /*
   * The argmax pair of each row, by the definition of removal (DropKV page, "Methodology
   * in Plain English"): drop j*, renormalise the softmax over the survivors and measure
   * ||a - a^(-j*)||. The survivors' weights are taken relative to their own max, so a^(-j*)
   * keeps full precision even where p* rounds to 1 in fp64 (the rest's total weight below
   * 2^-53); the closed form p/(1-p)*||a - v_j|| used for the other pairs divides by 1 - p*,
   * which cancels for this pair (every other pair has p <= 1/2). Row r sees keys 0..t with
   * t >= n - W >= 1, so at least one key survives.
   */
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < R; ++r) {
    const int64_t t = n - W + r % W;
    const int64_t js = JS[r];
    const double *srow = S + (int64_t)r * n;
    if (sh->mode == 2) { /* the argmax pair's attention weight p* */
      TERM[r] = exp(srow[js] - LSE[r]);
      continue;
    }
    double m2 = -INFINITY;
    for (int64_t j = 0; j <= t; ++j)
      if (j != js && srow[j] > m2) m2 = srow[j];
    double *am = AM + (int64_t)r * d;
    for (int c = 0; c < d; ++c) am[c] = 0.0;
    double lrest = 0.0;
    for (int64_t j = 0; j <= t; ++j) {
      if (j == js) continue;
      const double w = exp(srow[j] - m2);
      lrest += w;
      for (int c = 0; c < d; ++c) am[c] += w * V[j * d + c];
    }
    const double *ar = A + (int64_t)r * d;
    double dist2 = 0.0;
    for (int c = 0; c < d; ++c) {
      const double df = ar[c] - am[c] / lrest;
      dist2 += df * df;
    }
    const double shift = sqrt(dist2); /* ||a - a^(-j*)||_2 */
    TERM[r] = (sh->mode == 1) ? shift * shift : shift;
  }

  /* Per-pair term and the window/head sum, one output token j at a time. */
  if (score_unit) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int r = 0; r < R; ++r) {
        const int i = r % W;
        const int64_t t = n - W + i;
        if (j > t) continue; /* causal: row r never saw key j */
        if (j == JS[r]) { /* the row's argmax pair, by removal above */
          acc += TERM[r];
          continue;
        }
        const double x = S[(int64_t)r * n + j] - LSE[r];
        const double p = exp(x);
        if (sh->mode == 2) { /* attention sum (PyramidKV aggregated window score) */
          acc += p;
          continue;
        }
        const double one_minus_p = -expm1(x);
        const double c = p / one_minus_p;
        const double *ar = A + (int64_t)r * d;
        double dist2 = 0.0;
        for (int cc = 0; cc < d; ++cc) {
          const double df = ar[cc] - V[j * d + cc];
          dist2 += df * df;
        }
        const double shift = c * sqrt(dist2); /* ||a - a^(-j)||_2 */
        acc += (sh->mode == 1) ? shift * shift : shift;
      }
      score_unit[j] += acc;
    }
  }

  if (jstar_rows) memcpy(jstar_rows, JS, sizeof(int32_t) * (size_t)R);
  if (dom_rows) memcpy(dom_rows, TERM, sizeof(double) * (size_t)R);
  if (a_rows) memcpy(a_rows, A, sizeof(double) * (size_t)R * d);
  if (lse_rows) memcpy(lse_rows, LSE, sizeof(double) * (size_t)R);
  if (pmax_out) *pmax_out = pmax;

  free(K); free(V); free(Q); free(S); free(A); free(LSE); free(TERM); free(AM); free(JS);
  return 0;
}

/*
 * Evaluate a list of units u = (l*S + s)*Hkv + g (all units when units == NULL).
 *   score : [L][Hkv][N] doubles; each selected unit's n_s entries are overwritten.
 *   a, lse, jstar, dom : per-row outputs in the [L][S][Hq][W](x d) layout, or NULL.
 *   pmax : [n_units or all] max softmax probability per unit, or NULL.
 * Returns 0, or a negative code on a bad shape / allocation failure.
 */
int oracle_eval(const int32_t *dims /* S,L,Hq,Hkv,d,W,mode */, const int64_t *cu,
                const int64_t *kv_strides /* ksl,ksh,kst,vsl,vsh,vst */, double scale,
                const uint16_t *q, const uint16_t *k, const uint16_t *v,
                const int32_t *units, int32_t n_units,
                double *score, double *a, double *lse, int32_t *jstar, double *dom, double *pmax) {
  oracle_shape sh;
  sh.S = dims[0]; sh.L = dims[1]; sh.Hq = dims[2]; sh.Hkv = dims[3]; sh.d = dims[4]; sh.W = dims[5];
  sh.mode = dims[6];
  sh.cu = cu;
  sh.ksl = kv_strides[0]; sh.ksh = kv_strides[1]; sh.kst = kv_strides[2];
  sh.vsl = kv_strides[3]; sh.vsh = kv_strides[4]; sh.vst = kv_strides[5];
  sh.scale = scale;
  if (sh.Hkv <= 0 || sh.Hq % sh.Hkv != 0 || sh.d <= 0 || sh.W <= 0) return -1;
  const int G = sh.Hq / sh.Hkv, R = G * sh.W;
  const int64_t N = cu[sh.S];
  const int32_t total_units = sh.S * sh.L * sh.Hkv;
  const int32_t nu = units ? n_units : total_units;
  int32_t *jbuf = (int32_t *)malloc(sizeof(int32_t) * R);
  double *abuf = (double *)malloc(sizeof(double) * (size_t)R * sh.d);
  double *lbuf = (double *)malloc(sizeof(double) * R);
  double *dbuf = (double *)malloc(sizeof(double) * R);
  if (!jbuf || !abuf || !lbuf || !dbuf) { free(jbuf); free(abuf); free(lbuf); free(dbuf); return -2; }
  int rc = 0;
  for (int32_t ui = 0; ui < nu && rc == 0; ++ui) {
    const int32_t u = units ? units[ui] : ui;
    if (u < 0 || u >= total_units) { rc = -1; break; }
    const int g = u % sh.Hkv, s = (u / sh.Hkv) % sh.S, l = u / (sh.Hkv * sh.S);
    const int64_t n = cu[s + 1] - cu[s];
    double *su = NULL;
    if (score) {
      su = score + ((int64_t)l * sh.Hkv + g) * N + cu[s];
      for (int64_t j = 0; j < n; ++j) su[j] = 0.0;
    }
    double pm = 0.0;
    rc = unit_eval(&sh, q, k, v, s, l, g, su, abuf, lbuf, jbuf, dbuf, &pm);
    if (rc) break;
    if (pmax) pmax[ui] = pm;
    for (int hl = 0; hl < G; ++hl) {
      const int h = g * G + hl;
      for (int i = 0; i < sh.W; ++i) {
        const int r = hl * sh.W + i;
        const int64_t row = (((int64_t)l * sh.S + s) * sh.Hq + h) * sh.W + i;
        if (a) memcpy(a + row * sh.d, abuf + (int64_t)r * sh.d, sizeof(double) * sh.d);
        if (lse) lse[row] = lbuf[r];
        if (jstar) jstar[row] = jbuf[r];
        if (dom) dom[row] = dbuf[r];
      }
    }
  }
  free(jbuf); free(abuf); free(lbuf); free(dbuf);
  return rc;
}
