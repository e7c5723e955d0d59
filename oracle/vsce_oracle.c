/*
 * vsce_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU reference ("the oracle") for the large-vocabulary
 * softmax cross-entropy: per-row loss with ignore_index, class weights and
 * label smoothing, its reduction, the per-row statistics of the split mode,
 * the token accuracy, and the logits gradient rounded once to the buffer type.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this file.  It shares no code, header, table or constant with the HIP
 * library, and the library never calls it.
 *
 * Every function here is pinned by the CPU tests (tests/test_oracle.py)
 * against library routines, closed forms, invariants, brute force at 50
 * digits and the accuracy table printed on the pages; none is "parity
 * unpinned".
 *
 * Sources (page title, then the part of the page):
 *  [L1268]  Liger-Kernel PR #1268 "perf(ce): single-shot dx_y gradient
 *           correction": the review hunks of the pass-2 gradient
 *           (X_block += -eps, then -(1 - label_smoothing) at the target), and
 *           the embedded commit message of linkedin#1329 (fp32 dx_y fold).
 *  [L1622]  Liger-Kernel PR #1622 "perf(flce): drop host syncs that do not
 *           feed the computation", Summary: count and target-weight sum for
 *           "mean", class-weight sum times eps = label_smoothing / V,
 *           accuracy divided by the count.
 *  [TE2325] TransformerEngine PR #2325 "change fused cross entropy backward
 *           grad to fp32 and reduce one read/write", Greptile summary and
 *           sequence diagram: saved per-row (max, sum, target logit,
 *           scaled_x_sum).
 *
 * Where the pages give only fragments, the reading is that of PyTorch's
 * cross_entropy (the pages validate loss, gradients and accuracy against
 * PyTorch: [L1622] Testing Done).
 *
 * Logit soft-capping and the z-loss are named by [L1268] (What changed: the
 * target correction keeps the softcap factor; Correctness: the CE suite
 * covers softcap and z-loss) with no formula, so both take their plain
 * definitions: capped logits s * tanh(x / s) replace the logits everywhere
 * (s = 0: off), and a valid row adds lambda * lse^2 with lse taken over the
 * capped logits (lambda = 0: off).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC vsce_oracle.c -o liboracle.so -lm
 * (no -ffast-math: the arithmetic must be IEEE fp64 as written).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Row classes. */
#define ORACLE_VALID 0
#define ORACLE_IGNORED 1
#define ORACLE_INVALID 2

/* Buffer types the gradient is rounded to. */
#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F16 2

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of the later parallel loops (rows are independent, so the
 * results do not depend on it). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Round-to-nearest, ties-to-even, of an fp64 value to a binary format with
 * `p` significand bits (hidden bit included), minimum normal exponent `emin`
 * and maximum exponent `emax`; subnormals keep the quantum 2^(emin - p + 1);
 * values at or past the overflow threshold become infinities.  The result is
 * returned as an fp64 holding the rounded value exactly.
 *
 * The gradient element the buffer must hold is this rounding of the exact
 * (fp64) gradient: [L1268] linkedin#1329, "before the result is rounded to
 * the buffer dtype"; [TE2325] "grad_input (in original dtype)".
 */
static double round_to_format(double x, int p, int emin, int emax) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e;
  frexp(x, &e);          /* |x| = f * 2^e with f in [0.5, 1) */
  int lead = e - 1;      /* exponent of the leading bit */
  if (lead < emin) lead = emin;
  double quantum = ldexp(1.0, lead - (p - 1));
  double r = nearbyint(x / quantum) * quantum; /* default mode: ties-to-even */
  double max_finite = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
  if (fabs(r) > max_finite) r = copysign(INFINITY, x);
  return r;
}

double oracle_round_one(double x, int dtype) {
  switch (dtype) {
    case ORACLE_F32: return round_to_format(x, 24, -126, 127);
    case ORACLE_BF16: return round_to_format(x, 8, -126, 127);
    case ORACLE_F16: return round_to_format(x, 11, -14, 15);
    default: return NAN;
  }
}

void oracle_round(const double *in, double *out, int64_t n, int dtype) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = oracle_round_one(in[i], dtype);
}

/*
 * Row class ([L1268] "ignore_index" in the CE suite; [L1622] "non-ignored
 * count"): a row whose target equals ignore_index is ignored (tested first,
 * so an ignore_index inside [0, V) still ignores); a target outside [0, V)
 * that is not ignore_index is invalid; any other row is valid.
 */
static int row_class(int64_t y, int64_t V, int64_t ignore_index) {
  if (y == ignore_index) return ORACLE_IGNORED;
  if (y < 0 || y >= V) return ORACLE_INVALID;
  return ORACLE_VALID;
}

/*
 * Batch normalizers ([L1622] Summary, forward bullet): the number of valid
 * rows, the target-weight sum W = sum over valid rows of w[y] (the count when
 * there are no weights), the class-weight sum sum_c w[c] (V without weights)
 * that multiplies eps = label_smoothing / V, and the number of invalid rows.
 */
void oracle_normalizer(int64_t BT, const int64_t *target, int64_t V,
                       const double *weight, int64_t ignore_index,
                       int64_t *n_valid, double *W, double *sum_w,
                       int64_t *n_invalid) {
  int64_t nv = 0, ni = 0;
  double w_total = 0.0, sw = 0.0;
  for (int64_t n = 0; n < BT; ++n) {
    int cls = row_class(target[n], V, ignore_index);
    if (cls == ORACLE_VALID) {
      nv += 1;
      w_total += weight ? weight[target[n]] : 1.0;
    } else if (cls == ORACLE_INVALID) {
      ni += 1;
    }
  }
  for (int64_t c = 0; c < V; ++c) sw += weight ? weight[c] : 1.0;
  *n_valid = nv;
  *W = w_total;
  *sum_w = sw;
  *n_invalid = ni;
}

/*
 * Per-row forward and gradient, for `nrows` rows of `V` logits (x is
 * row-major with row stride V, the stored values upcast exactly).
 *
 * Soft-capping first: with softcap s > 0 every logit is replaced by
 *   xt[c] = s tanh(x[c] / s),   dxt[c]/dx[c] = 1 / cosh^2(x[c] / s)
 * (s = 0: xt = x, factor 1).  Everything below reads xt.
 *
 * For a valid row with target y, weights w (all ones when weight == NULL),
 * eps = label_smoothing and eta = eps / V:
 *   m    = max_c xt[c]; cstar = the first index attaining it
 *   d'   = sum over c != cstar of exp(xt[c] - m)          (d = 1 + d')
 *   lse  = m + log1p(d')
 *   ce   = (1 - eps) w[y] (lse - xt[y]) + eta * sum_c w[c] (lse - xt[c])
 *   z    = z_loss * lse^2
 *   loss = ce + z
 *   p[c] = exp(xt[c] - lse)
 * Every lse - xt[c] is evaluated as (m - xt[c]) + log1p(d'), the same
 * quantity without the cancellation of lse against xt[c] when the loss is
 * small.
 *   dce/dxt[c] = p[c] ((1 - eps) w[y] + eta sum_k w[k]) - eta w[c]
 *                - (1 - eps) w[y] [c == y]
 *   dz/dxt[c]  = 2 z_loss lse p[c]
 * The cross-entropy part is PyTorch's smoothed, weighted cross-entropy for
 * one row; its gradient has the structure of [L1268]'s pass 2 (softmax,
 * X_block += -eps, then -(1 - label_smoothing) at the target) with the class
 * weights of [L1622].
 *
 * The gradient written is, per row n,
 *   grad[c] = (scale_ce[n] dce/dxt[c] + scale_z[n] dz/dxt[c]) dxt[c]/dx[c]
 * (scale_ce / scale_z NULL: 1), so that a reduction may normalise the two
 * parts differently.
 *
 * Per-row statistics, as saved by the split forward ([TE2325] m_d_X_y):
 *   stats = (m, d', xt[y], S) with S = sum_c w[c] xt[c] when eps > 0, else 0.
 * The second slot holds d' = d - 1 rather than d (same information; d' keeps
 * its relative precision when one class dominates).
 *
 * Ignored rows: loss 0, gradient 0, stats 0.  Invalid rows: loss NaN,
 * gradient 0, stats 0.  argmax is the first index of the maximum of the
 * stored logits x (soft-capping is increasing, so it names the same class),
 * for every row.  row_z (may be NULL) receives z alone.
 *
 * `grad` may be NULL (no gradient wanted).
 */
void oracle_rows(int64_t nrows, int64_t V, const double *x,
                 const int64_t *target, const double *weight,
                 int64_t ignore_index, double label_smoothing, double softcap,
                 double z_loss, const double *scale_ce, const double *scale_z,
                 double *row_loss, double *row_z, double *stats, int64_t *argmax,
                 int32_t *cls_out, double *grad) {
  const double eps = label_smoothing;
  const double eta = eps / (double)V;
  double sum_w = 0.0;
  for (int64_t c = 0; c < V; ++c) sum_w += weight ? weight[c] : 1.0;

  int64_t n;
#pragma omp parallel
  {
    double *xt = (double *)malloc((size_t)V * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (n = 0; n < nrows; ++n) {
      const double *xr = x + n * V;
      double *gr = grad ? grad + n * V : NULL;
      const int64_t y = target[n];
      const int cls = row_class(y, V, ignore_index);
      cls_out[n] = cls;

      /* argmax of the stored logits, first index (NaN never compares greater) */
      double mx = -INFINITY;
      int64_t am = 0;
      for (int64_t c = 0; c < V; ++c) {
        if (xr[c] > mx) {
          mx = xr[c];
          am = c;
        }
      }
      argmax[n] = am;

      if (cls != ORACLE_VALID) {
        row_loss[n] = (cls == ORACLE_IGNORED) ? 0.0 : NAN;
        if (row_z) row_z[n] = (cls == ORACLE_IGNORED) ? 0.0 : NAN;
        for (int k = 0; k < 4; ++k) stats[4 * n + k] = 0.0;
        if (gr)
          for (int64_t c = 0; c < V; ++c) gr[c] = 0.0;
        continue;
      }

      for (int64_t c = 0; c < V; ++c)
        xt[c] = (softcap > 0.0) ? softcap * tanh(xr[c] / softcap) : xr[c];

      /* max of the (capped) logits and its first index */
      double m = -INFINITY;
      int64_t cstar = 0;
      for (int64_t c = 0; c < V; ++c) {
        if (xt[c] > m) {
          m = xt[c];
          cstar = c;
        }
      }

      double dprime = 0.0;
      for (int64_t c = 0; c < V; ++c)
        if (c != cstar) dprime += exp(xt[c] - m);
      /* a NaN anywhere in the row must reach the loss and the gradient (the
         max scan above never selects a NaN) */
      for (int64_t c = 0; c < V; ++c)
        if (isnan(xt[c])) dprime = NAN;
      const double lg = log1p(dprime); /* lse - m */
      const double lse = m + lg;

      const double wy = weight ? weight[y] : 1.0;
      double smooth = 0.0, S = 0.0;
      for (int64_t c = 0; c < V; ++c) {
        const double wc = weight ? weight[c] : 1.0;
        smooth += wc * ((m - xt[c]) + lg);
        S += wc * xt[c];
      }
      const double z = z_loss * lse * lse;
      row_loss[n] = (1.0 - eps) * wy * ((m - xt[y]) + lg) + eta * smooth + z;
      if (row_z) row_z[n] = z;

      stats[4 * n + 0] = m;
      stats[4 * n + 1] = dprime;
      stats[4 * n + 2] = xt[y];
      stats[4 * n + 3] = (eps > 0.0) ? S : 0.0;

      if (gr) {
        const double sc = scale_ce ? scale_ce[n] : 1.0;
        const double sz = scale_z ? scale_z[n] : 1.0;
        const double A = (1.0 - eps) * wy + eta * sum_w;
        for (int64_t c = 0; c < V; ++c) {
          const double wc = weight ? weight[c] : 1.0;
          const double p = exp((xt[c] - m) - lg);
          double g = p * A - eta * wc;
          if (c == y) g -= (1.0 - eps) * wy;
          g = sc * g + sz * (2.0 * z_loss * lse * p);
          if (softcap > 0.0) {
            const double ch = cosh(xr[c] / softcap);
            g /= ch * ch;
          }
          gr[c] = g;
        }
      }
    }
    free(xt);
  }
}

/*
 * Vocab-parallel statistics ([TE2325] Greptile summary: with a process group
 * of world_size > 1 each rank holds a slice of the vocabulary, and the per-row
 * m_d_X_y record -- max, sum, target logit and, under label smoothing,
 * scaled_x_sum as a 4th value -- is gathered from every rank; its review
 * comment asks that the 4th value be gathered and summed too).
 *
 * oracle_partials: the record of one shard holding columns [v0, v0 + Vs) of a
 * V-column vocabulary (x is the shard's [nrows, Vs] slice; targets and the
 * class weights are global, weight has V entries or is NULL).  Per valid row,
 * with xt the (soft-capped) logits of the shard:
 *   [0] m_s   = max over the shard of xt;  cs = the first column attaining it
 *   [1] d'_s  = sum over the shard's other columns of exp(xt[c] - m_s)
 *   [2] xt[y] if the shard holds column y, else 0
 *   [3] S_s   = sum over the shard of w[c] xt[c] (0 when eps == 0)
 *   [4] the maximum of the stored logits x over the shard
 *   [5] the global column of its first occurrence
 * Rows that are not valid get zeros.
 */
void oracle_partials(int64_t nrows, int64_t Vs, int64_t v0, int64_t V, const double *x,
                     const int64_t *target, const double *weight, int64_t ignore_index,
                     double label_smoothing, double softcap, double *part /* [nrows][6] */) {
  int64_t n;
#pragma omp parallel for schedule(dynamic, 1)
  for (n = 0; n < nrows; ++n) {
    const double *xr = x + n * Vs;
    double *pr = part + 6 * n;
    const int64_t y = target[n];
    for (int k = 0; k < 6; ++k) pr[k] = 0.0;
    if (row_class(y, V, ignore_index) != ORACLE_VALID) continue;
    double m = -INFINITY, mx = -INFINITY;
    int64_t cs = 0, am = 0;
    for (int64_t c = 0; c < Vs; ++c) {
      const double xt = (softcap > 0.0) ? softcap * tanh(xr[c] / softcap) : xr[c];
      if (xt > m) {
        m = xt;
        cs = c;
      }
      if (xr[c] > mx) {
        mx = xr[c];
        am = c;
      }
    }
    double dp = 0.0, S = 0.0;
    for (int64_t c = 0; c < Vs; ++c) {
      const double xt = (softcap > 0.0) ? softcap * tanh(xr[c] / softcap) : xr[c];
      if (c != cs) dp += exp(xt - m);
      S += (weight ? weight[v0 + c] : 1.0) * xt;
    }
    pr[0] = m;
    pr[1] = dp;
    if (y >= v0 && y < v0 + Vs)
      pr[2] = (softcap > 0.0) ? softcap * tanh(xr[y - v0] / softcap) : xr[y - v0];
    pr[3] = (label_smoothing > 0.0) ? S : 0.0;
    pr[4] = mx;
    pr[5] = (double)(v0 + am);
  }
}

/*
 * oracle_merge: the records of P shards (part[s] = [nrows][6], shards in
 * increasing column order) into the full row's statistics and argmax:
 *   m  = max_s m_s;  s* = the first shard attaining it
 *   d' = d'_{s*} + sum over s != s* of (1 + d'_s) exp(m_s - m)
 *   x[y] = sum_s of the shards' [2] (only the owner's is not 0)
 *   S  = sum_s S_s
 *   argmax = [5] of the first shard whose [4] attains the maximum of [4]
 * (the first column of the global maximum, as the unsharded row has it).
 * Rows that are not valid keep zeros.
 */
void oracle_merge(int64_t nrows, int64_t P, const double *part /* [P][nrows][6] */,
                  const int64_t *target, int64_t V, int64_t ignore_index,
                  double *stats /* [nrows][4] */, int64_t *argmax) {
  for (int64_t n = 0; n < nrows; ++n) {
    double *st = stats + 4 * n;
    for (int k = 0; k < 4; ++k) st[k] = 0.0;
    argmax[n] = 0;
    if (row_class(target[n], V, ignore_index) != ORACLE_VALID) continue;
    double m = -INFINITY, mx = -INFINITY;
    int64_t sstar = 0, sarg = 0;
    for (int64_t s = 0; s < P; ++s) {
      const double *pr = part + (s * nrows + n) * 6;
      if (pr[0] > m) {
        m = pr[0];
        sstar = s;
      }
      if (pr[4] > mx) {
        mx = pr[4];
        sarg = s;
      }
    }
    double dp = part[(sstar * nrows + n) * 6 + 1], xy = 0.0, S = 0.0;
    for (int64_t s = 0; s < P; ++s) {
      const double *pr = part + (s * nrows + n) * 6;
      if (s != sstar) dp += (1.0 + pr[1]) * exp(pr[0] - m);
      xy += pr[2];
      S += pr[3];
    }
    st[0] = m;
    st[1] = dp;
    st[2] = xy;
    st[3] = S;
    argmax[n] = (int64_t)part[(sarg * nrows + n) * 6 + 5];
  }
}
