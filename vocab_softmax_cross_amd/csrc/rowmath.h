// Per-row scalar arithmetic shared by the forward and backward kernels: the
// row loss from (m, d', x[y], S) and the fp32 gradient coefficients,
// including the true-class element folded once from the live statistics.
#pragma once

#include "common.h"

namespace vsce {

// Row loss, Liger-Kernel PR #1622 (eps = label_smoothing / V times the
// class-weight sum) with the PyTorch reading of the smoothed, weighted loss:
//   l = (1 - eps) w_y ((m - x_y) + log1p(d')) + eta (sum_w (m + log1p(d')) - S)
// (m - x_y) + log1p(d') is lse - x_y without cancelling lse against x_y.
// lg = log1p(d') = lse - m, computed once per row by the caller.
__device__ inline float row_loss(float m, float lg, float xy, float S, float wy, float sum_w,
                                 float eps, float eta) {
  float l = (1.0f - eps) * wy * ((m - xy) + lg);
  if (eps > 0.0f) l += eta * (sum_w * (m + lg) - S);
  return l;
}

// z-loss of a valid row: lambda lse^2 with lse = m + log1p(d') (the z-loss
// Liger-Kernel PR #1268 lists among the features its CE suite covers;
// Correctness).  0 when lambda is 0.
__device__ inline float row_z(float m, float lg, float zl) {
  const float lse = m + lg;
  const float z = zl * lse * lse;
  return zl != 0.0f ? z : 0.0f;  // a select, not a branch: no second code path
}

// Gradient coefficients of one row, all in fp32:
//   g[c] = K * exp(x[c] - m) - B * w[c]  for c != y,   g[y] = dxy,
// with K = (sigma A + Z) / (1 + d'), A = (1 - eps) w_y + eta sum_w,
// B = sigma eta, and the z-loss term Z = sigma_z 2 lambda lse (0 without a
// z-loss; its gradient 2 lambda lse p[c] rides on the softmax term).
// dxy is evaluated once from the live m, d' and x_y (Liger-Kernel PR #1268,
// commit message of linkedin#1329): when x_y is the maximum, p_y - 1 is
// -d' / (1 + d') exactly, so nothing cancels as softmax(x_y) -> 1.
// Under soft-capping, m and x_y are capped values and the caller multiplies
// every g by the slope of the cap at its own stored logit.
struct RowTerms {
  float ML;   // m * log2(e)
  float K;
  float B;
  float dxy;
};

__device__ inline RowTerms row_terms(float m, float dp, float lg, float xy, float wy,
                                     float sum_w, float eps, float eta, float sigma,
                                     float zl = 0.0f, float sigma_z = 0.0f) {
  RowTerms t;
  const float inv_d = 1.0f / (1.0f + dp);
  const float A = (1.0f - eps) * wy + eta * sum_w;
  const float Zv = sigma_z * 2.0f * zl * (m + lg);
  const float Z = zl != 0.0f ? Zv : 0.0f;
  t.ML = m * kLog2e;
  t.K = (sigma * A + Z) * inv_d;
  t.B = sigma * eta;
  float py, py_m1;
  if (xy == m) {
    py = inv_d;
    py_m1 = -dp * inv_d;
  } else {
    py = exp_shifted(xy, t.ML) * inv_d;
    py_m1 = py - 1.0f;
  }
  t.dxy = sigma * (py_m1 * (1.0f - eps) * wy + eta * (sum_w * py - wy)) + Z * py;
  return t;
}

// Row class: ignored rows are tested first (ignore_index may lie in [0, V)).
enum RowClass { kValid = 0, kIgnored = 1, kInvalid = 2 };

__device__ inline int row_class(int64_t y, int64_t V, int64_t ignore_index) {
  if (y == ignore_index) return kIgnored;
  if (y < 0 || y >= V) return kInvalid;
  return kValid;
}

// Writes the per-row outputs of a forward kernel (one thread per row): the
// row loss (cross-entropy plus z-loss), its z-loss part and the accuracy.
template <class Args>
__device__ inline void store_row(const Args& a, int64_t n, float loss, float acc, float z = 0.0f) {
  a.loss_rows[n] = loss;
  if (a.loss_rows2) a.loss_rows2[n] = loss;
  if (a.acc_rows) a.acc_rows[n] = acc;
  if (a.z_rows) a.z_rows[n] = z;
}

// The z-loss's gradient scale: 1 / valid rows for mean, else 1.
template <class Args>
__device__ inline float z_sigma(const Args& a) {
  return a.mean ? a.ws->inv_n_valid : 1.0f;
}

}  // namespace vsce
