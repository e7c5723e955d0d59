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
__device__ inline float row_loss(float m, float dp, float xy, float S, float wy, float sum_w,
                                 float eps, float eta) {
  const float lg = log1pf(dp);
  float l = (1.0f - eps) * wy * ((m - xy) + lg);
  if (eps > 0.0f) l += eta * (sum_w * (m + lg) - S);
  return l;
}

// Gradient coefficients of one row, all in fp32:
//   g[c] = K * exp(x[c] - m) - B * w[c]  for c != y,   g[y] = dxy,
// with K = sigma A / (1 + d'), A = (1 - eps) w_y + eta sum_w, B = sigma eta.
// dxy is evaluated once from the live m, d' and x_y (Liger-Kernel PR #1268,
// commit message of linkedin#1329): when x_y is the maximum, p_y - 1 is
// -d' / (1 + d') exactly, so nothing cancels as softmax(x_y) -> 1.
struct RowTerms {
  float ML;   // m * log2(e)
  float K;
  float B;
  float dxy;
};

__device__ inline RowTerms row_terms(float m, float dp, float xy, float wy, float sum_w,
                                     float eps, float eta, float sigma) {
  RowTerms t;
  const float inv_d = 1.0f / (1.0f + dp);
  const float A = (1.0f - eps) * wy + eta * sum_w;
  t.ML = m * kLog2e;
  t.K = sigma * A * inv_d;
  t.B = sigma * eta;
  float py, py_m1;
  if (xy == m) {
    py = inv_d;
    py_m1 = -dp * inv_d;
  } else {
    py = exp_shifted(xy, t.ML) * inv_d;
    py_m1 = py - 1.0f;
  }
  t.dxy = sigma * (py_m1 * (1.0f - eps) * wy + eta * (sum_w * py - wy));
  return t;
}

// Row class: ignored rows are tested first (ignore_index may lie in [0, V)).
enum RowClass { kValid = 0, kIgnored = 1, kInvalid = 2 };

__device__ inline int row_class(int64_t y, int64_t V, int64_t ignore_index) {
  if (y == ignore_index) return kIgnored;
  if (y < 0 || y >= V) return kInvalid;
  return kValid;
}

// Writes the per-row outputs of a forward kernel (one thread per row).
template <class Args>
__device__ inline void store_row(const Args& a, int64_t n, float loss, float acc) {
  a.loss_rows[n] = loss;
  if (a.loss_rows2) a.loss_rows2[n] = loss;
  if (a.acc_rows) a.acc_rows[n] = acc;
}

}  // namespace vsce
