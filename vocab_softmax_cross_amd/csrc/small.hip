// The two single-workgroup kernels around each forward:
//
//  prologue_kernel  the batch normalizers on the device (Liger-Kernel PR
//                   #1622, Summary: the non-ignored count and target-weight
//                   sum that "mean" divides by, the class-weight sum that eps
//                   multiplies; its Details note that avoiding the host sync
//                   needs the count passed to the kernel as a device pointer,
//                   which is what this header in the workspace is), plus the
//                   bad-target status bit and the fp32 reciprocals of W and of
//                   the valid count that the row kernels scale by.
//  finalize_kernel  the none / sum / mean reduction of the per-row losses (a
//                   mean divides the cross-entropy part by W and the z-loss
//                   part by the valid-row count) and the accuracy mean
//                   (accuracy divided by the count on the device, same
//                   Summary).
//
// Both sum in fp64 in a fixed order (per-thread strided partial sums, then a
// fixed tree), so results do not depend on scheduling and need no atomics.
#include "common.h"
#include "launch.h"
#include "rowmath.h"

namespace vsce {
namespace {

constexpr int kSmallNT = 1024;

// Fixed-order workgroup sum of doubles; every thread gets the result.
__device__ inline double block_sum_d(double v, double* sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  __syncthreads();  // `sh` may still be read by a previous call
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < kSmallNT / kWave; ++w) r += sh[w];
  return r;
}

__global__ __launch_bounds__(kSmallNT) void prologue_kernel(const int64_t* target, int64_t rows,
                                                           int64_t V, const float* weight,
                                                           int64_t ignore_index, WsHeader* ws) {
  __shared__ double sh[kSmallNT / kWave];
  double W = 0.0, nv = 0.0, ni = 0.0, sw = 0.0;
  // Unrolled so that several independent target loads are in flight.
#pragma unroll 8
  for (int64_t n = threadIdx.x; n < rows; n += kSmallNT) {
    const int64_t y = target[n];
    const int cls = row_class(y, V, ignore_index);
    if (cls == kValid) {
      nv += 1.0;
      W += weight ? static_cast<double>(weight[y]) : 1.0;
    } else if (cls == kInvalid) {
      ni += 1.0;
    }
  }
  if (weight) {
#pragma unroll 8
    for (int64_t c = threadIdx.x; c < V; c += kSmallNT) sw += static_cast<double>(weight[c]);
  }
  W = block_sum_d(W, sh);
  nv = block_sum_d(nv, sh);
  ni = block_sum_d(ni, sh);
  sw = weight ? block_sum_d(sw, sh) : static_cast<double>(V);
  if (threadIdx.x == 0) {
    ws->W = W;
    ws->sum_w = sw;
    ws->n_valid = static_cast<int64_t>(nv);
    ws->n_invalid = static_cast<int64_t>(ni);
    ws->status = (ni > 0.0) ? VSCE_STATUS_BAD_TARGET : 0u;
    ws->pad0 = 0u;
    // The row kernels' gradient scales, rounded once here rather than
    // divided in every workgroup.
    ws->inv_W = static_cast<float>(1.0 / W);
    ws->inv_n_valid = static_cast<float>(1.0 / nv);
  }
}

__global__ __launch_bounds__(kSmallNT) void finalize_kernel(const float* loss_rows,
                                                           const float* acc_rows,
                                                           const float* z_rows, int64_t rows,
                                                           int red, float* loss_out,
                                                           float* acc_mean_out, float* z_out,
                                                           const WsHeader* ws) {
  __shared__ double sh[kSmallNT / kWave];
  if (red != VSCE_REDUCTION_NONE) {
    double t = 0.0, z = 0.0;
#pragma unroll 8
    for (int64_t n = threadIdx.x; n < rows; n += kSmallNT) {
      t += static_cast<double>(loss_rows[n]);
      if (z_rows) z += static_cast<double>(z_rows[n]);
    }
    t = block_sum_d(t, sh);
    if (z_rows) z = block_sum_d(z, sh);
    if (threadIdx.x == 0) {
      if (red == VSCE_REDUCTION_MEAN) {
        // Cross-entropy over W, z-loss over the valid rows (they differ only
        // with class weights).
        const double W = ws->W;
        const double nv = static_cast<double>(ws->n_valid);
        const double ce = W != 0.0 ? (t - z) / W : __builtin_nan("");
        const double zm = nv != 0.0 ? z / nv : __builtin_nan("");
        loss_out[0] = static_cast<float>(z_rows ? ce + zm : ce);
        if (z_out) z_out[0] = static_cast<float>(z_rows ? zm : 0.0);
      } else {
        loss_out[0] = static_cast<float>(t);
        if (z_out) z_out[0] = static_cast<float>(z_rows ? z : 0.0);
      }
    }
  }
  if (acc_mean_out) {
    double h = 0.0;
#pragma unroll 8
    for (int64_t n = threadIdx.x; n < rows; n += kSmallNT) h += static_cast<double>(acc_rows[n]);
    h = block_sum_d(h, sh);
    if (threadIdx.x == 0) {
      const double nv = static_cast<double>(ws->n_valid);
      acc_mean_out[0] = static_cast<float>(nv != 0.0 ? h / nv : __builtin_nan(""));
    }
  }
}

// The merge of vocab-parallel shard records (TransformerEngine PR #2325: the
// per-row max, sum, target logit and scaled_x_sum gathered from every rank,
// the 4th value summed as its review asks), one thread per row:
//   m = max_s m_s, s* the first shard attaining it,
//   d' = d'_{s*} + sum over s != s* of (1 + d'_s) exp(m_s - m)
// (the shard that holds the first maximum keeps its exact d'; the others
// bring their maximum back as the 1), x[y] from its owner (the others hold
// 0), S summed, and the argmax of the stored logits from [4] and [5].  Then
// the row loss, z-loss and accuracy as the statistics kernel computes them.
constexpr int kMergeNT = 256;

__global__ __launch_bounds__(kMergeNT) void merge_kernel(const float* partials, int shards,
                                                        float* stats, const RowArgs a) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kMergeNT + threadIdx.x;
  if (n >= a.rows) return;
  const int64_t y = a.target[n];
  const int cls = row_class(y, a.Vt, a.ignore_index);
  float4* st = reinterpret_cast<float4*>(stats) + n;
  if (cls != kValid) {
    const float l = (cls == kIgnored) ? 0.0f : __builtin_nanf("");
    store_row(a, n, l, 0.0f, l);
    *st = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const int64_t shard_stride = a.rows * VSCE_PARTIAL_STRIDE;
  auto rec = [&](int s, int k) { return partials[s * shard_stride + n * VSCE_PARTIAL_STRIDE + k]; };
  float m = -__builtin_inff(), mx = -__builtin_inff();
  int ss = 0, sa = 0;
  for (int s = 0; s < shards; ++s) {
    const float ms = rec(s, 0), xs = rec(s, 4);
    if (ms > m) {
      m = ms;
      ss = s;
    }
    if (xs > mx) {
      mx = xs;
      sa = s;
    }
  }
  float dp = rec(ss, 1), xy = 0.0f, S = 0.0f;
  for (int s = 0; s < shards; ++s) {
    if (s != ss) dp += (1.0f + rec(s, 1)) * __builtin_amdgcn_exp2f((rec(s, 0) - m) * kLog2e);
    xy += rec(s, 2);
    S += rec(s, 3);
  }
  const int first = __float_as_int(rec(sa, 5));
  const float wy = a.weight ? a.weight[y] : 1.0f;
  const float sum_w = static_cast<float>(a.ws->sum_w);
  const float lg = log1pf(dp);
  const float z = row_z(m, lg, a.zl);
  store_row(a, n, row_loss(m, lg, xy, S, wy, sum_w, a.eps, a.eta) + z,
            (static_cast<int64_t>(first) == y) ? 1.0f : 0.0f, z);
  *st = make_float4(m, dp, xy, a.eps > 0.0f ? S : 0.0f);
}

}  // namespace

int launch_merge(const Prob& p, const float* partials, int shards, float* stats,
                 const RowArgs& a, hipStream_t s) {
  if (p.rows == 0) return VSCE_OK;
  const int64_t grid = (p.rows + kMergeNT - 1) / kMergeNT;
  hipLaunchKernelGGL(merge_kernel, dim3(static_cast<unsigned>(grid)), dim3(kMergeNT), 0, s,
                     partials, shards, stats, a);
  return hipGetLastError() == hipSuccess ? VSCE_OK : VSCE_ERR_LAUNCH;
}

int launch_prologue(const Prob& p, WsHeader* ws, hipStream_t s) {
  hipLaunchKernelGGL(prologue_kernel, dim3(1), dim3(kSmallNT), 0, s, p.target, p.rows, p.Vt,
                     p.weight, p.ignore_index, ws);
  return hipGetLastError() == hipSuccess ? VSCE_OK : VSCE_ERR_LAUNCH;
}

int launch_finalize(const Prob& p, const float* loss_rows, const float* acc_rows,
                    const float* z_rows, float* loss_out, float* acc_mean_out, float* z_out,
                    const WsHeader* ws, hipStream_t s) {
  if (p.red == VSCE_REDUCTION_NONE && acc_mean_out == nullptr) return VSCE_OK;
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kSmallNT), 0, s, loss_rows, acc_rows,
                     p.red == VSCE_REDUCTION_NONE ? nullptr : z_rows, p.rows, p.red, loss_out,
                     acc_mean_out, z_out, ws);
  return hipGetLastError() == hipSuccess ? VSCE_OK : VSCE_ERR_LAUNCH;
}

}  // namespace vsce
