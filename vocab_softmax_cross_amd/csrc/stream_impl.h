// Streaming kernels: rows are read from memory as they are consumed.
// (Template definitions; stream_<dtype>.hip instantiate one element type each.)
//
//  stats_kernel      split forward (TransformerEngine PR #2325: the forward
//                    saves the per-row max, sum, target logit and
//                    scaled_x_sum and computes the loss): one read per row.
//  backward_kernel   split backward (same PR: fp32 gradient from the saved
//                    statistics, grad_output applied, target handled once,
//                    written in the input type): one read + one write.
//  scale_kernel      in-place grad_output scale of a saved gradient
//                    (linkedin#1290 commit message; SKIP_IF_ONE of Liger-Kernel
//                    PR #1622): returns at once where grad_output == 1.0.
//  fused_stream_kernel  fused forward + gradient for rows too long to keep on
//                    chip: the statistics pass, then the gradient pass reading
//                    the row a second time.
//
// Each thread keeps an online (max, sum) pair per lane: a batch of U vectors
// raises the lane max once and rescales the sum once.  After the workgroup
// max M is known, the shares of the lanes whose own max equals M are summed
// again with the elements equal to M left out (re-read by the whole
// workgroup, one vector per thread), so d' = d - 1 never loses the small
// terms to the leading 1.
//
// CAP (soft-capped logits): maxima, ties and the first index are taken on the
// stored logits, sums on the capped ones (the shift of a lane's sum is the
// capped value of its stored maximum), and every gradient element is
// multiplied by the slope of the cap at its stored logit.
#pragma once

#include <tuple>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "rowmath.h"

namespace vsce {
namespace {

// Elements of one "group": a 16-byte vector on the vector path, one element
// on the scalar path (rows that are not 16-byte aligned).
template <int DT, bool VECP>
struct Grp {
  using D = Dt<DT>;
  static constexpr int E = VECP ? D::VEC : 1;
  __device__ static inline void load(const char* row, int64_t g, float (&f)[E]) {
    if constexpr (VECP) {
      D::unpack(nt_load16(row + g * 16), f);
    } else {
      f[0] = D::load1(row, g);
    }
  }
  __device__ static inline void store(char* row, int64_t g, const float (&f)[E]) {
    if constexpr (VECP) {
      nt_store16(row + g * 16, D::pack(f));
    } else {
      D::store1(row, g, f[0]);
    }
  }
  __device__ static inline void weights(const float* w, int64_t g, float (&wv)[E]) {
    if constexpr (VECP) {
      const float4* p = reinterpret_cast<const float4*>(w + g * E);
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        const float4 t = p[q];
        wv[4 * q] = t.x;
        wv[4 * q + 1] = t.y;
        wv[4 * q + 2] = t.z;
        wv[4 * q + 3] = t.w;
      }
    } else {
      wv[0] = w[g];
    }
  }
};

// Per-row statistics by streaming: returns (M, d', S, first) on every thread,
// M being the (capped) maximum the loss reads, and the maximum of the stored
// logits in *Mraw_out.  Must be called by the whole workgroup (it contains
// barriers).
template <int DT, int NT, int U, bool WEIGHTED, bool VECP, bool CAP>
__device__ inline void stream_stats(const RowArgs& a, const char* row, float& M_out,
                                    float& dp_out, float& S_out, int& first_out, float* red_max,
                                    float4* red_sum, float* Mraw_out = nullptr) {
  using G = Grp<DT, VECP>;
  constexpr int E = G::E;
  const int tid = threadIdx.x;
  const int64_t ng = a.nvec;
  const SoftCap cap{a.cap, a.cap_k};
  auto capped = [&](float v) { return CAP ? cap.value(v) : v; };
  float m = -__builtin_inff(), s = 0.0f, S = 0.0f;

  for (int64_t g0 = 0; g0 < ng; g0 += static_cast<int64_t>(NT) * U) {
    float f[U][E];
    bool ok[U];
    static_for<U>([&](auto u) {
      const int64_t g = g0 + u * NT + tid;
      ok[u] = g < ng;
      if (ok[u]) G::load(row, g, f[u]);
    });
    float bm = -__builtin_inff();
    static_for<U>([&](auto u) {
      if (ok[u]) {
#pragma unroll
        for (int i = 0; i < E; ++i) bm = fmaxf(bm, f[u][i]);
      }
    });
    if (bm > m) {
      s *= __builtin_amdgcn_exp2f((capped(m) - capped(bm)) * kLog2e);
      m = bm;
    }
    const float ML = (m == -__builtin_inff()) ? 0.0f : capped(m) * kLog2e;
    static_for<U>([&](auto u) {
      if (ok[u]) {
        float wv[E];
        if constexpr (WEIGHTED) G::weights(a.weight, g0 + u * NT + tid, wv);
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const float fc = capped(f[u][i]);
          s += exp_shifted(fc, ML);
          if constexpr (WEIGHTED) S = __builtin_fmaf(wv[i], fc, S);
          else S += fc;
        }
      }
    });
  }

  const float M = block_max<NT>(m, red_max);     // of the stored logits
  const float Mc = capped(M);                    // of the logits the loss reads
  const float ML = (M == -__builtin_inff()) ? 0.0f : Mc * kLog2e;
  RowSums rs = {0.0f, S, 0, 0x7fffffff};
  const bool owner = (m == M);  // this lane's share holds the row maximum
  if (!owner)
    rs.s = (m == -__builtin_inff()) ? 0.0f
                                    : s * __builtin_amdgcn_exp2f((capped(m) - Mc) * kLog2e);
  // The shares of the lanes that hold the maximum are summed again with every
  // element equal to M left out -- by the whole workgroup, one vector per
  // thread, so the second look costs one memory round trip rather than one per
  // batch of the owner's share.  Owners are listed in lane order (a prefix
  // count over the wavefronts' ballots), so the sum order is fixed.
  constexpr int NW = NT / kWave;
  __shared__ uint64_t owner_mask[NW];
  __shared__ int owners[NT];
  const int lane = tid & (kWave - 1), wave = uniform(tid / kWave);
  const uint64_t ball = __ballot(owner);
  if (lane == 0) owner_mask[wave] = ball;
  lds_barrier();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = __builtin_popcountll(owner_mask[w]);
    base += (w < wave) ? c : 0;
    total += c;
  }
  if (owner) {
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(ball >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(ball), 0));
    owners[base + below] = tid;
  }
  lds_barrier();
  // Vectors of a lane's share: lane t holds groups t, t + NT, ... below ng.
  const int share = static_cast<int>((ng + NT - 1) / NT);
  const int items = total * share;
  for (int w = tid; w < items; w += NT) {
    const int o = w / share;
    const int64_t g = owners[o] + static_cast<int64_t>(w - o * share) * NT;
    if (g < ng) {
      float f[E];
      G::load(row, g, f);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const bool eq = (f[i] == M);
        rs.s += eq ? 0.0f : exp_shifted(capped(f[i]), ML);
        rs.cnt += eq ? 1 : 0;
        if (eq) rs.first = min(rs.first, static_cast<int>(g * E + i));
      }
    }
  }
  rs = block_sums<NT>(rs, red_sum);
  M_out = Mc;
  if (Mraw_out) *Mraw_out = M;
  dp_out = rs.s + static_cast<float>(rs.cnt - 1);
  S_out = rs.S;
  first_out = rs.first;
}

// Writes the gradient of one row segment [g_begin, g_end) of groups, with
// the true-class element substituted by its owner (t.dxy is final: under CAP
// the caller has multiplied it by the slope at the stored x[y]).
template <int DT, int NT, int U, bool WEIGHTED, bool VECP, bool CAP>
__device__ inline void stream_grad(const RowArgs& a, const char* src, char* dst, int64_t g_begin,
                                   int64_t g_end, const RowTerms& t, int64_t y) {
  using G = Grp<DT, VECP>;
  constexpr int E = G::E;
  const int tid = threadIdx.x;
  const SoftCap cap{a.cap, a.cap_k};
  const int64_t gy = y >= 0 ? y / E : -1;  // y < 0: no element here owns the target
  const int iy = static_cast<int>(y >= 0 ? y % E : 0);
  for (int64_t g0 = g_begin; g0 < g_end; g0 += static_cast<int64_t>(NT) * U) {
    float f[U][E];
    static_for<U>([&](auto u) {
      const int64_t g = g0 + u * NT + tid;
      if (g < g_end) G::load(src, g, f[u]);
    });
    static_for<U>([&](auto u) {
      const int64_t g = g0 + u * NT + tid;
      if (g < g_end) {
        float wv[E];
        if constexpr (WEIGHTED) G::weights(a.weight, g, wv);
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const float b = WEIGHTED ? t.B * wv[i] : t.B;
          if constexpr (CAP) {
            float slope;
            const float fc = cap.value(f[u][i], slope);
            f[u][i] = __builtin_fmaf(exp_shifted(fc, t.ML), t.K, -b) * slope;
          } else {
            f[u][i] = __builtin_fmaf(exp_shifted(f[u][i], t.ML), t.K, -b);
          }
        }
        if (g == gy) {  // the owner stores the finished true-class value
#pragma unroll
          for (int i = 0; i < E; ++i)
            if (i == iy) f[u][i] = t.dxy;
        }
        G::store(dst, g, f[u]);
      }
    });
  }
}

template <int DT, bool VECP>
__device__ inline void stream_zero(char* dst, int64_t g_begin, int64_t g_end, int nt, int u_) {
  using G = Grp<DT, VECP>;
  float z[G::E];
#pragma unroll
  for (int i = 0; i < G::E; ++i) z[i] = 0.0f;
  for (int64_t g = g_begin + threadIdx.x; g < g_end; g += nt) G::store(dst, g, z);
}

// w[y] for a global class y (a.weight points at this buffer's first column
// of the full weight vector).
__device__ inline float row_weight(const RowArgs& a, int64_t y, bool weighted) {
  return weighted ? a.weight[y - a.voff] : 1.0f;
}

// Slope of the soft-cap at the stored true-class logit (1 without CAP).
template <bool CAP>
__device__ inline float cap_slope(const RowArgs& a, float x) {
  if constexpr (!CAP) return 1.0f;
  float slope;
  SoftCap{a.cap, a.cap_k}.value(x, slope);
  return slope;
}

template <int DT, int NT, int U, bool WEIGHTED, bool VECP, bool CAP>
__global__ __launch_bounds__(NT) void stats_kernel(const RowArgs a) {
  using D = Dt<DT>;
  __shared__ float red_max[NT / kWave];
  __shared__ float4 red_sum[NT / kWave];
  const int64_t n = xcd_contiguous(blockIdx.x, a.rows);
  const char* row = static_cast<const char*>(a.x) + n * a.stride * D::BYTES;
  const int64_t y = a.target[n];
  const int cls = row_class(y, a.Vt, a.ignore_index);
  if (cls != kValid) {
    if (threadIdx.x == 0) {
      if (a.partial) {
        float4* pr = reinterpret_cast<float4*>(a.partial + n * VSCE_PARTIAL_STRIDE);
        pr[0] = make_float4(0.f, 0.f, 0.f, 0.f);
        pr[1] = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
      }
      const float l = (cls == kIgnored) ? 0.0f : __builtin_nanf("");
      store_row(a, n, l, 0.0f, l);
      if (a.stats) reinterpret_cast<float4*>(a.stats)[n] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  float M, dp, S, Mraw;
  int first;
  stream_stats<DT, NT, U, WEIGHTED, VECP, CAP>(a, row, M, dp, S, first, red_max, red_sum, &Mraw);
  if (a.partial) {
    // One shard's record (vocab-parallel): the target logit only where this
    // shard holds column y, the first maximum as a global column.
    if (threadIdx.x == 0) {
      const int64_t yl = y - a.voff;
      float xy = 0.0f;
      if (yl >= 0 && yl < a.V) {
        const float xs = D::load1(row, yl);
        xy = CAP ? SoftCap{a.cap, a.cap_k}.value(xs) : xs;
      }
      float4* pr = reinterpret_cast<float4*>(a.partial + n * VSCE_PARTIAL_STRIDE);
      pr[0] = make_float4(M, dp, xy, a.eps > 0.0f ? S : 0.0f);
      pr[1] = make_float4(Mraw, __int_as_float(static_cast<int>(a.voff) + first), 0.f, 0.f);
    }
    return;
  }
  if (threadIdx.x == 0) {
    const float xs = D::load1(row, y);
    const float xy = CAP ? SoftCap{a.cap, a.cap_k}.value(xs) : xs;
    const float sum_w = static_cast<float>(a.ws->sum_w);
    const float lg = log1pf(dp);
    const float zrow = row_z(M, lg, a.zl);
    store_row(a, n,
              row_loss(M, lg, xy, S, row_weight(a, y, WEIGHTED), sum_w, a.eps, a.eta) + zrow,
              (static_cast<int64_t>(first) == y) ? 1.0f : 0.0f, zrow);
    if (a.stats)
      reinterpret_cast<float4*>(a.stats)[n] = make_float4(M, dp, xy, a.eps > 0.0f ? S : 0.0f);
  }
}

template <int DT, int NT, int U, bool WEIGHTED, bool VECP, bool CAP>
__global__ __launch_bounds__(NT) void fused_stream_kernel(const RowArgs a) {
  using D = Dt<DT>;
  __shared__ float red_max[NT / kWave];
  __shared__ float4 red_sum[NT / kWave];
  const int64_t n = xcd_contiguous(blockIdx.x, a.rows);
  char* row = static_cast<char*>(a.x) + n * a.stride * D::BYTES;
  const int64_t y = a.target[n];
  const int cls = row_class(y, a.Vt, a.ignore_index);
  if (cls != kValid) {
    stream_zero<DT, VECP>(row, 0, a.nvec, NT, U);
    const float l = (cls == kIgnored) ? 0.0f : __builtin_nanf("");
    if (threadIdx.x == 0) store_row(a, n, l, 0.0f, l);
    return;
  }
  float M, dp, S;
  int first;
  stream_stats<DT, NT, U, WEIGHTED, VECP, CAP>(a, row, M, dp, S, first, red_max, red_sum);
  const float xs = D::load1(row, y);
  const float xy = CAP ? SoftCap{a.cap, a.cap_k}.value(xs) : xs;
  const float sum_w = static_cast<float>(a.ws->sum_w);
  const float wy = row_weight(a, y, WEIGHTED);
  const float lg = log1pf(dp);
  if (threadIdx.x == 0) {
    const float zrow = row_z(M, lg, a.zl);
    store_row(a, n, row_loss(M, lg, xy, S, wy, sum_w, a.eps, a.eta) + zrow,
              (static_cast<int64_t>(first) == y) ? 1.0f : 0.0f, zrow);
  }
  // Every thread has read x[y] before any thread overwrites it: the block
  // reduction inside stream_stats ended with a barrier, and x[y] is re-read
  // here, so order the read before the first store of the gradient pass.
  __syncthreads();
  const float sigma = a.mean ? a.ws->inv_W : 1.0f;
  RowTerms t = row_terms(M, dp, lg, xy, wy, sum_w, a.eps, a.eta, sigma, a.zl, z_sigma(a));
  t.dxy *= cap_slope<CAP>(a, xs);
  stream_grad<DT, NT, U, WEIGHTED, VECP, CAP>(a, row, row, 0, a.nvec, t, y);
}

// Split backward over (row, column chunk) workgroups.
template <int DT, int NT, int U, bool WEIGHTED, bool VECP, bool CAP>
__global__ __launch_bounds__(NT) void backward_kernel(const RowArgs a) {
  using D = Dt<DT>;
  const int64_t b = xcd_contiguous(blockIdx.x, a.rows * a.chunks);
  const int64_t n = b / a.chunks;
  const int64_t c = b - n * a.chunks;
  const int64_t per = static_cast<int64_t>(NT) * U;
  const int64_t g_begin = c * per;
  const int64_t g_end = min(a.nvec, g_begin + per);
  const char* src = static_cast<const char*>(a.x) + n * a.stride * D::BYTES;
  char* dst = static_cast<char*>(a.g) + n * a.stride * D::BYTES;
  const int64_t y = a.target[n];
  const int cls = row_class(y, a.Vt, a.ignore_index);
  if (cls != kValid) {
    stream_zero<DT, VECP>(dst, g_begin, g_end, NT, U);
    return;
  }
  const float4 st = reinterpret_cast<const float4*>(a.stats)[n];
  const float go = a.go[n * a.go_stride];
  const float sigma = (a.mean ? a.ws->inv_W : 1.0f) * go;
  const float sum_w = static_cast<float>(a.ws->sum_w);
  RowTerms t = row_terms(st.x, st.y, log1pf(st.y), st.z, row_weight(a, y, WEIGHTED), sum_w,
                         a.eps, a.eta, sigma, a.zl, z_sigma(a) * go);
  // The target's column in this buffer (a vocab-parallel shard may not hold
  // it: then no element of the row takes the true-class value).
  const int64_t yl = (y - a.voff >= 0 && y - a.voff < a.V) ? y - a.voff : -1;
  // The saved x[y] is capped; the slope needs the stored one.  Only the
  // chunk that holds column y reads it (src is not yet overwritten: each
  // workgroup writes its own chunk only, after this read).
  if constexpr (CAP) {
    const int64_t per_elems = static_cast<int64_t>(NT) * U * Grp<DT, VECP>::E;
    if (yl >= 0 && yl / per_elems == c) t.dxy *= cap_slope<CAP>(a, D::load1(src, yl));
  }
  stream_grad<DT, NT, U, WEIGHTED, VECP, CAP>(a, src, dst, g_begin, g_end, t, yl);
}

// Grid-stride over (row, column chunk) work items, so that a grad_output of
// 1.0 costs one small launch: every workgroup reads the scalar once and
// returns.
template <int DT, int NT, int U, bool VECP>
__global__ __launch_bounds__(NT) void scale_kernel(const RowArgs a) {
  using D = Dt<DT>;
  using G = Grp<DT, VECP>;
  if (a.skip_if_one && a.go_stride == 0 && a.go[0] == 1.0f) return;
  const int64_t per = static_cast<int64_t>(NT) * U;
  const int64_t items = a.rows * a.chunks;
  for (int64_t b = blockIdx.x; b < items; b += gridDim.x) {
    const int64_t n = b / a.chunks;
    const int64_t c = b - n * a.chunks;
    const float go = a.go[n * a.go_stride];
    if (a.skip_if_one && go == 1.0f) continue;
    const int64_t g_begin = c * per;
    const int64_t g_end = min(a.nvec, g_begin + per);
    char* row = static_cast<char*>(a.g) + n * a.stride * D::BYTES;
    float f[U][G::E];
    static_for<U>([&](auto u) {
      const int64_t g = g_begin + u * NT + threadIdx.x;
      if (g < g_end) G::load(row, g, f[u]);
    });
    static_for<U>([&](auto u) {
      const int64_t g = g_begin + u * NT + threadIdx.x;
      if (g < g_end) {
#pragma unroll
        for (int i = 0; i < G::E; ++i) f[u][i] *= go;
        G::store(row, g, f[u]);
      }
    });
  }
}

constexpr int kStreamNT = 256;
constexpr int kStreamU = 4;
constexpr int64_t kScaleGrid = 2048;  // 8 workgroups per CU

template <int DT>
int64_t groups(const Prob& p) {
  return p.vec_ok ? p.V / Dt<DT>::VEC : p.V;
}

template <class K>
int launch(K kernel, int64_t grid, int nt, const RowArgs& a, hipStream_t s) {
  if (grid <= 0) return VSCE_OK;
  if (grid > 0x7fffffffLL) return VSCE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(nt), 0, s, a);
  return hipGetLastError() == hipSuccess ? VSCE_OK : VSCE_ERR_LAUNCH;
}

enum Which { kStats, kFusedStream, kBackward, kScale };

template <int DT, bool W, bool VECP, bool CAP>
int launch_which(Which which, const Prob& p, RowArgs a, hipStream_t s) {
  constexpr int NT = kStreamNT, U = kStreamU;
  a.nvec = groups<DT>(p);
  const int64_t per = static_cast<int64_t>(NT) * U;
  a.chunks = (a.nvec + per - 1) / per;
  switch (which) {
    case kStats: return launch(stats_kernel<DT, NT, U, W, VECP, CAP>, p.rows, NT, a, s);
    case kFusedStream:
      return launch(fused_stream_kernel<DT, NT, U, W, VECP, CAP>, p.rows, NT, a, s);
    case kBackward:
      return launch(backward_kernel<DT, NT, U, W, VECP, CAP>, p.rows * a.chunks, NT, a, s);
    case kScale:
      if constexpr (CAP) return VSCE_ERR_INVALID;  // the scale does not depend on the cap
      else
        return launch(scale_kernel<DT, NT, U, VECP>, min(p.rows * a.chunks, kScaleGrid), NT, a,
                      s);
  }
  return VSCE_ERR_INVALID;
}

template <int DT, bool CAP>
int dispatch(Which which, const Prob& p, const RowArgs& a, hipStream_t s) {
  const bool w = p.weight != nullptr && which != kScale;
  if (p.vec_ok) {
    return w ? launch_which<DT, true, true, CAP>(which, p, a, s)
             : launch_which<DT, false, true, CAP>(which, p, a, s);
  }
  return w ? launch_which<DT, true, false, CAP>(which, p, a, s)
           : launch_which<DT, false, false, CAP>(which, p, a, s);
}

}  // namespace

template <int DT, bool CAP>
int stream_dt(int which, const Prob& p, const RowArgs& a, hipStream_t s) {
  return dispatch<DT, CAP>(static_cast<Which>(which), p, a, s);
}

}  // namespace vsce
