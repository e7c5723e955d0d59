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
//  fused_ring_kernel fused forward + gradient in one launch for rows too long
//                    to keep on chip: the statistics pass, then the gradient
//                    pass reading the row a second time, both fed through a
//                    ring of LDS stages filled by direct-to-LDS loads (16-byte
//                    vector path, no class weights).  The default for such
//                    rows is the stats_kernel + backward_kernel pair in place.
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

// The end of a row's statistics, once every lane holds its online (m, s, S)
// over its share of the row (m the lane's maximum of the stored logits, s the
// sum of exp(capped(x) - capped(m)) over its elements, S its logit sum):
// returns (M, d', S, first) on every thread, M being the (capped) maximum the
// loss reads, and the maximum of the stored logits in *Mraw_out (if given).
// Lane t's share must be the groups t, t + NT, t + 2 NT, ... below a.nvec:
// the owners' shares are re-read in that layout.  Must be called by the whole
// workgroup (it contains barriers).
template <int DT, int NT, bool VECP, bool CAP>
__device__ inline void finish_stats(const RowArgs& a, const char* row, float m, float s, float S,
                                    float& M_out, float& dp_out, float& S_out, int& first_out,
                                    float* red_max, float4* red_sum, float* Mraw_out) {
  using G = Grp<DT, VECP>;
  constexpr int E = G::E;
  const int tid = threadIdx.x;
  const int64_t ng = a.nvec;
  const SoftCap cap = soft_cap(a);
  auto capped = [&](float v) { return CAP ? cap.value(v) : v; };
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
  const SoftCap cap = soft_cap(a);
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

  finish_stats<DT, NT, VECP, CAP>(a, row, m, s, S, M_out, dp_out, S_out, first_out, red_max,
                                  red_sum, Mraw_out);
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
  const SoftCap cap = soft_cap(a);
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
__device__ inline void stream_zero(char* dst, int64_t g_begin, int64_t g_end, int nt) {
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
  soft_cap(a).value(x, slope);
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
        xy = CAP ? soft_cap(a).value(xs) : xs;
      }
      float4* pr = reinterpret_cast<float4*>(a.partial + n * VSCE_PARTIAL_STRIDE);
      pr[0] = make_float4(M, dp, xy, a.eps > 0.0f ? S : 0.0f);
      pr[1] = make_float4(Mraw, __int_as_float(static_cast<int>(a.voff) + first), 0.f, 0.f);
    }
    return;
  }
  if (threadIdx.x == 0) {
    const float xs = D::load1(row, y);
    const float xy = CAP ? soft_cap(a).value(xs) : xs;
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

// ---------------------------------------------------------------- LDS ring
// 16 bytes from LDS, complete on return.  The read is opaque to the compiler
// (no wait for the direct-to-LDS loads it cannot tell apart), and it has
// finished before the caller refills the slot.
__device__ __forceinline__ uint4 lds_read16_now(const uint4* p) {
  const uint32_t addr = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint4*)p));
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Keeps the compiler from moving memory operations across this point, so the
// order of loads and stores the wait counts assume is the issue order.
__device__ __forceinline__ void issue_order() { asm volatile("" ::: "memory"); }

// Fused forward + in-place gradient for rows too long to keep on chip, on the
// 16-byte vector path without class weights: the statistics pass, then the
// gradient pass, each fed through a ring of LDS stages.  Each wavefront owns
// NS slots of 64 x 16 bytes and keeps its next NS stages in flight as
// direct-to-LDS loads (buffer_load_dwordx4 ... lds) while it works on the
// current one: the multi-stage, prologue-prefetched load ring that the
// linkedin#1290 commit message (Liger-Kernel PR #1268, "Source of the gains vs
// Triton", item 1) credits for hiding HBM latency, here without the register
// cost of holding the stages in flight.  The gradient pass also keeps its
// stores off the critical path: the wait for stage k counts exactly the loads
// and stores issued after it, so the stores of the last NS stages stay in
// flight (a wait on a load would otherwise also wait for every older store).
//
// Stage k of wavefront w holds vectors (k NW + w) 64 + lane, so thread t holds
// vectors t, t + NT, t + 2 NT, ... as finish_stats expects.  Stages past the
// row (the last stages of some wavefronts, and the NS stages each pass loads
// beyond its end) are dropped by the buffer range check: no memory is read.
template <int DT, int NT, int NS, bool CAP>
__global__ __launch_bounds__(NT) void fused_ring_kernel(const RowArgs a) {
  using D = Dt<DT>;
  constexpr int E = D::VEC;
  constexpr int NW = NT / kWave;
  static_assert((NS & (NS - 1)) == 0 && 2 * NS - 1 <= 63, "NS: a power of 2, at most 32");
  __shared__ uint4 ring[NW * NS * kWave];
  __shared__ float red_max[NW];
  __shared__ float4 red_sum[NW];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = uniform(tid / kWave);
  const int64_t n = xcd_contiguous(blockIdx.x, a.rows);
  char* row = static_cast<char*>(a.x) + n * a.stride * D::BYTES;
  const auto rsrc = make_rsrc(row, static_cast<uint32_t>(a.V * D::BYTES));
  const int64_t y = a.target[n];
  const int cls = row_class(y, a.Vt, a.ignore_index);
  if (cls != kValid) {
    stream_zero<DT, true>(row, 0, a.nvec, NT);
    const float l = (cls == kIgnored) ? 0.0f : __builtin_nanf("");
    if (tid == 0) store_row(a, n, l, 0.0f, l);
    return;
  }
  const int nvec = static_cast<int>(a.nvec);
  const int stages = (nvec + NT - 1) / NT;
  uint4* const mine = ring + wave * NS * kWave;
  auto slot = [&](int k) { return mine + (k & (NS - 1)) * kWave; };
  auto vec = [&](int k) { return (k * NW + wave) * kWave + lane; };
  auto fetch = [&](int k) {
    buf_load16_lds(rsrc, slot(k), static_cast<uint32_t>(vec(k)) * 16u, 0);
  };
  const SoftCap cap = soft_cap(a);
  auto capped = [&](float v) { return CAP ? cap.value(v) : v; };

  // ---- pass 1: online (max, sum, logit sum) per lane
  float m = -__builtin_inff(), s = 0.0f, S = 0.0f;
  for (int k = 0; k < NS; ++k) fetch(k);
  for (int k = 0; k < stages; ++k) {
    wait_vm<NS - 1>();  // stage k has landed; NS - 1 later loads may not have
    const uint4 v = lds_read16_now(slot(k) + lane);
    fetch(k + NS);
    issue_order();
    if (vec(k) < nvec) {
      float f[E];
      D::unpack(v, f);
      float bm = f[0];
#pragma unroll
      for (int i = 1; i < E; ++i) bm = fmaxf(bm, f[i]);
      if (bm > m) {
        s *= __builtin_amdgcn_exp2f((capped(m) - capped(bm)) * kLog2e);
        m = bm;
      }
      const float ML = (m == -__builtin_inff()) ? 0.0f : capped(m) * kLog2e;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float fc = capped(f[i]);
        s += exp_shifted(fc, ML);
        S += fc;
      }
    }
  }
  wait_vm<0>();  // the loads past the end write their (empty) slots too

  float M, dp, Sr;
  int first;
  finish_stats<DT, NT, true, CAP>(a, row, m, s, S, M, dp, Sr, first, red_max, red_sum, nullptr);
  const float xs = D::load1(row, y);
  const float xy = CAP ? cap.value(xs) : xs;
  const float sum_w = static_cast<float>(a.ws->sum_w);
  const float lg = log1pf(dp);
  if (tid == 0) {
    const float zrow = row_z(M, lg, a.zl);
    store_row(a, n, row_loss(M, lg, xy, Sr, 1.0f, sum_w, a.eps, a.eta) + zrow,
              (static_cast<int64_t>(first) == y) ? 1.0f : 0.0f, zrow);
  }
  const float sigma = a.mean ? a.ws->inv_W : 1.0f;
  RowTerms t = row_terms(M, dp, lg, xy, 1.0f, sum_w, a.eps, a.eta, sigma, a.zl, z_sigma(a));
  t.dxy *= cap_slope<CAP>(a, xs);
  // Every thread has its x[y] (used above) before any thread overwrites the
  // row.
  __syncthreads();

  // ---- pass 2: the gradient, stage by stage, stored over the logits
  const int jy = static_cast<int>(y / E);  // vector, stage and thread holding column y
  const int ky = jy / NT, ty = jy % NT, iy = static_cast<int>(y % E);
  for (int k = 0; k < NS; ++k) fetch(k);
  for (int k = 0; k < stages; ++k) {
    // Issued after stage k: the rest of the prologue and two operations per
    // earlier iteration (at least NS - 1 while k < NS), or stage k's own
    // iteration's store and two per later one (exactly 2 NS - 1).
    if (k < NS) wait_vm<NS - 1>();
    else wait_vm<2 * NS - 1>();
    const uint4 v = lds_read16_now(slot(k) + lane);
    fetch(k + NS);
    issue_order();
    float f[E];
    D::unpack(v, f);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if constexpr (CAP) {
        float slope;
        const float fc = cap.value(f[i], slope);
        f[i] = __builtin_fmaf(exp_shifted(fc, t.ML), t.K, -t.B) * slope;
      } else {
        f[i] = __builtin_fmaf(exp_shifted(f[i], t.ML), t.K, -t.B);
      }
    }
    if (k == ky && tid == ty) {
#pragma unroll
      for (int i = 0; i < E; ++i)
        if (i == iy) f[i] = t.dxy;
    }
    buf_store16(rsrc, static_cast<uint32_t>(vec(k)) * 16u, 0, D::pack(f));
    issue_order();
  }
  wait_vm<0>();  // no direct-to-LDS write may land after the workgroup ends
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
    stream_zero<DT, VECP>(dst, g_begin, g_end, NT);
    return;
  }
  const float4 st = reinterpret_cast<const float4*>(a.stats)[n];
  const float go = a.go ? a.go[n * a.go_stride] : 1.0f;  // null: the fused mode's pair
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
// The LDS ring: 256 threads, 8 stages of 1 KB per wavefront (32 KB of LDS
// per row, five rows per CU).
constexpr int kRingNT = 256;
constexpr int kRingNS = 8;
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

enum Which { kStats, kRing, kBackward, kScale };

template <int DT, bool W, bool VECP, bool CAP>
int launch_which(Which which, const Prob& p, RowArgs a, hipStream_t s) {
  constexpr int NT = kStreamNT, U = kStreamU;
  a.nvec = groups<DT>(p);
  const int64_t per = static_cast<int64_t>(NT) * U;
  a.chunks = (a.nvec + per - 1) / per;
  switch (which) {
    case kStats: return launch(stats_kernel<DT, NT, U, W, VECP, CAP>, p.rows, NT, a, s);
    case kRing:
      // The ring needs whole 16-byte vectors; per-element class weights would
      // add loads the ring's wait counts do not cover.
      if constexpr (VECP && !W)
        return launch(fused_ring_kernel<DT, kRingNT, kRingNS, CAP>, p.rows, kRingNT, a, s);
      else
        return VSCE_ERR_UNSUPPORTED;
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
