// Fused forward + in-place gradient with the whole row held on chip.
// (Template definitions; fused_<dtype>.hip instantiate one element type each.)
//
// One workgroup per row.  The row is read from HBM once, with 16-byte
// vector loads: thread t holds vectors t, t + NT, t + 2 NT, ... of the row,
// the first NREG of them in registers and the next NLDS in LDS (loaded
// straight into LDS with global_load_lds_dwordx4).  Three passes then run
// over the on-chip copy:
//   1. the row maximum M (workgroup max, one barrier);
//   2. the sum of exp(x - M) with every element equal to M left out, the
//      number of such elements and the first index of M (only the wavefronts
//      holding M take this careful path; the others just add), plus the
//      (weighted) logit sum for label smoothing (workgroup sum, one barrier);
//   3. the gradient, written over the logits with one store per vector; the
//      lane that owns the target column substitutes the fp32 true-class value
//      before its store.
// Rows a little longer than the chip holds (NOV > 0, uncapped logits): the
// first NT * NREG + LDS_CAP vectors are held as above and the rest, the
// overflow (thread t: vectors ONCHIP + k NT + t, k < NOV), is read twice
// instead: once before the row's first register slots are loaded, folded
// into an online (maximum, sum below it, count of it, first index of it,
// logit sum), merged over the wavefront and parked in LDS, which joins the
// row maximum in pass 1 and the pass-2 sums once that maximum is known; and
// once more in pass 3, for its gradient.  Two rows per CU stay resident, at
// the cost of reading the overflow twice.
// The design follows the fused kernel of Liger-Kernel PR #1268 ("pass 1"
// online statistics, "pass 2" in-place gradient, one O(1) true-class
// correction, fp32 per the linkedin#1329 commit message), with the second
// read of the logits served from registers and LDS instead of memory.
#pragma once

#include <tuple>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "rowmath.h"

namespace vsce {
namespace {

// LDS_CAP: vectors of LDS actually allocated (<= NLDS * NT).  The last LDS
// slot may be partial: the shape then serves rows of at most NT * NREG +
// LDS_CAP vectors, and no lane past that ever touches LDS.
// CAP: soft-capped logits.  The row maximum, its ties and its first index
// are taken on the stored logits (capping does not reorder them); every sum,
// the loss and the gradient read the capped values, and each gradient element
// is multiplied by the slope of the cap at its own stored logit.
// NOV: overflow vectors per thread (0: the row fits on chip).
template <int DT, int NT, int NREG, int NLDS, int LDS_CAP, int NOV, bool WEIGHTED, bool CAP,
          int WPE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE)))
void fused_resident_kernel(const RowArgs a) {
  using D = Dt<DT>;
  constexpr int VEC = D::VEC;
  constexpr int NW = NT / kWave;
  constexpr uint32_t SLOT_BYTES = NT * 16u;  // bytes between a thread's vectors
  static_assert(LDS_CAP <= NLDS * NT && LDS_CAP > (NLDS - 1) * NT - (NLDS == 0 ? 1 : 0),
                "the capped LDS must still reach into the last LDS slot");
  static_assert(NOV == 0 || (!CAP && !WEIGHTED && NOV <= NREG),
                "overflow: uncapped, unweighted rows, reusing registers");
  constexpr int ONCHIP = NT * NREG + LDS_CAP;  // vectors held on chip
  __shared__ uint4 xl[NLDS > 0 ? LDS_CAP : 1];
  __shared__ float red_max[NW];
  __shared__ float4 red_sum[NW];
  __shared__ float xy_sh;  // the stored target logit, posted by its owner lane
  __shared__ float4 red_sum3[WEIGHTED ? NW : 1];  // pass 3's weighted logit sum
  // Each wavefront's overflow state (NOV > 0): maximum, sum below it, logit
  // sum, count at it, first index of it.
  constexpr int NWO = NOV > 0 ? NW : 1;
  __shared__ float ov_m[NWO], ov_s[NWO], ov_S[NWO];
  __shared__ int ov_c[NWO], ov_f[NWO];

  const int tid = threadIdx.x;
  const int64_t n = xcd_contiguous(blockIdx.x, a.rows);
  const int nvec = static_cast<int>(a.nvec);
  char* rowb = static_cast<char*>(a.x) + n * a.stride * D::BYTES;
  const auto rsrc = make_rsrc(rowb, static_cast<uint32_t>(a.V * D::BYTES));
  const uint32_t voff = static_cast<uint32_t>(tid) * 16u;
  // On-chip slot k of this thread is in the row (with an overflow, only the
  // first ONCHIP vectors are on chip: no lane past LDS_CAP touches LDS).
  const int nchip = NOV > 0 ? min(nvec, ONCHIP) : nvec;
  auto in_row = [&](int k) { return k * NT + tid < nchip; };
  // Lanes past the end of the row get a per-lane offset beyond num_records,
  // so the buffer range check drops them whether or not it counts soffset.
  auto lane_off = [&](int k) { return in_row(k) ? voff : kOutOfRange; };
  // Overflow vector k of thread t.  A valid row's overflow loads and stores
  // are exec-masked, with one per-lane offset and slot k in soffset; ov_off
  // (each lane's own offset, past num_records beyond the row) serves the
  // stores of an ignored row.  Callers pass a fresh_tid() of their own, so
  // that these are computed where used instead of held in registers.
  auto ov_col = [&](int k, int t) { return ONCHIP + k * NT + t; };
  auto ov_off = [&](int k, int t) {
    return ov_col(k, t) < nvec ? static_cast<uint32_t>(ov_col(k, t)) * 16u : kOutOfRange;
  };
  const int64_t y = a.target[n];
  const int cls = row_class(y, a.Vt, a.ignore_index);
  const SoftCap cap = soft_cap(a);

  if (cls != kValid) {  // uniform over the workgroup: zero gradient, no read
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    static_for<NREG + NLDS>([&](auto k) { buf_store16(rsrc, lane_off(k), k * SLOT_BYTES, z); });
    static_for<NOV>([&](auto k) { buf_store16(rsrc, ov_off(k, tid), 0u, z); });
    const float l = (cls == kIgnored) ? 0.0f : __builtin_nanf("");
    if (tid == 0) store_row(a, n, l, 0.0f, l);
    return;
  }


  // ---- one read of the row: registers, then LDS (lanes past the row read 0
  //      and are masked out of every pass below)
  // (With an overflow, slots 0 .. NOV-1 are loaded after it: their registers
  // first carry the overflow.)
  uint4 r[NREG];
  static_for<NREG>([&](auto k) {
    if constexpr (k >= NOV) r[k] = buf_load16(rsrc, lane_off(k), k * SLOT_BYTES);
  });
  if constexpr (NLDS > 0) {
    const int wave_base = __builtin_amdgcn_readfirstlane(tid & ~(kWave - 1));
    // Exec-masked rather than range-checked: lanes past the row write nothing
    // to LDS (the last slot's allocation may end before them).
    static_for<NLDS>([&](auto k) {
      if (in_row(NREG + k))
        buf_load16_lds(rsrc, xl + k * NT + wave_base, voff, (NREG + k) * SLOT_BYTES);
    });
  }


  // Every pass works on one 32-bit word (EPW elements) at a time, so only a
  // few fp32 temporaries are live next to the resident row.
  constexpr int EPW = D::EPW;
  auto words = [](const uint4 v) {
    struct W4 { uint32_t w[4]; };
    return W4{{v.x, v.y, v.z, v.w}};
  };
  // ---- the overflow, read for the first time: an online maximum om, the sum
  //      osum of exp(x - om) over elements below it, their count oc at it, the
  //      first index of it and the logit sum.  A vector that raises om rescales
  //      what came before once (the elements then at the old maximum join the
  //      sum).  The owner of the target column posts x[y] here.  The lanes'
  //      states are merged over the wavefront (the same rescaling) and lane 0
  //      parks the result in LDS, so no register carries it through pass 1.
  if constexpr (NOV > 0) {
    float om = -__builtin_inff(), osum = 0.0f, oS = 0.0f;
    int oc = 0, ofirst = 0x7fffffff;
    const int jy_ov = static_cast<int>(y / VEC) - ONCHIP;  // < 0: on chip
    const int iy_ov = static_cast<int>(y % VEC);
    auto online = [&](const uint4 v, int j) {
      // Word by word, as the passes below: few fp32 temporaries next to the
      // register slots already in flight.
      const auto w = words(v);
      float bm = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float f[EPW];
        D::word_fresh(w.w[q], f);
#pragma unroll
        for (int e = 0; e < EPW; ++e) bm = fmaxf(bm, f[e]);
      }
      if (bm > om) {
        osum = (osum + static_cast<float>(oc)) * __builtin_amdgcn_exp2f((om - bm) * kLog2e);
        om = bm;
        oc = 0;
        ofirst = 0x7fffffff;
      }
      const float mL = om * kLog2e;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float f[EPW];
        D::word_fresh(w.w[q], f);
#pragma unroll
        for (int e = 0; e < EPW; ++e) {
          const int i = q * EPW + e;
          const bool eq = f[e] == om;
          osum += eq ? 0.0f : exp_shifted(f[e], mL);
          oc += eq ? 1 : 0;
          if (eq) ofirst = min(ofirst, j * VEC + i);
          if constexpr (WEIGHTED) oS = __builtin_fmaf(a.weight[j * VEC + i], f[e], oS);
          else oS += f[e];
          if (j - ONCHIP == jy_ov && i == iy_ov) xy_sh = f[e];
        }
      }
    };
    // Exec-masked loads: one per-lane offset for all k, slot k in soffset.
    const int t1 = fresh_tid();
    const uint32_t vo1 = static_cast<uint32_t>(ONCHIP + t1) * 16u;
    uint4 ov[NOV];
    static_for<NOV>([&](auto k) {
      if (ov_col(k, t1) < nvec) ov[k] = buf_load16(rsrc, vo1, k * SLOT_BYTES);
    });
    // One overflow vector at a time, its column from a fresh thread id: the
    // six columns and the unpacked elements of two vectors need not be held
    // beside the 44 registers of loads in flight.
    static_for<NOV>([&](auto k) {
      const int tk = fresh_tid();
      if (ov_col(k, tk) < nvec) online(ov[k], ov_col(k, tk));
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int d = kWave / 2; d >= 1; d /= 2) {  // fixed order
      const float m2 = __shfl_xor(om, d), s2 = __shfl_xor(osum, d), S2 = __shfl_xor(oS, d);
      const int c2 = __shfl_xor(oc, d), f2 = __shfl_xor(ofirst, d);
      const float mm = fmaxf(om, m2);
      const float s1 = om == mm ? osum
                                : (osum + static_cast<float>(oc)) *
                                      __builtin_amdgcn_exp2f((om - mm) * kLog2e);
      const float s2m = m2 == mm ? s2
                                 : (s2 + static_cast<float>(c2)) *
                                       __builtin_amdgcn_exp2f((m2 - mm) * kLog2e);
      oc = (om == mm ? oc : 0) + (m2 == mm ? c2 : 0);
      ofirst = min(om == mm ? ofirst : 0x7fffffff, m2 == mm ? f2 : 0x7fffffff);
      om = mm;
      osum = s1 + s2m;
      oS += S2;
    }
    if ((tid & (kWave - 1)) == 0) {
      const int wv = tid / kWave;
      ov_m[wv] = om;
      ov_s[wv] = osum;
      ov_S[wv] = oS;
      ov_c[wv] = oc;
      ov_f[wv] = ofirst;
    }
    static_for<NOV>([&](auto k) { r[k] = buf_load16(rsrc, lane_off(k), k * SLOT_BYTES); });
  }

  // ---- pass 1: row maximum (and, with a soft-cap, each lane's largest |x|)
  // With one row per CU (and uncapped logits), passes 1 and 2 are one online
  // pass instead (ONLINE): each register slot is folded in as its load lands,
  // so the statistics' arithmetic overlaps the rest of the row's read, where
  // two passes would start only once the whole row had arrived and leave the
  // CU's memory idle while they run.  Per lane: the maximum om so far, the
  // sum osum of exp(x - om) over elements below it and the count oc at it,
  // rescaled once whenever a vector raises om (the elements then at the old
  // maximum join the sum); merged over the wavefront and the workgroup in a
  // fixed order, with the same rescaling.  (The overflow pass's scheme.)
  // Measured faster on the 24-slot shape only (rows of 20481-32768 vectors);
  // on the 16-slot one the gradient pass grew by what the statistics saved.
  constexpr bool ONLINE = !CAP && NOV == 0 && NT == 1024 && NREG >= 24;
  __shared__ float4 red_on[ONLINE ? NW : 1];
  float lane_m = -__builtin_inff();  // ONLINE: this lane's maximum
  float M_on = 0.0f;
  RowSums rs_on = {0.0f, 0.0f, 0, 0x7fffffff};
  float mx = -__builtin_inff();
  float amax = 0.0f;
  auto max_vec = [&](const uint4 v) {
    const auto w = words(v);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f[EPW];
      D::word_fresh(w.w[q], f);
#pragma unroll
      for (int e = 0; e < EPW; ++e) {
        mx = fmaxf(mx, f[e]);
        if constexpr (CAP) amax = fmaxf(amax, __builtin_fabsf(f[e]));
      }
    }
  };
  float om = -__builtin_inff(), osum = 0.0f, oS = 0.0f;
  int oc = 0;
  auto online_vec = [&](const uint4 v) {
    float f[VEC];
    D::unpack(v, f);
    float bm = f[0];
#pragma unroll
    for (int e = 1; e < VEC; ++e) bm = fmaxf(bm, f[e]);
    const float nm = fmaxf(om, bm);
    const bool up = nm > om;  // select, not branch: the lanes stay together
    const float sc = __builtin_amdgcn_exp2f((om - nm) * kLog2e);
    osum = up ? (osum + static_cast<float>(oc)) * sc : osum;
    oc = up ? 0 : oc;
    om = nm;
    const float mL = om * kLog2e;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const bool eq = f[e] == om;
      osum += eq ? 0.0f : exp_shifted(f[e], mL);
      oc += eq ? 1 : 0;
      if constexpr (!WEIGHTED) oS += f[e];  // weighted: summed in pass 3
    }
  };
  if constexpr (ONLINE) {
    // One slot at a time (the scheduler would otherwise unpack several
    // slots' elements at once beside the row's registers).
    static_for<NREG>([&](auto k) {
      if (in_row(k)) online_vec(r[k]);
      __builtin_amdgcn_sched_barrier(0);
    });
  } else {
    static_for<NREG>([&](auto k) {
      if (in_row(k)) max_vec(r[k]);
    });
  }
  if constexpr (NLDS > 0) {
    // Each lane reads back only the LDS slots its own wavefront loaded.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    static_for<NLDS>([&](auto k) {
      if (in_row(NREG + k)) {
        if constexpr (ONLINE) online_vec(xl[k * NT + tid]);
        else max_vec(xl[k * NT + tid]);
      }
      if constexpr (ONLINE) __builtin_amdgcn_sched_barrier(0);
    });
  }
  // The lane that holds column y posts x[y] to LDS (read by every wavefront
  // after the next barrier): no second load of it, and no register holding
  // it through pass 2.
  const int64_t jy = y / VEC;
  const int ky = static_cast<int>(jy / NT);  // slot and lane owning the target
  const int ty = static_cast<int>(jy % NT);
  const int iy = static_cast<int>(y % VEC);
  const bool y_chip = NOV == 0 || jy < ONCHIP;  // else posted by the overflow pass
  if (tid == ty && y_chip) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (ky < NREG) {
      static_for<NREG>([&](auto k) {
        if (k == ky) v = r[k];
      });
    } else if constexpr (NLDS > 0) {
      v = xl[(ky - NREG) * NT + ty];
    }
    float f[VEC];
    D::unpack(v, f);
    float xv = f[0];
#pragma unroll
    for (int e = 1; e < VEC; ++e)
      if (e == iy) xv = f[e];
    xy_sh = xv;
  }
  if constexpr (NOV > 0) mx = fmaxf(mx, ov_m[tid / kWave]);  // this wavefront's lane 0 wrote it
  if constexpr (ONLINE) {
    lane_m = om;
    // (maximum, sum below it, count at it, logit sum) merged over the
    // wavefront's lanes in a fixed order; every lane gets the result.
    auto merge_wave = [&](float& m, float& sm, int& c, float& S) {
#pragma unroll
      for (int d = kWave / 2; d >= 1; d /= 2) {
        const float m2 = __shfl_xor(m, d), s2 = __shfl_xor(sm, d), S2 = __shfl_xor(S, d);
        const int c2 = __shfl_xor(c, d);
        const float mm = fmaxf(m, m2);
        const float s1 = m == mm ? sm
                                 : (sm + static_cast<float>(c)) *
                                       __builtin_amdgcn_exp2f((m - mm) * kLog2e);
        const float s2m = m2 == mm ? s2
                                   : (s2 + static_cast<float>(c2)) *
                                         __builtin_amdgcn_exp2f((m2 - mm) * kLog2e);
        c = (m == mm ? c : 0) + (m2 == mm ? c2 : 0);
        m = mm;
        sm = s1 + s2m;
        S += S2;
      }
    };
    merge_wave(om, osum, oc, oS);
    if ((tid & (kWave - 1)) == 0)
      red_on[tid / kWave] = make_float4(om, osum, __int_as_float(oc), oS);
    lds_barrier();
    // The wavefronts' states: lane w of every wavefront takes wavefront w's
    // (the other lanes an empty state), merged again the same way.
    const int l = tid & (kWave - 1);
    const float4 q = red_on[l < NW ? l : 0];
    float m = l < NW ? q.x : -__builtin_inff();
    float sm = l < NW ? q.y : 0.0f;
    int c = l < NW ? __float_as_int(q.z) : 0;
    float S = l < NW ? q.w : 0.0f;
    merge_wave(m, sm, c, S);
    M_on = uniform(m);
    rs_on = {uniform(sm), uniform(S), uniform(c), 0x7fffffff};
  }
  // A wavefront whose logits all lie in the soft-cap's central range takes
  // its polynomial alone in passes 2 and 3 (no per-element choice).  fmaxf
  // drops NaN, which the polynomial turns into NaN like the general path.
  const bool central = CAP && __ballot(amax > cap.x0) == 0ull;
  const float M = ONLINE ? M_on : block_max<NT>(mx, red_max);  // of the stored logits
  // The shift of the exponents, in base-2 units, and the maximum of the logits
  // the loss reads (capped ones are read as l2(x) = log2(e) s tanh(x / s)).
  const float ML = CAP ? uniform(cap.l2(M)) : M * kLog2e;
  const float Mc = CAP ? ML * kLn2 : M;

  // ---- pass 2: sums below the maximum, ties, first index, logit sum
  RowSums rs = {0.0f, 0.0f, 0, 0x7fffffff};
  auto accumulate = [&](auto careful, auto cen, const uint4 v) {
    const auto w = words(v);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f[EPW];
      D::word_fresh(w.w[q], f);
#pragma unroll
      for (int e = 0; e < EPW; ++e) {
        // ex = exp(x - M) of the (capped) logits; fc joins the logit sum (in
        // base-2 units when capped: scaled back once per row)
        float ex, fc;
        if constexpr (!CAP) {
          fc = f[e];
          ex = exp_shifted(fc, ML);
        } else if constexpr (decltype(cen)::value) {
          const float P = cap.central_p(f[e]);  // l2(x) = x P
          ex = __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], P, -ML));
          fc = f[e] * P;
        } else {
          fc = cap.l2(f[e]);
          ex = __builtin_amdgcn_exp2f(fc - ML);
        }
        if constexpr (decltype(careful)::value) {
          const bool eq = (f[e] == M);
          rs.s += eq ? 0.0f : ex;
          rs.cnt += eq ? 1 : 0;
        } else {
          rs.s += ex;
        }
        if constexpr (!WEIGHTED) rs.S += fc;  // weighted: summed in pass 3
      }
    }
  };
  auto sum_pass = [&](auto careful, auto cen) {
    static_for<NREG>([&](auto k) {
      if (in_row(k)) accumulate(careful, cen, r[k]);
    });
    static_for<NLDS>([&](auto k) {
      if (in_row(NREG + k)) accumulate(careful, cen, xl[k * NT + tid]);
    });
  };
  // Wavefront-uniform choices: only wavefronts that hold the maximum need the
  // compare per element, and a wavefront whose logits all lie in the
  // soft-cap's central range takes the polynomial alone.
  using T_ = std::true_type;
  using F_ = std::false_type;
  if constexpr (ONLINE) {
    rs = rs_on;
  } else if (__ballot(mx == M) != 0ull) {
    if (CAP && central) sum_pass(T_{}, T_{});
    else sum_pass(T_{}, F_{});
    // The first index of M (for the accuracy output only): only lanes that
    // hold it look for it, over their own vectors from the last back to the
    // first, so the last match found is the smallest index.
    if (rs.cnt > 0 && a.acc_rows != nullptr) {
      int first = 0x7fffffff;
      auto scan = [&](const uint4 v, int k) {
        const auto w = words(v);
        const int j = k * NT + fresh_tid();
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          float f[EPW];
          D::word_fresh(w.w[q], f);
#pragma unroll
          for (int e = EPW - 1; e >= 0; --e)
            if (f[e] == M) first = j * VEC + q * EPW + e;
        }
      };
      static_for<NLDS>([&](auto kk) {
        constexpr int k = NLDS - 1 - decltype(kk)::value;
        if (in_row(NREG + k)) scan(xl[k * NT + tid], NREG + k);
      });
      static_for<NREG>([&](auto kk) {
        constexpr int k = NREG - 1 - decltype(kk)::value;
        if (in_row(k)) scan(r[k], k);
      });
      rs.first = first;
    }
  } else {
    if (CAP && central) sum_pass(F_{}, T_{});
    else sum_pass(F_{}, F_{});
  }
  if constexpr (NOV > 0) {  // the wavefront's overflow share, at the row maximum, on lane 0
    if ((tid & (kWave - 1)) == 0) {
      const int wv = tid / kWave;
      const float om = ov_m[wv];
      if (om == M) {
        rs.s += ov_s[wv];
        rs.cnt += ov_c[wv];
        rs.first = min(rs.first, ov_f[wv]);
      } else {
        rs.s += (ov_s[wv] + static_cast<float>(ov_c[wv])) *
                __builtin_amdgcn_exp2f((om - M) * kLog2e);
      }
      rs.S += ov_S[wv];
    }
  }
  if constexpr (ONLINE) {
    // The first index of M (for the accuracy output only), by the lanes that
    // hold it, as pass 2 finds it.
    if (a.acc_rows != nullptr) {
      int first = 0x7fffffff;
      if (lane_m == M) {
        auto scan = [&](const uint4 v, int k) {
          const auto w = words(v);
          const int j = k * NT + fresh_tid();
#pragma unroll
          for (int q = 3; q >= 0; --q) {
            float f[EPW];
            D::word_fresh(w.w[q], f);
#pragma unroll
            for (int e = EPW - 1; e >= 0; --e)
              if (f[e] == M) first = j * VEC + q * EPW + e;
          }
        };
        static_for<NLDS>([&](auto kk) {
          constexpr int k = NLDS - 1 - decltype(kk)::value;
          if (in_row(NREG + k)) scan(xl[k * NT + tid], NREG + k);
        });
        static_for<NREG>([&](auto kk) {
          constexpr int k = NREG - 1 - decltype(kk)::value;
          if (in_row(k)) scan(r[k], k);
        });
      }
      rs.first = block_sums<NT>(RowSums{0.0f, 0.0f, 0, first}, red_sum).first;
    }
  } else {
    rs = block_sums<NT>(rs, red_sum);
  }

  const float dp = rs.s + static_cast<float>(rs.cnt - 1);  // d' = d - 1
  // What only the row's end needs (normalizers, outputs, z-loss) is read from
  // the arguments here rather than held in registers since the kernel began.
  const RowArgs& a0 = a;
  const RowArgs ra = fresh_args<RowArgs>();
  {
  const RowArgs& a = ra;
  const float xy_stored = uniform(xy_sh);  // posted before the pass-1 barrier
  float xy = xy_stored, slope_y = 1.0f;
  if constexpr (CAP) {
    xy = uniform(cap.l2(xy_stored, slope_y)) * kLn2;
    slope_y = uniform(slope_y);
    rs.S *= kLn2;  // the capped logit sum, summed in base-2 units
  }
  const float sum_w = uniform(static_cast<float>(a.ws->sum_w));
  const float wy = uniform(WEIGHTED ? a.weight[y] : 1.0f);
  const float lg = uniform(log1pf(dp));  // lse - m, once per row
  // The row's outputs.  With class weights the logit sum S = sum w x is
  // taken in pass 3, which loads every weight anyway (the weights are read
  // once per row instead of twice): the loss is first written without its
  // -eta S term, which pass 3's end subtracts.
  float l0 = 0.0f;
  if constexpr (WEIGHTED) {
    l0 = uniform(row_loss(Mc, lg, xy, 0.0f, wy, sum_w, a.eps, a.eta) + row_z(Mc, lg, a.zl));
  }
  if (tid == 0) {
    const float zrow = row_z(Mc, lg, a.zl);
    store_row(a, n, WEIGHTED ? l0 : row_loss(Mc, lg, xy, rs.S, wy, sum_w, a.eps, a.eta) + zrow,
              (static_cast<int64_t>(rs.first) == y) ? 1.0f : 0.0f, zrow);
  }

  // ---- pass 3: gradient over the on-chip row, one store per vector
  const float sigma = uniform(a.mean ? a.ws->inv_W : 1.0f);
  RowTerms t = row_terms(Mc, dp, lg, xy, wy, sum_w, a.eps, a.eta, sigma, a.zl, z_sigma(a));
  if constexpr (CAP) {
    t.dxy *= slope_y;  // the owner stores the finished value
    t.ML = ML;         // the shift pass 2 took, in base-2 units
  }
  t.ML = uniform(t.ML);
  t.K = uniform(t.K);
  t.B = uniform(t.B);
  t.dxy = uniform(t.dxy);
  float Sw = 0.0f;  // this thread's share of sum w x (class weights)
  // The class weights of a vector's VEC columns: 16 bytes (4 weights) per
  // load, through a buffer resource over the weights (kept in L2: every row
  // reads them).
  const auto wrsrc = make_rsrc(a.weight, WEIGHTED ? static_cast<uint32_t>(a.V * 4) : 0u);
  constexpr int NWV = WEIGHTED ? VEC / 4 : 1;
  auto grad_vec = [&](auto cen, const uint4 v, int k) {
    auto w = words(v);
    uint4 wv[NWV];  // weights of vector j = k NT + tid: columns j VEC .. j VEC + VEC - 1
    if constexpr (WEIGHTED) {
      static_for<NWV>([&](auto h) {
        wv[h] = buf_load16_cached(wrsrc, static_cast<uint32_t>(tid) * (VEC * 4u) + h * 16u,
                                  static_cast<uint32_t>(k) * (NT * VEC * 4u));
      });
    }
    auto weight_of = [&](int i) {  // the weight of column j VEC + i, i < VEC
      const uint4 q4 = wv[i / 4];
      const int c = i % 4;
      return __uint_as_float(c == 0 ? q4.x : c == 1 ? q4.y : c == 2 ? q4.z : q4.w);
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f[EPW];
      D::word_fresh(w.w[q], f);
#pragma unroll
      for (int e = 0; e < EPW; ++e) {
        const float wc = WEIGHTED ? weight_of(q * EPW + e) : 1.0f;
        const float b = WEIGHTED ? t.B * wc : t.B;
        if constexpr (CAP) {
          float slope;
          const float xl =
              decltype(cen)::value ? cap.central_l2(f[e], slope) : cap.l2(f[e], slope);
          if constexpr (WEIGHTED) Sw = __builtin_fmaf(wc, xl, Sw);  // base-2 units
          f[e] = __builtin_fmaf(__builtin_amdgcn_exp2f(xl - t.ML), t.K, -b) * slope;
        } else {
          if constexpr (WEIGHTED) Sw = __builtin_fmaf(wc, f[e], Sw);
          f[e] = __builtin_fmaf(exp_shifted(f[e], t.ML), t.K, -b);
        }
      }
      w.w[q] = D::pack_word(f);  // the result word replaces the input word
    }
    if (k == ky && tid == ty && y_chip) {
      // The owner of the target column writes the fp32 true-class value,
      // rounded once, in place of its softmax term.
      float f[EPW];
      const int q = iy / EPW;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        if (qq == q) {
          D::word_fresh(w.w[qq], f);
#pragma unroll
          for (int e = 0; e < EPW; ++e)
            if (qq * EPW + e == iy) f[e] = t.dxy;
          w.w[qq] = D::pack_word(f);
        }
      }
    }
    buf_store16(rsrc, voff, static_cast<uint32_t>(k) * SLOT_BYTES,
                make_uint4(w.w[0], w.w[1], w.w[2], w.w[3]));
  };
  auto grad_pass = [&](auto cen) {
    static_for<NREG>([&](auto k) {
      if (in_row(k)) grad_vec(cen, r[k], k);
    });
    static_for<NLDS>([&](auto k) {
      if (in_row(NREG + k)) grad_vec(cen, xl[k * NT + tid], NREG + k);
    });
  };
  if (CAP && central) grad_pass(std::true_type{});
  else grad_pass(std::false_type{});
  if constexpr (WEIGHTED) {  // summed in the order pass 2 sums the unweighted S
    const RowSums sw = block_sums<NT>(RowSums{0.0f, Sw, 0, 0x7fffffff}, red_sum3);
    if (tid == 0 && a.eps > 0.0f) {
      const float l = l0 - a.eta * (CAP ? sw.S * kLn2 : sw.S);
      a.loss_rows[n] = l;
      if (a.loss_rows2) a.loss_rows2[n] = l;
    }
  }
  // The overflow (unweighted rows only) is read again after the on-chip
  // row's stores, and its gradient is written last.
  if constexpr (NOV > 0) {
    const int t3 = fresh_tid();
    const uint32_t vo3 = static_cast<uint32_t>(ONCHIP + t3) * 16u;
    uint4 ov2[NOV];
    static_for<NOV>([&](auto q) {
      if (ov_col(q, t3) < nvec) ov2[q] = buf_load16(rsrc, vo3, q * SLOT_BYTES);
    });
    static_for<NOV>([&](auto q) {
      const int j = ov_col(q, t3);
      if (j >= nvec) return;
      auto w = words(ov2[q]);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        float f[EPW];
        D::word_fresh(w.w[qq], f);
#pragma unroll
        for (int e = 0; e < EPW; ++e) {
          const float b = WEIGHTED ? t.B * a.weight[j * VEC + qq * EPW + e] : t.B;
          f[e] = __builtin_fmaf(exp_shifted(f[e], t.ML), t.K, -b);
          if (static_cast<int64_t>(j) * VEC + qq * EPW + e == y) f[e] = t.dxy;
        }
        w.w[qq] = D::pack_word(f);
      }
      buf_store16(rsrc, vo3, q * SLOT_BYTES, make_uint4(w.w[0], w.w[1], w.w[2], w.w[3]));
    });
  }
  }
  (void)a0;
}

// Shapes of the resident kernel: threads per workgroup, vectors per thread in
// registers and in LDS, and the minimum wavefronts per SIMD to compile for
// (which caps the registers per wavefront at 512 / WPE).
template <int NT_, int NREG_, int NLDS_, int WPE_, int LDS_CAP_ = NT_ * NLDS_, int NOV_ = 0>
struct Shape {
  static constexpr int NT = NT_, NREG = NREG_, NLDS = NLDS_, WPE = WPE_, LDS_CAP = LDS_CAP_;
  static constexpr int NOV = NOV_;
  static constexpr int64_t CAPACITY = static_cast<int64_t>(NT_) * (NREG_ + NOV_) + LDS_CAP_;
};

using Shapes = std::tuple<Shape<64, 4, 0, 4>,       // rows up to 256 vectors
                          Shape<256, 8, 0, 4>,      // 2048 vectors
                          // 4096 vectors (bf16 V <= 32768): 512 threads at 8
                          // waves per SIMD, 1-3% ahead of 256 threads x 16
                          // vectors at V = 32000
                          Shape<512, 8, 0, 8>,
                          Shape<512, 16, 0, 4>,     // 8192 vectors
                          // 16320 vectors (bf16 V <= 130560): 2 workgroups per CU,
                          // 64 VGPRs and 79 KB of LDS each
                          Shape<1024, 11, 5, 8, 5056>,
                          // the same with an overflow read twice (uncapped,
                          // unweighted rows): 19392 / 22464 vectors (bf16 V
                          // <= 155136 / 179712).  Past about a third of the
                          // row in the overflow, one row per CU is faster.
                          Shape<1024, 11, 5, 8, 5056, 3>,
                          Shape<1024, 11, 5, 8, 5056, 6>,
                          Shape<1024, 16, 4, 4>,    // 20480 vectors
                          Shape<1024, 24, 8, 4>>;   // 32768 vectors

template <int DT, bool W, bool CAP, class SH>
int launch_shape(const Prob& p, const RowArgs& a, hipStream_t s) {
  if (p.rows <= 0) return VSCE_OK;
  hipLaunchKernelGGL(
      (fused_resident_kernel<DT, SH::NT, SH::NREG, SH::NLDS, SH::LDS_CAP, SH::NOV, W, CAP,
                             SH::WPE>),
                     dim3(static_cast<unsigned>(p.rows)), dim3(SH::NT), 0, s, a);
  return hipGetLastError() == hipSuccess ? VSCE_OK : VSCE_ERR_LAUNCH;
}

template <int DT, bool W, bool CAP, size_t I = 0>
int pick_shape(const Prob& p, const RowArgs& a, hipStream_t s) {
  if constexpr (I == std::tuple_size<Shapes>::value) {
    return VSCE_ERR_UNSUPPORTED;
  } else {
    using SH = std::tuple_element_t<I, Shapes>;
    if constexpr ((CAP || W) && SH::NOV > 0) {  // overflow: uncapped, unweighted rows
      return pick_shape<DT, W, CAP, I + 1>(p, a, s);
    } else {
      if (a.nvec <= SH::CAPACITY) return launch_shape<DT, W, CAP, SH>(p, a, s);
    }
    return pick_shape<DT, W, CAP, I + 1>(p, a, s);
  }
}

}  // namespace

template <int DT, bool CAP>
int fused_resident_dt(const Prob& p, const RowArgs& a, hipStream_t s) {
  return p.weight ? pick_shape<DT, true, CAP>(p, a, s) : pick_shape<DT, false, CAP>(p, a, s);
}

}  // namespace vsce
