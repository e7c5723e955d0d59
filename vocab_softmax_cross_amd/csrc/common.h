// Device-side building blocks shared by the cross-entropy kernels (gfx950).
//
// Element types, 16-byte vector pack/unpack, the workspace header, and
// wavefront / workgroup reductions.  Nothing here is specific to one kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "vsce.h"

namespace vsce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWave = 64;

// Workspace header; field offsets are part of the C ABI (VSCE_WS_*).
struct WsHeader {
  double W;           // target-weight sum over valid rows
  double sum_w;       // class-weight sum over the vocabulary
  int64_t n_valid;    // rows with a target in [0, V)
  int64_t n_invalid;  // rows with a target neither ignore_index nor in [0, V)
  uint32_t status;    // VSCE_STATUS_* bits
  uint32_t pad0;
  float inv_W;        // 1 / W in fp32 (the mean's gradient scale)
  float inv_n_valid;  // 1 / n_valid in fp32 (the mean's z-loss gradient scale)
};
static_assert(offsetof(WsHeader, W) == VSCE_WS_W, "header layout");
static_assert(offsetof(WsHeader, sum_w) == VSCE_WS_SUM_W, "header layout");
static_assert(offsetof(WsHeader, n_valid) == VSCE_WS_N_VALID, "header layout");
static_assert(offsetof(WsHeader, n_invalid) == VSCE_WS_N_INVALID, "header layout");
static_assert(offsetof(WsHeader, status) == VSCE_WS_STATUS, "header layout");
static_assert(offsetof(WsHeader, inv_W) == VSCE_WS_INV_W, "header layout");
static_assert(offsetof(WsHeader, inv_n_valid) == VSCE_WS_INV_N_VALID, "header layout");
static_assert(sizeof(WsHeader) <= VSCE_WS_HEADER_BYTES, "header layout");

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Element type traits.  VEC = elements per 16-byte vector.
template <int DT>
struct Dt;

template <>
struct Dt<VSCE_F32> {
  static constexpr int VEC = 4;
  static constexpr int BYTES = 4;
  __device__ static inline void unpack(const uint4 v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  // one 32-bit word = EPW elements
  static constexpr int EPW = 1;
  __device__ static inline void word_fresh(uint32_t w, float (&f)[1]) { f[0] = __uint_as_float(w); }
  __device__ static inline uint32_t pack_word(const float (&f)[1]) { return __float_as_uint(f[0]); }
  __device__ static inline uint4 pack(const float (&f)[4]) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
  __device__ static inline float load1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static inline void store1(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};

// bf16 -> fp32 is exact: the 16 bits become the high half of the fp32 word.
// fp32 -> bf16 rounds to nearest even with gfx950's v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <>
struct Dt<VSCE_BF16> {
  static constexpr int VEC = 8;
  static constexpr int BYTES = 2;
  __device__ static inline void unpack(const uint4 v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  // The same conversion of one 32-bit word as volatile asm: each pass over a
  // register-held row unpacks again instead of the compiler keeping the fp32
  // copies of an earlier pass alive, which would double the registers the
  // row needs.
  static constexpr int EPW = 2;
  __device__ static inline void word_fresh(uint32_t w, float (&f)[2]) {
    uint32_t lo, hi;
    asm volatile("v_lshlrev_b32 %0, 16, %2\n\tv_and_b32 %1, 0xffff0000, %2"
                 : "=&v"(lo), "=v"(hi)
                 : "v"(w));
    f[0] = __uint_as_float(lo);
    f[1] = __uint_as_float(hi);
  }
  __device__ static inline uint32_t pack_word(const float (&f)[2]) {
    return pack_bf16x2(f[0], f[1]);
  }
  __device__ static inline uint4 pack(const float (&f)[8]) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
  __device__ static inline float load1(const void* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  __device__ static inline void store1(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xffffu);
  }
};

// fp16 <-> fp32 with the hardware converts (round to nearest even, fp16
// subnormals kept).
__device__ inline uint32_t pack_f16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

template <>
struct Dt<VSCE_F16> {
  static constexpr int VEC = 8;
  static constexpr int BYTES = 2;
  __device__ static inline void unpack(const uint4 v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2_t h = __builtin_bit_cast(f16x2_t, w[i]);
      f[2 * i] = static_cast<float>(h[0]);
      f[2 * i + 1] = static_cast<float>(h[1]);
    }
  }
  // Volatile-asm conversion of one word (see Dt<VSCE_BF16>::word_fresh).
  static constexpr int EPW = 2;
  __device__ static inline void word_fresh(uint32_t w, float (&f)[2]) {
    float lo, hi;
    asm volatile(
        "v_cvt_f32_f16 %0, %2\n\t"
        "v_cvt_f32_f16_sdwa %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1"
        : "=&v"(lo), "=v"(hi)
        : "v"(w));
    f[0] = lo;
    f[1] = hi;
  }
  __device__ static inline uint32_t pack_word(const float (&f)[2]) {
    return pack_f16x2(f[0], f[1]);
  }
  __device__ static inline uint4 pack(const float (&f)[8]) {
    return make_uint4(pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]), pack_f16x2(f[4], f[5]),
                      pack_f16x2(f[6], f[7]));
  }
  __device__ static inline float load1(const void* p, int64_t i) {
    return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  }
  __device__ static inline void store1(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(pack_f16x2(v, 0.0f) & 0xffffu);
  }
};

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1, so
// that register arrays indexed by I stay in registers.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A workgroup barrier that orders LDS only: each wavefront waits for its own
// LDS operations, not for its global stores to complete (which a full
// __syncthreads() would, and which a kernel that streams its output need
// never wait for).  For exchanges through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// threadIdx.x passed through an empty asm: in a loop, what is derived from
// it per lane (masks, LDS addresses) is then rebuilt where it is used instead
// of being held in registers across the whole loop.
__device__ __forceinline__ int fresh_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// A kernel's single by-value argument, read again from the kernel-argument
// segment (where it sits at offset 0).  The segment pointer goes through an
// empty asm, so the fields are loaded (scalar loads) where they are used
// after that point, instead of being loaded at kernel entry and held in
// scalar registers through the whole kernel.
template <class T>
__device__ __forceinline__ T fresh_args() {
#if defined(__HIP_DEVICE_COMPILE__)
  using KT = const __attribute__((address_space(4))) T;
  KT* p = __builtin_bit_cast(KT*, __builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(p));
  return *p;
#else  // the host pass only parses device code
  return T{};
#endif
}

// ---------------------------------------------------------------- soft-capping
// Logit soft-capping x -> s tanh(x / s) and its slope 1 - tanh^2(x / s), each
// with a relative error of a few units of 2^-24 for every x (u = x / s).  The
// kernels read the capped logit in base-2 units, l2(x) = log2(e) s tanh(u),
// since every use is an exponent of 2 (or a sum that is scaled back once).
//
// Central range |u| <= kCapCentral: tanh(u) / u = 1 + w Q(w), w = u^2, with Q
// the quadratic that minimizes the largest relative error of 1 + w Q(w) on
// that range (Remez exchange: 0.68 units of 2^-24).  So
//   l2(x) = x P,  P = log2(e) (1 + w Q(w)) = P0 + P1 w + P2 w^2 + P3 w^3
// (the constants below), evaluated in x^2 itself:
//   P = D0 + D1 x^2 + D2 x^4 + D3 x^6,  Di = Pi / s^(2i),
// the Di taken once per launch in fp64 and rounded to fp32, so that an element
// costs x^2 and three fused multiply-adds.  The slope is 1 - t^2 with
// t = l2(x) / (log2(e) s) (t <= 0.34: nothing cancels).  In fp32 (emulated on
// the host, one rounding per operation) on a grid of 2e5 points per cap, caps
// 1 to 1e3: at most 2.6 units for the capped logit and 1.3 for the slope.  No
// exp and no reciprocal; at a cap of 30 the range holds every |x| <= 10.5.
//
// Outside it, from q = exp(-2 |u|), taken as q4 = 4 q = 2^(-2 |x| log2(e) / s + 2):
//   s tanh(|u|) = (s - (s / 4) q4) r,   slope = q4 r^2,   r = 1 / (1 + q4 / 4),
// a relative error of at most about 5 units for the value (at the range's
// edge, where 1 - q cancels a little) and about 4 |u| + 5 for the slope (the
// exponent argument's own rounding, scaled by its size, dominates far out).
//
// l2(x) and central_l2(x) give the same bits for a central x, so the
// statistics pass and the gradient pass see the same capped logits whichever
// form each takes.  A NaN logit stays NaN; +-inf caps to +-s with slope 0.
constexpr float kCapCentral = 0.35f;
constexpr double kCapP0 = 1.4426950408889634;     // log2(e)
constexpr double kCapP1 = -0.48088867846443684;
constexpr double kCapP2 = 0.19187592127303182;
constexpr double kCapP3 = -0.07090630044946303;

struct SoftCap {
  float s;      // the cap, > 0
  float k;      // -2 log2(e) / s
  float ct;     // 1 / (log2(e) s): t = l2(x) ct
  float x0;     // kCapCentral * s: where the central range ends
  float qs;     // -s / 4
  // P's coefficients D0..D3 in x^2, passed as kernel arguments: each Horner
  // step then reads one scalar register instead of a constant copied into a
  // vector register.
  float c0, c1, c2, c3;

  // P for a central x, as a polynomial in x^2: l2(x) = x P.
  __device__ __forceinline__ float central_p(float x) const {
    const float w = x * x;
    const float q = __builtin_fmaf(w, c3, c2);
    return __builtin_fmaf(__builtin_fmaf(q, w, c1), w, c0);
  }
  // The central range's formulas alone: for |x| <= x0 (a caller that knows
  // every logit it passes lies there; NaN gives NaN).
  __device__ __forceinline__ float central_l2(float x, float& slope) const {
    const float xl = x * central_p(x);
    const float t = xl * ct;
    slope = __builtin_fmaf(-t, t, 1.0f);
    return xl;
  }
  __device__ __forceinline__ float central_l2(float x) const { return x * central_p(x); }
  // Any x, in base-2 units: both forms, then a select (no branch per
  // element: the exec-mask juggling of one costs registers the resident row
  // needs).
  __device__ __forceinline__ float l2(float x, float& slope) const {
    float sc;
    const float xc = central_l2(x, sc);
    const float q4 = __builtin_amdgcn_exp2f(__builtin_fmaf(__builtin_fabsf(x), k, 2.0f));
    const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(q4, 0.25f, 1.0f));
    const bool c = __builtin_fabsf(x) <= x0;
    slope = c ? sc : q4 * r * r;
    return c ? xc : __builtin_copysignf(__builtin_fmaf(qs, q4, s) * r, x) * kLog2e;
  }
  __device__ __forceinline__ float l2(float x) const {
    const float xc = central_l2(x);
    const float q4 = __builtin_amdgcn_exp2f(__builtin_fmaf(__builtin_fabsf(x), k, 2.0f));
    const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(q4, 0.25f, 1.0f));
    const float xr = __builtin_copysignf(__builtin_fmaf(qs, q4, s) * r, x) * kLog2e;
    return __builtin_fabsf(x) <= x0 ? xc : xr;
  }
  // The capped logit s tanh(x / s) itself (for per-row values: the maximum,
  // the target logit, the statistics).
  __device__ __forceinline__ float value(float x) const {
    if (__builtin_fabsf(x) <= x0) return central_l2(x) * kLn2;
    const float q4 = __builtin_amdgcn_exp2f(__builtin_fmaf(__builtin_fabsf(x), k, 2.0f));
    const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(q4, 0.25f, 1.0f));
    return __builtin_copysignf(__builtin_fmaf(qs, q4, s) * r, x);
  }
  __device__ __forceinline__ float value(float x, float& slope) const {
    float xt = central_l2(x, slope) * kLn2;
    if (!(__builtin_fabsf(x) <= x0)) {
      const float q4 = __builtin_amdgcn_exp2f(__builtin_fmaf(__builtin_fabsf(x), k, 2.0f));
      const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(q4, 0.25f, 1.0f));
      slope = q4 * r * r;
      xt = __builtin_copysignf(__builtin_fmaf(qs, q4, s) * r, x);
    }
    return xt;
  }
};

// The soft-cap of a kernel's arguments (its field cap_c: the constants of
// a SoftCap, filled on the host by soft_cap_constants()).
template <class Args>
__device__ __forceinline__ SoftCap soft_cap(const Args& a) {
  return a.cap_c;
}

// ---------------------------------------------------------------- XCD-aware order
// The chip hands consecutive workgroups of a launch to its 8 XCDs in turn
// (workgroup b runs on XCD b mod 8), and each XCD has its own L2 and its own
// address-translation caches.  xcd_contiguous() renumbers a one-item-per-
// workgroup grid so that the workgroups one XCD runs take one contiguous range
// of items: the rows an XCD has in flight then lie side by side in memory
// instead of every 8th row of a window 8 times wider.  It is a bijection on
// [0, items) for every items (XCD x takes items/8 items, one more if x is
// below items mod 8), so results never depend on the dispatch order; only the
// speed does.
constexpr int64_t kXcds = 8;

__device__ __forceinline__ int64_t xcd_contiguous(int64_t b, int64_t items) {
  const int64_t q = items / kXcds, r = items % kXcds;
  const int64_t x = b % kXcds;
  return x * q + (x < r ? x : r) + b / kXcds;
}

// ---------------------------------------------------------------- buffer access
// A buffer resource covers one row: a 32-bit byte offset per lane (VGPR) plus
// a per-instruction constant (SGPR), and lanes past num_records read zeros and
// drop their stores instead of touching memory outside the row.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer (gfx9 data format)
// A per-lane byte offset past any row this library addresses (rows are
// < 2^31 bytes): loads from it return zeros and stores to it are dropped.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}
// Cache policy of the logits and gradient streams: non-temporal (the "nt"
// bit), since every byte is touched once per pass and the tensors are far
// larger than the caches.
constexpr int kNT = 2;

__device__ inline uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                   const uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, soff, kNT);
}
// 16 bytes per lane with the default cache policy: data that every row
// reads again (class weights), kept in L2.
__device__ inline uint4 buf_load16_cached(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                          uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 16 bytes per lane straight into LDS; lane i of the wavefront lands at
// lds_wave + 16 i, so `lds_wave` must be the same for the whole wavefront.
// POLICY: kNT for a stream read once; 0 (default) for data other workgroups
// read again.
template <int POLICY = kNT>
__device__ inline void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_wave, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave,
                                           16, voff, soff, 0, POLICY);
}

// Waits until at most N vector-memory operations of this wavefront are still
// outstanding.  The counter covers loads (those into LDS too) and stores, and
// they leave it in the order they were issued.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "the counter holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Plain-pointer 16-byte loads and stores with the same non-temporal policy.
__device__ inline uint4 nt_load16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void nt_store16(void* p, const uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, static_cast<u32x4_t*>(p));
}

// exp(x - m) as 2^(x*log2e - m*log2e) on the hardware base-2 exponential.
__device__ inline float exp_shifted(float x, float m_log2e) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -m_log2e));
}

// ---------------------------------------------------------------- reductions
// Wavefront all-reduce on the DPP crossbar: within each row of 16 lanes in
// four steps (swap neighbours, swap pairs, mirror halves, mirror the row),
// then the four row results are read into scalar registers and combined.
// Fixed order, so the result does not depend on scheduling.

template <int CTRL>
__device__ inline int dpp_mov(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppSwap1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

template <class Op>
__device__ inline float wave_reduce(float v, Op op) {
  v = op(v, __int_as_float(dpp_mov<kDppSwap1>(__float_as_int(v))));
  v = op(v, __int_as_float(dpp_mov<kDppSwap2>(__float_as_int(v))));
  v = op(v, __int_as_float(dpp_mov<kDppHalfMirror>(__float_as_int(v))));
  v = op(v, __int_as_float(dpp_mov<kDppMirror>(__float_as_int(v))));
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return op(op(r0, r1), op(r2, r3));
}

template <class Op>
__device__ inline int wave_reduce(int v, Op op) {
  v = op(v, dpp_mov<kDppSwap1>(v));
  v = op(v, dpp_mov<kDppSwap2>(v));
  v = op(v, dpp_mov<kDppHalfMirror>(v));
  v = op(v, dpp_mov<kDppMirror>(v));
  const int r0 = __builtin_amdgcn_readlane(v, 0);
  const int r1 = __builtin_amdgcn_readlane(v, 16);
  const int r2 = __builtin_amdgcn_readlane(v, 32);
  const int r3 = __builtin_amdgcn_readlane(v, 48);
  return op(op(r0, r1), op(r2, r3));
}

__device__ inline float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

__device__ inline float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

__device__ inline int wave_sum(int v) {
  return wave_reduce(v, [](int a, int b) { return a + b; });
}

__device__ inline int wave_min(int v) {
  return wave_reduce(v, [](int a, int b) { return min(a, b); });
}

// fp64 sums (the single-workgroup normalizer and reduction kernels only).
__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// A value every lane of the wavefront holds, moved to a scalar register (it
// frees a vector register for the resident row).
__device__ inline float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup max over NT threads; every thread gets the result.  `sh` holds
// NT/64 floats and is not reused until the next barrier.
template <int NT>
__device__ inline float block_max(float v, float* sh, int t = fresh_tid()) {
  constexpr int NW = NT / kWave;
  v = wave_max(v);
  if (NW == 1) return v;
  const int lane = t & (kWave - 1), wave = uniform(t / kWave);
  if (lane == 0) sh[wave] = v;
  lds_barrier();
  float r = sh[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, sh[w]);
  return uniform(r);
}

// The per-row sums merged once the row maximum is known: the sum of the
// exponentials with every element equal to the maximum left out, the number
// of such elements, the (weighted) logit sum, and the first index of the
// maximum.  Summed over lanes in a fixed order.
struct RowSums {
  float s;    // sum of exp(x - M) over elements below M
  float S;    // sum of w[c] x[c]
  int cnt;    // elements equal to M
  int first;  // first index of M (INT32_MAX if none seen)
};

template <int NT>
__device__ inline RowSums block_sums(RowSums v, float4* sh, int t = fresh_tid()) {
  constexpr int NW = NT / kWave;
  v.s = wave_sum(v.s);
  v.S = wave_sum(v.S);
  v.cnt = wave_sum(v.cnt);
  v.first = wave_min(v.first);
  if (NW == 1) return v;
  const int lane = t & (kWave - 1), wave = uniform(t / kWave);
  if (lane == 0)
    sh[wave] = make_float4(v.s, v.S, __int_as_float(v.cnt), __int_as_float(v.first));
  lds_barrier();
  RowSums r = {0.f, 0.f, 0, 0x7fffffff};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float4 q = sh[w];
    r.s += q.x;
    r.S += q.y;
    r.cnt += __float_as_int(q.z);
    r.first = min(r.first, __float_as_int(q.w));
  }
  r.s = uniform(r.s);
  r.S = uniform(r.S);
  r.cnt = uniform(r.cnt);
  r.first = uniform(r.first);
  return r;
}

}  // namespace vsce
