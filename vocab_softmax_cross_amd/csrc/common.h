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
constexpr int kWave = 64;

// Workspace header; field offsets are part of the C ABI (VSCE_WS_*).
struct WsHeader {
  double W;           // target-weight sum over valid rows
  double sum_w;       // class-weight sum over the vocabulary
  int64_t n_valid;    // rows with a target in [0, V)
  int64_t n_invalid;  // rows with a target neither ignore_index nor in [0, V)
  uint32_t status;    // VSCE_STATUS_* bits
  uint32_t pad0;
};
static_assert(offsetof(WsHeader, W) == VSCE_WS_W, "header layout");
static_assert(offsetof(WsHeader, sum_w) == VSCE_WS_SUM_W, "header layout");
static_assert(offsetof(WsHeader, n_valid) == VSCE_WS_N_VALID, "header layout");
static_assert(offsetof(WsHeader, n_invalid) == VSCE_WS_N_INVALID, "header layout");
static_assert(offsetof(WsHeader, status) == VSCE_WS_STATUS, "header layout");

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
// 16 bytes per lane straight into LDS; lane i of the wavefront lands at
// lds_wave + 16 i, so `lds_wave` must be the same for the whole wavefront.
__device__ inline void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_wave, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave,
                                           16, voff, soff, 0, kNT);
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

// Hides a register-held vector from the optimizer so that a pass over the
// row unpacks it again instead of keeping the previous pass's fp32 copies
// alive (which would double the registers a resident row needs).
__device__ inline void opaque(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// exp(x - m) as 2^(x*log2e - m*log2e) on the hardware base-2 exponential.
__device__ inline float exp_shifted(float x, float m_log2e) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -m_log2e));
}

// ---------------------------------------------------------------- reductions

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline int wave_min(int v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// Workgroup max over NT threads; every thread gets the result.  `sh` holds
// NT/64 floats and is not reused until the next barrier.
template <int NT>
__device__ inline float block_max(float v, float* sh) {
  constexpr int NW = NT / kWave;
  v = wave_max(v);
  if (NW == 1) return v;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, sh[w]);
  return r;
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
__device__ inline RowSums block_sums(RowSums v, float4* sh) {
  constexpr int NW = NT / kWave;
  v.s = wave_sum(v.s);
  v.S = wave_sum(v.S);
  v.cnt = wave_sum(v.cnt);
  v.first = wave_min(v.first);
  if (NW == 1) return v;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0)
    sh[wave] = make_float4(v.s, v.S, __int_as_float(v.cnt), __int_as_float(v.first));
  __syncthreads();
  RowSums r = {0.f, 0.f, 0, 0x7fffffff};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float4 q = sh[w];
    r.s += q.x;
    r.S += q.y;
    r.cnt += __float_as_int(q.z);
    r.first = min(r.first, __float_as_int(q.w));
  }
  return r;
}

}  // namespace vsce
