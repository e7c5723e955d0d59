// bf16 GEMM on the gfx950 matrix cores, C[m, n] = sum_k A[m, k] B[n, k], for
// the projection products of the linear head fused with the cross-entropy
// (Liger-Kernel PR #1622, FLCE: logits = h W^T, dL/dh = G W, dL/dW = G^T h,
// each arranged so that both operands are contiguous along k).
//
// One workgroup of 256 threads computes a 128 x 128 tile of C.  Its four
// wavefronts each own a 64 x 64 quarter, as 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  k advances 64 at a time
// through two LDS stages of A and B (16 KB each): the next stage is loaded
// straight into LDS (buffer_load_dwordx4 ... lds) while the current one is
// multiplied.  In LDS each tile row is 8 chunks of 16 bytes, the chunk
// index XOR-ed with the row (mod 8), so that the 32 rows one MFMA operand
// reads sit in different banks; the swizzle is applied by choosing which
// global chunk each lane loads, since a direct-to-LDS load writes lane i at
// base + 16 i.
//
// Operand lane layout of the 32x32x16 bf16 MFMA (checked on the hardware):
// lane l supplies row l mod 32 and the 8 k-values 8 (l / 32) .. + 7 of each
// operand; result element i of lane l is (row 8 (i / 4) + 4 (l / 32) + i mod 4,
// column l mod 32).  B goes in as the first operand and A as the second, so
// the result's rows are n and its columns m: each lane then holds 4
// consecutive n of one m, stored as one 8-byte (bf16) or 16-byte (fp32) write.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "launch.h"

namespace vsce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int kChunks = BM * BK * 2 / 16;  // 16-byte chunks per operand stage (1024)
static_assert(BM == BN, "A and B stages share one layout");

// LDS chunk of (row, 16-byte k-chunk kc) in a stage.
__device__ __forceinline__ int swz(int row, int kc) { return row * 8 + (kc ^ (row & 7)); }

// A stage is read with ordinary LDS loads (the compiler places their waits
// and the MFMA register hazards); the direct-to-LDS loads that fill it are
// waited for by hand (wait_vm) and published to the workgroup by barrier().
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 as_bf16(const u32x4_t v) { return __builtin_bit_cast(bf16x8, v); }

// Tile (tm, tn) of linear tile index t: groups of group_m m-tiles by all
// n-tiles, m fastest inside a group (tile indices are first made contiguous
// per XCD, so one XCD works on neighbouring tiles and shares their panels in
// its L2).
__device__ __forceinline__ void tile_of(int64_t t, int tiles_m, int tiles_n, int group_m, int& tm,
                                        int& tn) {
  const int64_t per_group = static_cast<int64_t>(group_m) * tiles_n;
  const int grp = static_cast<int>(t / per_group);
  const int first = grp * group_m;
  const int gm = min(group_m, tiles_m - first);
  const int in = static_cast<int>(t - grp * per_group);
  tm = first + in % gm;
  tn = in / gm;
}

template <int OUT>
__global__ __launch_bounds__(NT, 2) void gemm_nt_kernel(const GemmArgs g) {
  __shared__ uint4 lds[2][2][kChunks];  // [stage][A, B][chunk]: 64 KB
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = uniform(tid / kWave);
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  tile_of(xcd_contiguous(blockIdx.x, static_cast<int64_t>(tiles_m) * tiles_n), tiles_m, tiles_n,
          g.group_m, tm, tn);
  const int m_eff = g.m_count ? min(max(*g.m_count, 0), g.M) : g.M;
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= m_eff) return;  // rows past the device-side count: nothing to do
  const int k_eff = g.k_count ? min(g.K, (max(*g.k_count, 0) + BK - 1) / BK * BK) : g.K;
  const int nk = k_eff / BK;

  // One resource per operand tile: rows past those in memory read as zeros.
  const int rows_a = max(0, min(BM, g.a_rows - m0)), rows_b = max(0, min(BN, g.b_rows - n0));
  const auto ra = make_rsrc(static_cast<const uint16_t*>(g.A) + static_cast<int64_t>(m0) * g.lda,
                            static_cast<uint32_t>(rows_a * g.lda * 2));
  const auto rb = make_rsrc(static_cast<const uint16_t*>(g.B) + static_cast<int64_t>(n0) * g.ldb,
                            static_cast<uint32_t>(rows_b * g.ldb * 2));
  // This lane's chunk of each of the wavefront's 4 loads per operand: chunk
  // j = q 64 + lane of the stage holds (row j / 8, k-chunk (j mod 8) xor row).
  uint32_t offa[4], offb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = (wave * 4 + i) * kWave + lane;
    const int row = j >> 3, kc = (j & 7) ^ (row & 7);
    offa[i] = static_cast<uint32_t>((row * g.lda + kc * 8) * 2);  // < 2^31: lda <= 2^23
    offb[i] = static_cast<uint32_t>((row * g.ldb + kc * 8) * 2);
  }
  auto load_stage = [&](int s, int k0) {
    const uint32_t kb = static_cast<uint32_t>(k0) * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = wave * 4 + i;
      buf_load16_lds(ra, &lds[s][0][q * kWave], offa[i] + kb, 0);
      buf_load16_lds(rb, &lds[s][1][q * kWave], offb[i] + kb, 0);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;  // this wavefront's 64 x 64 quarter
  const int r32 = lane & 31, khalf = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  if (nk > 0) load_stage(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < nk) {
      load_stage(s ^ 1, (kt + 1) * BK);
      wait_vm<8>();  // this stage's 8 loads have landed; the next stage's may not
    } else {
      wait_vm<0>();
    }
    barrier();  // every wavefront's part of stage s is in LDS
    const uint4* As = lds[s][0];
    const uint4* Bs = lds[s][1];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kc = ks * 2 + khalf;  // this lane's 8 k-values of the step
      u32x4_t fa[2], fb[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        fa[b] = *reinterpret_cast<const u32x4_t*>(As + swz(wm * 64 + b * 32 + r32, kc));
        fb[b] = *reinterpret_cast<const u32x4_t*>(Bs + swz(wn * 64 + b * 32 + r32, kc));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(fb[b]), as_bf16(fa[a]),
                                                              acc[a][b], 0, 0, 0);
    }
    barrier();  // every wavefront is done with stage s before it is refilled
  }

  // Epilogue: lane holds, per block, m = r32 and n = 8 j + 4 khalf + (0..3).
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int m = m0 + wm * 64 + a * 32 + r32;
    if (m >= m_eff) continue;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + b * 32 + j * 8 + khalf * 4;
        if (n >= g.N) continue;
        const float v0 = acc[a][b][4 * j], v1 = acc[a][b][4 * j + 1];
        const float v2 = acc[a][b][4 * j + 2], v3 = acc[a][b][4 * j + 3];
        const int64_t off = static_cast<int64_t>(m) * g.ldc + n;
        if constexpr (OUT == kGemmOutBf16) {
          const float lo[2] = {v0, v1}, hi[2] = {v2, v3};
          uint2 w;
          w.x = Dt<VSCE_BF16>::pack_word(lo);
          w.y = Dt<VSCE_BF16>::pack_word(hi);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.C) + off) = w;
        } else {
          float4* p = reinterpret_cast<float4*>(static_cast<float*>(g.C) + off);
          if constexpr (OUT == kGemmOutF32Add) {
            const float4 o = *p;
            *p = make_float4(o.x + v0, o.y + v1, o.z + v2, o.w + v3);
          } else {
            *p = make_float4(v0, v1, v2, v3);
          }
        }
      }
    }
  }
}

}  // namespace

int launch_gemm_nt(int out, const GemmArgs& g, hipStream_t s) {
  if (g.M < 0 || g.N < 0 || g.K < 0 || g.K % BK != 0 || g.N % 4 != 0 || g.ldc % 4 != 0 ||
      g.lda % 8 != 0 || g.ldb % 8 != 0 || g.lda < g.K || g.ldb < g.K || g.ldc < g.N ||
      g.lda > (int64_t(1) << 23) || g.ldb > (int64_t(1) << 23) || g.group_m < 1 ||
      g.a_rows < 0 || g.b_rows < 0)
    return VSCE_ERR_INVALID;
  if (g.M == 0 || g.N == 0) return VSCE_OK;
  const int64_t tiles = static_cast<int64_t>((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  if (tiles > 0x7fffffffLL) return VSCE_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(tiles)), block(NT);
  switch (out) {
    case kGemmOutBf16: hipLaunchKernelGGL(gemm_nt_kernel<kGemmOutBf16>, grid, block, 0, s, g); break;
    case kGemmOutF32: hipLaunchKernelGGL(gemm_nt_kernel<kGemmOutF32>, grid, block, 0, s, g); break;
    case kGemmOutF32Add:
      hipLaunchKernelGGL(gemm_nt_kernel<kGemmOutF32Add>, grid, block, 0, s, g);
      break;
    default: return VSCE_ERR_INVALID;
  }
  return hipGetLastError() == hipSuccess ? VSCE_OK : VSCE_ERR_LAUNCH;
}

}  // namespace vsce
