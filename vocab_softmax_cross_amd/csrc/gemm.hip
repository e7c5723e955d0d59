// bf16 GEMM on the gfx950 matrix cores, C[m, n] = sum_k A[m, k] B[n, k], for
// the projection products of the linear head fused with the cross-entropy
// (Liger-Kernel PR #1622, FLCE: logits = h W^T, dL/dh = G W, dL/dW = G^T h,
// each arranged so that both operands are contiguous along k).
//
// Large products: one workgroup of 16 wavefronts (1024 threads, one per CU,
// four per SIMD) computes a 256 x 256 block of C, each wavefront a 64 x 64
// part as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
// Small products (M or N below 256): 128 x 128 blocks of 4 wavefronts, two
// workgroups per CU.  k advances 64 at a time through two LDS stages of A and
// B (64 KB per stage for 256 x 256): the next stage is loaded straight into
// LDS (buffer_load_dwordx4 ... lds) while the current one is multiplied, with
// one workgroup barrier per stage.  In LDS each tile row is 8 chunks of 16
// bytes, the chunk index XOR-ed with a function of the row (swz below) so the
// rows one MFMA operand read touches sit in different banks; the swizzle is
// applied by choosing which global chunk each lane loads, since a
// direct-to-LDS load writes lane i at base + 16 i.
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

constexpr int kKMult = 64;  // K must be a multiple of kKMult

// LDS chunk of (row, 16-byte k-chunk kc) in a stage whose rows hold BK
// k-values (BK / 8 chunks).  A 16-byte-per-lane LDS read is served 16 lanes
// at a time across 64 four-byte banks (a 256-byte window; the bank-conflict
// counter confirms it), and an MFMA operand read has 16 consecutive rows at
// one kc in each such group.  The chunk index is XOR-ed with a function of
// the row so that those 16 rows fill the 16 slots of the window: rows of 128
// bytes (BK 64, two per window) use (row / 2) mod 8; rows of 64 bytes (BK 32,
// four per window) use (row / 4) mod 4.
template <int BK>
__device__ __forceinline__ int swz(int row, int kc) {
  if constexpr (BK == 64) return row * 8 + (kc ^ ((row >> 1) & 7));
  else return row * 4 + (kc ^ ((row >> 2) & 3));
}

// A stage is read with ordinary LDS loads (the compiler places their waits
// and the MFMA register hazards); the direct-to-LDS loads that fill it are
// waited for by hand (wait_vm) and published to the workgroup by barrier().
// Operand stages are loaded with the default cache policy: unlike the
// cross-entropy's single pass over the logits, every operand panel is read
// again by the other tiles of its row or column, so it should stay in L2 and
// the infinity cache.
__device__ __forceinline__ void load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_wave,
                                           uint32_t voff) {
  buf_load16_lds<0>(r, lds_wave, voff, 0);
}

// A buffer resource from values every lane holds, passed through
// readfirstlane so that the compiler keeps it in scalar registers (otherwise
// it may treat it as per-lane and wrap every load in a loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bytes));
  return make_rsrc(reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo), n);
}

// Workgroup barrier after this wavefront's LDS reads have completed (so a
// stage is refilled only once every wavefront is done reading it).
__device__ __forceinline__ void barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
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

// BM x BN block, WGM x WGN wavefronts, each a (BM / WGM) x (BN / WGN) part of
// R x S 32 x 32 MFMA blocks; NS LDS stages of BK k-values (NS - 1 of them in
// flight while one is multiplied); WPE wavefronts per SIMD to compile for.
template <int OUT, int BM, int BN, int BK, int NS, int WGM, int WGN, int WPE>
__global__ __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void gemm_nt_kernel(const GemmArgs g) {
  constexpr int NW = WGM * WGN, NT = NW * 64;
  constexpr int R = BM / (32 * WGM), S = BN / (32 * WGN);
  constexpr int CPR = BK / 8;                      // 16-byte chunks per tile row
  constexpr int LA = BM * CPR / NT, LB = BN * CPR / NT;
  static_assert(LA * NT == BM * CPR && LB * NT == BN * CPR, "loads per wavefront");
  constexpr int L = LA + LB;                       // loads per wavefront per stage
  static_assert(NS >= 2 && NS <= 4 && (NS - 2) * L <= 63, "stages");
  __shared__ uint4 lds[NS][(BM + BN) * CPR];       // [stage][A rows, then B rows][chunk]
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = uniform(tid / kWave);
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  tile_of(xcd_contiguous(blockIdx.x, static_cast<int64_t>(tiles_m) * tiles_n), tiles_m, tiles_n,
          g.group_m, tm, tn);
  const int m_eff = g.m_count ? min(max(*g.m_count, 0), g.M) : g.M;
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= m_eff) return;  // rows past the device-side count: nothing to do
  const int k_eff =
      g.k_count ? min(g.K, (max(*g.k_count, 0) + kKMult - 1) / kKMult * kKMult) : g.K;
  const int nk = k_eff / BK;

  // One resource per operand tile: rows past those in memory read as zeros.
  const int rows_a = max(0, min(BM, g.a_rows - m0)), rows_b = max(0, min(BN, g.b_rows - n0));
  const auto ra = uniform_rsrc(
      static_cast<const uint16_t*>(g.A) + static_cast<int64_t>(m0) * g.lda, rows_a * g.lda * 2);
  const auto rb = uniform_rsrc(
      static_cast<const uint16_t*>(g.B) + static_cast<int64_t>(n0) * g.ldb, rows_b * g.ldb * 2);
  // This lane's chunk of each of the wavefront's loads: chunk j = q 64 + lane
  // of an operand's stage is LDS position j, which swz() assigns to (row
  // j / CPR, k-chunk (j mod CPR) xor f(row)); the XOR is its own inverse.
  uint32_t offa[LA], offb[LB];
  auto chunk_offset = [&](int j, int64_t ld) {
    const int row = j / CPR;
    const int kc = swz<BK>(row, j % CPR) - row * CPR;
    return static_cast<uint32_t>((row * ld + kc * 8) * 2);  // < 2^31: ld <= 2^23
  };
#pragma unroll
  for (int i = 0; i < LA; ++i) offa[i] = chunk_offset((wave * LA + i) * kWave + lane, g.lda);
#pragma unroll
  for (int i = 0; i < LB; ++i) offb[i] = chunk_offset((wave * LB + i) * kWave + lane, g.ldb);
  auto load_stage = [&](int s, int k0) {
    const uint32_t kb = static_cast<uint32_t>(k0) * 2u;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      load16_lds(ra, &lds[s][(wave * LA + i) * kWave], offa[i] + kb);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      load16_lds(rb, &lds[s][BM * CPR + (wave * LB + i) * kWave], offb[i] + kb);
  };

  const int wm = wave / WGN, wn = wave % WGN;  // this wavefront's part
  const int r32 = lane & 31, khalf = lane >> 5;
  f32x16 acc[R][S];
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < S; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  // NS - 1 stages in flight ahead of the one being multiplied.
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) load_stage(st, st * BK);
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt % NS;
    // Loads issued after stage kt's: the stages kt + 1 .. kt + NS - 2 that exist.
    const int later = min(NS - 2, nk - 1 - kt);
    if (later >= 2) wait_vm<(NS >= 4 ? 2 : 0) * L>();
    else if (later == 1) wait_vm<L>();
    else wait_vm<0>();
    barrier();  // stage kt is in LDS; every wavefront is done with stage kt - 1
    if (kt + NS - 1 < nk) load_stage((kt + NS - 1) % NS, (kt + NS - 1) * BK);
    const uint4* As = lds[s];
    const uint4* Bs = lds[s] + BM * CPR;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kc = ks * 2 + khalf;  // this lane's 8 k-values of the step
      u32x4_t fa[R], fb[S];
#pragma unroll
      for (int a = 0; a < R; ++a)
        fa[a] = *reinterpret_cast<const u32x4_t*>(
            As + swz<BK>(wm * (BM / WGM) + a * 32 + r32, kc));
#pragma unroll
      for (int b = 0; b < S; ++b)
        fb[b] = *reinterpret_cast<const u32x4_t*>(
            Bs + swz<BK>(wn * (BN / WGN) + b * 32 + r32, kc));
#pragma unroll
      for (int a = 0; a < R; ++a)
#pragma unroll
        for (int b = 0; b < S; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(fb[b]), as_bf16(fa[a]),
                                                              acc[a][b], 0, 0, 0);
    }
  }

  // Epilogue: lane holds, per block, m = r32 and n = 8 j + 4 khalf + (0..3).
#pragma unroll
  for (int a = 0; a < R; ++a) {
    const int m = m0 + wm * (BM / WGM) + a * 32 + r32;
    if (m >= m_eff) continue;
#pragma unroll
    for (int b = 0; b < S; ++b) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * (BN / WGN) + b * 32 + j * 8 + khalf * 4;
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

namespace {

template <int BM, int BN, int BK, int NS, int WGM, int WGN, int WPE>
int launch_blocks(int out, const GemmArgs& g, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  if (tiles > 0x7fffffffLL) return VSCE_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(tiles)), block(WGM * WGN * 64);
  switch (out) {
    case kGemmOutBf16:
      hipLaunchKernelGGL((gemm_nt_kernel<kGemmOutBf16, BM, BN, BK, NS, WGM, WGN, WPE>), grid, block, 0, s, g);
      break;
    case kGemmOutF32:
      hipLaunchKernelGGL((gemm_nt_kernel<kGemmOutF32, BM, BN, BK, NS, WGM, WGN, WPE>), grid, block, 0, s, g);
      break;
    case kGemmOutF32Add:
      hipLaunchKernelGGL((gemm_nt_kernel<kGemmOutF32Add, BM, BN, BK, NS, WGM, WGN, WPE>), grid, block, 0, s, g);
      break;
    default: return VSCE_ERR_INVALID;
  }
  return hipGetLastError() == hipSuccess ? VSCE_OK : VSCE_ERR_LAUNCH;
}

}  // namespace

int launch_gemm_nt(int out, const GemmArgs& g, hipStream_t s) {
  if (g.M < 0 || g.N < 0 || g.K < 0 || g.K % kKMult != 0 || g.N % 4 != 0 || g.ldc % 4 != 0 ||
      g.lda % 8 != 0 || g.ldb % 8 != 0 || g.lda < g.K || g.ldb < g.K || g.ldc < g.N ||
      g.lda > (int64_t(1) << 23) || g.ldb > (int64_t(1) << 23) || g.group_m < 1 ||
      g.a_rows < 0 || g.b_rows < 0)
    return VSCE_ERR_INVALID;
  if (g.M == 0 || g.N == 0) return VSCE_OK;
  // Large products: 256 x 256 blocks, one per CU, 2 stages of 64 k-values
  // (128 KB of LDS, 128 x 128 per wavefront); small ones: 128 x 128 blocks,
  // two per CU, 2 stages of 64.
  if (g.M >= 256 && g.N >= 256) return launch_blocks<256, 256, 64, 2, 4, 4, 4>(out, g, s);
  return launch_blocks<128, 128, 64, 2, 2, 2, 2>(out, g, s);
}

}  // namespace vsce
