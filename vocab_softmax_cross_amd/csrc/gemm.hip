// bf16 GEMM on the gfx950 matrix cores, C[m, n] = sum_k A[m, k] B[n, k], for
// the projection products of the linear head fused with the cross-entropy
// (Liger-Kernel PR #1622, FLCE: logits = h W^T, dL/dh = G W, dL/dW = G^T h,
// each arranged so that both operands are contiguous along k).
//
// Large products: workgroups of 16 wavefronts (1024 threads, one per CU,
// four per SIMD) compute 256 x 256 blocks of C, each wavefront a 64 x 64
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
// An operand is stored either with k contiguous ([rows][ld], the row layout)
// or k-major ([k][ld], its rows contiguous: G and h for dL/dW = G^T h, W for
// dL/dh = G W), so that no product needs a transposed copy.  A k-major stage
// holds BK k-rows of the tile's rows and is read with the transposing LDS
// load (fragment() below), which gives the MFMA the same operand, k in the
// same order, as the row layout: the results do not depend on the layout.
//
// Operand lane layout of the 32x32x16 bf16 MFMA (checked on the hardware):
// lane l supplies row l mod 32 and the 8 k-values 8 (l / 32) .. + 7 of each
// operand; result element i of lane l is (row 8 (i / 4) + 4 (l / 32) + i mod 4,
// column l mod 32).  B goes in as the first operand and A as the second, so
// the result's rows are n and its columns m: each lane then holds 4
// consecutive n of one m, stored as one 8-byte (bf16) or 16-byte (fp32) write.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "common.h"
#include "launch.h"

namespace vsce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

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

// This lane's MFMA operand for the 32 rows rb.. of a stage X at k-step ks
// (k-values 16 ks ..): 8 k-values of row rb + (lane mod 32), from k-value
// 16 ks + 8 (lane / 32).
// Row layout (tile rows of BK / 8 chunks, swz): one 16-byte LDS read.
// k-major layout (BK k-rows of CPM chunks; chunk c of k-row k kept at
// c xor 4 (k mod 4), so the 4 k-rows one read touches fill all 64 banks): two
// ds_read_b64_tr_b16.  That load treats the 8 bytes each lane of a group of
// 16 addresses as a 16 x 4 matrix D of 16-bit values (row i from lane i) and
// gives lane t the 4 values D[4 j + t / 4][t mod 4], j = 0..3 (measured on
// gfx950).  Lane i of a group addresses k-row k0 + i / 4 at rows
// r0 + 4 (i mod 4) .. + 3, so lane t receives row r0 + t at k-rows k0 .. k0 + 3.
// One ds_read_b64_tr_b16.  The restrict pointer of this inlined function
// gives the load alias-scope metadata, from which the compiler can tell it
// apart from the direct-to-LDS loads in flight into the other stage; without
// any, it would wait for all of those before every transposing read.
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ s16x4 read_tr(lds_s16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}

// LDS accesses of the epilogue, through restrict pointers for the same
// reason: the stage they use is not the one the loads in flight fill.
template <typename T>
__device__ __forceinline__ void lds_put(T* __restrict__ p, const T v) { *p = v; }
template <typename T>
__device__ __forceinline__ T lds_get(const T* __restrict__ p) { return *p; }

template <bool KM, int BK, int CPM>
__device__ __forceinline__ u32x4_t fragment(const uint4* X, int rb, int ks, int lane) {
  if constexpr (!KM) {
    return *reinterpret_cast<const u32x4_t*>(X + swz<BK>(rb + (lane & 31), ks * 2 + (lane >> 5)));
  } else {
    const int grp = lane >> 4, t = lane & 15;
    const int r = rb + 16 * (grp & 1) + 4 * (t & 3);   // rows this lane addresses
    const int k = ks * 16 + 8 * (grp >> 1) + (t >> 2);  // its k-row; k mod 4 = t / 4
    const int c = (r >> 3) ^ (4 * (t >> 2));
    const char* p = reinterpret_cast<const char*>(X + k * CPM + c) + (r & 7) * 2;
    const s16x4 lo = read_tr((lds_s16x4*)(p));
    const s16x4 hi = read_tr((lds_s16x4*)(p + 4 * CPM * 16));  // k-rows + 4
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return u32x4_t{a.x, a.y, b.x, b.y};
  }
}

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

// BM x BN blocks, WGM x WGN wavefronts, each a (BM / WGM) x (BN / WGN) part of
// R x S 32 x 32 MFMA blocks; two LDS stages of BK k-values (one in flight
// while the other is multiplied); WPE wavefronts per SIMD to compile for.
// LAYOUT: bit 0, A k-major; bit 1, B k-major.
//
// Persistent: the grid holds as many workgroups as the chip runs at once, and
// each walks its own sequence of tiles as one flat loop over (tile, k-step),
// so the first stage of its next tile is loaded while the last stage of the
// current one is multiplied and while that tile's C is stored.  Workgroup b
// runs on XCD b mod 8; XCD x takes a contiguous range of the tile order and
// its gridDim / 8 workgroups every (gridDim / 8)-th tile of it, so the tiles
// one XCD has in flight are neighbours in the order (tile_of) and share
// operand panels in that XCD's L2.
template <int OUT, int LAYOUT, int BM, int BN, int BK, int NS, int WGM, int WGN, int WPE>
__global__ __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void gemm_nt_kernel(const GemmArgs g) {
  constexpr bool AKM = LAYOUT & 1, BKM = LAYOUT & 2;
  constexpr int CPA = BM / 8, CPB = BN / 8;        // 16-byte chunks per k-major k-row
  static_assert(CPA >= 16 && CPB >= 16, "the k-major swizzle spans 16 chunks");
  constexpr int NW = WGM * WGN, NT = NW * 64;
  constexpr int R = BM / (32 * WGM), S = BN / (32 * WGN);
  constexpr int CPR = BK / 8;                      // 16-byte chunks per tile row
  constexpr int LA = BM * CPR / NT, LB = BN * CPR / NT;
  static_assert(LA * NT == BM * CPR && LB * NT == BN * CPR, "loads per wavefront");
  static_assert(NS == 2, "the waits below assume one stage in flight");
  // Vector-memory stores of one tile's epilogue per wavefront, at least: every
  // one is issued (lanes outside C are dropped by the buffer's range check,
  // not skipped), so the count of operations issued after a stage's loads is
  // known.  4 per round of the epilogue below.
  static_assert(R == 2 && S == 2, "the epilogue stages 64 x 64 per wavefront");
  static_assert((BM + BN) * CPR >= NW * 256, "4 KB of a stage per wavefront");
  constexpr int kEpilogueStores = (OUT == kGemmOutBf16 ? R : R * S) * 4;
  constexpr int ES = OUT == kGemmOutBf16 ? 2 : 4;  // bytes per element of C
  __shared__ uint4 lds[NS][(BM + BN) * CPR];       // [stage][A rows, then B rows][chunk]
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = uniform(tid / kWave);
  const int m_eff = g.m_count ? min(max(*g.m_count, 0), g.M) : g.M;
  const int k_eff =
      g.k_count ? min(g.K, (max(*g.k_count, 0) + kKMult - 1) / kKMult * kKMult) : g.K;
  const int nk = k_eff / BK;
  // Tiles with rows past the device-side count are left out of the order.
  const int tiles_m = (m_eff + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int64_t xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds, slot = blockIdx.x / kXcds;
  const int64_t q = tiles / kXcds, rem = tiles % kXcds;
  const int64_t first = xcd * q + (xcd < rem ? xcd : rem) + slot;  // this workgroup's first tile
  const int64_t range = q + (xcd < rem ? 1 : 0);         // tiles of this XCD
  const int64_t mine = range > slot ? (range - 1 - slot) / per_xcd + 1 : 0;
  if (mine == 0) return;
  auto origin = [&](int64_t ord, int& m0, int& n0) {  // of this workgroup's tile ord
    int tm, tn;
    tile_of(first + ord * per_xcd, tiles_m, tiles_n, g.group_m, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
  };

  const int wm = wave / WGN, wn = wave % WGN;  // this wavefront's part
  const int r32 = lane & 31, khalf = lane >> 5;
  f32x16 acc[R][S];
  auto clear = [&]() {
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < S; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  };
  // C of the tile at (m0, n0) from acc, staged through this wavefront's 4 KB
  // of LDS stage s (free once every wavefront is done multiplying it) so that
  // each store writes whole 128-byte row segments, 8 rows per instruction,
  // instead of 16 bytes in each of 32 rows.  acc holds, per 32 x 32 block,
  // m = r32 and n = 8 j + 4 khalf + (0..3).  A round stages 32 rows: bf16, one
  // block row (S blocks, 64 n); fp32, one block (32 n); each row is 128 bytes,
  // its 16-byte chunk c kept at c xor (row mod 8) so that the writes of a
  // column of rows and the reads of 2 rows at a time spread over the banks.
  // One resource spans the tile's rows of C (< 2^31 bytes: ldc bytes <= 2^23);
  // chunks past N get an offset outside it.
  auto epilogue = [&](int m0, int n0, int s) {
    const int rows_c = min(BM, m_eff - m0);
    const auto rc = uniform_rsrc(static_cast<char*>(g.C) + static_cast<int64_t>(m0) * g.ldc * ES,
                                 static_cast<int64_t>(rows_c) * g.ldc * ES);
    // bf16 chunks are 8 n: one 16-byte store each when N and ldc allow it,
    // else two 8-byte stores that stop at N.
    const bool whole = OUT != kGemmOutBf16 || (g.N % 8 == 0 && g.ldc % 8 == 0);
    barrier();  // every wavefront is done reading stage s
    uint4* const buf = lds[s] + wave * 256;
    const int rrow = lane >> 3, rc8 = lane & 7;  // read-back: row in 8, chunk
    constexpr int kRounds = OUT == kGemmOutBf16 ? R : R * S;
#pragma unroll
    for (int round = 0; round < kRounds; ++round) {
      const int a = OUT == kGemmOutBf16 ? round : round / S;
      const int b0 = OUT == kGemmOutBf16 ? 0 : round % S;
      if constexpr (OUT == kGemmOutBf16) {
#pragma unroll
        for (int b = 0; b < S; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float lo[2] = {acc[a][b][4 * j], acc[a][b][4 * j + 1]};
            const float hi[2] = {acc[a][b][4 * j + 2], acc[a][b][4 * j + 3]};
            const uint2 w = make_uint2(Dt<VSCE_BF16>::pack_word(lo), Dt<VSCE_BF16>::pack_word(hi));
            lds_put(reinterpret_cast<uint2*>(buf + r32 * 8 + ((b * 4 + j) ^ (r32 & 7))) + khalf, w);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          lds_put(buf + r32 * 8 + ((2 * j + khalf) ^ (r32 & 7)),
              make_uint4(__float_as_uint(acc[a][b0][4 * j]), __float_as_uint(acc[a][b0][4 * j + 1]),
                         __float_as_uint(acc[a][b0][4 * j + 2]),
                         __float_as_uint(acc[a][b0][4 * j + 3])));
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = rr * 8 + rrow;
        const uint4 v = lds_get(buf + row * 8 + (rc8 ^ (row & 7)));
        const int64_t mrow = static_cast<int64_t>(wm * (BM / WGM) + a * 32 + row) * g.ldc;
        const int n = n0 + wn * (BN / WGN) + (OUT == kGemmOutBf16 ? rc8 * 8 : b0 * 32 + rc8 * 4);
        const uint32_t off = n < g.N ? static_cast<uint32_t>((mrow + n) * ES) : kOutOfRange;
        if constexpr (OUT == kGemmOutBf16) {
          if (whole) {
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, rc, off, 0, 0);
          } else {
            const uint32_t off2 =
                n + 4 < g.N ? static_cast<uint32_t>((mrow + n + 4) * ES) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v.x, v.y}, rc, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v.z, v.w}, rc, off2, 0, 0);
          }
        } else {
          float4 o = __builtin_bit_cast(float4, v);
          if constexpr (OUT == kGemmOutF32Add) {
            const float4 c =
                __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0));
            o = make_float4(c.x + o.x, c.y + o.y, c.z + o.z, c.w + o.w);
          }
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), rc, off, 0, 0);
        }
      }
    }
  };
  if (nk == 0) {  // empty k: C = 0 (or C unchanged when adding)
    clear();
    for (int64_t ord = 0; ord < mine; ++ord) {
      int m0, n0;
      origin(ord, m0, n0);
      epilogue(m0, n0, 0);
    }
    return;
  }

  // This lane's chunk of each of the wavefront's loads: chunk j = q 64 + lane
  // of an operand's stage is LDS position j.  Row layout: swz() assigns it to
  // (row j / CPR, k-chunk (j mod CPR) xor f(row)); k-major: to (k-row j / CP,
  // chunk (j mod CP) xor 4 (k-row mod 4)).  Each XOR is its own inverse.
  uint32_t offa[LA], offb[LB];
  auto chunk_offset = [&](int j, int64_t ld, bool km, int cp) {
    if (km) {
      const int k = j / cp;
      const int c = (j % cp) ^ (4 * (k & 3));
      return static_cast<uint32_t>((k * ld + c * 8) * 2);  // < 2^30: k < 64, ld < 2^23
    }
    const int row = j / CPR;
    const int kc = swz<BK>(row, j % CPR) - row * CPR;
    return static_cast<uint32_t>((row * ld + kc * 8) * 2);  // < 2^32: ld < 2^23
  };
#pragma unroll
  for (int i = 0; i < LA; ++i)
    offa[i] = chunk_offset((wave * LA + i) * kWave + lane, g.lda, AKM, CPA);
#pragma unroll
  for (int i = 0; i < LB; ++i)
    offb[i] = chunk_offset((wave * LB + i) * kWave + lane, g.ldb, BKM, CPB);
  // The load cursor: tile ordinal and k-step of the next stage to load, and
  // one resource per operand: per tile for the row layout (rows past a_rows /
  // b_rows read as zeros), per stage for k-major (k-rows past a_rows / b_rows,
  // and columns past M / N of the last k-row, read as zeros; other columns
  // past M / N only reach rows of C that are not stored).
  int64_t l_ord = 0;
  int l_k = 0, l_m0 = 0, l_n0 = 0;
  __amdgpu_buffer_rsrc_t ra, rb;
  auto row_rsrc = [&](const void* X, int64_t ld, int rows_mem, int r0, int rows) {
    const int n = max(0, min(rows, rows_mem - r0));
    return uniform_rsrc(static_cast<const uint16_t*>(X) + static_cast<int64_t>(r0) * ld,
                        static_cast<int64_t>(n) * ld * 2);
  };
  auto km_rsrc = [&](const void* X, int64_t ld, int krows_mem, int cols, int k0, int c0) {
    const int64_t left = (static_cast<int64_t>(krows_mem - 1 - k0) * ld + (cols - c0)) * 2;
    const int64_t cap = int64_t(1) << 31;  // past every offset of a stage (< 2^30)
    return uniform_rsrc(static_cast<const uint16_t*>(X) + static_cast<int64_t>(k0) * ld + c0,
                        left <= 0 ? 0 : (left < cap ? left : cap));
  };
  auto aim = [&](int64_t ord) {
    origin(ord, l_m0, l_n0);
    if constexpr (!AKM) ra = row_rsrc(g.A, g.lda, g.a_rows, l_m0, BM);
    if constexpr (!BKM) rb = row_rsrc(g.B, g.ldb, g.b_rows, l_n0, BN);
  };
  auto load_next = [&](int s) {
    if (l_ord == mine) return;
    const int k0 = l_k * BK;
    if constexpr (AKM) ra = km_rsrc(g.A, g.lda, g.a_rows, g.M, k0, l_m0);
    if constexpr (BKM) rb = km_rsrc(g.B, g.ldb, g.b_rows, g.N, k0, l_n0);
    const uint32_t ka = AKM ? 0u : static_cast<uint32_t>(k0) * 2u;
    const uint32_t kb = BKM ? 0u : static_cast<uint32_t>(k0) * 2u;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      load16_lds(ra, &lds[s][(wave * LA + i) * kWave], offa[i] + ka);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      load16_lds(rb, &lds[s][BM * CPR + (wave * LB + i) * kWave], offb[i] + kb);
    if (++l_k == nk) {
      l_k = 0;
      if (++l_ord < mine) aim(l_ord);
    }
  };

  aim(0);
  load_next(0);
  int64_t c_ord = 0;  // tile being multiplied, and its k-step
  int c_k = 0, cm0, cn0;
  origin(0, cm0, cn0);
  clear();
  const int64_t steps = mine * nk;
  for (int64_t it = 0; it < steps; ++it) {
    const int s = static_cast<int>(it & 1);
    // Stage it was loaded during step it - 1; when that step ended a tile,
    // the tile's epilogue stores were issued after it and may stay in flight.
    if (c_k == 0 && it > 0) wait_vm<kEpilogueStores>();
    else wait_vm<0>();
    barrier();  // stage it is in LDS; every wavefront is done with stage it - 1
    load_next(s ^ 1);
    const uint4* As = lds[s];
    const uint4* Bs = lds[s] + BM * CPR;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4_t fa[R], fb[S];
#pragma unroll
      for (int a = 0; a < R; ++a)
        fa[a] = fragment<AKM, BK, CPA>(As, wm * (BM / WGM) + a * 32, ks, lane);
#pragma unroll
      for (int b = 0; b < S; ++b)
        fb[b] = fragment<BKM, BK, CPB>(Bs, wn * (BN / WGN) + b * 32, ks, lane);
#pragma unroll
      for (int a = 0; a < R; ++a)
#pragma unroll
        for (int b = 0; b < S; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(fb[b]), as_bf16(fa[a]),
                                                              acc[a][b], 0, 0, 0);
    }
    if (++c_k == nk) {
      epilogue(cm0, cn0, s);
      clear();
      c_k = 0;
      if (++c_ord < mine) origin(c_ord, cm0, cn0);
    }
  }
}

}  // namespace

namespace {

constexpr int kMaxDevices = 64;

// Workgroups of `kernel` the current device runs at once (CUs x workgroups
// per CU), cached per device.
template <typename Kernel>
int resident_workgroups(Kernel kernel, int threads) {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 0;
  const int n = cus * per_cu;
  if (n > 0 && dev >= 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int OUT, int LAYOUT, int BM, int BN, int BK, int NS, int WGM, int WGN, int WPE>
int launch_persistent(const GemmArgs& g, hipStream_t s) {
  auto kernel = gemm_nt_kernel<OUT, LAYOUT, BM, BN, BK, NS, WGM, WGN, WPE>;
  const int threads = WGM * WGN * 64;
  const int64_t tiles = static_cast<int64_t>((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  const int resident = resident_workgroups(kernel, threads);
  if (resident <= 0) return VSCE_ERR_LAUNCH;
  // A multiple of 8 (the tile ranges are split by XCD), no more than the
  // chip holds at once nor than the tiles need.
  const int64_t cap = std::max<int64_t>(kXcds, resident / kXcds * kXcds);
  const int64_t grid = std::min<int64_t>(cap, (tiles + kXcds - 1) / kXcds * kXcds);
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(threads), 0, s, g);
  return hipGetLastError() == hipSuccess ? VSCE_OK : VSCE_ERR_LAUNCH;
}

template <int OUT, int BM, int BN, int BK, int NS, int WGM, int WGN, int WPE>
int launch_layout(const GemmArgs& g, hipStream_t s) {
  switch (g.layout) {
    case 0: return launch_persistent<OUT, 0, BM, BN, BK, NS, WGM, WGN, WPE>(g, s);
    case 1: return launch_persistent<OUT, 1, BM, BN, BK, NS, WGM, WGN, WPE>(g, s);
    case 2: return launch_persistent<OUT, 2, BM, BN, BK, NS, WGM, WGN, WPE>(g, s);
    case 3: return launch_persistent<OUT, 3, BM, BN, BK, NS, WGM, WGN, WPE>(g, s);
    default: return VSCE_ERR_INVALID;
  }
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, int WPE>
int launch_blocks(int out, const GemmArgs& g, hipStream_t s) {
  switch (out) {
    case kGemmOutBf16: return launch_layout<kGemmOutBf16, BM, BN, BK, NS, WGM, WGN, WPE>(g, s);
    case kGemmOutF32: return launch_layout<kGemmOutF32, BM, BN, BK, NS, WGM, WGN, WPE>(g, s);
    case kGemmOutF32Add: return launch_layout<kGemmOutF32Add, BM, BN, BK, NS, WGM, WGN, WPE>(g, s);
    default: return VSCE_ERR_INVALID;
  }
}

// An operand's leading dimension: a multiple of 8, below 2^23, and at least
// its contiguous extent (K in the row layout, its rows when k-major).
bool ld_ok(int64_t ld, int64_t contiguous) {
  return ld % 8 == 0 && ld >= contiguous && ld < (int64_t(1) << 23);
}

}  // namespace

int launch_gemm_nt(int out, const GemmArgs& g, hipStream_t s) {
  if (g.M < 0 || g.N < 0 || g.K < 0 || g.K % kKMult != 0 || g.N % 4 != 0 || g.ldc % 4 != 0 ||
      g.layout < 0 || g.layout > 3 || !ld_ok(g.lda, (g.layout & 1) ? g.M : g.K) ||
      !ld_ok(g.ldb, (g.layout & 2) ? g.N : g.K) || g.ldc < g.N || g.group_m < 1 ||
      g.a_rows < 0 || g.b_rows < 0 ||
      g.ldc * (out == kGemmOutBf16 ? 2 : 4) > (int64_t(1) << 23))
    return VSCE_ERR_INVALID;
  if (g.M == 0 || g.N == 0) return VSCE_OK;
  // Large products: 256 x 256 blocks, one per CU, 2 stages of 64 k-values
  // (128 KB of LDS, 64 x 64 per wavefront); small ones: 128 x 128 blocks,
  // two per CU, 2 stages of 64.
  if (g.M >= 256 && g.N >= 256) return launch_blocks<256, 256, 64, 2, 4, 4, 4>(out, g, s);
  return launch_blocks<128, 128, 64, 2, 2, 2, 2>(out, g, s);
}

}  // namespace vsce
