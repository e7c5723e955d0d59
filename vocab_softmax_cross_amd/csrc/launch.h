// Internal interface between the C-ABI layer (abi.cpp) and the kernel
// translation units.  Host code only; every function enqueues work on the
// given stream and returns a VSCE_* code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "vsce.h"

namespace vsce {

// A validated problem with the derived quantities the launchers need.
struct Prob {
  int64_t rows;
  int64_t V;       // columns of this buffer
  int64_t voff;    // global column of its first column (vocab-parallel shard)
  int64_t Vt;      // full vocabulary (= V unless sharded)
  int64_t stride;  // elements
  int dt;          // vsce_dtype
  int red;         // vsce_reduction
  const int64_t* target;
  const float* weight;
  int64_t ignore_index;
  float eps;
  float eta;       // eps / V
  float cap;       // soft-cap s (0: off)
  float zl;        // z-loss lambda (0: off)
  int elem_bytes;
  bool vec_ok;     // rows start 16-byte aligned and V fills whole 16-byte vectors
  uint32_t flags;  // VSCE_FLAG_* bits
};

// Arguments of every per-row kernel (passed by value).
struct RowArgs {
  void* x;              // logits (the gradient is written here by the fused kernels)
  void* g;              // gradient output of the split backward (may equal x)
  int64_t stride;       // elements between rows
  int64_t V;            // columns of this buffer
  int64_t voff;         // global column of its first column (shard), else 0
  int64_t Vt;           // full vocabulary: targets are classes of [0, Vt)
  int64_t nvec;         // 16-byte vectors per row (vector path) or V (scalar path)
  const int64_t* target;
  const float* weight;  // [V] or null
  int64_t ignore_index;
  float eps;
  float eta;
  SoftCap cap_c;        // the soft-cap's constants (the CAP kernels only)
  float zl;             // z-loss lambda (0: off)
  int mean;             // sigma = 1 / W (mean) else 1
  float* loss_rows;     // [rows] per-row loss (never null)
  float* loss_rows2;    // [rows] second copy of the per-row loss, or null
  float* acc_rows;      // [rows] or null
  float* z_rows;        // [rows] per-row z-loss, or null
  float* stats;         // [rows][4] or null
  float* partial;       // [rows][8] shard records (partial statistics mode), or null
  const float* go;      // grad_output (backward / scale); null: 1.0 (backward)
  int64_t go_stride;    // 0 (scalar) or 1 (per row)
  int skip_if_one;
  int64_t rows;
  int64_t chunks;       // column chunks per row (chunked kernels)
  const WsHeader* ws;
};

// Checks a problem descriptor (with the logits pointer it will be used
// with) and fills the derived fields; VSCE_OK or the error to return.
int check_problem(const vsce_problem* pb, const void* logits, Prob& p);
// The problem's fields every per-row kernel reads.
void problem_args(const Prob& p, RowArgs& a);
// The constants of a soft-cap s (zeros for s = 0).
SoftCap soft_cap_constants(float s);
// Byte offset, in a workspace of vsce_workspace_bytes(rows), of its [rows]
// float4 statistics area (the fused mode's rows that are read twice).
int64_t stats_scratch_offset(int64_t rows);

int launch_prologue(const Prob& p, WsHeader* ws, hipStream_t s);
int launch_finalize(const Prob& p, const float* loss_rows, const float* acc_rows,
                    const float* z_rows, float* loss_out, float* acc_mean_out, float* z_out,
                    const WsHeader* ws, hipStream_t s);

// Row held on chip (registers + LDS) between its passes: one logits read and
// one gradient write.  VSCE_ERR_UNSUPPORTED when the row does not fit.
int launch_fused_resident(const Prob& p, RowArgs a, hipStream_t s);
template <int DT, bool CAP>
int fused_resident_dt(const Prob& p, const RowArgs& a, hipStream_t s);
// Streaming kernels by element type; `which` is kStreamStats .. kStreamScale.
enum { kStreamStats = 0, kStreamRing = 1, kStreamBackward = 2, kStreamScale = 3 };
template <int DT, bool CAP>
int stream_dt(int which, const Prob& p, const RowArgs& a, hipStream_t s);
// Fused, one launch, any row length on 16-byte vectors without class
// weights: the row is streamed twice (statistics, then gradient) through an
// LDS ring.  VSCE_ERR_UNSUPPORTED for other rows.
int launch_fused_ring(const Prob& p, RowArgs a, hipStream_t s);
// Split forward: one logits read, statistics + loss.
int launch_stats(const Prob& p, RowArgs a, hipStream_t s);
// Split backward: logits read + gradient write from the saved statistics.
int launch_backward(const Prob& p, RowArgs a, hipStream_t s);
// Merge of shard records into full statistics and row losses.
int launch_merge(const Prob& p, const float* partials, int shards, float* stats,
                 const RowArgs& a, hipStream_t s);
// In-place grad_output scale.
int launch_scale(const Prob& p, RowArgs a, hipStream_t s);

// bf16 GEMM on the matrix cores: C[m, n] = sum_k A[m, k] B[n, k] with fp32
// accumulation.  A is [M, K] and B [N, K], each either contiguous along k
// (the row layout) or stored k-major as [K][M] / [K][N] (layout); leading
// dimensions lda, ldb in elements, multiples of 8, below 2^23, at least K in
// the row layout and M / N when k-major; 16-byte aligned; K a multiple of 64;
// N and ldc multiples of 4, a row of C at most 2^23 bytes.  Device-side counts
// (optional) narrow the work without a host read: rows m >= *m_count are
// neither computed nor stored, and k runs to *k_count rounded up to 64 (the
// caller keeps A and B zero between the count and that bound).
struct GemmArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C;
  int64_t ldc;
  int M, N, K;
  // Rows of A and B in memory, rows past them read as zeros: m- / n-rows in
  // the row layout ([M][lda], [N][ldb]), k-rows when k-major ([K][lda], [K][ldb]).
  int a_rows, b_rows;
  int layout;             // bit 0: A k-major; bit 1: B k-major
  int group_m;            // m-tiles per group of the tile order (>= 1)
  const int* m_count;     // device, or null (all M rows)
  const int* k_count;     // device, or null (all K)
};
enum { kGemmOutBf16 = 0, kGemmOutF32 = 1, kGemmOutF32Add = 2 };
enum { kGemmAKMajor = 1, kGemmBKMajor = 2 };
int launch_gemm_nt(int out, const GemmArgs& g, hipStream_t s);

}  // namespace vsce
