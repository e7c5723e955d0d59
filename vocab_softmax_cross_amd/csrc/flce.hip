// The linear head fused with the cross-entropy (Liger-Kernel PR #1622,
// "perf(flce): drop host syncs that do not feed the computation": the FLCE
// forward computes the loss and both gradients, chunk by chunk of rows; the
// #1554 compaction it discusses keeps ignored rows out of the projection
// products).  For a chunk of rows with hidden states h and the weight W:
//   logits z = h W^T            (bf16 GEMM on the matrix cores, bf16 logits)
//   the fused cross-entropy     (loss rows; G = dL/dz written over z)
//   dL/dh = G W,  dL/dW += G^T h   (two more GEMMs that read W, G and h
//                                  k-major where they need it: no transposed
//                                  copies)
// Ignored rows are compacted out on the device first (a prefix count over the
// targets): the products skip them through device-side row counts, so no
// count is read on the host, and their dL/dh rows are written as zeros at the
// end.  The loss normalizers come from one prologue over all kept rows, so a
// chunked run reduces exactly like an unchunked one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "launch.h"
#include "vsce.h"

namespace vsce {
namespace {

constexpr int64_t kAlignB = 256;
int64_t al(int64_t v) { return (v + kAlignB - 1) / kAlignB * kAlignB; }
int64_t up64(int64_t v) { return (v + 63) / 64 * 64; }

// Workspace layout of one FLCE problem (byte offsets from its start).
struct FlceLayout {
  int64_t C;      // rows per chunk (a multiple of 64)
  int64_t nch;    // chunks
  int64_t R;      // compacted rows held: nch * C
  int64_t Vp;     // vocabulary padded to a multiple of 64
  int64_t ce, ints, tc, goc, lossc, zc, accc, xc, dxc, logits, end;
};

FlceLayout layout(int64_t rows, int64_t H, int64_t V, int64_t chunk_rows) {
  FlceLayout L;
  const int64_t all = up64(rows > 0 ? rows : 1);
  L.C = (chunk_rows <= 0) ? all : (up64(chunk_rows) < all ? up64(chunk_rows) : all);
  L.nch = (rows + L.C - 1) / L.C;
  if (L.nch < 1) L.nch = 1;
  L.R = L.nch * L.C;
  L.Vp = up64(V);
  int64_t o = 0;
  L.ce = o;     o += al(static_cast<int64_t>(vsce_workspace_bytes(L.R)));
  L.ints = o;   o += al(4 * (1 + L.nch + L.R + rows));  // n_valid, counts, src_of, row_of
  L.tc = o;     o += al(8 * L.R);
  L.goc = o;    o += al(4 * L.R);
  L.lossc = o;  o += al(4 * L.R);
  L.zc = o;     o += al(4 * L.R);
  L.accc = o;   o += al(4 * L.R);
  L.xc = o;     o += al(2 * L.R * H);
  L.dxc = o;    o += al(2 * L.R * H);
  L.logits = o; o += al(2 * L.C * L.Vp);
  L.end = o;
  return L;
}

// ---------------------------------------------------------------- compaction
constexpr int kScanNT = 1024;

// One workgroup: the kept rows (target != ignore_index; a bad target is kept
// so that the cross-entropy flags it) in order, by a fixed-order prefix count.
// Writes n_valid, the kept rows per chunk, src_of[i] (original row of kept row
// i) and row_of[r] (kept index of row r, or -1).
__global__ __launch_bounds__(kScanNT) void compact_kernel(const int64_t* target, int64_t rows,
                                                          int64_t ignore_index, int64_t C,
                                                          int64_t nch, int* n_valid, int* counts,
                                                          int* src_of, int* row_of) {
  __shared__ int part[kScanNT];
  const int t = threadIdx.x;
  const int64_t per = (rows + kScanNT - 1) / kScanNT;
  const int64_t r0 = t * per, r1 = min(rows, r0 + per);
  int c = 0;
  for (int64_t r = r0; r < r1; ++r) c += (target[r] != ignore_index) ? 1 : 0;
  part[t] = c;
  __syncthreads();
  // Inclusive scan of part[] (Hillis-Steele; fixed order, deterministic).
  for (int d = 1; d < kScanNT; d <<= 1) {
    const int v = (t >= d) ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int pos = part[t] - c;  // exclusive prefix
  for (int64_t r = r0; r < r1; ++r) {
    if (target[r] != ignore_index) {
      src_of[pos] = static_cast<int>(r);
      row_of[r] = pos++;
    } else {
      row_of[r] = -1;
    }
  }
  const int total = part[kScanNT - 1];
  if (t == 0) *n_valid = total;
  for (int64_t ch = t; ch < nch; ch += kScanNT) {
    const int64_t left = total - ch * C;
    counts[ch] = static_cast<int>(left < 0 ? 0 : (left > C ? C : left));
  }
}

// One workgroup per compacted row i < R: the kept row's hidden state (zeros
// past n_valid), its target (ignore_index past n_valid) and, for a per-row
// grad_output, its value.
__global__ __launch_bounds__(256) void gather_kernel(const uint4* hidden, int64_t hvec,
                                                     const int64_t* target, const float* go,
                                                     int64_t go_stride, int64_t ignore_index,
                                                     const int* n_valid, const int* src_of,
                                                     uint4* xc, int64_t* tc, float* goc) {
  const int64_t i = blockIdx.x;
  const int src = (i < *n_valid) ? src_of[i] : -1;
  if (src >= 0) {
    for (int64_t v = threadIdx.x; v < hvec; v += blockDim.x)
      xc[i * hvec + v] = hidden[static_cast<int64_t>(src) * hvec + v];
  } else {
    for (int64_t v = threadIdx.x; v < hvec; v += blockDim.x)
      xc[i * hvec + v] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (threadIdx.x == 0) {
    tc[i] = src >= 0 ? target[src] : ignore_index;
    if (go && go_stride) goc[i] = src >= 0 ? go[src] : 0.0f;
  }
}

// Row r of dL/dh: the kept row's gradient, or zeros for an ignored row.
__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint4* dxc, int64_t hvec,
                                                           const int* row_of, uint4* out) {
  const int64_t r = blockIdx.x;
  const int i = row_of[r];
  if (i >= 0) {
    for (int64_t v = threadIdx.x; v < hvec; v += blockDim.x)
      out[r * hvec + v] = dxc[static_cast<int64_t>(i) * hvec + v];
  } else {
    for (int64_t v = threadIdx.x; v < hvec; v += blockDim.x)
      out[r * hvec + v] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Per-row outputs back in the caller's row order (0 for ignored rows).
__global__ __launch_bounds__(256) void scatter_floats_kernel(const float* in, const int* row_of,
                                                             int64_t rows, float* out) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int i = row_of[r];
  out[r] = i >= 0 ? in[i] : 0.0f;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_flce(const vsce_flce_problem* fp) {
  if (!fp) return VSCE_ERR_INVALID;
  if (fp->rows < 0 || fp->hidden < 64 || fp->hidden % 64 != 0 || fp->vocab < 1 ||
      fp->chunk_rows < 0)
    return VSCE_ERR_INVALID;
  if (fp->hidden > (int64_t(1) << 20) || fp->vocab > (int64_t(1) << 22) ||
      fp->rows > (int64_t(1) << 28))
    return VSCE_ERR_UNSUPPORTED;
  return VSCE_OK;
}

}  // namespace
}  // namespace vsce

using namespace vsce;

extern "C" {

int vsce_gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                   int64_t ldc, int64_t M, int64_t N, int64_t K, uint32_t layout,
                   int32_t out_mode, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || M > 0x7fffffffLL || N > 0x7fffffffLL || K > 0x7fffffffLL)
    return VSCE_ERR_INVALID;
  if (M > 0 && N > 0 && (!A || !B || !C || !al16(A) || !al16(B) || !al16(C)))
    return VSCE_ERR_INVALID;
  if (out_mode < VSCE_GEMM_OUT_BF16 || out_mode > VSCE_GEMM_OUT_F32_ADD) return VSCE_ERR_INVALID;
  if (layout & ~(VSCE_GEMM_A_K_MAJOR | VSCE_GEMM_B_K_MAJOR)) return VSCE_ERR_INVALID;
  GemmArgs g = {};
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  g.M = static_cast<int>(M);
  g.N = static_cast<int>(N);
  g.K = static_cast<int>(K);
  g.layout = static_cast<int>(layout);
  g.a_rows = (layout & VSCE_GEMM_A_K_MAJOR) ? g.K : g.M;
  g.b_rows = (layout & VSCE_GEMM_B_K_MAJOR) ? g.K : g.N;
  g.group_m = 8;
  return launch_gemm_nt(out_mode, g, stream);
}

int vsce_gemm_bf16_nt(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                      int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t out_mode,
                      hipStream_t stream) {
  return vsce_gemm_bf16(A, lda, B, ldb, C, ldc, M, N, K, 0u, out_mode, stream);
}

size_t vsce_flce_workspace_bytes(const vsce_flce_problem* problem) {
  if (check_flce(problem) != VSCE_OK) return 0;
  return static_cast<size_t>(
      layout(problem->rows, problem->hidden, problem->vocab, problem->chunk_rows).end);
}

int flce_forward_backward(const vsce_flce_problem* fp, const void* hidden, const void* weight,
                          const vsce_outputs* out, const float* grad_output,
                          int64_t grad_output_stride, void* grad_hidden, float* grad_weight,
                          void* workspace, hipStream_t stream) {
  int rc = check_flce(fp);
  if (rc != VSCE_OK) return rc;
  if (!out || !out->loss || !weight || !grad_weight || !workspace) return VSCE_ERR_INVALID;
  if (!al16(weight) || !al16(grad_weight) || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return VSCE_ERR_INVALID;
  if (fp->rows > 0 && (!fp->target || !hidden || !al16(hidden) || !grad_hidden ||
                      !al16(grad_hidden)))
    return VSCE_ERR_INVALID;
  if (grad_output_stride != 0 && grad_output_stride != 1) return VSCE_ERR_INVALID;
  const int64_t rows = fp->rows, H = fp->hidden, V = fp->vocab;
  const FlceLayout Lw = layout(rows, H, V, fp->chunk_rows);
  // The chunk's rows are the k extent of dL/dW's product (below 2^23).
  if (Lw.C >= (int64_t(1) << 23)) return VSCE_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);

  // The cross-entropy of one chunk of compacted rows: a [C, Vp] bf16 logits
  // buffer whose columns past V the products keep at zero.
  vsce_problem cp = {};
  cp.rows = Lw.C;
  cp.vocab = V;
  cp.row_stride = Lw.Vp;
  cp.dtype = VSCE_BF16;
  cp.reduction = fp->reduction;
  cp.target = reinterpret_cast<const int64_t*>(ws + Lw.tc);
  cp.class_weight = fp->class_weight;
  cp.ignore_index = fp->ignore_index;
  cp.label_smoothing = fp->label_smoothing;
  cp.softcap = fp->softcap;
  cp.z_loss = fp->z_loss;
  Prob pc;
  rc = check_problem(&cp, ws + Lw.logits, pc);
  if (rc != VSCE_OK) return rc;
  Prob pall = pc;  // the normalizers and the reduction see all R compacted rows
  pall.rows = Lw.R;

  int* n_valid = reinterpret_cast<int*>(ws + Lw.ints);
  int* counts = n_valid + 1;
  int* src_of = counts + Lw.nch;
  int* row_of = src_of + Lw.R;
  int64_t* tc = reinterpret_cast<int64_t*>(ws + Lw.tc);
  float* goc = reinterpret_cast<float*>(ws + Lw.goc);
  float* lossc = reinterpret_cast<float*>(ws + Lw.lossc);
  float* zc = reinterpret_cast<float*>(ws + Lw.zc);
  float* accc = reinterpret_cast<float*>(ws + Lw.accc);
  uint16_t* xc = reinterpret_cast<uint16_t*>(ws + Lw.xc);
  uint16_t* dxc = reinterpret_cast<uint16_t*>(ws + Lw.dxc);
  uint16_t* logits = reinterpret_cast<uint16_t*>(ws + Lw.logits);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws + Lw.ce);
  const int64_t hvec = H / 8;
  const bool none = fp->reduction == VSCE_REDUCTION_NONE;

  // 1. Compaction of the kept rows.
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(kScanNT), 0, stream, fp->target, rows,
                     fp->ignore_index, Lw.C, Lw.nch, n_valid, counts, src_of, row_of);
  hipLaunchKernelGGL(gather_kernel, dim3(static_cast<unsigned>(Lw.R)), dim3(256), 0, stream,
                     static_cast<const uint4*>(hidden), hvec, fp->target, grad_output,
                     grad_output_stride, fp->ignore_index, n_valid, src_of,
                     reinterpret_cast<uint4*>(xc), tc, goc);
  if (hipGetLastError() != hipSuccess) return VSCE_ERR_LAUNCH;
  // 2. Normalizers over all kept rows.
  rc = launch_prologue(pall, hdr, stream);
  if (rc != VSCE_OK) return rc;

  // Tile order of the products: groups of 8 m-tiles by all n-tiles, so the
  // 32 tiles one XCD runs at a time form an 8 x 4 block and share each
  // operand stage through that XCD's L2 (12 panels of A and B per stage
  // instead of 33 when the 32 tiles span one whole column of m-tiles).
  constexpr int kGroupM = 8;
  for (int64_t ch = 0; ch < Lw.nch; ++ch) {
    const int64_t c0 = ch * Lw.C;
    // 3. z = h W^T for the chunk's kept rows (bf16).
    GemmArgs g = {};
    g.A = xc + c0 * H;
    g.lda = H;
    g.a_rows = static_cast<int>(Lw.C);
    g.B = weight;
    g.ldb = H;
    g.b_rows = static_cast<int>(V);
    g.C = logits;
    g.ldc = Lw.Vp;
    g.M = static_cast<int>(Lw.C);
    g.N = static_cast<int>(Lw.Vp);
    g.K = static_cast<int>(H);
    g.group_m = kGroupM;
    g.m_count = counts + ch;
    rc = launch_gemm_nt(kGemmOutBf16, g, stream);
    if (rc != VSCE_OK) return rc;
    // 4. The cross-entropy; G = dL/dz over the logits.
    Prob p = pc;
    p.target = tc + c0;
    RowArgs a = {};
    a.x = logits;
    a.g = logits;
    problem_args(p, a);
    a.loss_rows = lossc + c0;
    a.acc_rows = accc + c0;
    a.z_rows = zc + c0;
    a.ws = hdr;
    rc = launch_fused_resident(p, a, stream);
    if (rc == VSCE_ERR_UNSUPPORTED) {  // rows too long for the chip: read twice
      a.stats = reinterpret_cast<float*>(ws + Lw.ce + stats_scratch_offset(Lw.R));
      rc = launch_stats(p, a, stream);
      if (rc == VSCE_OK) {
        RowArgs b = a;
        b.go = nullptr;
        rc = launch_backward(p, b, stream);
      }
    }
    if (rc != VSCE_OK) return rc;
    if (grad_output) {
      RowArgs sa = {};
      sa.g = logits;
      sa.stride = Lw.Vp;
      sa.V = V;
      sa.go = grad_output_stride ? goc + c0 : grad_output;
      sa.go_stride = grad_output_stride;
      sa.skip_if_one = 1;
      sa.rows = Lw.C;
      rc = launch_scale(p, sa, stream);
      if (rc != VSCE_OK) return rc;
    }
    // 5. dL/dh = G W for the kept rows: W read k-major (k = vocabulary
    // entry), its k-rows past V as zeros.
    GemmArgs d = {};
    d.A = logits;
    d.lda = Lw.Vp;
    d.a_rows = static_cast<int>(Lw.C);
    d.B = weight;
    d.ldb = H;
    d.b_rows = static_cast<int>(V);
    d.layout = kGemmBKMajor;
    d.C = dxc + c0 * H;
    d.ldc = H;
    d.M = static_cast<int>(Lw.C);
    d.N = static_cast<int>(H);
    d.K = static_cast<int>(Lw.Vp);
    d.group_m = kGroupM;
    d.m_count = counts + ch;
    rc = launch_gemm_nt(kGemmOutBf16, d, stream);
    if (rc != VSCE_OK) return rc;
    // 6. dL/dW (+)= G^T h over the chunk's kept rows: G and h read k-major
    // (k = kept row).
    GemmArgs w = {};
    w.A = logits;
    w.lda = Lw.Vp;
    w.a_rows = static_cast<int>(Lw.C);
    w.B = xc + c0 * H;
    w.ldb = H;
    w.b_rows = static_cast<int>(Lw.C);
    w.layout = kGemmAKMajor | kGemmBKMajor;
    w.C = grad_weight;
    w.ldc = H;
    w.M = static_cast<int>(V);
    w.N = static_cast<int>(H);
    w.K = static_cast<int>(Lw.C);
    w.group_m = kGroupM;
    w.k_count = counts + ch;
    rc = launch_gemm_nt(ch == 0 ? kGemmOutF32 : kGemmOutF32Add, w, stream);
    if (rc != VSCE_OK) return rc;
  }

  // 7. The reduction over all kept rows, then everything per row back in the
  // caller's order.
  rc = launch_finalize(pall, lossc, accc, zc, none ? nullptr : out->loss, out->acc_mean,
                       none ? nullptr : out->z_loss, hdr, stream);
  if (rc != VSCE_OK) return rc;
  if (rows > 0) {
    hipLaunchKernelGGL(scatter_rows_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0,
                       stream, reinterpret_cast<const uint4*>(dxc), hvec, row_of,
                       static_cast<uint4*>(grad_hidden));
    const dim3 fg(static_cast<unsigned>((rows + 255) / 256));
    float* per_row[4] = {none ? out->loss : nullptr, out->row_loss, out->token_acc,
                         none ? out->z_loss : nullptr};
    const float* src[4] = {lossc, lossc, accc, zc};
    for (int k = 0; k < 4; ++k)
      if (per_row[k])
        hipLaunchKernelGGL(scatter_floats_kernel, fg, dim3(256), 0, stream, src[k], row_of, rows,
                           per_row[k]);
    if (hipGetLastError() != hipSuccess) return VSCE_ERR_LAUNCH;
  }
  return VSCE_OK;
}

}  // extern "C"
