// The C ABI of libvsce.so (declared in include/vsce.h): argument checks,
// workspace layout and the launch sequence of each entry point.
//
// Every check happens before the first HIP call, so a rejected call enqueues
// nothing; the entry points never allocate, synchronize or read device data.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "common.h"
#include "launch.h"
#include "vsce.h"

namespace vsce {
namespace {

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int dt) {
  switch (dt) {
    case VSCE_F32: return 4;
    case VSCE_BF16:
    case VSCE_F16: return 2;
    default: return 0;
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

// Checks a problem descriptor and fills the derived fields.
int check_problem(const vsce_problem* pb, const void* logits, Prob& p) {
  if (!pb) return VSCE_ERR_INVALID;
  const int eb = elem_bytes(pb->dtype);
  if (eb == 0) return VSCE_ERR_INVALID;
  if (pb->rows < 0 || pb->vocab < 1 || pb->row_stride < pb->vocab) return VSCE_ERR_INVALID;
  if (pb->reduction < VSCE_REDUCTION_NONE || pb->reduction > VSCE_REDUCTION_SUM)
    return VSCE_ERR_INVALID;
  if ((pb->flags & ~VSCE_FLAG_LONG_ROWS_RING) != 0) return VSCE_ERR_INVALID;
  const float eps = pb->label_smoothing;
  if (!(eps >= 0.0f && eps <= 1.0f)) return VSCE_ERR_INVALID;  // also rejects NaN
  const float cap = pb->softcap, zl = pb->z_loss;
  if (!(cap >= 0.0f && cap <= 3.0e38f)) return VSCE_ERR_INVALID;  // finite, not NaN
  if (!(zl >= 0.0f && zl <= 3.0e38f)) return VSCE_ERR_INVALID;
  const int64_t voff = pb->vocab_offset;
  const int64_t Vt = pb->vocab_total == 0 ? pb->vocab : pb->vocab_total;
  if (voff < 0 || Vt < pb->vocab || voff > Vt - pb->vocab) return VSCE_ERR_INVALID;
  if (pb->rows > 0 && (!pb->target || !logits)) return VSCE_ERR_INVALID;
  if (logits && !aligned(logits, static_cast<uintptr_t>(eb))) return VSCE_ERR_INVALID;
  if (pb->class_weight && !aligned(pb->class_weight, 4)) return VSCE_ERR_INVALID;
  // Row byte offsets are 32-bit in the kernels; grids are 31-bit.
  if (pb->vocab * eb >= (int64_t(1) << 31) || Vt >= (int64_t(1) << 31)) return VSCE_ERR_UNSUPPORTED;
  if (pb->rows > 0x7fffffffLL) return VSCE_ERR_UNSUPPORTED;

  p.rows = pb->rows;
  p.V = pb->vocab;
  p.voff = voff;
  p.Vt = Vt;
  p.stride = pb->row_stride;
  p.dt = pb->dtype;
  p.red = pb->reduction;
  p.target = pb->target;
  p.weight = pb->class_weight;
  p.ignore_index = pb->ignore_index;
  p.eps = eps;
  p.eta = eps / static_cast<float>(Vt);
  p.cap = cap;
  p.zl = zl;
  p.elem_bytes = eb;
  p.flags = pb->flags;
  const int vec = 16 / eb;
  p.vec_ok = aligned(logits, 16) && (pb->row_stride * eb) % 16 == 0 && pb->vocab % vec == 0 &&
             (!pb->class_weight || aligned(pb->class_weight + voff, 16));
  return VSCE_OK;
}

// The constants of the soft-cap s (all zero when s = 0: no cap).
SoftCap soft_cap_constants(float s) {
  SoftCap c = {};
  if (s > 0.0f) {
    constexpr double log2e = 1.4426950408889634;
    c.s = s;
    c.k = static_cast<float>(-2.0 * log2e / s);
    c.ct = static_cast<float>(1.0 / (log2e * s));
    c.x0 = kCapCentral * s;
    c.qs = -0.25f * s;
    const double is2 = 1.0 / (static_cast<double>(s) * s);  // 1 / s^2
    c.c0 = static_cast<float>(kCapP0);
    c.c1 = static_cast<float>(kCapP1 * is2);
    c.c2 = static_cast<float>(kCapP2 * is2 * is2);
    c.c3 = static_cast<float>(kCapP3 * is2 * is2 * is2);
  }
  return c;
}

// The problem's fields every per-row kernel reads.  The kernels index the
// weights by this buffer's columns, so a shard sees its slice of them.
void problem_args(const Prob& p, RowArgs& a) {
  a.stride = p.stride;
  a.V = p.V;
  a.voff = p.voff;
  a.Vt = p.Vt;
  a.target = p.target;
  a.weight = p.weight ? p.weight + p.voff : nullptr;
  a.ignore_index = p.ignore_index;
  a.eps = p.eps;
  a.eta = p.eta;
  a.cap_c = soft_cap_constants(p.cap);
  a.zl = p.zl;
  a.mean = (p.red == VSCE_REDUCTION_MEAN);
  a.rows = p.rows;
}

int64_t stats_scratch_offset(int64_t rows) { return VSCE_WS_HEADER_BYTES + 3 * align_up(4 * rows); }

namespace {

// The entry points that see whole rows (loss, fused gradient) take no shard.
bool whole_rows(const Prob& p) { return p.voff == 0 && p.Vt == p.V; }

int check_workspace(const void* ws) {
  if (!ws || !aligned(ws, kAlign)) return VSCE_ERR_INVALID;
  return VSCE_OK;
}

int check_outputs(const vsce_outputs* out) {
  if (!out || !out->loss) return VSCE_ERR_INVALID;
  return VSCE_OK;
}

// The workspace after its header: [rows] fp32 scratch for the row losses, the
// accuracies and the z-losses (each used when the caller's outputs do not take
// its place), then [rows] float4 statistics (the fused mode's rows that are
// read twice).

// Per-row destinations of the forward kernels.
RowArgs row_args(const Prob& p, void* x, const vsce_outputs* out, void* workspace) {
  RowArgs a = {};
  char* ws = static_cast<char*>(workspace);
  float* loss_scratch = reinterpret_cast<float*>(ws + VSCE_WS_HEADER_BYTES);
  float* acc_scratch =
      reinterpret_cast<float*>(ws + VSCE_WS_HEADER_BYTES + align_up(4 * p.rows));
  float* z_scratch =
      reinterpret_cast<float*>(ws + VSCE_WS_HEADER_BYTES + 2 * align_up(4 * p.rows));
  a.x = x;
  a.g = x;
  problem_args(p, a);
  if (p.red == VSCE_REDUCTION_NONE) {
    a.loss_rows = out->loss;
    a.loss_rows2 = out->row_loss;
    a.z_rows = out->z_loss;
  } else {
    a.loss_rows = out->row_loss ? out->row_loss : loss_scratch;
    // The mean splits the loss into its parts; the sum only needs them for
    // the z-loss output.
    a.z_rows = (p.zl != 0.0f || out->z_loss) ? z_scratch : nullptr;
  }
  a.acc_rows = out->token_acc ? out->token_acc : (out->acc_mean ? acc_scratch : nullptr);
  a.ws = reinterpret_cast<const WsHeader*>(ws);
  return a;
}

int forward_common(const Prob& p, RowArgs a, const vsce_outputs* out, void* workspace,
                   bool fused, hipStream_t stream, hipEvent_t ev_begin = nullptr,
                   hipEvent_t ev_end = nullptr) {
  WsHeader* hdr = reinterpret_cast<WsHeader*>(workspace);
  int rc = launch_prologue(p, hdr, stream);
  if (rc != VSCE_OK) return rc;
  if (ev_begin && hipEventRecord(ev_begin, stream) != hipSuccess) return VSCE_ERR_LAUNCH;
  if (p.rows > 0) {
    if (fused) {
      rc = launch_fused_resident(p, a, stream);
      if (rc == VSCE_ERR_UNSUPPORTED && (p.flags & VSCE_FLAG_LONG_ROWS_RING))
        rc = launch_fused_ring(p, a, stream);
      if (rc == VSCE_ERR_UNSUPPORTED) {
        // Rows read twice: the statistics into the workspace, then the
        // gradient in place (grad_output 1).
        a.stats = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           stats_scratch_offset(p.rows));
        rc = launch_stats(p, a, stream);
        if (rc == VSCE_OK) {
          RowArgs b = a;
          b.g = a.x;
          b.go = nullptr;
          b.go_stride = 0;
          rc = launch_backward(p, b, stream);
        }
      }
    } else {
      rc = launch_stats(p, a, stream);
    }
    if (rc != VSCE_OK) return rc;
  }
  if (ev_end && hipEventRecord(ev_end, stream) != hipSuccess) return VSCE_ERR_LAUNCH;
  return launch_finalize(p, a.loss_rows, a.acc_rows, a.z_rows, out->loss, out->acc_mean,
                         p.red == VSCE_REDUCTION_NONE ? nullptr : out->z_loss, hdr, stream);
}

}  // namespace

int launch_fused_resident(const Prob& p, RowArgs a, hipStream_t s) {
  if (!p.vec_ok) return VSCE_ERR_UNSUPPORTED;
  a.nvec = p.V / (16 / p.elem_bytes);
  const bool cap = p.cap > 0.0f;
  switch (p.dt) {
    case VSCE_F32:
      return cap ? fused_resident_dt<VSCE_F32, true>(p, a, s)
                 : fused_resident_dt<VSCE_F32, false>(p, a, s);
    case VSCE_BF16:
      return cap ? fused_resident_dt<VSCE_BF16, true>(p, a, s)
                 : fused_resident_dt<VSCE_BF16, false>(p, a, s);
    case VSCE_F16:
      return cap ? fused_resident_dt<VSCE_F16, true>(p, a, s)
                 : fused_resident_dt<VSCE_F16, false>(p, a, s);
    default: return VSCE_ERR_INVALID;
  }
}

namespace {
int stream_any(int which, const Prob& p, const RowArgs& a, hipStream_t s) {
  const bool cap = p.cap > 0.0f && which != kStreamScale;
  switch (p.dt) {
    case VSCE_F32:
      return cap ? stream_dt<VSCE_F32, true>(which, p, a, s)
                 : stream_dt<VSCE_F32, false>(which, p, a, s);
    case VSCE_BF16:
      return cap ? stream_dt<VSCE_BF16, true>(which, p, a, s)
                 : stream_dt<VSCE_BF16, false>(which, p, a, s);
    case VSCE_F16:
      return cap ? stream_dt<VSCE_F16, true>(which, p, a, s)
                 : stream_dt<VSCE_F16, false>(which, p, a, s);
    default: return VSCE_ERR_INVALID;
  }
}
}  // namespace

int launch_stats(const Prob& p, RowArgs a, hipStream_t s) {
  return stream_any(kStreamStats, p, a, s);
}
int launch_fused_ring(const Prob& p, RowArgs a, hipStream_t s) {
  if (!p.vec_ok || p.weight) return VSCE_ERR_UNSUPPORTED;
  return stream_any(kStreamRing, p, a, s);
}
int launch_backward(const Prob& p, RowArgs a, hipStream_t s) {
  return stream_any(kStreamBackward, p, a, s);
}
int launch_scale(const Prob& p, RowArgs a, hipStream_t s) {
  return stream_any(kStreamScale, p, a, s);
}

// ---------------------------------------------------------------- static workspace
// The workspace of ce_forward_fused_inplace_noalloc: one array per device, in
// the library's device code object, sized for kStaticMaxRows rows.  In host
// code `scratch` names a host-side stand-in, not device memory: host code
// only ever uses the device address hipGetSymbolAddress gives for it, looked
// up once per device (with that device current) and kept.
namespace {

constexpr int64_t kStaticMaxRows = VSCE_NOALLOC_MAX_ROWS;
constexpr int64_t kStaticBytes =
    VSCE_WS_HEADER_BYTES + 3 * ((4 * kStaticMaxRows + kAlign - 1) / kAlign * kAlign) +
    (16 * kStaticMaxRows + kAlign - 1) / kAlign * kAlign;

__device__ __align__(256) unsigned char scratch[kStaticBytes];

constexpr int kMaxDevices = 64;

// This device's copy of `scratch`, or null if the lookup fails.
void* static_scratch() {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace

}  // namespace vsce

using namespace vsce;

extern "C" {

size_t vsce_workspace_bytes(int64_t rows) {
  if (rows < 0) return 0;
  return static_cast<size_t>(stats_scratch_offset(rows) + align_up(16 * rows));
}

int ce_forward_fused_inplace(const vsce_problem* problem, void* logits_inout,
                             const vsce_outputs* out, void* workspace, hipStream_t stream) {
  Prob p;
  int rc = check_problem(problem, logits_inout, p);
  if (rc == VSCE_OK && !whole_rows(p)) rc = VSCE_ERR_INVALID;
  if (rc == VSCE_OK) rc = check_outputs(out);
  if (rc == VSCE_OK) rc = check_workspace(workspace);
  if (rc != VSCE_OK) return rc;
  return forward_common(p, row_args(p, logits_inout, out, workspace), out, workspace, true,
                        stream);
}

int ce_forward_fused_inplace_timed(const vsce_problem* problem, void* logits_inout,
                                   const vsce_outputs* out, void* workspace, hipStream_t stream,
                                   hipEvent_t begin, hipEvent_t end) {
  Prob p;
  int rc = check_problem(problem, logits_inout, p);
  if (rc == VSCE_OK && !whole_rows(p)) rc = VSCE_ERR_INVALID;
  if (rc == VSCE_OK) rc = check_outputs(out);
  if (rc == VSCE_OK) rc = check_workspace(workspace);
  if (rc != VSCE_OK) return rc;
  return forward_common(p, row_args(p, logits_inout, out, workspace), out, workspace, true,
                        stream, begin, end);
}

int ce_forward_fused_inplace_noalloc(const vsce_problem* problem, void* logits_inout,
                                     const vsce_outputs* out, hipStream_t stream) {
  static_assert(kStaticBytes >= VSCE_WS_HEADER_BYTES, "static workspace");
  Prob p;
  int rc = check_problem(problem, logits_inout, p);
  if (rc == VSCE_OK && !whole_rows(p)) rc = VSCE_ERR_INVALID;
  if (rc == VSCE_OK) rc = check_outputs(out);
  if (rc != VSCE_OK) return rc;
  if (p.rows > kStaticMaxRows) return VSCE_ERR_TOO_LARGE;
  // The layout of a workspace of vsce_workspace_bytes(rows) bytes, inside
  // the array sized for kStaticMaxRows (every offset grows with rows).
  void* ws = static_scratch();
  if (ws == nullptr) return VSCE_ERR_LAUNCH;
  return forward_common(p, row_args(p, logits_inout, out, ws), out, ws, true, stream);
}

int ce_forward_stats(const vsce_problem* problem, const void* logits, float* stats,
                     const vsce_outputs* out, void* workspace, hipStream_t stream) {
  Prob p;
  int rc = check_problem(problem, logits, p);
  if (rc == VSCE_OK && !whole_rows(p)) rc = VSCE_ERR_INVALID;
  if (rc == VSCE_OK) rc = check_outputs(out);
  if (rc == VSCE_OK) rc = check_workspace(workspace);
  if (rc == VSCE_OK && p.rows > 0 && (!stats || !aligned(stats, 16))) rc = VSCE_ERR_INVALID;
  if (rc != VSCE_OK) return rc;
  RowArgs a = row_args(p, const_cast<void*>(logits), out, workspace);
  a.stats = stats;
  return forward_common(p, a, out, workspace, false, stream);
}

int ce_forward_stats_partial(const vsce_problem* problem, const void* logits, float* partial,
                             hipStream_t stream) {
  Prob p;
  int rc = check_problem(problem, logits, p);
  if (rc != VSCE_OK) return rc;
  if (p.rows == 0) return VSCE_OK;
  if (!partial || !aligned(partial, 16)) return VSCE_ERR_INVALID;
  RowArgs a = {};
  a.x = const_cast<void*>(logits);
  problem_args(p, a);
  a.partial = partial;
  return launch_stats(p, a, stream);
}

int ce_merge_stats(const vsce_problem* problem, const float* partials, int32_t shards,
                   float* stats, const vsce_outputs* out, void* workspace, hipStream_t stream) {
  Prob p;
  // The merge reads no logits: check the problem as if it had an aligned buffer.
  int rc = check_problem(problem, reinterpret_cast<const void*>(uintptr_t{256}), p);
  if (rc == VSCE_OK && !whole_rows(p)) rc = VSCE_ERR_INVALID;
  if (rc == VSCE_OK) rc = check_outputs(out);
  if (rc == VSCE_OK) rc = check_workspace(workspace);
  if (rc != VSCE_OK) return rc;
  if (shards < 1) return VSCE_ERR_INVALID;
  if (p.rows > 0 && (!partials || !stats || !aligned(partials, 16) || !aligned(stats, 16)))
    return VSCE_ERR_INVALID;
  RowArgs a = row_args(p, nullptr, out, workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(workspace);
  rc = launch_prologue(p, hdr, stream);
  if (rc == VSCE_OK) rc = launch_merge(p, partials, shards, stats, a, stream);
  if (rc != VSCE_OK) return rc;
  return launch_finalize(p, a.loss_rows, a.acc_rows, a.z_rows, out->loss, out->acc_mean,
                         p.red == VSCE_REDUCTION_NONE ? nullptr : out->z_loss, hdr, stream);
}

int ce_backward_from_stats(const vsce_problem* problem, const void* logits, void* grad,
                           const float* stats, const float* grad_output,
                           int64_t grad_output_stride, const void* workspace,
                           hipStream_t stream) {
  Prob p;
  int rc = check_problem(problem, logits, p);
  if (rc == VSCE_OK) rc = check_workspace(workspace);
  if (rc != VSCE_OK) return rc;
  if (p.rows == 0) return VSCE_OK;
  if (!grad || !aligned(grad, static_cast<uintptr_t>(p.elem_bytes))) return VSCE_ERR_INVALID;
  if (!stats || !aligned(stats, 16) || !grad_output) return VSCE_ERR_INVALID;
  if (grad_output_stride != 0 && grad_output_stride != 1) return VSCE_ERR_INVALID;
  // The vector path needs the output aligned like the input.
  if (p.vec_ok && !aligned(grad, 16)) p.vec_ok = false;
  RowArgs a = {};
  a.x = const_cast<void*>(logits);
  a.g = grad;
  problem_args(p, a);
  a.stats = const_cast<float*>(stats);
  a.go = grad_output;
  a.go_stride = grad_output_stride;
  a.ws = static_cast<const WsHeader*>(workspace);
  return launch_backward(p, a, stream);
}

int ce_scale_grad(void* grad, int64_t rows, int64_t vocab, int64_t row_stride, int32_t dtype,
                  const float* grad_output, int64_t grad_output_stride, int32_t skip_if_one,
                  hipStream_t stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0 || rows < 0 || vocab < 1 || row_stride < vocab) return VSCE_ERR_INVALID;
  if (grad_output_stride != 0 && grad_output_stride != 1) return VSCE_ERR_INVALID;
  if (rows == 0) return VSCE_OK;
  if (!grad || !grad_output || !aligned(grad, static_cast<uintptr_t>(eb))) return VSCE_ERR_INVALID;
  if (vocab * eb >= (int64_t(1) << 31) || rows > 0x7fffffffLL) return VSCE_ERR_UNSUPPORTED;
  Prob p = {};
  p.rows = rows;
  p.V = vocab;
  p.stride = row_stride;
  p.dt = dtype;
  p.elem_bytes = eb;
  p.vec_ok = aligned(grad, 16) && (row_stride * eb) % 16 == 0 && vocab % (16 / eb) == 0;
  RowArgs a = {};
  a.g = grad;
  a.stride = row_stride;
  a.V = vocab;
  a.go = grad_output;
  a.go_stride = grad_output_stride;
  a.skip_if_one = skip_if_one != 0;
  a.rows = rows;
  return launch_scale(p, a, stream);
}

const char* vsce_strerror(int code) {
  switch (code) {
    case VSCE_OK: return "ok";
    case VSCE_ERR_INVALID: return "invalid argument";
    case VSCE_ERR_UNSUPPORTED: return "unsupported combination";
    case VSCE_ERR_LAUNCH: return "kernel launch failed";
    case VSCE_ERR_TOO_LARGE: return "more rows than the static workspace holds";
    default: return "unknown error";
  }
}

int vsce_version(void) { return 300; }

}  // extern "C"
