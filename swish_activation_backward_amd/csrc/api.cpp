// C ABI of the SwiGLU backward / Swish-gradient library: argument validation, launch
// planning and dispatch.  Every check happens on the host before anything is enqueued;
// the rules follow the SwishGrad page's aclnn interface (section 3.3: NULL tensors ->
// null-pointer error, bad dtype or shape -> invalid-parameter error; section 3.5:
// empty tensors return success without running anything; a missing beta means 1.0)
// and the Fused SwiGLU backward page's kernel signatures (section "Kernel 签名与参数规格").
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "../../include/swiglu_bwd.h"
#include "launch.hpp"
#include "plan.hpp"

using namespace swg;

namespace {

thread_local int g_last_hip_error = 0;

bool dtype_ok(int dt) { return dt == SWG_BF16 || dt == SWG_FP16 || dt == SWG_FP32; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

swg_status hip_status(hipError_t e) {
  if (e == hipSuccess) return SWG_OK;
  g_last_hip_error = (int)e;
  return SWG_ERR_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

thread_local swg::CallTiming g_timing;

// Clears the timing events when an entry point returns (they time one call only).
struct TimedCall {
  ~TimedCall() { g_timing = swg::CallTiming{}; }
};

// A buffer as a byte range [p, p + bytes); bytes = 0 marks an absent buffer.
struct Span {
  const void* p;
  int64_t bytes;
};

// rows x cols elements of es bytes; -1 when the byte count overflows int64
int64_t span_bytes(int64_t rows, int64_t cols, int64_t es) {
  int64_t n;
  if (__builtin_mul_overflow(rows, cols, &n) || __builtin_mul_overflow(n, es, &n)) return -1;
  return n;
}

bool spans_meet(const Span& a, const Span& b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes <= 0 || b.bytes <= 0) return false;
  const __int128 a0 = (__int128)reinterpret_cast<uintptr_t>(a.p), b0 =
      (__int128)reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Every output span must be disjoint from every other span (inputs may share memory with
// each other: they are only read).  False also when a byte count overflowed.
template <size_t NO, size_t NI>
bool outputs_disjoint(const Span (&outs)[NO], const Span (&ins)[NI]) {
  for (const Span& o : outs)
    if (o.bytes < 0) return false;
  for (const Span& i : ins)
    if (i.bytes < 0) return false;
  for (size_t a = 0; a < NO; ++a) {
    for (size_t b = a + 1; b < NO; ++b)
      if (spans_meet(outs[a], outs[b])) return false;
    for (size_t b = 0; b < NI; ++b)
      if (spans_meet(outs[a], ins[b])) return false;
  }
  return true;
}

// Compute units of the current device (cached per device; 0 if the query fails, in
// which case the launch uses one workgroup per tile).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int gemm_grid_cap() {
  const int cus = device_cus();
  return cus > 0 ? cus : (1 << 30);
}

}  // namespace

swg::CallTiming& swg::call_timing() { return g_timing; }

namespace {
// swg_set_gemm_tile's setting for this thread: 4 or 2 (tile edge / 64), 0 = planner
thread_local int g_tile_f = 0;
}  // namespace

extern "C" {

swg_status swg_set_gemm_tile(int edge) {
  if (edge != 0 && edge != 128 && edge != 256) return SWG_ERR_INVALID;
  g_tile_f = edge / 64;
  return SWG_OK;
}

swg_status swg_time_next_call(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return SWG_ERR_INVALID;
  g_timing.start = reinterpret_cast<hipEvent_t>(start_event);
  g_timing.stop = reinterpret_cast<hipEvent_t>(stop_event);
  return SWG_OK;
}

const char* swg_version(void) { return "swiglu_bwd 0.1.0 gfx950"; }

const char* swg_status_string(int status) {
  switch (status) {
    case SWG_OK: return "SWG_OK";
    case SWG_ERR_NULLPTR: return "SWG_ERR_NULLPTR: a required pointer is NULL";
    case SWG_ERR_INVALID: return "SWG_ERR_INVALID: negative size, unknown dtype or misaligned pointer";
    case SWG_ERR_UNSUPPORTED: return "SWG_ERR_UNSUPPORTED: dtype or shape not implemented by this call";
    case SWG_ERR_WORKSPACE: return "SWG_ERR_WORKSPACE: workspace smaller than the size query";
    case SWG_ERR_HIP: return "SWG_ERR_HIP: a HIP launch failed (see swg_last_hip_error)";
    default: return "unknown swg_status";
  }
}

int swg_last_hip_error(void) { return g_last_hip_error; }

// ------------------------------------------------------------------- swish_grad
swg_status swish_grad(const void* grad, const void* x, void* grad_x, int64_t n, swg_dtype dtype,
                      const float* beta, void* stream) {
  TimedCall timed_;
  if (!dtype_ok(dtype) || n < 0) return SWG_ERR_INVALID;
  if (n == 0) return SWG_OK;
  if (grad == nullptr || x == nullptr || grad_x == nullptr) return SWG_ERR_NULLPTR;
  const size_t es = (size_t)elem_size(dtype);
  if (!aligned(grad, es) || !aligned(x, es) || !aligned(grad_x, es)) return SWG_ERR_INVALID;
  // only exact aliasing of the output with an input is allowed
  const uintptr_t o = reinterpret_cast<uintptr_t>(grad_x);
  const uintptr_t bytes = (uintptr_t)n * es;
  for (const void* in : {grad, x}) {
    const uintptr_t i = reinterpret_cast<uintptr_t>(in);
    if (i != o && i < o + bytes && o < i + bytes) return SWG_ERR_INVALID;
  }
  const float b = beta ? *beta : 1.0f;
  const bool vec = aligned(grad, 16) && aligned(x, 16) && aligned(grad_x, 16);
  return hip_status(launch_swish_grad(dtype, grad, x, grad_x, n, b, vec, as_stream(stream)));
}

// ------------------------------------------------------------------- strided swish_grad
swg_status swish_grad_strided(const void* grad, const void* x, void* grad_x, int ndim,
                              const int64_t* sizes, const int64_t* grad_strides,
                              const int64_t* x_strides, const int64_t* out_strides,
                              swg_dtype dtype, const float* beta, void* stream) {
  TimedCall timed_;
  if (!dtype_ok(dtype) || ndim < 0 || ndim > SWG_MAX_NDIM) return SWG_ERR_INVALID;
  if (ndim > 0 && (!sizes || !grad_strides || !x_strides || !out_strides))
    return SWG_ERR_NULLPTR;
  int64_t n = 1;
  for (int d = 0; d < ndim; ++d) {
    if (sizes[d] < 0) return SWG_ERR_INVALID;
    if (__builtin_mul_overflow(n, sizes[d], &n)) return SWG_ERR_INVALID;
  }
  if (n == 0) return SWG_OK;
  if (!grad || !x || !grad_x) return SWG_ERR_NULLPTR;
  const int64_t es = elem_size(dtype);
  if (!aligned(grad, (size_t)es) || !aligned(x, (size_t)es) || !aligned(grad_x, (size_t)es))
    return SWG_ERR_INVALID;
  const int64_t* st[3] = {grad_strides, x_strides, out_strides};
  // every view's byte span must be representable: |stride| and (size - 1) * stride * es
  // for each dimension, and their sums, without int64 overflow
  for (int t = 0; t < 3; ++t) {
    int64_t lo = 0, hi = 0;
    for (int d = 0; d < ndim; ++d) {
      int64_t e;
      if (st[t][d] == INT64_MIN || __builtin_mul_overflow(sizes[d] - 1, st[t][d], &e) ||
          __builtin_mul_overflow(e, es, &e) ||
          __builtin_add_overflow(e < 0 ? lo : hi, e, e < 0 ? &lo : &hi))
        return SWG_ERR_INVALID;
    }
  }

  // the output's elements must not overlap each other: with its dimensions of size > 1
  // sorted by |stride|, each stride must exceed the extent spanned by the smaller ones
  {
    int64_t ord[SWG_MAX_NDIM];
    int m = 0;
    for (int d = 0; d < ndim; ++d)
      if (sizes[d] > 1) {
        const int64_t a = out_strides[d] < 0 ? -out_strides[d] : out_strides[d];
        int k = m++;
        while (k > 0) {
          const int64_t b = out_strides[ord[k - 1]] < 0 ? -out_strides[ord[k - 1]]
                                                       : out_strides[ord[k - 1]];
          if (b <= a) break;
          ord[k] = ord[k - 1];
          --k;
        }
        ord[k] = d;
      }
    int64_t extent = 0;
    for (int k = 0; k < m; ++k) {
      const int d = (int)ord[k];
      const int64_t a = out_strides[d] < 0 ? -out_strides[d] : out_strides[d];
      if (a <= extent) return SWG_ERR_INVALID;
      int64_t span;
      if (__builtin_mul_overflow(sizes[d] - 1, a, &span) ||
          __builtin_add_overflow(extent, span, &extent))
        return SWG_ERR_INVALID;
    }
  }
  // byte span [lo, hi] of each view; the output may meet an input only as the same view
  {
    auto span = [&](const void* p, const int64_t* s, __int128& lo, __int128& hi) {
      int64_t a = 0, b = 0;   // no overflow: checked above
      for (int d = 0; d < ndim; ++d) {
        const int64_t e = (sizes[d] - 1) * s[d] * es;
        if (e < 0) a += e; else b += e;
      }
      lo = (__int128)reinterpret_cast<uintptr_t>(p) + a;
      hi = (__int128)reinterpret_cast<uintptr_t>(p) + b + es - 1;
    };
    __int128 olo, ohi;
    span(grad_x, out_strides, olo, ohi);
    const void* ins[2] = {grad, x};
    for (int t = 0; t < 2; ++t) {
      __int128 lo, hi;
      span(ins[t], st[t], lo, hi);
      if (lo > ohi || olo > hi) continue;   // disjoint
      bool same = ins[t] == grad_x;
      for (int d = 0; same && d < ndim; ++d) same = sizes[d] == 1 || st[t][d] == out_strides[d];
      if (!same) return SWG_ERR_INVALID;
    }
  }
  // merge dimensions (innermost first) that are contiguous in all three tensors; drop
  // dimensions of size 1
  StridedView v;
  int64_t msize[SWG_MAX_NDIM], mst[3][SWG_MAX_NDIM];
  int nd = 0;
  for (int d = ndim - 1; d >= 0; --d) {
    if (sizes[d] == 1) continue;
    if (nd > 0) {
      const int c = nd - 1;
      bool merge = true;
      for (int t = 0; t < 3; ++t) merge = merge && st[t][d] == mst[t][c] * msize[c];
      if (merge) {
        msize[c] *= sizes[d];
        continue;
      }
    }
    msize[nd] = sizes[d];
    for (int t = 0; t < 3; ++t) mst[t][nd] = st[t][d];
    ++nd;
  }
  const float b = beta ? *beta : 1.0f;
  if (nd == 0 || (nd == 1 && mst[0][0] == 1 && mst[1][0] == 1 && mst[2][0] == 1)) {
    const bool vec = aligned(grad, 16) && aligned(x, 16) && aligned(grad_x, 16);
    return hip_status(launch_swish_grad(dtype, grad, x, grad_x, n, b, vec, as_stream(stream)));
  }
  if (nd > kMaxStridedDims) return SWG_ERR_UNSUPPORTED;
  v.nd = nd;
  for (int k = 0; k < nd; ++k) {   // back to outermost-first order
    v.size[k] = msize[nd - 1 - k];
    for (int t = 0; t < 3; ++t) v.stride[t][k] = mst[t][nd - 1 - k];
  }
  return hip_status(launch_swish_grad_strided(dtype, grad, x, grad_x, v, n, b,
                                              as_stream(stream)));
}

// ------------------------------------------------------------------- b stage
size_t swiglu_bwd_b_workspace_size(int64_t M, int64_t N, swg_dtype dtype) {
  if (!dtype_ok(dtype) || M <= 0 || N <= 0) return 0;
  return plan_b(M, N, dtype, true).ws_bytes;
}

// Argument checks shared by swiglu_bwd_b and swiglu_bwd_b_noalloc (workspace: the
// caller's, or NULL with ws_bytes 0 for the static scratch); fills the plan.
static swg_status b_checks(const void* dy, const void* g, const void* fc, void* dg, void* dfc,
                           void* db_g, void* db_fc, int64_t M, int64_t N, int dtype,
                           const void* workspace, size_t workspace_bytes, bool own_ws,
                           BPlan* plan) {
  if (!dtype_ok(dtype) || M < 0 || N < 0) return SWG_ERR_INVALID;
  if (M == 0 || N == 0) return SWG_OK;  // dg/dfc empty; db += empty sum
  if (!dy || !g || !fc || !dg || !dfc || !db_g || !db_fc) return SWG_ERR_NULLPTR;
  const size_t es = (size_t)elem_size(dtype);
  for (const void* p : {dy, g, fc, (const void*)dg, (const void*)dfc, (const void*)db_g,
                        (const void*)db_fc})
    if (!aligned(p, es)) return SWG_ERR_INVALID;
  const bool vec = aligned(dy, 16) && aligned(g, 16) && aligned(fc, 16) && aligned(dg, 16) &&
                   aligned(dfc, 16);
  *plan = plan_b(M, N, dtype, vec);
  if (own_ws) {
    if (workspace_bytes < plan->ws_bytes) return SWG_ERR_WORKSPACE;
    if (plan->ws_bytes > 0 && workspace == nullptr) return SWG_ERR_NULLPTR;
    if (!aligned(workspace, 16)) return SWG_ERR_INVALID;
  } else if (plan->ws_bytes > kBScratchBytes) {
    return SWG_ERR_WORKSPACE;   // the partials would not fit the static scratch
  }
  const int64_t t = span_bytes(M, N, (int64_t)es), v = span_bytes(1, N, (int64_t)es);
  const Span outs[] = {{dg, t}, {dfc, t}, {db_g, v}, {db_fc, v},
                       {own_ws ? workspace : nullptr, (int64_t)plan->ws_bytes}};
  const Span ins[] = {{dy, t}, {g, t}, {fc, t}};
  if (!outputs_disjoint(outs, ins)) return SWG_ERR_INVALID;
  return SWG_OK;
}

swg_status swiglu_bwd_b(const void* dy, const void* g, const void* fc, void* dg, void* dfc,
                        void* db_g, void* db_fc, int64_t M, int64_t N, swg_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  TimedCall timed_;
  BPlan p{};
  const swg_status st = b_checks(dy, g, fc, dg, dfc, db_g, db_fc, M, N, dtype, workspace,
                                 workspace_bytes, true, &p);
  if (st != SWG_OK || M == 0 || N == 0) return st;
  return hip_status(launch_b_stage(dtype, p, dy, g, fc, dg, dfc, db_g, db_fc, M, N,
                                   static_cast<float*>(workspace), as_stream(stream)));
}

swg_status swiglu_bwd_b_noalloc(const void* dy, const void* g, const void* fc, void* dg,
                                void* dfc, void* db_g, void* db_fc, int64_t M, int64_t N,
                                swg_dtype dtype, void* stream) {
  TimedCall timed_;
  BPlan p{};
  const swg_status st = b_checks(dy, g, fc, dg, dfc, db_g, db_fc, M, N, dtype, nullptr, 0,
                                 false, &p);
  if (st != SWG_OK || M == 0 || N == 0) return st;
  // every walker writes its whole partial row, so the scratch needs no clearing
  float* part = nullptr;
  const hipError_t e = b_scratch(&part);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_b_stage(dtype, p, dy, g, fc, dg, dfc, db_g, db_fc, M, N, part,
                                   as_stream(stream)));
}

// ------------------------------------------------------------------- GEMM stages
// fp32_ok: the w and x stages have an fp32 path (K, N multiples of 4: 16-byte vectors);
// the 16-bit paths need K, N multiples of 8.
static swg_status gemm_shape_check(int dtype, int64_t M, int64_t K, int64_t N,
                                   bool fp32_ok = false) {
  if (!dtype_ok(dtype) || M < 0 || K < 0 || N < 0) return SWG_ERR_INVALID;
  if (dtype == SWG_FP32 && !fp32_ok) return SWG_ERR_UNSUPPORTED;
  const int64_t vec = dtype == SWG_FP32 ? 4 : 8;
  if (K % vec != 0 || N % vec != 0) return SWG_ERR_UNSUPPORTED;
  // tile windows are addressed with 32-bit byte offsets (256 rows of 2N bytes) and
  // row indices in 32 bits
  if (K >= kMaxGemmDim || N >= kMaxGemmDim || M >= (int64_t(1) << 31)) return SWG_ERR_UNSUPPORTED;
  return SWG_OK;
}

size_t swiglu_bwd_w_workspace_size(int64_t M, int64_t K, int64_t N, swg_dtype dtype) {
  if (gemm_shape_check(dtype, M, K, N, true) != SWG_OK || M == 0 || K == 0 || N == 0) return 0;
  return plan_w(M, K, N, g_tile_f).ws_bytes;
}

swg_status swiglu_bwd_w(const void* x, const void* dg, const void* dfc, void* dw_g, void* dw_fc,
                        int64_t M, int64_t K, int64_t N, swg_dtype dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  TimedCall timed_;
  swg_status st = gemm_shape_check(dtype, M, K, N, true);
  if (st != SWG_OK) return st;
  if (M == 0 || K == 0 || N == 0) return SWG_OK;  // dw += empty sum
  if (!x || !dg || !dfc || !dw_g || !dw_fc) return SWG_ERR_NULLPTR;
  for (const void* p : {x, dg, dfc}) if (!aligned(p, 16)) return SWG_ERR_UNSUPPORTED;
  for (const void* p : {(const void*)dw_g, (const void*)dw_fc}) if (!aligned(p, 8)) return SWG_ERR_UNSUPPORTED;
  const WPlan p = plan_w(M, K, N, g_tile_f);
  if (workspace_bytes < p.ws_bytes) return SWG_ERR_WORKSPACE;
  if (p.ws_bytes > 0 && workspace == nullptr) return SWG_ERR_NULLPTR;
  if (!aligned(workspace, 16)) return SWG_ERR_INVALID;
  {
    const int64_t es = elem_size(dtype);
    const int64_t w = span_bytes(K, N, es), d = span_bytes(M, N, es);
    const Span outs[] = {{dw_g, w}, {dw_fc, w}, {workspace, (int64_t)p.ws_bytes}};
    const Span ins[] = {{x, span_bytes(M, K, es)}, {dg, d}, {dfc, d}};
    if (!outputs_disjoint(outs, ins)) return SWG_ERR_INVALID;
  }
  return hip_status(launch_w_stage(dtype, p, x, dg, dfc, dw_g, dw_fc, M, K, N,
                                   static_cast<float*>(workspace), gemm_grid_cap(),
                                   as_stream(stream)));
}

swg_status swiglu_bwd_x(const void* dg, const void* dfc, const void* w_g, const void* w_fc,
                        void* dx, int64_t M, int64_t K, int64_t N, swg_dtype dtype, void* stream) {
  TimedCall timed_;
  swg_status st = gemm_shape_check(dtype, M, K, N, true);
  if (st != SWG_OK) return st;
  if (M == 0 || K == 0) return SWG_OK;  // dx is empty
  if (!dx) return SWG_ERR_NULLPTR;
  if (!aligned(dx, 16)) return SWG_ERR_UNSUPPORTED;
  if (N == 0)  // the empty sum: dx = 0
    return hip_status(launch_zero(dx, (size_t)M * (size_t)K * (size_t)elem_size(dtype),
                                  as_stream(stream)));
  if (!dg || !dfc || !w_g || !w_fc) return SWG_ERR_NULLPTR;
  for (const void* p : {dg, dfc, w_g, w_fc}) if (!aligned(p, 16)) return SWG_ERR_UNSUPPORTED;
  {
    const int64_t es = elem_size(dtype);
    const int64_t d = span_bytes(M, N, es), w = span_bytes(K, N, es);
    const Span outs[] = {{dx, span_bytes(M, K, es)}};
    const Span ins[] = {{dg, d}, {dfc, d}, {w_g, w}, {w_fc, w}};
    if (!outputs_disjoint(outs, ins)) return SWG_ERR_INVALID;
  }
  return hip_status(launch_x_stage(dtype, dg, dfc, w_g, w_fc, dx, M, K, N, g_tile_f,
                                   gemm_grid_cap(), as_stream(stream)));
}

int swiglu_bwd_gemm_tile(int stage, int64_t M, int64_t K, int64_t N, swg_dtype dtype) {
  if (dtype == SWG_FP32 || gemm_shape_check(dtype, M, K, N) != SWG_OK || M == 0 || K == 0 ||
      N == 0)
    return 0;
  int f = 0;
  if (stage == 0) f = plan_w(M, K, N, g_tile_f).f;
  else if (stage == 1) f = plan_x(M, K, N, g_tile_f).f;
  else if (stage == 2) {
    const WXPlan p = plan_wx(M, K, N, g_tile_f);
    f = p.separate ? plan_x(M, K, N, g_tile_f).f : p.f;
  }
  return (int)tile_edge(f);
}

// ------------------------------------------------------------------- fused w + x
// fp32 has no fused kernel: it always runs the two stages (the fp32 w and x kernels)
static WXPlan wx_plan(int dtype, int64_t M, int64_t K, int64_t N) {
  WXPlan p = plan_wx(M, K, N, g_tile_f);
  if (dtype == SWG_FP32) {
    p.separate = true;
    p.ws_bytes = plan_w(M, K, N, g_tile_f).ws_bytes;
  }
  return p;
}

size_t swiglu_bwd_wx_workspace_size(int64_t M, int64_t K, int64_t N, swg_dtype dtype) {
  if (gemm_shape_check(dtype, M, K, N, true) != SWG_OK || M == 0 || K == 0 || N == 0) return 0;
  return wx_plan(dtype, M, K, N).ws_bytes;
}

swg_status swiglu_bwd_wx(const void* x, const void* dg, const void* dfc, const void* w_g,
                         const void* w_fc, void* dw_g, void* dw_fc, void* dx, int64_t M,
                         int64_t K, int64_t N, swg_dtype dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  TimedCall timed_;
  swg_status st = gemm_shape_check(dtype, M, K, N, true);
  if (st != SWG_OK) return st;
  if (M == 0 || K == 0) return SWG_OK;   // dx and dW are empty
  if (!dx) return SWG_ERR_NULLPTR;
  if (!aligned(dx, 16)) return SWG_ERR_UNSUPPORTED;
  const int64_t es = elem_size(dtype);
  if (N == 0)   // dx = 0 (the empty sum); dW is empty
    return hip_status(launch_zero(dx, (size_t)M * (size_t)K * (size_t)es, as_stream(stream)));
  if (!x || !dg || !dfc || !w_g || !w_fc || !dw_g || !dw_fc) return SWG_ERR_NULLPTR;
  for (const void* p : {(const void*)dw_g, (const void*)dw_fc})
    if (!aligned(p, 8)) return SWG_ERR_UNSUPPORTED;
  for (const void* p : {x, dg, dfc, w_g, w_fc}) if (!aligned(p, 16)) return SWG_ERR_UNSUPPORTED;
  const WXPlan p = wx_plan(dtype, M, K, N);
  if (workspace_bytes < p.ws_bytes) return SWG_ERR_WORKSPACE;
  if (p.ws_bytes > 0 && workspace == nullptr) return SWG_ERR_NULLPTR;
  if (!aligned(workspace, 16)) return SWG_ERR_INVALID;
  {
    const int64_t w = span_bytes(K, N, es), d = span_bytes(M, N, es);
    const Span outs[] = {{dx, span_bytes(M, K, es)}, {dw_g, w}, {dw_fc, w},
                         {workspace, (int64_t)p.ws_bytes}};
    const Span ins[] = {{x, span_bytes(M, K, es)}, {dg, d}, {dfc, d}, {w_g, w}, {w_fc, w}};
    if (!outputs_disjoint(outs, ins)) return SWG_ERR_INVALID;
  }
  if (p.separate) {   // no M split to share rows: the two stages, one launch each
    const hipError_t e = launch_w_stage(dtype, plan_w(M, K, N, g_tile_f), x, dg, dfc, dw_g,
                                        dw_fc, M, K, N, static_cast<float*>(workspace),
                                        gemm_grid_cap(), as_stream(stream));
    if (e != hipSuccess) return hip_status(e);
    return hip_status(launch_x_stage(dtype, dg, dfc, w_g, w_fc, dx, M, K, N, g_tile_f,
                                     gemm_grid_cap(), as_stream(stream)));
  }
  return hip_status(launch_wx(dtype, p, x, dg, dfc, w_g, w_fc, dw_g, dw_fc, dx, M, K, N,
                              static_cast<float*>(workspace), as_stream(stream)));
}

// ------------------------------------------------------------------- forward
swg_status swiglu_fwd(const void* x, const void* w_g, const void* w_fc, const void* b_g,
                      const void* b_fc, void* g, void* fc, void* y, int64_t M, int64_t K,
                      int64_t N, swg_dtype dtype, void* stream) {
  TimedCall timed_;
  swg_status st = gemm_shape_check(dtype, M, K, N, true);
  if (st != SWG_OK) return st;
  if (M == 0 || N == 0) return SWG_OK;  // outputs are empty
  if (!g || !fc || !y) return SWG_ERR_NULLPTR;
  if (K > 0 && (!x || !w_g || !w_fc)) return SWG_ERR_NULLPTR;
  for (const void* p : {x, w_g, w_fc, (const void*)g, (const void*)fc, (const void*)y})
    if (!aligned(p, 16)) return SWG_ERR_UNSUPPORTED;
  for (const void* p : {b_g, b_fc})
    if (!aligned(p, (size_t)elem_size(dtype))) return SWG_ERR_INVALID;
  {
    const int64_t es = elem_size(dtype);
    const int64_t o = span_bytes(M, N, es), w = span_bytes(K, N, es), v = span_bytes(1, N, es);
    const Span outs[] = {{g, o}, {fc, o}, {y, o}};
    const Span ins[] = {{x, span_bytes(M, K, es)}, {w_g, w}, {w_fc, w}, {b_g, v}, {b_fc, v}};
    if (!outputs_disjoint(outs, ins)) return SWG_ERR_INVALID;
  }
  return hip_status(launch_fwd(dtype, x, w_g, w_fc, b_g, b_fc, g, fc, y, M, K, N,
                               gemm_grid_cap(), as_stream(stream)));
}

}  // extern "C"
