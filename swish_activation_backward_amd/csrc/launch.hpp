// Internal launchers (C++ linkage) called by the C ABI layer after validation.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace swg {

// Kernel-duration timing of one entry-point call (swg_time_next_call): caller-created HIP
// events, per host thread, cleared when the timed call returns.
struct CallTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
CallTiming& call_timing();

// Every kernel of the library is dispatched through this.  While a call is timed, the
// dispatch carries the call's events (hipExtLaunchKernelGGL): the first dispatch records
// `start` when it begins and every dispatch records `stop` when it ends, so the pair spans
// the call's kernels from the first one's start to the last one's end.
#define SWG_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                 \
  do {                                                                                    \
    ::swg::CallTiming& t_ = ::swg::call_timing();                                         \
    if (t_.stop == nullptr) {                                                             \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                 \
    } else {                                                                              \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, t_.start, t_.stop, 0,       \
                            __VA_ARGS__);                                                 \
      t_.start = nullptr;                                                                 \
    }                                                                                     \
  } while (0)

constexpr int64_t kMaxStreamBlocks = 8192;

hipError_t launch_swish_grad(int dtype, const void* grad, const void* x, void* out, int64_t n,
                             float beta, bool vector_path, hipStream_t stream);

// Strided views for swish_grad: a logical shape in row-major order (after merging the
// dimensions that are contiguous in all three tensors) and each tensor's element strides.
constexpr int kMaxStridedDims = 8;
struct StridedView {
  int nd;
  int64_t size[kMaxStridedDims];
  int64_t stride[3][kMaxStridedDims];   // grad, x, grad_x
};

// grad_x[i] for every logical index i of the view (n = product of the sizes > 0)
hipError_t launch_swish_grad_strided(int dtype, const void* grad, const void* x, void* out,
                                     const StridedView& v, int64_t n, float beta,
                                     hipStream_t stream);

// The device address of the b stage's static scratch array on the current device
// (kBScratchBytes; resolved on the first call per device, no allocation).
hipError_t b_scratch(float** out);

hipError_t launch_b_stage(int dtype, const BPlan& p, const void* dy, const void* g,
                          const void* fc, void* dg, void* dfc, void* db_g, void* db_fc,
                          int64_t M, int64_t N, float* part, hipStream_t stream);

// `cus`: compute units of the device: the GEMM stages launch one persistent workgroup
// per CU (fewer when there is less work).
hipError_t launch_w_stage(int dtype, const WPlan& p, const void* x, const void* dg,
                          const void* dfc, void* dw_g, void* dw_fc, int64_t M, int64_t K,
                          int64_t N, float* ws, int cus, hipStream_t stream);

// fused w + x pass (bf16 / fp16): dx and [dw_g | dw_fc] += x^T [dg | dfc] in one launch
hipError_t launch_wx(int dtype, const WXPlan& p, const void* x, const void* dg, const void* dfc,
                     const void* w_g, const void* w_fc, void* dw_g, void* dw_fc, void* dx,
                     int64_t M, int64_t K, int64_t N, float* ws, hipStream_t stream);

// force_f: tile configuration override (4 or 2; 0 = the planner's choice)
hipError_t launch_x_stage(int dtype, const void* dg, const void* dfc, const void* w_g,
                          const void* w_fc, void* dx, int64_t M, int64_t K, int64_t N,
                          int force_f, int cus, hipStream_t stream);

// fp32 tensors (dtype 2) of the GEMMs; called by launch_x_stage / launch_w_stage / launch_fwd
hipError_t launch_x_stage32(const void* dg, const void* dfc, const void* w_g, const void* w_fc,
                            void* dx, int64_t M, int64_t K, int64_t N, hipStream_t stream);
hipError_t launch_w_stage32(const WPlan& p, const void* x, const void* dg, const void* dfc,
                            void* dw_g, void* dw_fc, int64_t M, int64_t K, int64_t N, float* ws,
                            hipStream_t stream);
hipError_t launch_fwd32(const void* x, const void* w_g, const void* w_fc, const void* b_g,
                        const void* b_fc, void* g, void* fc, void* y, int64_t M, int64_t K,
                        int64_t N, hipStream_t stream);

// SwiGLU forward: g, fc, y [M, N] from x [M, K], W_g, W_fc [K, N], b_g, b_fc [N] (may be
// null); one persistent workgroup per CU.
hipError_t launch_fwd(int dtype, const void* x, const void* w_g, const void* w_fc,
                      const void* b_g, const void* b_fc, void* g, void* fc, void* y, int64_t M,
                      int64_t K, int64_t N, int cus, hipStream_t stream);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

}  // namespace swg
