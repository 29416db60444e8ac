/*
 * swiglu_bwd.h — C ABI of the MI355X (gfx950) SwiGLU backward and Swish-gradient library.
 *
 * Sources (web pages; cited by title and section):
 *   [SwiGLU page]  "PyPTO-Gym 实战: Fused SwiGLU 反向传播算子 (Ascend NPU 三 Kernel 融合实现)",
 *                  sections "算法概述与数学公式" (formulas 1-4), "Kernel 概览与调用链" (call
 *                  chain b -> w -> x), "Kernel 签名与参数规格" (shapes, dtypes, zero-init
 *                  accumulators), "动态轴" (dynamic M), "Dtype 转换流程" (bf16 storage,
 *                  fp32 arithmetic).
 *   [Swish page]   "CANN ops-nn 中 SwishGrad 算子解析: 原理、实现与 aclnnSwishBackward 调用指南",
 *                  sections 1.2 (formula), 1.3 (parameters, optional scale = beta, default 1.0),
 *                  2.4 (fp16/bf16 widened to fp32, rounded back to nearest even),
 *                  3.3 / 3.5 (argument checks, empty tensors return success with no work).
 *
 * Conventions shared by every call:
 *   - All tensors are dense, row-major, contiguous device buffers (hipMalloc'd or any
 *     device-accessible pointer).  The library never allocates, frees or copies device
 *     memory and never synchronises; every call only validates its arguments on the host
 *     and enqueues kernels on `stream` (a hipStream_t; NULL = the null stream).
 *   - Sizes are int64_t element counts.  The batch size M (and the Swish length n) is a
 *     run-time argument of any value >= 0: there is no per-size compilation and the last
 *     partial tile is masked, never padded.
 *   - Arithmetic is fp32; results are rounded once to the storage dtype with
 *     round-to-nearest-even.
 *   - Every pointer must be aligned to its element size.  Buffers may not overlap unless
 *     a call says otherwise.
 *   - Errors are reported before anything is enqueued: SWG_ERR_NULLPTR for a NULL
 *     pointer that the call would touch, SWG_ERR_INVALID for a negative size, an unknown
 *     dtype or a misaligned pointer, SWG_ERR_UNSUPPORTED for a dtype/shape combination
 *     the call does not implement, SWG_ERR_WORKSPACE for a workspace smaller than the
 *     matching *_workspace_size query.  SWG_ERR_HIP means a launch failed; the HIP error
 *     code is then available from swg_last_hip_error().  Calls whose work is empty return
 *     SWG_OK without launching anything.
 *   - Calls are thread-safe: the library keeps no state apart from the last HIP error, the
 *     timing events of swg_time_next_call and the tile setting of swg_set_gemm_tile (all
 *     per host thread), the cached compute-unit count of each device and the device
 *     scratch of swiglu_bwd_b_noalloc.
 *   - A workspace is in use until the call's kernels have finished on its stream: calls
 *     that may run at the same time (on different streams) need distinct workspaces.
 */
#ifndef SWIGLU_BWD_H
#define SWIGLU_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SWG_BF16 = 0, SWG_FP16 = 1, SWG_FP32 = 2 } swg_dtype;

typedef enum {
  SWG_OK = 0,
  SWG_ERR_NULLPTR = 1,
  SWG_ERR_INVALID = 2,
  SWG_ERR_UNSUPPORTED = 3,
  SWG_ERR_WORKSPACE = 4,
  SWG_ERR_HIP = 5
} swg_status;

/*
 * b stage [SwiGLU page, formulas 1 and 2; kernel 1 of the call chain]:
 *   s = sigma(g) = 1 / (1 + exp(-g))
 *   dg[m,n]  = dy[m,n] * fc[m,n] * s * (1 + g[m,n] * (1 - s))
 *   dfc[m,n] = dy[m,n] * g[m,n] * s
 *   db_g[n]  = RNE(db_g[n]  + sum_m dg[m,n])     (accumulated, see below)
 *   db_fc[n] = RNE(db_fc[n] + sum_m dfc[m,n])
 * dy, g, fc, dg, dfc: [M, N]; db_g, db_fc: [N] (the page's [1, N]).  dtype: bf16, fp16
 * or fp32, the same for every tensor.  dg and dfc are overwritten.  db_g and db_fc are
 * ACCUMULATED: the column sums are formed from the fp32 values of dg/dfc (before their
 * rounding), in a fixed order (run-to-run deterministic, no atomics), added to the
 * current contents and rounded once; the caller zeroes them for a plain gradient.
 * `workspace` must hold swiglu_bwd_b_workspace_size(M, N, dtype) bytes of device memory
 * (fp32 column partials; contents on entry are ignored, contents on return unspecified);
 * it may be NULL when that size is 0.  No output (dg, dfc, db_g, db_fc, workspace) may
 * overlap another buffer (SWG_ERR_INVALID); the inputs are only read and may share memory.
 */
swg_status swiglu_bwd_b(const void* dy, const void* g, const void* fc,
                        void* dg, void* dfc, void* db_g, void* db_fc,
                        int64_t M, int64_t N, swg_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream);
size_t swiglu_bwd_b_workspace_size(int64_t M, int64_t N, swg_dtype dtype);

/*
 * The b stage for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation,
 * kernels and results as swiglu_bwd_b, bit for bit, with the fp32 column partials kept
 * in a static device array of SWG_B_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends, instead of a caller workspace.  The call itself
 * allocates nothing (no hipMalloc, no allocating library routine).  Its first call on a
 * device resolves that device's array address once.  Shapes whose partials exceed the
 * array (swiglu_bwd_b_workspace_size(M, N, dtype) > SWG_B_SCRATCH_BYTES, i.e. N above 2^21)
 * return SWG_ERR_WORKSPACE; the other errors are those of swiglu_bwd_b.
 * Every call on one GPU uses that GPU's one array: two calls that run at the same time on
 * one GPU (on different streams, or from different threads) race on it and give wrong
 * db; serialise them on one stream.  The array is fully rewritten by each call (nothing
 * in it has to start at zero).
 */
#define SWG_B_SCRATCH_BYTES (16u << 20)
swg_status swiglu_bwd_b_noalloc(const void* dy, const void* g, const void* fc,
                                void* dg, void* dfc, void* db_g, void* db_fc,
                                int64_t M, int64_t N, swg_dtype dtype, void* stream);

/*
 * w stage [SwiGLU page, formula 3; kernel 2]:  [dw_g | dw_fc] += x^T [dg | dfc]
 * one GEMM [K, M] x [M, 2N] whose right operand is the column concatenation of dg and dfc.
 *   dw_g[k,n]  = RNE(dw_g[k,n]  + sum_m x[m,k] * dg[m,n])
 *   dw_fc[k,n] = RNE(dw_fc[k,n] + sum_m x[m,k] * dfc[m,n])
 * x: [M, K]; dg, dfc: [M, N]; dw_g, dw_fc: [K, N].  dtype: bf16, fp16 or fp32.  K and N
 * must be multiples of 8 (bf16 / fp16) or of 4 (fp32), i.e. 16-byte rows, and below 2^22,
 * and M below 2^31; x, dg and dfc must be 16-byte aligned and dw_g, dw_fc 8-byte aligned;
 * otherwise SWG_ERR_UNSUPPORTED.  Products are formed on the matrix
 * cores, accumulated in fp32 (split over M in fixed-order fp32 partials when the output is
 * small), added to the current dw and rounded once (fp32: not rounded): dw is ACCUMULATED
 * like db.  `workspace` holds swiglu_bwd_w_workspace_size(M, K, N, dtype) bytes (0 when
 * no split is needed; the same for every dtype).  dw_g, dw_fc and the workspace may not
 * overlap each other or an input (SWG_ERR_INVALID).
 */
swg_status swiglu_bwd_w(const void* x, const void* dg, const void* dfc,
                        void* dw_g, void* dw_fc,
                        int64_t M, int64_t K, int64_t N, swg_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream);
size_t swiglu_bwd_w_workspace_size(int64_t M, int64_t K, int64_t N, swg_dtype dtype);

/*
 * x stage [SwiGLU page, formula 4; kernel 3]:  dx = [dg | dfc] [W_g | W_fc]^T
 * one GEMM [M, 2N] x [2N, K]:  dx[m,k] = sum_n dg[m,n] W_g[k,n] + dfc[m,n] W_fc[k,n].
 * dg, dfc: [M, N]; w_g, w_fc: [K, N] (row-major, as on the page); dx: [M, K], OVERWRITTEN.
 * dtype: bf16, fp16 or fp32; K and N multiples of 8 (bf16 / fp16) or of 4 (fp32) and
 * below 2^22, M below 2^31, every pointer 16-byte aligned (else SWG_ERR_UNSUPPORTED).  fp32 accumulation, one rounding
 * (none for fp32).  N = 0 with M*K > 0 writes dx = 0 (the empty sum).  dx may not overlap
 * an input (SWG_ERR_INVALID).
 */
swg_status swiglu_bwd_x(const void* dg, const void* dfc, const void* w_g, const void* w_fc,
                        void* dx, int64_t M, int64_t K, int64_t N, swg_dtype dtype,
                        void* stream);

/*
 * Tile configuration of the matrix-core stages: the edge of the square output tile (rows
 * = columns per workgroup) that swiglu_bwd_w (stage 0), swiglu_bwd_x (stage 1) or
 * swiglu_bwd_wx (stage 2) uses for a bf16 or fp16 problem of this shape: 256, or 128 where
 * 256 x 256 tiles would leave CUs of the MI355X idle (small M, small outputs) or, in the w
 * stage, need many fp32 M-split partials.  Host-only arithmetic: the planner the calls
 * themselves use, independent of the device.  Where swiglu_bwd_wx runs the two stages
 * as separate launches, stage 2 reports the x stage's tile.  Results do not depend on the tile size
 * beyond rounding order.  0 for fp32 (its own kernels), empty or unsupported shapes and an
 * unknown stage.
 */
int swiglu_bwd_gemm_tile(int stage, int64_t M, int64_t K, int64_t N, swg_dtype dtype);

/*
 * Tile override, for tuning and tests: edge 256 or 128 makes swiglu_bwd_w, swiglu_bwd_x,
 * swiglu_bwd_wx, their workspace-size queries and swiglu_bwd_gemm_tile, when called
 * afterwards on the calling thread, use that tile edge instead of the planner's choice
 * (bf16 / fp16; the w stage's M splits follow the tile count, so query the workspace size
 * under the same setting); 0 restores the planner.  SWG_ERR_INVALID for other values.
 */
swg_status swg_set_gemm_tile(int edge);

/*
 * Fused w + x pass [SwiGLU page, formulas 3 and 4, which contract the same [dg | dfc], and
 * the operator background's motive for fusion: intermediates should not make repeated
 * trips through memory]: the results of swiglu_bwd_w followed by swiglu_bwd_x from one
 * kernel launch (plus, when M is split, the in-order reduction of the fp32 partials):
 *   [dw_g | dw_fc] += x^T [dg | dfc]   (accumulated, one rounding, as swiglu_bwd_w)
 *   dx = [dg | dfc] [W_g | W_fc]^T     (overwritten, as swiglu_bwd_x)
 * Half of the workgroups compute dx tiles row block after row block while the other half
 * compute dW tiles over 256-row chunks of [dg | dfc] taken round-robin by S splits, so
 * that both halves read the same rows at about the same time and [dg | dfc] crosses HBM
 * about once (the separate calls read it twice).  dx is bit-identical to swiglu_bwd_x;
 * dW groups its fp32 partial sums by chunk and may differ from swiglu_bwd_w in the last
 * bit.  Shapes whose dW grid needs no M split and where each stage alone fills the GPU
 * (e.g. M = 16384, K = 4096, N = 14336) gain nothing from sharing rows: there the call runs
 * swiglu_bwd_w and then swiglu_bwd_x (two launches on the stream, the same bits as those
 * calls).  dtype bf16, fp16 or fp32 (fp32 has no fused kernel: the call runs the fp32
 * swiglu_bwd_w and then swiglu_bwd_x); the shape and alignment rules of swiglu_bwd_w and
 * swiglu_bwd_x; dx, dw_g, dw_fc and the workspace may not overlap each
 * other or an input (SWG_ERR_INVALID).  `workspace`: swiglu_bwd_wx_workspace_size(M, K, N,
 * dtype) bytes (S * K * 2N fp32 partials; 0 when S = 1).  N = 0 writes dx = 0 (the
 * inputs and dW, all empty, may then be NULL).
 */
swg_status swiglu_bwd_wx(const void* x, const void* dg, const void* dfc,
                         const void* w_g, const void* w_fc,
                         void* dw_g, void* dw_fc, void* dx,
                         int64_t M, int64_t K, int64_t N, swg_dtype dtype,
                         void* workspace, size_t workspace_bytes, void* stream);
size_t swiglu_bwd_wx_workspace_size(int64_t M, int64_t K, int64_t N, swg_dtype dtype);

/*
 * SwiGLU forward [SwiGLU page, operator background: the function the three stages above
 * differentiate]:
 *   g[m,n]  = sum_k x[m,k] W_g[k,n]  + b_g[n]
 *   fc[m,n] = sum_k x[m,k] W_fc[k,n] + b_fc[n]
 *   y[m,n]  = SiLU(g[m,n]) * fc[m,n] = g sigma(g) fc
 * x: [M, K]; w_g, w_fc: [K, N]; b_g, b_fc: [N], or NULL for no bias; g, fc, y: [M, N],
 * OVERWRITTEN (g and fc are what swiglu_bwd_b takes).  dtype: bf16, fp16 or fp32; K and N
 * multiples of 8 (bf16 / fp16) or of 4 (fp32) and below 2^22, M below 2^31, and x, w_g,
 * w_fc, g, fc, y 16-byte aligned, else SWG_ERR_UNSUPPORTED (a bias that is not aligned to
 * its element size: SWG_ERR_INVALID).  Products on the matrix cores with fp32 accumulation; the bias is
 * added in fp32; y is formed from the fp32 values of g and fc (before their rounding); each
 * output is rounded once (fp32: not rounded).  K = 0 gives g = b_g, fc = b_fc (the empty sums); x, w_g and
 * w_fc may then be NULL.  g, fc and y may not overlap each other or an input
 * (SWG_ERR_INVALID).
 */
swg_status swiglu_fwd(const void* x, const void* w_g, const void* w_fc,
                      const void* b_g, const void* b_fc, void* g, void* fc, void* y,
                      int64_t M, int64_t K, int64_t N, swg_dtype dtype, void* stream);

/*
 * Swish gradient with a scalar beta [Swish page, sections 1.2 and 2.4]:
 *   t = beta * x,  s = sigma(t),  grad_x = grad * s * (1 + t * (1 - s))
 * grad, x, grad_x: n elements of one dtype (bf16, fp16 or fp32).  `beta` points to a
 * host float; NULL means 1.0 (the page's default when the scale is absent).  Any finite
 * beta is valid (beta = 0 gives grad / 2).  grad_x may alias grad or x exactly (in-place);
 * no other overlap is allowed.
 */
swg_status swish_grad(const void* grad, const void* x, void* grad_x, int64_t n,
                      swg_dtype dtype, const float* beta, void* stream);

/*
 * Swish gradient over strided (non-contiguous) tensors [Swish page, sections 3.5 and 4.2:
 * non-contiguous inputs are accepted, tensors of more than 8 dimensions are flattened,
 * and the result is written into a possibly non-contiguous output].  The three tensors
 * share one logical shape sizes[0..ndim) (row-major order; ndim 0 is a scalar, up to
 * SWG_MAX_NDIM dimensions); grad_strides, x_strides and out_strides give each tensor's
 * element strides per dimension (host arrays; negative strides allowed; input strides
 * may be 0, i.e. broadcast views).  The pointers address each tensor's element at
 * logical index (0, ..., 0).  Dimensions that are contiguous in all three tensors are
 * merged first; a view that is contiguous after merging runs the contiguous kernel.
 * Errors: SWG_ERR_INVALID for a negative size, an element count that overflows int64,
 * a view whose byte span overflows int64 (or a stride of INT64_MIN), misaligned pointers, an output whose elements overlap each other, or an output that
 * overlaps an input other than as the exact same view (same pointer and strides, which
 * is in-place); SWG_ERR_UNSUPPORTED when more than 8 dimensions remain after merging.
 * Empty views (a size of 0) return SWG_OK without touching the pointers.
 */
#define SWG_MAX_NDIM 64
swg_status swish_grad_strided(const void* grad, const void* x, void* grad_x, int ndim,
                              const int64_t* sizes, const int64_t* grad_strides,
                              const int64_t* x_strides, const int64_t* out_strides,
                              swg_dtype dtype, const float* beta, void* stream);

/*
 * Kernel-duration timing for measurement harnesses.  The next entry-point call made on
 * the calling thread dispatches its kernels with these two events attached
 * (hipExtLaunchKernel): `start_event` is recorded when its first kernel begins and
 * `stop_event` when its last kernel ends, so hipEventElapsedTime(start, stop) after that
 * call is the span of its kernels on the GPU, without the dispatch gaps that events
 * recorded around the call include.  Both are hipEvent_t handles created by the caller
 * (timing enabled) on the device of the call; both NULL cancels.  The setting applies to
 * that one call and is cleared when it returns; a call that launches nothing (empty
 * input, argument error) records neither event.  SWG_ERR_INVALID if only one is NULL.
 */
swg_status swg_time_next_call(void* start_event, void* stop_event);

/* Human-readable name of a status code (static storage; never NULL). */
const char* swg_status_string(int status);

/* The hipError_t of the most recent SWG_ERR_HIP on the calling thread (0 if none). */
int swg_last_hip_error(void);

/* Library version, e.g. "swiglu_bwd 0.1.0 gfx950". */
const char* swg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_BWD_H */
