// Memory-bound kernels for gfx950: the beta-scaled Swish gradient and the SwiGLU
// backward b stage (dg, dfc and the column partials of db), plus the finalize kernel
// that turns the db partials into the accumulated bias gradients.
//
// Math sources: the SwishGrad page (ops-nn), section 1.2 formula and section 2.4
// (widen 16-bit inputs to fp32, compute, round back to nearest even); the Fused
// SwiGLU backward page (PyPTO-Gym), formulas 1 and 2 and the "Dtype 转换流程" table
// (bf16 storage, fp32 arithmetic).
//
// Both streaming kernels read each input once with 16-byte non-temporal loads
// (8 bf16/fp16 or 4 fp32 per lane, so one wave instruction moves 1 KiB), keep several
// independent loads in flight per lane, and write each output once.
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace swg {

// ------------------------------------------------------------------ b-stage scratch
// Column partials of the b stage for callers that cannot allocate (swiglu_bwd_b_noalloc):
// a file-scope device array, one copy per GPU, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address hipGetSymbolAddress returns, resolved once per
// device with that device current.
static __device__ __align__(256) float scratch[kBScratchBytes / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t b_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------------ swish_grad
// grid-stride over 16-byte vectors; U vectors per lane per step, coalesced so that a
// fixed u addresses 1 KiB of contiguous memory per wave.  The last block also handles
// the n % VEC scalar tail (the first blocks to start are the first to be given more
// work when the grid strides).
template <typename T, int U>
__global__ __launch_bounds__(256) void swish_grad_vec_kernel(const T* grad, const T* x, T* out,
                                                             int64_t n, float beta) {
  using VT = Vec16<T>;
  constexpr int V = VT::VEC;
  const int64_t nvec = n / V;
  const int64_t step = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U; base < nvec; base += step) {
    u32x4 rg[U], rx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      if (i < nvec) {
        rg[u] = ld16_stream(grad + i * V);
        rx[u] = ld16_stream(x + i * V);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      if (i < nvec) {
        float fg[V], fx[V], fo[V];
        VT::widen(rg[u], fg);
        VT::widen(rx[u], fx);
#pragma unroll
        for (int e = 0; e < V; ++e) fo[e] = fg[e] * swish_factor(beta * fx[e]);
        st16_stream(out + i * V, VT::narrow(fo));
      }
    }
  }
  if (blockIdx.x == gridDim.x - 1) {
    const int64_t i = nvec * V + threadIdx.x;
    if (i < n) out[i] = from_f32<T>(to_f32(grad[i]) * swish_factor(beta * to_f32(x[i])));
  }
}

// element-wise fallback for pointers that are not 16-byte aligned
template <typename T>
__global__ __launch_bounds__(256) void swish_grad_scalar_kernel(const T* grad, const T* x, T* out,
                                                                int64_t n, float beta) {
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += step)
    out[i] = from_f32<T>(to_f32(grad[i]) * swish_factor(beta * to_f32(x[i])));
}

template <typename T>
static hipError_t swish_grad_t(const void* grad, const void* x, void* out, int64_t n,
                               float beta, bool vector_path, hipStream_t stream) {
  const T* g = static_cast<const T*>(grad);
  const T* xx = static_cast<const T*>(x);
  T* o = static_cast<T*>(out);
  if (vector_path) {
    // one 16-byte vector of each input per lane and a grid that covers the whole tensor
    // in one pass (measured on MI355X at 2^24 + 37 elements: 2 vectors per lane over at
    // most 4096 workgroups was about 1 us slower in fp16 and in fp32); the grid strides
    // only past 2^20 workgroups
    constexpr int U = 1;
    constexpr int64_t kMaxBlocks = int64_t(1) << 20;
    constexpr int V = Vec16<T>::VEC;
    const int64_t nvec = n / V;
    int64_t blocks = ceil_div(nvec, 256 * U);
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    if (blocks < 1) blocks = 1;
    SWG_LAUNCH((swish_grad_vec_kernel<T, U>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, g, xx, o, n, beta);
  } else {
    int64_t blocks = ceil_div(n, 256);
    if (blocks > kMaxStreamBlocks) blocks = kMaxStreamBlocks;
    SWG_LAUNCH((swish_grad_scalar_kernel<T>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, g, xx, o, n, beta);
  }
  return hipGetLastError();
}

hipError_t launch_swish_grad(int dtype, const void* grad, const void* x, void* out, int64_t n,
                             float beta, bool vector_path, hipStream_t stream) {
  switch (dtype) {
    case 0: return swish_grad_t<bf16>(grad, x, out, n, beta, vector_path, stream);
    case 1: return swish_grad_t<fp16>(grad, x, out, n, beta, vector_path, stream);
    default: return swish_grad_t<float>(grad, x, out, n, beta, vector_path, stream);
  }
}

// ------------------------------------------------------------------ b stage
// Workgroup = 256 lanes laid out as TY rows x TX vector-columns (TX = 2^txlog2).
// blockIdx.x picks the column strip; blockIdx.y is the walker, which takes the row units
// blockIdx.y, blockIdx.y + gridDim.y, ... (unit_rows rows each, a multiple of R * TY on
// the vector path).  Inside a unit each lane walks the rows with stride TY; on the vector
// path it first issues the loads of R rows (3R independent 16-byte loads in flight per
// lane), then computes and stores them.
// dg and dfc are written with non-temporal stores: the next stage reads them back from
// HBM anyway (they are far larger than the caches).  The lane keeps fp32 column sums
// over all its units; the workgroup reduces them over TY in LDS (fixed order) and writes
// one partial row: part[walker][0:N] = sum dg, part[walker][N:2N] = sum dfc.
template <typename T, bool VECTOR>
struct BAccess {
  static constexpr int V = VECTOR ? Vec16<T>::VEC : 1;
  using Raw = typename std::conditional<VECTOR, u32x4, T>::type;
  __device__ static inline Raw load(const T* p) {
    if constexpr (VECTOR) return ld16_stream(p);
    else return *p;
  }
  __device__ static inline void widen(const Raw& r, float* f) {
    if constexpr (VECTOR) Vec16<T>::widen(r, f);
    else f[0] = to_f32(r);
  }
  __device__ static inline void store(T* p, const float* f) {
    if constexpr (VECTOR) st16_stream(p, Vec16<T>::narrow(f));
    else *p = from_f32<T>(f[0]);
  }
};

// dg = dy fc s (1 + g (1 - s)),  dfc = dy g s  (SwiGLU page, formulas 1 and 2)
template <typename T, bool VECTOR>
__device__ inline void b_compute(const typename BAccess<T, VECTOR>::Raw& rdy,
                                 const typename BAccess<T, VECTOR>::Raw& rg,
                                 const typename BAccess<T, VECTOR>::Raw& rfc, T* dg, T* dfc,
                                 int64_t off, float* sg, float* sf) {
  using A = BAccess<T, VECTOR>;
  constexpr int V = A::V;
  float fdy[V], fg[V], ffc[V], odg[V], odfc[V];
  A::widen(rdy, fdy);
  A::widen(rg, fg);
  A::widen(rfc, ffc);
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const SigmoidParts p = sigmoid_parts(fg[e]);
    const float dyfc = fdy[e] * ffc[e];
    odg[e] = dyfc * __builtin_fmaf(fg[e], p.s1ms, p.s);
    odfc[e] = fdy[e] * (fg[e] * p.s);
    sg[e] += odg[e];
    sf[e] += odfc[e];
  }
  A::store(dg + off, odg);
  A::store(dfc + off, odfc);
}

template <typename T, bool VECTOR, int R>
__global__ __launch_bounds__(256) void b_stage_kernel(const T* dy, const T* g, const T* fc, T* dg,
                                                      T* dfc, float* part, int64_t M, int64_t N,
                                                      int64_t cv, int64_t unit_rows,
                                                      int64_t nunits, int txlog2) {
  using A = BAccess<T, VECTOR>;
  constexpr int V = A::V;
  const int tid = threadIdx.x;
  const int TX = 1 << txlog2;
  const int TY = 256 >> txlog2;
  const int tx = tid & (TX - 1);
  const int ty = tid >> txlog2;
  const int64_t c = (int64_t)blockIdx.x * TX + tx;

  float sg[V], sf[V];
#pragma unroll
  for (int e = 0; e < V; ++e) sg[e] = sf[e] = 0.0f;

  const int64_t col = c * V;
  for (int64_t unit = blockIdx.y; c < cv && unit < nunits; unit += gridDim.y) {
    const int64_t r0 = unit * unit_rows;
    const int64_t r1 = (r0 + unit_rows < M) ? r0 + unit_rows : M;
    int64_t r = r0 + ty;
    for (; r + (R - 1) * TY < r1; r += R * TY) {
      typename A::Raw a[R], b[R], d[R];
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int64_t off = (r + u * TY) * N + col;
        a[u] = A::load(dy + off);
        b[u] = A::load(g + off);
        d[u] = A::load(fc + off);
      }
#pragma unroll
      for (int u = 0; u < R; ++u)
        b_compute<T, VECTOR>(a[u], b[u], d[u], dg, dfc, (r + u * TY) * N + col, sg, sf);
    }
    for (; r < r1; r += TY) {
      const int64_t off = r * N + col;
      b_compute<T, VECTOR>(A::load(dy + off), A::load(g + off), A::load(fc + off), dg, dfc, off,
                           sg, sf);
    }
  }

  __shared__ float red[2 * 8 * 256];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    red[e * 256 + tid] = sg[e];
    red[(V + e) * 256 + tid] = sf[e];
  }
  __syncthreads();
  if (ty == 0 && c < cv) {
    float* dst = part + (int64_t)blockIdx.y * 2 * N;
#pragma unroll
    for (int e = 0; e < 2 * V; ++e) {
      float acc = 0.0f;
      for (int y = 0; y < TY; ++y) acc += red[e * 256 + y * TX + tx];
      const int64_t n = c * V + (e % V);
      dst[(e < V ? 0 : N) + n] = acc;
    }
  }
}

// db[n] = RNE(db[n] + sum_chunks part[chunk][n]).  A workgroup owns 16 columns of the
// [nchunks, 2N] partial matrix; its 16 lane groups split the chunks round-robin
// (group j takes chunks j, j+16, ...), each lane keeping kFinUnroll loads in flight
// and adding them in chunk order; the 16 group sums are then added in group order.
// The summation tree depends only on nchunks: results are run-to-run deterministic.
constexpr int kFinUnroll = 16;

template <typename T>
__global__ __launch_bounds__(256) void db_finalize_kernel(const float* part, T* db_g, T* db_fc,
                                                          int64_t N, int64_t nchunks) {
  const int lane = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const int64_t col = (int64_t)blockIdx.x * 16 + lane;
  const int64_t W = 2 * N;
  float s = 0.0f;
  if (col < W) {
    for (int64_t ch0 = grp; ch0 < nchunks; ch0 += 16 * kFinUnroll) {
      float v[kFinUnroll];
#pragma unroll
      for (int u = 0; u < kFinUnroll; ++u) {
        const int64_t ch = ch0 + 16 * u;
        v[u] = ch < nchunks ? part[ch * W + col] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kFinUnroll; ++u) s += v[u];
    }
  }
  __shared__ float red[16][17];
  red[grp][lane] = s;
  __syncthreads();
  if (grp == 0 && col < W) {
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) t += red[j][lane];
    T* dst = col < N ? db_g + col : db_fc + (col - N);
    *dst = from_f32<T>(to_f32(*dst) + t);
  }
}

template <typename T>
static hipError_t b_stage_t(const BPlan& p, const void* dy, const void* g, const void* fc,
                            void* dg, void* dfc, void* db_g, void* db_fc, int64_t M, int64_t N,
                            float* part, hipStream_t stream) {
  int txlog2 = 0;
  while ((1 << txlog2) < p.tx) ++txlog2;
  const dim3 grid((unsigned)p.nstrips, (unsigned)p.nwalk);
  const T* a = static_cast<const T*>(dy);
  const T* b = static_cast<const T*>(g);
  const T* c = static_cast<const T*>(fc);
  if (p.vec > 1 && p.rif == kBRowsInFlight) {
    SWG_LAUNCH((b_stage_kernel<T, true, kBRowsInFlight>), grid, dim3(256), 0, stream, a, b, c,
                       static_cast<T*>(dg), static_cast<T*>(dfc), part, M, N, p.cv, p.unit_rows,
                       p.nunits, txlog2);
  } else if (p.vec > 1) {
    SWG_LAUNCH((b_stage_kernel<T, true, kBSmallRows>), grid, dim3(256), 0, stream, a, b, c,
               static_cast<T*>(dg), static_cast<T*>(dfc), part, M, N, p.cv, p.unit_rows,
               p.nunits, txlog2);
  } else {
    SWG_LAUNCH((b_stage_kernel<T, false, 1>), grid, dim3(256), 0, stream, a, b, c,
                       static_cast<T*>(dg), static_cast<T*>(dfc), part, M, N, p.cv, p.unit_rows,
                       p.nunits, txlog2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SWG_LAUNCH((db_finalize_kernel<T>), dim3((unsigned)ceil_div(2 * N, 16)), dim3(256), 0,
                     stream, part, static_cast<T*>(db_g), static_cast<T*>(db_fc), N, p.nwalk);
  return hipGetLastError();
}

hipError_t launch_b_stage(int dtype, const BPlan& p, const void* dy, const void* g,
                          const void* fc, void* dg, void* dfc, void* db_g, void* db_fc,
                          int64_t M, int64_t N, float* part, hipStream_t stream) {
  switch (dtype) {
    case 0: return b_stage_t<bf16>(p, dy, g, fc, dg, dfc, db_g, db_fc, M, N, part, stream);
    case 1: return b_stage_t<fp16>(p, dy, g, fc, dg, dfc, db_g, db_fc, M, N, part, stream);
    default: return b_stage_t<float>(p, dy, g, fc, dg, dfc, db_g, db_fc, M, N, part, stream);
  }
}

}  // namespace swg
