// Swish gradient over strided (non-contiguous) tensors: the gather / scatter kernel for
// any view and the LDS-tiled kernel for two-dimensional views with a column-contiguous
// tensor.  Math: the SwishGrad page (ops-nn), section 1.2 formula and section 2.4 (widen
// 16-bit inputs to fp32, compute, round back to nearest even).
#include "common.hpp"
#include "launch.hpp"

namespace swg {

// ------------------------------------------------------------------ strided swish_grad
// Non-contiguous tensors (the SwishGrad page's aclnn interface, sections 3.5 and 4.2:
// non-contiguous inputs are accepted and the result is written back into a possibly
// non-contiguous output).
// Instead of copying the inputs to contiguous buffers and the result back, one kernel
// walks the logical index space and gathers / scatters through each tensor's strides.
//
// Index decomposition: per dimension (innermost first) q = i / size, r = i - q size.  When
// n < 2^32 the division is a multiply-high by a precomputed magic number (unsigned
// division by an invariant integer, Granlund and Montgomery, PLDI 1994: for divisor d,
// s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1, q = (mulhi(i, m) + i) >> s).
struct FastDiv32 {
  uint32_t d, m, s;
};

struct StridedArgs {
  int nd;
  FastDiv32 div[kMaxStridedDims];
  int64_t size[kMaxStridedDims];
  int64_t sg[kMaxStridedDims], sx[kMaxStridedDims], so[kMaxStridedDims];
};

static FastDiv32 make_fastdiv(uint32_t d) {
  FastDiv32 f;
  f.d = d;
  uint32_t s = 0;
  while (s < 32 && (uint64_t(1) << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
  return f;
}

__device__ inline uint32_t fastdiv(uint32_t i, const FastDiv32& f) {
  const uint64_t t = ((uint64_t)i * f.m) >> 32;
  return (uint32_t)((t + i) >> f.s);
}

template <typename T, bool WIDE>
__global__ __launch_bounds__(256) void swish_grad_strided_kernel(const T* grad, const T* x,
                                                                 T* out, StridedArgs a,
                                                                 int64_t n, float beta) {
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += step) {
    int64_t og = 0, ox = 0, oo = 0;
    if (WIDE) {
      int64_t idx = i;
#pragma unroll
      for (int k = kMaxStridedDims - 1; k >= 0; --k) {
        if (k < a.nd) {
          const int64_t q = idx / a.size[k], r = idx - q * a.size[k];
          og += r * a.sg[k];
          ox += r * a.sx[k];
          oo += r * a.so[k];
          idx = q;
        }
      }
    } else {
      uint32_t idx = (uint32_t)i;
#pragma unroll
      for (int k = kMaxStridedDims - 1; k >= 0; --k) {
        if (k < a.nd) {
          const uint32_t q = fastdiv(idx, a.div[k]), r = idx - q * a.div[k].d;
          og += (int64_t)r * a.sg[k];
          ox += (int64_t)r * a.sx[k];
          oo += (int64_t)r * a.so[k];
          idx = q;
        }
      }
    }
    out[oo] = from_f32<T>(to_f32(grad[og]) * swish_factor(beta * to_f32(x[ox])));
  }
}

// Two-dimensional views in which some tensor runs down the columns (stride 1 on the outer
// dimension, e.g. a transposed matrix): element-at-a-time gathering would read or write
// 2-byte elements a whole row apart.  Each workgroup takes a 64 x 64 tile of the logical
// index space instead; each input is read along its own contiguous dimension into an LDS
// tile (widened to fp32), and the output is written along its contiguous dimension, so
// every global access of a wave covers consecutive addresses.
constexpr int kTrTile = 64;

template <typename T>
__global__ __launch_bounds__(256) void swish_grad_tr2d_kernel(const T* grad, const T* x, T* out,
                                                              int64_t R, int64_t C,
                                                              int64_t sg0, int64_t sg1,
                                                              int64_t sx0, int64_t sx1,
                                                              int64_t so0, int64_t so1,
                                                              float beta) {
  __shared__ float tg[kTrTile][kTrTile + 1], tx[kTrTile][kTrTile + 1];
  const int lo = threadIdx.x & 63, hi = threadIdx.x >> 6;   // 64 x 4 threads
  const int64_t tc = (C + kTrTile - 1) / kTrTile;
  const int64_t tiles = ((R + kTrTile - 1) / kTrTile) * tc;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t r0 = (t / tc) * kTrTile, c0 = (t % tc) * kTrTile;
    // loads: along columns (lo -> c) for a row-contiguous tensor, else along rows
#pragma unroll 4
    for (int k = 0; k < kTrTile / 4; ++k) {
      const int a = hi + 4 * k;
      {
        const bool down = sg1 != 1 && sg0 == 1;
        const int rr = down ? lo : a, cc = down ? a : lo;
        const int64_t r = r0 + rr, c = c0 + cc;
        tg[rr][cc] = (r < R && c < C) ? to_f32(grad[r * sg0 + c * sg1]) : 0.0f;
      }
      {
        const bool down = sx1 != 1 && sx0 == 1;
        const int rr = down ? lo : a, cc = down ? a : lo;
        const int64_t r = r0 + rr, c = c0 + cc;
        tx[rr][cc] = (r < R && c < C) ? to_f32(x[r * sx0 + c * sx1]) : 0.0f;
      }
    }
    __syncthreads();
    const bool down = so1 != 1 && so0 == 1;
#pragma unroll 4
    for (int k = 0; k < kTrTile / 4; ++k) {
      const int a = hi + 4 * k;
      const int rr = down ? lo : a, cc = down ? a : lo;
      const int64_t r = r0 + rr, c = c0 + cc;
      if (r < R && c < C)
        out[r * so0 + c * so1] = from_f32<T>(tg[rr][cc] * swish_factor(beta * tx[rr][cc]));
    }
    __syncthreads();
  }
}

// The same tile with 4-element vectors: a lane moves 4 consecutive elements along its
// tensor's contiguous dimension (8 bytes for 16-bit types, 16 for fp32), 16 lanes cover a
// 64-element line of the tile, four passes the whole tile.  Used when every tensor's other
// stride is a multiple of 4 and its pointer 4-element aligned; a vector that crosses the
// edge of the view falls back to element accesses.
template <typename T>
struct Line4 {
  typedef T V __attribute__((ext_vector_type(4)));
  // direction 0: along columns (stride 1 on dimension 1), 1: along rows
  __device__ static void load(const T* p, int64_t s0, int64_t s1, int dir, int64_t r, int64_t c,
                              int64_t R, int64_t C, float (&v)[4]) {
    const int64_t lim = dir == 0 ? C - c : R - r;   // elements left on the line
    if (r < R && c < C && lim >= 4) {
      const V t = *reinterpret_cast<const V*>(p + r * s0 + c * s1);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = to_f32(t[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t rr = dir == 0 ? r : r + e, cc = dir == 0 ? c + e : c;
        v[e] = (rr < R && cc < C) ? to_f32(p[rr * s0 + cc * s1]) : 0.0f;
      }
    }
  }
  __device__ static void store(T* p, int64_t s0, int64_t s1, int dir, int64_t r, int64_t c,
                               int64_t R, int64_t C, const float (&v)[4]) {
    const int64_t lim = dir == 0 ? C - c : R - r;
    if (r < R && c < C && lim >= 4) {
      V t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = from_f32<T>(v[e]);
      *reinterpret_cast<V*>(p + r * s0 + c * s1) = t;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t rr = dir == 0 ? r : r + e, cc = dir == 0 ? c + e : c;
        if (rr < R && cc < C) p[rr * s0 + cc * s1] = from_f32<T>(v[e]);
      }
    }
  }
};

template <typename T>
__global__ __launch_bounds__(256) void swish_grad_tr2d_vec_kernel(
    const T* grad, const T* x, T* out, int64_t R, int64_t C, int64_t sg0, int64_t sg1,
    int64_t sx0, int64_t sx1, int64_t so0, int64_t so1, float beta) {
  __shared__ float tg[kTrTile][kTrTile + 1], tx[kTrTile][kTrTile + 1];
  const int idx = threadIdx.x & 15, grp = threadIdx.x >> 4;   // 16 lanes per line
  const int dg = (sg1 != 1 && sg0 == 1) ? 1 : 0;
  const int dx = (sx1 != 1 && sx0 == 1) ? 1 : 0;
  const int dout = (so1 != 1 && so0 == 1) ? 1 : 0;
  const int64_t tc = (C + kTrTile - 1) / kTrTile;
  const int64_t tiles = ((R + kTrTile - 1) / kTrTile) * tc;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t r0 = (t / tc) * kTrTile, c0 = (t % tc) * kTrTile;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int line = grp + 16 * pass, off = idx * 4;
      float v[4];
      {
        const int rr = dg == 0 ? line : off, cc = dg == 0 ? off : line;
        Line4<T>::load(grad, sg0, sg1, dg, r0 + rr, c0 + cc, R, C, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) tg[dg == 0 ? rr : rr + e][dg == 0 ? cc + e : cc] = v[e];
      }
      {
        const int rr = dx == 0 ? line : off, cc = dx == 0 ? off : line;
        Line4<T>::load(x, sx0, sx1, dx, r0 + rr, c0 + cc, R, C, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) tx[dx == 0 ? rr : rr + e][dx == 0 ? cc + e : cc] = v[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int line = grp + 16 * pass, off = idx * 4;
      const int rr = dout == 0 ? line : off, cc = dout == 0 ? off : line;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ar = dout == 0 ? rr : rr + e, ac = dout == 0 ? cc + e : cc;
        v[e] = tg[ar][ac] * swish_factor(beta * tx[ar][ac]);
      }
      Line4<T>::store(out, so0, so1, dout, r0 + rr, c0 + cc, R, C, v);
    }
    __syncthreads();
  }
}

// Vector accesses are safe for a tensor when the stride of its other dimension is a
// multiple of 4 and its pointer is aligned to 4 elements.
static bool line4_ok(const void* p, int64_t s0, int64_t s1, int64_t es) {
  const bool down = s1 != 1 && s0 == 1;
  const int64_t other = down ? s1 : s0;
  if (!down && s1 != 1) return false;   // neither dimension contiguous
  return other % 4 == 0 && (reinterpret_cast<uintptr_t>(p) % (uintptr_t)(4 * es)) == 0;
}

template <typename T>
static hipError_t swish_grad_strided_t(const void* grad, const void* x, void* out,
                                       const StridedView& v, int64_t n, float beta,
                                       hipStream_t stream) {
  if (v.nd == 2 && (v.stride[0][0] == 1 || v.stride[1][0] == 1 || v.stride[2][0] == 1)) {
    const int64_t R = v.size[0], C = v.size[1];
    int64_t tiles = ceil_div(R, kTrTile) * ceil_div(C, kTrTile);
    if (tiles > kMaxStreamBlocks) tiles = kMaxStreamBlocks;
    const int64_t es = (int64_t)sizeof(T);
    if (line4_ok(grad, v.stride[0][0], v.stride[0][1], es) &&
        line4_ok(x, v.stride[1][0], v.stride[1][1], es) &&
        line4_ok(out, v.stride[2][0], v.stride[2][1], es)) {
      SWG_LAUNCH((swish_grad_tr2d_vec_kernel<T>), dim3((unsigned)tiles), dim3(256), 0,
                         stream, static_cast<const T*>(grad), static_cast<const T*>(x),
                         static_cast<T*>(out), R, C, v.stride[0][0], v.stride[0][1],
                         v.stride[1][0], v.stride[1][1], v.stride[2][0], v.stride[2][1], beta);
      return hipGetLastError();
    }
    SWG_LAUNCH((swish_grad_tr2d_kernel<T>), dim3((unsigned)tiles), dim3(256), 0, stream,
                       static_cast<const T*>(grad), static_cast<const T*>(x),
                       static_cast<T*>(out), R, C, v.stride[0][0], v.stride[0][1],
                       v.stride[1][0], v.stride[1][1], v.stride[2][0], v.stride[2][1], beta);
    return hipGetLastError();
  }
  StridedArgs a;
  a.nd = v.nd;
  // 32-bit path: every index below 2^32 and every divisor at most 2^31 (the magic
  // number then fits in 32 bits)
  bool narrow = n <= 0xFFFFFFFFll;
  for (int k = 0; k < kMaxStridedDims; ++k) {
    const bool used = k < v.nd;
    narrow = narrow && (!used || v.size[k] <= (int64_t(1) << 31));
    a.size[k] = used ? v.size[k] : 1;
    a.div[k] = make_fastdiv(used && v.size[k] <= (int64_t(1) << 31) ? (uint32_t)v.size[k] : 1u);
    a.sg[k] = used ? v.stride[0][k] : 0;
    a.sx[k] = used ? v.stride[1][k] : 0;
    a.so[k] = used ? v.stride[2][k] : 0;
  }
  int64_t blocks = ceil_div(n, 256);
  if (blocks > kMaxStreamBlocks) blocks = kMaxStreamBlocks;
  const T* g = static_cast<const T*>(grad);
  const T* xx = static_cast<const T*>(x);
  T* o = static_cast<T*>(out);
  if (narrow)
    SWG_LAUNCH((swish_grad_strided_kernel<T, false>), dim3((unsigned)blocks), dim3(256),
                       0, stream, g, xx, o, a, n, beta);
  else
    SWG_LAUNCH((swish_grad_strided_kernel<T, true>), dim3((unsigned)blocks), dim3(256),
                       0, stream, g, xx, o, a, n, beta);
  return hipGetLastError();
}

hipError_t launch_swish_grad_strided(int dtype, const void* grad, const void* x, void* out,
                                     const StridedView& v, int64_t n, float beta,
                                     hipStream_t stream) {
  switch (dtype) {
    case 0: return swish_grad_strided_t<bf16>(grad, x, out, v, n, beta, stream);
    case 1: return swish_grad_strided_t<fp16>(grad, x, out, v, n, beta, stream);
    default: return swish_grad_strided_t<float>(grad, x, out, v, n, beta, stream);
  }
}

}  // namespace swg
