// Matrix-core kernels for gfx950: the w stage [dw_g | dw_fc] += x^T [dg | dfc]
// (one TN GEMM [K, M] x [M, 2N]) and the x stage dx = [dg | dfc] [W_g | W_fc]^T
// (one NT GEMM [M, 2N] x [2N, K]).  Source: the Fused SwiGLU backward page
// (PyPTO-Gym), formulas 3 and 4, and its matmul transposition flags (w: a
// transposed, b not; x: a not, b transposed); fp32 accumulation as in its dtype table.
//
// Both kernels compute a 256 x 256 output tile per workgroup from LDS tiles laid out
// as [rows][contraction] with a 16-byte pad per row, so that every lane fetches its
// MFMA operand (8 consecutive contraction elements) with one 16-byte LDS read and the
// 32 rows of a 32 x 32 x 16 MFMA hit distinct banks.  Two LDS stages: while the matrix
// cores work on stage t, the lanes hold the global loads of stage t + 1 in registers.
//
//   x stage: both operands are contraction-contiguous in memory, copied as is.
//   w stage: both operands are contraction-strided (the contraction runs over rows of
//            x and dg), so each lane loads an 8 x 8 block (8 rows x 16 bytes, fully
//            coalesced along the row) and transposes it in registers before the LDS
//            store.
//
// Workgroup ids are remapped so that consecutive logical tiles run on one XCD
// (the hardware deals consecutive ids round-robin over the 8 XCDs): tiles that share
// an operand panel then share that XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace swg {

template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  typedef bf16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<fp16> {
  typedef fp16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int BP = kTileP, BQ = kTileQ, BR = kTileR;
constexpr int LDR = BR + 8;            // LDS row stride (elements): 144 bytes
constexpr int STAGE = (BP + BQ) * LDR;  // elements per LDS stage
constexpr int LDC = BQ + 8;            // LDS row stride of the staged output tile
static_assert(BP * LDC <= 2 * STAGE, "output staging must fit in the operand stages");

// consecutive logical tiles -> same XCD
__device__ inline int64_t xcd_remap(int64_t b, int64_t nblocks) {
  const int64_t per = nblocks / 8;
  if (b >= per * 8) return b;
  return (b % 8) * per + b / 8;
}

// ----------------------------------------------------------------- compute core
// WP x WQ wavefronts; each owns a (BP / WP) x (BQ / WQ) block of 32 x 32 MFMA tiles.
// MFMA 32x32x16 operand layout: lane l supplies row (l % 32), contraction elements
// 8 (l / 32) .. 8 (l / 32) + 7; the accumulator lane l holds column (l % 32) and rows
// 8 (r / 4) + 4 (l / 32) + (r % 4) for r = 0..15.
template <int WP_, int WQ_>
struct Waves {
  static constexpr int WP = WP_, WQ = WQ_;
  static constexpr int NT = 64 * WP * WQ;
  static constexpr int FP = BP / WP / 32, FQ = BQ / WQ / 32;
};
// 8 wavefronts (2 per SIMD), each 128 x 64: 128 accumulator registers per lane.
typedef Waves<2, 4> GemmWaves;

template <typename T, class C>
__device__ inline void mma_stage(const uint16_t* As, const uint16_t* Bs, int wp, int wq, int lane,
                                 f32x16 (&acc)[C::FP][C::FQ]) {
  constexpr int WP = C::WP, WQ = C::WQ, FP = C::FP, FQ = C::FQ;
  using F = typename Mfma<T>::frag;
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < BR; kk += 16) {
    F a[FP], b[FQ];
#pragma unroll
    for (int i = 0; i < FP; ++i)
      a[i] = *reinterpret_cast<const F*>(As + (wp * (BP / WP) + i * 32 + lrow) * LDR + kk + lk);
#pragma unroll
    for (int j = 0; j < FQ; ++j)
      b[j] = *reinterpret_cast<const F*>(Bs + (wq * (BQ / WQ) + j * 32 + lrow) * LDR + kk + lk);
#pragma unroll
    for (int i = 0; i < FP; ++i)
#pragma unroll
      for (int j = 0; j < FQ; ++j) acc[i][j] = Mfma<T>::mma(a[i], b[j], acc[i][j]);
  }
}

// ----------------------------------------------------------------- x stage (NT)
// A = [dg | dfc] rows p (M), B = [W_g | W_fc] rows q (K); contraction over 2N.
template <typename T, class C>
__global__ __launch_bounds__(C::NT) void x_stage_kernel(
    const T* __restrict__ dg, const T* __restrict__ dfc, const T* __restrict__ wg,
    const T* __restrict__ wfc, T* __restrict__ dx, int64_t M, int64_t K, int64_t N,
    int64_t nq) {
  constexpr int WP = C::WP, WQ = C::WQ, FP = C::FP, FQ = C::FQ, NT = C::NT;
  constexpr int XCH = (BP * BR / 8) / NT;  // 16-byte chunks per lane per operand
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave / WQ, wq = wave % WQ;
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t p0 = (L / nq) * BP, q0 = (L % nq) * BQ;
  const int64_t R = 2 * N;
  const int64_t nsteps = (R + BR - 1) / BR;

  f32x16 acc[FP][FQ];
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x4 ra[XCH], rb[XCH];
  auto load = [&](int64_t r0) {
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int id = tid + c * NT;
      const int row = id >> 3, ch = id & 7;
      const int64_t rr = r0 + ch * 8;
      const int64_t p = p0 + row, q = q0 + row;
      u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
      if (rr < R) {
        const bool lo = rr < N;
        const int64_t col = lo ? rr : rr - N;
        if (p < M) va = ld16((lo ? dg : dfc) + p * N + col);
        if (q < K) vb = ld16((lo ? wg : wfc) + q * N + col);
      }
      ra[c] = va;
      rb[c] = vb;
    }
  };
  auto store = [&](int buf) {
    uint16_t* As = lds + buf * STAGE;
    uint16_t* Bs = As + BP * LDR;
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int id = tid + c * NT;
      const int row = id >> 3, ch = id & 7;
      st16(As + row * LDR + ch * 8, ra[c]);
      st16(Bs + row * LDR + ch * 8, rb[c]);
    }
  };

  load(0);
  store(0);
  __syncthreads();
  for (int64_t t = 0; t < nsteps; ++t) {
    const int buf = (int)(t & 1);
    if (t + 1 < nsteps) load((t + 1) * BR);
    mma_stage<T, C>(lds + buf * STAGE, lds + buf * STAGE + BP * LDR, wp, wq, lane, acc);
    if (t + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }

  // epilogue: round to T, stage the 256 x 256 tile in LDS, write 16-byte rows
  T* Cs = reinterpret_cast<T*>(lds);
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wp * (BP / WP) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wq * (BQ / WQ) + j * 32 + (lane & 31);
        Cs[row * LDC + col] = from_f32<T>(acc[i][j][r]);
      }
  __syncthreads();
  constexpr int CCH = BP * BQ / 8 / NT;
#pragma unroll 4
  for (int c = 0; c < CCH; ++c) {
    const int id = tid + c * NT;
    const int row = id / (BQ / 8), ch = id % (BQ / 8);
    const int64_t p = p0 + row, q = q0 + ch * 8;
    if (p < M && q < K)
      st16(dx + p * K + q, *reinterpret_cast<const u32x4*>(Cs + row * LDC + ch * 8));
  }
}

// ----------------------------------------------------------------- w stage (TN)
// A = x^T: rows k (K), contraction m;  B = [dg | dfc]^T: rows n (2N), contraction m.
// 8 x 8 blocks of 16-bit elements: 256 per operand per stage.
static_assert(BP == BQ, "w-stage block split assumes square tiles");

__device__ inline void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
  // in[i]: 8 halves of source row i; out[j]: the 8 rows' half j
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = j >> 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a = in[2 * e][d], b = in[2 * e + 1][d];
      out[j][e] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

template <typename T, class C>
__global__ __launch_bounds__(C::NT) void w_stage_kernel(
    const T* __restrict__ x, const T* __restrict__ dg, const T* __restrict__ dfc,
    T* __restrict__ dwg, T* __restrict__ dwfc, float* __restrict__ ws, int64_t M, int64_t K,
    int64_t N, int64_t tn, int64_t tiles, int64_t split_rows) {
  constexpr int WP = C::WP, WQ = C::WQ, FP = C::FP, FQ = C::FQ, NT = C::NT;
  constexpr int WBLK = (2 * (BP * BR / 64)) / NT;  // 8 x 8 blocks per lane per stage
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave / WQ, wq = wave % WQ;
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t s = L / tiles, tt = L % tiles;
  const int64_t k0 = (tt / tn) * BP, n0 = (tt % tn) * BQ;
  const int64_t m_begin = s * split_rows;
  const int64_t m_end = (m_begin + split_rows < M) ? m_begin + split_rows : M;
  const int64_t R2 = 2 * N;
  const int64_t nsteps = (m_end - m_begin + BR - 1) / BR;

  f32x16 acc[FP][FQ];
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x4 rin[WBLK][8];
  auto load = [&](int64_t m0) {
#pragma unroll
    for (int bI = 0; bI < WBLK; ++bI) {
      const int id = tid + bI * NT;
      const bool isA = id < (BP * BR / 64);
      const int bid = isA ? id : id - (BP * BR / 64);
      const int bc = bid & 31, bm = bid >> 5;  // 8-column group, 8-row group
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t m = m0 + bm * 8 + i;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m < m_end) {
          if (isA) {
            const int64_t k = k0 + bc * 8;
            if (k < K) v = ld16(x + m * K + k);
          } else {
            const int64_t n = n0 + bc * 8;
            if (n < R2) v = ld16(n < N ? dg + m * N + n : dfc + m * N + (n - N));
          }
        }
        rin[bI][i] = v;
      }
    }
  };
  auto store = [&](int buf) {
    uint16_t* As = lds + buf * STAGE;
    uint16_t* Bs = As + BP * LDR;
#pragma unroll
    for (int bI = 0; bI < WBLK; ++bI) {
      const int id = tid + bI * NT;
      const bool isA = id < (BP * BR / 64);
      const int bid = isA ? id : id - (BP * BR / 64);
      const int bc = bid & 31, bm = bid >> 5;
      u32x4 out[8];
      transpose8x8(rin[bI], out);
      uint16_t* base = (isA ? As : Bs) + (bc * 8) * LDR + bm * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) st16(base + j * LDR, out[j]);
    }
  };

  if (nsteps > 0) {
    load(m_begin);
    store(0);
  }
  __syncthreads();
  for (int64_t t = 0; t < nsteps; ++t) {
    const int buf = (int)(t & 1);
    if (t + 1 < nsteps) load(m_begin + (t + 1) * BR);
    mma_stage<T, C>(lds + buf * STAGE, lds + buf * STAGE + BP * LDR, wp, wq, lane, acc);
    if (t + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }

  // epilogue: rows k, cols n of the [K, 2N] result
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t k = k0 + wp * (BP / WP) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wq * (BQ / WQ) + j * 32 + (lane & 31);
        if (k < K && n < R2) {
          if (ws != nullptr) {
            ws[(s * K + k) * R2 + n] = acc[i][j][r];
          } else {
            T* dst = n < N ? dwg + k * N + n : dwfc + k * N + (n - N);
            *dst = from_f32<T>(to_f32(*dst) + acc[i][j][r]);
          }
        }
      }
}

// dw = RNE(dw + sum_s ws[s]) in split order; 4 consecutive columns per lane (N % 8 == 0,
// so a group never straddles the dg | dfc boundary).
template <typename T>
__global__ __launch_bounds__(256) void w_reduce_kernel(const float* __restrict__ ws,
                                                       T* __restrict__ dwg, T* __restrict__ dwfc,
                                                       int64_t K, int64_t N, int64_t S) {
  const int64_t W = 2 * N;
  const int64_t total4 = K * W / 4;
  const int64_t plane = K * W;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total4;
       i += (int64_t)gridDim.x * 256) {
    const int64_t e = i * 4;
    f32x4 acc = *reinterpret_cast<const f32x4*>(ws + e);
    for (int64_t si = 1; si < S; ++si) acc += *reinterpret_cast<const f32x4*>(ws + si * plane + e);
    const int64_t k = e / W, n = e % W;
    T* dst = n < N ? dwg + k * N + n : dwfc + k * N + (n - N);
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = from_f32<T>(to_f32(dst[c]) + acc[c]);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

template <typename T>
static hipError_t x_stage_t(const void* dg, const void* dfc, const void* wg, const void* wfc,
                            void* dx, int64_t M, int64_t K, int64_t N, hipStream_t stream) {
  const int64_t np = ceil_div(M, BP), nq = ceil_div(K, BQ);
  hipLaunchKernelGGL((x_stage_kernel<T, GemmWaves>), dim3((unsigned)(np * nq)),
                     dim3(GemmWaves::NT), 0,
                     stream, static_cast<const T*>(dg), static_cast<const T*>(dfc),
                     static_cast<const T*>(wg), static_cast<const T*>(wfc), static_cast<T*>(dx),
                     M, K, N, nq);
  return hipGetLastError();
}

hipError_t launch_x_stage(int dtype, const void* dg, const void* dfc, const void* w_g,
                          const void* w_fc, void* dx, int64_t M, int64_t K, int64_t N,
                          hipStream_t stream) {
  if (dtype == 0) return x_stage_t<bf16>(dg, dfc, w_g, w_fc, dx, M, K, N, stream);
  return x_stage_t<fp16>(dg, dfc, w_g, w_fc, dx, M, K, N, stream);
}

template <typename T>
static hipError_t w_stage_t(const WPlan& p, const void* x, const void* dg, const void* dfc,
                            void* dwg, void* dwfc, int64_t M, int64_t K, int64_t N, float* ws,
                            hipStream_t stream) {
  float* wsp = p.splits > 1 ? ws : nullptr;
  hipLaunchKernelGGL((w_stage_kernel<T, GemmWaves>), dim3((unsigned)(p.splits * p.tiles)),
                     dim3(GemmWaves::NT), 0, stream, static_cast<const T*>(x),
                     static_cast<const T*>(dg), static_cast<const T*>(dfc), static_cast<T*>(dwg),
                     static_cast<T*>(dwfc), wsp, M, K, N, p.tn, p.tiles, p.rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  int64_t blocks = ceil_div(K * 2 * N / 4, 256);
  if (blocks > kMaxStreamBlocks) blocks = kMaxStreamBlocks;
  hipLaunchKernelGGL((w_reduce_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, stream, ws,
                     static_cast<T*>(dwg), static_cast<T*>(dwfc), K, N, p.splits);
  return hipGetLastError();
}

hipError_t launch_w_stage(int dtype, const WPlan& p, const void* x, const void* dg,
                          const void* dfc, void* dw_g, void* dw_fc, int64_t M, int64_t K,
                          int64_t N, float* ws, hipStream_t stream) {
  if (dtype == 0) return w_stage_t<bf16>(p, x, dg, dfc, dw_g, dw_fc, M, K, N, ws, stream);
  return w_stage_t<fp16>(p, x, dg, dfc, dw_g, dw_fc, M, K, N, ws, stream);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t words = (int64_t)(bytes / 4);
  int64_t blocks = ceil_div(words, 256);
  if (blocks > kMaxStreamBlocks) blocks = kMaxStreamBlocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((fill_zero_kernel<int>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace swg
