// fp32 path of the w and x stages and of the SwiGLU forward (fp32 tensors): the same
// GEMMs as the bf16 / fp16 kernels [Fused SwiGLU backward page, formulas 3 and 4; SwiGLU
// page, operator background], on the fp32 matrix cores (v_mfma_f32_32x32x2_f32), fp32
// accumulation, one rounding-free store per output.
//
// Output tiles of 128 x 128 per workgroup of four waves (2 x 2, each 64 x 64 = 2 x 2
// blocks of 32 x 32 accumulators); the contraction advances 32 at a time through a
// double-buffered LDS stage (operands loaded as 16-byte vectors into registers, written
// to LDS as [32 contraction][128] so that each lane's MFMA operand is one 4-byte read
// from a row of 128 consecutive floats).  The next stage's global loads are issued before
// the current stage's MFMAs and written to the other LDS buffer after them.
//
// Operand layouts: element (p, r) (row p of the output side, contraction index r) sits
//   at src[p * ld + r] when the contraction is contiguous (CK: dg / dfc and W in the x
//   stage), at src[r * ld + p] when the rows are (x, dg, dfc in the w stage).
// Rows and contraction indices past the tensors load as zeros; K and N are multiples of
// 4, so a 16-byte vector is either wholly inside or wholly outside.
#include <utility>

#include "common.hpp"
#include "launch.hpp"

namespace swg {

namespace {

constexpr int T32 = 128;            // output tile rows and columns
constexpr int K32 = 32;             // contraction per stage
constexpr int LD32 = T32 + 4;       // LDS row pitch in floats (rows 16 bytes apart in bank)
constexpr int NT32 = 256;

// Four 16-byte vectors per lane cover a [128 rows][32 contraction] operand tile.
template <bool CK>
struct Tile32 {
  static constexpr int NV = K32 / 8;   // 16-byte vectors per lane
  static constexpr int RV = K32 / 4;   // 16-byte vectors per row (contraction-contiguous)
  f32x4 v[NV];

  // rows [p0, p0 + 128) limited to plim, contraction [r0, r0 + K32) limited to rlim
  __device__ void load(const float* src, int64_t ld, int64_t p0, int64_t r0, int64_t plim,
                       int64_t rlim, int tid) {
#pragma unroll
    for (int h = 0; h < NV; ++h) {
      int64_t p, r;
      if (CK) {
        p = p0 + (tid / RV) + (256 / RV) * h;
        r = r0 + (tid % RV) * 4;
      } else {
        r = r0 + (tid >> 5) + 8 * h;
        p = p0 + (tid & 31) * 4;
      }
      const bool ok = p < plim && r < rlim;
      v[h] = ok ? *reinterpret_cast<const f32x4*>(src + (CK ? p * ld + r : r * ld + p))
                : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  // to LDS [K32][LD32]: element (p, r) at r * LD32 + p
  __device__ void store(float* lds, int tid) const {
#pragma unroll
    for (int h = 0; h < NV; ++h) {
      if (CK) {
        const int p = (tid / RV) + (256 / RV) * h, r = (tid % RV) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) lds[(r + e) * LD32 + p] = v[h][e];
      } else {
        const int r = (tid >> 5) + 8 * h, p = (tid & 31) * 4;
        *reinterpret_cast<f32x4*>(lds + r * LD32 + p) = v[h];
      }
    }
  }
};

// The 32 MFMAs of one stage: per contraction pair s, lane l supplies row l % 32 and
// contraction index 2 s + l / 32 of each operand block.
__device__ inline void stage32(const float* la, const float* lb, int wp, int wq, int lane,
                               f32x16 (&acc)[2][2]) {
#pragma unroll
  for (int s = 0; s < K32 / 2; ++s) {
    const int k = 2 * s + (lane >> 5);
    float a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = la[k * LD32 + wp * 64 + i * 32 + (lane & 31)];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = lb[k * LD32 + wq * 64 + j * 32 + (lane & 31)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Contraction over one operand pair: A rows [pa0, ...) (limit plim), B rows [qb0, ...)
// (limit qlim), contraction [rb, re).  LDS: two buffers of A and B stages.
template <bool ACK, bool BCK>
__device__ inline void contract32(const float* A, int64_t lda, int64_t pa0, int64_t plim,
                                  const float* B, int64_t ldb, int64_t qb0, int64_t qlim,
                                  int64_t rb, int64_t re, float* lds, int tid, int wp, int wq,
                                  int lane, f32x16 (&acc)[2][2]) {
  if (re <= rb) return;
  float* la[2] = {lds, lds + 2 * K32 * LD32};
  float* lb[2] = {lds + K32 * LD32, lds + 3 * K32 * LD32};
  Tile32<ACK> ta;
  Tile32<BCK> tb;
  ta.load(A, lda, pa0, rb, plim, re, tid);
  tb.load(B, ldb, qb0, rb, qlim, re, tid);
  __syncthreads();   // the previous contraction's last reads of buffer 0 are done
  ta.store(la[0], tid);
  tb.store(lb[0], tid);
  __syncthreads();
  int cur = 0;
  for (int64_t r0 = rb; r0 < re; r0 += K32) {
    const bool more = r0 + K32 < re;
    if (more) {
      ta.load(A, lda, pa0, r0 + K32, plim, re, tid);
      tb.load(B, ldb, qb0, r0 + K32, qlim, re, tid);
    }
    stage32(la[cur], lb[cur], wp, wq, lane, acc);
    if (more) {
      ta.store(la[cur ^ 1], tid);
      tb.store(lb[cur ^ 1], tid);
    }
    __syncthreads();
    cur ^= 1;
  }
}

// Visit every accumulator: fn(row, col, value) in tile coordinates.
template <typename Fn>
__device__ inline void for_each_acc32(const f32x16 (&acc)[2][2], int wp, int wq, int lane,
                                      Fn&& fn) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        fn(wp * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3),
           wq * 64 + j * 32 + (lane & 31), acc[i][j][r]);
}

__device__ inline void zero32(f32x16 (&acc)[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// x stage, fp32: dx[m, k] = sum_n dg[m, n] W_g[k, n] + sum_n dfc[m, n] W_fc[k, n]
__global__ __launch_bounds__(NT32) void x_stage32_kernel(const float* __restrict__ dg,
                                                         const float* __restrict__ dfc,
                                                         const float* __restrict__ wg,
                                                         const float* __restrict__ wfc,
                                                         float* __restrict__ dx, int64_t M,
                                                         int64_t K, int64_t N, int64_t nq) {
  __shared__ __attribute__((aligned(16))) float lds[4 * K32 * LD32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave >> 1, wq = wave & 1;
  const int64_t m0 = (int64_t)(blockIdx.x / nq) * T32, k0 = (int64_t)(blockIdx.x % nq) * T32;
  f32x16 acc[2][2];
  zero32(acc);
  contract32<true, true>(dg, N, m0, M, wg, N, k0, K, 0, N, lds, tid, wp, wq, lane, acc);
  contract32<true, true>(dfc, N, m0, M, wfc, N, k0, K, 0, N, lds, tid, wp, wq, lane, acc);
  for_each_acc32(acc, wp, wq, lane, [&](int row, int col, float v) {
    const int64_t m = m0 + row, k = k0 + col;
    if (m < M && k < K) dx[m * K + k] = v;
  });
}

// w stage, fp32: item (split s, tile): C[k, n] = sum over rows m of split s of
// x[m, k] d[m, n] (d = dg for the first tn / 2 column tiles, dfc for the rest); with
// splits the fp32 partial goes to ws[s][k][2N], otherwise dw[k, n] += C.
__global__ __launch_bounds__(NT32) void w_stage32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ dg,
                                                         const float* __restrict__ dfc,
                                                         float* __restrict__ dwg,
                                                         float* __restrict__ dwfc,
                                                         float* __restrict__ ws, int64_t M,
                                                         int64_t K, int64_t N, int64_t tk,
                                                         int64_t tnh, int64_t split_rows) {
  __shared__ __attribute__((aligned(16))) float lds[4 * K32 * LD32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave >> 1, wq = wave & 1;
  const int64_t tiles = tk * 2 * tnh;
  const int64_t s = blockIdx.x / tiles, tt = blockIdx.x % tiles;
  const int64_t kb = tt / (2 * tnh), nb = tt % (2 * tnh);
  const bool hi = nb >= tnh;
  const int64_t k0 = kb * T32, n0 = (hi ? nb - tnh : nb) * T32;
  const int64_t mb = s * split_rows;
  const int64_t me = mb + split_rows < M ? mb + split_rows : M;
  const float* d = hi ? dfc : dg;
  f32x16 acc[2][2];
  zero32(acc);
  contract32<false, false>(x, K, k0, K, d, N, n0, N, mb, me, lds, tid, wp, wq, lane, acc);
  if (ws != nullptr) {
    float* dst = ws + s * K * 2 * N + (hi ? N : 0);
    for_each_acc32(acc, wp, wq, lane, [&](int row, int col, float v) {
      const int64_t k = k0 + row, n = n0 + col;
      if (k < K && n < N) dst[k * 2 * N + n] = v;
    });
  } else {
    // dw += C: every old value is loaded before any store (a load-add-store per element
    // would be one memory round trip each, since loads of dw cannot move above its stores)
    float* dw = hi ? dwfc : dwg;
    float old[64];
    int e = 0;
    for_each_acc32(acc, wp, wq, lane, [&](int row, int col, float) {
      const int64_t k = k0 + row, n = n0 + col;
      old[e++] = (k < K && n < N) ? dw[k * N + n] : 0.0f;
    });
    e = 0;
    for_each_acc32(acc, wp, wq, lane, [&](int row, int col, float v) {
      const int64_t k = k0 + row, n = n0 + col;
      if (k < K && n < N) dw[k * N + n] = old[e] + v;
      ++e;
    });
  }
}

// SwiGLU forward, fp32 [SwiGLU page, operator background]: g = x W_g + b_g,
// fc = x W_fc + b_fc, y = g sigma(g) fc.  A = x rows m (contraction k contiguous);
// B = W_g then W_fc, element (n, k) at W[k N + n] (rows n contiguous).  Biases may be
// null (zero).
__global__ __launch_bounds__(NT32) void fwd32_kernel(const float* __restrict__ x,
                                                     const float* __restrict__ wg,
                                                     const float* __restrict__ wfc,
                                                     const float* __restrict__ bg,
                                                     const float* __restrict__ bfc,
                                                     float* __restrict__ g,
                                                     float* __restrict__ fc,
                                                     float* __restrict__ y, int64_t M,
                                                     int64_t K, int64_t N, int64_t nn) {
  __shared__ __attribute__((aligned(16))) float lds[4 * K32 * LD32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave >> 1, wq = wave & 1;
  const int64_t m0 = (int64_t)(blockIdx.x / nn) * T32, n0 = (int64_t)(blockIdx.x % nn) * T32;
  f32x16 ag[2][2], af[2][2];
  zero32(ag);
  zero32(af);
  contract32<true, false>(x, K, m0, M, wg, N, n0, N, 0, K, lds, tid, wp, wq, lane, ag);
  contract32<true, false>(x, K, m0, M, wfc, N, n0, N, 0, K, lds, tid, wp, wq, lane, af);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wq * 64 + j * 32 + (lane & 31);
      const int64_t n = n0 + col;
      const float bgv = (bg != nullptr && n < N) ? bg[n] : 0.0f;
      const float bfv = (bfc != nullptr && n < N) ? bfc[n] : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wp * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < N) {
          const float gv = ag[i][j][r] + bgv, fv = af[i][j][r] + bfv;
          const int64_t o = m * N + n;
          // written once and not read again here: non-temporal stores keep the x and W
          // panels in the caches (as in the 16-bit forward)
          __builtin_nontemporal_store(gv, g + o);
          __builtin_nontemporal_store(fv, fc + o);
          __builtin_nontemporal_store(gv * sigmoid_only(gv) * fv, y + o);
        }
      }
    }
}

}  // namespace

hipError_t launch_fwd32(const void* x, const void* w_g, const void* w_fc, const void* b_g,
                        const void* b_fc, void* g, void* fc, void* y, int64_t M, int64_t K,
                        int64_t N, hipStream_t stream) {
  const int64_t np = ceil_div(M, T32), nn = ceil_div(N, T32);
  SWG_LAUNCH(fwd32_kernel, dim3((unsigned)(np * nn)), dim3(NT32), 0, stream,
                     static_cast<const float*>(x), static_cast<const float*>(w_g),
                     static_cast<const float*>(w_fc), static_cast<const float*>(b_g),
                     static_cast<const float*>(b_fc), static_cast<float*>(g),
                     static_cast<float*>(fc), static_cast<float*>(y), M, K, N, nn);
  return hipGetLastError();
}

hipError_t launch_x_stage32(const void* dg, const void* dfc, const void* w_g, const void* w_fc,
                            void* dx, int64_t M, int64_t K, int64_t N, hipStream_t stream) {
  const int64_t np = ceil_div(M, T32), nq = ceil_div(K, T32);
  SWG_LAUNCH(x_stage32_kernel, dim3((unsigned)(np * nq)), dim3(NT32), 0, stream,
                     static_cast<const float*>(dg), static_cast<const float*>(dfc),
                     static_cast<const float*>(w_g), static_cast<const float*>(w_fc),
                     static_cast<float*>(dx), M, K, N, nq);
  return hipGetLastError();
}

hipError_t launch_w_stage32(const WPlan& p, const void* x, const void* dg, const void* dfc,
                            void* dw_g, void* dw_fc, int64_t M, int64_t K, int64_t N, float* ws,
                            hipStream_t stream) {
  const int64_t tk = ceil_div(K, T32), tnh = ceil_div(N, T32);
  const int64_t items = p.splits * tk * 2 * tnh;
  float* wsp = p.splits > 1 ? ws : nullptr;
  SWG_LAUNCH(w_stage32_kernel, dim3((unsigned)items), dim3(NT32), 0, stream,
                     static_cast<const float*>(x), static_cast<const float*>(dg),
                     static_cast<const float*>(dfc), static_cast<float*>(dw_g),
                     static_cast<float*>(dw_fc), wsp, M, K, N, tk, tnh, p.rows);
  return hipGetLastError();
}

}  // namespace swg
