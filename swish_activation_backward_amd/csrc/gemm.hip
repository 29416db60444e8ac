// Matrix-core kernels for gfx950: the w stage [dw_g | dw_fc] += x^T [dg | dfc]
// (one TN GEMM [K, M] x [M, 2N]) and the x stage dx = [dg | dfc] [W_g | W_fc]^T
// (one NT GEMM [M, 2N] x [2N, K]).  Source: the Fused SwiGLU backward page
// (PyPTO-Gym), formulas 3 and 4 and its matmul transposition flags (w: first operand
// transposed; x: second operand transposed); fp32 accumulation as in its dtype flow.
//
// Both kernels compute a 256 x 256 output tile per workgroup of four wavefronts (one
// per SIMD); each wave owns a 128 x 128 block = 4 x 4 tiles of v_mfma_f32_32x32x16 whose
// 256 fp32 accumulators live in the AGPR file.  A second configuration halves every edge
// (128 x 128 tiles, 64 x 64 per wave) for outputs that 256 x 256 tiles would spread over
// too few CUs (see Tc below).
//
// Operands move global -> LDS with buffer_load ... lds (the load unit writes LDS
// directly; no registers, no ds_write), and operand fragments are double-buffered in
// registers: while the matrix cores multiply one 32-deep stage from registers, the
// fragments of the next stage are read from LDS and later stages are in flight.  A stage
// is read only after `s_waitcnt vmcnt` says this wave's part of it landed and a barrier
// says every wave's part did.  The loads of a step and the next stage's LDS reads are
// spread between that step's MFMAs (scheduling fences fix the order), so the load issue
// does not stall the matrix cores behind the barrier.  Rows and columns outside the
// tensors (ragged M, partial tiles, stages past the end) are fetched at offsets beyond
// the buffer window and arrive as zeros from the hardware range check: the loop has no
// data-path branches.
//
//   x stage: both operands are contraction-contiguous in memory; LDS holds three 64-deep
//            slots of [dg | dfc] rows and two of [W_g | W_fc] rows, [row][64] each, and
//            each lane reads one MFMA operand (8 consecutive contraction elements) with
//            a 16-byte ds_read_b128.
//   w stage: both operands are contraction-strided (the contraction runs over the rows
//            of x and dg); LDS is a ring of four 32-deep stages kept as loaded,
//            [32 contraction][256 columns] per operand, and the operands are read with
//            the gfx950 transposing LDS read ds_read_b64_tr_b16 (two per operand).
// Every LDS tile is XOR-swizzled in 16-byte chunks (the swizzle is applied to the
// global address each lane fetches, since the LDS write order is fixed by the load
// unit) so that the operand reads of one instruction hit distinct banks.
//
// The concatenations [dg | dfc] and [W_g | W_fc] are never materialised: the x stage
// runs its contraction over dg/W_g and then dfc/W_fc, and the w stage gives each
// output tile one of dg or dfc.
//
// Both kernels are persistent: one workgroup per CU walks a list of output tiles and the
// ring keeps streaming across tile boundaries (the first stages of the next tile are in
// flight while the current tile finishes and writes its result straight from the
// accumulators).  Work is dealt so that concurrently running tiles with neighbouring
// indices sit on one XCD (the hardware deals workgroup ids round-robin over the 8
// XCDs): tiles sharing an operand panel then share that XCD's L2.
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "launch.hpp"

namespace swg {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
#define LDS_AS __attribute__((address_space(3)))

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

constexpr int BP = kTileP, BQ = kTileQ, BR = kTileR;   // 256 x 256 tile, 32-deep stages
constexpr int NT = 256;                                 // 4 wavefronts, 2 x 2
constexpr int WP = 2, WQ = 2;
constexpr int FP = BP / WP / 32, FQ = BQ / WQ / 32;     // 4 x 4 MFMA tiles per wave
constexpr int SLOT = (BP + BQ) * BR;                    // elements per ring slot (32 KiB)
constexpr int LOADS_PER_STAGE = SLOT * 2 / 1024 / (NT / 64);   // 1 KiB loads per wave: 8
constexpr uint32_t kOOB = 0x80000000u;  // offset past every window: loads zeros
static_assert(BR == 32 && BP == 256 && BQ == 256, "swizzles below assume 256 x 256 x 32");
constexpr int XA_BR = 2 * BR;   // x stage: contraction elements per double stage

// Workgroup tile configurations of the w and x stages.  F = 4: 256 x 256 outputs, each
// wave 128 x 128 (4 x 4 MFMA tiles, 256 accumulators); F = 2: 128 x 128 outputs, each wave
// 64 x 64 (2 x 2 tiles), for outputs whose 256 x 256 tiles would leave most CUs idle.  The
// loops, swizzles and ring layouts are the same; only the tile edge changes.
template <int F> struct Tc {
  static_assert(F == 2 || F == 4, "tile configurations");
  static constexpr int P = 64 * F;                       // tile edge (rows = columns)
  static constexpr int WR = 32 * F;                      // rows / columns per wave
  static constexpr int XSLOT = P * XA_BR;                // x stage: elements per A or B slot
  static constexpr int XLOADS = XSLOT * 2 / 1024 / (NT / 64);   // 1 KiB loads per wave: 2F
  static constexpr int X_RING = 5 * XSLOT;               // 3 A slots + 2 B slots
  static constexpr int WSLOT = 2 * P * BR;               // w stage: elements per ring slot
  static constexpr int WLOADS = WSLOT * 2 / 1024 / (NT / 64);   // 1 KiB loads per wave: 2F
  static constexpr int W_RING = 4 * WSLOT;
  static constexpr int RPL = 1024 / (2 * P);             // w-stage rows per 1 KiB load
  static constexpr int RING = X_RING > W_RING ? X_RING : W_RING;
  // x-stage workgroups per CU: at F = 2 the ring (80 KiB) and the registers fit twice, and
  // a second wave per SIMD raises the LDS read rate the 128 x 128 tile is bound by
  static constexpr int XOCC = F == 4 ? 1 : 2;
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
constexpr int vmcnt_le(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }
constexpr int kLgkmcnt0 = 0xC07F;   // s_waitcnt lgkmcnt(0), other counters free

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer, no stride: offsets >= bytes return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ inline uint32_t clamp_bytes(int64_t rows, int64_t row_bytes) {
  return rows > 0 ? (uint32_t)(rows * row_bytes) : 0u;
}
// 16 bytes per lane from window `r` at soffset + voffset to LDS at dst + OFS + 16 * lane
// (dst must be wave-uniform).  The hardware range check applies to voffset (plus the
// instruction offset) against the window's size, not to soffset: a wave-uniform column or
// stage offset can go into soffset while the per-lane row term in voffset keeps rows past
// the window reading zeros.  Issued as inline asm: the loads' completion is tracked by
// the explicit vmcnt waits of the pipeline (the compiler's own tracking of LDS-DMA stores
// would add conservative waits that drain the ring).  The constant OFS is added to M0
// inside the asm so one scalar base serves all loads of a stage.
template <int OFS>
__device__ inline void dma16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                              const uint16_t* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(LDS_AS const void*)dst);
  asm volatile("s_add_u32 m0, %2, %3\n\tbuffer_load_dwordx4 %0, %1, %4 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds), "i"(OFS), "s"(soff)
               : "memory", "scc");   // s_add_u32 writes SCC
}
// Compiler-only fence: keeps LDS reads and writes on their side of a barrier without
// emitting the memory-model waits of __syncthreads (which would drain the ring).
#define SWG_COMPILER_FENCE() asm volatile("" ::: "memory")

// consecutive logical tiles -> same XCD
__device__ inline int64_t xcd_remap(int64_t b, int64_t nblocks) {
  const int64_t per = nblocks / 8;
  if (b >= per * 8) return b;
  return (b % 8) * per + b / 8;
}

template <int F>
__device__ inline void zero_acc(f32x16 (&acc)[F][F]) {
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// MFMA 32x32x16 layout: lane l supplies row (l % 32) and contraction elements
// 8 (l / 32) .. 8 (l / 32) + 7 of each operand; accumulator register r of lane l holds
// row 8 (r / 4) + 4 (l / 32) + (r % 4), column l % 32.

// ------------------------------------------------------------------ 32-deep row tiles
// (the forward's x operand) Slot layout: [256 rows][32]; a row is 4 chunks of 16 B.
// Chunk c of row r sits at position c ^ xsw(r), xsw(r) = (r / 4) % 4: within 16
// consecutive rows (one group of 16 lanes of a 16-byte read) the four rows that share a
// 64-byte bank window take four different chunks (measured: full LDS read rate, no bank
// conflict cycles).
__device__ inline int xsw(int r) { return (r >> 2) & 3; }

// Scheduling hint for one pipeline step: the LDS reads of the next stage (READS of them)
// spread evenly between the MFMAS MFMAs of the current stage.  sched_group_barrier(mask, n,
// 0) asks the scheduler for n instructions of the class next (0x008 MFMA, 0x100 LDS read).
#define SWG_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
template <int MFMAS, int READS>
__device__ inline void step_schedule() {
  static_assert((MFMAS == 32 && READS == 16) || (MFMAS == 8 && READS == 8), "per step");
  // groups of (MFMAs, reads) that cover the step's MFMAs and reads evenly
  constexpr int kGroups = READS;
  constexpr int kMfma = MFMAS / kGroups, kReads = READS / kGroups;
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    SWG_SCHED(0x008, kMfma);
    SWG_SCHED(0x100, kReads);
  }
}

// Operand fragments of one stage, per wave: [contraction half][block]; FragSet[2] holds
// the stage being multiplied and the stage being read.
template <typename T, int F = 4> struct FragSet {
  typename Mfma<T>::frag a[2][F], b[2][F];
};

// x-stage LDS: both operands move 64 contraction elements (128-byte row segments) per
// load, into "double stages" (pipeline stage 2d + h is half h of double stage d).  A ring
// (dg | dfc, streamed from HBM): three slots of [P rows][64]; B ring (W, resident in L2):
// two slots of [P rows][64]; 160 KiB in all at P = 256.  A row is 8 chunks of 16 B, chunk
// c of row r at position c ^ xsw8(r): within 16 consecutive rows the pairs of rows that
// share a 256-byte bank window take different chunks.
__device__ inline int xsw8(int r) { return (r >> 1) & 7; }

// Fragments of one pipeline stage: half HALF of an A slot and of a B slot.
template <typename T, int F, int HALF>
__device__ inline void x_read(const uint16_t* aslot, const uint16_t* bslot, int wp, int wq,
                              int lane, FragSet<T, F>& f) {
  using Fr = typename Mfma<T>::frag;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int lc = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < F; ++i) {
      const int r = wp * Tc<F>::WR + i * 32 + (lane & 31);
      f.a[kk][i] = *reinterpret_cast<const Fr*>(aslot + r * XA_BR + (((4 * HALF + lc) ^ xsw8(r)) << 3));
    }
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const int r = wq * Tc<F>::WR + j * 32 + (lane & 31);
      f.b[kk][j] = *reinterpret_cast<const Fr*>(bslot + r * XA_BR + (((4 * HALF + lc) ^ xsw8(r)) << 3));
    }
  }
}

// ------------------------------------------------------------------ w-stage tiles
// Slot layout: [32 contraction rows of A][P] then [32 rows of B][P]; a row is P / 8
// chunks of 16 B (32 or 16), chunk c of row m at position c ^ wsw(m).  A transposing read
// covers 4 rows x 32 bytes per 16 lanes (64 bytes for 32 lanes); wsw spreads them over
// distinct banks (rows are a multiple of 256 bytes apart at either P).
__device__ inline int wsw(int m) {
  const int t = m & 3;
  return t == 0 ? 0 : t == 1 ? 6 : t == 2 ? 12 : 10;
}

// ds_read_b64_tr_b16: within each 16-lane group, lane s supplies 4 consecutive 16-bit
// elements E[s][0..3]; lane i receives E[4 j + i / 4][i % 4] for j = 0..3.  With lane s
// pointing at row m0 + s / 4, column c0 + 4 (s % 4), lane i gets column c0 + i of rows
// m0 .. m0 + 3: four consecutive contraction elements of one operand row.
__device__ inline i16x4 tr_read(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p);
}

// Per-lane part of the transposing-read address of operand block i (rows 32 i .. of the
// wave's WR), in elements, for contraction rows 0..3 of a 16-row step, in a [k][P] tile
// whose wave part starts at chunk wchunk:
//   lane = 16 grp + s:  row 8 (grp / 2) + s / 4, column 32 i + 16 (grp % 2) + 4 (s % 4)
// with the column's chunk swizzled by wsw(row) (row % 4 = s / 4: the swizzle does not
// depend on the step, so every other term is a compile-time offset).
template <int F, int P>
__device__ inline void w_lane_offsets(int lane, int wchunk, int (&off)[F]) {
  const int grp = lane >> 4, s = lane & 15;
  const int q = 2 * (grp & 1) + ((s & 3) >> 1);    // chunk inside the 32-column block
  const int sw = wsw(s >> 2);
  const int row = 8 * (grp >> 1) + (s >> 2);
#pragma unroll
  for (int i = 0; i < F; ++i)
    off[i] = row * P + (((wchunk + 4 * i + q) ^ sw) << 3) + 4 * (s & 1);
}

// Transposing-read fragment of 16 contraction rows from a [k][RL] tile: p is this lane's
// address for contraction rows 0..3; rows 4..7 are 4 rows further.
template <typename T, int RL>
__device__ inline typename Mfma<T>::frag tr_frag(const uint16_t* p) {
  const i16x4 lo = tr_read(p);
  const i16x4 hi = tr_read(p + 4 * RL);
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename Mfma<T>::frag, v);
}

template <typename T, int F>
__device__ inline void w_read(const uint16_t* slot, const int (&aoff)[F], const int (&boff)[F],
                              FragSet<T, F>& f) {
  constexpr int P = Tc<F>::P;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int i = 0; i < F; ++i) f.a[ks][i] = tr_frag<T, P>(slot + 16 * ks * P + aoff[i]);
#pragma unroll
    for (int j = 0; j < F; ++j) f.b[ks][j] = tr_frag<T, P>(slot + BR * P + 16 * ks * P + boff[j]);
  }
}

// The 2 F^2 MFMAs of one stage.
template <typename T, int F>
__device__ inline void stage_mma(const FragSet<T, F>& f, f32x16 (&acc)[F][F]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int j = 0; j < F; ++j) acc[i][j] = Mfma<T>::mma(f.a[kk][i], f.b[kk][j], acc[i][j]);
}

// Swap a value with the neighbouring lane (lane ^ 1): DPP quad_perm [1, 0, 3, 2].
__device__ inline float swap_adjacent(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// Two adjacent columns of one row, rounded to T (nearest even) and packed in 32 bits.
template <typename T> __device__ inline uint32_t pack2(float lo, float hi);
template <> __device__ inline uint32_t pack2<bf16>(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
template <> __device__ inline uint32_t pack2<fp16>(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}
template <typename T> __device__ inline float2 unpack2(uint32_t v);
template <> __device__ inline float2 unpack2<bf16>(uint32_t v) {
  return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}
template <> __device__ inline float2 unpack2<fp16>(uint32_t v) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 h = __builtin_bit_cast(f16x2, v);
  return make_float2((float)h[0], (float)h[1]);
}

// Row pairs of adjacent columns: accumulator registers r and r + 1 of a 32 x 32 tile are
// rows R and R + 1 of one column; after a swap with the neighbouring lane, even lanes hold
// (row R, columns c, c + 1) and odd lanes (row R + 1, columns c - 1, c), so that each lane
// writes two adjacent columns of one row (the read-add-write and partial stores below).

// dW[row, col] += accumulators of block row I (32 rows of the wave's WR), for a tile
// without an M split.  `r` is a buffer window over the wave's valid dW rows (rows past K
// are dropped by the range check); columns past N are pushed out of the window
// (cols_left: columns left from the wave's first).  The old values of all of the block's
// pairs are loaded before any of them is stored: the compiler cannot move a load of dW
// above a store to dW, so a load-add-store per pair would cost one memory round trip each
// (128 per wave at F = 4); batched, the wave makes F.  Offsets are 32-bit (128 rows of
// < 2^23 bytes).
template <typename T, int F, int I>
__device__ inline void rmw_block_rows(const f32x16 (&acc)[F][F], int lane,
                                      __amdgpu_buffer_rsrc_t r, uint32_t row_bytes,
                                      int cols_left) {
  const int odd = lane & 1;
  const uint32_t loff = (uint32_t)(4 * (lane >> 5) + odd) * row_bytes +
                        (uint32_t)((lane & 31) & ~1) * 2u;
  uint32_t voff[F][8], old[F][8];
#pragma unroll
  for (int j = 0; j < F; ++j) {
    const uint32_t cbad = j * 32 + ((lane & 31) & ~1) < cols_left ? 0u : kOOB;
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2) {
      const int rr = 2 * r2;
      voff[j][r2] = (loff + (uint32_t)(I * 32 + 8 * (rr >> 2) + (rr & 3)) * row_bytes +
                     64u * j) | cbad;
      old[j][r2] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff[j][r2], 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < F; ++j)
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2) {
      const int rr = 2 * r2;
      const float v0 = acc[I][j][rr], v1 = acc[I][j][rr + 1];
      const float recv = swap_adjacent(odd ? v0 : v1);
      const float lo = odd ? recv : v0, hi = odd ? v1 : recv;
      const float2 o = unpack2<T>(old[j][r2]);
      __builtin_amdgcn_raw_buffer_store_b32(pack2<T>(o.x + lo, o.y + hi), r, (int)voff[j][r2],
                                            0, 0);
    }
}

// fp32 partials of block row I (32 rows of the wave's WR) straight from the accumulators:
// after the swap with the neighbouring lane (row pairs above) each lane writes two
// adjacent columns of one row, 8 bytes.  `r` is a buffer window over the block's valid
// rows only, so rows past K are dropped by the range check, and so are columns past N,
// whose offsets are pushed out of the window (cols_left: columns left from the wave's
// first) - no branch per store.  row_bytes = 8 N < 2^25 and 32 rows keep every offset
// below 2^30.
template <int F, int I>
__device__ inline void store_partial_block(const f32x16 (&acc)[F][F], int lane,
                                           __amdgpu_buffer_rsrc_t r, uint32_t row_bytes,
                                           int cols_left) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const int odd = lane & 1;
  const uint32_t loff = (uint32_t)(4 * (lane >> 5) + odd) * row_bytes +
                        (uint32_t)((lane & 31) & ~1) * 4u;
#pragma unroll
  for (int j = 0; j < F; ++j) {
    const uint32_t cbad = j * 32 + ((lane & 31) & ~1) < cols_left ? 0u : kOOB;
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2) {
      const int rr = 2 * r2;
      const float v0 = acc[I][j][rr], v1 = acc[I][j][rr + 1];
      const float recv = swap_adjacent(odd ? v0 : v1);
      const float lo = odd ? recv : v0, hi = odd ? v1 : recv;
      const uint32_t voff =
          (loff + (uint32_t)(8 * (rr >> 2) + (rr & 3)) * row_bytes + 128u * j) | cbad;
      const u32x2 v = {__float_as_uint(lo), __float_as_uint(hi)};
      __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, 0, 0);
    }
  }
}

// Tile store straight from the accumulators: every lane pair turns its two rows x two
// columns into one row each (pack to 16 bits, swap the packed words with the neighbouring
// lane, byte-permute: even lanes keep row R, odd lanes row R + 1) and writes 32 bits per
// row.  `r` is a buffer window over the tile's valid rows only, so stores to rows past the
// output are dropped by the hardware range check, and so are stores to columns past the
// output's right edge, whose offsets are pushed out of the window (cols_left: columns left
// from the tile's first; a multiple of 8, so a pair never straddles it).  wrow0 / wcol0:
// the wave's first row / column inside the tile.  All offsets are 32-bit (256 rows x 2^23
// bytes < 2^31).
template <typename T, int F>
__device__ inline void store_tile_rows(const f32x16 (&acc)[F][F], int lane,
                                       __amdgpu_buffer_rsrc_t r, uint32_t row_bytes, int wrow0,
                                       int wcol0, int cols_left) {
  const int odd = lane & 1;
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;   // odd: (nb.hi, own.hi)
  uint32_t loff = (uint32_t)(4 * (lane >> 5) + odd) * row_bytes +
                  (uint32_t)(wcol0 + ((lane & 31) & ~1)) * 2u;
  asm volatile("" : "+v"(loff));   // keeps the 32 row offsets below from being hoisted out of
                                   // the tile loop (they would stay live, and spill)
  // columns past the tensor's edge: the offset is pushed past the window and the store is
  // dropped by the range check (no branch per store)
  uint32_t cbad[F];
#pragma unroll
  for (int j = 0; j < F; ++j) {
    cbad[j] = wcol0 + j * 32 + ((lane & 31) & ~1) < cols_left ? 0u : kOOB;
    asm volatile("" : "+v"(cbad[j]));   // formed here, not hoisted (see loff)
  }
  asm volatile("" : "+s"(row_bytes));  // the row offsets below likewise
  // An always-true wave-uniform test the compiler cannot fold: each row pair's stores sit
  // in a block of their own, so the accumulators are copied out a few at a time (in
  // straight-line code the copies of all 256 are hoisted together, and spill).
  int go = 1;
  asm volatile("" : "+s"(go));
#pragma unroll
  for (int i = 0; i < F; ++i) {
#pragma unroll
    for (int rr = 0; rr < 16; rr += 2) {
      asm volatile("" : "+s"(go));   // a fresh value per block (no threading of the tests)
      if (go) {
        const uint32_t voff =
            loff + (uint32_t)(wrow0 + i * 32 + 8 * (rr >> 2) + (rr & 3)) * row_bytes;
#pragma unroll
        for (int j = 0; j < F; ++j) {
          const uint32_t own = pack2<T>(acc[i][j][rr], acc[i][j][rr + 1]);
          const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, false);
          const uint32_t out = __builtin_amdgcn_perm(nb, own, sel);
          __builtin_amdgcn_raw_buffer_store_b32(out, r, (int)((voff | cbad[j]) + 64u * j), 0, 0);
        }
      }
    }
  }
}

// ----------------------------------------------------------------- x stage (NT)
// A = [dg | dfc] rows p (M), B = [W_g | W_fc] rows q (K).  Double stage d < sD contracts
// over columns 64 d .. of dg / W_g, d >= sD over the same columns of dfc / W_fc
// (sD = max(2, ceil(N / 64)); columns past N read zeros).  Tile L covers rows (L / nq) * P
// and columns (L % nq) * P (P = 256 or 128).
//
// Two steps per double stage d (stages t = 2d, 2d + 1):
//   even t: read stage t + 1 (the second halves of the A and B slots of double stage d,
//           which landed with the first) into the other register set while the MFMAs run
//           on stage t; no wait, no barrier, no load;
//   odd t:  wait until this wave's loads of double stage d + 1 landed and its own LDS
//           reads are done; barrier (every wave's loads landed; every wave finished reading
//           both slots of double stage d); then, spread between the MFMAs of stage t, issue
//           B double stage d + 2 into the B slot and A double stage d + 3 into the A slot of
//           double stage d, and read stage t + 1 (first halves of double stage d + 1).
// Every wave issues 8 B then 8 A loads per odd step, so "double stage d + 1 landed" is "at
// most 8 loads outstanding" (only A of d + 3 was issued after B of d + 1); the prologue
// issues in the same order (A0 B0 A1 B1 A2).  Issues past the tile's last double stage
// fetch the next tile's first ones (uniform selects, no branch).
//
// Issue cost: a load's address is window base + soffset + voffset.  The window (the
// operand panel of a tile, dg or dfc half) is formed once per tile; the column of the
// double stage goes into the scalar soffset; the per-lane voffset (row and swizzled chunk)
// is fixed.  The hardware range check applies to voffset only, against the window's rows,
// so rows past the end still read zeros.  Only when some double stage reaches past N
// (N not a multiple of 64, or N = 64) does a per-lane column test remain (template
// RAGGED).
struct XTile {   // first row of the dg/dfc panel and of the W panel; 32-bit (M < 2^31)
  int p0, q0;
  bool live;
};

template <int F>
__device__ inline XTile x_tile(int64_t L, bool live, int64_t nq) {
  XTile c;
  c.live = live;
  const int64_t LL = live ? L : 0;
  c.p0 = (int)(LL / nq) * Tc<F>::P;
  c.q0 = (int)(LL % nq) * Tc<F>::P;
  return c;
}

// 64-bit pointer pinned to scalar registers (a buffer resource must be wave-uniform)
template <typename P>
__device__ inline P* uniform_ptr(P* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Operand windows of one tile: the dg and dfc row panels and the W_g and W_fc row panels,
// each with its valid byte count (0 for a tile that does not exist: every load reads 0).
struct XWin {
  int64_t a_off, b_off;        // element offsets of the panels (p0 N, q0 N)
  uint32_t a_bytes, b_bytes;
};

template <int F>
__device__ inline XWin x_win(const XTile& c, int64_t M, int64_t K, int64_t N) {
  XWin w;
  constexpr int P = Tc<F>::P;
  const int64_t ra = c.live ? (M - c.p0 < P ? M - c.p0 : P) : 0;
  const int64_t rb = c.live ? (K - c.q0 < P ? K - c.q0 : P) : 0;
  w.a_off = (int64_t)c.p0 * N;
  w.b_off = (int64_t)c.q0 * N;
  w.a_bytes = (uint32_t)(ra * N * 2);
  w.b_bytes = (uint32_t)(rb * N * 2);
  return w;
}

// One issue: window, soffset (column of the double stage, bytes) and LDS destination.
struct XIssue {
  __amdgpu_buffer_rsrc_t r;
  uint32_t soff;
  int lim;                 // columns left in the half from this double stage on
  const uint16_t* dst;
};

// Double stage d of operand A (IS_A) or B of the current tile (d >= nds: double stage
// d - nds of the next tile).
template <typename T>
__device__ inline XIssue x_issue(const T* lo, const T* hi_arr, XWin wc, XWin wn, bool is_a, int d,
                                 int nds, int sD, int64_t N, uint16_t* slot) {
  const bool nx = d >= nds;
  const int dd = nx ? d - nds : d;
  const bool hi = dd >= sD;
  const int col = (hi ? dd - sD : dd) * XA_BR;
  const int64_t off = is_a ? (nx ? wn.a_off : wc.a_off) : (nx ? wn.b_off : wc.b_off);
  const uint32_t bytes = is_a ? (nx ? wn.a_bytes : wc.a_bytes) : (nx ? wn.b_bytes : wc.b_bytes);
  XIssue is;
  is.r = make_rsrc(uniform_ptr((hi ? hi_arr : lo) + off), __builtin_amdgcn_readfirstlane(bytes));
  is.soff = __builtin_amdgcn_readfirstlane((uint32_t)col * 2u);
  is.lim = (int)N - col;
  is.dst = slot;
  return is;
}

// This lane's voffset for load i (0 .. 2F - 1) of an issue.
template <bool RAGGED, int L>
__device__ inline uint32_t x_voff(const XIssue& is, const uint32_t (&aoff)[L], const int (&acol)[2],
                                  int i) {
  if (!RAGGED) return aoff[i];
  return acol[i & 1] < is.lim ? aoff[i] : kOOB;
}

template <bool RAGGED, int L, int... I>
__device__ inline void x_issue_loads(std::integer_sequence<int, I...>, const XIssue& is,
                                     const uint32_t (&aoff)[L], const int (&acol)[2]) {
  (dma16s<I * 1024>(is.r, x_voff<RAGGED>(is, aoff, acol, I), is.soff, is.dst), ...);
}

template <bool RAGGED, int L>
__device__ inline void x_issue_all(const XIssue& is, const uint32_t (&aoff)[L],
                                   const int (&acol)[2]) {
  x_issue_loads<RAGGED>(std::make_integer_sequence<int, L>{}, is, aoff, acol);
}

// Fragment G (0 .. 4F - 1, in x_read's order: kk = G / 2F; G % 2F < F: A block G % 2F,
// else B block G % 2F - F) of stage half HALF.
template <typename T, int F, int HALF, int G>
__device__ inline void x_read_one(const uint16_t* aslot, const uint16_t* bslot, int wp, int wq,
                                  int lane, FragSet<T, F>& f) {
  using Fr = typename Mfma<T>::frag;
  constexpr int kk = G / (2 * F), idx = G % (2 * F);
  const int lc = 2 * kk + (lane >> 5);
  if constexpr (idx < F) {
    const int r = wp * Tc<F>::WR + idx * 32 + (lane & 31);
    f.a[kk][idx] = *reinterpret_cast<const Fr*>(aslot + r * XA_BR + (((4 * HALF + lc) ^ xsw8(r)) << 3));
  } else {
    const int r = wq * Tc<F>::WR + (idx - F) * 32 + (lane & 31);
    f.b[kk][idx - F] = *reinterpret_cast<const Fr*>(bslot + r * XA_BR + (((4 * HALF + lc) ^ xsw8(r)) << 3));
  }
}

// MFMA q (stage_mma's order) of the stage in f.
template <typename T, int F, int Q>
__device__ inline void mma_q(f32x16 (&acc)[F][F], const FragSet<T, F>& f) {
  constexpr int kk = Q / (F * F), i = (Q / F) % F, j = Q % F;
  acc[i][j] = Mfma<T>::mma(f.a[kk][i], f.b[kk][j], acc[i][j]);
}

// Group G (0 .. 4F - 1) of an odd step: MFMAs F/2 G .. F/2 G + F/2 - 1 of the stage in f
// (stage_mma's order), fragment G of the next stage (READ_NEXT), and load G % 2F of the B
// issue (G < 2F) or of the A issue.  The scheduling fence keeps the groups in this order,
// so that the 4F loads and the address work around them are spread over the step instead
// of stalling the matrix cores behind the barrier.
template <typename T, int F, bool RAGGED, bool READ_NEXT, int G>
__device__ inline void x_odd_group(f32x16 (&acc)[F][F], const FragSet<T, F>& f,
                                   FragSet<T, F>& fn, const uint16_t* aslot,
                                   const uint16_t* bslot, int wp, int wq, int lane,
                                   const XIssue& is, const uint32_t (&aoff)[2 * F],
                                   const int (&acol)[2]) {
  mma_q<T, F, G * (F / 2)>(acc, f);
  if constexpr (F == 4) mma_q<T, F, G * (F / 2) + 1>(acc, f);
  if (READ_NEXT) x_read_one<T, F, 0, G>(aslot, bslot, wp, wq, lane, fn);
  constexpr int e = G % (2 * F);
  dma16s<e * 1024>(is.r, x_voff<RAGGED>(is, aoff, acol, e), is.soff, is.dst);
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T, int F, bool RAGGED, bool READ_NEXT, int OFS, int... G>
__device__ inline void x_odd_groups(std::integer_sequence<int, G...>, f32x16 (&acc)[F][F],
                                    const FragSet<T, F>& f, FragSet<T, F>& fn,
                                    const uint16_t* aslot, const uint16_t* bslot, int wp, int wq,
                                    int lane, const XIssue& is, const uint32_t (&aoff)[2 * F],
                                    const int (&acol)[2]) {
  (x_odd_group<T, F, RAGGED, READ_NEXT, OFS + G>(acc, f, fn, aslot, bslot, wp, wq, lane, is,
                                                 aoff, acol),
   ...);
}

// The x-stage tile walk of one workgroup: tiles f0, f0 + G, f0 + 2G, ... of the ntiles
// output tiles, through the LDS ring at `ring` (3 A slots then 2 B slots).
template <typename T, int F, bool RAGGED>
__device__ __attribute__((always_inline)) inline void x_tiles(
    uint16_t* ring, const T* __restrict__ dg, const T* __restrict__ dfc,
    const T* __restrict__ wg, const T* __restrict__ wfc, T* __restrict__ dx, int64_t M,
    int64_t K, int64_t N, int64_t nq, int64_t ntiles, int64_t f0, int64_t G) {
  constexpr int P = Tc<F>::P, XSLOT = Tc<F>::XSLOT, XLOADS = Tc<F>::XLOADS;
  uint16_t* const ra0 = ring;
  uint16_t* const rb0 = ring + 3 * XSLOT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave / WQ, wq = wave % WQ;
  const int64_t my_tiles = ntiles > f0 ? (ntiles - f0 + G - 1) / G : 0;
  // double stages per dg (or dfc) half, at least 2 so that a tile has at least 4: the A
  // loads run up to three double stages ahead and must stay within the next tile
  int sD = (int)((N + XA_BR - 1) / XA_BR);
  if (sD < 2) sD = 2;
  const int nds = 2 * sD;                          // double stages per tile (even, >= 4)

  // A and B alike: a 1 KiB load covers 8 rows x 8 chunks, rows P / 4 wave + 8 i + lane / 8
  // (i = 0 .. 2F - 1); the lane fetches the logical chunk that its LDS position holds under
  // the swizzle.  xsw8(P / 4 wave + 8 i + lane / 8) = (4 i + lane / 16) % 8, so the column
  // term takes two values per lane; dg, dfc, W_g and W_fc all have rows of N elements, so
  // the offsets serve both operands.
  uint32_t aoff[XLOADS];
  int acol[2];
  acol[0] = ((lane & 7) ^ ((lane >> 4) & 7)) * 8;
  acol[1] = ((lane & 7) ^ ((4 + (lane >> 4)) & 7)) * 8;
#pragma unroll
  for (int i = 0; i < XLOADS; ++i) {
    const int row = (P / 4) * wave + 8 * i + (lane >> 3);
    aoff[i] = (uint32_t)row * (uint32_t)(N * 2) + (uint32_t)acol[i & 1] * 2u;
  }
  const int wofs = (P / 4) * wave * XA_BR;   // this wave's rows in a slot
  auto issue_a = [&](XWin wc, XWin wn, int d, uint16_t* slot) {
    asm volatile("" : "+s"(d));   // keep per-stage values from being hoisted (they would
                                  // stay live across the tile loop, and spill)
    return x_issue<T>(dg, dfc, wc, wn, true, d, nds, sD, N, slot + wofs);
  };
  auto issue_b = [&](XWin wc, XWin wn, int d, uint16_t* slot) {
    asm volatile("" : "+s"(d));
    return x_issue<T>(wg, wfc, wc, wn, false, d, nds, sD, N, slot + wofs);
  };
#define X_READ(h, as, bs, f) x_read<T, F, (h)>((as), (bs), wp, wq, lane, (f))
  // even step: second halves of the current double stage
#define X_STEP_EVEN()                                                                     \
  do {                                                                                    \
    X_READ(1, ra0 + as * XSLOT, rb0 + bs * XSLOT, frags[1]);                               \
    stage_mma<T, F>(frags[0], acc);                                                       \
    step_schedule<2 * F * F, 4 * F>();                                                    \
  } while (0)
  // odd step t = 2d + 1 (d = t0 / 2 + (u - 1) / 2); READ_NEXT = 0 on the last step of a tile
#define X_STEP_ODD(d, READ_NEXT)                                                           \
  do {                                                                                    \
    __builtin_amdgcn_s_waitcnt(vmcnt_le(XLOADS));                                         \
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);                                                \
    SWG_COMPILER_FENCE();                                                                 \
    __builtin_amdgcn_s_barrier();                                                         \
    SWG_COMPILER_FENCE();                                                                 \
    uint16_t* const bfree_ = rb0 + bs * XSLOT;                                            \
    uint16_t* const afree_ = ra0 + as * XSLOT;                                            \
    as = (as == 2 ? 0 : as + 1);                                                          \
    bs ^= 1;                                                                              \
    const XIssue ib_ = issue_b(wc, wn, (d) + 2, bfree_);                                   \
    x_odd_groups<T, F, RAGGED, (READ_NEXT), 0>(std::make_integer_sequence<int, 2 * F>{},   \
                                               acc, frags[1], frags[0], ra0 + as * XSLOT,  \
                                               rb0 + bs * XSLOT, wp, wq, lane, ib_, aoff,  \
                                               acol);                                     \
    const XIssue ia_ = issue_a(wc, wn, (d) + 3, afree_);                                   \
    x_odd_groups<T, F, RAGGED, (READ_NEXT), 2 * F>(std::make_integer_sequence<int, 2 * F>{}, \
                                                   acc, frags[1], frags[0],                \
                                                   ra0 + as * XSLOT, rb0 + bs * XSLOT, wp, \
                                                   wq, lane, ia_, aoff, acol);            \
  } while (0)

  f32x16 acc[F][F];
  FragSet<T, F> frags[2];
  XTile nxt = x_tile<F>(f0 + G, my_tiles > 1, nq);
  XWin wc = x_win<F>(x_tile<F>(f0, my_tiles > 0, nq), M, K, N);
  XWin wn = x_win<F>(nxt, M, K, N);
  int as = 0, bs = 0;   // A and B slots of the double stage holding the current stage
  // prologue, in the steady-state issue order: A0 B0 A1 B1 A2
  x_issue_all<RAGGED>(issue_a(wc, wn, 0, ra0), aoff, acol);
  x_issue_all<RAGGED>(issue_b(wc, wn, 0, rb0), aoff, acol);
  x_issue_all<RAGGED>(issue_a(wc, wn, 1, ra0 + XSLOT), aoff, acol);
  x_issue_all<RAGGED>(issue_b(wc, wn, 1, rb0 + XSLOT), aoff, acol);
  x_issue_all<RAGGED>(issue_a(wc, wn, 2, ra0 + 2 * XSLOT), aoff, acol);
  __builtin_amdgcn_s_waitcnt(vmcnt_le(3 * XLOADS));   // A0 and B0 landed
  SWG_COMPILER_FENCE();
  __builtin_amdgcn_s_barrier();
  SWG_COMPILER_FENCE();
  for (int64_t j = 0; j < my_tiles; ++j) {
    const XTile cur = x_tile<F>(f0 + j * G, true, nq);
    if (j > 0) {
      nxt = x_tile<F>(f0 + (j + 1) * G, j + 1 < my_tiles, nq);
      wc = wn;
      wn = x_win<F>(nxt, M, K, N);
    }
    __builtin_amdgcn_sched_barrier(0);   // the epilogue stays ahead of the next reads
    zero_acc(acc);
    X_READ(0, ra0 + as * XSLOT, rb0 + bs * XSLOT, frags[0]);   // stage 0
    int d0 = 0;
    for (; d0 + 2 < nds; d0 += 2) {
      X_STEP_EVEN();
      X_STEP_ODD(d0, true);
      X_STEP_EVEN();
      X_STEP_ODD(d0 + 1, true);
    }
    X_STEP_EVEN();
    X_STEP_ODD(d0, true);
    X_STEP_EVEN();
    X_STEP_ODD(d0 + 1, false);
    // epilogue: straight from the accumulators, two adjacent columns per 32-bit store
    {
      const int rows = (int)M - cur.p0 < P ? (int)M - cur.p0 : P;
      store_tile_rows<T, F>(acc, lane,
                            make_rsrc(dx + (int64_t)cur.p0 * K + cur.q0, clamp_bytes(rows, K * 2)),
                            (uint32_t)(K * 2), wp * Tc<F>::WR, wq * Tc<F>::WR, (int)K - cur.q0);
    }
  }
#undef X_STEP_EVEN
#undef X_STEP_ODD
#undef X_READ
  __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
}

template <typename T, int F, bool RAGGED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(Tc<F>::XOCC, Tc<F>::XOCC))) void x_stage_kernel(
    const T* __restrict__ dg, const T* __restrict__ dfc, const T* __restrict__ wg,
    const T* __restrict__ wfc, T* __restrict__ dx, int64_t M, int64_t K, int64_t N, int64_t nq,
    int64_t ntiles) {
  __shared__ __attribute__((aligned(1024))) uint16_t ring[Tc<F>::X_RING];
  const int64_t G = gridDim.x;
  x_tiles<T, F, RAGGED>(ring, dg, dfc, wg, wfc, dx, M, K, N, nq, ntiles,
                        xcd_remap(blockIdx.x, G), G);
}

// ----------------------------------------------------------------- w stage (TN)
// A = x^T: rows k (K), contraction m;  B = d^T (d = dg or dfc): rows n, contraction m.
// Work item L = (split s, tile tt): output rows k0 = (tt / (2 tnh)) * P, columns n0 of
// dg (tt % (2 tnh) < tnh) or of dfc, contracting over the rows of split s.  A split's rows
// are either one range [s R, min(M, (s + 1) R)) (the w stage) or chunks of CH rows taken
// every S chunks: chunk j of split s covers rows (s + j S) CH .. (the fused pass, whose
// x-stage workgroups sweep the same rows at the same time).  Stage st (BR rows) starts at
//   m_begin + (st >> cs_log2) * stride + (st & (2^cs_log2 - 1)) * BR
// with cs_log2 = log2(CH / BR) and stride = S CH for chunks, cs_log2 = 30 for one range.
struct WItem {   // 32-bit fields: M < 2^31 and K, N < 2^22 are checked on the host
  int s, k0, n0, m_begin, m_end, nst, stride, cs_log2;
  bool hi, live;
};

struct WMap {          // how items map to rows (see WItem)
  int64_t split_rows;  // R (one range per split), or 0 for chunked splits
  int64_t chunk_rows;  // CH (chunked splits; a power of two times BR)
  int64_t nsplit;      // S
};

template <int F>
__device__ inline WItem w_item(int64_t L, bool live, int64_t tiles, int64_t tnh,
                               const WMap& mp, int64_t M) {
  WItem w;
  w.live = live;
  const int64_t LL = live ? L : 0;
  w.s = (int)(LL / tiles);
  const int tt = (int)(LL % tiles);
  const int kb = tt / (int)(2 * tnh), nb = tt % (int)(2 * tnh);
  w.hi = nb >= tnh;
  w.k0 = kb * Tc<F>::P;
  w.n0 = (w.hi ? nb - (int)tnh : nb) * Tc<F>::P;
  if (mp.split_rows > 0) {
    w.m_begin = w.s * (int)mp.split_rows;
    w.m_end = (w.m_begin + mp.split_rows < M) ? w.m_begin + (int)mp.split_rows : (int)M;
    w.stride = 0;
    w.cs_log2 = 30;
    w.nst = 4 * ((w.m_end - w.m_begin + 4 * BR - 1) / (4 * BR));   // whole ring rounds
  } else {
    const int ch = (int)mp.chunk_rows;
    const int chunks = (int)((M + ch - 1) / ch);
    const int mine = chunks > w.s ? (chunks - w.s + (int)mp.nsplit - 1) / (int)mp.nsplit : 0;
    w.m_begin = w.s * ch;
    w.m_end = (int)M;
    w.stride = (int)mp.nsplit * ch;
    w.cs_log2 = 31 - __builtin_clz((unsigned)(ch / BR));
    w.nst = (ch / BR) * mine;                 // a multiple of 4: CH is at least 4 stages
    // wave-uniform values computed through divisions: pinned to scalar registers, since
    // they address buffer windows (scalar operands)
    w.m_begin = __builtin_amdgcn_readfirstlane(w.m_begin);
    w.stride = __builtin_amdgcn_readfirstlane(w.stride);
    w.cs_log2 = __builtin_amdgcn_readfirstlane(w.cs_log2);
    w.nst = __builtin_amdgcn_readfirstlane(w.nst);
  }
  if (w.nst < 4) w.nst = 4;                   // one ring round at least (zeros past the end)
  return w;
}

// One w-stage issue: the stage's row windows of x and of dg (or dfc), the tile's first
// columns as scalar soffsets (bytes) and the columns left in the tile (ragged edges only).
struct WIssue {
  __amdgpu_buffer_rsrc_t rx, rd;
  uint32_t sx, sd;
  int kleft, nleft;
  const uint16_t* dst;
};

// Load e (0 .. 2F - 1) of a w-stage issue: e < F fetches rows of x, e >= F rows of
// dg / dfc; each load is 1 KiB of the wave's part of the slot.
template <bool RAGGED, int F, int E>
__device__ inline void w_dma(const WIssue& is, const uint32_t (&xbase)[F],
                             const uint32_t (&dbase)[F], const int (&lcol)[F]) {
  constexpr int i = E % F;
  if (E < F) {
    const uint32_t v = !RAGGED || lcol[i] < is.kleft ? xbase[i] : kOOB;
    dma16s<i * 1024>(is.rx, v, is.sx, is.dst);
  } else {
    const uint32_t v = !RAGGED || lcol[i] < is.nleft ? dbase[i] : kOOB;
    dma16s<BR * Tc<F>::P * 2 + i * 1024>(is.rd, v, is.sd, is.dst);
  }
}

template <bool RAGGED, int F, int... E>
__device__ inline void w_issue_loads(std::integer_sequence<int, E...>, const WIssue& is,
                                     const uint32_t (&xbase)[F], const uint32_t (&dbase)[F],
                                     const int (&lcol)[F]) {
  (w_dma<RAGGED, F, E>(is, xbase, dbase, lcol), ...);
}

template <bool RAGGED, int F>
__device__ inline void w_issue_all(const WIssue& is, const uint32_t (&xbase)[F],
                                   const uint32_t (&dbase)[F], const int (&lcol)[F]) {
  w_issue_loads<RAGGED, F>(std::make_integer_sequence<int, 2 * F>{}, is, xbase, dbase, lcol);
}

// Fragment G (0 .. 4F - 1, w_read's order) of a w-stage slot.
template <typename T, int F, int G>
__device__ inline void w_read_one(const uint16_t* slot, const int (&aoff)[F],
                                  const int (&boff)[F], FragSet<T, F>& f) {
  constexpr int P = Tc<F>::P;
  constexpr int ks = G / (2 * F), idx = G % (2 * F);
  if constexpr (idx < F) f.a[ks][idx] = tr_frag<T, P>(slot + 16 * ks * P + aoff[idx]);
  else f.b[ks][idx - F] = tr_frag<T, P>(slot + BR * P + 16 * ks * P + boff[idx - F]);
}

// Group G (0 .. 4F - 1) of a w step: MFMAs F/2 G .. F/2 G + F/2 - 1 of the stage in f,
// fragment G of the next stage (READ_NEXT) and, in odd groups, load G / 2 of the issue,
// kept in this order by the scheduling fence (see x_odd_group).
template <typename T, int F, bool RAGGED, bool READ_NEXT, int G>
__device__ inline void w_group(f32x16 (&acc)[F][F], const FragSet<T, F>& f, FragSet<T, F>& fn,
                               const uint16_t* next_slot, const int (&aoff)[F],
                               const int (&boff)[F], const WIssue& is,
                               const uint32_t (&xbase)[F], const uint32_t (&dbase)[F],
                               const int (&lcol)[F]) {
  mma_q<T, F, G * (F / 2)>(acc, f);
  if constexpr (F == 4) mma_q<T, F, G * (F / 2) + 1>(acc, f);
  if (READ_NEXT) w_read_one<T, F, G>(next_slot, aoff, boff, fn);
  if constexpr ((G & 1) != 0) w_dma<RAGGED, F, (G >> 1)>(is, xbase, dbase, lcol);
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T, int F, bool RAGGED, bool READ_NEXT, int... G>
__device__ inline void w_groups(std::integer_sequence<int, G...>, f32x16 (&acc)[F][F],
                                const FragSet<T, F>& f, FragSet<T, F>& fn,
                                const uint16_t* next_slot, const int (&aoff)[F],
                                const int (&boff)[F], const WIssue& is,
                                const uint32_t (&xbase)[F], const uint32_t (&dbase)[F],
                                const int (&lcol)[F]) {
  (w_group<T, F, RAGGED, READ_NEXT, G>(acc, f, fn, next_slot, aoff, boff, is, xbase, dbase,
                                       lcol),
   ...);
}

// The w-stage item walk of one workgroup: items f0, f0 + G, ... of the nitems items,
// through the LDS ring at `ring` (four slots).
template <typename T, int F, bool RAGGED>
__device__ __attribute__((always_inline)) inline void w_items(
    uint16_t* ring, const T* __restrict__ x, const T* __restrict__ dg,
    const T* __restrict__ dfc, T* __restrict__ dwg, T* __restrict__ dwfc,
    float* __restrict__ ws, int64_t M, int64_t K, int64_t N, int64_t tnh, int64_t tiles,
    const WMap& mp, int64_t nitems, int64_t f0, int64_t G) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave / WQ, wq = wave % WQ;
  const int64_t my_items = nitems > f0 ? (nitems - f0 + G - 1) / G : 0;
  constexpr int P = Tc<F>::P, WR = Tc<F>::WR, WSLOT = Tc<F>::WSLOT, WLOADS = Tc<F>::WLOADS;
  constexpr int RPL = Tc<F>::RPL, LPR = 64 / RPL;   // rows per load, lanes per row

  // A 1 KiB load covers RPL rows x P / 8 chunks; this wave's loads are rows 8 wave +
  // RPL i + lane / LPR (i = 0 .. F - 1) of A and of B, logical chunk (lane % LPR) ^
  // wsw(row).  The lane parts of the offsets are fixed; the tile adds k0 / n0 (uniform).
  // One buffer window per stage: rows m0 .. m0 + 32 (rows past m_end, and every row of a
  // dead item, read 0).
  uint32_t xbase[F], dbase[F];
  int lcol[F];
#pragma unroll
  for (int i = 0; i < F; ++i) {
    const int row = 8 * wave + RPL * i + lane / LPR;
    lcol[i] = ((lane % LPR) ^ wsw(row)) * 8;
    xbase[i] = (uint32_t)row * (uint32_t)(K * 2) + (uint32_t)lcol[i] * 2u;
    dbase[i] = (uint32_t)row * (uint32_t)(N * 2) + (uint32_t)lcol[i] * 2u;
  }
  auto issue = [&](const WItem& w, int64_t st, uint16_t* slot) {
    int m0 = w.m_begin + ((int)st >> w.cs_log2) * w.stride +
             ((int)st & ((1 << w.cs_log2) - 1)) * BR;
    asm volatile("" : "+s"(m0));   // keep per-stage offsets from being hoisted (see x stage)
    const int rows = w.live ? ((w.m_end - m0 < BR) ? w.m_end - m0 : BR) : 0;
    const int64_t mb = rows > 0 ? m0 : 0;
    const T* d = w.hi ? dfc : dg;
    WIssue is;
    is.rx = make_rsrc(uniform_ptr(x + mb * K), __builtin_amdgcn_readfirstlane(clamp_bytes(rows, K * 2)));
    is.rd = make_rsrc(uniform_ptr(d + mb * N), __builtin_amdgcn_readfirstlane(clamp_bytes(rows, N * 2)));
    is.sx = __builtin_amdgcn_readfirstlane((uint32_t)w.k0 * 2u);
    is.sd = __builtin_amdgcn_readfirstlane((uint32_t)w.n0 * 2u);
    is.kleft = (int)K - w.k0;   // columns left in the tile
    is.nleft = (int)N - w.n0;
    is.dst = slot + 8 * wave * P;   // this wave's 8 rows
    return is;
  };

  int aoff[F], boff[F];
  w_lane_offsets<F, P>(lane, wp * (WR / 8), aoff);
  w_lane_offsets<F, P>(lane, wq * (WR / 8), boff);
#define W_READ(slot, f) w_read<T, F>((slot), aoff, boff, (f))
  // One pipeline step u (0..3) of a ring round.  On entry the fragments of the stage in
  // slot u are in registers (set u % 2) and the three following stages are in flight.  The
  // step waits until this wave's loads of the stage in slot u + 1 have landed and its own
  // LDS reads are complete; the barrier then says that every wave's loads landed and that
  // every wave has finished reading slot u, which is refilled with the stage four ahead
  // (of the next item once the current one runs out).  The MFMAs of the current stage run
  // from registers while the next stage's fragments are read from LDS into the other set;
  // loads and reads are spread between the MFMAs (w_group).  Every issue is
  // WLOADS (2F) loads per wave, always issued (stages past the end of the work load
  // zeros), so "the stage in slot u + 1 has landed" is exactly "at most 2 stages of loads
  // outstanding".  The last step of an item reads nothing: the next item's first stage is
  // read after the epilogue, so that no operand fragments are live while the accumulators
  // are written out.
#define W_STEP(ctx, st, u, READ_NEXT)                                                       \
  do {                                                                                    \
    __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * WLOADS));                                     \
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);                                                \
    SWG_COMPILER_FENCE();                                                                 \
    __builtin_amdgcn_s_barrier();                                                         \
    SWG_COMPILER_FENCE();                                                                 \
    const WIssue is_ = issue((ctx), (st), ring + (u) * WSLOT);                             \
    w_groups<T, F, RAGGED, (READ_NEXT)>(std::make_integer_sequence<int, 4 * F>{}, acc,     \
                                        frags[(u) & 1], frags[((u) + 1) & 1],             \
                                        ring + (((u) + 1) & 3) * WSLOT, aoff, boff, is_,   \
                                        xbase, dbase, lcol);                              \
  } while (0)

  f32x16 acc[F][F];
  FragSet<T, F> frags[2];
  WItem cur = w_item<F>(f0, my_items > 0, tiles, tnh, mp, M);
  // prologue: the first four stages in flight, the first landed for every wave
  w_issue_all<RAGGED>(issue(cur, 0, ring), xbase, dbase, lcol);
  w_issue_all<RAGGED>(issue(cur, 1, ring + WSLOT), xbase, dbase, lcol);
  w_issue_all<RAGGED>(issue(cur, 2, ring + 2 * WSLOT), xbase, dbase, lcol);
  w_issue_all<RAGGED>(issue(cur, 3, ring + 3 * WSLOT), xbase, dbase, lcol);
  __builtin_amdgcn_s_waitcnt(vmcnt_le(3 * WLOADS));
  SWG_COMPILER_FENCE();
  __builtin_amdgcn_s_barrier();
  SWG_COMPILER_FENCE();
  const int64_t R2 = 2 * N;
  for (int64_t j = 0; j < my_items; ++j) {
    const WItem nxt = w_item<F>(f0 + (j + 1) * G, j + 1 < my_items, tiles, tnh, mp, M);
    zero_acc(acc);
    W_READ(ring, frags[0]);
    int64_t t = 0;
    for (; t + 4 < cur.nst; t += 4) {
      W_STEP(cur, t + 4, 0, true);
      W_STEP(cur, t + 5, 1, true);
      W_STEP(cur, t + 6, 2, true);
      W_STEP(cur, t + 7, 3, true);
    }
    W_STEP(nxt, 0, 0, true);
    W_STEP(nxt, 1, 1, true);
    W_STEP(nxt, 2, 2, true);
    W_STEP(nxt, 3, 3, false);   // the next tile's first stage is read after the epilogue
    // epilogue: rows k, columns n (of dg or dfc) straight from the accumulators
    const int64_t k0 = (int64_t)cur.k0 + wp * WR, n0 = (int64_t)cur.n0 + wq * WR;
    if (ws != nullptr) {
      // fp32 partials in the [K, 2N] layout of split s, one window per 32-row block
      float* dst = ws + (int64_t)cur.s * K * R2 + (cur.hi ? N : 0) + n0;
      int ln = lane;
      asm volatile("" : "+v"(ln));   // lane terms formed here: hoisted out of the tile
                                     // loop they would stay live, and spill
      const uint32_t row_bytes = (uint32_t)(R2 * 4);
      const int cols_left = (int)(N - n0);
      auto block = [&](auto I) {
        constexpr int i = decltype(I)::value;
        const int64_t kb = k0 + 32 * i;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(dst + kb * R2, clamp_bytes(K - kb < 32 ? K - kb : 32, R2 * 4));
        store_partial_block<F, i>(acc, ln, r, row_bytes, cols_left);
      };
      block(std::integral_constant<int, 0>{});
      block(std::integral_constant<int, 1>{});
      if constexpr (F == 4) {
        block(std::integral_constant<int, 2>{});
        block(std::integral_constant<int, 3>{});
      }
    } else {
      T* dw = cur.hi ? dwfc : dwg;
      int ln = lane;
      asm volatile("" : "+v"(ln));   // lane terms formed here: hoisted out of the tile
                                     // loop they would stay live, and spill
      const int64_t krows = K - k0 < WR ? K - k0 : WR;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(dw + k0 * N + n0, clamp_bytes(krows, N * 2));
      const uint32_t row_bytes = (uint32_t)(N * 2);
      const int cols_left = (int)(N - n0);
      rmw_block_rows<T, F, 0>(acc, ln, r, row_bytes, cols_left);
      rmw_block_rows<T, F, 1>(acc, ln, r, row_bytes, cols_left);
      if constexpr (F == 4) {
        rmw_block_rows<T, F, 2>(acc, ln, r, row_bytes, cols_left);
        rmw_block_rows<T, F, 3>(acc, ln, r, row_bytes, cols_left);
      }
    }
    cur = nxt;
  }
#undef W_STEP
#undef W_READ
  __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
}

template <typename T, int F, bool RAGGED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void w_stage_kernel(
    const T* __restrict__ x, const T* __restrict__ dg, const T* __restrict__ dfc,
    T* __restrict__ dwg, T* __restrict__ dwfc, float* __restrict__ ws, int64_t M, int64_t K,
    int64_t N, int64_t tnh, int64_t tiles, int64_t split_rows, int64_t nitems) {
  __shared__ __attribute__((aligned(1024))) uint16_t ring[Tc<F>::W_RING];
  const int64_t G = gridDim.x;
  const WMap mp{split_rows, 0, 0};
  w_items<T, F, RAGGED>(ring, x, dg, dfc, dwg, dwfc, ws, M, K, N, tnh, tiles, mp, nitems,
                        xcd_remap(blockIdx.x, G), G);
}

// ------------------------------------------------------------- fused w + x pass
// One launch for both GEMMs over [dg | dfc] [SwiGLU page, formulas 3 and 4, and the fusion
// motive of its operator background: no second trip through HBM for an intermediate].
// Workgroups 0 .. gx - 1 walk the x-stage tiles (row blocks of dx, in order), workgroups
// gx .. gx + gw - 1 walk w-stage items whose splits take 256-row chunks round-robin, so
// that in one round both halves of the grid read the same stretch of dg | dfc (at the
// large-batch shape: 128 x-stage tiles cover 64 row blocks while the 8 splits x 16 dW
// tiles cover the same 64 chunks); the stretch is read from HBM once and found again in
// the last-level cache.  The w items' fp32 partials per split are summed by
// w_reduce_kernel in split order, as in the w stage.
template <typename T, int F, bool RAGGED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void wx_fused_kernel(
    const T* __restrict__ x, const T* __restrict__ dg, const T* __restrict__ dfc,
    const T* __restrict__ wg, const T* __restrict__ wfc, T* __restrict__ dx,
    T* __restrict__ dwg, T* __restrict__ dwfc, float* __restrict__ ws, int64_t M, int64_t K,
    int64_t N, int64_t nq, int64_t x_ntiles, int64_t gx, int64_t tnh, int64_t w_tiles,
    int64_t chunk_rows, int64_t nsplit, int64_t w_nitems) {
  __shared__ __attribute__((aligned(1024))) uint16_t ring[Tc<F>::RING];
  const int64_t b = blockIdx.x;
  if (b < gx) {
    x_tiles<T, F, RAGGED>(ring, dg, dfc, wg, wfc, dx, M, K, N, nq, x_ntiles, xcd_remap(b, gx),
                          gx);
  } else {
    const int64_t gw = (int64_t)gridDim.x - gx;
    const WMap mp{0, chunk_rows, nsplit};
    w_items<T, F, RAGGED>(ring, x, dg, dfc, dwg, dwfc, ws, M, K, N, tnh, w_tiles, mp, w_nitems,
                          xcd_remap(b - gx, gw), gw);
  }
}

// dw = RNE(dw + sum_s ws[s]) in split order (fp32 dw: no rounding); 4 consecutive columns
// per lane (N % 4 == 0, so a group never straddles the dg | dfc boundary).
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

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// ----------------------------------------------------------------- forward (NN)
// SwiGLU forward [SwiGLU page, operator background]: g = x W_g + b_g, fc = x W_fc + b_fc,
// y = SiLU(g) fc, one GEMM [M, K] x [K, 2N] with a fused epilogue.  A = x rows m,
// contraction k contiguous (the x stage's operand A layout); B = W_g | W_fc rows k,
// columns n contiguous (the w stage's operand B layout, read with transposing reads).
// A workgroup owns 256 rows x 128 columns of g AND the same 128 columns of fc, so the
// epilogue has both at hand; each wave 128 rows x 64 columns of each (4 x 2 + 4 x 2 MFMA
// tiles: 256 accumulators, as in the backward GEMMs).  Slot layout: [256 rows of x][32]
// then [32 k-rows of W_g][128] then [32 k-rows of W_fc][128] (32 KiB).
constexpr int FN = 128;   // output columns of g (and of fc) per tile

struct FTile {   // first row of x / of the outputs, first column of W / of the outputs
  int p0, n0;
  bool live;
};

__device__ inline FTile f_tile(int64_t L, bool live, int64_t nn) {
  FTile c;
  c.live = live;
  const int64_t LL = live ? L : 0;
  c.p0 = (int)(LL / nn) * BP;
  c.n0 = (int)(LL % nn) * FN;
  return c;
}

template <typename T>
__device__ inline void f_read(const uint16_t* slot, int wp, int lane, const int (&boff)[2],
                              FragSet<T>& f) {
  using F = typename Mfma<T>::frag;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int lc = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FP; ++i) {
      const int r = wp * 128 + i * 32 + (lane & 31);
      f.a[kk][i] = *reinterpret_cast<const F*>(slot + r * BR + ((lc ^ xsw(r)) << 3));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f.b[kk][j] = tr_frag<T, FN>(slot + BP * BR + 16 * kk * FN + boff[j]);
      f.b[kk][2 + j] = tr_frag<T, FN>(slot + BP * BR + BR * FN + 16 * kk * FN + boff[j]);
    }
  }
}

// Store one output of the epilogue: values v0 (row R) and v1 (row R + 1) of one column per
// lane become 32-bit row pairs exactly as in store_tile_rows.  Non-temporal (cache policy
// nt): g, fc and y, 1.35 GB at the large-batch shape, are not read again by this kernel,
// and keeping them out of the caches leaves the x and W panels there (forward 679-683 ->
// 629-632 us in a same-board comparison; the x stage's dx stores gained nothing from it).
// Unconditional: columns past N carry offsets outside the window (the caller ORs in
// kOOB), which the range check drops; a per-lane branch around each store (three per
// element pair, exec-mask save and restore each) cost 602-612 against 557-572 us.
template <typename T>
__device__ inline void f_store_pair(float v0, float v1, uint32_t sel, __amdgpu_buffer_rsrc_t r,
                                    uint32_t voff) {
  const uint32_t own = pack2<T>(v0, v1);
  const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, false);
  const uint32_t out = __builtin_amdgcn_perm(nb, own, sel);
  __builtin_amdgcn_raw_buffer_store_b32(out, r, (int)voff, 0, 2);
}

// One forward issue: the tile's x window with the stage's first column as soffset, the
// stage's k-row windows of W_g and W_fc with the tile's first column as soffset.
struct FIssue {
  __amdgpu_buffer_rsrc_t ra, rg, rf;
  uint32_t sa, sw;
  int kleft, nleft;
  const uint16_t* dst;
  const uint16_t* dstw;
};

template <bool RAGGED, int E>
__device__ inline void f_dma(const FIssue& is, const uint32_t (&roff)[4], const int (&lcol)[4],
                             const uint32_t (&wbase)[2], const int (&wcol)[2]) {
  if (E < 4) {
    constexpr int i = E;
    const uint32_t v = !RAGGED || lcol[i] < is.kleft ? roff[i] : kOOB;
    dma16s<i * 16 * BR * 2>(is.ra, v, is.sa, is.dst);
  } else {
    constexpr int t = E & 1;
    const uint32_t v = !RAGGED || wcol[t] < is.nleft ? wbase[t] : kOOB;
    if (E < 6) dma16s<t * 4 * FN * 2>(is.rg, v, is.sw, is.dstw);
    else dma16s<BR * FN * 2 + t * 4 * FN * 2>(is.rf, v, is.sw, is.dstw);
  }
}

template <bool RAGGED>
__device__ inline void f_issue_all(const FIssue& is, const uint32_t (&roff)[4],
                                   const int (&lcol)[4], const uint32_t (&wbase)[2],
                                   const int (&wcol)[2]) {
  f_dma<RAGGED, 0>(is, roff, lcol, wbase, wcol);
  f_dma<RAGGED, 1>(is, roff, lcol, wbase, wcol);
  f_dma<RAGGED, 2>(is, roff, lcol, wbase, wcol);
  f_dma<RAGGED, 3>(is, roff, lcol, wbase, wcol);
  f_dma<RAGGED, 4>(is, roff, lcol, wbase, wcol);
  f_dma<RAGGED, 5>(is, roff, lcol, wbase, wcol);
  f_dma<RAGGED, 6>(is, roff, lcol, wbase, wcol);
  f_dma<RAGGED, 7>(is, roff, lcol, wbase, wcol);
}

// Fragment G (0..15, f_read's order: kk = G / 8; G % 8 < 4: x block G % 4, else W block
// G % 4, the first two of W_g, the last two of W_fc).
template <typename T, int G>
__device__ inline void f_read_one(const uint16_t* slot, int wp, int lane, const int (&boff)[2],
                                  FragSet<T>& f) {
  using F = typename Mfma<T>::frag;
  constexpr int kk = G / 8, blk = G % 4;
  if (G % 8 < 4) {
    const int lc = 2 * kk + (lane >> 5);
    const int r = wp * 128 + blk * 32 + (lane & 31);
    f.a[kk][blk] = *reinterpret_cast<const F*>(slot + r * BR + ((lc ^ xsw(r)) << 3));
  } else {
    f.b[kk][blk] = tr_frag<T, FN>(slot + BP * BR + (blk >= 2 ? BR * FN : 0) + 16 * kk * FN +
                                  boff[blk & 1]);
  }
}

template <typename T, bool RAGGED, bool READ_NEXT, int G>
__device__ inline void f_group(f32x16 (&acc)[FP][FQ], const FragSet<T>& f, FragSet<T>& fn,
                               const uint16_t* next_slot, int wp, int lane, const int (&boff)[2],
                               const FIssue& is, const uint32_t (&roff)[4], const int (&lcol)[4],
                               const uint32_t (&wbase)[2], const int (&wcol)[2]) {
  constexpr int kk = G >> 3, i = (G >> 1) & 3, j = (G & 1) * 2;
  acc[i][j] = Mfma<T>::mma(f.a[kk][i], f.b[kk][j], acc[i][j]);
  acc[i][j + 1] = Mfma<T>::mma(f.a[kk][i], f.b[kk][j + 1], acc[i][j + 1]);
  if (READ_NEXT) f_read_one<T, G>(next_slot, wp, lane, boff, fn);
  if (G & 1) f_dma<RAGGED, (G >> 1)>(is, roff, lcol, wbase, wcol);
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T, bool RAGGED, bool READ_NEXT, int... G>
__device__ inline void f_groups(std::integer_sequence<int, G...>, f32x16 (&acc)[FP][FQ],
                                const FragSet<T>& f, FragSet<T>& fn, const uint16_t* next_slot,
                                int wp, int lane, const int (&boff)[2], const FIssue& is,
                                const uint32_t (&roff)[4], const int (&lcol)[4],
                                const uint32_t (&wbase)[2], const int (&wcol)[2]) {
  (f_group<T, RAGGED, READ_NEXT, G>(acc, f, fn, next_slot, wp, lane, boff, is, roff, lcol, wbase,
                                     wcol),
   ...);
}

template <typename T, bool RAGGED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_kernel(
    const T* __restrict__ x, const T* __restrict__ wg, const T* __restrict__ wfc,
    const T* __restrict__ bg, const T* __restrict__ bfc, T* __restrict__ g, T* __restrict__ fc,
    T* __restrict__ y, int64_t M, int64_t K, int64_t N, int64_t nn, int64_t ntiles) {
  __shared__ __attribute__((aligned(1024))) uint16_t ring[4 * SLOT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave / WQ, wq = wave % WQ;
  const int64_t G = gridDim.x;
  const int64_t f0 = xcd_remap(blockIdx.x, G);
  const int64_t my_tiles = ntiles > f0 ? (ntiles - f0 + G - 1) / G : 0;
  int64_t nst = 4 * ((K + 4 * BR - 1) / (4 * BR));   // whole ring rounds (K = 0: one round
  if (nst < 4) nst = 4;                                  // of zeros, outputs = bias terms)

  // x: a 1 KiB load covers 16 rows x 4 chunks (rows 64 wave + 16 i + lane / 4), as in the
  // x stage.  W: a 1 KiB load covers 4 k-rows x 16 chunks (rows 8 wave + 4 t + lane / 16),
  // logical chunk (lane % 16) ^ wsw(row).
  uint32_t roff[4];
  int lcol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 64 * wave + 16 * i + (lane >> 2);
    lcol[i] = ((lane & 3) ^ xsw(row)) * 8;
    roff[i] = (uint32_t)row * (uint32_t)(K * 2) + (uint32_t)lcol[i] * 2u;
  }
  uint32_t wbase[2];
  int wcol[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 8 * wave + 4 * t + (lane >> 4);
    wcol[t] = ((lane & 15) ^ wsw(row)) * 8;
    wbase[t] = (uint32_t)row * (uint32_t)(N * 2) + (uint32_t)wcol[t] * 2u;
  }
  auto issue = [&](const FTile& c, int64_t st, uint16_t* slot) {
    int k0 = (int)st * BR;
    asm volatile("" : "+s"(k0));   // keep per-stage offsets from being hoisted (x stage)
    const int rows_a = c.live ? ((int)M - c.p0 < BP ? (int)M - c.p0 : BP) : 0;
    const int rows_w = c.live ? ((int)K - k0 < BR ? (int)K - k0 : BR) : 0;
    const int64_t kb = rows_w > 0 ? k0 : 0;
    FIssue is;
    is.ra = make_rsrc(uniform_ptr(x + (int64_t)c.p0 * K),
                      __builtin_amdgcn_readfirstlane(clamp_bytes(rows_a, K * 2)));
    const uint32_t wbytes = __builtin_amdgcn_readfirstlane(clamp_bytes(rows_w, N * 2));
    is.rg = make_rsrc(uniform_ptr(wg + kb * N), wbytes);
    is.rf = make_rsrc(uniform_ptr(wfc + kb * N), wbytes);
    is.sa = __builtin_amdgcn_readfirstlane((uint32_t)k0 * 2u);
    is.sw = __builtin_amdgcn_readfirstlane((uint32_t)c.n0 * 2u);
    is.kleft = (int)K - k0;
    is.nleft = (int)N - c.n0;
    is.dst = slot + 64 * wave * BR;
    is.dstw = slot + BP * BR + 8 * wave * FN;
    return is;
  };
  // transposing-read offsets of this wave's two 32-column blocks (see w_lane_offsets)
  int boff[2];
  {
    const int grp = lane >> 4, sl = lane & 15;
    const int q = 2 * (grp & 1) + ((sl & 3) >> 1);
    const int sw = wsw(sl >> 2);
    const int row = 8 * (grp >> 1) + (sl >> 2);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      boff[j] = row * FN + (((4 * (2 * wq + j) + q) ^ sw) << 3) + 4 * (sl & 1);
  }
#define F_READ(slot, f) f_read<T>((slot), wp, lane, boff, (f))
  // one pipeline step u (0..3), as the w stage's W_STEP
#define F_STEP(ctx, st, u, READ_NEXT)                                                       \
  do {                                                                                    \
    __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * LOADS_PER_STAGE));                            \
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);                                                \
    SWG_COMPILER_FENCE();                                                                 \
    __builtin_amdgcn_s_barrier();                                                         \
    SWG_COMPILER_FENCE();                                                                 \
    const FIssue is_ = issue((ctx), (st), ring + (u) * SLOT);                              \
    f_groups<T, RAGGED, (READ_NEXT)>(std::make_integer_sequence<int, 16>{}, acc,           \
                                     frags[(u) & 1], frags[((u) + 1) & 1],                \
                                     ring + (((u) + 1) & 3) * SLOT, wp, lane, boff, is_,   \
                                     roff, lcol, wbase, wcol);                            \
  } while (0)

  f32x16 acc[FP][FQ];
  FragSet<T> frags[2];
  FTile cur = f_tile(f0, my_tiles > 0, nn);
  f_issue_all<RAGGED>(issue(cur, 0, ring), roff, lcol, wbase, wcol);
  f_issue_all<RAGGED>(issue(cur, 1, ring + SLOT), roff, lcol, wbase, wcol);
  f_issue_all<RAGGED>(issue(cur, 2, ring + 2 * SLOT), roff, lcol, wbase, wcol);
  f_issue_all<RAGGED>(issue(cur, 3, ring + 3 * SLOT), roff, lcol, wbase, wcol);
  __builtin_amdgcn_s_waitcnt(vmcnt_le(3 * LOADS_PER_STAGE));
  SWG_COMPILER_FENCE();
  __builtin_amdgcn_s_barrier();
  SWG_COMPILER_FENCE();
  for (int64_t j = 0; j < my_tiles; ++j) {
    const FTile nxt = f_tile(f0 + (j + 1) * G, j + 1 < my_tiles, nn);
    zero_acc(acc);
    // the cleared accumulators pinned in AGPRs here: otherwise the register allocator
    // gives the loop's first steps another AGPR set and copies between them (192 moves
    // per tile; 584 -> 555 us without them, same bits)
#pragma unroll
    for (int i = 0; i < FP; ++i)
#pragma unroll
      for (int q = 0; q < FQ; ++q) asm volatile("" : "+a"(acc[i][q]));
    F_READ(ring, frags[0]);
    int64_t t = 0;
    for (; t + 4 < nst; t += 4) {
      F_STEP(cur, t + 4, 0, true);
      F_STEP(cur, t + 5, 1, true);
      F_STEP(cur, t + 6, 2, true);
      F_STEP(cur, t + 7, 3, true);
    }
    F_STEP(nxt, 0, 0, true);
    F_STEP(nxt, 1, 1, true);
    F_STEP(nxt, 2, 2, true);
    F_STEP(nxt, 3, 3, false);   // the next tile's first stage is read after the epilogue
    // epilogue: bias, SiLU, product, three outputs
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int odd = ln & 1;
      const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
      const int rows = (int)M - cur.p0 < BP ? (int)M - cur.p0 : BP;
      const uint32_t bytes = clamp_bytes(rows, N * 2);
      const int64_t base = (int64_t)cur.p0 * N + cur.n0;
      const __amdgpu_buffer_rsrc_t rgo = make_rsrc(g + base, bytes);
      const __amdgpu_buffer_rsrc_t rfo = make_rsrc(fc + base, bytes);
      const __amdgpu_buffer_rsrc_t ryo = make_rsrc(y + base, bytes);
      const int nleft = (int)N - cur.n0;
      const uint32_t row_bytes = (uint32_t)(N * 2);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int colv = wq * 64 + jj * 32 + (ln & 31);          // this lane's column
        const int colp = wq * 64 + jj * 32 + ((ln & 31) & ~1);   // its pair's first column
        // columns past N: offsets pushed out of the window, dropped by the range check
        uint32_t cbad = colp < nleft ? 0u : kOOB;
        asm volatile("" : "+v"(cbad));
        const float bgv = (bg != nullptr && colv < nleft) ? to_f32(bg[cur.n0 + colv]) : 0.0f;
        const float bfv = (bfc != nullptr && colv < nleft) ? to_f32(bfc[cur.n0 + colv]) : 0.0f;
        const uint32_t loff = (uint32_t)(4 * (ln >> 5) + odd) * row_bytes + (uint32_t)colp * 2u;
#pragma unroll
        for (int i = 0; i < FP; ++i)
#pragma unroll
          for (int rr = 0; rr < 16; rr += 2) {
            const uint32_t voff =
                (loff + (uint32_t)(wp * 128 + i * 32 + 8 * (rr >> 2) + (rr & 3)) * row_bytes) | cbad;
            const float g0 = acc[i][jj][rr] + bgv, g1 = acc[i][jj][rr + 1] + bgv;
            const float c0 = acc[i][2 + jj][rr] + bfv, c1 = acc[i][2 + jj][rr + 1] + bfv;
            const float s0 = sigmoid_only(g0), s1 = sigmoid_only(g1);
            f_store_pair<T>(g0, g1, sel, rgo, voff);
            f_store_pair<T>(c0, c1, sel, rfo, voff);
            f_store_pair<T>(g0 * s0 * c0, g1 * s1 * c1, sel, ryo, voff);
          }
      }
    }
    cur = nxt;
  }
#undef F_STEP
#undef F_READ
  __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
}

template <typename T, int F>
static void x_stage_f(const XPlan& p, const void* dg, const void* dfc, const void* wg,
                      const void* wfc, void* dx, int64_t M, int64_t K, int64_t N, int cus,
                      hipStream_t stream) {
  const int64_t slots = (int64_t)cus * Tc<F>::XOCC;
  const int64_t grid = p.tiles < slots ? p.tiles : slots;
  // per-lane column tests unless every double stage is whole: N a multiple of 64 and at
  // least two double stages per half (N = 64 pads the half with a stage past N)
  if (N % XA_BR == 0 && N >= 2 * XA_BR)
    SWG_LAUNCH((x_stage_kernel<T, F, false>), dim3((unsigned)grid), dim3(NT), 0, stream,
               static_cast<const T*>(dg), static_cast<const T*>(dfc),
               static_cast<const T*>(wg), static_cast<const T*>(wfc), static_cast<T*>(dx), M,
               K, N, p.nq, p.tiles);
  else
    SWG_LAUNCH((x_stage_kernel<T, F, true>), dim3((unsigned)grid), dim3(NT), 0, stream,
               static_cast<const T*>(dg), static_cast<const T*>(dfc),
               static_cast<const T*>(wg), static_cast<const T*>(wfc), static_cast<T*>(dx), M,
               K, N, p.nq, p.tiles);
}

template <typename T>
static hipError_t x_stage_t(const void* dg, const void* dfc, const void* wg, const void* wfc,
                            void* dx, int64_t M, int64_t K, int64_t N, int force_f, int cus,
                            hipStream_t stream) {
  const XPlan p = plan_x(M, K, N, force_f);
  if (p.f == 4) x_stage_f<T, 4>(p, dg, dfc, wg, wfc, dx, M, K, N, cus, stream);
  else x_stage_f<T, 2>(p, dg, dfc, wg, wfc, dx, M, K, N, cus, stream);
  return hipGetLastError();
}

hipError_t launch_x_stage(int dtype, const void* dg, const void* dfc, const void* w_g,
                          const void* w_fc, void* dx, int64_t M, int64_t K, int64_t N,
                          int force_f, int cus, hipStream_t stream) {
  if (dtype == 0) return x_stage_t<bf16>(dg, dfc, w_g, w_fc, dx, M, K, N, force_f, cus, stream);
  if (dtype == 1) return x_stage_t<fp16>(dg, dfc, w_g, w_fc, dx, M, K, N, force_f, cus, stream);
  return launch_x_stage32(dg, dfc, w_g, w_fc, dx, M, K, N, stream);
}

template <typename T, int F>
static void w_stage_f(const WPlan& p, const void* x, const void* dg, const void* dfc,
                      void* dwg, void* dwfc, int64_t M, int64_t K, int64_t N, float* wsp,
                      int cus, hipStream_t stream) {
  const int64_t nitems = p.splits * p.tiles;
  const int64_t grid = nitems < cus ? nitems : cus;
  // per-lane column tests only for tiles cut by the right or bottom edge of dW
  if (K % Tc<F>::P == 0 && N % Tc<F>::P == 0)
    SWG_LAUNCH((w_stage_kernel<T, F, false>), dim3((unsigned)grid), dim3(NT), 0, stream,
               static_cast<const T*>(x), static_cast<const T*>(dg), static_cast<const T*>(dfc),
               static_cast<T*>(dwg), static_cast<T*>(dwfc), wsp, M, K, N, p.tn / 2, p.tiles,
               p.rows, nitems);
  else
    SWG_LAUNCH((w_stage_kernel<T, F, true>), dim3((unsigned)grid), dim3(NT), 0, stream,
               static_cast<const T*>(x), static_cast<const T*>(dg), static_cast<const T*>(dfc),
               static_cast<T*>(dwg), static_cast<T*>(dwfc), wsp, M, K, N, p.tn / 2, p.tiles,
               p.rows, nitems);
}

template <typename T>
static hipError_t w_stage_t(const WPlan& p, const void* x, const void* dg, const void* dfc,
                            void* dwg, void* dwfc, int64_t M, int64_t K, int64_t N, float* ws,
                            int cus, hipStream_t stream) {
  float* wsp = p.splits > 1 ? ws : nullptr;
  if (p.f == 4) w_stage_f<T, 4>(p, x, dg, dfc, dwg, dwfc, M, K, N, wsp, cus, stream);
  else w_stage_f<T, 2>(p, x, dg, dfc, dwg, dwfc, M, K, N, wsp, cus, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  int64_t blocks = ceil_div(K * 2 * N / 4, 256);
  if (blocks > kMaxStreamBlocks) blocks = kMaxStreamBlocks;
  SWG_LAUNCH((w_reduce_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, stream, ws,
                     static_cast<T*>(dwg), static_cast<T*>(dwfc), K, N, p.splits);
  return hipGetLastError();
}

hipError_t launch_w_stage(int dtype, const WPlan& p, const void* x, const void* dg,
                          const void* dfc, void* dw_g, void* dw_fc, int64_t M, int64_t K,
                          int64_t N, float* ws, int cus, hipStream_t stream) {
  if (dtype == 0) return w_stage_t<bf16>(p, x, dg, dfc, dw_g, dw_fc, M, K, N, ws, cus, stream);
  if (dtype == 1) return w_stage_t<fp16>(p, x, dg, dfc, dw_g, dw_fc, M, K, N, ws, cus, stream);
  // fp32: the fp32 GEMM writes the same split partials, reduced in the same order
  hipError_t e = launch_w_stage32(p, x, dg, dfc, dw_g, dw_fc, M, K, N, ws, stream);
  if (e != hipSuccess || p.splits == 1) return e;
  int64_t blocks = ceil_div(K * 2 * N / 4, 256);
  if (blocks > kMaxStreamBlocks) blocks = kMaxStreamBlocks;
  SWG_LAUNCH((w_reduce_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, stream, ws,
                     static_cast<float*>(dw_g), static_cast<float*>(dw_fc), K, N, p.splits);
  return hipGetLastError();
}

template <typename T>
static hipError_t wx_t(const WXPlan& p, const void* x, const void* dg, const void* dfc,
                       const void* wg, const void* wfc, void* dwg, void* dwfc, void* dx,
                       int64_t M, int64_t K, int64_t N, float* ws, hipStream_t stream) {
  float* wsp = p.splits > 1 ? ws : nullptr;
  const int64_t grid = p.gx + p.gw;
  // the fast (non-ragged) walks need whole x-stage double stages and whole dW tiles
  const int64_t edge = tile_edge(p.f);
  const bool whole = N % XA_BR == 0 && N >= 2 * XA_BR && K % edge == 0 && N % edge == 0;
#define SWG_WX_ARGS                                                                          \
  static_cast<const T*>(x), static_cast<const T*>(dg), static_cast<const T*>(dfc),          \
      static_cast<const T*>(wg), static_cast<const T*>(wfc), static_cast<T*>(dx),            \
      static_cast<T*>(dwg), static_cast<T*>(dwfc), wsp, M, K, N, p.nq, p.x_tiles, p.gx,      \
      p.tn / 2, p.w_tiles, p.chunk_rows, p.splits, p.w_items
#define SWG_WX_LAUNCH(F_, R_)                                                                \
  SWG_LAUNCH((wx_fused_kernel<T, F_, R_>), dim3((unsigned)grid), dim3(NT), 0, stream, SWG_WX_ARGS)
  if (p.f == 4) {
    if (whole) SWG_WX_LAUNCH(4, false);
    else SWG_WX_LAUNCH(4, true);
  } else {
    if (whole) SWG_WX_LAUNCH(2, false);
    else SWG_WX_LAUNCH(2, true);
  }
#undef SWG_WX_LAUNCH
#undef SWG_WX_ARGS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  int64_t blocks = ceil_div(K * 2 * N / 4, 256);
  if (blocks > kMaxStreamBlocks) blocks = kMaxStreamBlocks;
  SWG_LAUNCH((w_reduce_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, stream, ws,
             static_cast<T*>(dwg), static_cast<T*>(dwfc), K, N, p.splits);
  return hipGetLastError();
}

hipError_t launch_wx(int dtype, const WXPlan& p, const void* x, const void* dg, const void* dfc,
                     const void* w_g, const void* w_fc, void* dw_g, void* dw_fc, void* dx,
                     int64_t M, int64_t K, int64_t N, float* ws, hipStream_t stream) {
  if (dtype == 0) return wx_t<bf16>(p, x, dg, dfc, w_g, w_fc, dw_g, dw_fc, dx, M, K, N, ws, stream);
  return wx_t<fp16>(p, x, dg, dfc, w_g, w_fc, dw_g, dw_fc, dx, M, K, N, ws, stream);
}

template <typename T>
static hipError_t fwd_t(const void* x, const void* wg, const void* wfc, const void* bg,
                        const void* bfc, void* g, void* fc, void* y, int64_t M, int64_t K,
                        int64_t N, int cus, hipStream_t stream) {
  const int64_t np = ceil_div(M, BP), nn = ceil_div(N, FN);
  const int64_t ntiles = np * nn;
  const int64_t grid = ntiles < cus ? ntiles : cus;
  // per-lane column tests unless every stage is whole: K a multiple of a ring round
  // (stages past K would otherwise read the next row of x) and N of the tile width
  if (K % (4 * BR) == 0 && N % FN == 0)
    SWG_LAUNCH((fwd_kernel<T, false>), dim3((unsigned)grid), dim3(NT), 0, stream,
                       static_cast<const T*>(x), static_cast<const T*>(wg),
                       static_cast<const T*>(wfc), static_cast<const T*>(bg),
                       static_cast<const T*>(bfc), static_cast<T*>(g), static_cast<T*>(fc),
                       static_cast<T*>(y), M, K, N, nn, ntiles);
  else
    SWG_LAUNCH((fwd_kernel<T, true>), dim3((unsigned)grid), dim3(NT), 0, stream,
                       static_cast<const T*>(x), static_cast<const T*>(wg),
                       static_cast<const T*>(wfc), static_cast<const T*>(bg),
                       static_cast<const T*>(bfc), static_cast<T*>(g), static_cast<T*>(fc),
                       static_cast<T*>(y), M, K, N, nn, ntiles);
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, const void* x, const void* w_g, const void* w_fc,
                      const void* b_g, const void* b_fc, void* g, void* fc, void* y, int64_t M,
                      int64_t K, int64_t N, int cus, hipStream_t stream) {
  if (dtype == 0) return fwd_t<bf16>(x, w_g, w_fc, b_g, b_fc, g, fc, y, M, K, N, cus, stream);
  if (dtype == 1) return fwd_t<fp16>(x, w_g, w_fc, b_g, b_fc, g, fc, y, M, K, N, cus, stream);
  return launch_fwd32(x, w_g, w_fc, b_g, b_fc, g, fc, y, M, K, N, stream);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t words = (int64_t)(bytes / 4);
  int64_t blocks = ceil_div(words, 256);
  if (blocks > kMaxStreamBlocks) blocks = kMaxStreamBlocks;
  if (blocks < 1) blocks = 1;
  SWG_LAUNCH(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace swg
