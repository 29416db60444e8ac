// Host-side launch planning, shared by the workspace-size queries and the launches so
// the two always agree.  Pure integer arithmetic: no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace swg {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int elem_size(int dtype) { return dtype == 2 ? 4 : 2; }
inline int vec_of(int dtype) { return 16 / elem_size(dtype); }

// ---------------------------------------------------------------- b stage
// A workgroup of 256 threads owns a strip of TX vector-columns (TX a power of two
// <= 32; TY = 256 / TX rows per pass, each lane issuing the loads of kBRowsInFlight rows
// before it computes them).  The rows are cut into units of unit_rows = max(64,
// kBRowsInFlight * TY) rows, so a unit is whole passes; the workgroups of a strip
// ("walkers", grid.y of them) take the units round-robin (walker w: units w, w + walkers,
// ...), a static assignment that keeps the column sums run-to-run deterministic while
// every walker ends within one unit of the others.  Each walker leaves one fp32 partial
// row [2N] (dg sums, then dfc sums) in the workspace, which the finalize kernel sums in
// walker order.  Measured on MI355X at M = 220000, N = 1024 bf16 (inputs in HBM, finalize
// included): 32-wide strips, 8 rows in flight and 64-row units with 256 walkers per strip
// run 384 us; 64-wide strips, 4 rows and 32-row units ran 403-406 us; walker counts that
// are not a power of two (balanced to whole rounds) ran slower.
struct BPlan {
  int vec;             // elements per 16-byte access (1 when the scalar path is used)
  int rif;             // rows whose loads a lane issues before computing (vector path)
  int tx, ty;          // thread layout inside the 256-thread workgroup
  int64_t cv;          // vector columns per row = N / vec
  int64_t nstrips;     // ceil(cv / tx)
  int64_t unit_rows;   // rows per work unit (a multiple of the rows one pass covers)
  int64_t nunits;      // ceil(M / unit_rows)
  int64_t nwalk;       // walkers per strip (grid.y) = partial rows
  size_t ws_bytes;     // nwalk * 2N * sizeof(float)
};

constexpr int kBThreads = 256;
constexpr int kBMaxTx = 32;              // widest strip, in 16-byte vector columns
constexpr int64_t kBMinUnitRows = 64;    // smallest work unit
// Walkers per strip: of the smallest power of two that launches at least kBMinBlocks
// workgroups in all and the next two (each capped at the number of units), the one that
// minimises rounds x units per walker, where a round is kBSlots workgroups (one resident
// per CU of the MI355X: the vector kernel holds 300 VGPRs).  More walkers would also add
// partial rows for the finalize to read.  Counts that are not a power of two ran
// slower even when balanced (measured at N = 1024); at N = 14336 bf16 the rule gives 56
// strips x 32 walkers (seven full rounds of 8 units, 434 us) where 56 x 19 ran 474 us and
// 56 x 18 441-444 us.
constexpr int64_t kBSlots = 256;
// Size of the static partial-row array used by swiglu_bwd_b_noalloc (16 MiB: every shape
// up to N = 2^21 columns fits; at N = 1024 the plan needs 2 MiB, at N = 14336 3.5 MiB).
constexpr size_t kBScratchBytes = size_t(16) << 20;
constexpr int64_t kBMinBlocks = 1024;
constexpr int kBRowsInFlight = 8;        // rows whose loads a lane issues before computing
// Small batches (at most kBSmallBlocks workgroups with kBRowsInFlight rows per lane): the
// vector kernel holds 300 registers, so one workgroup per CU runs its single pass of
// loads, then its arithmetic, with nothing to overlap them.  There the plan takes
// kBSmallRows rows in flight (a kernel several workgroups of which share a CU), units of
// one pass and one walker per unit (at most kBSmallMaxBlocks workgroups).
constexpr int kBSmallRows = 4;
constexpr int64_t kBSmallBlocks = 4096;
constexpr int64_t kBSmallMaxBlocks = 4096;

inline BPlan plan_b(int64_t M, int64_t N, int dtype, bool vector_path) {
  BPlan p{};
  // the unit size and the walker count depend only on (M, N, dtype), never on pointer
  // alignment (the workspace query cannot see the pointers)
  const int vref = vec_of(dtype);
  const int64_t cv_ref = (N % vref == 0) ? N / vref : N;
  int tx_ref = 1;
  while (tx_ref < kBMaxTx && tx_ref < cv_ref) tx_ref <<= 1;
  const int64_t strips_ref = ceil_div(cv_ref, tx_ref);
  const int64_t pass_rows = (int64_t)kBRowsInFlight * (kBThreads / tx_ref);
  p.rif = kBRowsInFlight;
  p.unit_rows = pass_rows > kBMinUnitRows ? pass_rows : kBMinUnitRows;
  p.nunits = M > 0 ? ceil_div(M, p.unit_rows) : 0;
  int64_t nwalk = 1;
  if (p.nunits > 0 && strips_ref * p.nunits <= kBSmallBlocks) {
    p.rif = kBSmallRows;
    p.unit_rows = (int64_t)kBSmallRows * (kBThreads / tx_ref);
    p.nunits = ceil_div(M, p.unit_rows);
    const int64_t cap = kBSmallMaxBlocks / strips_ref;
    nwalk = p.nunits < cap ? p.nunits : (cap > 0 ? cap : 1);
  } else if (p.nunits > 0) {
    int64_t w0 = 1;   // smallest power of two reaching kBMinBlocks workgroups
    while (strips_ref * w0 < kBMinBlocks) w0 *= 2;
    int64_t best_cost = -1;
    for (int64_t w = w0; w <= 4 * w0; w *= 2) {
      const int64_t ww = w < p.nunits ? w : p.nunits;
      const int64_t cost = ceil_div(strips_ref * ww, kBSlots) * ceil_div(p.nunits, ww);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        nwalk = ww;
      }
      if (ww == p.nunits) break;
    }
  }
  p.nwalk = nwalk;
  p.ws_bytes = (M > 0 && N > 0) ? (size_t)p.nwalk * (size_t)(2 * N) * sizeof(float) : 0;

  p.vec = (vector_path && N % vref == 0) ? vref : 1;
  p.cv = N / p.vec;
  int tx = 1;
  while (tx < kBMaxTx && tx < p.cv) tx <<= 1;
  p.tx = tx;
  p.ty = kBThreads / tx;
  p.nstrips = ceil_div(p.cv, tx);
  return p;
}

// ---------------------------------------------------------------- GEMM tiles
// Both GEMMs use square output tiles of edge 64 F per workgroup of four waves: F = 4
// (256 x 256) or F = 2 (128 x 128), and a 32-deep contraction step per LDS stage (the
// x stage moves two stages per load).
constexpr int kTileP = 256;     // output rows per workgroup at F = 4
constexpr int kTileQ = 256;     // output cols per workgroup at F = 4
constexpr int kTileR = 32;      // contraction depth per LDS stage
constexpr int64_t kMaxGemmDim = int64_t(1) << 22;  // K, N limit of the GEMM stages
inline int64_t tile_edge(int f) { return 64 * (int64_t)f; }

// Tile choice.  256 x 256 tiles load half the operand bytes per flop of 128 x 128 tiles
// and run faster per flop; 128 x 128 tiles win when the large ones leave CUs idle (small
// batches) or, in the w stage, need many M splits whose fp32 partials cost a round trip
// through memory.  The planner takes the configuration with the smaller time estimate:
// rounds of work items over the CUs x pipeline stages per item x the time of one stage
// at that configuration, plus, for the w stage, the partials' write and read at the
// streaming rate and the reduce launch.  Stage times from kernel spans on MI355X (bf16,
// both tile sizes forced, M = 256 .. 220000 at K = 512, N = 1024 and four shapes with K, N
// up to 4096 and 14336): at 128 x 128 one workgroup per CU is bound by LDS traffic (the
// DMA writes plus the fragment reads of twice as many bytes per flop), so its stage takes
// 0.4-0.45 of a 256 x 256 stage for a quarter of the work.  The x stage at 128 x 128 runs
// two workgroups per CU when it has more tiles than CUs: a double stage then takes 1.15 us
// per workgroup (two progress at once), against 0.75 us for a workgroup alone.
constexpr int64_t kGemmSlots = 256;        // one persistent workgroup per CU of the MI355X
constexpr int64_t kXStageNs[2] = {1700, 750};   // x: one 64-deep double stage, F = 4 / F = 2
constexpr int64_t kXStageNsShared = 1150;       // x, F = 2, two workgroups per CU
constexpr int64_t kWStageNs[2] = {850, 320};    // w: one 32-deep stage, F = 4 / F = 2
constexpr int64_t kReduceLaunchNs = 2000;       // w_reduce launch and ramp
constexpr int64_t kStreamBytesPerNs = 5000;     // partials' round trip, ~5 TB/s
inline int64_t stage_ns(const int64_t (&t)[2], int f) { return f == 4 ? t[0] : t[1]; }

// x stage: output [M, K] in tiles of edge 64 F; every tile runs nds double stages.
struct XPlan {
  int f;
  int64_t nq, tiles;       // column tiles per row block, tiles
};

inline int64_t x_double_stages(int64_t N) {
  const int64_t sd = ceil_div(N, 2 * kTileR);
  return 2 * (sd < 2 ? 2 : sd);
}

inline XPlan plan_x_f(int64_t M, int64_t K, int f) {
  XPlan p{};
  p.f = f;
  p.nq = ceil_div(K, tile_edge(f));
  p.tiles = ceil_div(M, tile_edge(f)) * p.nq;
  return p;
}

inline int64_t x_time_ns(const XPlan& p, int64_t N, int64_t slots) {
  const int64_t nds = x_double_stages(N);
  if (p.f == 4) return ceil_div(p.tiles, slots) * nds * kXStageNs[0];
  if (p.tiles <= slots) return nds * kXStageNs[1];   // one workgroup per CU
  return ceil_div(p.tiles, 2 * slots) * nds * kXStageNsShared;
}

// force_f: 4 or 2 overrides the estimate (0: the planner's choice); likewise below.
inline XPlan plan_x(int64_t M, int64_t K, int64_t N, int force_f = 0) {
  if (force_f == 4 || force_f == 2) return plan_x_f(M, K, force_f);
  const XPlan big = plan_x_f(M, K, 4), small = plan_x_f(M, K, 2);
  return x_time_ns(small, N, kGemmSlots) < x_time_ns(big, N, kGemmSlots) ? small : big;
}

// w stage: output [K, 2N]; when it has too few tiles to fill the chip the batch
// dimension M is split into S ranges whose fp32 partials are summed in order.
struct WPlan {
  int f;                   // tile configuration
  int64_t tk, tn, tiles;   // tile grid over [K, 2N]: tn / 2 column tiles in dg, tn / 2 in dfc
  int64_t splits;          // S
  int64_t rows;            // rows of M per split (multiple of kTileR)
  size_t ws_bytes;         // S > 1: S * K * 2N * sizeof(float)
};

constexpr int64_t kWTargetBlocks = kGemmSlots;
constexpr int64_t kWMinRowsPerSplit = 512;

inline WPlan plan_w_f(int64_t M, int64_t K, int64_t N, int f) {
  WPlan p{};
  p.f = f;
  p.tk = ceil_div(K, tile_edge(f));
  p.tn = 2 * ceil_div(N, tile_edge(f));
  p.tiles = p.tk * p.tn;
  // splits that keep tiles x S within one round of workgroups
  int64_t s = p.tiles > 0 ? kWTargetBlocks / p.tiles : 1;
  const int64_t smax = M / kWMinRowsPerSplit;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  p.rows = ceil_div(ceil_div(M, s), kTileR) * kTileR;
  if (p.rows < kTileR) p.rows = kTileR;
  p.splits = M > 0 ? ceil_div(M, p.rows) : 1;
  if (p.splits < 1) p.splits = 1;
  p.ws_bytes = (p.splits > 1 && K > 0 && N > 0)
                   ? (size_t)p.splits * (size_t)K * (size_t)(2 * N) * sizeof(float)
                   : 0;
  return p;
}

inline int64_t w_time_ns(const WPlan& p) {
  const int64_t nst = 4 * ceil_div(p.rows, 4 * kTileR);   // whole ring rounds per item
  int64_t t = ceil_div(p.splits * p.tiles, kWTargetBlocks) * nst * stage_ns(kWStageNs, p.f);
  if (p.splits > 1) t += kReduceLaunchNs + 2 * (int64_t)p.ws_bytes / kStreamBytesPerNs;
  return t;
}

inline WPlan plan_w(int64_t M, int64_t K, int64_t N, int force_f = 0) {
  if (force_f == 4 || force_f == 2) return plan_w_f(M, K, N, force_f);
  const WPlan big = plan_w_f(M, K, N, 4), small = plan_w_f(M, K, N, 2);
  return w_time_ns(small) < w_time_ns(big) ? small : big;
}

// fused w + x pass: the grid is split between x-stage tiles (gx workgroups) and w-stage
// items (gw workgroups).  Both GEMMs have the same flop count, so half of the workgroups
// go to each; the w items are the dW tiles times S splits over 256-row chunks taken
// round-robin, S chosen so the w half of the grid is filled (and at least 512 rows per
// split, as in the w stage).  With 128 + 128 workgroups both halves advance through the
// rows of [dg | dfc] at the same rate.  Both halves use 128 x 128 tiles when the x stage
// has fewer 256 x 256 tiles than its half of the grid.
struct WXPlan {
  bool separate;                   // run the w stage and the x stage as two launches
  int f;                           // tile configuration of both halves
  int64_t nq, x_tiles, gx;         // x stage: column tiles per row block, tiles, workgroups
  int64_t tn, w_tiles, splits;     // w stage: tile grid, tiles, S
  int64_t w_items, gw;             // items (tiles x S), workgroups
  int64_t chunk_rows;              // 256
  size_t ws_bytes;                 // S > 1: S * K * 2N * sizeof(float); separate: plan_w's
};

constexpr int64_t kWXChunkRows = 256;
constexpr int64_t kWXWorkgroups = 256;

inline WXPlan plan_wx(int64_t M, int64_t K, int64_t N, int force_f = 0) {
  WXPlan p{};
  p.f = ceil_div(M, tile_edge(4)) * ceil_div(K, tile_edge(4)) < kWXWorkgroups / 2 ? 2 : 4;
  if (force_f == 4 || force_f == 2) p.f = force_f;
  const int64_t edge = tile_edge(p.f);
  p.nq = ceil_div(K, edge);
  p.x_tiles = ceil_div(M, edge) * p.nq;
  p.gx = p.x_tiles < kWXWorkgroups / 2 ? p.x_tiles : kWXWorkgroups / 2;
  if (p.gx < 1) p.gx = 1;
  p.tn = 2 * ceil_div(N, edge);
  p.w_tiles = ceil_div(K, edge) * p.tn;
  const int64_t target = kWXWorkgroups - p.gx;
  int64_t s = p.w_tiles > 0 ? target / p.w_tiles : 1;
  const int64_t smax = M / kWMinRowsPerSplit;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  p.splits = s;
  p.chunk_rows = kWXChunkRows;
  p.w_items = p.w_tiles * p.splits;
  p.gw = p.w_items < target ? p.w_items : target;
  if (p.gw < 1) p.gw = 1;
  p.ws_bytes = (p.splits > 1 && K > 0 && N > 0)
                   ? (size_t)p.splits * (size_t)K * (size_t)(2 * N) * sizeof(float)
                   : 0;
  // Without an M split the w items each walk all of M while the x tiles walk row blocks,
  // so the two halves never read the same rows at the same time; when each stage also
  // fills the GPU on its own (two rounds or more of each half), fusing gives no traffic
  // back and only shares the chip: measured 1.68 ms against 1.53 ms for w + x at
  // M = 4096, K = 4096, N = 14336, and 6.6 ms against 6.2 ms at M = 16384.  Those shapes
  // run the two stages as separate launches.
  p.separate = p.splits == 1 && p.x_tiles >= 2 * p.gx && p.w_items >= 2 * p.gw;
  if (p.separate) p.ws_bytes = plan_w(M, K, N, force_f).ws_bytes;
  return p;
}

}  // namespace swg
