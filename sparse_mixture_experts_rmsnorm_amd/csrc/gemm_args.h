// Tile lists and arguments of the expert GEMM kernels (gemm.hip), and their
// host launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// One output tile of a grouped / BCSR / dense GEMM:  Y[row, ocol0 + f] =
// epilogue(sum_k X[row, xk + k] * W[wrow0 + f, kofs + k]),  rows [row0, row_end).
//
// A tile of the last round of a persistent launch may be cut along K into
// nparts pieces (part = 0 .. nparts - 1) that run on different compute
// units: each piece stores its fp32 partial sums at piece slot pslot0 + part;
// the fixup kernel that follows the GEMM adds the nparts partials in part
// order and applies the tile's epilogue.
struct Tile {
  int row0, row_end;  // GEMM rows (permuted rows, or tokens)
  int wrow0;          // first packed weight row (feature) of the tile
  int kofs;           // K offset into the weight rows
  int klen;           // K length (multiple of 64)
  int ocol0;          // first output column
  int expert;
  int spare;
  int xk;             // K offset into the activation rows (a K piece's start)
  int part, nparts;   // K piece of the tile (0, 1 for a whole tile)
  int pslot0;         // partial-buffer slot of part 0 (pieces only)
};

// EPI_STORE_T: the plain accumulator in bf16 over a tile whose last
// features may be missing (tile.spare = the features that exist, a multiple
// of 32; the backward of the second linear).  EPI_SCALE_F32 with row_r NULL
// stores the plain fp32 accumulator (the weight-gradient GEMMs).
enum Epi {
  EPI_ACT = 0, EPI_SWIGLU = 1, EPI_GATE = 2, EPI_SCALE_F32 = 3, EPI_STORE_T = 5
};

struct GemmArgs {
  const void* X; int64_t ldx;      // activations, row = GEMM row
  const void* W; int64_t ldw;      // packed weights, row = feature
  const Tile* tiles; const int* ntiles;
  void* Y; int64_t ldy;            // output (dtype, or fp32 for EPI_SCALE_F32)
  const float* row_r;              // r per GEMM row (EPI_ACT / SWIGLU / SCALE)
  const float* row_w;              // gate per GEMM row (EPI_GATE), NULL = 1
  int epi; int act;                // act: 0 GELU erf, 1 GELU tanh
  int64_t ysplit;                  // EPI_SCALE_F32: elements between the K-split
                                   // planes (tile.spare = split)
  const int32_t* xrow;             // NULL, or X row of each GEMM row (-1: any row;
                                   // its result is never read)
  // First linear (EPI_ACT / EPI_SWIGLU): when non-NULL, the pre-activations
  // r * acc are also stored (bf16) at pre[row * ldpre + packed feature], in
  // the expert-local packed order of the weights (for the backward pass).
  void* pre; int64_t ldpre;
  // Persistent launches planned per XCD (PlanArgs.grid > 0): ntiles[0] is
  // the list length and ntiles[1 .. NX + 1] the first tile of each XCD's run
  // (NX = 8 when the grid is a multiple of 8, else 1); workgroup b runs
  // entries base[b % NX] + b / NX, + grid / NX, ... of its run; ntiles[10]
  // is the number of split tiles.  part: fp32 partials of K pieces (grid x
  // BF x BT floats); counters: the list entry of each split tile's part 0
  // (read by the fixup kernel).
  int xcd_runs;
  float* part;
  int* counters;
  // Bytes of X and W from their bases that the launch may read.  The bf16
  // kernel reads both through buffer resources with 32-bit offsets, so both
  // must be below 4 GiB (launch_gemm refuses the launch otherwise); the
  // hardware returns zeros for anything past them, so every call sets them.
  int64_t x_bytes, w_bytes;
};

// Plan of GEMM tiles for grouped experts.  gemm = 1: first linear (features
// = packed rows of the expert, K = d); gemm = 2: second linear (features = d,
// K = f_e).  rows of expert e: [offsets[e], offsets[e+1]).
struct PlanArgs {
  const int32_t* offsets;    // [E+1]; NULL = one dense group of dense_rows rows
  int dense_rows;            // dense: GEMM rows (tokens)
  int dense_n;               // dense: packed features
  const int32_t* foff;       // [E+1] hidden-unit offsets (device)
  int E; int gemm; int swiglu; int d;
  int bt;                    // tokens per tile
  int bf;                    // packed features per tile
  int fold;                  // output columns per packed feature divisor (2 for SwiGLU GEMM1)
  Tile* tiles; int* ntiles; int max_tiles;
  int ksplit;                // second linear: K parts per tile (1, 2 or 4, equal and whole
                             // K stages); tile.spare = part
  int kmul;                  // second linear: K = kmul * f_e at kmul * foff[e] (0 means 1)
  int ragged;                // first linear: last feature tile of a group may be partial
                             // (tile.spare = its valid features, a multiple of 32)
  // BCSR (topology walk) when row_offsets != NULL
  const int32_t* row_offsets; const int32_t* column_indices; const int32_t* block_offsets;
  int block;
  // grid > 0: the list is laid out for a persistent launch of `grid`
  // workgroups: each XCD's run of tiles (as the XCD remap splits the list)
  // ends with its last-round remainder cut along K into up to max_parts
  // pieces so that the run fills its last round (ntiles[1..9] get the runs'
  // bases, ntiles[10] the number of split tiles, counters[g] the list entry
  // of split tile g's part 0).  The tile buffer must hold max_tiles + grid
  // entries.  Pieces are cut at whole K stages of kstage elements (the GEMM
  // kernel's stage: 64 for bf16, 128 for MXFP8; 0 means 64).  cost_split:
  // the runs of a grouped list (ksplit 1) end at equal shares of the list's
  // modelled cost (row blocks and K stages of each tile) instead of at equal
  // tile counts, so that XCDs whose experts end in short row tiles take more
  // tiles.
  int grid; int max_parts; int* counters;
  int kstage;
  int cost_split;
};

// MXFP8 GEMM: X and W hold E4M3 codes (ldx / ldw in bytes).  ws / xs: the
// weights' and the activation rows' E8M0 block scales, both stage-major (the
// four bytes of row r in 128-element K stage s at s * ld + 4 r, ld = ldws /
// ldxs = 4 x the rows of the array).  The first-linear epilogues write MXFP8
// h (codes to Y with ldy bytes, scales stage-major to ys with ldys bytes
// between stages), the gate epilogues bf16 Y.
struct MxGemmArgs {
  GemmArgs g;
  const uint8_t* xs; int64_t ldxs;
  const uint8_t* ws; int64_t ldws;
  uint8_t* ys; int64_t ldys;
  // byte extents of X, W, xs and ws (each below 2 GiB: the kernel reads
  // them through buffer resources with 32-bit offsets)
  int64_t x_bytes, w_bytes, xs_bytes, ws_bytes;
};

hipError_t launch_plan(const PlanArgs& p, hipStream_t s);
// Two tile lists (independent outputs) in one launch.
hipError_t launch_plan_pair(const PlanArgs& p0, const PlanArgs& p1, hipStream_t s);
hipError_t launch_gemm(int dtype, const GemmArgs& a, int bf, int bt, int grid, hipStream_t s);
// Workgroups of a persistent launch of the bf16 GEMM over at most `tiles`
// tiles (one per compute unit, a multiple of 8 when there are enough tiles).
int gemm_persistent_grid(int tiles);
// The epilogue of the split tiles of a persistent launch planned for it
// (grid: workgroups, at least the number of split tiles).
hipError_t launch_piece_fixup(const GemmArgs& a, int bf, int bt, int grid, int max_parts,
                              hipStream_t s);

}  // namespace moe
