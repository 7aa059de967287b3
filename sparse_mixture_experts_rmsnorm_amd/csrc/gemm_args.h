// Tile lists and arguments of the expert GEMM kernels (gemm.hip), and their
// host launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// One output tile of a grouped / BCSR / dense GEMM:  Y[row, ocol0 + f] =
// epilogue(sum_k X[row, k] * W[wrow0 + f, kofs + k]),  rows [row0, row_end).
struct Tile {
  int row0, row_end;  // GEMM rows (permuted rows, or tokens)
  int wrow0;          // first packed weight row (feature) of the tile
  int kofs;           // K offset into the weight rows
  int klen;           // K length (multiple of 64)
  int ocol0;          // first output column
  int expert;
  int spare;
};

// EPI_GATE_SPLIT: gated partial of one K split, written to Y + split * ysplit.
// EPI_STORE_T: the plain accumulator in bf16 over a tile whose last
// features may be missing (tile.spare = the features that exist, a multiple
// of 32; the backward of the second linear).  EPI_SCALE_F32 with row_r NULL
// stores the plain fp32 accumulator (the weight-gradient GEMMs).
enum Epi {
  EPI_ACT = 0, EPI_SWIGLU = 1, EPI_GATE = 2, EPI_SCALE_F32 = 3, EPI_GATE_SPLIT = 4,
  EPI_STORE_T = 5
};

struct GemmArgs {
  const void* X; int64_t ldx;      // activations, row = GEMM row
  const void* W; int64_t ldw;      // packed weights, row = feature
  const Tile* tiles; const int* ntiles;
  void* Y; int64_t ldy;            // output (dtype, or fp32 for EPI_SCALE_F32)
  const float* row_r;              // r per GEMM row (EPI_ACT / SWIGLU / SCALE)
  const float* row_w;              // gate per GEMM row (EPI_GATE), NULL = 1
  int epi; int act;                // act: 0 GELU erf, 1 GELU tanh
  int64_t ysplit;                  // EPI_GATE_SPLIT / EPI_SCALE_F32: elements between the
                                   // K-split planes (tile.spare = split)
  const int32_t* xrow;             // NULL, or X row of each GEMM row (-1: any row;
                                   // its result is never read)
  // First linear (EPI_ACT / EPI_SWIGLU): when non-NULL, the pre-activations
  // r * acc are also stored (bf16) at pre[row * ldpre + packed feature], in
  // the expert-local packed order of the weights (for the backward pass).
  void* pre; int64_t ldpre;
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
};

// MXFP8 GEMM: X and W hold E4M3 codes (ldx / ldw in bytes), xs / ws their
// E8M0 block scales [rows, K / 32]; the first-linear epilogues write MXFP8 h
// (codes to Y with ldy bytes, scales to ys), the gate epilogues bf16 Y.
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
int gemm_tile_bf(int dtype);   // packed features per tile the GEMM kernels use
int gemm_tile_bt(int dtype, int bcsr);

}  // namespace moe
