// Host-side launchers implemented in the .hip files; called by api.cpp.
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
enum Epi { EPI_ACT = 0, EPI_SWIGLU = 1, EPI_GATE = 2, EPI_SCALE_F32 = 3, EPI_GATE_SPLIT = 4 };

struct GemmArgs {
  const void* X; int64_t ldx;      // activations, row = GEMM row
  const void* W; int64_t ldw;      // packed weights, row = feature
  const Tile* tiles; const int* ntiles;
  void* Y; int64_t ldy;            // output (dtype, or fp32 for EPI_SCALE_F32)
  const float* row_r;              // r per GEMM row (EPI_ACT / SWIGLU / SCALE)
  const float* row_w;              // gate per GEMM row (EPI_GATE), NULL = 1
  int epi; int act;                // act: 0 GELU erf, 1 GELU tanh
  int64_t ysplit;                  // EPI_GATE_SPLIT: elements between split planes
  const int32_t* xrow;             // NULL, or X row of each GEMM row (-1: any row;
                                   // its result is never read)
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
  int ksplit;                // second linear: K halves per tile (1 or 2); tile.spare = split
  // BCSR (topology walk) when row_offsets != NULL
  const int32_t* row_offsets; const int32_t* column_indices; const int32_t* block_offsets;
  int block;
};

hipError_t launch_plan(const PlanArgs& p, hipStream_t s);
hipError_t launch_gemm(int dtype, const GemmArgs& a, int bf, int bt, int grid, hipStream_t s);
int gemm_tile_bf(int dtype);   // packed features per tile the GEMM kernels use
int gemm_tile_bt(int dtype, int bcsr);

hipError_t launch_pack_transpose(const void* src, int dtype, int64_t K, int64_t N, void* dst,
                                 hipStream_t s);
hipError_t launch_pack_swiglu(const void* w1, const void* w3, int dtype, int64_t d, int64_t F,
                              const int32_t* foff_dev, const int64_t* sizes_host, int64_t E,
                              void* dst, hipStream_t s);

hipError_t launch_rmsnorm(const void* x, int dtype, int64_t T, int64_t d, const void* gamma,
                          float eps, float* r, void* xg, hipStream_t s);
// Noise and statistics of the dense router (all nullable).  part_p /
// part_g: per-workgroup partial sums [blocks][E] (workspace).
struct RouterExtras {
  const float* noise = nullptr;
  float noise_std = 0.f;
  float* part_p = nullptr;
  float* part_g = nullptr;
  float* prob_sum = nullptr;
  float* gate_sum = nullptr;
  float* aux = nullptr;
};
// Workgroups of the dense router launch for T tokens (the rows of the
// partial-sum arrays).
int64_t router_dense_blocks(int dtype, int64_t T);
hipError_t launch_router_dense(const void* x, int dtype, int64_t T, int64_t d, const void* wr_t,
                               const float* bias, int64_t E, const float* r_in, float eps,
                               float* r_out, int k, int renorm, int32_t* ids, float* w,
                               float* logits, const RouterExtras& ex, hipStream_t s);
hipError_t launch_cartesian_topk(const float* scores, int64_t T, int64_t Nr, int64_t Nc, int k,
                                 int renorm, int32_t* ids, float* w, hipStream_t s);

struct DispatchArgs {
  const int32_t* ids; const float* w; const float* r; const void* x; int dtype;
  int64_t T, d, E; int k; int64_t cap; int pad; int64_t rows_max;
  int32_t* counts; int32_t* offsets; int32_t* pos; int32_t* row_token; float* row_r;
  float* row_w; int32_t* row_expert; void* x_perm; void* stats;
  void* ws; size_t ws_bytes;
};
size_t dispatch_ws_bytes(int64_t T, int k, int64_t E);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);

hipError_t launch_topology(const int32_t* offsets, const int32_t* size_blocks,
                           const int32_t* block_offsets, int64_t E, int block, int64_t rows_max,
                           int32_t* row_offsets, int32_t* column_indices, int32_t* nnz,
                           hipStream_t s);

hipError_t launch_combine(const void* y, const int32_t* pos, const void* x, const void* shared,
                          int dtype, int64_t T, int64_t d, int k, void* out, hipStream_t s);
// Combine over the two K-split partial planes (y0, y0 + rows_max * d), dtype.
hipError_t launch_combine_split(const void* y0, int64_t rows_max, const int32_t* pos, const void* x,
                                const void* shared, int dtype, int64_t T, int64_t d, int k,
                                void* out, hipStream_t s);

struct AtomicArgs {
  const void* xhat; int dtype; int64_t T, d; int k; int64_t N;
  const void* W; const void* V; int act;
  const int32_t* ids; const int32_t* pos; const int32_t* row_token; const int32_t* row_expert;
  const float* row_r; const float* row_w;
  const int32_t* rows_used;   // device: rows in use (offsets[E])
  int64_t rows;               // host upper bound on rows
  float* a_rows;   // [rows] workspace: gated activation per task
  void* routed;    // [T, d]
};
hipError_t launch_atomic(const AtomicArgs& a, hipStream_t s);

}  // namespace moe
