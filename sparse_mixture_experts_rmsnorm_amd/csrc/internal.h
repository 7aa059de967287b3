// Host-side launchers implemented in the .hip files; called by api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gemm_args.h"

namespace moe {

// MXFP8 (gemm_mx.hip): bf16 rows [R, K] (row stride lds) -> E4M3 codes
// [R, K] (stride ldc) and E8M0 scales [R, K / 32] (stride ldsc); the GEMM.
// Output row r reads source row map[r] (map NULL: r; -1: zeros); rows at or
// past *rows_used (when given) are left untouched.
// sstage > 0: the scales stage-major instead, the four bytes of row r in
// the 128-element K stage s at s * sstage + 4 r (the GEMM's activation
// operand; K a multiple of 128).
hipError_t launch_quant_mx(const void* src, int64_t R, int64_t K, int64_t lds, const int32_t* map,
                           const int32_t* rows_used, void* codes, int64_t ldc, void* scales,
                           int64_t ldsc, int64_t sstage, hipStream_t s);
hipError_t launch_gemm_mx(const MxGemmArgs& m, int grid, hipStream_t s);

hipError_t launch_pack_transpose(const void* src, int dtype, int64_t K, int64_t N, void* dst,
                                 hipStream_t s);
hipError_t launch_pack_swiglu(const void* w1, const void* w3, int dtype, int64_t d, int64_t F,
                              const int32_t* foff_dev, const int64_t* sizes_host, int64_t E,
                              void* dst, hipStream_t s);

hipError_t launch_rmsnorm(const void* x, int dtype, int64_t T, int64_t d, const void* gamma,
                          float eps, float* r, void* xg, hipStream_t s);
// Noise and statistics of the dense router (all nullable).  part_p /
// part_g / part_c: per-workgroup partial sums [blocks][E] (workspace).
struct RouterExtras {
  const float* noise = nullptr;
  float noise_std = 0.f;
  float* part_p = nullptr;
  float* part_g = nullptr;
  int* part_c = nullptr;
  float* sum_p = nullptr;       // [E] workspace: per-expert totals
  float* sum_g = nullptr;
  long long* sum_c = nullptr;
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

// Sets the message moe_last_error() returns and gives back `code` (for
// entry points outside api.cpp).
int report_error(int code, const char* msg);

struct AtomicArgs {
  const void* xhat; int dtype; int64_t T, d; int k; int64_t N;
  const void* W; const void* V; int act;
  const int32_t* ids; const int32_t* pos; const int32_t* row_token; const int32_t* row_expert;
  const float* row_r; const float* row_w;
  const int32_t* rows_used;   // device: rows in use (offsets[E])
  int64_t rows;               // host upper bound on rows
  float* a_rows;   // [rows] workspace: gated activation per task
  void* routed;    // [T, d]
  // token-centric form (one pass per token over its slots, no task list):
  // the router's gates and the RMSNorm statistic by token
  int token_centric = 0;
  const float* w_tok = nullptr;   // [T, k]
  const float* r_tok = nullptr;   // [T]
  int32_t* errors = nullptr;      // device, nullable: += slots with ids outside [0, N)
};
hipError_t launch_atomic(const AtomicArgs& a, hipStream_t s);

// ---- backward pass (backward.hip)
// out[base_e + m, j] = rscale[row] * src[rowmap[row], m], row = offsets[e] + j,
// for j < rows_e (zero rows past the map's -1 and for rows_e <= j <
// pad64(rows_e)), m < width_e: width_e = wfix (base e * wfix) when wfix > 0,
// else wmul * f_e (base wmul * foff[e]).  offsets NULL: one segment of
// dense_rows rows.  Every width is a multiple of 64.
struct GatherTArgs {
  const uint16_t* src; int64_t lds;
  const int32_t* rowmap;    // NULL: the row itself
  const float* rscale;      // NULL: 1
  const int32_t* offsets; int dense_rows; int E;
  const int32_t* foff; int wmul; int wfix;
  uint16_t* out; int64_t ldo;
};
hipError_t launch_gather_t(const GatherTArgs& a, int max_width, int max_rows, int units,
                           hipStream_t s);
// Activation backward over expert segments (offsets NULL: one segment of
// dense_rows rows); foff gives each segment's hidden units (multiples of 64).
struct ActBwdArgs {
  const uint16_t* t; int64_t ldt;       // [rows, Fmax] dout . w2^T (ungated)
  const uint16_t* h; int64_t ldh;       // saved h
  const uint16_t* pre; int64_t ldpre;   // saved pre-activations (packed order)
  const float* row_w; const float* row_r;
  const int32_t* offsets; int dense_rows; int E;
  const int32_t* foff; int swiglu; int act;
  uint16_t* dpre; int64_t lddp;         // [rows, pf Fmax]
  uint16_t* dpreT; uint16_t* hT; int64_t ldo;
  float* part; int64_t ldpart;          // [rows, 2 ceil(Fmax / 64)]
};
hipError_t launch_act_bwd(const ActBwdArgs& a, int max_units, int max_rows, int units,
                          hipStream_t s);
// Weight-gradient tiles: X rows xmul * foff[e] .. xmul * foff[e+1] (or xfix
// rows from 0), W rows e * wstride + [0, d), K = pad64(rows of segment e).
struct WgradPlanArgs {
  const int32_t* offsets; int dense_rows; int E;
  const int32_t* foff; int xmul; int xfix;
  int wstride; int d;
  int tile;                 // tile edge: 128 or 256
  Tile* tiles; int* ntiles; int max_tiles;
};
hipError_t launch_plan_wgrad(const WgradPlanArgs& p, hipStream_t s);
hipError_t launch_reduce_part(const float* part, int64_t ldpart, int64_t rows,
                              const int32_t* row_expert, const int32_t* foff, int dense_nft,
                              float* dg_row, float* dr_row, hipStream_t s);
hipError_t launch_colsum(const float* in, int64_t n, int64_t ld, int64_t cols, float* out,
                         hipStream_t s);
struct RouterBwdArgs {
  int64_t T, Tpad; int E, k, renorm;
  const float* logits; const int32_t* ids; const float* w; const int32_t* pos;
  const float* dg_row; const float* bias; const float* r;
  float* dl; uint16_t* dlT; int64_t ldt; float* dr;
};
hipError_t launch_router_bwd(const RouterBwdArgs& a, hipStream_t s);
struct TokenBwdArgs {
  int64_t T, d; int k, E, residual;
  const uint16_t* x; const uint16_t* dout; const uint16_t* gamma; const float* r;
  const int32_t* pos; const float* dxperm; int ksplit; int64_t plane; const float* dr_row;
  const float* dxs; const float* dr_shared;
  const float* dl; const uint16_t* wr; const float* dr_router;
  uint16_t* dx; float* dgamma_part;   // [token_bwd_blocks(T), d] or NULL
};
int token_bwd_blocks(int64_t T);
hipError_t launch_token_bwd(const TokenBwdArgs& a, hipStream_t s);
// Slot counters of a layer that runs no dispatch (its router's ids are in
// range by construction): rows = n, dropped = 0, max_load = -1, errors = 0.
hipError_t launch_slot_stats(int64_t n, void* stats, hipStream_t s);

}  // namespace moe
