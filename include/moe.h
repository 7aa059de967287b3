/*
 * moe.h -- C ABI of libmoe_mi355x.so: the forward pass of one sparse
 * mixture-of-experts FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The pass (and the pages that define each step):
 *   1. RMSNorm statistic r[t] = (mean_i x[t,i]^2 + eps)^-1/2.  Following the
 *      CODA sparse-MoE thread (the paragraph on commuting the RMSNorm scale
 *      across the GEMM), r is never applied to the activations: it multiplies
 *      the fp32 accumulator in the epilogue of every GEMM that consumes the
 *      normed input (the router and the first expert linear).
 *   2. Router GEMM + top-k gating ("Mixture of Experts (MoE)" glossary:
 *      gating network, top-k / switch routing), or the Cartesian-product
 *      router of the OmniMoE summary (section 2.2).
 *   3. Expert capacity (glossary, expert-capacity entry) and dispatch: a
 *      histogram, a prefix sum and a stable permutation of the (token, slot)
 *      assignments into expert-contiguous order.  The dispatch carries r and
 *      the gate with every permuted row (CODA thread: r travels with the
 *      tokens to the experts).
 *   4. Expert FFNs as grouped GEMMs, or walked over the block-sparse (BCSR)
 *      topology of the "Variable-size experts" nanoMOE notes (sections 3-4),
 *      or as atomic experts (OmniMoE 2.1) scheduled expert-centrically
 *      (OmniMoE 2.2).  Always-on shared experts are a one-group GEMM.
 *   5. Combine: the gated expert outputs summed back into token order.
 *
 * Conventions
 *   - Every pointer is a DEVICE pointer unless marked [host].
 *   - Nothing allocates device memory: the caller owns every buffer and
 *     passes a workspace sized by the matching *_workspace_size call.
 *   - All work is enqueued on the given stream; no call synchronises with
 *     the host, so a whole layer can be captured in a HIP graph.  Inputs and
 *     weights are never written.
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns a negative MOE_E* code, leaves every output untouched
 *     and sets the message returned by moe_last_error().  No silent fallback:
 *     an unsupported case returns MOE_EUNSUPPORTED.
 *   - Data errors found on the device (an expert id out of range) are counted
 *     in moe_stats.errors; the offending slot is dropped.
 *   - Calls are reentrant as long as callers use distinct workspaces and
 *     outputs.
 *   - Indices are int32 (the nanoMOE notes' int16 indices overflowed; see the
 *     output-array-indexing bug-fix section there).
 *
 * Data types: MOE_F32 (everything fp32) or MOE_BF16 (activations, weights,
 * hidden h, expert outputs and the layer output stored as bf16 with
 * round-to-nearest-even; r, logits, gates and every accumulator fp32).
 *
 * Weight layouts.  The pages store w1, w3 as [d, sum f] and w2 as [sum f, d]
 * with one slice per expert ("Variable-size experts", weight allocation).
 * The kernels read every operand K-contiguous, so a one-time pack converts
 * them (moe_pack_*; not part of the per-token work):
 *   router        w_router [d, E]    -> wr_t  [E, d]
 *   Cartesian     k_rows [d, Nr], k_cols [d, Nc] -> keys_t [Nr + Nc, d]
 *   GELU experts  w1 [d, F]          -> w13_t [F, d]       (F = sum f_e)
 *   SwiGLU        w1, w3 [d, F]      -> w13_t [2F, d], per expert in groups
 *                 of 32 rows: 32 rows of w1^T then the same 32 rows of w3^T
 *   all experts   w2 [F, d]          -> w2_t  [d, F]
 *   atomic        W, V [N, d]        used as given (rows are K-contiguous)
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---- */
enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* null pointer or out-of-range scalar            */
  MOE_ESHAPE = -2,        /* sizes inconsistent or not a supported multiple */
  MOE_EDTYPE = -3,        /* unknown dtype / activation / kind              */
  MOE_EUNSUPPORTED = -4,  /* valid request this build does not implement    */
  MOE_EWORKSPACE = -5,    /* workspace null or smaller than required        */
  MOE_EHIP = -6           /* a HIP runtime call failed                      */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };
enum { MOE_ACT_GELU = 0, MOE_ACT_GELU_TANH = 1, MOE_ACT_SWIGLU = 2 };
enum { MOE_ROUTER_DENSE = 0, MOE_ROUTER_CARTESIAN = 1 };
enum { MOE_EXPERTS_GROUPED = 0, MOE_EXPERTS_BCSR = 1, MOE_EXPERTS_ATOMIC = 2 };
enum { MOE_QUANT_NONE = 0, MOE_QUANT_MXFP8 = 1 };

/* Counters written by moe_dispatch (device memory, overwritten each call).
 * A layer of ATOMIC experts runs no dispatch: it writes rows = T*k slots,
 * dropped = 0, max_load = -1 (not counted) and errors = 0 (its Cartesian
 * router produces ids in range by construction). */
typedef struct moe_stats {
  int32_t rows;      /* permuted rows in use: offsets[E]                     */
  int32_t dropped;   /* (token, slot) assignments over capacity              */
  int32_t max_load;  /* largest per-expert count before the capacity rule    */
  int32_t errors;    /* expert ids out of [0, E) (those slots are dropped)   */
} moe_stats;

/* Router.  DENSE: logits l[t,e] = r[t] * (xhat[t] . W_r[:,e]) + bias[e].
 * CARTESIAN (OmniMoE 2.2): E = Nr * Nc experts on a row-major grid,
 * expert n = i*Nc + j scores s1[t,i] + s2[t,j] with s1 = r * xhat.K_rows and
 * s2 = r * xhat.K_cols. */
typedef struct moe_router_desc {
  int kind;               /* MOE_ROUTER_DENSE or MOE_ROUTER_CARTESIAN        */
  int64_t E;              /* number of experts (CARTESIAN: Nr * Nc)          */
  const void* wr_t;       /* DENSE: packed router [E, d], dtype of x         */
  const float* bias;      /* DENSE: [E] fp32 or NULL                         */
  int64_t Nr, Nc;         /* CARTESIAN grid                                   */
  const void* keys_t;     /* CARTESIAN: packed [Nr + Nc, d], dtype of x      */
} moe_router_desc;

/* Experts.
 * GROUPED: expert e has ffn_sizes[e] hidden units; weights packed as above.
 * BCSR:    same weights, but the GEMMs walk a BCSR topology built by
 *          moe_build_topology over block x block tiles (dispatch pad = block).
 * ATOMIC:  N = E single-unit experts: routed[t] = sum_j g * act(r xhat.W[n]) V[n].
 * Constraints (else MOE_ESHAPE): d % 256 == 0 for bf16 (d % 64 for f32);
 * every ffn size a multiple of 128 (of 32 for f32); ATOMIC d % 512 == 0.
 * The bf16 GEMMs address each operand array (the GEMM rows, x or its
 * gathered token rows, the hidden activation h, each packed weight matrix)
 * with 32-bit byte offsets: each must stay below 4 GiB, else the GEMM's
 * launch is refused and the call returns MOE_EHIP (invalid argument). */
typedef struct moe_experts_desc {
  int kind;                     /* MOE_EXPERTS_*                             */
  int act;                      /* MOE_ACT_* (ATOMIC: GELU or GELU_TANH)     */
  int64_t E;                    /* experts                                    */
  const int64_t* ffn_sizes;     /* [host] [E] hidden sizes (not ATOMIC)      */
  const int32_t* ffn_offsets;   /* [E+1] device copy of their prefix sum     */
  const void* w13_t;            /* packed first linear(s)                    */
  const void* w2_t;             /* packed second linear [d, F]               */
  int64_t w2_ld;                /* row stride of w2_t in elements; 0: F.
                                 * >= F, a multiple of 16 bytes, d * w2_ld
                                 * below 2 GiB for MXFP8.  The MXFP8 second
                                 * linear ran 13% faster on a Mixtral-sized
                                 * layer with F + 256 (what the layer uses)
                                 * than with F = 114688, where every row
                                 * starts on the same low 14 address bits    */
  const void* W;                /* ATOMIC: [E, d]                             */
  const void* V;                /* ATOMIC: [E, d]                             */
  int block;                    /* BCSR block size (128)                     */
  /* BCSR per-expert block buffers (device, int32) and the topology built by
   * moe_build_topology; ignored for the other kinds.  moe_layer_forward
   * builds the topology itself (in its workspace) and ignores the last two. */
  const int32_t* size_blocks;   /* [E] f_e / block                            */
  const int32_t* block_offsets; /* [E+1] prefix sum of size_blocks            */
  const int32_t* row_offsets;   /* [rows_max/block + 1] CSR row pointer       */
  const int32_t* column_indices;/* [nnz_max] column block of each nonzero     */
  /* MOE_QUANT_MXFP8 (GROUPED or BCSR, bf16 layers only): w13_t and w2_t hold E4M3
   * codes (one byte per element, same packed layouts) and w13_scale,
   * w2_scale their E8M0 block scales in the stage-major layout written by
   * moe_pack_mxfp8_weights from the bf16 packs: w13_scale [d/128][P][4],
   * w2_scale [F/128][d][4] (P = F, or 2F for SwiGLU).  Following the CODA
   * thread's point that low-precision conversions are free in epilogues, the
   * expert rows are quantised once per (token, slot) as they are gathered,
   * the first linear's epilogue writes the hidden activation h as MXFP8, and
   * both GEMMs run on the scaled MFMA with fp32 accumulators; r, gates,
   * expert outputs and the layer output stay as in the bf16 path.  Needs
   * every ffn size a multiple of 128.  MOE_QUANT_NONE: the fields below are
   * ignored. */
  int quant;
  const uint8_t* w13_scale;
  const uint8_t* w2_scale;
  /* Needed by moe_layer_backward only (GROUPED / BCSR, bf16): the second
   * linear as the pages store it, w2 [F, d] (= w2_t transposed), and the
   * packed first linear transposed, w13_dk [d, P] (moe_pack_transpose of
   * w13_t viewed as [P, d]).  Ignored by the forward calls. */
  const void* w2_fk;
  const void* w13_dk;
} moe_experts_desc;

/* Results of moe_dispatch, consumed by moe_expert_gemm and moe_combine. */
typedef struct moe_routing {
  int64_t T;                 /* tokens                                         */
  int k;                     /* slots per token                                */
  int64_t E;                 /* experts                                        */
  int64_t rows_max;          /* capacity of the permuted-row buffers           */
  int pad;                   /* row padding per expert (1 or the BCSR block)   */
  const int32_t* ids;        /* [T, k] expert of each slot                     */
  const float* w;            /* [T, k] gate of each slot                       */
  const float* r;            /* [T] RMSNorm statistic                          */
  const int32_t* counts;     /* [E] load before the capacity rule              */
  const int32_t* offsets;    /* [E+1] first permuted row of each expert        */
  const int32_t* pos;        /* [T, k] permuted row of each slot, -1 = dropped */
  const int32_t* row_token;  /* [rows_max] token of each row, -1 = padding     */
  const float* row_r;        /* [rows_max] r of the row's token (0 on padding) */
  const float* row_w;        /* [rows_max] gate of the row (0 on padding)      */
  const int32_t* row_expert; /* [rows_max] expert of the row, -1 = padding     */
} moe_routing;

typedef struct moe_timer moe_timer;  /* opaque per-stage hipEvent timer */

/* Stages timed by a moe_timer attached to moe_layer_forward. */
enum {
  MOE_STAGE_ROUTER = 0,   /* RMSNorm statistic + router + top-k             */
  MOE_STAGE_DISPATCH,     /* histogram, scan, rank, gather                  */
  MOE_STAGE_PLAN,         /* topology / GEMM tile lists                     */
  MOE_STAGE_GEMM1,        /* first expert linear + r-scale + activation     */
  MOE_STAGE_GEMM2,        /* second expert linear + gate                    */
  MOE_STAGE_SHARED,       /* always-on shared experts                       */
  MOE_STAGE_COMBINE,      /* weighted sum back to token order               */
  MOE_STAGE_COUNT
};

/* Router extras (dense router): noise top-k and routing statistics.
 * Glossary "Mixture of Experts (MoE)": the gating-network entry (noise
 * top-k: tunable Gaussian noise added to the logits before selection) and
 * the load-balancing / auxiliary-loss entries (the squared coefficient of
 * variation of the routing probability across experts); the CODA thread's
 * point that metrics ride in epilogues.  All pointers are device pointers
 * and may be NULL.  The noise is an input: the caller draws it.  With noise,
 * selection, gates, the logits output and the statistics all use
 * logits + noise_std * noise.  Statistics are summed per workgroup and then
 * over workgroups in a fixed order, so they are deterministic. */
typedef struct moe_router_extras {
  const float* noise;   /* [T, E] fp32 standard-normal draws, or NULL        */
  float noise_std;      /* scale of the noise                                */
  float* prob_sum;      /* [E] out: sum over tokens of the full-softmax
                           router probability of each expert                */
  float* gate_sum;      /* [E] out: sum over tokens of the gate each expert
                           receives in the selected slots                   */
  float* aux;           /* [3] out: squared CV across experts (population
                           variance / mean^2) of prob_sum (the auxiliary
                           load loss), of gate_sum, and of the per-expert
                           slot counts (before capacity); NaN for a zero
                           mean                                              */
} moe_router_extras;

typedef struct moe_layer_desc {
  int64_t d;                       /* model width                              */
  int dtype;                       /* MOE_F32 or MOE_BF16                      */
  const void* gamma;               /* [d] RMSNorm gain (dtype) or NULL = 1     */
  float eps;                       /* RMSNorm epsilon                          */
  moe_router_desc router;
  int k;                           /* experts per token                        */
  int renorm;                      /* 1: softmax over the k selected logits;
                                      0: full-softmax probability              */
  double capacity_factor;          /* <= 0: no capacity limit                  */
  moe_experts_desc experts;
  const moe_experts_desc* shared;  /* [host] always-on shared FFN or NULL:
                                      kind GROUPED, E = 1, gate 1             */
  int residual;                    /* 1: out includes x (dropped tokens pass
                                      through); 0: experts only                */
  moe_timer* timer;                /* NULL, or per-stage event timing          */
  const moe_router_extras* router_extras;  /* [host] NULL, or noise / statistics
                                               of the dense router            */
  int save_for_backward;           /* 1: moe_layer_forward also keeps in its
                                      workspace what moe_layer_backward needs
                                      (pre-activations, router logits); bf16,
                                      dense router, unquantised grouped or
                                      BCSR experts only                       */
} moe_layer_desc;

/* Gradients written by moe_layer_backward (device pointers; fp32 unless
 * noted).  Weight gradients are in the layouts the forward reads (packed
 * rows are features, K = d contiguous), so that an optimizer updates the
 * packed weights in place:
 *   dw13  [P, d]  gradient of w13_t (P = F, or 2F for SwiGLU)
 *   dw2   [F, d]  gradient of the pages' w2 (the transpose of w2_t)
 *   dw_router [E, d]  gradient of wr_t
 * Every pointer that applies is required: dbias with a router bias, dgamma
 * with a gain, dws13 / dws2 with shared experts. */
typedef struct moe_layer_grads {
  void* dx;          /* [T, d] dtype                                          */
  float* dgamma;     /* [d]                                                   */
  float* dw_router;  /* [E, d]                                                */
  float* dbias;      /* [E]                                                   */
  float* dw13;       /* [P, d]                                                */
  float* dw2;        /* [F, d]                                                */
  float* dws13;      /* [P_s, d]                                              */
  float* dws2;       /* [F_s, d]                                              */
} moe_layer_grads;

/* Last error message of the calling thread ("" after success). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

/* [host] Expert capacity, glossary expert-capacity entry:
 * ceil(T*k*cf/E) evaluated exactly for the binary value of cf, clamped to
 * [0, T]; cf <= 0 means no limit and returns T.  Returns -1 on bad input. */
int64_t moe_capacity(int64_t T, int k, int64_t E, double cf);

/* [host] Rows the permuted buffers must hold: min(T*k, E*capacity) plus
 * E*(pad-1) for padding.  -1 on bad input. */
int64_t moe_rows_max(int64_t T, int k, int64_t E, int64_t capacity, int pad);

/* ---- weight packing (one-time; see the layout note above) ---- */

/* dst[n, kk] = src[kk, n] for a [K, N] source (dtype elements). */
int moe_pack_transpose(const void* src, int dtype, int64_t K, int64_t N, void* dst,
                       hipStream_t stream);

/* SwiGLU pack: w1, w3 [d, F] -> w13_t [2F, d] interleaved per expert in
 * groups of 32 rows (ffn_sizes [host] [E], each a multiple of 32). */
int moe_pack_swiglu(const void* w1, const void* w3, int dtype, int64_t d,
                    const int64_t* ffn_sizes, int64_t E, void* w13_t, hipStream_t stream);

/* MXFP8 pack (OCP Microscaling format, MXFP8 with E4M3 elements): each row
 * of the bf16 matrix src [R, K] (row stride lds elements) is cut into blocks
 * of 32 consecutive elements; a block's shared exponent is
 * s = floor(log2(max |v|)) - 8 (the largest E4M3 normal is 1.75 * 2^8),
 * clamped to [-127, 127] (-127 for an all-zero block), stored as the E8M0
 * byte s + 127 in scales [R, K/32] (row stride ldsc bytes); its elements are
 * stored as the E4M3 code (bias 7, 3 mantissa bits, subnormals on the 2^-9
 * grid) of v * 2^-s rounded to nearest-even, magnitudes of 448 and above
 * saturated to 448, in codes [R, K] (row stride ldc bytes).  K % 32 == 0,
 * ldc % 8 == 0.  The layer quantises its activations with the same kernel;
 * the expert weights take moe_pack_mxfp8_weights (below), which writes the
 * same values with the scales in the GEMMs' layout. */
int moe_pack_mxfp8(const void* src, int64_t R, int64_t K, int64_t lds, void* codes, int64_t ldc,
                   void* scales, int64_t ldsc, hipStream_t stream);

/* MXFP8 pack of packed expert weights (w13_t [P, d] or w2_t [d, F], bf16) for
 * the expert GEMMs: the same codes and block scales as moe_pack_mxfp8 (same
 * format and rounding), with the scales stored stage-major, scales
 * [K/128][R][4]: the E8M0 byte of row r for elements 32 j .. 32 j + 31 at
 * byte 4 (floor(j/4) R + r) + j % 4, so that the four scales of one row
 * over 128 consecutive elements form one 32-bit word and the words of
 * consecutive rows are adjacent (a 256-row weight tile's scales for one
 * 128-element K step are 1 KB of contiguous bytes).  This is the layout
 * moe_experts_desc.w13_scale and w2_scale hold.  K % 128 == 0, lds and ldc
 * multiples of 8, src 16-byte and codes 8-byte aligned; scales holds
 * R * K / 32 bytes (below 2 GiB).  Errors: MOE_ESHAPE, MOE_EINVAL. */
int moe_pack_mxfp8_weights(const void* src, int64_t R, int64_t K, int64_t lds, void* codes,
                           int64_t ldc, void* scales, hipStream_t stream);

/* ---- step 1: RMSNorm statistic ----
 * r[T] fp32.  If gamma is non-NULL, also writes xg[T, d] = x * gamma (dtype,
 * rounded once), the input of the GEMMs that follow. */
int moe_rmsnorm_stats(const void* x, int dtype, int64_t T, int64_t d, const void* gamma,
                      float eps, float* r, void* xg, hipStream_t stream);

/* ---- step 2: router + top-k ----
 * x is the GEMM input xhat (x, or xg when a gain is used).  If r_in is NULL
 * the statistic is computed from x in the same pass (valid only without a
 * gain) and written to r_out; otherwise r_in is used.  Writes ids [T, k]
 * (int32, slot 0 = best, ordered by logit descending with ties to the lower
 * expert index), w [T, k] gates (renorm as in moe_layer_desc), and, when
 * non-NULL, logits: DENSE [T, E]; CARTESIAN [T, Nr + Nc] = (s1 | s2).
 * DENSE supports E <= 256 and k <= E; f32 needs logits (non-NULL).
 * CARTESIAN needs k <= 64, Nr, Nc >= k, Nr + Nc a multiple of 256.  Both
 * take a workspace of moe_router_workspace_size bytes (DENSE: room for the
 * per-workgroup statistics of moe_router_topk_ex). */
size_t moe_router_workspace_size(const moe_router_desc* R, int64_t T);
int moe_router_topk(const moe_router_desc* R, const void* x, int dtype, int64_t T, int64_t d,
                    const float* r_in, float eps, float* r_out, int k, int renorm,
                    int32_t* ids, float* w, float* logits, void* ws, size_t ws_bytes,
                    hipStream_t stream);
/* moe_router_topk with extras [host, may be NULL]: noise top-k and the
 * routing statistics of moe_router_extras.  DENSE router only, k <= 64;
 * otherwise MOE_EUNSUPPORTED when any extra is requested. */
int moe_router_topk_ex(const moe_router_desc* R, const void* x, int dtype, int64_t T, int64_t d,
                       const float* r_in, float eps, float* r_out, int k, int renorm,
                       int32_t* ids, float* w, float* logits,
                       const moe_router_extras* extras, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* ---- step 3: capacity + dispatch ----
 * Deterministic and stable: within an expert, slots keep token order; a
 * slot whose rank reaches `capacity` is dropped (pos = -1).  offsets is the
 * exclusive prefix sum of min(counts, capacity) each rounded up to `pad`.
 * row_token/row_r/row_w/row_expert (row_expert may be NULL) are written for
 * all rows_max rows (-1/0/0/-1 beyond the rows in use and on padding).
 * x_perm [rows_max, d] receives the token rows (zero rows on padding); pass
 * NULL for index-only dispatch.  E > 2048 switches to a two-pass LSD radix
 * sort of the slots by expert id (the expert-centric task sort of OmniMoE
 * 2.2); that path needs pad == 1 and no capacity limit (capacity >= T) and
 * supports E < 2^22. */
size_t moe_dispatch_workspace_size(int64_t T, int k, int64_t E);
int moe_dispatch(const int32_t* ids, const float* w, const float* r, const void* x, int dtype,
                 int64_t T, int64_t d, int64_t E, int k, int64_t capacity, int pad,
                 int64_t rows_max, int32_t* counts, int32_t* offsets, int32_t* pos,
                 int32_t* row_token, float* row_r, float* row_w, int32_t* row_expert,
                 void* x_perm, moe_stats* stats, void* ws, size_t ws_bytes,
                 hipStream_t stream);

/* ---- allocation-free dispatch ----
 * For callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same operation, checks, outputs and error codes as moe_dispatch, with the
 * workspace replaced by a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * that each GPU the library runs on holds until the process ends (its
 * address is looked up on the first call on each device).  No call
 * allocates.  A (T, k, E) whose moe_dispatch_workspace_size exceeds
 * MOE_NOALLOC_SCRATCH_BYTES returns MOE_EWORKSPACE with a message naming
 * both sizes (8 MiB covers every dense dispatch with E * ceil(T / 256) below
 * about two million, and the radix dispatch of up to about 300k slots).
 * Calls on one GPU share its array: calls that overlap on one GPU (streams
 * with no ordering between them) race; calls ordered on one stream do not. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_dispatch_noalloc(const int32_t* ids, const float* w, const float* r, const void* x,
                         int dtype, int64_t T, int64_t d, int64_t E, int k, int64_t capacity,
                         int pad, int64_t rows_max, int32_t* counts, int32_t* offsets,
                         int32_t* pos, int32_t* row_token, float* row_r, float* row_w,
                         int32_t* row_expert, void* x_perm, moe_stats* stats,
                         hipStream_t stream);

/* ---- BCSR topology ("Variable-size experts", sections 3-4) ----
 * From offsets [E+1] (padded to `block`), size_blocks [E] and block_offsets
 * [E+1] build row_offsets [rows_max/block + 1] and column_indices: token
 * block y of expert e gets column blocks block_offsets[e] ..
 * block_offsets[e] + size_blocks[e] - 1, written at the exclusive prefix sum
 * over experts of token_blocks * size_blocks (never a uniform stride).
 * nnz (one device int32) receives the nonzero count; row_offsets is filled
 * with the final count past the last row block in use. */
int64_t moe_topology_nnz_max(int64_t rows_max, int block, const int64_t* ffn_sizes /*[host]*/,
                             int64_t E);
int moe_build_topology(const int32_t* offsets, const int32_t* size_blocks,
                       const int32_t* block_offsets, int64_t E, int block, int64_t rows_max,
                       int32_t* row_offsets, int32_t* column_indices, int32_t* nnz,
                       hipStream_t stream);

/* ---- step 4: expert FFNs ----
 * GROUPED / BCSR: x_in = x_perm [rows_max, d]; y = y_perm [rows_max, d],
 *   y[row] = row_w[row] * FFN_e(row_r[row] * x_perm[row]) for rows in use
 *   (the gate and r epilogues; rows past offsets[E] are not written).
 * ATOMIC: x_in = xhat [T, d]; y = routed [T, d],
 *   routed[t] = sum_j w[t,j] * act(r[t] xhat[t].W[n]) V[n], n = ids[t,j],
 *   summed in slot order.  With the dispatch's task list (row_expert, sorted
 *   by expert as OmniMoE 2.2 schedules it) the two-phase expert-centric
 *   form runs; with row_expert NULL the single-pass token-centric form runs
 *   from ids, w and r alone (moe_layer_forward uses it).  Both give the same
 *   bits.  A slot whose id lies outside [0, N) is dropped (no row is read)
 *   and added to stats->errors (stats nullable; the count is added to what
 *   stats holds, never reset here); a task row whose token lies outside
 *   [0, T) is dropped.  The workspace holds the hidden activations, the
 *   device-built tile lists and, for bf16 experts whose second linear cuts
 *   its last round of tiles along K, the pieces' fp32 partial sums (added in
 *   a fixed order, so y is rounded to the dtype once and repeats bit for bit).
 * stats is not used by the GROUPED / BCSR kinds (they read no expert ids). */
size_t moe_expert_workspace_size(const moe_experts_desc* X, int dtype, int64_t d,
                                 int64_t T, int k, int64_t rows_max);
int moe_expert_gemm(const moe_experts_desc* X, int dtype, int64_t d, const moe_routing* rt,
                    const void* x_in, void* y, moe_stats* stats, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Always-on shared FFN over all T tokens with gate 1 (one expert, kind
 * GROUPED): s[t] = FFN(r[t] * xhat[t]). */
size_t moe_shared_workspace_size(const moe_experts_desc* S, int dtype, int64_t d, int64_t T);
int moe_shared_ffn(const moe_experts_desc* S, int dtype, int64_t d, int64_t T, const void* xhat,
                   const float* r, void* s, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- step 5: combine ----
 * "Mixture of Experts (MoE)" glossary: the layer output is the sum of the
 * selected experts' outputs weighted by their router scores (gating-network
 * and top-k entries), and a token that overflows every chosen expert's
 * capacity skips the experts and passes through unchanged (expert-capacity
 * and dropped-token entries); OmniMoE summary 2.1: the shared dense MLP's
 * output is added to the routed branch.  The gate is already applied by the
 * second expert linear's epilogue, so here:
 *   out[t] = x[t] + shared[t] + sum_{j : pos[t,j] >= 0} y[pos[t,j]],
 * summed in fp32 in exactly that order and stored once.
 *   y        [rows_max, d] expert outputs in permuted order (dtype), or with
 *            pos == NULL [T, d] in token order (the atomic branch);
 *   pos      [T, k] int32 rows of the token's slots, -1 = dropped;
 *   residual [T, d] (nullable: no residual), shared [T, d] (nullable);
 *   out      [T, d], fully overwritten; may not alias y.
 * A token whose slots are all dropped gets out = x bit-exactly.  Errors:
 * MOE_EDTYPE for an unknown dtype, MOE_ESHAPE for T < 0, d < 1, k < 1 or a
 * row that does not fill 16-byte vectors, MOE_EUNSUPPORTED for k > 256,
 * MOE_EINVAL for a NULL y / out with T > 0. */
int moe_combine(const void* y, const int32_t* pos, const void* residual, const void* shared,
                int dtype, int64_t T, int64_t d, int k, void* out, hipStream_t stream);

/* ---- the whole layer ----
 * The forward pass the pages compose: the CODA sparse-MoE thread's RMSNorm
 * with the r-scale commuted into the router's and the first expert linear's
 * epilogues, the glossary's gating network with top-k / switch routing and
 * the expert-capacity rule, the dispatch (the glossary's fused-MoE-kernels
 * entry: routing, permutation and expert GEMMs without host round trips),
 * the expert FFNs (grouped, the nanoMOE notes' variable-size BCSR walk, or
 * OmniMoE 2.1 atomic experts behind the 2.2 Cartesian router), the shared
 * experts (OmniMoE 2.1) and the combine above.  Steps 1-5 run on `stream`
 * with every tile list built on the device: no host read-back of the loads.
 *   L     [host] layer descriptor (weights packed as described at the top);
 *   x     [T, d] in L->dtype; out [T, d], fully overwritten (not aliasing x);
 *   stats nullable: rows, dropped slots, max load, data errors (int32 x 4);
 *   ws    moe_layer_workspace_size(L, T) bytes, caller-owned; it also keeps
 *         the routing for moe_layer_routing and, with save_for_backward,
 *         what moe_layer_backward reads.
 * Errors (nothing enqueued): MOE_EINVAL / MOE_ESHAPE for a bad descriptor or
 * T < 0, MOE_EWORKSPACE when ws_bytes is too small, MOE_EUNSUPPORTED for a
 * combination no kernel covers, MOE_EHIP for a failed launch. */
size_t moe_layer_workspace_size(const moe_layer_desc* L, int64_t T);
int moe_layer_forward(const moe_layer_desc* L, const void* x, int64_t T, void* out,
                      moe_stats* stats, void* ws, size_t ws_bytes, hipStream_t stream);

/* Read back the routing of the last moe_layer_forward on this workspace:
 * fills *rt with pointers into ws (valid until the workspace is reused). */
int moe_layer_routing(const moe_layer_desc* L, int64_t T, void* ws, size_t ws_bytes,
                      moe_routing* rt);

/* ---- backward pass ----
 * CODA thread, the paragraph on the backward: the RMSNorm backward is fused
 * into the backward of the linear that consumed the normed input, using the
 * saved r.  For an upstream gradient dout [T, d] of the layer output, after
 * moe_layer_forward(L with save_for_backward = 1, x, T, ...) on the same
 * fwd_ws (untouched since), writes the gradients of moe_layer_grads:
 *   expert rows:  dy = g dout,  dg = dout . y,  dh = dy w2^T,
 *                 da = dh act'(a)  (SwiGLU: da = dh u silu'(a), du = dh silu(a)),
 *                 dw2 += h^T dy,  dw13 += [da | du]^T (r xhat),
 *                 dxhat += r [da | du] w13,  dr += (xhat w13) . [da | du]
 *   shared experts: the same with gate 1 over all tokens
 *   router:       top-k selection and the capacity rule are piecewise
 *                 constant; dl from dg through the gate softmax (renorm 1:
 *                 over the k selected; renorm 0: over all E);
 *                 dw_router = dl^T (r xhat), dbias = sum_t dl,
 *                 dxhat += r dl wr, dr += (xhat wr) . dl
 *   RMSNorm:      dx = dout (residual) + gamma dxhat - (r^3 / d) dr x,
 *                 dgamma = sum_t dxhat x
 * Dropped slots get no gradient.  Needs w2_fk and w13_dk in the expert
 * descriptors; router extras with noise are not supported.  Every sum is in
 * a fixed order (deterministic).  ws: moe_layer_backward_workspace_size bytes. */
size_t moe_layer_backward_workspace_size(const moe_layer_desc* L, int64_t T);
int moe_layer_backward(const moe_layer_desc* L, const void* x, int64_t T, const void* dout,
                       const void* fwd_ws, size_t fwd_ws_bytes, const moe_layer_grads* grads,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- per-stage timing (hipEvents; the only calls here that synchronise) ---- */
int moe_timer_create(moe_timer** out, int max_calls);
int moe_timer_destroy(moe_timer* t);
int moe_timer_reset(moe_timer* t);
/* Sum over recorded calls of the elapsed time of `stage`, in ms; waits for
 * the recorded events.  *calls receives the number of calls summed. */
int moe_timer_stage_ms(moe_timer* t, int stage, double* total_ms, int* calls);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
