// Host side of libmoe_mi355x: argument checks, workspace carving and the
// launch sequence of the MoE layer forward.  Nothing here allocates device
// memory or waits for the device (except the explicit timer read-out).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"
#include "moe.h"

using namespace moe;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
int ok() {
  g_err.clear();
  return MOE_OK;
}

}  // namespace

// Error reporting for entry points defined in other source files.
int moe::report_error(int code, const char* msg) {
  g_err = msg;
  return code;
}

namespace {

#define MOE_HIP(call)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) return fail(MOE_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
size_t esize(int dtype) { return dtype == MOE_F32 ? 4 : 2; }

// Bump allocator over a caller workspace (or a null base to measure).
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += align_up(std::max<size_t>(bytes, 1));
    return p;
  }
  template <typename T> T* take_n(int64_t n) { return static_cast<T*>(take(size_t(n) * sizeof(T))); }
};

bool valid_dtype(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }

// ---------------------------------------------------------------- expert geometry

struct ExpertGeo {
  int64_t E = 0, F = 0, Fmax = 0;
  int pf = 1;          // packed rows per hidden unit in the first linear
  int bf1 = 256;       // packed weight rows per first-linear tile
  int bf2 = 256;       // output features per second-linear tile
  int bt = 256;        // GEMM rows per tile
  int bt2 = 256;       // rows per tile of the second linear (128 fills a small dense layer)
  int fold = 1;        // first-linear output columns = packed features / fold
  bool bcsr = false, atomic = false;
  bool mx = false;     // MXFP8 operands (E4M3 codes + E8M0 block scales)
  int kdiv = 1;        // largest second-linear K split (1, 2 or 4) whose parts are
                       // whole K stages of every expert
  int64_t ld2 = 0;     // row stride of w2_t (elements)
};

int check_experts(const moe_experts_desc* X, int dtype, int64_t d, ExpertGeo* g) {
  REQUIRE(X, MOE_EINVAL, "experts descriptor is NULL");
  REQUIRE(valid_dtype(dtype), MOE_EDTYPE, "unknown dtype %d", dtype);
  REQUIRE(X->kind >= MOE_EXPERTS_GROUPED && X->kind <= MOE_EXPERTS_ATOMIC, MOE_EDTYPE,
          "unknown experts kind %d", X->kind);
  REQUIRE(X->act >= MOE_ACT_GELU && X->act <= MOE_ACT_SWIGLU, MOE_EDTYPE, "unknown activation %d",
          X->act);
  REQUIRE(X->E >= 1, MOE_EINVAL, "experts E must be >= 1 (got %lld)", (long long)X->E);
  ExpertGeo geo;
  geo.E = X->E;
  geo.bcsr = X->kind == MOE_EXPERTS_BCSR;
  geo.atomic = X->kind == MOE_EXPERTS_ATOMIC;
  if (geo.atomic) {
    REQUIRE(dtype == MOE_BF16, MOE_EUNSUPPORTED, "atomic experts are implemented for bf16 only");
    REQUIRE(X->act != MOE_ACT_SWIGLU, MOE_EUNSUPPORTED, "atomic experts take GELU activations");
    REQUIRE(d == 512 || d == 1024 || d == 2048 || d == 4096, MOE_ESHAPE,
            "atomic experts need d in {512, 1024, 2048, 4096} (got %lld)", (long long)d);
    REQUIRE(X->W && X->V, MOE_EINVAL, "atomic experts need W and V");
    *g = geo;
    return MOE_OK;
  }
  REQUIRE(X->ffn_sizes, MOE_EINVAL, "ffn_sizes is NULL");
  REQUIRE(X->ffn_offsets, MOE_EINVAL, "ffn_offsets (device prefix sum) is NULL");
  REQUIRE(X->w13_t && X->w2_t, MOE_EINVAL, "packed expert weights are NULL");
  REQUIRE(X->E <= 2048, MOE_EUNSUPPORTED, "grouped / BCSR experts support E <= 2048");
  geo.pf = X->act == MOE_ACT_SWIGLU ? 2 : 1;
  if (dtype == MOE_F32) {
    REQUIRE(!geo.bcsr, MOE_EUNSUPPORTED, "the BCSR walk is implemented for bf16 only");
    REQUIRE(d % 64 == 0 && d > 0, MOE_ESHAPE, "f32 experts need d %% 64 == 0 (got %lld)", (long long)d);
    geo.bf1 = 64 * geo.pf;
    geo.bf2 = 64;
    geo.bt = 64;
  } else {
    REQUIRE(d % 256 == 0 && d > 0, MOE_ESHAPE, "bf16 experts need d %% 256 == 0 (got %lld)", (long long)d);
    geo.bf1 = 256;
    geo.bf2 = 256;
    // BCSR: tiles of two 128-row token blocks of one expert (a lone last
    // block makes a 128-row tile), so both walks run the 8-wave kernel
    geo.bt = 256;
  }
  geo.bt2 = geo.bt;
  geo.fold = geo.pf;
  for (int64_t e = 0; e < X->E; ++e) {
    const int64_t f = X->ffn_sizes[e];
    REQUIRE(f > 0, MOE_ESHAPE, "ffn_sizes[%lld] must be positive", (long long)e);
    if (dtype == MOE_F32)
      REQUIRE(f % 64 == 0, MOE_ESHAPE, "f32 ffn sizes must be multiples of 64 (expert %lld: %lld)",
              (long long)e, (long long)f);
    else
      REQUIRE((f * geo.pf) % geo.bf1 == 0, MOE_ESHAPE,
              "bf16 ffn sizes must be multiples of %d for this activation (expert %lld: %lld)",
              256 / geo.pf, (long long)e, (long long)f);
    geo.F += f;
    geo.Fmax = std::max(geo.Fmax, f);
  }
  REQUIRE(geo.F < (int64_t(1) << 31) / 2, MOE_ESHAPE, "total ffn width too large");
  REQUIRE(X->quant == MOE_QUANT_NONE || X->quant == MOE_QUANT_MXFP8, MOE_EDTYPE,
          "unknown quant %d", X->quant);
  if (X->quant == MOE_QUANT_MXFP8) {
    REQUIRE(dtype == MOE_BF16, MOE_EUNSUPPORTED,
            "MXFP8 experts are implemented for bf16 grouped and BCSR experts");
    REQUIRE(X->w13_scale && X->w2_scale, MOE_EINVAL, "MXFP8 experts need w13_scale and w2_scale");
    geo.mx = true;
    for (int64_t e = 0; e < X->E; ++e)
      REQUIRE(X->ffn_sizes[e] % 128 == 0, MOE_ESHAPE,
              "MXFP8 ffn sizes must be multiples of 128 (expert %lld: %lld)", (long long)e,
              (long long)X->ffn_sizes[e]);
    // the kernels address operands with 32-bit byte offsets
    REQUIRE(geo.F * geo.pf * d < (int64_t(1) << 31) && geo.F * d < (int64_t(1) << 31), MOE_ESHAPE,
            "MXFP8 weights must stay below 2 GiB per matrix");
  }
  geo.ld2 = X->w2_ld ? X->w2_ld : geo.F;
  {
    const int64_t eb = geo.mx ? 1 : esize(dtype);
    REQUIRE(geo.ld2 >= geo.F && (geo.ld2 * eb) % 16 == 0, MOE_ESHAPE,
            "w2_ld must be >= F (%lld) and a multiple of 16 bytes (got %lld)", (long long)geo.F,
            (long long)X->w2_ld);
    REQUIRE(!geo.mx || geo.ld2 * d < (int64_t(1) << 31), MOE_ESHAPE,
            "MXFP8 weights must stay below 2 GiB per matrix");
  }
  // K stage of the second linear: 64 elements (bf16), 128 (MXFP8)
  const int64_t kstage = geo.mx ? 128 : 64;
  for (int div = 4; div >= 2 && geo.kdiv == 1; div /= 2) {
    bool whole = true;
    for (int64_t e = 0; e < X->E; ++e) whole = whole && X->ffn_sizes[e] % (div * kstage) == 0;
    if (whole) geo.kdiv = div;
  }
  if (geo.bcsr) {
    REQUIRE(X->block == 128, MOE_EUNSUPPORTED, "BCSR block must be 128 (got %d)", X->block);
    REQUIRE(X->size_blocks && X->block_offsets, MOE_EINVAL, "BCSR needs size_blocks and block_offsets");
  }
  *g = geo;
  return MOE_OK;
}

// Upper bounds on the tile lists (the real counts are only known on the
// device): sum_e ceil(rows_e / bt) * nf_e <= (rows_max / bt + E) * max_e nf_e.
int64_t max_tiles_gemm1(const ExpertGeo& g, int64_t rows_max, int64_t nnz_max) {
  if (g.bcsr) return nnz_max * 128 * g.pf / g.bf1;
  return (rows_max / g.bt + g.E) * ((g.Fmax * g.pf + g.bf1 - 1) / g.bf1);
}
// (bf16 grouped sets are bounded for 128-row tiles, which a dense layer may
// choose for its second linear.)
int64_t max_tiles_gemm2(const ExpertGeo& g, int64_t d, int64_t rows_max) {
  const int64_t nf = d / g.bf2;
  if (g.bcsr) return (rows_max / 128) * nf;
  return (rows_max / std::min(g.bt, 128) + g.E) * nf;
}

int64_t nnz_max_of(const moe_experts_desc* X, int64_t rows_max) {
  int64_t sbmax = 0;
  for (int64_t e = 0; e < X->E; ++e) sbmax = std::max(sbmax, X->ffn_sizes[e] / 128);
  return (rows_max / 128) * sbmax;
}

constexpr int64_t kMxRowPad = 256;   // rows per MXFP8 GEMM tile

struct ExpertWs {
  void* h = nullptr;
  Tile* tiles1 = nullptr;
  Tile* tiles2 = nullptr;
  int* nt = nullptr;   // [32]: the first list's counts at nt, the second's at nt + 16
  // persistent launches planned per XCD: workgroups of each GEMM (0: the
  // kernel splits the list itself); the second GEMM may cut its last round's
  // tiles into K pieces for exactly its grid (pieces2), with fp32 partials
  // and the list entry of each split tile (grid2 ints)
  int grid1 = 0, grid2 = 0;
  bool pieces2 = false;
  float* part = nullptr;
  int* counters = nullptr;
  float* a_rows = nullptr;
  int64_t mt1 = 0, mt2 = 0;
  int64_t rows_max = 0;
  // MXFP8: the quantised GEMM rows and hidden activation with their scales
  // (rp = rows_max + one tile of padding rows; the scales are stage-major:
  // the four bytes of row r in 128-element K stage s at s * 4 rp + 4 r)
  uint8_t* xq = nullptr;   // [rp, d]
  uint8_t* xqs = nullptr;  // [d / 128, rp, 4]
  uint8_t* hq = nullptr;   // [rp, Fmax]
  uint8_t* hqs = nullptr;  // [Fmax / 128, rp, 4]
  bool xq_ready = false;   // the caller already quantised the rows into xq (the layer
                           // does it as its dispatch gather)
  // saved for the backward pass: pre-activations [rows_max, pf * Fmax] (bf16)
  void* pre = nullptr;
  int64_t ldpre = 0;
};

// Compute units of the current device (cached; a host query, no sync).
int device_cus() {
  static thread_local int dev_cached = -1, cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return cus;
  if (dev != dev_cached) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    dev_cached = dev;
  }
  return cus;
}

// A dense layer (the shared FFN) whose second linear has fewer 256-row tiles
// than compute units takes 128-row tiles there instead.
void fit_dense_tiles(ExpertGeo* g, int dtype, int64_t d, int64_t T) {
  if (dtype != MOE_BF16 || g->bcsr || g->atomic || g->mx) return;
  const int64_t tiles = (T + 255) / 256 * (d / g->bf2);
  if (tiles < device_cus()) g->bt2 = 128;
}

// Whether the second linear's last round of tiles is worth cutting into K
// pieces.  The tile count of a grouped layer is only known on the device, so
// the host estimates it (T k / bt + E / 2 row tiles per output slice) and
// models the time of splitting every tile in s parts, in units of one full-K
// tile: the rounds of tiles over the compute units, each 1 / s of a tile, plus
// a fixed cost per round (a tile's prologue and epilogue) and per extra part
// (its partial stores and their reduction).  Splits of 1, 2 or 4 whose parts
// are whole K stages of every expert are considered; a split that beats whole
// tiles says that the last round leaves compute units idle, and then only
// that round's tiles are cut (carve_expert_ws).
constexpr bool kCostRuns = true;
constexpr int kMaxParts2 = 8;   // K pieces per split tile of the second linear
bool want_pieces(const ExpertGeo& g, int dtype, int64_t d, int64_t rows_used_est) {
  if (g.bcsr || g.atomic || dtype != MOE_BF16 || g.kdiv < 2) return false;
  constexpr double kRoundCost = 0.017, kPartCost = 0.031;
  const double cus = device_cus();
  const double n = (double(rows_used_est) / g.bt + 0.5 * double(g.E)) * double(d / g.bf2);
  int best = 1;
  double best_t = 0;
  for (int s = 1; s <= g.kdiv; s *= 2) {
    const double rounds = std::ceil(s * n / cus);
    const double t = rounds / s + kRoundCost * rounds + kPartCost * (s - 1);
    if (s == 1 || t < best_t) {
      best = s;
      best_t = t;
    }
  }
  return best > 1;
}

void carve_expert_ws(Carve& c, const ExpertGeo& g, int dtype, int64_t d, int64_t rows_max,
                     int64_t nnz_max, ExpertWs* w, bool pieces = false, bool save = false,
                     bool runs = false) {
  if (g.atomic) {
    w->a_rows = c.take_n<float>(rows_max);
    return;
  }
  // bf16 and MXFP8 experts whose second linear leaves compute units idle in
  // its last round of tiles (pieces) cut only that round's tiles into K
  // pieces, summed in fp32 by the fixup kernel (measured against splitting
  // every tile into partial planes that combine adds: the same balance with
  // one quarter of the partial traffic and a single rounding of y).
  // Elsewhere the pieces' partial stores and fixup cost more than the idle
  // compute units of the last round.
  // Grouped bf16 / MXFP8 layers (runs) also plan both GEMMs' XCD runs on the
  // device, split by the tiles' modelled cost rather than by count.
  pieces = pieces && dtype == MOE_BF16;
  runs = runs && dtype == MOE_BF16 && !g.bcsr;
  w->mt1 = std::max<int64_t>(1, max_tiles_gemm1(g, rows_max, nnz_max));
  w->mt2 = std::max<int64_t>(1, max_tiles_gemm2(g, d, rows_max));
  if (runs) w->grid1 = gemm_persistent_grid(int(std::min<int64_t>(w->mt1, 1 << 30)));
  if (runs || pieces) w->grid2 = gemm_persistent_grid(int(std::min<int64_t>(w->mt2, 1 << 30)));
  w->pieces2 = pieces;
  if (pieces) {
    w->part = c.take_n<float>(int64_t(w->grid2) * g.bf2 * g.bt2);
    w->counters = c.take_n<int>(w->grid2);
  }
  w->rows_max = rows_max;
  if (g.mx) {
    // a tile reads all of its 256 rows (the ones past the group's end are
    // never stored), so the MXFP8 row buffers carry one tile of spare rows
    const int64_t rp = rows_max + kMxRowPad;
    w->xq = c.take_n<uint8_t>(rp * d);
    w->xqs = c.take_n<uint8_t>(rp * (d / 32));
    w->hq = c.take_n<uint8_t>(rp * g.Fmax);
    w->hqs = c.take_n<uint8_t>(rp * (g.Fmax / 32));
  } else {
    w->h = c.take(size_t(rows_max) * g.Fmax * esize(dtype));
  }
  if (save) {
    w->ldpre = g.pf * g.Fmax;
    w->pre = c.take(size_t(rows_max) * w->ldpre * esize(dtype));
  }
  // a plan for a persistent grid adds at most one entry per workgroup
  w->tiles1 = c.take_n<Tile>(w->mt1 + w->grid1);
  w->tiles2 = c.take_n<Tile>(w->mt2 + w->grid2);
  w->nt = c.take_n<int>(32);
}

// Launch the two expert GEMMs of a grouped / BCSR expert set over the rows of
// a routing (or, for the shared FFN, one dense group of T rows).
// x_rows: the rows of x_in (the token rows when xrow gathers them).
int run_expert_gemms(const moe_experts_desc* X, const ExpertGeo& g, int dtype, int64_t d,
                     const int32_t* offsets, int dense_rows, const int32_t* row_offsets,
                     const int32_t* column_indices, const void* x_in, int64_t x_rows,
                     const float* row_r, const float* row_w, void* y, const ExpertWs& w,
                     hipStream_t s, moe_timer* timer, int call, const int32_t* xrow = nullptr);

}  // namespace

// ---------------------------------------------------------------- timer

struct moe_timer {
  int max_calls = 0;
  int ncalls = 0;
  std::vector<hipEvent_t> ev;   // max_calls x (MOE_STAGE_COUNT + 1)
};

namespace {
void timer_mark(moe_timer* t, int call, int idx, hipStream_t s) {
  if (!t || call < 0) return;
  (void)hipEventRecord(t->ev[size_t(call) * (MOE_STAGE_COUNT + 1) + idx], s);
}

// MXFP8 experts: the GEMM rows are quantised as they are gathered (xrow, or
// the rows themselves), the first linear writes MXFP8 h, the second reads it.
int run_expert_gemms_mx(const moe_experts_desc* X, const ExpertGeo& g, int64_t d,
                        const int32_t* offsets, int dense_rows, const void* x_in,
                        const float* row_r, const float* row_w, void* y, const ExpertWs& w,
                        hipStream_t s, moe_timer* timer, int call, const int32_t* xrow) {
  const int64_t R = w.rows_max, RP = R + kMxRowPad;
  const int64_t P = g.F * g.pf;
  if (std::max(RP * d, RP * g.Fmax) >= (int64_t(1) << 31))
    return fail(MOE_ESHAPE, "MXFP8 row buffers must stay below 2 GiB (rows %lld)", (long long)R);
  if (!w.xq_ready)
    MOE_HIP(launch_quant_mx(x_in, R, d, d, xrow, offsets ? offsets + X->E : nullptr, w.xq, d,
                            w.xqs, d / 32, RP * 4, s));
  MxGemmArgs a{};
  a.g.X = w.xq;
  a.g.ldx = d;
  a.g.W = X->w13_t;
  a.g.ldw = d;
  a.g.tiles = w.tiles1;
  a.g.ntiles = w.nt;
  a.g.Y = w.hq;
  a.g.ldy = g.Fmax;
  a.g.row_r = row_r;
  a.g.epi = X->act == MOE_ACT_SWIGLU ? EPI_SWIGLU : EPI_ACT;
  a.g.act = X->act == MOE_ACT_GELU_TANH ? 1 : 0;
  a.xs = w.xqs;
  a.ldxs = RP * 4;                 // activation scales stage-major: bytes between stages
  a.ws = X->w13_scale;
  a.ldws = P * 4;                  // weight scales stage-major (moe_pack_mxfp8_weights)
  a.ys = w.hqs;
  a.ldys = RP * 4;                 // h's scales written stage-major
  a.x_bytes = RP * d;
  a.w_bytes = P * d;
  a.xs_bytes = RP * (d / 32);
  a.ws_bytes = P * (d / 32);
  // (no K pieces here: the epilogue quantises h, which needs the whole K)
  a.g.xcd_runs = w.grid1 > 0;
  MOE_HIP(launch_gemm_mx(a, w.grid1 > 0 ? w.grid1 : int(w.mt1), s));
  timer_mark(timer, call, MOE_STAGE_GEMM1 + 1, s);

  MxGemmArgs b{};
  b.g.X = w.hq;
  b.g.ldx = g.Fmax;
  b.g.W = X->w2_t;
  b.g.ldw = g.ld2;
  b.g.tiles = w.tiles2;
  b.g.ntiles = w.nt + 16;
  b.g.Y = y;
  b.g.ldy = d;
  b.g.row_w = row_w;
  b.g.epi = EPI_GATE;
  b.g.xcd_runs = w.grid2 > 0;
  b.g.part = w.part;
  b.g.counters = w.counters;
  b.xs = w.hqs;
  b.ldxs = RP * 4;
  b.ws = X->w2_scale;
  b.ldws = d * 4;
  b.x_bytes = RP * g.Fmax;
  b.w_bytes = d * g.ld2;
  b.xs_bytes = RP * (g.Fmax / 32);
  b.ws_bytes = d * (g.F / 32);
  MOE_HIP(launch_gemm_mx(b, w.grid2 > 0 ? w.grid2 : int(w.mt2), s));
  if (w.pieces2) MOE_HIP(launch_piece_fixup(b.g, g.bf2, g.bt2, w.grid2, kMaxParts2, s));
  timer_mark(timer, call, MOE_STAGE_GEMM2 + 1, s);
  (void)dense_rows;
  return MOE_OK;
}

int run_expert_gemms(const moe_experts_desc* X, const ExpertGeo& g, int dtype, int64_t d,
                     const int32_t* offsets, int dense_rows, const int32_t* row_offsets,
                     const int32_t* column_indices, const void* x_in, int64_t x_rows,
                     const float* row_r, const float* row_w, void* y, const ExpertWs& w,
                     hipStream_t s, moe_timer* timer, int call, const int32_t* xrow) {
  PlanArgs p{};
  p.offsets = offsets;
  p.dense_rows = dense_rows;
  p.foff = X->ffn_offsets;
  p.E = int(X->E);
  p.swiglu = X->act == MOE_ACT_SWIGLU;
  p.d = int(d);
  p.bt = g.bt;
  p.row_offsets = g.bcsr ? row_offsets : nullptr;
  p.column_indices = column_indices;
  p.block_offsets = X->block_offsets;
  p.block = 128;
  p.ksplit = 1;
  // first linear
  p.gemm = 1;
  p.bf = g.bf1;
  p.fold = g.fold;
  p.dense_n = int(g.Fmax * g.pf);
  p.tiles = w.tiles1;
  p.ntiles = w.nt;
  p.max_tiles = int(w.mt1);
  p.grid = w.grid1;
  p.max_parts = 1;                 // the first GEMM's epilogue needs the whole K
  p.counters = nullptr;
  p.cost_split = 1;
  p.kstage = g.mx ? 128 : 64;   // the GEMM kernel's K stage (pieces are whole stages)
  // second linear
  PlanArgs p2 = p;
  p2.gemm = 2;
  p2.bf = g.bf2;
  p2.fold = 1;
  p2.dense_n = int(d);
  p2.tiles = w.tiles2;
  p2.ntiles = w.nt + 16;
  p2.max_tiles = int(w.mt2);
  p2.ksplit = 1;
  p2.bt = g.bt2;
  p2.grid = w.grid2;
  p2.max_parts = w.pieces2 ? kMaxParts2 : 1;
  p2.cost_split = 0;
  p2.counters = w.counters;
  MOE_HIP(launch_plan_pair(p, p2, s));
  timer_mark(timer, call, MOE_STAGE_PLAN + 1, s);

  if (g.mx) return run_expert_gemms_mx(X, g, d, offsets, dense_rows, x_in, row_r, row_w, y, w, s,
                                       timer, call, xrow);

  GemmArgs a{};
  a.X = x_in;
  a.ldx = d;
  a.W = X->w13_t;
  a.ldw = d;
  a.tiles = w.tiles1;
  a.ntiles = w.nt;
  a.Y = w.h;
  a.ldy = g.Fmax;
  a.row_r = row_r;
  a.row_w = nullptr;
  a.xrow = xrow;
  a.epi = X->act == MOE_ACT_SWIGLU ? EPI_SWIGLU : EPI_ACT;
  a.act = X->act == MOE_ACT_GELU_TANH ? 1 : 0;
  a.pre = w.pre;
  a.ldpre = w.ldpre;
  a.xcd_runs = w.grid1 > 0;
  a.part = w.part;
  a.counters = w.counters;
  a.x_bytes = x_rows * d * int64_t(esize(dtype));
  a.w_bytes = g.F * g.pf * d * int64_t(esize(dtype));
  MOE_HIP(launch_gemm(dtype, a, g.bf1, g.bt, w.grid1 > 0 ? w.grid1 : int(w.mt1), s));
  timer_mark(timer, call, MOE_STAGE_GEMM1 + 1, s);

  GemmArgs b{};
  b.X = w.h;
  b.ldx = g.Fmax;
  b.W = X->w2_t;
  b.ldw = g.ld2;
  b.tiles = w.tiles2;
  b.ntiles = w.nt + 16;
  b.Y = y;
  b.ldy = d;
  b.row_r = nullptr;
  b.row_w = row_w;
  b.epi = EPI_GATE;
  b.xcd_runs = w.grid2 > 0;
  b.part = w.part;
  b.counters = w.counters;
  b.x_bytes = w.rows_max * g.Fmax * int64_t(esize(dtype));
  b.w_bytes = d * g.ld2 * int64_t(esize(dtype));
  MOE_HIP(launch_gemm(dtype, b, g.bf2, g.bt2, w.grid2 > 0 ? w.grid2 : int(w.mt2), s));
  if (w.pieces2) MOE_HIP(launch_piece_fixup(b, g.bf2, g.bt2, w.grid2, kMaxParts2, s));
  timer_mark(timer, call, MOE_STAGE_GEMM2 + 1, s);
  return MOE_OK;
}

__int128 i128(int64_t v) { return __int128(v); }

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe_mi355x 0.1 (gfx950)"; }

int64_t moe_capacity(int64_t T, int k, int64_t E, double cf) {
  if (T < 0 || k <= 0 || E <= 0 || std::isnan(cf)) return -1;
  if (!(cf > 0)) return T;
  if (T == 0) return 0;
  const double est = double(T) * double(k) * cf / double(E);
  if (!(est < double(T) + 2.0)) return T;          // includes +inf
  if (est < 0.25) return std::min<int64_t>(1, T);  // 0 < exact <= 1
  // exact: cf = m * 2^e2 with integer m
  int ex = 0;
  const double mant = std::frexp(cf, &ex);
  int64_t m = int64_t(std::ldexp(mant, 53));
  int e2 = ex - 53;
  while (m % 2 == 0 && e2 < 0) {
    m /= 2;
    ++e2;
  }
  unsigned __int128 num = (unsigned __int128)(i128(T) * k) * (unsigned __int128)m;
  unsigned __int128 den = (unsigned __int128)E;
  if (e2 >= 0) num <<= e2;
  else den <<= -e2;
  const unsigned __int128 c = (num + den - 1) / den;
  return c > (unsigned __int128)T ? T : int64_t(c);
}

int64_t moe_rows_max(int64_t T, int k, int64_t E, int64_t capacity, int pad) {
  if (T < 0 || k <= 0 || E <= 0 || capacity < 0 || pad < 1) return -1;
  const int64_t kept = std::min(T * k, E * std::min(capacity, T));
  return kept + E * (pad - 1);
}

// ---------------------------------------------------------------- packing

int moe_pack_transpose(const void* src, int dtype, int64_t K, int64_t N, void* dst,
                       hipStream_t stream) {
  REQUIRE(valid_dtype(dtype), MOE_EDTYPE, "unknown dtype %d", dtype);
  REQUIRE(K >= 0 && N >= 0, MOE_ESHAPE, "negative size");
  REQUIRE((src && dst) || K * N == 0, MOE_EINVAL, "NULL pointer");
  REQUIRE(src != dst || K * N == 0, MOE_EINVAL, "transpose cannot run in place");
  MOE_HIP(launch_pack_transpose(src, dtype, K, N, dst, stream));
  return ok();
}

int moe_pack_swiglu(const void* w1, const void* w3, int dtype, int64_t d, const int64_t* ffn_sizes,
                    int64_t E, void* w13_t, hipStream_t stream) {
  REQUIRE(valid_dtype(dtype), MOE_EDTYPE, "unknown dtype %d", dtype);
  REQUIRE(w1 && w3 && w13_t && ffn_sizes, MOE_EINVAL, "NULL pointer");
  REQUIRE(d > 0 && E > 0, MOE_ESHAPE, "d and E must be positive");
  int64_t F = 0;
  for (int64_t e = 0; e < E; ++e) {
    REQUIRE(ffn_sizes[e] > 0 && ffn_sizes[e] % 32 == 0, MOE_ESHAPE,
            "SwiGLU pack needs ffn sizes that are positive multiples of 32 (expert %lld: %lld)",
            (long long)e, (long long)ffn_sizes[e]);
    F += ffn_sizes[e];
  }
  MOE_HIP(launch_pack_swiglu(w1, w3, dtype, d, F, nullptr, ffn_sizes, E, w13_t, stream));
  return ok();
}

int moe_pack_mxfp8(const void* src, int64_t R, int64_t K, int64_t lds, void* codes, int64_t ldc,
                   void* scales, int64_t ldsc, hipStream_t stream) {
  REQUIRE(R >= 0 && K > 0 && K % 32 == 0, MOE_ESHAPE, "MXFP8 pack needs K %% 32 == 0 (K=%lld)",
          (long long)K);
  REQUIRE(lds >= K && lds % 8 == 0 && ldc >= K && ldc % 8 == 0 && ldsc >= K / 32, MOE_ESHAPE,
          "bad row strides (lds %% 8 == 0 and ldc %% 8 == 0 needed)");
  REQUIRE(R == 0 || (src && codes && scales), MOE_EINVAL, "NULL pointer");
  REQUIRE(reinterpret_cast<uintptr_t>(src) % 16 == 0 && reinterpret_cast<uintptr_t>(codes) % 8 == 0,
          MOE_EINVAL, "src must be 16-byte and codes 8-byte aligned");
  MOE_HIP(launch_quant_mx(src, R, K, lds, nullptr, nullptr, codes, ldc, scales, ldsc, 0, stream));
  return ok();
}

int moe_pack_mxfp8_weights(const void* src, int64_t R, int64_t K, int64_t lds, void* codes,
                           int64_t ldc, void* scales, hipStream_t stream) {
  REQUIRE(R >= 0 && K > 0 && K % 128 == 0, MOE_ESHAPE,
          "MXFP8 weight pack needs K %% 128 == 0 (K=%lld)", (long long)K);
  REQUIRE(lds >= K && lds % 8 == 0 && ldc >= K && ldc % 8 == 0, MOE_ESHAPE,
          "bad row strides (lds %% 8 == 0 and ldc %% 8 == 0 needed)");
  REQUIRE(R * (K / 32) < (int64_t(1) << 31), MOE_ESHAPE, "MXFP8 weight scales must stay below 2 GiB");
  REQUIRE(R == 0 || (src && codes && scales), MOE_EINVAL, "NULL pointer");
  REQUIRE(reinterpret_cast<uintptr_t>(src) % 16 == 0 && reinterpret_cast<uintptr_t>(codes) % 8 == 0,
          MOE_EINVAL, "src must be 16-byte and codes 8-byte aligned");
  MOE_HIP(launch_quant_mx(src, R, K, lds, nullptr, nullptr, codes, ldc, scales, K / 32, R * 4, stream));
  return ok();
}

// ---------------------------------------------------------------- stages

int moe_rmsnorm_stats(const void* x, int dtype, int64_t T, int64_t d, const void* gamma, float eps,
                      float* r, void* xg, hipStream_t stream) {
  REQUIRE(valid_dtype(dtype), MOE_EDTYPE, "unknown dtype %d", dtype);
  REQUIRE(T >= 0 && d > 0, MOE_ESHAPE, "bad sizes T=%lld d=%lld", (long long)T, (long long)d);
  REQUIRE(d % (16 / esize(dtype)) == 0, MOE_ESHAPE, "d must fill 16-byte vectors");
  REQUIRE(T == 0 || (x && r), MOE_EINVAL, "x and r are required");
  REQUIRE(!gamma || xg, MOE_EINVAL, "a gain needs the xg output");
  REQUIRE(eps >= 0.f, MOE_EINVAL, "eps must be >= 0");
  MOE_HIP(launch_rmsnorm(x, dtype, T, d, gamma, eps, r, gamma ? xg : nullptr, stream));
  return ok();
}

size_t moe_router_workspace_size(const moe_router_desc* R, int64_t T) {
  if (!R || T < 0) return 0;
  if (R->kind == MOE_ROUTER_CARTESIAN) {
    Carve c(nullptr);
    c.take(size_t(T) * (R->Nr + R->Nc) * sizeof(float));   // scores
    c.take_n<Tile>(std::max<int64_t>(1, ((T + 255) / 256) * ((R->Nr + R->Nc) / 256)));
    c.take_n<int>(1);
    return c.used;
  }
  // dense: per-workgroup partial sums of the routing statistics (the f32
  // router's 4-token workgroups bound the bf16 router's 16-token ones)
  Carve c(nullptr);
  c.take_n<float>(((T + 3) / 4) * R->E);
  c.take_n<float>(((T + 3) / 4) * R->E);
  c.take_n<int>(((T + 3) / 4) * R->E);
  c.take_n<float>(R->E);
  c.take_n<float>(R->E);
  c.take_n<long long>(R->E);
  return c.used;
}

namespace {
int check_router(const moe_router_desc* R, int dtype, int64_t T, int64_t d, int k) {
  REQUIRE(R, MOE_EINVAL, "router descriptor is NULL");
  REQUIRE(valid_dtype(dtype), MOE_EDTYPE, "unknown dtype %d", dtype);
  REQUIRE(T >= 0 && d > 0, MOE_ESHAPE, "bad sizes");
  if (R->kind == MOE_ROUTER_DENSE) {
    REQUIRE(R->E >= 1 && R->E <= 256, MOE_EUNSUPPORTED, "dense router supports 1 <= E <= 256 (got %lld)",
            (long long)R->E);
    REQUIRE(k >= 1 && k <= R->E, MOE_EINVAL, "k must be in [1, E] (k=%d, E=%lld)", k, (long long)R->E);
    REQUIRE(R->wr_t, MOE_EINVAL, "router weights are NULL");
    if (dtype == MOE_BF16)
      REQUIRE(d % 128 == 0, MOE_ESHAPE, "bf16 router needs d %% 128 == 0");
    return MOE_OK;
  }
  REQUIRE(R->kind == MOE_ROUTER_CARTESIAN, MOE_EDTYPE, "unknown router kind %d", R->kind);
  REQUIRE(dtype == MOE_BF16, MOE_EUNSUPPORTED, "the Cartesian router is implemented for bf16 only");
  REQUIRE(R->Nr >= 1 && R->Nc >= 1 && R->E == R->Nr * R->Nc, MOE_ESHAPE, "Cartesian router needs E = Nr*Nc");
  REQUIRE(k >= 1 && k <= 64 && k <= R->Nr && k <= R->Nc, MOE_EINVAL,
          "Cartesian router needs 1 <= k <= min(64, Nr, Nc)");
  REQUIRE((R->Nr + R->Nc) % 256 == 0 && R->Nr + R->Nc <= 8192, MOE_ESHAPE,
          "Cartesian router needs Nr + Nc a multiple of 256 (at most 8192)");
  REQUIRE(int64_t(k) * k <= 4096, MOE_EUNSUPPORTED, "k*k too large");
  REQUIRE(d % 256 == 0, MOE_ESHAPE, "Cartesian router needs d %% 256 == 0");
  REQUIRE(R->keys_t, MOE_EINVAL, "router keys are NULL");
  REQUIRE(R->E < (int64_t(1) << 31), MOE_ESHAPE, "too many experts");
  return MOE_OK;
}

bool extras_requested(const moe_router_extras* ex) {
  return ex && (ex->noise || ex->prob_sum || ex->gate_sum || ex->aux);
}

int check_extras(const moe_router_desc* R, int k, const moe_router_extras* ex) {
  if (!extras_requested(ex)) return MOE_OK;
  REQUIRE(R->kind == MOE_ROUTER_DENSE, MOE_EUNSUPPORTED,
          "router noise / statistics are implemented for the dense router");
  REQUIRE(k <= 64, MOE_EUNSUPPORTED, "router noise / statistics need k <= 64");
  REQUIRE(std::isfinite(ex->noise_std), MOE_EINVAL, "noise_std must be finite");
  return MOE_OK;
}

int router_run(const moe_router_desc* R, const void* x, int dtype, int64_t T, int64_t d,
               const float* r_in, float eps, float* r_out, int k, int renorm, int32_t* ids, float* w,
               float* logits, void* ws, hipStream_t stream, const moe_router_extras* extras) {
  if (R->kind == MOE_ROUTER_DENSE) {
    RouterExtras ex;
    if (extras) {
      ex.noise = extras->noise;
      ex.noise_std = extras->noise_std;
      if (extras->prob_sum || extras->gate_sum || extras->aux) {
        Carve c(ws);
        ex.part_p = c.take_n<float>(((T + 3) / 4) * R->E);
        ex.part_g = c.take_n<float>(((T + 3) / 4) * R->E);
        ex.part_c = c.take_n<int>(((T + 3) / 4) * R->E);
        ex.sum_p = c.take_n<float>(R->E);
        ex.sum_g = c.take_n<float>(R->E);
        ex.sum_c = c.take_n<long long>(R->E);
        ex.prob_sum = extras->prob_sum;
        ex.gate_sum = extras->gate_sum;
        ex.aux = extras->aux;
      }
    }
    MOE_HIP(launch_router_dense(x, dtype, T, d, R->wr_t, R->bias, R->E, r_in, eps, r_out, k, renorm,
                                ids, w, logits, ex, stream));
    return MOE_OK;
  }
  Carve c(ws);
  float* scores = logits ? logits : c.take_n<float>(T * (R->Nr + R->Nc));
  if (logits) c.take_n<float>(T * (R->Nr + R->Nc));
  const int64_t ntile_max = std::max<int64_t>(1, ((T + 255) / 256) * ((R->Nr + R->Nc) / 256));
  Tile* tiles = c.take_n<Tile>(ntile_max);
  int* nt = c.take_n<int>(1);
  const float* r = r_in;
  if (!r) {
    MOE_HIP(launch_rmsnorm(x, dtype, T, d, nullptr, eps, r_out, nullptr, stream));
    r = r_out;
  }
  if (T > 0) {
    PlanArgs p{};
    p.offsets = nullptr;
    p.dense_rows = int(T);
    p.dense_n = int(R->Nr + R->Nc);
    p.gemm = 1;
    p.d = int(d);
    p.bt = 256;
    p.bf = 256;
    p.fold = 1;
    p.tiles = tiles;
    p.ntiles = nt;
    p.max_tiles = int(ntile_max);
    p.ksplit = 1;
    MOE_HIP(launch_plan(p, stream));
    GemmArgs a{};
    a.X = x;
    a.ldx = d;
    a.W = R->keys_t;
    a.ldw = d;
    a.tiles = tiles;
    a.ntiles = nt;
    a.Y = scores;
    a.ldy = R->Nr + R->Nc;
    a.row_r = r;
    a.epi = EPI_SCALE_F32;
    a.x_bytes = T * d * int64_t(esize(dtype));
    a.w_bytes = (R->Nr + R->Nc) * d * int64_t(esize(dtype));
    MOE_HIP(launch_gemm(dtype, a, 256, 256, int(ntile_max), stream));
  }
  MOE_HIP(launch_cartesian_topk(scores, T, R->Nr, R->Nc, k, renorm, ids, w, stream));
  return MOE_OK;
}
}  // namespace

int moe_router_topk(const moe_router_desc* R, const void* x, int dtype, int64_t T, int64_t d,
                    const float* r_in, float eps, float* r_out, int k, int renorm, int32_t* ids,
                    float* w, float* logits, void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_router_topk_ex(R, x, dtype, T, d, r_in, eps, r_out, k, renorm, ids, w, logits, nullptr,
                            ws, ws_bytes, stream);
}

int moe_router_topk_ex(const moe_router_desc* R, const void* x, int dtype, int64_t T, int64_t d,
                       const float* r_in, float eps, float* r_out, int k, int renorm, int32_t* ids,
                       float* w, float* logits, const moe_router_extras* extras, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  int rc = check_router(R, dtype, T, d, k);
  if (rc) return rc;
  rc = check_extras(R, k, extras);
  if (rc) return rc;
  REQUIRE(T == 0 || (x && ids && w), MOE_EINVAL, "x, ids and w are required");
  REQUIRE(r_in || r_out || T == 0, MOE_EINVAL, "r_in or r_out is required");
  REQUIRE(renorm == 0 || renorm == 1, MOE_EINVAL, "renorm must be 0 or 1");
  if (R->kind == MOE_ROUTER_DENSE && dtype == MOE_F32)
    REQUIRE(logits || T == 0, MOE_EINVAL, "the f32 router needs the logits buffer");
  const size_t need = moe_router_workspace_size(R, T);
  REQUIRE(ws_bytes >= need && (need == 0 || ws), MOE_EWORKSPACE, "router workspace needs %zu bytes",
          need);
  rc = router_run(R, x, dtype, T, d, r_in, eps, r_out, k, renorm, ids, w, logits, ws, stream, extras);
  return rc ? rc : ok();
}

size_t moe_dispatch_workspace_size(int64_t T, int k, int64_t E) {
  if (T < 0 || k <= 0 || E <= 0) return 0;
  return dispatch_ws_bytes(T, k, E);
}

int moe_dispatch(const int32_t* ids, const float* w, const float* r, const void* x, int dtype,
                 int64_t T, int64_t d, int64_t E, int k, int64_t capacity, int pad, int64_t rows_max,
                 int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* row_token, float* row_r,
                 float* row_w, int32_t* row_expert, void* x_perm, moe_stats* stats, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  REQUIRE(valid_dtype(dtype), MOE_EDTYPE, "unknown dtype %d", dtype);
  REQUIRE(T >= 0 && k >= 1 && E >= 1 && E < (int64_t(1) << 22), MOE_ESHAPE,
          "bad sizes T=%lld k=%d E=%lld", (long long)T, k, (long long)E);
  REQUIRE(T * k < (int64_t(1) << 31), MOE_ESHAPE, "T*k too large");
  REQUIRE(capacity >= 0, MOE_EINVAL, "capacity must be >= 0");
  REQUIRE(pad >= 1 && pad <= 1024, MOE_EINVAL, "pad must be in [1, 1024]");
  const int64_t need_rows = moe_rows_max(T, k, E, capacity, pad);
  REQUIRE(rows_max >= need_rows, MOE_ESHAPE, "rows_max %lld < required %lld", (long long)rows_max,
          (long long)need_rows);
  REQUIRE(rows_max < (int64_t(1) << 31), MOE_ESHAPE, "rows_max too large");
  REQUIRE(counts && offsets && (T == 0 || (ids && w && r && pos)) &&
              (rows_max == 0 || (row_token && row_r && row_w)),
          MOE_EINVAL, "NULL output");
  REQUIRE(!x_perm || (x && d > 0 && d % (16 / esize(dtype)) == 0), MOE_EINVAL,
          "x_perm needs x and d filling 16-byte vectors");
  if (E > 2048) {
    REQUIRE(pad == 1 && capacity >= T, MOE_EUNSUPPORTED,
            "the radix-sort dispatch (E > 2048) supports pad 1 and no capacity limit only");
  }
  const size_t need = moe_dispatch_workspace_size(T, k, E);
  REQUIRE(ws && ws_bytes >= need, MOE_EWORKSPACE, "dispatch workspace needs %zu bytes", need);
  DispatchArgs a{};
  a.ids = ids;
  a.w = w;
  a.r = r;
  a.x = x;
  a.dtype = dtype;
  a.T = T;
  a.d = d;
  a.E = E;
  a.k = k;
  a.cap = std::min(capacity, T);
  a.pad = pad;
  a.rows_max = rows_max;
  a.counts = counts;
  a.offsets = offsets;
  a.pos = pos;
  a.row_token = row_token;
  a.row_r = row_r;
  a.row_w = row_w;
  a.row_expert = row_expert;
  a.x_perm = x_perm;
  a.stats = stats;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  MOE_HIP(launch_dispatch(a, stream));
  return ok();
}

int64_t moe_topology_nnz_max(int64_t rows_max, int block, const int64_t* ffn_sizes, int64_t E) {
  if (rows_max < 0 || block <= 0 || !ffn_sizes || E <= 0) return -1;
  int64_t sbmax = 0;
  for (int64_t e = 0; e < E; ++e) sbmax = std::max(sbmax, (ffn_sizes[e] + block - 1) / block);
  return (rows_max / block) * sbmax;
}

int moe_build_topology(const int32_t* offsets, const int32_t* size_blocks,
                       const int32_t* block_offsets, int64_t E, int block, int64_t rows_max,
                       int32_t* row_offsets, int32_t* column_indices, int32_t* nnz,
                       hipStream_t stream) {
  REQUIRE(E >= 1 && E <= 2048, MOE_EUNSUPPORTED, "topology supports 1 <= E <= 2048");
  REQUIRE(block > 0 && rows_max >= 0 && rows_max % block == 0, MOE_ESHAPE,
          "rows_max must be a multiple of the block");
  REQUIRE(offsets && size_blocks && block_offsets && row_offsets && column_indices && nnz,
          MOE_EINVAL, "NULL pointer");
  MOE_HIP(launch_topology(offsets, size_blocks, block_offsets, E, block, rows_max, row_offsets,
                          column_indices, nnz, stream));
  return ok();
}

size_t moe_expert_workspace_size(const moe_experts_desc* X, int dtype, int64_t d, int64_t T, int k,
                                 int64_t rows_max) {
  ExpertGeo g;
  if (check_experts(X, dtype, d, &g) || T < 0 || k <= 0 || rows_max < 0) return 0;
  Carve c(nullptr);
  ExpertWs w;
  carve_expert_ws(c, g, dtype, d, rows_max, g.bcsr ? nnz_max_of(X, rows_max) : 0, &w);
  return c.used;
}

int moe_expert_gemm(const moe_experts_desc* X, int dtype, int64_t d, const moe_routing* rt,
                    const void* x_in, void* y, moe_stats* stats, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  ExpertGeo g;
  int rc = check_experts(X, dtype, d, &g);
  if (rc) return rc;
  REQUIRE(rt, MOE_EINVAL, "routing is NULL");
  REQUIRE(rt->E == X->E, MOE_ESHAPE, "routing E %lld != experts E %lld", (long long)rt->E,
          (long long)X->E);
  REQUIRE(rt->T >= 0 && rt->k >= 1 && rt->rows_max >= 0 && rt->rows_max < (int64_t(1) << 31),
          MOE_ESHAPE, "bad routing sizes");
  if (g.atomic && !rt->row_expert)
    REQUIRE(x_in && y && rt->ids && rt->w && rt->r, MOE_EINVAL,
            "token-centric atomic experts need ids, w and r");
  else
    REQUIRE(x_in && y && rt->offsets && rt->row_r && rt->row_w, MOE_EINVAL, "NULL pointer");
  if (g.bcsr) {
    REQUIRE(rt->pad == 128, MOE_ESHAPE, "BCSR experts need a dispatch padded to 128");
    REQUIRE(X->row_offsets && X->column_indices, MOE_EINVAL, "BCSR needs the topology");
    REQUIRE(rt->rows_max % 128 == 0, MOE_ESHAPE, "BCSR rows_max must be a multiple of 128");
    REQUIRE(rt->rows_max / 128 <= 4096, MOE_EUNSUPPORTED, "BCSR supports at most 4096 token blocks");
  }
  if (g.atomic && rt->row_expert)
    REQUIRE(rt->ids && rt->pos && rt->row_token, MOE_EINVAL,
            "expert-centric atomic experts need ids, pos, row_token and row_expert");
  const size_t need = moe_expert_workspace_size(X, dtype, d, rt->T, rt->k, rt->rows_max);
  REQUIRE(ws && ws_bytes >= need, MOE_EWORKSPACE, "expert workspace needs %zu bytes", need);
  Carve c(ws);
  ExpertWs w;
  carve_expert_ws(c, g, dtype, d, rt->rows_max, g.bcsr ? nnz_max_of(X, rt->rows_max) : 0, &w);
  if (g.atomic) {
    AtomicArgs a{};
    a.xhat = x_in;
    a.dtype = dtype;
    a.T = rt->T;
    a.d = d;
    a.k = rt->k;
    a.N = X->E;
    a.W = X->W;
    a.V = X->V;
    a.act = X->act == MOE_ACT_GELU_TANH ? 1 : 0;
    a.ids = rt->ids;
    a.pos = rt->pos;
    a.row_token = rt->row_token;
    a.row_expert = rt->row_expert;
    a.row_r = rt->row_r;
    a.row_w = rt->row_w;
    a.rows_used = rt->offsets ? rt->offsets + rt->E : nullptr;
    a.rows = rt->rows_max;
    a.a_rows = w.a_rows;
    a.routed = y;
    a.token_centric = rt->row_expert ? 0 : 1;
    a.w_tok = rt->w;
    a.r_tok = rt->r;
    a.errors = stats ? &stats->errors : nullptr;
    MOE_HIP(launch_atomic(a, stream));
    return ok();
  }
  rc = run_expert_gemms(X, g, dtype, d, rt->offsets, 0, X->row_offsets, X->column_indices, x_in,
                        rt->rows_max, rt->row_r, rt->row_w, y, w, stream, nullptr, -1);
  return rc ? rc : ok();
}

size_t moe_shared_workspace_size(const moe_experts_desc* S, int dtype, int64_t d, int64_t T) {
  ExpertGeo g;
  if (check_experts(S, dtype, d, &g) || S->E != 1 || S->kind != MOE_EXPERTS_GROUPED || T < 0) return 0;
  Carve c(nullptr);
  ExpertWs w;
  // dense group of T rows: rows_max = T
  carve_expert_ws(c, g, dtype, d, T, 0, &w);
  return c.used;
}

int moe_shared_ffn(const moe_experts_desc* S, int dtype, int64_t d, int64_t T, const void* xhat,
                   const float* r, void* s, void* ws, size_t ws_bytes, hipStream_t stream) {
  ExpertGeo g;
  int rc = check_experts(S, dtype, d, &g);
  if (rc) return rc;
  REQUIRE(S->kind == MOE_EXPERTS_GROUPED && S->E == 1, MOE_EUNSUPPORTED,
          "the shared FFN is one grouped expert");
  REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ESHAPE, "bad T");
  REQUIRE(T == 0 || (xhat && r && s), MOE_EINVAL, "NULL pointer");
  const size_t need = moe_shared_workspace_size(S, dtype, d, T);
  REQUIRE(ws && ws_bytes >= need, MOE_EWORKSPACE, "shared workspace needs %zu bytes", need);
  if (T == 0) return ok();
  Carve c(ws);
  ExpertWs w;
  carve_expert_ws(c, g, dtype, d, T, 0, &w);
  fit_dense_tiles(&g, dtype, d, T);
  rc = run_expert_gemms(S, g, dtype, d, nullptr, int(T), nullptr, nullptr, xhat, T, r, nullptr, s,
                        w, stream, nullptr, -1);
  return rc ? rc : ok();
}

int moe_combine(const void* y, const int32_t* pos, const void* residual, const void* shared,
                int dtype, int64_t T, int64_t d, int k, void* out, hipStream_t stream) {
  REQUIRE(valid_dtype(dtype), MOE_EDTYPE, "unknown dtype %d", dtype);
  REQUIRE(T >= 0 && d > 0 && k >= 1, MOE_ESHAPE, "bad sizes");
  REQUIRE(k <= 256, MOE_EUNSUPPORTED, "combine supports k <= 256");
  REQUIRE(d % (16 / esize(dtype)) == 0, MOE_ESHAPE, "d must fill 16-byte vectors");
  REQUIRE(T == 0 || (y && out), MOE_EINVAL, "NULL pointer");
  MOE_HIP(launch_combine(y, pos, residual, shared, dtype, T, d, k, out, stream));
  return ok();
}

// ---------------------------------------------------------------- the layer

}  // extern "C"

namespace {

struct LayerWs {
  float* r;
  void* xg;
  int32_t* ids;
  float* w;
  float* logits;
  void* router_ws;
  int32_t* counts;
  int32_t* offsets;
  int32_t* pos;
  int32_t* row_token;
  float* row_r;
  float* row_w;
  int32_t* row_expert;
  void* x_perm;
  moe_stats* stats;
  void* disp_ws;
  size_t disp_ws_bytes;
  int32_t* row_offsets;
  int32_t* column_indices;
  int32_t* nnz;
  ExpertWs ex;
  void* y;          // y_perm [rows_max, d] or routed [T, d]
  ExpertWs sh;
  void* s;          // shared output [T, d]
  int64_t rows_max, cap;
};

bool d_ok_for_backward(int64_t d) { return d > 0 && d % 256 == 0; }

int check_layer(const moe_layer_desc* L, int64_t T, ExpertGeo* g, ExpertGeo* gs) {
  REQUIRE(L, MOE_EINVAL, "layer descriptor is NULL");
  REQUIRE(T >= 0 && T < (int64_t(1) << 30), MOE_ESHAPE, "bad T");
  int rc = check_router(&L->router, L->dtype, T, L->d, L->k);
  if (rc) return rc;
  rc = check_extras(&L->router, L->k, L->router_extras);
  if (rc) return rc;
  rc = check_experts(&L->experts, L->dtype, L->d, g);
  if (rc) return rc;
  REQUIRE(L->experts.E == L->router.E, MOE_ESHAPE, "router E %lld != experts E %lld",
          (long long)L->router.E, (long long)L->experts.E);
  REQUIRE((L->router.kind == MOE_ROUTER_CARTESIAN) == g->atomic, MOE_EUNSUPPORTED,
          "the Cartesian router pairs with atomic experts (and only with them)");
  REQUIRE(L->renorm == 0 || L->renorm == 1, MOE_EINVAL, "renorm must be 0 or 1");
  REQUIRE(L->eps >= 0.f, MOE_EINVAL, "eps must be >= 0");
  if (L->shared) {
    rc = check_experts(L->shared, L->dtype, L->d, gs);
    if (rc) return rc;
    REQUIRE(L->shared->kind == MOE_EXPERTS_GROUPED && L->shared->E == 1, MOE_EUNSUPPORTED,
            "the shared FFN is one grouped expert");
  }
  if (g->bcsr) {
    const int64_t cap = moe_capacity(T, L->k, L->experts.E, L->capacity_factor);
    REQUIRE(moe_rows_max(T, L->k, L->experts.E, cap, 128) / 128 < 4096, MOE_EUNSUPPORTED,
            "BCSR supports at most 4096 token blocks");
  }
  if (g->atomic)
    REQUIRE(!(L->capacity_factor > 0) || moe_capacity(T, L->k, L->experts.E, L->capacity_factor) >= T,
            MOE_EUNSUPPORTED, "atomic experts run without a capacity limit");
  REQUIRE(L->save_for_backward == 0 || L->save_for_backward == 1, MOE_EINVAL,
          "save_for_backward must be 0 or 1");
  if (L->save_for_backward) {
    REQUIRE(L->dtype == MOE_BF16 && L->router.kind == MOE_ROUTER_DENSE && !g->atomic && !g->mx &&
                !(L->shared && gs->mx),
            MOE_EUNSUPPORTED,
            "the backward pass covers bf16 layers with a dense router and unquantised grouped "
            "or BCSR experts");
    REQUIRE(d_ok_for_backward(L->d), MOE_ESHAPE, "bad d");
  }
  return MOE_OK;
}

void carve_layer(Carve& c, const moe_layer_desc* L, int64_t T, const ExpertGeo& g,
                 const ExpertGeo& gs, LayerWs* w) {
  const int64_t d = L->d, E = L->experts.E;
  const int k = L->k;
  const size_t es = esize(L->dtype);
  const int pad = g.bcsr ? 128 : 1;
  w->cap = moe_capacity(T, k, E, L->capacity_factor);
  w->rows_max = moe_rows_max(T, k, E, w->cap, pad);
  if (g.bcsr) w->rows_max = (w->rows_max + 127) / 128 * 128;
  w->r = c.take_n<float>(T);
  w->xg = L->gamma ? c.take(size_t(T) * d * es) : nullptr;
  w->ids = c.take_n<int32_t>(T * k);
  w->w = c.take_n<float>(T * k);
  w->logits = (L->router.kind == MOE_ROUTER_DENSE && (L->dtype == MOE_F32 || L->save_for_backward))
                  ? c.take_n<float>(T * E)
                  : nullptr;
  const size_t rws = moe_router_workspace_size(&L->router, T);
  w->router_ws = rws ? c.take(rws) : nullptr;
  w->counts = c.take_n<int32_t>(E);
  w->offsets = c.take_n<int32_t>(E + 1);
  w->pos = c.take_n<int32_t>(T * k);
  w->row_token = c.take_n<int32_t>(w->rows_max);
  w->row_r = c.take_n<float>(w->rows_max);
  w->row_w = c.take_n<float>(w->rows_max);
  w->row_expert = c.take_n<int32_t>(w->rows_max);
  // the first expert GEMM gathers its rows from x through row_token, so the
  // layer never materialises x_perm
  w->x_perm = nullptr;
  w->stats = c.take_n<moe_stats>(1);
  w->disp_ws_bytes = moe_dispatch_workspace_size(T, k, E);
  w->disp_ws = c.take(w->disp_ws_bytes);
  int64_t nnz_max = 0;
  if (g.bcsr) {
    nnz_max = nnz_max_of(&L->experts, w->rows_max);
    w->row_offsets = c.take_n<int32_t>(w->rows_max / 128 + 1);
    w->column_indices = c.take_n<int32_t>(std::max<int64_t>(1, nnz_max));
    w->nnz = c.take_n<int32_t>(1);
  } else {
    w->row_offsets = w->column_indices = w->nnz = nullptr;
  }
  const int64_t rows_est = std::min(T * k, E * std::min(w->cap, T));
  const bool pieces = want_pieces(g, L->dtype, d, rows_est);
  carve_expert_ws(c, g, L->dtype, d, w->rows_max, nnz_max, &w->ex, pieces,
                  L->save_for_backward != 0, kCostRuns && !g.atomic);
  w->y = c.take(size_t(g.atomic ? T : w->rows_max) * d * es);
  if (L->shared) {
    carve_expert_ws(c, gs, L->dtype, d, T, 0, &w->sh, false, L->save_for_backward != 0);
    w->s = c.take(size_t(T) * d * es);
  } else {
    w->s = nullptr;
  }
}

}  // namespace

extern "C" {

size_t moe_layer_workspace_size(const moe_layer_desc* L, int64_t T) {
  ExpertGeo g, gs;
  if (check_layer(L, T, &g, &gs)) return 0;
  Carve c(nullptr);
  LayerWs w;
  carve_layer(c, L, T, g, gs, &w);
  return c.used;
}

int moe_layer_routing(const moe_layer_desc* L, int64_t T, void* ws, size_t ws_bytes, moe_routing* rt) {
  ExpertGeo g, gs;
  int rc = check_layer(L, T, &g, &gs);
  if (rc) return rc;
  REQUIRE(ws && rt, MOE_EINVAL, "NULL pointer");
  Carve c(ws);
  LayerWs w;
  carve_layer(c, L, T, g, gs, &w);
  REQUIRE(ws_bytes >= c.used, MOE_EWORKSPACE, "workspace too small");
  rt->T = T;
  rt->k = L->k;
  rt->E = L->experts.E;
  rt->rows_max = w.rows_max;
  rt->pad = g.bcsr ? 128 : 1;
  rt->ids = w.ids;
  rt->w = w.w;
  rt->r = w.r;
  rt->counts = w.counts;
  rt->offsets = w.offsets;
  rt->pos = w.pos;
  rt->row_token = w.row_token;
  rt->row_r = w.row_r;
  rt->row_w = w.row_w;
  rt->row_expert = w.row_expert;
  return ok();
}

int moe_layer_forward(const moe_layer_desc* L, const void* x, int64_t T, void* out, moe_stats* stats,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  ExpertGeo g, gs;
  int rc = check_layer(L, T, &g, &gs);
  if (rc) return rc;
  REQUIRE(T == 0 || (x && out), MOE_EINVAL, "x and out are required");
  Carve c(ws);
  LayerWs w;
  carve_layer(c, L, T, g, gs, &w);
  REQUIRE(ws && ws_bytes >= c.used, MOE_EWORKSPACE, "layer workspace needs %zu bytes (got %zu)",
          c.used, ws_bytes);
  const int64_t d = L->d, E = L->experts.E;
  const int k = L->k;
  moe_timer* tm = L->timer;
  int call = -1;
  if (tm && tm->ncalls < tm->max_calls) call = tm->ncalls++;
  timer_mark(tm, call, 0, stream);

  // 1-2. RMSNorm statistic, router, top-k
  const void* xhat = x;
  if (L->gamma) {
    MOE_HIP(launch_rmsnorm(x, L->dtype, T, d, L->gamma, L->eps, w.r, w.xg, stream));
    xhat = w.xg;
    rc = router_run(&L->router, xhat, L->dtype, T, d, w.r, L->eps, nullptr, k, L->renorm, w.ids, w.w,
                    w.logits, w.router_ws, stream, L->router_extras);
  } else {
    rc = router_run(&L->router, xhat, L->dtype, T, d, nullptr, L->eps, w.r, k, L->renorm, w.ids, w.w,
                    w.logits, w.router_ws, stream, L->router_extras);
  }
  if (rc) return rc;
  timer_mark(tm, call, MOE_STAGE_ROUTER + 1, stream);

  // 3. capacity + dispatch (atomic experts read the routing by token and need
  // no task list: only their slot counters are written)
  moe_stats* st = stats ? stats : w.stats;
  if (g.atomic) {
    MOE_HIP(launch_slot_stats(T * k, st, stream));
  } else {
    DispatchArgs a{};
    a.ids = w.ids;
    a.w = w.w;
    a.r = w.r;
    a.x = xhat;
    a.dtype = L->dtype;
    a.T = T;
    a.d = d;
    a.E = E;
    a.k = k;
    a.cap = w.cap;
    a.pad = g.bcsr ? 128 : 1;
    a.rows_max = w.rows_max;
    a.counts = w.counts;
    a.offsets = w.offsets;
    a.pos = w.pos;
    a.row_token = w.row_token;
    a.row_r = w.row_r;
    a.row_w = w.row_w;
    a.row_expert = w.row_expert;
    a.x_perm = w.x_perm;
    a.stats = st;
    a.ws = w.disp_ws;
    a.ws_bytes = w.disp_ws_bytes;
    MOE_HIP(launch_dispatch(a, stream));
    if (g.mx) {
      // the MXFP8 path's gather: each routed row quantised once as it is read
      MOE_HIP(launch_quant_mx(xhat, w.rows_max, d, d, w.row_token, w.offsets + E, w.ex.xq, d,
                              w.ex.xqs, d / 32, (w.rows_max + kMxRowPad) * 4, stream));
      w.ex.xq_ready = true;
    }
  }
  timer_mark(tm, call, MOE_STAGE_DISPATCH + 1, stream);

  // 4. experts
  if (g.atomic) {
    timer_mark(tm, call, MOE_STAGE_PLAN + 1, stream);
    AtomicArgs a{};
    a.xhat = xhat;
    a.dtype = L->dtype;
    a.T = T;
    a.d = d;
    a.k = k;
    a.N = E;
    a.W = L->experts.W;
    a.V = L->experts.V;
    a.act = L->experts.act == MOE_ACT_GELU_TANH ? 1 : 0;
    a.ids = w.ids;
    a.pos = w.pos;
    a.row_token = w.row_token;
    a.routed = w.y;
    a.token_centric = 1;
    a.w_tok = w.w;
    a.r_tok = w.r;
    a.errors = &st->errors;
    MOE_HIP(launch_atomic(a, stream));
    timer_mark(tm, call, MOE_STAGE_GEMM1 + 1, stream);
    timer_mark(tm, call, MOE_STAGE_GEMM2 + 1, stream);
  } else {
    if (g.bcsr)
      MOE_HIP(launch_topology(w.offsets, L->experts.size_blocks, L->experts.block_offsets, E, 128,
                              w.rows_max, w.row_offsets, w.column_indices, w.nnz, stream));
    rc = run_expert_gemms(&L->experts, g, L->dtype, d, w.offsets, 0, w.row_offsets, w.column_indices,
                          xhat, T, w.row_r, w.row_w, w.y, w.ex, stream, tm, call, w.row_token);
    if (rc) return rc;
  }
  // shared experts: dense, gate 1, r in the first epilogue
  if (L->shared && T > 0) {
    ExpertGeo gt = gs;
    fit_dense_tiles(&gt, L->dtype, d, T);
    rc = run_expert_gemms(L->shared, gt, L->dtype, d, nullptr, int(T), nullptr, nullptr, xhat, T,
                          w.r, nullptr, w.s, w.sh, stream, nullptr, -1);
    if (rc) return rc;
  }
  timer_mark(tm, call, MOE_STAGE_SHARED + 1, stream);

  // 5. combine
  MOE_HIP(launch_combine(w.y, g.atomic ? nullptr : w.pos, L->residual ? x : nullptr, w.s,
                         L->dtype, T, d, k, out, stream));
  timer_mark(tm, call, MOE_STAGE_COMBINE + 1, stream);
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------- backward pass

namespace {

int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

// Tile edge of the weight-gradient GEMMs (256 x 256; 128 x 128 tiles with
// two workgroups per compute unit measured slower: 4.9 against 3.85 ms for
// the Mixtral-shaped layer's two weight gradients).
constexpr int kWgTile = 256;

// Pointers into the backward workspace.
struct BwdWs {
  int64_t L = 0, Tpad = 0;     // K extents of the routed / token-wide weight-gradient GEMMs
  int nft = 0;                 // routed 64-unit blocks per row (ceil(Fmax / 64))
  void* tbuf = nullptr;        // [rows_max, Fmax] bf16: dout . w2^T per row
  void* dpre = nullptr;        // [rows_max, pf Fmax] bf16
  float* part = nullptr;       // [rows_max, 2 nft]
  float* dg_row = nullptr;     // [rows_max]
  float* dr_row = nullptr;
  float* dxperm = nullptr;     // [ksplit][rows_max, d]
  int ksplit = 1;              // K halves of the dxhat GEMM (partial planes summed by the
                               // token pass)
  uint16_t* hT = nullptr;      // [F, L]
  uint16_t* dpreT = nullptr;   // [P, L]
  uint16_t* dyT = nullptr;     // [E d, L]
  uint16_t* rxT = nullptr;     // [E d, L]
  float* dl = nullptr;         // [T, E]
  uint16_t* dlT = nullptr;     // [E, Tpad]
  float* drr = nullptr;        // [T]
  uint16_t* rxT_all = nullptr; // [d, Tpad]
  float* dgamma_part = nullptr;
  // shared experts
  int nft_s = 0;
  void* tbuf_s = nullptr;      // [T, F_s]
  void* dpre_s = nullptr;      // [T, P_s]
  float* part_s = nullptr;     // [T, 2 nft_s]
  float* dr_s = nullptr;       // [T]
  float* dxs = nullptr;        // [T, d]
  uint16_t* hT_s = nullptr;    // [F_s, Tpad]
  uint16_t* dpreT_s = nullptr; // [P_s, Tpad]
  uint16_t* GT = nullptr;      // [d, Tpad]
  // tile lists: B1, B2, dW13, dW2 (routed), router, B1s, B2s, dW13s, dW2s
  Tile* tiles[9] = {};
  int64_t mt[9] = {};
  int* nt = nullptr;           // [9]
};

void carve_backward(Carve& c, const moe_layer_desc* L, int64_t T, const ExpertGeo& g,
                    const ExpertGeo& gs, const LayerWs& fw, BwdWs* b) {
  const int64_t d = L->d, E = L->experts.E;
  const int pad = g.bcsr ? 128 : 1;
  const int64_t rm = fw.rows_max;
  const int64_t P = g.F * g.pf, Pmax = g.Fmax * g.pf;
  b->L = pad64((std::min(fw.cap, T) + pad - 1) / pad * pad);
  b->Tpad = pad64(T);
  b->nft = int((g.Fmax + 63) / 64);
  b->tbuf = c.take(size_t(rm) * g.Fmax * 2);
  b->dpre = c.take(size_t(rm) * Pmax * 2);
  b->part = c.take_n<float>(rm * 2 * b->nft);
  b->dg_row = c.take_n<float>(rm);
  b->dr_row = c.take_n<float>(rm);
  {
    // split K of the dxhat GEMM when its tile count leaves the last round of
    // tiles badly filled (each half a whole number of 64-wide stages)
    bool halves = true;
    for (int64_t e = 0; e < E; ++e)
      halves = halves && (L->experts.ffn_sizes[e] * g.pf) % 128 == 0;
    const double cus = device_cus();
    const int64_t rows_est = std::min(T * L->k, E * std::min(fw.cap, T));
    const double n = (double(rows_est) / 256 + 0.5 * double(E)) * double(d / 256);
    auto eff = [&](double t) { return t <= 0 ? 1.0 : (t / cus) / std::ceil(t / cus); };
    b->ksplit = halves && eff(2 * n) > eff(n) + 0.08 ? 2 : 1;
  }
  b->dxperm = c.take_n<float>(b->ksplit * rm * d);
  b->hT = c.take_n<uint16_t>(g.F * b->L);
  b->dpreT = c.take_n<uint16_t>(P * b->L);
  b->dyT = c.take_n<uint16_t>(E * d * b->L);
  b->rxT = c.take_n<uint16_t>(E * d * b->L);
  b->dl = c.take_n<float>(T * E);
  b->dlT = c.take_n<uint16_t>(E * b->Tpad);
  b->drr = c.take_n<float>(T);
  b->rxT_all = c.take_n<uint16_t>(d * b->Tpad);
  b->dgamma_part = L->gamma ? c.take_n<float>(int64_t(token_bwd_blocks(T)) * d) : nullptr;
  const int64_t nd = d / 256;
  b->mt[0] = (rm / 256 + E) * ((g.Fmax + 255) / 256);
  b->mt[1] = (rm / 256 + E) * nd * b->ksplit;
  // weight-gradient GEMMs: 128 x 128 tiles (kWgTile)
  const int64_t ndw = d / kWgTile;
  b->mt[2] = (P / kWgTile + E) * ndw;
  b->mt[3] = (g.F / kWgTile + E) * ndw;
  b->mt[4] = ((E + kWgTile - 1) / kWgTile) * ndw;
  if (L->shared) {
    const int64_t Ps = gs.F * gs.pf;
    b->nft_s = int((gs.F + 63) / 64);
    b->tbuf_s = c.take(size_t(T) * gs.F * 2);
    b->dpre_s = c.take(size_t(T) * Ps * 2);
    b->part_s = c.take_n<float>(T * 2 * b->nft_s);
    b->dr_s = c.take_n<float>(T);
    b->dxs = c.take_n<float>(T * d);
    b->hT_s = c.take_n<uint16_t>(gs.F * b->Tpad);
    b->dpreT_s = c.take_n<uint16_t>(Ps * b->Tpad);
    b->GT = c.take_n<uint16_t>(d * b->Tpad);
    const int64_t mtT = (T + 255) / 256;
    b->mt[5] = mtT * ((gs.F + 255) / 256);
    b->mt[6] = mtT * nd;
    b->mt[7] = ((Ps + kWgTile - 1) / kWgTile) * (d / kWgTile);
    b->mt[8] = ((gs.F + kWgTile - 1) / kWgTile) * (d / kWgTile);
  }
  for (int i = 0; i < 9; ++i) {
    b->mt[i] = std::max<int64_t>(1, b->mt[i]);
    b->tiles[i] = c.take_n<Tile>(b->mt[i]);
  }
  b->nt = c.take_n<int>(9);
}

int check_backward(const moe_layer_desc* L, int64_t T, ExpertGeo* g, ExpertGeo* gs) {
  int rc = check_layer(L, T, g, gs);
  if (rc) return rc;
  REQUIRE(L->save_for_backward == 1, MOE_EINVAL,
          "the backward needs a layer descriptor with save_for_backward = 1");
  REQUIRE(L->experts.w2_fk && L->experts.w13_dk, MOE_EINVAL,
          "the backward needs w2_fk and w13_dk in the expert descriptor");
  REQUIRE(!L->shared || (L->shared->w2_fk && L->shared->w13_dk), MOE_EINVAL,
          "the backward needs w2_fk and w13_dk in the shared-expert descriptor");
  REQUIRE(!L->router_extras || !L->router_extras->noise, MOE_EUNSUPPORTED,
          "the backward does not take noise top-k");
  REQUIRE(L->experts.E <= 4096, MOE_EUNSUPPORTED, "the backward supports E <= 4096");
  REQUIRE(L->d % 256 == 0, MOE_ESHAPE, "the backward needs d %% 256 == 0");
  return MOE_OK;
}

// The two GEMMs of one expert set's backward on the rows of its segments
// (routed: the dispatch's offsets; shared: one dense group of T rows).
struct ExpertBwdIo {
  const moe_experts_desc* X;
  const ExpertGeo* g;
  const int32_t* offsets;      // NULL: dense group of T rows
  int64_t rows;                // rows_max, or T
  const int32_t* xrow;         // row -> token (routed) or NULL
  const float* row_w;          // gate per row, NULL = 1
  const float* row_r;          // r per row
  const int32_t* row_expert;   // routed rows' expert (for the partial reduction)
  const void* h;               // saved h [rows, Fmax]
  const void* pre;             // saved pre-activations [rows, pf Fmax]
  void* tbuf; void* dpre; float* part; int nft; float* dg_row; float* dr_row; float* dx_rows;
  uint16_t* hT; uint16_t* dpreT; int64_t ldo; int64_t seg_rows;   // transposed outputs
  int ksplit; int64_t plane;   // K halves of the dxhat GEMM, elements between planes
  Tile* t_b1; int64_t mt_b1; int* nt_b1;
  Tile* t_b2; int64_t mt_b2; int* nt_b2;
};

int run_expert_bwd(const ExpertBwdIo& io, int64_t d, int64_t T, const void* dout, hipStream_t s) {
  const ExpertGeo& g = *io.g;
  const int64_t Pmax = g.pf * g.Fmax;
  PlanArgs p{};
  p.offsets = io.offsets;
  p.dense_rows = int(T);
  p.dense_n = int(g.Fmax);
  p.foff = io.X->ffn_offsets;
  p.E = int(io.X->E);
  p.swiglu = 0;
  p.d = int(d);
  p.bt = 256;
  p.bf = 256;
  p.fold = 1;
  p.ksplit = 1;
  p.block = 128;
  p.gemm = 1;
  p.ragged = 1;
  p.tiles = io.t_b1;
  p.ntiles = io.nt_b1;
  p.max_tiles = int(io.mt_b1);
  PlanArgs p2 = p;
  p2.gemm = 2;
  p2.ragged = 0;
  p2.kmul = g.pf;
  p2.ksplit = std::max(1, io.ksplit);
  p2.dense_n = int(d);
  p2.tiles = io.t_b2;
  p2.ntiles = io.nt_b2;
  p2.max_tiles = int(io.mt_b2);
  MOE_HIP(launch_plan_pair(p, p2, s));

  GemmArgs a{};
  a.X = dout;
  a.ldx = d;
  a.xrow = io.xrow;
  a.W = io.X->w2_fk;
  a.ldw = d;
  a.tiles = io.t_b1;
  a.ntiles = io.nt_b1;
  a.Y = io.tbuf;
  a.ldy = g.Fmax;
  a.epi = EPI_STORE_T;
  a.x_bytes = T * d * 2;
  a.w_bytes = g.F * d * 2;
  MOE_HIP(launch_gemm(MOE_BF16, a, 256, 256, int(io.mt_b1), s));
  ActBwdArgs ab{};
  ab.t = static_cast<const uint16_t*>(io.tbuf);
  ab.ldt = g.Fmax;
  ab.h = static_cast<const uint16_t*>(io.h);
  ab.ldh = g.Fmax;
  ab.pre = static_cast<const uint16_t*>(io.pre);
  ab.ldpre = Pmax;
  ab.row_w = io.row_w;
  ab.row_r = io.row_r;
  ab.offsets = io.offsets;
  ab.dense_rows = int(T);
  ab.E = int(io.X->E);
  ab.foff = io.X->ffn_offsets;
  ab.swiglu = io.X->act == MOE_ACT_SWIGLU;
  ab.act = io.X->act == MOE_ACT_GELU_TANH ? 1 : 0;
  ab.dpre = static_cast<uint16_t*>(io.dpre);
  ab.lddp = Pmax;
  ab.dpreT = io.dpreT;
  ab.hT = io.hT;
  ab.ldo = io.ldo;
  ab.part = io.part;
  ab.ldpart = 2 * io.nft;
  MOE_HIP(launch_act_bwd(ab, int(g.Fmax), int(io.seg_rows), int(io.offsets ? io.X->E : 1), s));
  MOE_HIP(launch_reduce_part(io.part, 2 * io.nft, io.rows, io.row_expert, io.X->ffn_offsets,
                             io.nft, io.dg_row, io.dr_row, s));
  GemmArgs b{};
  b.X = io.dpre;
  b.ldx = Pmax;
  b.W = io.X->w13_dk;
  b.ldw = g.F * g.pf;
  b.tiles = io.t_b2;
  b.ntiles = io.nt_b2;
  b.Y = io.dx_rows;
  b.ldy = d;
  b.ysplit = io.plane;
  b.row_r = io.row_r;
  b.epi = EPI_SCALE_F32;
  b.x_bytes = io.rows * Pmax * 2;
  b.w_bytes = d * g.F * g.pf * 2;
  MOE_HIP(launch_gemm(MOE_BF16, b, 256, 256, int(io.mt_b2), s));
  return MOE_OK;
}

// Y [xrows, d] = sum over each segment's rows of X^T W (fp32, plain); X has
// xrows rows and W wrows rows.
int run_wgrad(WgradPlanArgs wp, const uint16_t* X, int64_t ldx, int64_t xrows, const uint16_t* W,
              int64_t ldw, int64_t wrows, float* Y, int64_t ldy, hipStream_t s) {
  wp.tile = kWgTile;
  MOE_HIP(launch_plan_wgrad(wp, s));
  GemmArgs a{};
  a.X = X;
  a.ldx = ldx;
  a.W = W;
  a.ldw = ldw;
  a.tiles = wp.tiles;
  a.ntiles = wp.ntiles;
  a.Y = Y;
  a.ldy = ldy;
  a.epi = EPI_SCALE_F32;
  a.x_bytes = xrows * ldx * 2;
  a.w_bytes = wrows * ldw * 2;
  MOE_HIP(launch_gemm(MOE_BF16, a, kWgTile, kWgTile, wp.max_tiles, s));
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_layer_backward_workspace_size(const moe_layer_desc* L, int64_t T) {
  ExpertGeo g, gs;
  if (check_backward(L, T, &g, &gs)) return 0;
  Carve c0(nullptr);
  LayerWs fw;
  carve_layer(c0, L, T, g, gs, &fw);
  Carve c(nullptr);
  BwdWs b;
  carve_backward(c, L, T, g, gs, fw, &b);
  return c.used;
}

int moe_layer_backward(const moe_layer_desc* L, const void* x, int64_t T, const void* dout,
                       const void* fwd_ws, size_t fwd_ws_bytes, const moe_layer_grads* grads,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  ExpertGeo g, gs;
  int rc = check_backward(L, T, &g, &gs);
  if (rc) return rc;
  REQUIRE(grads, MOE_EINVAL, "grads is NULL");
  REQUIRE(T == 0 || (x && dout && grads->dx && grads->dw_router && grads->dw13 && grads->dw2),
          MOE_EINVAL, "x, dout, dx, dw_router, dw13 and dw2 are required");
  REQUIRE(!L->router.bias || grads->dbias, MOE_EINVAL, "a router bias needs dbias");
  REQUIRE(!L->gamma || grads->dgamma, MOE_EINVAL, "a gain needs dgamma");
  REQUIRE(!L->shared || (grads->dws13 && grads->dws2), MOE_EINVAL,
          "shared experts need dws13 and dws2");
  Carve c0(const_cast<void*>(fwd_ws));
  LayerWs fw;
  carve_layer(c0, L, T, g, gs, &fw);
  REQUIRE(fwd_ws && fwd_ws_bytes >= c0.used, MOE_EWORKSPACE,
          "the forward workspace needs %zu bytes (got %zu)", c0.used, fwd_ws_bytes);
  Carve c(ws);
  BwdWs b;
  carve_backward(c, L, T, g, gs, fw, &b);
  REQUIRE(ws && ws_bytes >= c.used, MOE_EWORKSPACE, "backward workspace needs %zu bytes (got %zu)",
          c.used, ws_bytes);
  if (T == 0) return ok();
  const int64_t d = L->d, E = L->experts.E;
  const int k = L->k;
  const void* xhat = L->gamma ? fw.xg : x;
  const uint16_t* dout16 = static_cast<const uint16_t*>(dout);
  const uint16_t* xhat16 = static_cast<const uint16_t*>(xhat);

  // 1. routed experts: dh / da (and the gate's and r's per-row sums), dxhat rows
  ExpertBwdIo io{};
  io.X = &L->experts;
  io.g = &g;
  io.offsets = fw.offsets;
  io.rows = fw.rows_max;
  io.xrow = fw.row_token;
  io.row_w = fw.row_w;
  io.row_r = fw.row_r;
  io.row_expert = fw.row_expert;
  io.h = fw.ex.h;
  io.pre = fw.ex.pre;
  io.tbuf = b.tbuf;
  io.dpre = b.dpre;
  io.hT = b.hT;
  io.dpreT = b.dpreT;
  io.ldo = b.L;
  io.seg_rows = b.L;
  io.part = b.part;
  io.nft = b.nft;
  io.dg_row = b.dg_row;
  io.dr_row = b.dr_row;
  io.dx_rows = b.dxperm;
  io.ksplit = b.ksplit;
  io.plane = fw.rows_max * d;
  io.t_b1 = b.tiles[0];
  io.mt_b1 = b.mt[0];
  io.nt_b1 = b.nt;
  io.t_b2 = b.tiles[1];
  io.mt_b2 = b.mt[1];
  io.nt_b2 = b.nt + 1;
  rc = run_expert_bwd(io, d, T, dout, stream);
  if (rc) return rc;

  // 2. routed weight gradients over each expert's rows
  {
    GatherTArgs t{};
    t.offsets = fw.offsets;
    t.E = int(E);
    t.foff = L->experts.ffn_offsets;
    t.ldo = b.L;
    t.wfix = int(d);
    t.rowmap = fw.row_token;
    t.src = dout16;
    t.lds = d;
    t.rscale = fw.row_w;
    t.out = b.dyT;
    MOE_HIP(launch_gather_t(t, int(d), int(b.L), int(E), stream));
    t.src = xhat16;
    t.rscale = fw.row_r;
    t.out = b.rxT;
    MOE_HIP(launch_gather_t(t, int(d), int(b.L), int(E), stream));
    WgradPlanArgs wp{};
    wp.offsets = fw.offsets;
    wp.E = int(E);
    wp.foff = L->experts.ffn_offsets;
    wp.xmul = g.pf;
    wp.wstride = int(d);
    wp.d = int(d);
    wp.tiles = b.tiles[2];
    wp.ntiles = b.nt + 2;
    wp.max_tiles = int(b.mt[2]);
    rc = run_wgrad(wp, b.dpreT, b.L, g.F * g.pf, b.rxT, b.L, E * d, grads->dw13, d, stream);
    if (rc) return rc;
    wp.xmul = 1;
    wp.tiles = b.tiles[3];
    wp.ntiles = b.nt + 3;
    wp.max_tiles = int(b.mt[3]);
    rc = run_wgrad(wp, b.hT, b.L, g.F, b.dyT, b.L, E * d, grads->dw2, d, stream);
    if (rc) return rc;
  }

  // 3. token-wide operands: r xhat transposed (router and shared experts)
  {
    GatherTArgs t{};
    t.dense_rows = int(T);
    t.E = 1;
    t.wfix = int(d);
    t.src = xhat16;
    t.lds = d;
    t.rscale = fw.r;
    t.out = b.rxT_all;
    t.ldo = b.Tpad;
    MOE_HIP(launch_gather_t(t, int(d), int(b.Tpad), 1, stream));
  }

  // 4. shared experts (gate 1, every token)
  if (L->shared) {
    const int64_t Ps = gs.F * gs.pf;
    ExpertBwdIo si{};
    si.X = L->shared;
    si.g = &gs;
    si.offsets = nullptr;
    si.rows = T;
    si.row_r = fw.r;
    si.h = fw.sh.h;
    si.pre = fw.sh.pre;
    si.tbuf = b.tbuf_s;
    si.dpre = b.dpre_s;
    si.hT = b.hT_s;
    si.dpreT = b.dpreT_s;
    si.ldo = b.Tpad;
    si.seg_rows = b.Tpad;
    si.part = b.part_s;
    si.nft = b.nft_s;
    si.dr_row = b.dr_s;
    si.dx_rows = b.dxs;
    si.ksplit = 1;
    si.t_b1 = b.tiles[5];
    si.mt_b1 = b.mt[5];
    si.nt_b1 = b.nt + 5;
    si.t_b2 = b.tiles[6];
    si.mt_b2 = b.mt[6];
    si.nt_b2 = b.nt + 6;
    rc = run_expert_bwd(si, d, T, dout, stream);
    if (rc) return rc;
    GatherTArgs t{};
    t.dense_rows = int(T);
    t.E = 1;
    t.ldo = b.Tpad;
    t.src = dout16;
    t.lds = d;
    t.wfix = int(d);
    t.out = b.GT;
    MOE_HIP(launch_gather_t(t, int(d), int(b.Tpad), 1, stream));
    WgradPlanArgs wp{};
    wp.dense_rows = int(T);
    wp.E = 1;
    wp.wstride = 0;
    wp.d = int(d);
    wp.xfix = int(Ps);
    wp.tiles = b.tiles[7];
    wp.ntiles = b.nt + 7;
    wp.max_tiles = int(b.mt[7]);
    rc = run_wgrad(wp, b.dpreT_s, b.Tpad, Ps, b.rxT_all, b.Tpad, d, grads->dws13, d, stream);
    if (rc) return rc;
    wp.xfix = int(gs.F);
    wp.tiles = b.tiles[8];
    wp.ntiles = b.nt + 8;
    wp.max_tiles = int(b.mt[8]);
    rc = run_wgrad(wp, b.hT_s, b.Tpad, gs.F, b.GT, b.Tpad, d, grads->dws2, d, stream);
    if (rc) return rc;
  }

  // 5. router: gate -> logit gradients, its weight / bias gradients
  {
    RouterBwdArgs r{};
    r.T = T;
    r.Tpad = b.Tpad;
    r.E = int(E);
    r.k = k;
    r.renorm = L->renorm;
    r.logits = fw.logits;
    r.ids = fw.ids;
    r.w = fw.w;
    r.pos = fw.pos;
    r.dg_row = b.dg_row;
    r.bias = L->router.bias;
    r.r = fw.r;
    r.dl = b.dl;
    r.dlT = b.dlT;
    r.ldt = b.Tpad;
    r.dr = b.drr;
    MOE_HIP(launch_router_bwd(r, stream));
    WgradPlanArgs wp{};
    wp.dense_rows = int(T);
    wp.E = 1;
    wp.xfix = int(E);
    wp.wstride = 0;
    wp.d = int(d);
    wp.tiles = b.tiles[4];
    wp.ntiles = b.nt + 4;
    wp.max_tiles = int(b.mt[4]);
    rc = run_wgrad(wp, b.dlT, b.Tpad, E, b.rxT_all, b.Tpad, d, grads->dw_router, d, stream);
    if (rc) return rc;
    if (grads->dbias) MOE_HIP(launch_colsum(b.dl, T, E, E, grads->dbias, stream));
  }

  // 6. back to token order, with the RMSNorm backward (saved r)
  {
    TokenBwdArgs t{};
    t.T = T;
    t.d = d;
    t.k = k;
    t.E = int(E);
    t.residual = L->residual;
    t.x = static_cast<const uint16_t*>(x);
    t.dout = dout16;
    t.gamma = static_cast<const uint16_t*>(L->gamma);
    t.r = fw.r;
    t.pos = fw.pos;
    t.dxperm = b.dxperm;
    t.ksplit = b.ksplit;
    t.plane = fw.rows_max * d;
    t.dr_row = b.dr_row;
    t.dxs = L->shared ? b.dxs : nullptr;
    t.dr_shared = L->shared ? b.dr_s : nullptr;
    t.dl = b.dl;
    t.wr = static_cast<const uint16_t*>(L->router.wr_t);
    t.dr_router = b.drr;
    t.dx = static_cast<uint16_t*>(grads->dx);
    t.dgamma_part = b.dgamma_part;
    MOE_HIP(launch_token_bwd(t, stream));
    if (L->gamma)
      MOE_HIP(launch_colsum(b.dgamma_part, token_bwd_blocks(T), d, d, grads->dgamma, stream));
  }
  return ok();
}

}  // extern "C"

extern "C" {

// ---------------------------------------------------------------- timer

int moe_timer_create(moe_timer** out, int max_calls) {
  REQUIRE(out && max_calls > 0 && max_calls <= 100000, MOE_EINVAL, "bad timer arguments");
  moe_timer* t = new moe_timer;
  t->max_calls = max_calls;
  t->ev.resize(size_t(max_calls) * (MOE_STAGE_COUNT + 1));
  for (auto& e : t->ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto& f : t->ev)
        if (f) (void)hipEventDestroy(f);
      delete t;
      return fail(MOE_EHIP, "hipEventCreate failed");
    }
  }
  *out = t;
  return ok();
}

int moe_timer_destroy(moe_timer* t) {
  if (!t) return ok();
  for (auto& e : t->ev) (void)hipEventDestroy(e);
  delete t;
  return ok();
}

int moe_timer_reset(moe_timer* t) {
  REQUIRE(t, MOE_EINVAL, "timer is NULL");
  t->ncalls = 0;
  return ok();
}

int moe_timer_stage_ms(moe_timer* t, int stage, double* total_ms, int* calls) {
  REQUIRE(t && total_ms && stage >= 0 && stage < MOE_STAGE_COUNT, MOE_EINVAL, "bad timer query");
  double tot = 0;
  for (int c = 0; c < t->ncalls; ++c) {
    hipEvent_t a = t->ev[size_t(c) * (MOE_STAGE_COUNT + 1) + stage];
    hipEvent_t b = t->ev[size_t(c) * (MOE_STAGE_COUNT + 1) + stage + 1];
    MOE_HIP(hipEventSynchronize(b));
    float ms = 0;
    MOE_HIP(hipEventElapsedTime(&ms, a, b));
    tot += ms;
  }
  *total_ms = tot;
  if (calls) *calls = t->ncalls;
  return ok();
}

}  // extern "C"
