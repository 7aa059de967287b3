// Expert GEMMs: grouped / block-sparse (BCSR) / dense tiles on bf16 MFMA,
// with the epilogues that carry the layer's elementwise work.
//
//   first linear   h = act(r * (x_perm . W1_e))   or, SwiGLU,
//                  h = silu(r * x_perm.W1_e) * (r * x_perm.W3_e)
//   second linear  y = g * (h . W2_e)
//   router scores  s = r * (x . K)                (fp32 output)
//
// CODA sparse-MoE thread: the RMSNorm statistic r is commuted across the
// first expert GEMM into its epilogue (it reaches the experts with the
// dispatched rows), and the other per-row factors that straddle the
// dispatch / combine boundary -- the gate -- go into the second GEMM's
// epilogue, so combine is a plain sum.
//
// Every tile of every group comes from a device-built tile list (expert row
// counts are only known on the device), so one launch covers all experts
// with no host round trip.  For the BCSR kind the list is produced by
// walking the topology of the "Variable-size experts" nanoMOE notes
// (sections 3-4): first linear = one tile per run of nonzero column blocks
// of a token-block row (SDD), second linear = one tile per token-block row
// and output slice, with K over that row's nonzero blocks (DSD); two
// consecutive token-block rows of an expert that hold the same column blocks
// share their tiles (256 rows).  The last round of a persistent launch may
// cut its tiles along K into pieces whose fp32 partials k_piece_fixup sums.
//
// Tiling for gfx950: a 256 x 256 output tile per workgroup of 8 wave64s (a
// 4 x 2 grid of 64 x 128 wave tiles; a 4-wave 256 x 128 variant serves
// dense second linears with fewer 256-row tiles than compute units).
// Operands are both K-contiguous (weights packed as [features, K]) and move
// global -> LDS by the buffer_load_dwordx4 ... lds DMA into LDS rings (three
// stages of weights, two of activations) with a 16-byte-chunk XOR swizzle
// (conflict-free for the 64-bank LDS), so no registers are spent on staging.
// v_mfma_f32_32x32x16_bf16 takes the
// weights as the A operand (features = MFMA rows) and tokens as B (MFMA
// columns), so a lane's accumulators hold four consecutive features of one
// token and the epilogue stores 8 bytes per group.  Fragments of the next
// K sub-step are read from LDS while the current MFMAs run.  Tiles are
// remapped so that each XCD (workgroup id mod 8) runs a contiguous run of
// the list: the row tiles that share a weight tile run together in one L2.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {
namespace {


__device__ __forceinline__ float apply_act(float z, int act) {
  return act == 1 ? gelu_tanh(z) : gelu_erf(z);
}

// Epilogue shared by the GEMM kernels: lane holds token column (lane & 31) of
// each 32x32 block and features 8 g + 4 (lane >> 5) + {0..3} for g = 0..3.
template <int BF, int BT, int WGF, int WGT, int EPI, int MF, int MT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, const Tile& tile,
                                              f32x16 (&acc)[MF][MT], int wf, int wt, int fr,
                                              int fh) {
  constexpr int WTF = BF / WGF, WTT = BT / WGT;
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int row = tile.row0 + wt * WTT + j * 32 + fr;
    if (row >= tile.row_end) continue;
    float rs = 1.f;
    if (EPI == EPI_ACT || EPI == EPI_SWIGLU) rs = a.row_r[row];
    if (EPI == EPI_SCALE_F32) rs = a.row_r ? a.row_r[row] : 1.f;
    if (EPI == EPI_GATE) rs = a.row_w ? a.row_w[row] : 1.f;
    if ((EPI == EPI_SWIGLU || EPI == EPI_ACT) && a.pre) {
      // pre-activations for the backward pass, in the packed feature order
      uint16_t* P = static_cast<uint16_t*>(a.pre) + int64_t(row) * a.ldpre +
                    (EPI == EPI_SWIGLU ? 2 : 1) * tile.ocol0 + wf * WTF;
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int v = g * 4;
          const uint32_t lo = pk_bf16(rs * acc[i][j][v], rs * acc[i][j][v + 1]);
          const uint32_t hi = pk_bf16(rs * acc[i][j][v + 2], rs * acc[i][j][v + 3]);
          *reinterpret_cast<uint2*>(P + i * 32 + g * 8 + fh * 4) = make_uint2(lo, hi);
        }
    }
    if (EPI == EPI_SWIGLU) {
      uint16_t* Y = static_cast<uint16_t*>(a.Y) + int64_t(row) * a.ldy + tile.ocol0 + wf * (WTF / 2);
#pragma unroll
      for (int p = 0; p < MF / 2; ++p)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t pk[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float o[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int v = g * 4 + h * 2 + e;
              const float gate = rs * acc[2 * p][j][v];
              const float up = rs * acc[2 * p + 1][j][v];
              o[e] = silu(gate) * up;
            }
            pk[h] = pk_bf16(o[0], o[1]);
          }
          *reinterpret_cast<uint2*>(Y + p * 32 + g * 8 + fh * 4) = make_uint2(pk[0], pk[1]);
        }
    } else if (EPI == EPI_SCALE_F32) {
      float* Y = static_cast<float*>(a.Y) + int64_t(row) * a.ldy + tile.ocol0 + wf * WTF +
                 int64_t(tile.spare) * a.ysplit;
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 o;
          o.x = rs * acc[i][j][g * 4 + 0];
          o.y = rs * acc[i][j][g * 4 + 1];
          o.z = rs * acc[i][j][g * 4 + 2];
          o.w = rs * acc[i][j][g * 4 + 3];
          *reinterpret_cast<float4*>(Y + i * 32 + g * 8 + fh * 4) = o;
        }
    } else {
      uint16_t* Y = static_cast<uint16_t*>(a.Y) + int64_t(row) * a.ldy + tile.ocol0 + wf * WTF;
      // one loop nest per activation, chosen by a uniform branch: inside the
      // unrolled loop a runtime choice would be if-converted into computing
      // both activations of every value
      auto store_rows = [&](auto act_c) __attribute__((always_inline)) {
        constexpr int ACT = decltype(act_c)::value;
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if (EPI == EPI_STORE_T && wf * WTF + i * 32 >= tile.spare) continue;   // missing features
            uint32_t pk[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float o[2];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const float z = rs * acc[i][j][g * 4 + h * 2 + e];
                o[e] = EPI != EPI_ACT ? z : ACT == 1 ? gelu_tanh(z) : gelu_erf(z);
              }
              pk[h] = pk_bf16(o[0], o[1]);
            }
            *reinterpret_cast<uint2*>(Y + i * 32 + g * 8 + fh * 4) = make_uint2(pk[0], pk[1]);
          }
      };
      if (EPI == EPI_ACT && a.act == 1) store_rows(std::integral_constant<int, 1>{});
      else store_rows(std::integral_constant<int, 0>{});
    }
  }
}

// EPI_SCALE_F32 epilogue through LDS: the tile's fp32 rows are written by
// the waves that hold them (one 128-row half at a time, 128 KB), then every
// wave stores whole rows (1 KB per instruction, contiguous) instead of 32
// bytes of each of 32 rows.  r scales each row as it is stored.  The row
// pitch carries 4 floats of padding, so the fragment writes (32 rows at a
// time) spread over the banks.
template <int BF, int BT, int WGF, int WGT, int MF, int MT>
__device__ __forceinline__ void epilogue_f32_lds(const GemmArgs& a, const Tile& tile,
                                                 f32x16 (&acc)[MF][MT], int wf, int wt, int fr,
                                                 int fh, int lane, int wid, float* st) {
  constexpr int WTF = BF / WGF, WTT = BT / WGT, NW = WGF * WGT;
  constexpr int P = BF + 4;                     // row pitch (floats)
  static_assert(BF == 256 && WTT * P * 4 <= 160 * 1024, "one 256-feature half tile in LDS");
#pragma unroll
  for (int h = 0; h < WGT; ++h) {
    if (wt == h) {
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 o = {acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                             acc[i][j][g * 4 + 3]};
            *reinterpret_cast<f32x4*>(st + (j * 32 + fr) * P + wf * WTF + i * 32 + g * 8 + fh * 4) = o;
          }
    }
    __syncthreads();
    for (int r = wid; r < WTT; r += NW) {
      const int row = tile.row0 + h * WTT + r;
      if (row >= tile.row_end) break;
      const float rs = a.row_r ? a.row_r[row] : 1.f;
      f32x4 v = *reinterpret_cast<const f32x4*>(st + r * P + lane * 4);
      v *= rs;
      float* Y = static_cast<float*>(a.Y) + int64_t(row) * a.ldy + tile.ocol0 +
                 int64_t(tile.spare) * a.ysplit;
      *reinterpret_cast<f32x4*>(Y + lane * 4) = v;
    }
    __syncthreads();
  }
}

// Fixup of split tiles (the second linear's gate epilogue): one wave per
// 32 x 32 block of a split tile -- item (g, w, i, j): tile g, GEMM wave w,
// its block (i, j) -- four items per workgroup, so that the loads of every
// part of a block are in flight together.  The parts are summed in part order
// (part 0 first: the same fp32 sum every run), then the block is gated and
// stored as the GEMM's own epilogue stores it.  counters[g] is the list entry
// of the tile's part 0; a.ntiles[10] holds the number of split tiles.
constexpr int kFixupMaxParts = 8;

template <int BF, int BT, int WGF, int WGT>
__global__ void __launch_bounds__(256) k_piece_fixup(GemmArgs a) {
  constexpr int WTF = BF / WGF, WTT = BT / WGT;
  constexpr int MF = WTF / 32, MT = WTT / 32;
  constexpr int NI = WGF * WGT * MF * MT;       // items per tile
  const int item = int(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int g = item / NI;
  if (g >= a.ntiles[10]) return;
  const int r = item - g * NI;
  const int wid = r / (MF * MT), ij = r - wid * (MF * MT);
  const int i = ij / MT, j = ij - i * MT;
  const Tile tile = a.tiles[a.counters[g]];
  const int lane = threadIdx.x & 63, fr = lane & 31, fh = lane >> 5;
  const int wt = wid / WGF, wf = wid % WGF;
  const int np = tile.nparts;
  const f32x4* const src = reinterpret_cast<const f32x4*>(
      a.part + int64_t(tile.pslot0) * (int64_t(BF) * BT) + piece_frag_offset<BF, BT, MF, MT>(wid, lane, i, j));
  constexpr int PS = BF * BT / 4;               // f32x4 between parts
  f32x4 v[kFixupMaxParts][4];
#pragma unroll
  for (int pt = 0; pt < kFixupMaxParts; ++pt)
    if (pt < np)
#pragma unroll
      for (int q = 0; q < 4; ++q) v[pt][q] = src[pt * PS + q];
  f32x4 acc[4] = {v[0][0], v[0][1], v[0][2], v[0][3]};
#pragma unroll
  for (int pt = 1; pt < kFixupMaxParts; ++pt)
    if (pt < np)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += v[pt][q];
  const int row = tile.row0 + wt * WTT + j * 32 + fr;
  if (row >= tile.row_end) return;
  const float rs = a.row_w ? a.row_w[row] : 1.f;
  uint16_t* Y = static_cast<uint16_t*>(a.Y) + int64_t(row) * a.ldy + tile.ocol0 + wf * WTF + i * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<uint2*>(Y + q * 8 + fh * 4) =
        make_uint2(pk_bf16(rs * acc[q][0], rs * acc[q][1]), pk_bf16(rs * acc[q][2], rs * acc[q][3]));
}

// Word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle;
// reads past num_records return zero).
constexpr int kRsrcWord3Raw = 0x00020000;

// One 16-byte-per-lane DMA from a buffer resource into LDS (lane i's bytes
// at dst + 16 i).  Kept out of line of the kernel template: with the builtin
// written in the template's lambdas, the host pass emitted no launch stubs.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_void_ptr dst, uint32_t voff,
                                      int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// ---------------------------------------------------------------- bf16 MFMA GEMM, LDS-DMA ring

// BF features x BT rows per workgroup, WGF x WGT waves, each wave a
// (BF / WGF) x (BT / WGT) sub-tile of 32 x 32 MFMA blocks, K in stages of 64.
// Global -> LDS moves by the buffer_load_dwordx4 ... lds DMA (each wave
// instruction writes 1 KB of LDS, lane i at byte 16 i).  The weights go
// through a ring of three LDS stages and the activation rows through two
// (3 x 32 KB + 2 x 32 KB = the whole 160 KB of a CU at 256 x 256): the
// weights stream from HBM and get two stages of lookahead, the activation
// rows (L2-resident) one.  Every wave moves its share of both operands, the
// activation segments first, so at a barrier vmcnt(weight segments) leaves
// only the newest weight stage in flight.  One barrier per stage, before its
// last K sub-step: by then every wave holds that sub-step's fragments, so
// behind the barrier its MFMAs cover the next stage's first fragment reads
// and the refill of the two buffers just drained.
template <int BF, int BT, int WGF, int WGT, int EPI>
__global__ void __launch_bounds__(64 * WGF * WGT, 1) k_gemm_bf16_dma(GemmArgs a) {
  constexpr int NW = WGF * WGT;
  constexpr int WTF = BF / WGF, WTT = BT / WGT;
  constexpr int MF = WTF / 32, MT = WTT / 32;
  constexpr int BKD = 64;                       // K per stage
  constexpr int C = BKD / 8;                    // 16-byte chunks per LDS row
  constexpr int RSEG = 64 / C;                  // rows per 1 KB DMA segment
  constexpr int SPW = BF / RSEG / NW;           // weight segments per wave per stage
  constexpr int SPX = BT / RSEG / NW;           // activation segments per wave per stage
  constexpr int WS = BF * BKD, XS = BT * BKD;   // elements per stage buffer
  constexpr int KS = BKD / 16;                  // MFMA sub-steps per stage
  static_assert(SPW * RSEG * NW == BF && SPX * RSEG * NW == BT, "segments must divide among waves");
  static_assert(MF >= 1 && MT >= 1 && MT <= 4, "wave tile of 1..4 row blocks");
  static_assert(EPI != EPI_SWIGLU || MF % 2 == 0, "SwiGLU needs gate/up block pairs per wave");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[3 * WS + 2 * XS];
  uint16_t* const ldsx = lds + 3 * WS;

  // Persistent: workgroup b takes tiles b, b + G, b + 2 G, ... of the remapped
  // list (G a multiple of 8, so all of them come from its own XCD's run).
  // The first loads of the next tile are issued before this tile's
  // epilogue, so their latency hides behind the epilogue's arithmetic and
  // stores.
  // The tile list either follows the XCD remap of list index tb = b, b + G,
  // ... (remap_xcd), or, planned for this grid (xcd_runs), gives each XCD's
  // run explicitly: entries base[x] + slot, + S, ... with x = b % NX.
  const int nt = a.ntiles[0];
  const int G = gridDim.x;
  const int NX = a.xcd_runs && G % 8 == 0 ? 8 : 1;
  const int S = G / NX;
  const int run_end = a.xcd_runs ? a.ntiles[2 + int(blockIdx.x) % NX] : nt;
  int tb = a.xcd_runs ? a.ntiles[1 + int(blockIdx.x) % NX] + int(blockIdx.x) / NX : int(blockIdx.x);
  const int step = a.xcd_runs ? S : G;
  auto list_index = [&](int i) { return a.xcd_runs ? i : remap_xcd(i, nt); };
  if (tb >= run_end) return;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (the LDS destinations of the DMA are then scalar arithmetic)
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves wid and wid + 4 share a SIMD: give them the same feature rows and
  // the two row halves, so that a tile with few rows still keeps every SIMD
  // equally busy
  const int wt = wid / WGF, wf = wid % WGF;
  const uint16_t* __restrict__ X = static_cast<const uint16_t*>(a.X);
  const uint16_t* __restrict__ W = static_cast<const uint16_t*>(a.W);
  const int srow = lane / C;                  // row within a segment
  const int fr = lane & 31, fh = lane >> 5, fswz = chunk_swz<C>(lane & 15);

  // Operands through raw buffer resources over the whole weight and
  // activation arrays (x_bytes, w_bytes: each below 4 GiB): a 32-bit byte
  // offset per lane and segment, set per tile, and the stage step in the
  // scalar offset.  Every address stays inside the arrays (rows are clamped
  // to the tile's last row, gathered rows are token rows, weight rows end at
  // a whole tile); the extents make the hardware return zeros past them.
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(W), 0, int(uint32_t(a.w_bytes)), kRsrcWord3Raw);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, int(uint32_t(a.x_bytes)), kRsrcWord3Raw);
  uint32_t vw[SPW], vx[SPX];
  auto set_sources = [&](const Tile& t) {
    const int xlast = t.row_end - 1;
    // a K-split tile reads its own part of the activation row
    const int xk0 = (EPI == EPI_SCALE_F32 ? t.spare * t.klen : 0) + t.xk;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int row = (wid * SPW + u) * RSEG + srow;
      // a partial feature tile (EPI_STORE_T) reads its last existing weight
      // row in place of the missing ones
      const int wr = EPI == EPI_STORE_T ? min(row, t.spare - 1) : row;
      vw[u] = uint32_t((int64_t(t.wrow0 + wr) * a.ldw + t.kofs + ((lane % C) ^ chunk_swz<C>(row)) * 8) * 2);
    }
#pragma unroll
    for (int u = 0; u < SPX; ++u) {
      const int row = (wid * SPX + u) * RSEG + srow;
      // with a row map the rows are gathered from the token rows (dispatch
      // fused here)
      int xr = min(t.row0 + row, xlast);
      if (a.xrow) xr = max(a.xrow[xr], 0);
      vx[u] = uint32_t((int64_t(xr) * a.ldx + xk0 + ((lane % C) ^ chunk_swz<C>(row)) * 8) * 2);
    }
  };
  auto issue_w = [&](int kt, int buf) {
    uint16_t* base = lds + buf * WS;
#pragma unroll
    for (int u = 0; u < SPW; ++u)
      dma16(rw, (lds_void_ptr)(base + (wid * SPW + u) * 512), vw[u], kt * BKD * 2);
  };
  auto issue_x = [&](int kt, int buf) {
    uint16_t* base = ldsx + buf * XS;
#pragma unroll
    for (int u = 0; u < SPX; ++u)
      dma16(rx, (lds_void_ptr)(base + (wid * SPX + u) * 512), vx[u], kt * BKD * 2);
  };
  // stages 0 and 1 of both operands and stage 2 of the weights (past the
  // last stage a load repeats stage nk - 1, in bounds, into a buffer that is
  // not read again)
  auto prologue = [&](int nk) {
    issue_x(0, 0);
    issue_w(0, 0);
    issue_x(min(1, nk - 1), 1);
    issue_w(min(1, nk - 1), 1);
    issue_w(min(2, nk - 1), 2);
  };

  Tile tile = a.tiles[list_index(tb)];
  int nk = tile.klen / BKD;
  set_sources(tile);
  if (nk > 0) prologue(nk);
  bool first = true;
  f32x16 acc[MF][MT];
  for (;;) {
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    // Row blocks of this wave that hold rows of the tile: a partial tile (the
    // last rows of an expert) skips the MFMAs and fragment reads of the rest,
    // whose results the epilogue never stores.  One copy of the loop per count
    // keeps the inner loop free of branches.
    const int mta = __builtin_amdgcn_readfirstlane(
        max(0, min(MT, (tile.row_end - tile.row0 - wt * WTT + 31) / 32)));
    auto main_loop = [&](auto mta_c) {
      constexpr int MTA = decltype(mta_c)::value;
      bf16x8 af[2][MF], bfr[2][MT];
#define MOE_FRAGS2(SW, SX, KSV, SLOT)                                                          \
      {                                                                                      \
        const int qo_ = ((2 * (KSV) + fh) ^ fswz) * 8;                                       \
        _Pragma("unroll") for (int i = 0; i < MF; ++i)                                       \
          af[SLOT][i] = *reinterpret_cast<const bf16x8*>((SW) + (wf * WTF + i * 32 + fr) * BKD + qo_); \
        _Pragma("unroll") for (int j = 0; j < MTA; ++j)                                      \
          bfr[SLOT][j] = *reinterpret_cast<const bf16x8*>((SX) + (wt * WTT + j * 32 + fr) * BKD + qo_); \
      }
#define MOE_MFMA2(I, J, KSV)                                                                   \
      acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[(KSV) & 1][I], bfr[(KSV) & 1][J], \
                                                          acc[I][J], 0, 0, 0);
      if (nk > 0) {
        // stage 0 has landed (after the previous tile's epilogue its stores
        // are counted too, so everything is waited for)
        if (first) MOE_WAIT_VMCNT(SPX + 2 * SPW);
        else MOE_WAIT_VMCNT(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (MTA > 0) MOE_FRAGS2(lds, ldsx, 0, 0)
        __builtin_amdgcn_sched_barrier(0);
        int wb = 0;                              // weight buffer of stage kt (kt % 3)
        // every stage but the last; the body has no branch, so the refills and
        // the next stage's first fragment reads are scheduled between the last
        // sub-step's MFMAs
        for (int kt = 0; kt + 1 < nk; ++kt) {
          const uint16_t* sw = lds + wb * WS;
          const uint16_t* sx = ldsx + (kt & 1) * XS;
          const int wn = wb == 2 ? 0 : wb + 1;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) {
              if (MTA > 0) MOE_FRAGS2(sw, sx, ks + 1, (ks + 1) & 1)
#pragma unroll
              for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < MTA; ++j) MOE_MFMA2(i, j, ks)
              if (MTA > 0) sched_interleave<MF + MTA, MF * MTA>();
            } else {
              // this wave's reads of stage kt are in registers and its share
              // of stage kt + 1 has landed (in flight: the weights of stage
              // kt + 2); after the barrier the same holds for every wave, so
              // the buffers of stage kt may be refilled
              MOE_WAIT_VMCNT(SPW);
              __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
              asm volatile("" ::: "memory");
              __builtin_amdgcn_s_barrier();
              asm volatile("" ::: "memory");
              // the next stage's first fragment reads under the first row of
              // MFMAs, then the refills under the rest
              if (MTA > 0) MOE_FRAGS2(lds + wn * WS, ldsx + ((kt + 1) & 1) * XS, 0, 0)
#pragma unroll
              for (int j = 0; j < MTA; ++j) MOE_MFMA2(0, j, ks)
              if (MTA > 0) sched_interleave<MF + MTA, MTA>();
              __builtin_amdgcn_sched_barrier(0);
              issue_x(min(kt + 2, nk - 1), kt & 1);
              issue_w(min(kt + 3, nk - 1), wb);
#pragma unroll
              for (int i = 1; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < MTA; ++j) MOE_MFMA2(i, j, ks)
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          wb = wn;
        }
        {
          const uint16_t* sw = lds + wb * WS;
          const uint16_t* sx = ldsx + ((nk - 1) & 1) * XS;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS && MTA > 0) MOE_FRAGS2(sw, sx, ks + 1, (ks + 1) & 1)
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
              for (int j = 0; j < MTA; ++j) MOE_MFMA2(i, j, ks)
            if (ks + 1 < KS && MTA > 0) sched_interleave<MF + MTA, MF * MTA>();
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
#undef MOE_MFMA2
#undef MOE_FRAGS2
    };
    if (mta >= MT) main_loop(std::integral_constant<int, MT>{});
    else if (mta == 3) main_loop(std::integral_constant<int, (MT > 3 ? 3 : MT)>{});
    else if (mta == 2) main_loop(std::integral_constant<int, (MT > 2 ? 2 : MT)>{});
    else if (mta == 1) main_loop(std::integral_constant<int, 1>{});
    else main_loop(std::integral_constant<int, 0>{});
    // every wave's LDS reads of this tile are in registers and its DMA has
    // landed: after the barrier the next tile may refill any buffer
    MOE_WAIT_VMCNT(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int tn = tb + step;
    const bool more = tn < run_end;
    Tile next = tile;
    int nk2 = 0;
    if constexpr (EPI == EPI_SCALE_F32 && WGT == 2 && BT == 256) {
      // fp32 rows staged through the (now idle) LDS, so that every store
      // writes whole rows; the next tile's loads wait for the LDS
      epilogue_f32_lds<BF, BT, WGF, WGT>(a, tile, acc, wf, wt, fr, fh, lane, wid,
                                         reinterpret_cast<float*>(lds));
      if (!more) break;
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      next = a.tiles[list_index(tn)];
      nk2 = next.klen / BKD;
      set_sources(next);
      if (nk2 > 0) prologue(nk2);
    } else if (tile.nparts > 1) {
      // a K piece: its partial sums go to the partial buffer, and the fixup
      // kernel applies the epilogue to the sum of the tile's pieces
      if (more) {
        next = a.tiles[list_index(tn)];
        nk2 = next.klen / BKD;
        set_sources(next);
        if (nk2 > 0) prologue(nk2);
      }
      store_piece<BF, BT, MF, MT>(a, tile, acc, wid, lane);
      if (!more) break;
    } else {
      if (more) {
        next = a.tiles[list_index(tn)];
        nk2 = next.klen / BKD;
        set_sources(next);
        if (nk2 > 0) prologue(nk2);
      }
      gemm_epilogue<BF, BT, WGF, WGT, EPI>(a, tile, acc, wf, wt, fr, fh);
      if (!more) break;
    }
    tile = next;
    nk = nk2;
    tb = tn;
    first = false;
  }
}

// ---------------------------------------------------------------- fp32 SIMT GEMM

// Tile: 64 output columns x 64 rows, K step 16.  SwiGLU tiles read 128 packed
// rows (gate rows 32 g + c, up rows 32 g + 32 + c of each 64-row group).
template <int EPI>
__global__ void __launch_bounds__(256) k_gemm_f32(GemmArgs a) {
  constexpr int NW = EPI == EPI_SWIGLU ? 128 : 64;
  __shared__ float sW[16][NW + 4];
  __shared__ float sX[16][64 + 4];
  const int nt = *a.ntiles;
  if (int(blockIdx.x) >= nt) return;
  const Tile tile = a.tiles[remap_xcd(blockIdx.x, nt)];
  const float* __restrict__ X = static_cast<const float*>(a.X);
  const float* __restrict__ W = static_cast<const float*>(a.W);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4], accu[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = accu[i][j] = 0.f;
  const int lr = tid >> 2, lq = tid & 3;   // 64 rows x 4 float4 chunks
  for (int k0 = 0; k0 < tile.klen; k0 += 16) {
    // W rows -> sW[k][col]; col c < 64: gate (or plain) row; c >= 64: up row
#pragma unroll
    for (int half = 0; half < NW / 64; ++half) {
      const int c = lr;
      const int prow = EPI == EPI_SWIGLU ? (c / 32) * 64 + (c % 32) + half * 32 : c;
      const float4 v = *reinterpret_cast<const float4*>(
          W + int64_t(tile.wrow0 + prow) * a.ldw + tile.kofs + k0 + lq * 4);
      sW[lq * 4 + 0][half * 64 + c] = v.x;
      sW[lq * 4 + 1][half * 64 + c] = v.y;
      sW[lq * 4 + 2][half * 64 + c] = v.z;
      sW[lq * 4 + 3][half * 64 + c] = v.w;
    }
    {
      int row = min(tile.row0 + lr, tile.row_end - 1);
      if (a.xrow) row = max(a.xrow[row], 0);
      const float4 v = *reinterpret_cast<const float4*>(X + int64_t(row) * a.ldx + k0 + lq * 4);
      sX[lq * 4 + 0][lr] = v.x;
      sX[lq * 4 + 1][lr] = v.y;
      sX[lq * 4 + 2][lr] = v.z;
      sX[lq * 4 + 3][lr] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float wv[4], uv[4], xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wv[i] = sW[kk][tx + 16 * i];
        if (EPI == EPI_SWIGLU) uv[i] = sW[kk][64 + tx + 16 * i];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = sX[kk][ty + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(wv[i], xv[j], acc[i][j]);
          if (EPI == EPI_SWIGLU) accu[i][j] = fmaf(uv[i], xv[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = tile.row0 + ty + 16 * j;
    if (row >= tile.row_end) continue;
    float rs = 1.f;
    if (EPI == EPI_ACT || EPI == EPI_SWIGLU) rs = a.row_r[row];
    if (EPI == EPI_SCALE_F32) rs = a.row_r ? a.row_r[row] : 1.f;
    if (EPI == EPI_GATE) rs = a.row_w ? a.row_w[row] : 1.f;
    float* Y = static_cast<float*>(a.Y) + int64_t(row) * a.ldy + tile.ocol0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tx + 16 * i;
      float o;
      if (EPI == EPI_SWIGLU) o = silu(rs * acc[i][j]) * (rs * accu[i][j]);
      else if (EPI == EPI_ACT) o = apply_act(rs * acc[i][j], a.act);
      else o = rs * acc[i][j];
      Y[c] = o;
    }
  }
}

// ---------------------------------------------------------------- tile plans

__device__ __forceinline__ int upper_bound_i(const int* a, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

constexpr int kPlanMax = 4096;   // experts (grouped) or token-block rows (BCSR)
constexpr int kPlanOffsMax = 2048;   // experts of a grouped / BCSR layer

// Position of the n-th tile of a group of mt row tiles x nf column tiles.
// A group of at most kRowBlock row tiles runs row tile fastest, so the tiles
// an XCD runs together share each weight tile through L2 and hold all of the
// group's rows.  A taller group (a dense shared FFN over every token, a hot
// expert) runs in blocks of kRowBlock row tiles, column tile next, so that a
// window of 32 tiles reads 8 row tiles and 4 weight tiles instead of 32 row
// tiles and one weight tile.
constexpr int kRowBlock = 8;
__device__ __forceinline__ void tile_coords(int n, int mt, int nf_total, int* m, int* nf) {
  if (mt <= kRowBlock) {
    *nf = n / mt;
    *m = n - *nf * mt;
    return;
  }
  const int blk = n / (kRowBlock * nf_total);
  const int rem = n - blk * kRowBlock * nf_total;
  const int rows = min(kRowBlock, mt - blk * kRowBlock);
  *nf = rem / rows;
  *m = blk * kRowBlock + (rem - *nf * rows);
}

// Workgroup `slice` of `nslices` writes list entries slice * blockDim + tid,
// stepping by nslices * blockDim; every workgroup computes the per-unit
// counts and the XCD runs itself (a few reads of the offsets), and slice 0
// writes the list's header.
// BCSR with tiles of two token blocks (bt = 2 block): token-block rows pair
// up within an expert (its blocks 0-1, 2-3, ...), and a pair shares its tiles
// when both topology rows hold the same column blocks.  Returns the rows'
// share: 2 = first row of a pair (its tiles span both rows), 0 = second row
// of a pair (no tiles of its own), 1 = a row on its own.
__device__ __forceinline__ int bcsr_span(const PlanArgs& p, const int* offs, int u) {
  if (p.bt < 2 * p.block) return 1;
  const int row = u * p.block;
  const int e = upper_bound_i(offs, p.E + 1, row) - 1;
  const int i = (row - offs[e]) / p.block;
  const int u0 = u - (i & 1);
  if ((u0 + 1) * p.block >= offs[e + 1]) return 1;   // no second block
  const int f0 = p.row_offsets[u0], f1 = p.row_offsets[u0 + 1];
  const int nz = f1 - f0;
  if (p.row_offsets[u0 + 2] - f1 != nz) return 1;
  bool same = true;
#pragma unroll 4
  for (int c = 0; c < nz; ++c) same = same && p.column_indices[f0 + c] == p.column_indices[f1 + c];
  if (!same) return 1;
  return (i & 1) ? 0 : 2;
}

// Cost model of a grouped unit's tiles for splitting a list over the XCDs:
// a tile costs (kTileCost0 + its 32-row blocks) per K stage (the kernels skip
// the row blocks past a tile's end; kTileCost0 stands for the per-stage work
// that does not shrink with the rows: the weight stage and the barrier).  A
// unit with a single row tile shares no weight tile with another row tile,
// so each of its tiles streams its weights alone and is priced as a full
// tile.  The row tiles of a unit hold rt rows each but the last, which holds
// the rest (the even split of the planner below).
constexpr int kTileCost0 = 4;
struct UnitCost {
  int mt, nf;        // row tiles, column tiles
  int wf, wl;        // cost per K stage of a row tile that is not the last / of the last
  int nk;            // K stages per tile
};

__device__ __forceinline__ UnitCost unit_cost_shape(const PlanArgs& p, int rows, int nf, int fsize) {
  UnitCost c{};
  c.mt = (rows + p.bt - 1) / p.bt;
  c.nf = nf;
  if (c.mt == 0) return c;
  const int rt = min(p.bt, ((rows + c.mt - 1) / c.mt + 31) / 32 * 32);
  const int ks = p.kstage > 0 ? p.kstage : 64;
  const int km = p.kmul > 0 ? p.kmul : 1;
  c.wf = kTileCost0 + rt / 32;
  c.wl = c.mt == 1 ? kTileCost0 + p.bt / 32 : kTileCost0 + (rows - (c.mt - 1) * rt + 31) / 32;
  c.nk = p.gemm == 1 ? p.d / ks : km * fsize / ks;
  return c;
}

// Packed in two words for LDS: (mt, nf) and (wf, wl, nk).
__device__ __forceinline__ void unit_cost_pack(const UnitCost& c, int* w0, int* w1) {
  *w0 = (c.mt << 16) | c.nf;
  *w1 = (c.wf << 24) | (c.wl << 16) | c.nk;
}
__device__ __forceinline__ UnitCost unit_cost_unpack(int w0, int w1) {
  UnitCost c;
  c.mt = int(unsigned(w0) >> 16);
  c.nf = w0 & 0xFFFF;
  c.wf = int(unsigned(w1) >> 24);
  c.wl = (w1 >> 16) & 0xFF;
  c.nk = w1 & 0xFFFF;
  return c;
}

// Cost of the unit's first n tiles in list order (tile_coords), in K-stage
// units.
__device__ __forceinline__ long long unit_cost_prefix(const UnitCost& c, int n) {
  if (c.mt == 0 || n <= 0) return 0;
  if (n >= c.mt * c.nf) return (long long)c.nf * ((c.mt - 1) * c.wf + c.wl) * c.nk;
  long long pre;
  if (c.mt <= kRowBlock) {
    const int g = n / c.mt, i = n - g * c.mt;           // i < mt: tiles 0 .. i-1 are not the last
    pre = (long long)g * ((c.mt - 1) * c.wf + c.wl) + (long long)i * c.wf;
  } else {
    const int blk = n / (kRowBlock * c.nf);
    const int rem = n - blk * kRowBlock * c.nf;
    const int rows_b = min(kRowBlock, c.mt - blk * kRowBlock);
    const bool last_blk = (blk + 1) * kRowBlock >= c.mt;
    const long long wblk = (long long)(rows_b - 1) * c.wf + (last_blk ? c.wl : c.wf);
    const int col = rows_b > 0 ? rem / rows_b : 0, i = rem - col * rows_b;
    pre = (long long)blk * c.nf * kRowBlock * c.wf + col * wblk + (long long)i * c.wf;
  }
  return pre * c.nk;
}

// The unit's tile index (0 .. cnt) whose cost prefix is nearest to `want`
// (to within one tile), in closed form: whole blocks of row tiles, whole
// columns of the block, then row tiles of the column.  In double precision:
// the costs stay far below 2^53, and 64-bit integer division is a long
// software sequence on the GPU.
__device__ __forceinline__ int unit_cost_find(const UnitCost& c, int cnt, long long want) {
  if (c.mt == 0 || cnt == 0 || want <= 0) return 0;
  const double w = double(want) / c.nk;                 // in cost-per-stage units
  double blk = 0, rem = w;
  int rows_b = c.mt;
  if (c.mt > kRowBlock) {
    const int nblk = (c.mt + kRowBlock - 1) / kRowBlock;
    const double full = double(c.nf) * kRowBlock * c.wf;   // a block without the last row tile
    blk = fmin(double(nblk - 1), floor(w / full));
    rem = w - blk * full;
    rows_b = min(kRowBlock, c.mt - int(blk) * kRowBlock);
  }
  const bool last_blk = c.mt <= kRowBlock || (int(blk) + 1) * kRowBlock >= c.mt;
  const double gc = double(rows_b - 1) * c.wf + (last_blk ? c.wl : c.wf);   // one column
  const double col = fmin(double(c.nf - 1), floor(rem / gc));
  const double r = rem - col * gc;
  const double i = fmin(double(rows_b - 1), floor(r / c.wf + 0.5));
  const double n = blk * kRowBlock * c.nf + col * rows_b + i;
  return int(fmin(double(cnt), fmax(0.0, n)));
}

__device__ __forceinline__ void plan_tiles(const PlanArgs& p, int slice, int nslices) {
  __shared__ int base_s[kPlanMax + 1];
  __shared__ unsigned char span_s[kPlanMax];   // BCSR: bcsr_span of each token-block row
  __shared__ int offs_s[kPlanOffsMax + 1];      // BCSR: the expert row offsets
  __shared__ long long cost_s[kPlanOffsMax + 1];  // cost split: unit costs, then their prefix
  __shared__ int shape_s[kPlanOffsMax];           // cost split: second word of each unit's shape
  int* const shape0_s = offs_s;                   // (its first word; offs_s is BCSR-only)
  __shared__ long long sh[33];
  const bool dense = p.offsets == nullptr;
  const bool bcsr = !dense && p.row_offsets != nullptr;
  if (bcsr) {
    for (int e = threadIdx.x; e <= p.E; e += blockDim.x) offs_s[e] = p.offsets[e];
    __syncthreads();
  }
  const int pf = p.swiglu && p.gemm == 1 ? 2 : 1;   // packed rows per hidden unit
  const int km = p.kmul > 0 ? p.kmul : 1;            // second linear: K per hidden unit
  const int nunits = dense ? 1 : bcsr ? p.offsets[p.E] / p.block : p.E;
  // XCD runs split by cost (grouped lists of a persistent launch, no K split)
  const bool by_cost = p.cost_split && p.grid > 0 && !dense && !bcsr && p.ksplit <= 1 &&
                       nunits <= kPlanOffsMax;
  // per unit tile count, then exclusive scan (each thread owns a contiguous run)
  const int per = (nunits + blockDim.x - 1) / blockDim.x;
  const int lo = min(nunits, int(threadIdx.x) * per), hi = min(nunits, lo + per);
  long long local = 0, lcost = 0;
  for (int u = lo; u < hi; ++u) {
    int cnt;
    if (dense) {
      cnt = ((p.dense_rows + p.bt - 1) / p.bt) * ((p.dense_n + (p.ragged ? p.bf - 1 : 0)) / p.bf);
    } else if (bcsr) {
      const int nz = p.row_offsets[u + 1] - p.row_offsets[u];
      const int sp = bcsr_span(p, offs_s, u);
      span_s[u] = static_cast<unsigned char>(sp);
      cnt = sp == 0 ? 0 : p.gemm == 1 ? nz * p.block * pf / p.bf : p.d / p.bf;
    } else {
      const int rows = p.offsets[u + 1] - p.offsets[u];
      const int mt = (rows + p.bt - 1) / p.bt;
      const int nf = p.gemm == 1 ? ((p.foff[u + 1] - p.foff[u]) * pf + (p.ragged ? p.bf - 1 : 0)) / p.bf
                                 : p.d / p.bf;
      cnt = mt * nf * (p.gemm == 2 ? p.ksplit : 1);
      if (by_cost) {
        const UnitCost c = unit_cost_shape(p, rows, nf, p.foff[u + 1] - p.foff[u]);
        cost_s[u] = unit_cost_prefix(c, cnt);
        lcost += cost_s[u];
        unit_cost_pack(c, &shape0_s[u], &shape_s[u]);
      }
    }
    base_s[u] = cnt;
    local += cnt;
  }
  // exclusive scans of the tile counts and (by_cost) the unit costs
  long long total;
  {
    __shared__ long long shc[33];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    long long incl = local, inclc = lcost;
    for (int o = 1; o < 64; o <<= 1) {
      const long long u = __shfl_up(incl, o, 64);
      const long long uc = __shfl_up(inclc, o, 64);
      if (lane >= o) {
        incl += u;
        inclc += uc;
      }
    }
    if (lane == 63) {
      sh[wid] = incl;
      shc[wid] = inclc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      long long run = 0, runc = 0;
      for (int w = 0; w < nw; ++w) {
        const long long t = sh[w], tc = shc[w];
        sh[w] = run;
        shc[w] = runc;
        run += t;
        runc += tc;
      }
      sh[32] = run;
      shc[32] = runc;
    }
    __syncthreads();
    long long b = sh[wid] + incl - local, bc = shc[wid] + inclc - lcost;
    total = sh[32];
    for (int u = lo; u < hi; ++u) {
      const int c = base_s[u];
      base_s[u] = int(b);
      b += c;
      if (by_cost) {
        const long long cc = cost_s[u];
        cost_s[u] = bc;
        bc += cc;
      }
    }
    if (threadIdx.x == 0) {
      base_s[nunits] = int(total);
      if (by_cost) cost_s[nunits] = shc[32];
    }
  }
  __syncthreads();
  const int ntot = int(min<long long>(total, p.max_tiles));
  // Persistent launch of p.grid workgroups: the XCD remap gives each XCD a
  // contiguous run of the list, run S = grid / NX tiles at a time.  The
  // run's last round holds r = q % S tiles and leaves S - r compute units
  // idle for a whole tile; its r tiles are cut along K into P = S / r pieces
  // (at most max_parts), so the last round takes about 1 / P of a tile.
  __shared__ int xfirst_s[8], xfull_s[8], xp_s[8], xout_s[9], xgrp_s[8], xpc_s[8];
  int nout = ntot;
  const int NX = p.grid > 0 && p.grid % 8 == 0 ? 8 : 1;
  if (p.grid > 0) {
    const int S = p.grid / NX;
    // XCD x runs list entries [bound[x], bound[x + 1]): equal counts, or
    // (by_cost) boundaries at equal shares of the list's cost, each placed at
    // the tile boundary nearest to its share (one thread per boundary)
    __shared__ int bound_s[9];
    if (threadIdx.x <= NX) {
      const int x = threadIdx.x;
      const int q = ntot / NX, rem = ntot % NX;
      int bx = x == NX ? ntot : x * q + min(x, rem);
      if (by_cost && x > 0 && x < NX && cost_s[nunits] > 0) {
        const long long target = NX == 8 ? (cost_s[nunits] * x) >> 3 : cost_s[nunits] * x;
        int lo = 0, hi = nunits - 1;                    // last unit starting at or before target
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (cost_s[mid] <= target) lo = mid;
          else hi = mid - 1;
        }
        const UnitCost c = unit_cost_unpack(shape0_s[lo], shape_s[lo]);
        const int cnt = base_s[lo + 1] - base_s[lo];
        bx = min(ntot, base_s[lo] + unit_cost_find(c, cnt, target - cost_s[lo]));
      }
      bound_s[x] = bx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int bound[9];
      bound[0] = 0;
      for (int x = 1; x <= NX; ++x) bound[x] = max(bound[x - 1], min(ntot, bound_s[x]));
      bound[NX] = ntot;
      int out = 0, grp = 0, pcs = 0;
      for (int x = 0; x < NX; ++x) {
        const int qx = bound[x + 1] - bound[x];
        int r = qx % S;
        int P = r > 0 ? min(p.max_parts, S / r) : 1;
        if (P < 2) {
          P = 1;
          r = 0;
        }
        xfirst_s[x] = bound[x];
        xfull_s[x] = qx - r;
        xp_s[x] = P;
        xout_s[x] = out;
        xgrp_s[x] = grp;
        xpc_s[x] = pcs;
        out += (qx - r) + r * P;
        if (P > 1) {
          grp += r;
          pcs += r * P;
        }
      }
      xout_s[NX] = out;
      if (slice == 0) {
        p.ntiles[0] = out;
        for (int x = 0; x <= NX; ++x) p.ntiles[1 + x] = xout_s[x];
        p.ntiles[10] = grp;
      }
    }
    __syncthreads();
    nout = xout_s[NX];
  } else if (threadIdx.x == 0 && slice == 0) {
    *p.ntiles = ntot;
  }
  for (int o = slice * int(blockDim.x) + int(threadIdx.x); o < nout;
       o += nslices * int(blockDim.x)) {
    int idx = o, part = 0, nparts = 1, group = 0, pslot0 = 0;
    if (p.grid > 0) {
      int x = 0;
      while (x + 1 < NX && xout_s[x + 1] <= o) ++x;
      const int local = o - xout_s[x];
      if (local < xfull_s[x]) {
        idx = xfirst_s[x] + local;
      } else {
        const int j = local - xfull_s[x], P = xp_s[x], gl = j / P;
        part = j - gl * P;
        nparts = P;
        idx = xfirst_s[x] + xfull_s[x] + gl;
        group = xgrp_s[x] + gl;
        pslot0 = xpc_s[x] + gl * P;
      }
    }
    const int u = upper_bound_i(base_s, nunits + 1, idx) - 1;
    const int n = idx - base_s[u];
    Tile t{};
    t.spare = 0;
    if (dense) {
      const int mt = (p.dense_rows + p.bt - 1) / p.bt;
      const int nft = (p.dense_n + (p.ragged ? p.bf - 1 : 0)) / p.bf;
      int m, nf;
      tile_coords(n, mt, nft, &m, &nf);
      t.expert = 0;
      t.row0 = m * p.bt;
      t.row_end = min(p.dense_rows, t.row0 + p.bt);
      t.wrow0 = nf * p.bf;
      if (p.gemm == 1) {
        t.kofs = 0;
        t.klen = p.d;
        if (p.ragged) t.spare = min(p.bf, p.dense_n - nf * p.bf);
      } else {
        t.kofs = km * p.foff[0];
        t.klen = km * (p.foff[1] - p.foff[0]);
      }
      t.ocol0 = nf * p.bf / p.fold;
    } else if (bcsr) {
      const int first = p.row_offsets[u];
      const int cb0 = p.column_indices[first];
      const int e = upper_bound_i(p.block_offsets, p.E + 1, cb0) - 1;
      t.expert = e;
      t.row0 = u * p.block;
      t.row_end = t.row0 + span_s[u] * p.block;
      if (p.gemm == 1) {
        const int cb = p.column_indices[first + n * (p.bf / (p.block * pf))];
        t.wrow0 = cb * p.block * pf;
        t.kofs = 0;
        t.klen = p.d;
        t.ocol0 = (cb - p.block_offsets[e]) * p.block;
      } else {
        const int nz = p.row_offsets[u + 1] - first;
        t.wrow0 = n * p.bf;
        t.kofs = cb0 * p.block;
        t.klen = nz * p.block;
        t.ocol0 = n * p.bf;
      }
    } else {
      const int rows = p.offsets[u + 1] - p.offsets[u];
      const int mt = (rows + p.bt - 1) / p.bt;
      const int nfe = p.gemm == 1 ? ((p.foff[u + 1] - p.foff[u]) * pf + (p.ragged ? p.bf - 1 : 0)) / p.bf
                                  : p.d / p.bf;
      const int sp = n / (mt * nfe);           // K split (second linear only)
      const int nn = n - sp * mt * nfe;
      int m, nf;
      tile_coords(nn, mt, nfe, &m, &nf);
      t.expert = u;
      t.spare = sp;
      // the group's rows split evenly over its mt row tiles, in multiples of
      // 32 (the MFMA row block): tiles of one group then cost the same (the
      // kernels skip whole row blocks past a tile's end), so the row tiles
      // that share a weight tile stay in step and share it through L2
      // instead of one short tile running ahead; rt <= bt keeps every tile
      // non-empty
      const int rt = min(p.bt, ((rows + mt - 1) / max(mt, 1) + 31) / 32 * 32);
      t.row0 = p.offsets[u] + m * rt;
      t.row_end = min(p.offsets[u + 1], t.row0 + rt);
      if (p.gemm == 1) {
        t.wrow0 = p.foff[u] * pf + nf * p.bf;
        t.kofs = 0;
        t.klen = p.d;
        t.ocol0 = nf * p.bf / p.fold;
        if (p.ragged) t.spare = min(p.bf, (p.foff[u + 1] - p.foff[u]) * pf - nf * p.bf);
      } else {
        const int kl = km * (p.foff[u + 1] - p.foff[u]) / p.ksplit;
        t.wrow0 = nf * p.bf;
        t.kofs = km * p.foff[u] + sp * kl;
        t.klen = kl;
        t.ocol0 = nf * p.bf;
      }
    }
    t.part = part;
    t.nparts = nparts;
    t.pslot0 = pslot0;
    if (nparts > 1 && part == 0) p.counters[group] = o;
    if (nparts > 1) {
      // whole K stages: part j takes stages [j nk / P, (j + 1) nk / P)
      const int ks = p.kstage > 0 ? p.kstage : 64;
      const int nk = t.klen / ks;
      const int k0 = part * nk / nparts, k1 = (part + 1) * nk / nparts;
      t.kofs += k0 * ks;
      t.xk = k0 * ks;
      t.klen = (k1 - k0) * ks;
    }
    p.tiles[o] = t;
  }
}

// ---------------------------------------------------------------- packing

// dst[n, k] = src[k, n], 32 x 32 tiles through LDS.

constexpr int kPlanSlices = 8;   // workgroups writing one list

__global__ void __launch_bounds__(1024) k_plan(PlanArgs p) {
  plan_tiles(p, blockIdx.x, kPlanSlices);
}

// Both expert GEMMs' lists in one launch, kPlanSlices workgroups each.
__global__ void __launch_bounds__(1024) k_plan_pair(PlanArgs p0, PlanArgs p1) {
  if (int(blockIdx.x) < kPlanSlices) plan_tiles(p0, blockIdx.x, kPlanSlices);
  else plan_tiles(p1, blockIdx.x - kPlanSlices, kPlanSlices);
}

template <typename T>
__global__ void __launch_bounds__(256) k_transpose(const T* __restrict__ src, int64_t K, int64_t N,
                                                   T* __restrict__ dst) {
  __shared__ T tile[32][33];
  const int64_t n0 = int64_t(blockIdx.x) * 32, k0 = int64_t(blockIdx.y) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  for (int i = ty; i < 32; i += 8) {
    const int64_t kk = k0 + i, nn = n0 + tx;
    if (kk < K && nn < N) tile[i][tx] = src[kk * N + nn];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int64_t nn = n0 + i, kk = k0 + tx;
    if (kk < K && nn < N) dst[nn * K + kk] = tile[tx][i];
  }
}

// SwiGLU interleave: packed row p <- column 32 (p / 64) + p % 32 of w1 (p % 64 < 32)
// or of w3 (p % 64 >= 32); every expert width is a multiple of 32, so the
// mapping is the same for every expert.
template <typename T>
__global__ void __launch_bounds__(256) k_pack_swiglu(const T* __restrict__ w1,
                                                     const T* __restrict__ w3, int64_t d,
                                                     int64_t F, T* __restrict__ dst) {
  __shared__ T tile[32][33];
  const int64_t p0 = int64_t(blockIdx.x) * 32;   // 32 packed rows, one source matrix
  const int64_t k0 = int64_t(blockIdx.y) * 32;
  const T* src = ((p0 / 32) & 1) ? w3 : w1;
  const int64_t c0 = (p0 / 64) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int64_t kk = k0 + i;
    if (kk < d) tile[i][tx] = src[kk * F + c0 + tx];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int64_t kk = k0 + tx;
    if (kk < d) dst[(p0 + i) * d + kk] = tile[tx][i];
  }
}

}  // namespace


hipError_t launch_plan(const PlanArgs& p, hipStream_t s) {
  hipLaunchKernelGGL(k_plan, dim3(kPlanSlices), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_plan_pair(const PlanArgs& p0, const PlanArgs& p1, hipStream_t s) {
  hipLaunchKernelGGL(k_plan_pair, dim3(2 * kPlanSlices), dim3(1024), 0, s, p0, p1);
  return hipGetLastError();
}

// A persistent launch of the bf16 GEMM: one workgroup per compute unit (its
// LDS ring fills a CU), in a multiple of 8 so that each keeps to one XCD's
// tiles.  (With a grid of one workgroup per tile the kernel's tile loop runs
// once.)
int gemm_persistent_grid(int grid) {
  static thread_local int dev_cached = -1, cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev != dev_cached) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n >= 8)
      cus = n / 8 * 8;
    dev_cached = dev;
  }
  return std::min(grid, cus);
}

hipError_t launch_gemm(int dtype, const GemmArgs& a, int bf, int bt, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  // Persistent only for the forward epilogues: the next tile's first wait
  // also covers this tile's stores (vmcnt counts both), which costs more than
  // it saves when a tile stores 256 KB of fp32 (the backward's EPI_SCALE_F32
  // ran 4% slower persistent) or bf16 rows of the backward's EPI_STORE_T.
  if (dtype != 0 && a.epi != EPI_SCALE_F32 && a.epi != EPI_STORE_T) grid = gemm_persistent_grid(grid);
  const dim3 g(grid), b(256);
  if (dtype == 0) {
    switch (a.epi) {
      case EPI_ACT: hipLaunchKernelGGL(k_gemm_f32<EPI_ACT>, g, b, 0, s, a); break;
      case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_f32<EPI_SWIGLU>, g, b, 0, s, a); break;
      case EPI_GATE: hipLaunchKernelGGL(k_gemm_f32<EPI_GATE>, g, b, 0, s, a); break;
      case EPI_SCALE_F32: hipLaunchKernelGGL(k_gemm_f32<EPI_SCALE_F32>, g, b, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (bf != 256 || (bt != 256 && bt != 128)) return hipErrorInvalidValue;
  // (an extent of 0 is an empty operand: a launch over no rows reads nothing)
  if (a.x_bytes < 0 || a.w_bytes < 0 || a.x_bytes >= (int64_t(1) << 32) ||
      a.w_bytes >= (int64_t(1) << 32))
    return hipErrorInvalidValue;
  if (bt == 256) {
    const dim3 b8(512);
    switch (a.epi) {
      case EPI_ACT: hipLaunchKernelGGL((k_gemm_bf16_dma<256, 256, 4, 2, EPI_ACT>), g, b8, 0, s, a); break;
      case EPI_SWIGLU: hipLaunchKernelGGL((k_gemm_bf16_dma<256, 256, 4, 2, EPI_SWIGLU>), g, b8, 0, s, a); break;
      case EPI_GATE: hipLaunchKernelGGL((k_gemm_bf16_dma<256, 256, 4, 2, EPI_GATE>), g, b8, 0, s, a); break;
      case EPI_SCALE_F32: hipLaunchKernelGGL((k_gemm_bf16_dma<256, 256, 4, 2, EPI_SCALE_F32>), g, b8, 0, s, a); break;
      case EPI_STORE_T: hipLaunchKernelGGL((k_gemm_bf16_dma<256, 256, 4, 2, EPI_STORE_T>), g, b8, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.epi) {
      case EPI_ACT: hipLaunchKernelGGL((k_gemm_bf16_dma<256, 128, 2, 2, EPI_ACT>), g, b, 0, s, a); break;
      case EPI_SWIGLU: hipLaunchKernelGGL((k_gemm_bf16_dma<256, 128, 2, 2, EPI_SWIGLU>), g, b, 0, s, a); break;
      case EPI_GATE: hipLaunchKernelGGL((k_gemm_bf16_dma<256, 128, 2, 2, EPI_GATE>), g, b, 0, s, a); break;
      case EPI_SCALE_F32: hipLaunchKernelGGL((k_gemm_bf16_dma<256, 128, 2, 2, EPI_SCALE_F32>), g, b, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_piece_fixup(const GemmArgs& a, int bf, int bt, int grid, int max_parts,
                              hipStream_t s) {
  // grid = the GEMM's persistent grid; a split tile holds at least two of its
  // workgroups' pieces, so there are at most grid / 2 split tiles
  if (grid <= 0) return hipSuccess;
  if (bf != 256 || bt != 256 || a.epi != EPI_GATE || max_parts > kFixupMaxParts)
    return hipErrorInvalidValue;
  constexpr int NI = 8 * 2 * 4;                 // items per 256 x 256 tile, 4 per workgroup
  const dim3 g(unsigned((grid + 1) / 2 * NI / 4));
  hipLaunchKernelGGL((k_piece_fixup<256, 256, 4, 2>), g, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack_transpose(const void* src, int dtype, int64_t K, int64_t N, void* dst,
                                 hipStream_t s) {
  if (K == 0 || N == 0) return hipSuccess;
  const dim3 g(unsigned((N + 31) / 32), unsigned((K + 31) / 32));
  if (dtype == 0)
    hipLaunchKernelGGL(k_transpose<float>, g, dim3(256), 0, s, static_cast<const float*>(src), K,
                       N, static_cast<float*>(dst));
  else
    hipLaunchKernelGGL(k_transpose<uint16_t>, g, dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), K, N, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_pack_swiglu(const void* w1, const void* w3, int dtype, int64_t d, int64_t F,
                              const int32_t*, const int64_t*, int64_t, void* dst, hipStream_t s) {
  if (d == 0 || F == 0) return hipSuccess;
  const dim3 g(unsigned(2 * F / 32), unsigned((d + 31) / 32));
  if (dtype == 0)
    hipLaunchKernelGGL(k_pack_swiglu<float>, g, dim3(256), 0, s, static_cast<const float*>(w1),
                       static_cast<const float*>(w3), d, F, static_cast<float*>(dst));
  else
    hipLaunchKernelGGL(k_pack_swiglu<uint16_t>, g, dim3(256), 0, s,
                       static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3), d, F,
                       static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

}  // namespace moe
