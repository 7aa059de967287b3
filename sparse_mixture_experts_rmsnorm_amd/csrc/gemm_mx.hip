// MXFP8 expert GEMMs on the gfx950 scaled MFMA, and the MXFP8 quantiser.
//
// CODA sparse-MoE thread: low-precision conversions belong in epilogues.
// Format: OCP Microscaling MXFP8 -- blocks of 32 elements along K share an
// E8M0 power-of-two scale, elements are FP8 E4M3 (nearest-even, saturating
// at 448).  The activation rows are quantised once per token (k_quant_mx),
// the weights once at pack time, and the hidden activation h in the first
// GEMM's epilogue (one block = the 32 features a wave holds for a token),
// so the second GEMM reads MXFP8 h directly.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands; layout measured on the
// GPU): lane l covers row (A) / column (B) l % 32; register bytes 0-15 hold
// K = 16 (l / 32) + b and bytes 16-31 hold K = 32 + 16 (l / 32) + (b - 16),
// i.e. 16-byte chunks h and 2 + h of the 64-byte K sub-step, and byte 0 of
// the lane's scale operand is the E8M0 scale of its row's 32-element block
// l / 32.  The accumulator layout is that of the other 32 x 32 MFMAs.
//
// The tiling, LDS ring, swizzle, barrier placement and tile lists are those
// of the bf16 kernel: a stage is 128 bytes of K per row (128 FP8 elements,
// two MFMA sub-steps), so the LDS bytes per stage are the same and the
// MFMA work per stage doubles.
#include <algorithm>

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle;
// reads past num_records return zero).
constexpr int kRsrcWord3 = 0x00020000;

// E4M3 codes of four finite values, the first in the low byte: nearest-even
// on 3 mantissa bits, magnitudes of 448 and above saturated to 448,
// subnormals on the 2^-9 grid.  gfx950's v_cvt_pk_fp8_f32 converts a pair
// to OCP E4M3 with round-to-nearest-even; clamped to +-448 first (past the
// largest normal the instruction itself would give NaN), its codes equal this
// rounding exactly: the quantiser's parity test compares them with the
// oracle's encoder at every midpoint between neighbouring codes and the bf16
// values either side of it, both signs, at three block scales.
__device__ __forceinline__ uint32_t e4m3_pk_pair(float a, float b) {
  const float ca = __builtin_fminf(__builtin_fmaxf(a, -448.f), 448.f);
  const float cb = __builtin_fminf(__builtin_fmaxf(b, -448.f), 448.f);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false)) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t e4m3_x4(float a, float b, float c, float d) {
  return e4m3_pk_pair(a, b) | (e4m3_pk_pair(c, d) << 16);
}

// Shared exponent of a block whose largest magnitude is amax:
// floor(log2 amax) - 8 (the exponent of E4M3's largest normal), within the
// E8M0 range; -127 for an all-zero block.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  int e;
  (void)frexpf(amax, &e);                       // amax = m 2^e, m in [0.5, 1)
  return min(127, max(-127, e - 1 - 8));
}

// Rows of bf16 [R, K] -> E4M3 codes [R, K] and E8M0 scales, either row-major
// [R, K / 32] (sstage 0: row r's byte j at r ldsc + j) or stage-major for the
// GEMM's activation operand (sstage > 0: the four scale bytes of row r in the
// 128-element K stage s at s sstage + 4 r, so that one stage's scales of
// consecutive rows are contiguous and the GEMM's scale DMA is coalesced).
// Output row r reads source row map[r] (map NULL: r; -1: a zero row), so the
// quantiser is also the dispatch gather of the MXFP8 path.  One wave per
// row; a lane converts 8 consecutive elements, four lanes make a block.
__global__ void __launch_bounds__(256) k_quant_mx(const uint16_t* __restrict__ src, int64_t R,
                                                  int64_t K, int64_t lds,
                                                  const int32_t* __restrict__ map,
                                                  const int32_t* __restrict__ rows_used,
                                                  uint8_t* __restrict__ codes, int64_t ldc,
                                                  uint8_t* __restrict__ scales, int64_t ldsc,
                                                  int64_t sstage) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= R || (rows_used && row >= *rows_used)) return;
  const int64_t sr = map ? map[row] : row;
  for (int64_t k0 = lane * 8; k0 < K; k0 += 512) {
    float f[8];
    const uint4 v = sr >= 0 ? *reinterpret_cast<const uint4*>(src + sr * lds + k0)
                            : make_uint4(0, 0, 0, 0);
    unpack16(v, f, (const uint16_t*)nullptr);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    const int s = mx_shared_exp(m);
    const float inv = ldexpf(1.f, -s);
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[h] = e4m3_x4(f[4 * h] * inv, f[4 * h + 1] * inv, f[4 * h + 2] * inv, f[4 * h + 3] * inv);
    *reinterpret_cast<uint2*>(codes + row * ldc + k0) = make_uint2(w[0], w[1]);
    if ((lane & 3) == 0) {
      const int64_t at = sstage > 0 ? (k0 / 128) * sstage + row * 4 + (k0 / 32) % 4 : row * ldsc + k0 / 32;
      scales[at] = uint8_t(s + 127);
    }
  }
}

// 16 values a lane holds of one 32-element block (its partner lane, lane ^ 32,
// holds the other 16): the block's shared exponent and the values' codes,
// four bytes per group g (features 8 g + 4 (lane >> 5) + {0..3}).
__device__ __forceinline__ int mx_block_codes(const float (&o)[16], uint32_t (&w)[4]) {
  float m = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) m = fmaxf(m, fabsf(o[v]));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  const int s = mx_shared_exp(m);
  const float inv = ldexpf(1.f, -s);
#pragma unroll
  for (int g = 0; g < 4; ++g)
    w[g] = e4m3_x4(o[4 * g] * inv, o[4 * g + 1] * inv, o[4 * g + 2] * inv, o[4 * g + 3] * inv);
  return s;
}

// Scheduling of one MXFP8 sub-step: the NA reads of the next A fragments
// (and scale words) first, then per B block its MFN MFMAs followed by the two
// reads that refill that block for the next sub-step.
template <int NJ, int MFN>
__device__ __forceinline__ void sched_mx_blocks() {
  if constexpr (NJ > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, MFN, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    sched_mx_blocks<NJ - 1, MFN>();
  }
}
template <int NA, int NJ, int MFN>
__device__ __forceinline__ void sched_mx_step() {
  __builtin_amdgcn_sched_group_barrier(0x100, NA, 0);
  sched_mx_blocks<NJ, MFN>();
}

// 256 features x 256 rows per workgroup, 8 waves in a 4 x 2 grid of 64 x 128
// wave tiles (MF = 2, MT = 4 blocks of 32 x 32).  Each sub-step's fragments
// (32 bytes per block) are read under the MFMAs of the sub-step before: two
// sets of A fragments, and one set of B fragments in which a block is
// refilled as soon as its last MFMA has been issued, so the wave stays within
// the 256 registers two waves per SIMD allow (a second full B set would not).
//
// Persistent, as the bf16 kernel: workgroup b takes tiles b, b + G, ... of the
// XCD-remapped list, or of its XCD's run when the list was planned for this
// grid (xcd_runs), and issues the next tile's first two stages before this
// tile's epilogue.  A K piece (tile.nparts > 1) stores its fp32 partial tile
// for the fixup kernel, which applies the epilogue to the sum of the pieces.
template <int EPI>
__global__ void __launch_bounds__(512) k_gemm_mx(MxGemmArgs m) {
  constexpr int BF = 256, BT = 256, WGF = 4, WGT = 2, NW = 8;
  constexpr int WTF = BF / WGF, WTT = BT / WGT, MF = WTF / 32, MT = WTT / 32;
  constexpr int BK = 128;                       // bytes (= elements) of K per stage
  constexpr int C = BK / 16;                    // 16-byte chunks per LDS row
  constexpr int RSEG = 64 / C;                  // rows per 1 KB DMA segment
  constexpr int SEGW = BF / RSEG, SEGX = BT / RSEG;
  constexpr int SPW = (SEGW + SEGX) / NW;       // DMA instructions per wave per stage
  constexpr int LT = (BF + BT) * BK;            // operand bytes per stage
  constexpr int LS = LT + (BF + BT) * 4;        // + one E8M0 scale word per row
  constexpr int KS = BK / 64;                   // MFMA sub-steps per stage
  constexpr int SPI = SPW + 1;                  // DMA instructions per wave per stage
  static_assert(EPI != EPI_SWIGLU || MF % 2 == 0, "SwiGLU pairs gate and up blocks per wave");
  static_assert(KS == 2, "two sub-steps per stage");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * LS];
  const GemmArgs& a = m.g;

  const int nt = a.ntiles[0];
  const int G = gridDim.x;
  const int NX = a.xcd_runs && G % 8 == 0 ? 8 : 1;
  const int run_end = a.xcd_runs ? a.ntiles[2 + int(blockIdx.x) % NX] : nt;
  int tb = a.xcd_runs ? a.ntiles[1 + int(blockIdx.x) % NX] + int(blockIdx.x) / NX : int(blockIdx.x);
  const int step = a.xcd_runs ? G / NX : G;
  auto list_index = [&](int i) { return a.xcd_runs ? i : remap_xcd(i, nt); };
  if (tb >= run_end) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  // waves wid and wid + 4 share a SIMD: the same feature rows, the two row
  // halves (a tile with few rows keeps every SIMD equally busy)
  const int wt = wid / WGF, wf = wid % WGF;

  // Operands are read through buffer resources: uniform base and size in
  // scalar registers, a 32-bit per-lane offset, and every uniform part of the
  // address (stage, segment, block) in the scalar offset.  X rows are
  // contiguous (the quantiser gathered them); a tile reads all 256 of its
  // rows, and the rows past the group's end are never stored (the caller's
  // row buffers extend one tile past their last row, so those reads stay in
  // the allocation whether or not the scalar offset is range-checked).
  // Segment sg covers rows 8 sg .. 8 sg + 7: lane row srow = lane / 8, and the
  // chunk swizzle of that row is srow ^ (sg & 1).
  const int srow = lane / C;
  const bool wseg = wid * SPW < SEGW;
  const __amdgpu_buffer_rsrc_t rsrc =
      wseg ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(static_cast<const uint8_t*>(a.W)),
                                               0, int(m.w_bytes), kRsrcWord3)
           : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(static_cast<const uint8_t*>(a.X)),
                                               0, int(m.x_bytes), kRsrcWord3);
  const int64_t ld = wseg ? a.ldw : a.ldx;
  const int sg0 = wseg ? wid * SPW : wid * SPW - SEGW;      // first segment of this wave
  // Scale words ride with the operands: the 4 E8M0 bytes of a row's stage
  // (K offsets are multiples of 128, so they are one aligned 32-bit word)
  // land after the operand tiles, W rows then X rows, one 4-byte DMA per
  // wave (waves 0-3: W rows 64 w .. 64 w + 63, waves 4-7: X rows).  Both
  // operands' scales are stage-major (the words of consecutive rows for one
  // stage are adjacent), so each of these DMAs reads 256 contiguous bytes.
  // The weights have ldws / 4 rows; a tile whose features run past the last
  // row (a ragged last tile) reads the last row's word for them instead,
  // which stays inside the array at every stage (those features are never
  // stored).
  const bool wsc = wid < NW / 2;
  const __amdgpu_buffer_rsrc_t s_rsrc =
      wsc ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(m.ws), 0, int(m.ws_bytes), kRsrcWord3)
          : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(m.xs), 0, int(m.xs_bytes), kRsrcWord3);
  const int64_t srow_s = (wsc ? wid : wid - NW / 2) * 64 + lane;
  const int s_step = int(wsc ? m.ldws : m.ldxs);  // bytes between a row's consecutive stages
  // this lane's offsets into its operand and scale rows for a tile (a K
  // piece starts at tile.kofs in the weights and tile.xk in the rows)
  uint32_t voff[2];                              // even / odd segments (swizzle parity)
  uint32_t s_voff;
  auto set_sources = [&](const Tile& t) {
    const int xk0 = t.xk;
    const int64_t rbase = (wseg ? int64_t(t.wrow0) : int64_t(t.row0)) + srow;
    const int64_t kbase = wseg ? t.kofs : xk0;
#pragma unroll
    for (int p = 0; p < 2; ++p)
      voff[p] = uint32_t(rbase * ld + kbase + ((lane % C) ^ srow ^ p) * 16);
    s_voff = wsc ? uint32_t(min(int64_t(t.wrow0) + srow_s, m.ldws / 4 - 1) * 4 +
                            int64_t(t.kofs / 128) * m.ldws)
                 : uint32_t((int64_t(t.row0) + srow_s) * 4 + int64_t(xk0 / 128) * m.ldxs);
  };
  auto issue = [&](int kt, int stage) {
    uint8_t* base = lds + stage * LS;
#pragma unroll
    for (int u = 0; u < SPW; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_void_ptr)(base + (wid * SPW + u) * 1024), 16, voff[(sg0 + u) & 1],
          int(kt * BK + int64_t(sg0 + u) * RSEG * ld), 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_void_ptr)(base + LT + wid * 256), 4,
                                             s_voff, kt * s_step, 0, 0);
  };
  // stages 0 and 1 (a one-stage tile loads stage 0 twice, the second copy
  // into a buffer that is not read)
  auto prologue = [&](int nk) {
    issue(0, 0);
    issue(min(1, nk - 1), 1);
  };

  const int fr = lane & 31, fh = lane >> 5, fswz = chunk_swz<C>(lane & 15);
  // Fragment addresses: the 16-byte chunk c of a row sits at slot c ^ swz(row)
  // (the DMA wrote it there), and a lane's chunks in sub-step ksv are
  // 4 ksv + 2 h + fh, h = 0, 1.  Row offsets are multiples of the 128-byte row,
  // so the slot offset is one per-lane base XORed with 64 ksv + 32 h.
  const uint32_t a_off = uint32_t((wf * WTF + fr) * BK + ((fh ^ fswz) << 4));
  const uint32_t b_off = uint32_t(BF * BK + (wt * WTT + fr) * BK + ((fh ^ fswz) << 4));

  Tile tile = a.tiles[list_index(tb)];
  int nk = tile.klen / BK;
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

#define MOE_MX_LOAD(DST, SW, OFF, KSV)                                                         \
  {                                                                                            \
    const u32x4 lo_ = *reinterpret_cast<const u32x4*>((SW) + ((OFF) ^ (64u * (KSV))));         \
    const u32x4 hi_ = *reinterpret_cast<const u32x4*>((SW) + ((OFF) ^ (64u * (KSV) + 32u)));   \
    DST = i32x8{int(lo_.x), int(lo_.y), int(lo_.z), int(lo_.w),                               \
                int(hi_.x), int(hi_.y), int(hi_.z), int(hi_.w)};                              \
  }
#define MOE_MX_LOADA(AF, SW, KSV)                                                              \
  _Pragma("unroll") for (int i = 0; i < MF; ++i) MOE_MX_LOAD(AF[i], (SW) + i * 32 * BK, a_off, KSV)
#define MOE_MX_LOADB(J, SW, KSV) MOE_MX_LOAD(bfr[J], (SW) + (J) * 32 * BK, b_off, KSV)
// one sub-step's MFMAs, B block by B block; behind the last use of each B
// block its registers are refilled with the same block of the next sub-step
// (buffer SWN, sub-step KSVN), and the next sub-step's A fragments go to the
// other A set first
#define MOE_MX_STEP(AF, SA, SB, SWN, KSVN, AFN)                                                \
  {                                                                                            \
    MOE_MX_LOADA(AFN, SWN, KSVN)                                                               \
    _Pragma("unroll") for (int j = 0; j < MTA; ++j) {                                         \
      _Pragma("unroll") for (int i = 0; i < MF; ++i)                                          \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                           \
            AF[i], bfr[j], acc[i][j], 0, 0, 0, int(SA[i]), 0, int(SB[j]));                     \
      MOE_MX_LOADB(j, SWN, KSVN)                                                               \
    }                                                                                          \
  }
#define MOE_MX_MFMAS(AF, SA, SB)                                                               \
  {                                                                                            \
    _Pragma("unroll") for (int j = 0; j < MTA; ++j)                                           \
      _Pragma("unroll") for (int i = 0; i < MF; ++i)                                          \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                           \
            AF[i], bfr[j], acc[i][j], 0, 0, 0, int(SA[i]), 0, int(SB[j]));                     \
  }
// E8M0 bytes of this lane's 32-block (2 ksv + fh of the stage) in sub-step ksv
#define MOE_MX_BYTES(KSV, SA, SB)                                                              \
  {                                                                                            \
    const int sh_ = 8 * (2 * (KSV) + fh);                                                      \
    _Pragma("unroll") for (int i = 0; i < MF; ++i) SA[i] = (sa[i] >> sh_) & 0xFFu;            \
    _Pragma("unroll") for (int j = 0; j < MTA; ++j) SB[j] = (sb[j] >> sh_) & 0xFFu;            \
  }
#define MOE_MX_SCALES(SW)                                                                      \
  {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < MF; ++i)                                            \
      sa[i] = *reinterpret_cast<const uint32_t*>((SW) + LT + (wf * WTF + i * 32 + fr) * 4);    \
    _Pragma("unroll") for (int j = 0; j < MTA; ++j)                                           \
      sb[j] = *reinterpret_cast<const uint32_t*>((SW) + LT + BF * 4 + (wt * WTT + j * 32 + fr) * 4); \
  }

    // Two LDS stages and one barrier per stage, placed after the stage's last
    // fragments are in registers: behind it the drained buffer is refilled
    // (stage kt + 2) while the second sub-step's MFMAs run.  The fragments of
    // each sub-step are read under the MFMAs of the one before (two A sets,
    // one B set refilled block by block), so a wave's MFMAs never wait for
    // its own LDS reads except at the barrier.  The loop body has no branch:
    // past the last stage the refill repeats stage nk - 1, in bounds, into a
    // buffer that is not read again.
    // Row blocks of this wave that hold rows of the tile: the MFMAs, fragment
    // and scale reads of the rest (never stored) are skipped, one loop copy
    // per count.
    const int mta = __builtin_amdgcn_readfirstlane(
        max(0, min(MT, (tile.row_end - tile.row0 - wt * WTT + 31) / 32)));
    auto main_loop = [&](auto mta_c) {
      constexpr int MTA = decltype(mta_c)::value;
      uint32_t sa[MF], sb[MT];
      uint32_t s0a[MF], s0b[MT], s1a[MF], s1b[MT];
      i32x8 af0[MF], af1[MF], bfr[MT];
      if (nk > 0) {
        // stage 0 has landed (after a previous tile's epilogue its stores
        // are counted too, so everything is waited for)
        if (first) MOE_WAIT_VMCNT(SPI);
        else MOE_WAIT_VMCNT(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        MOE_MX_SCALES(lds)
        MOE_MX_LOADA(af0, lds, 0)
        _Pragma("unroll") for (int j = 0; j < MTA; ++j) MOE_MX_LOADB(j, lds, 0)
        MOE_MX_BYTES(0, s0a, s0b)
        __builtin_amdgcn_sched_barrier(0);
        for (int kt = 0; kt + 1 < nk; ++kt) {
          const uint8_t* sw = lds + (kt & 1) * LS;
          const uint8_t* swn = lds + ((kt + 1) & 1) * LS;
          const int knext = min(kt + 2, nk - 1);
          MOE_MX_STEP(af0, s0a, s0b, sw, 1, af1)
          sched_mx_step<2 * MF, MTA, MF>();
          __builtin_amdgcn_sched_barrier(0);
          MOE_MX_BYTES(1, s1a, s1b)
          // this wave's reads of stage kt are in registers and its share of
          // stage kt + 1 has landed; after the barrier both hold for every
          // wave, so stage kt's buffer may be refilled
          asm volatile("s_waitcnt 0x0070" ::: "memory");   // vmcnt(0) lgkmcnt(0)
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          issue(knext, kt & 1);
          __builtin_amdgcn_sched_barrier(0);
          MOE_MX_SCALES(swn)
          MOE_MX_STEP(af1, s1a, s1b, swn, 0, af0)
          sched_mx_step<2 * MF + MF + MTA, MTA, MF>();
          __builtin_amdgcn_sched_barrier(0);
          MOE_MX_BYTES(0, s0a, s0b)
        }
        const uint8_t* sw = lds + ((nk - 1) & 1) * LS;
        MOE_MX_STEP(af0, s0a, s0b, sw, 1, af1)
        sched_mx_step<2 * MF, MTA, MF>();
        __builtin_amdgcn_sched_barrier(0);
        MOE_MX_BYTES(1, s1a, s1b)
        MOE_MX_MFMAS(af1, s1a, s1b)
      }
    };
    static_assert(MT == 4, "one loop copy per row-block count");
    if (mta >= 4) main_loop(std::integral_constant<int, 4>{});
    else if (mta == 3) main_loop(std::integral_constant<int, 3>{});
    else if (mta == 2) main_loop(std::integral_constant<int, 2>{});
    else if (mta == 1) main_loop(std::integral_constant<int, 1>{});
    else main_loop(std::integral_constant<int, 0>{});

#undef MOE_MX_LOAD
#undef MOE_MX_LOADA
#undef MOE_MX_LOADB
#undef MOE_MX_STEP
#undef MOE_MX_MFMAS
#undef MOE_MX_SCALES
#undef MOE_MX_BYTES

    // the repeated refill may still be in flight, and every wave's LDS reads
    // of this tile must be done before the next tile's loads overwrite the
    // ring: after the barrier the next tile's first two stages are issued,
    // under this tile's epilogue
    MOE_WAIT_VMCNT(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int tn = tb + step;
    const bool more = tn < run_end;
    Tile next = tile;
    int nk2 = 0;
    if (more) {
      next = a.tiles[list_index(tn)];
      nk2 = next.klen / BK;
      set_sources(next);
      if (nk2 > 0) prologue(nk2);
    }

    if (tile.nparts > 1) {
      store_piece<BF, BT, MF, MT>(a, tile, acc, wid, lane);
    } else {
      // epilogues: lane holds token column fr of each block and features
      // 8 g + 4 fh + {0..3}, g = 0..3
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int row = tile.row0 + wt * WTT + j * 32 + fr;
        const bool live = row < tile.row_end;       // (the shuffles below need every lane)
        if (EPI == EPI_SWIGLU || EPI == EPI_ACT) {
          const float rs = live ? a.row_r[row] : 0.f;
          constexpr int NBLK = EPI == EPI_SWIGLU ? MF / 2 : MF;
#pragma unroll
          for (int p = 0; p < NBLK; ++p) {
            float o[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              if (EPI == EPI_SWIGLU) {
                o[v] = silu(rs * acc[2 * p][j][v]) * (rs * acc[2 * p + 1][j][v]);
              } else {
                const float z = rs * acc[p][j][v];
                o[v] = a.act == 1 ? gelu_tanh(z) : gelu_erf(z);
              }
            }
            uint32_t w[4];
            const int s = mx_block_codes(o, w);
            if (live) {
              const int col = tile.ocol0 + wf * (EPI == EPI_SWIGLU ? WTF / 2 : WTF) + p * 32;
              uint8_t* Y = static_cast<uint8_t*>(a.Y) + int64_t(row) * a.ldy + col;
#pragma unroll
              for (int g = 0; g < 4; ++g) *reinterpret_cast<uint32_t*>(Y + g * 8 + fh * 4) = w[g];
              if (fh == 0) m.ys[int64_t(col / 128) * m.ldys + int64_t(row) * 4 + (col / 32) % 4] = uint8_t(s + 127);
            }
          }
        } else if (live) {
          const float rs = a.row_w ? a.row_w[row] : 1.f;
          uint16_t* Y = static_cast<uint16_t*>(a.Y) + int64_t(row) * a.ldy + tile.ocol0 + wf * WTF;
#pragma unroll
          for (int i = 0; i < MF; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              uint32_t pk[2];
#pragma unroll
              for (int h = 0; h < 2; ++h)
                pk[h] = pk_bf16(rs * acc[i][j][g * 4 + h * 2], rs * acc[i][j][g * 4 + h * 2 + 1]);
              *reinterpret_cast<uint2*>(Y + i * 32 + g * 8 + fh * 4) = make_uint2(pk[0], pk[1]);
            }
        }
      }
    }
    if (!more) break;
    tile = next;
    nk = nk2;
    tb = tn;
    first = false;
  }
}

}  // namespace

hipError_t launch_quant_mx(const void* src, int64_t R, int64_t K, int64_t lds, const int32_t* map,
                           const int32_t* rows_used, void* codes, int64_t ldc, void* scales,
                           int64_t ldsc, int64_t sstage, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (K % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quant_mx, dim3(unsigned((R + 3) / 4)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(src), R, K, lds, map, rows_used,
                     static_cast<uint8_t*>(codes), ldc, static_cast<uint8_t*>(scales), ldsc, sstage);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const MxGemmArgs& m, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  // persistent: one workgroup per compute unit, as the bf16 kernel
  const dim3 g(gemm_persistent_grid(grid)), b(512);
  switch (m.g.epi) {
    case EPI_ACT: hipLaunchKernelGGL(k_gemm_mx<EPI_ACT>, g, b, 0, s, m); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_mx<EPI_SWIGLU>, g, b, 0, s, m); break;
    case EPI_GATE: hipLaunchKernelGGL(k_gemm_mx<EPI_GATE>, g, b, 0, s, m); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
