// Device helpers shared by the expert GEMM kernels (bf16 and MXFP8): the
// XCD-aware tile order, the LDS chunk swizzle, the DMA wait, the MFMA /
// fragment-read scheduling pattern and the K pieces' partial stores.
#pragma once
#include <hip/hip_runtime.h>

#include "common.h"
#include "gemm_args.h"

namespace moe {

// Tiles are remapped so that each XCD (workgroup id mod 8) runs a contiguous
// run of the tile list: the row tiles that share a weight tile run together
// in one L2.
__device__ __forceinline__ int remap_xcd(int b, int nt) {
  const int xcd = b & 7, slot = b >> 3;
  const int q = nt >> 3, rem = nt & 7;
  return xcd * q + min(xcd, rem) + slot;
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) const void* global_void_ptr;

// s_waitcnt vmcnt(n) with the other counters left free (gfx9 encoding).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// Swizzle of 16-byte chunk q in row r for C chunks per row: any 16 consecutive
// rows read at one logical chunk land in 16 distinct 16-byte bank groups.  It
// depends on r & 15 only, so a fragment read (rows base + lane & 31, base a
// multiple of 32) can compute it from the lane index.
template <int C>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (C == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return (r >> 2) & 3;
}

// Scheduling pattern for one K sub-step: NR fragment reads of the next
// sub-step spread over the first MFMAs of this one (one MFMA, two reads, ...),
// then the remaining MFMAs, so that the reads are in flight under MFMAs and
// have had most of the sub-step to land before they are waited for.
template <int NR, int NM>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (NR > 0 && NM > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NR >= 2 ? 2 : 1, 0);
    sched_interleave<NR - (NR >= 2 ? 2 : 1), NM - 1>();
  } else if constexpr (NR > 0) {
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
  } else if constexpr (NM > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  }
}

// K pieces of a split tile.  Each piece stores its fp32 partial sums at its
// slot of the partial buffer in fragment order (block (i, j) of wave w at
// ((w MF + i) MT + j) 1024 + 16 lane floats), so that the lane of the fixup
// kernel that reads them back holds exactly the values the same lane of a
// whole tile would.  No workgroup waits for another: the fixup kernel runs
// after the GEMM on the same stream.
template <int BF, int BT, int MF, int MT>
__device__ __forceinline__ int64_t piece_frag_offset(int wid, int lane, int i, int j) {
  return int64_t(wid) * (MF * MT * 1024) + (i * MT + j) * 1024 + lane * 16;
}

template <int BF, int BT, int MF, int MT>
__device__ __forceinline__ void store_piece(const GemmArgs& a, const Tile& tile,
                                            const f32x16 (&acc)[MF][MT], int wid, int lane) {
  float* const dst0 = a.part + (int64_t(tile.pslot0) + tile.part) * (int64_t(BF) * BT);
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      f32x4* dst = reinterpret_cast<f32x4*>(dst0 + piece_frag_offset<BF, BT, MF, MT>(wid, lane, i, j));
#pragma unroll
      for (int v = 0; v < 4; ++v)
        dst[v] = f32x4{acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2],
                       acc[i][j][4 * v + 3]};
    }
}

}  // namespace moe
