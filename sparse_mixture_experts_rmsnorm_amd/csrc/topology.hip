// BCSR topology of the expert FFN ("Variable-size experts" nanoMOE notes,
// section 3 on the indices kernel, the output-array-indexing bug fix, and
// section 4 on topology construction).
//
// Rows of the permuted activation form token blocks of `block` rows; expert
// e owns tb_e = (offsets[e+1] - offsets[e]) / block of them (dispatch pads
// each expert to the block).  Every token block of e connects to e's
// size_blocks[e] column blocks, starting at block_offsets[e].  Each expert's
// column indices start at the exclusive prefix sum over experts of
// tb_e * size_blocks[e] -- computed here on the device, so no host loop or
// read-back is needed -- never at a uniform per-expert stride.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kTopoMaxE = 2048;

__device__ __forceinline__ int upper_bound_rows(const int32_t* a, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(1024) k_topology(const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ size_blocks,
                                                   const int32_t* __restrict__ block_offsets,
                                                   int E, int block, int nrb_max,
                                                   int32_t* __restrict__ row_offsets,
                                                   int32_t* __restrict__ column_indices,
                                                   int32_t* __restrict__ nnz) {
  __shared__ int outoff[kTopoMaxE + 1];
  __shared__ long long sh[33];
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int lo = min(E, int(threadIdx.x) * per), hi = min(E, lo + per);
  long long local = 0;
  for (int e = lo; e < hi; ++e) {
    const int tb = (offsets[e + 1] - offsets[e]) / block;
    outoff[e] = tb * size_blocks[e];
    local += outoff[e];
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  long long incl = local;
  for (int o = 1; o < 64; o <<= 1) {
    const long long u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) sh[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long run = 0;
    for (int w = 0; w < nw; ++w) {
      const long long t = sh[w];
      sh[w] = run;
      run += t;
    }
    sh[32] = run;
  }
  __syncthreads();
  long long b = sh[wid] + incl - local;
  const int total = int(sh[32]);
  for (int e = lo; e < hi; ++e) {
    const int c = outoff[e];
    outoff[e] = int(b);
    b += c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    *nnz = total;
    row_offsets[0] = 0;
  }
  const int used = offsets[E] / block;
  for (int rb = threadIdx.x; rb < nrb_max; rb += blockDim.x) {
    if (rb < used) {
      const int e = upper_bound_rows(offsets, E + 1, rb * block) - 1;
      const int y = rb - offsets[e] / block;
      const int sb = size_blocks[e];
      const int start = outoff[e] + y * sb;
      row_offsets[rb + 1] = start + sb;
      for (int c = 0; c < sb; ++c) column_indices[start + c] = block_offsets[e] + c;
    } else {
      row_offsets[rb + 1] = total;
    }
  }
}

}  // namespace

hipError_t launch_topology(const int32_t* offsets, const int32_t* size_blocks,
                           const int32_t* block_offsets, int64_t E, int block, int64_t rows_max,
                           int32_t* row_offsets, int32_t* column_indices, int32_t* nnz,
                           hipStream_t s) {
  hipLaunchKernelGGL(k_topology, dim3(1), dim3(1024), 0, s, offsets, size_blocks, block_offsets,
                     int(E), block, int(rows_max / block), row_offsets, column_indices, nnz);
  return hipGetLastError();
}

}  // namespace moe
