// Combine: the gated expert outputs summed back into token order.
//
// "Mixture of Experts (MoE)" glossary, top-k gating: a token's output is the
// weighted sum of its selected experts' outputs.  The gate already sits in
// the second expert GEMM's epilogue (CODA thread: epilogues straddling the
// dispatch / combine boundary), so combine is a plain fixed-order sum:
//   out[t] = x[t] + shared[t] + sum_{j = 0..k-1, pos[t,j] >= 0} y[pos[t,j]]
// in fp32, stored once.  Dropped slots contribute nothing; a token whose
// slots were all dropped passes through unchanged (glossary, expert
// capacity), bit-exactly, because x + 0 rounds back to x.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) k_combine(const T* __restrict__ y,
                                                 const int32_t* __restrict__ pos,
                                                 const T* __restrict__ x, const T* __restrict__ sh,
                                                 int64_t Tn, int64_t d, int k, T* __restrict__ out) {
  constexpr int N = Vec16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int64_t nvec = d / N;
  const uint4* ys = reinterpret_cast<const uint4*>(y);
#pragma unroll 2
  for (int64_t v = lane; v < nvec; v += 64) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
    if (x) {
      float f[8];
      unpack16(reinterpret_cast<const uint4*>(x)[t * nvec + v], f, (const T*)nullptr);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += f[i];
    }
    if (sh) {
      float f[8];
      unpack16(reinterpret_cast<const uint4*>(sh)[t * nvec + v], f, (const T*)nullptr);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += f[i];
    }
    if (pos) {
      for (int j = 0; j < k; ++j) {
        const int p = pos[t * k + j];
        if (p < 0) continue;
        float f[8];
        unpack16(ys[int64_t(p) * nvec + v], f, (const T*)nullptr);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] += f[i];
      }
    } else {
      float f[8];
      unpack16(ys[t * nvec + v], f, (const T*)nullptr);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += f[i];
    }
    reinterpret_cast<uint4*>(out)[t * nvec + v] = pack16(acc, (const T*)nullptr);
  }
}

// Same sum with the expert outputs held as two partial planes of a K-split
// second GEMM: slot j adds (p0[pos] + p1[pos]).
template <typename T>
__global__ void __launch_bounds__(256) k_combine_split(const T* __restrict__ y0, int64_t plane,
                                                       const int32_t* __restrict__ pos,
                                                       const T* __restrict__ x,
                                                       const T* __restrict__ sh, int64_t Tn,
                                                       int64_t d, int k, T* __restrict__ out) {
  constexpr int N = Vec16<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int64_t nvec = d / N;
  const uint4* ys = reinterpret_cast<const uint4*>(y0);
  const int64_t pv = plane / N;
#pragma unroll 2
  for (int64_t v = lane; v < nvec; v += 64) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
    if (x) {
      float f[8];
      unpack16(reinterpret_cast<const uint4*>(x)[t * nvec + v], f, (const T*)nullptr);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += f[i];
    }
    if (sh) {
      float f[8];
      unpack16(reinterpret_cast<const uint4*>(sh)[t * nvec + v], f, (const T*)nullptr);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += f[i];
    }
    for (int j = 0; j < k; ++j) {
      const int p = pos[t * k + j];
      if (p < 0) continue;
      float f0[8], f1[8];
      unpack16(ys[int64_t(p) * nvec + v], f0, (const T*)nullptr);
      unpack16(ys[pv + int64_t(p) * nvec + v], f1, (const T*)nullptr);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += f0[i] + f1[i];
    }
    reinterpret_cast<uint4*>(out)[t * nvec + v] = pack16(acc, (const T*)nullptr);
  }
}

}  // namespace

hipError_t launch_combine_split(const void* y0, int64_t rows_max, const int32_t* pos,
                                const void* x, const void* shared, int dtype, int64_t T,
                                int64_t d, int k, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 g(unsigned((T + 3) / 4));
  if (dtype == 0)
    hipLaunchKernelGGL(k_combine_split<float>, g, dim3(256), 0, s, static_cast<const float*>(y0),
                       rows_max * d, pos,
                       static_cast<const float*>(x), static_cast<const float*>(shared), T, d, k,
                       static_cast<float*>(out));
  else
    hipLaunchKernelGGL(k_combine_split<uint16_t>, g, dim3(256), 0, s,
                       static_cast<const uint16_t*>(y0), rows_max * d, pos,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(shared), T,
                       d, k, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, const int32_t* pos, const void* x, const void* shared,
                          int dtype, int64_t T, int64_t d, int k, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 g(unsigned((T + 3) / 4));
  if (dtype == 0)
    hipLaunchKernelGGL(k_combine<float>, g, dim3(256), 0, s, static_cast<const float*>(y), pos,
                       static_cast<const float*>(x), static_cast<const float*>(shared), T, d, k,
                       static_cast<float*>(out));
  else
    hipLaunchKernelGGL(k_combine<uint16_t>, g, dim3(256), 0, s, static_cast<const uint16_t*>(y),
                       pos, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(shared),
                       T, d, k, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace moe
