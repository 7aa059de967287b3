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

// One wave per token and part of the row (P parts of d / P features, so that
// a wave's loads are few rounds deep and the whole grid has many loads in
// flight).  The token's slot positions are read once (lane j holds slot
// j + 64 q) and broadcast slot by slot; the expert rows of four slots are
// loaded together before they are added, so several gathers are in flight.
// The sum starts from x itself, so a token whose slots were all dropped
// stores x bit for bit.
template <typename T>
__global__ void __launch_bounds__(256) k_combine(const T* __restrict__ y,
                                                 const int32_t* __restrict__ pos,
                                                 const T* __restrict__ x, const T* __restrict__ sh,
                                                 int64_t Tn, int64_t d, int k, int parts,
                                                 T* __restrict__ out) {
  constexpr int N = Vec16<T>::N;
  constexpr int SB = 4;                         // slots per batch of loads
  const int lane = threadIdx.x & 63;
  const int64_t g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = g / parts;
  if (t >= Tn) return;
  const int64_t nvec = d / N;
  const int64_t vlen = nvec / parts, v0 = (g - t * parts) * vlen;
  const uint4* ys = reinterpret_cast<const uint4*>(y);
  int pl[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = lane + 64 * q;
    pl[q] = (pos && j < k) ? pos[t * k + j] : -1;
  }
#pragma unroll 2
  for (int64_t v = v0 + lane; v < v0 + vlen; v += 64) {
    float acc[8];
    if (x) {
      unpack16(reinterpret_cast<const uint4*>(x)[t * nvec + v], acc, (const T*)nullptr);
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] = 0.f;
    }
    if (sh) {
      float f[8];
      unpack16(reinterpret_cast<const uint4*>(sh)[t * nvec + v], f, (const T*)nullptr);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += f[i];
    }
    if (pos) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nq = min(64, k - 64 * q);
        for (int j0 = 0; j0 < nq; j0 += SB) {
          uint4 a[SB];
          bool ok[SB];
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            const int p = j0 + u < nq ? __builtin_amdgcn_readlane(pl[q], j0 + u) : -1;
            ok[u] = p >= 0;
            a[u] = ok[u] ? ys[int64_t(p) * nvec + v] : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            if (!ok[u]) continue;
            float f[8];
            unpack16(a[u], f, (const T*)nullptr);
#pragma unroll
            for (int i = 0; i < N; ++i) acc[i] += f[i];
          }
        }
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

}  // namespace

// parts per token row: as many as keep every wave's share a whole number of
// 64-lane rounds of 16-byte vectors, at most 4
static int combine_parts(int64_t d, int dtype) {
  const int64_t nvec = d / (dtype == 0 ? 4 : 8);
  int p = 4;
  while (p > 1 && nvec % (64 * p) != 0) p /= 2;
  return p;
}

hipError_t launch_combine(const void* y, const int32_t* pos, const void* x, const void* shared,
                          int dtype, int64_t T, int64_t d, int k, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int parts = combine_parts(d, dtype);
  const dim3 g(unsigned((T * parts + 3) / 4));
  if (dtype == 0)
    hipLaunchKernelGGL(k_combine<float>, g, dim3(256), 0, s, static_cast<const float*>(y), pos,
                       static_cast<const float*>(x), static_cast<const float*>(shared), T, d, k,
                       parts, static_cast<float*>(out));
  else
    hipLaunchKernelGGL(k_combine<uint16_t>, g, dim3(256), 0, s, static_cast<const uint16_t*>(y),
                       pos, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(shared),
                       T, d, k, parts, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace moe
