// Atomic experts (OmniMoE summary, 2.1) scheduled expert-centrically (2.2).
//
// An atomic expert n is one hidden unit: E_n(x) = act(x . W[n]) V[n].  With
// the RMSNorm scale in the epilogue (CODA thread) and the gate g of the
// Cartesian router, token t receives
//   routed[t] = sum_j g[t,j] * act(r[t] * xhat[t] . W[n_j]) * V[n_j].
//
// Phase 1 walks the task list sorted by expert id, tokens ascending inside
// each expert (the dispatch's radix sort produced it), so every W row is
// fetched once per run of tasks that share it; a wave keeps the row in
// registers while the run lasts and stores the gated activation a per task.
// Phase 2 gathers, per token and in slot order, a * V[n] -- a fixed summation
// order, so the result is deterministic without atomics.  (A fully
// expert-centric phase 2 would need a scatter-add into routed[t].)
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kTasksPerWave = 16;

// CH = d / 512 16-byte chunks per lane (bf16), d in {512, 1024, 2048, 4096}.
template <int CH>
__global__ void __launch_bounds__(256) k_atomic_phase1(
    const uint16_t* __restrict__ xhat, int d, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ rows_used, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ row_expert, const float* __restrict__ row_r,
    const float* __restrict__ row_w, int act, float* __restrict__ a_rows) {
  const int rows = *rows_used;
  const int lane = threadIdx.x & 63;
  const int64_t first = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kTasksPerWave;
  if (first >= rows) return;
  const int nvec = d / 8;
  int cur = -1;
  u32x4 wv[CH];
  for (int i = 0; i < kTasksPerWave; ++i) {
    const int64_t row = first + i;
    if (row >= rows) break;
    const int n = row_expert[row];
    const int t = row_token[row];
    if (n < 0 || t < 0) {
      if (lane == 0) a_rows[row] = 0.f;
      continue;
    }
    if (n != cur) {
      const u32x4* ws = reinterpret_cast<const u32x4*>(W + int64_t(n) * d);
#pragma unroll
      for (int c = 0; c < CH; ++c) wv[c] = ws[lane + 64 * c];
      cur = n;
    }
    const uint4* xs = reinterpret_cast<const uint4*>(xhat + int64_t(t) * d);
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float xf[8], wf[8];
      unpack16(xs[lane + 64 * c], xf, (const uint16_t*)nullptr);
      unpack16(make_uint4(wv[c].x, wv[c].y, wv[c].z, wv[c].w), wf, (const uint16_t*)nullptr);
#pragma unroll
      for (int q = 0; q < 8; ++q) dot = fmaf(xf[q], wf[q], dot);
    }
    dot = wave_sum(dot);
    if (lane == 0) {
      const float z = row_r[row] * dot;
      a_rows[row] = row_w[row] * (act == 1 ? gelu_tanh(z) : gelu_erf(z));
    }
  }
  (void)nvec;
}

template <int CH>
__global__ void __launch_bounds__(256) k_atomic_phase2(
    const uint16_t* __restrict__ V, int d, int64_t Tn, int k, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ pos, const float* __restrict__ a_rows,
    uint16_t* __restrict__ routed) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  float acc[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[c][q] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int p = pos[t * k + j];
    if (p < 0) continue;
    const float a = a_rows[p];
    const uint4* vs = reinterpret_cast<const uint4*>(V + int64_t(ids[t * k + j]) * d);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float vf[8];
      unpack16(vs[lane + 64 * c], vf, (const uint16_t*)nullptr);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[c][q] = fmaf(a, vf[q], acc[c][q]);
    }
  }
  uint4* out = reinterpret_cast<uint4*>(routed + t * d);
#pragma unroll
  for (int c = 0; c < CH; ++c) out[lane + 64 * c] = pack16(acc[c], (const uint16_t*)nullptr);
}

template <int CH>
hipError_t launch_ch(const AtomicArgs& a, hipStream_t s) {
  const int64_t waves1 = (a.rows + kTasksPerWave - 1) / kTasksPerWave;
  if (waves1 > 0)
    hipLaunchKernelGGL(k_atomic_phase1<CH>, dim3(unsigned((waves1 + 3) / 4)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.xhat), int(a.d),
                       static_cast<const uint16_t*>(a.W), a.rows_used, a.row_token, a.row_expert,
                       a.row_r, a.row_w, a.act, a.a_rows);
  if (a.T > 0)
    hipLaunchKernelGGL(k_atomic_phase2<CH>, dim3(unsigned((a.T + 3) / 4)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.V), int(a.d), a.T, a.k, a.ids, a.pos,
                       a.a_rows, static_cast<uint16_t*>(a.routed));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_atomic(const AtomicArgs& a, hipStream_t s) {
  switch (a.d) {
    case 512: return launch_ch<1>(a, s);
    case 1024: return launch_ch<2>(a, s);
    case 2048: return launch_ch<4>(a, s);
    case 4096: return launch_ch<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
