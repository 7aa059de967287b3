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

// Tasks (phase 1) or slots (phase 2) whose rows are in flight together: the
// row loads of a batch are all issued before any is used, so a wave keeps
// NB * 2 KB (d = 1024) of gathers outstanding instead of one row.
template <int CH>
constexpr int batch_of() { return CH >= 8 ? 1 : 8 / CH; }

// CH = d / 512 16-byte chunks per lane (bf16), d in {512, 1024, 2048, 4096}.
// Rows whose expert is outside [0, N) or whose token is outside [0, T) are
// dropped (a = 0, nothing loaded); the rows in use are clamped to rows_max.
template <int CH>
__global__ void __launch_bounds__(256) k_atomic_phase1(
    const uint16_t* __restrict__ xhat, int d, const uint16_t* __restrict__ W, int64_t N,
    int64_t Tn, const int32_t* __restrict__ rows_used, int64_t rows_max,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ row_expert,
    const float* __restrict__ row_r, const float* __restrict__ row_w, int act,
    float* __restrict__ a_rows) {
  constexpr int NB = batch_of<CH>();
  const int rows = int(min(int64_t(max(*rows_used, 0)), rows_max));
  const int lane = threadIdx.x & 63;
  const int64_t first = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kTasksPerWave;
  if (first >= rows) return;
  for (int i0 = 0; i0 < kTasksPerWave; i0 += NB) {
    u32x4 wv[NB][CH], xv[NB][CH];
    bool live[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t row = first + i0 + b;
      const int n = row < rows ? row_expert[row] : -1;
      const int t = row < rows ? row_token[row] : -1;
      live[b] = uint64_t(uint32_t(n)) < uint64_t(N) && uint64_t(uint32_t(t)) < uint64_t(Tn);
      const u32x4* ws = reinterpret_cast<const u32x4*>(W + int64_t(live[b] ? n : 0) * d);
      const u32x4* xs = reinterpret_cast<const u32x4*>(xhat + int64_t(live[b] ? t : 0) * d);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        wv[b][c] = live[b] ? ws[lane + 64 * c] : u32x4{0u, 0u, 0u, 0u};
        xv[b][c] = live[b] ? xs[lane + 64 * c] : u32x4{0u, 0u, 0u, 0u};
      }
    }
    float dot[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      dot[b] = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float xf[8], wf[8];
        unpack16(make_uint4(xv[b][c].x, xv[b][c].y, xv[b][c].z, xv[b][c].w), xf,
                 (const uint16_t*)nullptr);
        unpack16(make_uint4(wv[b][c].x, wv[b][c].y, wv[b][c].z, wv[b][c].w), wf,
                 (const uint16_t*)nullptr);
#pragma unroll
        for (int q = 0; q < 8; ++q) dot[b] = fmaf(xf[q], wf[q], dot[b]);
      }
    }
    // NB independent butterfly reductions, interleaved step by step
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
#pragma unroll
      for (int b = 0; b < NB; ++b) dot[b] += __shfl_xor(dot[b], o, 64);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t row = first + i0 + b;
      if (lane == b && row < rows) {
        float av = 0.f;
        if (live[b]) {
          const float z = row_r[row] * dot[b];
          av = row_w[row] * (act == 1 ? gelu_tanh(z) : gelu_erf(z));
        }
        a_rows[row] = av;
      }
    }
  }
}

// A kept slot (pos >= 0) whose expert id is outside [0, N), or whose row is
// past rows_max, is dropped and, for a bad id, counted in *errors.
template <int CH>
__global__ void __launch_bounds__(256) k_atomic_phase2(
    const uint16_t* __restrict__ V, int d, int64_t N, int64_t Tn, int k,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ pos, int64_t rows_max,
    const float* __restrict__ a_rows, uint16_t* __restrict__ routed, int32_t* __restrict__ errors) {
  constexpr int NB = batch_of<CH>();
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  float acc[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[c][q] = 0.f;
  int bad = 0;
  for (int j0 = 0; j0 < k; j0 += NB) {
    u32x4 vv[NB][CH];
    float a[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = j0 + b;
      const int p = j < k ? pos[t * k + j] : -1;
      const int n = p >= 0 ? ids[t * k + j] : 0;
      const bool id_ok = uint64_t(uint32_t(n)) < uint64_t(N);
      bad += (p >= 0 && !id_ok) ? 1 : 0;
      const bool live = p >= 0 && int64_t(p) < rows_max && id_ok;
      a[b] = live ? a_rows[p] : 0.f;
      const u32x4* vs = reinterpret_cast<const u32x4*>(V + int64_t(live ? n : 0) * d);
#pragma unroll
      for (int c = 0; c < CH; ++c) vv[b][c] = live ? vs[lane + 64 * c] : u32x4{0u, 0u, 0u, 0u};
    }
    // slots added in slot order: the sum is the same as one slot at a time
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float vf[8];
        unpack16(make_uint4(vv[b][c].x, vv[b][c].y, vv[b][c].z, vv[b][c].w), vf,
                 (const uint16_t*)nullptr);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[c][q] = fmaf(a[b], vf[q], acc[c][q]);
      }
  }
  if (bad && lane == 0 && errors) atomicAdd(errors, bad);
  uint4* out = reinterpret_cast<uint4*>(routed + t * d);
#pragma unroll
  for (int c = 0; c < CH; ++c) out[lane + 64 * c] = pack16(acc[c], (const uint16_t*)nullptr);
}

// Token-centric single pass: one wave per token keeps x[t] in registers and
// walks its k slots in order, NB at a time with all 2 NB row gathers (W[n]
// and V[n]) issued before any is used: a = g * act(r * x.W[n]), then
// routed[t] += a * V[n] in slot order (the same sum as the two phases).  A
// slot whose expert id is outside [0, N) is dropped (nothing loaded) and
// counted in *errors.
template <int CH>
__global__ void __launch_bounds__(256) k_atomic_token(
    const uint16_t* __restrict__ xhat, int d, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ V, int64_t N, int64_t Tn, int k,
    const int32_t* __restrict__ ids, const float* __restrict__ w_tok,
    const float* __restrict__ r_tok, int act, uint16_t* __restrict__ routed,
    int32_t* __restrict__ errors) {
  constexpr int NB = CH >= 4 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  u32x4 xv[CH];
  {
    const u32x4* xs = reinterpret_cast<const u32x4*>(xhat + t * d);
#pragma unroll
    for (int c = 0; c < CH; ++c) xv[c] = xs[lane + 64 * c];
  }
  const float rt = r_tok[t];
  float acc[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[c][q] = 0.f;
  int bad = 0;
  for (int j0 = 0; j0 < k; j0 += NB) {
    u32x4 wv[NB][CH], vv[NB][CH];
    float g[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = j0 + b;
      const int id = j < k ? ids[t * k + j] : 0;
      const bool id_ok = uint64_t(uint32_t(id)) < uint64_t(N);
      bad += (j < k && !id_ok) ? 1 : 0;
      const bool live = j < k && id_ok;
      const int n = live ? id : 0;
      g[b] = live ? w_tok[t * k + j] : 0.f;
      const u32x4* ws = reinterpret_cast<const u32x4*>(W + int64_t(n) * d);
      const u32x4* vs = reinterpret_cast<const u32x4*>(V + int64_t(n) * d);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        wv[b][c] = live ? ws[lane + 64 * c] : u32x4{0u, 0u, 0u, 0u};
        vv[b][c] = live ? vs[lane + 64 * c] : u32x4{0u, 0u, 0u, 0u};
      }
    }
    float dot[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      dot[b] = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float wf[8], xf[8];
        unpack16(make_uint4(wv[b][c].x, wv[b][c].y, wv[b][c].z, wv[b][c].w), wf,
                 (const uint16_t*)nullptr);
        unpack16(make_uint4(xv[c].x, xv[c].y, xv[c].z, xv[c].w), xf, (const uint16_t*)nullptr);
#pragma unroll
        for (int q = 0; q < 8; ++q) dot[b] = fmaf(xf[q], wf[q], dot[b]);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
#pragma unroll
      for (int b = 0; b < NB; ++b) dot[b] += __shfl_xor(dot[b], o, 64);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float z = rt * dot[b];
      const float a = g[b] * (act == 1 ? gelu_tanh(z) : gelu_erf(z));
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float vf[8];
        unpack16(make_uint4(vv[b][c].x, vv[b][c].y, vv[b][c].z, vv[b][c].w), vf,
                 (const uint16_t*)nullptr);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[c][q] = fmaf(a, vf[q], acc[c][q]);
      }
    }
  }
  if (bad && lane == 0 && errors) atomicAdd(errors, bad);
  uint4* out = reinterpret_cast<uint4*>(routed + t * d);
#pragma unroll
  for (int c = 0; c < CH; ++c) out[lane + 64 * c] = pack16(acc[c], (const uint16_t*)nullptr);
}

template <int CH>
hipError_t launch_ch(const AtomicArgs& a, hipStream_t s) {
  if (a.token_centric) {
    if (a.T > 0)
      hipLaunchKernelGGL(k_atomic_token<CH>, dim3(unsigned((a.T + 3) / 4)), dim3(256), 0, s,
                         static_cast<const uint16_t*>(a.xhat), int(a.d),
                         static_cast<const uint16_t*>(a.W), static_cast<const uint16_t*>(a.V), a.N,
                         a.T, a.k, a.ids, a.w_tok, a.r_tok, a.act,
                         static_cast<uint16_t*>(a.routed), a.errors);
    return hipGetLastError();
  }
  const int64_t waves1 = (a.rows + kTasksPerWave - 1) / kTasksPerWave;
  if (waves1 > 0)
    hipLaunchKernelGGL(k_atomic_phase1<CH>, dim3(unsigned((waves1 + 3) / 4)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.xhat), int(a.d),
                       static_cast<const uint16_t*>(a.W), a.N, a.T, a.rows_used, a.rows,
                       a.row_token, a.row_expert, a.row_r, a.row_w, a.act, a.a_rows);
  if (a.T > 0)
    hipLaunchKernelGGL(k_atomic_phase2<CH>, dim3(unsigned((a.T + 3) / 4)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.V), int(a.d), a.N, a.T, a.k, a.ids, a.pos,
                       a.rows, a.a_rows, static_cast<uint16_t*>(a.routed), a.errors);
  return hipGetLastError();
}

// The four counters of a layer whose ids come from its own router (in range
// by construction): all T k slots are rows, none dropped, load not counted.
__global__ void k_slot_stats(int64_t n, int32_t* __restrict__ st) {
  if (threadIdx.x == 0) {
    st[0] = int32_t(n);
    st[1] = 0;
    st[2] = -1;
    st[3] = 0;
  }
}

}  // namespace

hipError_t launch_slot_stats(int64_t n, void* stats, hipStream_t s) {
  hipLaunchKernelGGL(k_slot_stats, dim3(1), dim3(64), 0, s, n, static_cast<int32_t*>(stats));
  return hipGetLastError();
}

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
