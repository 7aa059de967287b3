// RMSNorm statistic, router GEMM with the r-scale epilogue, top-k gating,
// and the two-stage top-k of the Cartesian-product router.
//
// CODA sparse-MoE thread (router-fusion paragraph): the router is a plain
// GEMM right after the RMSNorm, and the per-token statistic r is applied to
// its output just before the top-k.  The GEMM therefore reads the raw rows
// of x once; the sum of squares that gives r is accumulated from the same
// registers that feed the matrix cores.
//
// "Mixture of Experts (MoE)" glossary, top-k gating: the k highest-scoring
// experts are selected (k = 1 is switch routing) and weighted by their
// scores -- here a softmax over the k selected logits (or the full-softmax
// probability).  Ties go to the lower expert index; slot 0 is the best.
//
// OmniMoE summary, 2.2 (Cartesian-product router): expert n = i*Nc + j
// scores s1[i] + s2[j].  The exact top-k over the Nr x Nc grid is found
// among the k x k pairs of the row top-k and the column top-k.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- RMSNorm

template <typename T>
__global__ void __launch_bounds__(256) k_rmsnorm(const T* __restrict__ x, int64_t T_, int64_t d,
                                                 const T* __restrict__ gamma, float eps,
                                                 float* __restrict__ r, T* __restrict__ xg) {
  const int lane = threadIdx.x & 63;
  const int64_t t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  constexpr int N = Vec16<T>::N;
  const int64_t nvec = d / N;
  const uint4* xs = reinterpret_cast<const uint4*>(x + t * d);
  float ss = 0.f;
  for (int64_t v = lane; v < nvec; v += 64) {
    float f[8];
    unpack16(xs[v], f, (const T*)nullptr);
#pragma unroll
    for (int i = 0; i < N; ++i) ss = fmaf(f[i], f[i], ss);
  }
  ss = wave_sum(ss);
  const float rr = 1.0f / sqrtf(ss / float(d) + eps);
  if (lane == 0) r[t] = rr;
  if (gamma && xg) {
    const uint4* gs = reinterpret_cast<const uint4*>(gamma);
    uint4* xo = reinterpret_cast<uint4*>(xg + t * d);
    for (int64_t v = lane; v < nvec; v += 64) {
      float f[8], g[8];
      unpack16(xs[v], f, (const T*)nullptr);
      unpack16(gs[v], g, (const T*)nullptr);
#pragma unroll
      for (int i = 0; i < N; ++i) f[i] *= g[i];
      xo[v] = pack16(f, (const T*)nullptr);
    }
  }
}

// ---------------------------------------------------------------- top-k helpers

struct KV {
  float v;
  int i;
};
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}
// Wave-wide best (value desc, index asc); every lane gets the result.
__device__ __forceinline__ KV wave_best(float v, int i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(i, o, 64);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
  return KV{v, i};
}

// Top-k of n values held as lane-strided registers vals[q] (index lane + 64q),
// q < Q.  Selection j (j < k <= 64*QS) lands in lane j % 64, register j / 64.
template <int Q, int QS>
__device__ void wave_topk(const float (&vals)[Q], int n, int k, float (&sv)[QS], int (&si)[QS]) {
  const int lane = threadIdx.x & 63;
  bool live[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) live[q] = lane + 64 * q < n;
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    sv[q] = -INFINITY;
    si[q] = 0;
  }
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int idx = lane + 64 * q;
      if (live[q] && better(vals[q], idx, bv, bi)) {
        bv = vals[q];
        bi = idx;
      }
    }
    const KV w = wave_best(bv, bi);
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (lane + 64 * q == w.i) live[q] = false;
#pragma unroll
    for (int q = 0; q < QS; ++q)
      if ((j >> 6) == q && (j & 63) == lane) {
        sv[q] = w.v;
        si[q] = w.i;
      }
  }
}

// Order-preserving map of an fp32 score to uint32 (larger score, larger
// key); NaN maps to 0, below every number, and so does padding.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t b = __float_as_uint(f);
  if (f != f) return 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Largest key th with at least k of the wave's keys >= th, i.e. the k-th
// largest key, found bit by bit from the top.  Counts come from ballots
// (one compare per held key, popcounts in scalar registers), so no
// cross-lane shuffles sit on the dependency chain.
template <int Q>
__device__ __forceinline__ uint32_t kth_largest_key(const uint32_t (&u)[Q], int k) {
  uint32_t th = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = th | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) cnt += __popcll(__ballot(u[q] >= cand));
    if (cnt >= k) th = cand;
  }
  return th;
}

// The same threshold, usually from far fewer ballots: the k-th largest of the
// 64 lane maxima is a lower bound L (k lane maxima are >= L); when at most 64
// keys reach L they are compacted one per lane (through the wave's LDS
// slice `cand`) and the threshold is searched among them alone.
template <int Q>
__device__ __forceinline__ uint32_t kth_largest_key_fast(const uint32_t (&u)[Q], int k,
                                                         uint32_t* cand) {
  uint32_t mx[1] = {u[0]};
#pragma unroll
  for (int q = 1; q < Q; ++q) mx[0] = max(mx[0], u[q]);
  const uint32_t lo = kth_largest_key<1>(mx, k);
  int c = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) c += __popcll(__ballot(u[q] >= lo));
  if (c > 64) return kth_largest_key<Q>(u, k);
  const int lane = threadIdx.x & 63;
  int base = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint64_t m = __ballot(u[q] >= lo);
    if (u[q] >= lo) cand[base + rank_below(m)] = u[q];
    base += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint32_t cu[1] = {lane < c ? cand[lane] : 0u};
  __builtin_amdgcn_wave_barrier();
  return kth_largest_key<1>(cu, k);
}

// Top-k of one token's n values (lane l holds index l + 64 q) for k <= 64,
// slots ordered by (value descending, index ascending), and their gates
// (softmax over the k, or over all n when renorm is 0); writes ids / w of
// token t.  Selection by threshold: the k-th largest key, everything above
// it and the lowest-index ties at it, compacted through the wave's LDS
// slices (64 entries each); a winner's slot is its rank among the k.
// pacc / gacc / cacc (the wave's LDS rows of n, or NULL) accumulate the
// token's full-softmax probabilities, its gates and its slots per expert.
template <int Q>
__device__ void wave_select_gates(const float (&vals)[Q], int n, int k, int renorm, int64_t t,
                                  int32_t* __restrict__ ids, float* __restrict__ wout,
                                  uint32_t* cand, float* selv, int* seli, float* pacc = nullptr,
                                  float* gacc = nullptr, int* cacc = nullptr) {
  const int lane = threadIdx.x & 63;
  uint32_t u[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) u[q] = lane + 64 * q < n ? score_key(vals[q]) : 0u;
  uint32_t th;
  if constexpr (Q == 1) th = kth_largest_key<1>(u, k);
  else th = kth_largest_key_fast<Q>(u, k, cand);
  int need = k;
#pragma unroll
  for (int q = 0; q < Q; ++q) need -= __popcll(__ballot(u[q] > th));
  int base = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint64_t eq = __ballot(u[q] == th);
    const bool take_eq = u[q] == th && rank_below(eq) < need;
    need -= min(need, __popcll(eq));
    const bool sel = u[q] > th || take_eq;
    const uint64_t sm = __ballot(sel);
    if (sel) {
      const int p = base + rank_below(sm);
      selv[p] = vals[q];
      seli[p] = lane + 64 * q;
    }
    base += __popcll(sm);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const bool mine = lane < k;
  const float sv = mine ? selv[lane] : -INFINITY;
  const int si = mine ? seli[lane] : 0x7fffffff;
  const uint32_t su = mine ? score_key(sv) : 0u;
  __builtin_amdgcn_wave_barrier();
  int rank = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t uj = __builtin_amdgcn_readlane(su, j);
    const int ij = __builtin_amdgcn_readlane(si, j);
    rank += (uj > su || (uj == su && ij < si)) ? 1 : 0;
  }
  const uint64_t top = __ballot(mine && rank == 0);
  const float mx =
      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), int(__builtin_ctzll(top))));
  float den = 0.f;
  if (renorm) {
    den = mine ? expf(sv - mx) : 0.f;
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (lane + 64 * q < n) den += expf(vals[q] - mx);
  }
  den = wave_sum(den);
  const float gate = expf(sv - mx) / den;
  if (mine) {
    ids[t * k + rank] = si;
    wout[t * k + rank] = gate;
  }
  if (pacc) {
    float zall = den;
    if (renorm) {
      float zz = 0.f;
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (lane + 64 * q < n) zz += expf(vals[q] - mx);
      zall = wave_sum(zz);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (lane + 64 * q < n) pacc[lane + 64 * q] += expf(vals[q] - mx) / zall;
  }
  if (gacc && mine) {
    gacc[si] += gate;
    cacc[si] += 1;
  }
}

// Gates of the k selections held as in wave_topk; writes ids / w of token t.
template <int QS, int Q>
__device__ void write_gates(const float (&sv)[QS], const int (&si)[QS], const float (&vals)[Q],
                            int n, int k, int renorm, int64_t t, int32_t* ids, float* wout) {
  const int lane = threadIdx.x & 63;
  const float mx = __shfl(sv[0], 0, 64);
  float denom = 0.f;
  if (renorm) {
#pragma unroll
    for (int q = 0; q < QS; ++q)
      if (lane + 64 * q < k) denom += expf(sv[q] - mx);
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (lane + 64 * q < n) denom += expf(vals[q] - mx);
  }
  denom = wave_sum(denom);
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    const int j = lane + 64 * q;
    if (j < k) {
      ids[t * k + j] = si[q];
      wout[t * k + j] = expf(sv[q] - mx) / denom;
    }
  }
}

// ---------------------------------------------------------------- dense router, bf16 (MFMA)

constexpr int kRouterTok = 16;  // tokens per workgroup (one 16-wide MFMA block)

// Workgroup: NW waves split K; each wave runs 16x16x32 MFMAs with the router
// rows as the A operand (16 experts per block) and 16 token rows as B.  More
// waves per workgroup keep fewer loads outstanding per wave and more per CU
// (the token rows are read once, so the kernel is bound by how many loads
// are in flight).
template <int NB, int NW>
__global__ void __launch_bounds__(64 * NW) k_router_bf16(
    const uint16_t* __restrict__ x, int T, int d, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int E, const float* __restrict__ r_in, float eps,
    float* __restrict__ r_out, int k, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ wout, float* __restrict__ logits, RouterExtras ex) {
  constexpr int QV = (NB * 16 + 63) / 64;   // logits per lane in the top-k
  __shared__ float lg[kRouterTok][NB * 16 + 1];
  __shared__ float ssq[kRouterTok];
  __shared__ float rs[kRouterTok];
  __shared__ uint32_t cand_s[NW][64];
  __shared__ float selv_s[NW][64];
  __shared__ int seli_s[NW][64];
  __shared__ float pacc_s[NW][NB * 16];
  __shared__ float gacc_s[NW][NB * 16];
  __shared__ int cacc_s[NW][NB * 16];
  static_assert(kRouterTok % NW == 0, "whole tokens per wave in the epilogue");
  const bool stats = ex.part_p != nullptr;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRouterTok;
  const int tl = lane & 15;       // token within the block (B column)
  const int kg = lane >> 4;       // which 8-element K group
  const int t = t0 + tl;
  const bool tok_ok = t < T;
  const int kw = d / NW;          // K range of this wave
  const int kb = wid * kw;
  if (stats)
    for (int e = lane; e < NB * 16; e += 64) {
      pacc_s[wid][e] = gacc_s[wid][e] = 0.f;
      cacc_s[wid][e] = 0;
    }

  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  const uint16_t* xrow = x + int64_t(tok_ok ? t : 0) * d + kb + kg * 8;
  const uint16_t* wrow[NB];
  bool wok[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = b * 16 + tl;
    wok[b] = e < E;
    wrow[b] = wr + int64_t(wok[b] ? e : 0) * d + kb + kg * 8;
  }
  // K steps of 32 in groups of U: the loads of a group are issued together
  // and unconditionally (rows past T or E read row 0, in bounds, and are
  // zeroed by a select), so no branch puts a wait between a load and the
  // next one; then the group's MFMAs run in K order.  With one expert block
  // a group of 8 (64 registers of loads) covers a 256-wide K range in one
  // round trip to memory.
  constexpr int U = NB == 1 ? 8 : 4;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  auto kstep = [&](const uint4& xv_in, const uint4 (&wv)[NB]) __attribute__((always_inline)) {
    const uint4 xv = tok_ok ? xv_in : zero4;
    float f[8];
    unpack16(xv, f, (const uint16_t*)nullptr);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
    const bf16x8 bx = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint4 wb = wok[b] ? wv[b] : zero4;
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wb), bx, acc[b], 0, 0, 0);
    }
  };
  const int nit = kw / 32;
  int it = 0;
  for (; it + U <= nit; it += U) {
    uint4 xv[U], wv[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xv[u] = *reinterpret_cast<const uint4*>(xrow + (it + u) * 32);
#pragma unroll
      for (int b = 0; b < NB; ++b) wv[u][b] = *reinterpret_cast<const uint4*>(wrow[b] + (it + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) kstep(xv[u], wv[u]);
  }
  for (; it < nit; ++it) {
    uint4 wv[NB];
    const uint4 xv = *reinterpret_cast<const uint4*>(xrow + it * 32);
#pragma unroll
    for (int b = 0; b < NB; ++b) wv[b] = *reinterpret_cast<const uint4*>(wrow[b] + it * 32);
    kstep(xv, wv);
  }
  // sum of squares of the token over this wave's K range (lanes tl, tl+16, ...)
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  // ordered cross-wave reduction (wave 0, then 1, 2, ...): deterministic.
  // With few experts every wave's partial goes to LDS at once and one pass
  // sums them in wave order; otherwise the waves add into one row in turn.
  constexpr bool kOnePass = NW * kRouterTok * (NB * 16 + 1) * 4 <= 40960;
  if constexpr (kOnePass) {
    __shared__ float part[kOnePass ? NW : 1][kRouterTok][NB * 16 + 1];
    __shared__ float sq_part[NW][kRouterTok];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[wid][tl][b * 16 + kg * 4 + v] = acc[b][v];
    if (lane < 16) sq_part[wid][tl] = ss;
    __syncthreads();
    for (int i = threadIdx.x; i < kRouterTok * NB * 16; i += 64 * NW) {
      const int t2 = i / (NB * 16), e = i - t2 * (NB * 16);
      float sum = part[0][t2][e];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += part[w][t2][e];
      lg[t2][e] = sum;
    }
    if (threadIdx.x < kRouterTok) {
      float sum = sq_part[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += sq_part[w][threadIdx.x];
      ssq[threadIdx.x] = sum;
    }
    __syncthreads();
  } else {
    for (int w = 0; w < NW; ++w) {
      if (wid == w) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int e = b * 16 + kg * 4 + v;
            if (w == 0) lg[tl][e] = acc[b][v];
            else lg[tl][e] += acc[b][v];
          }
        if (lane < 16) {
          if (w == 0) ssq[tl] = ss;
          else ssq[tl] += ss;
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x < kRouterTok) {
    const int tt = t0 + threadIdx.x;
    float rr = 0.f;
    if (tt < T) {
      rr = r_in ? r_in[tt] : 1.0f / sqrtf(ssq[threadIdx.x] / float(d) + eps);
      if (!r_in && r_out) r_out[tt] = rr;
    }
    rs[threadIdx.x] = rr;
  }
  __syncthreads();
  // epilogue: r-scale + bias, then top-k per token (each wave: 16 / NW tokens)
  for (int q = 0; q < kRouterTok / NW; ++q) {
    const int tl2 = wid * (kRouterTok / NW) + q;
    const int tt = t0 + tl2;
    if (tt >= T) break;
    const float rr = rs[tl2];
    float vals[QV];
#pragma unroll
    for (int qq = 0; qq < QV; ++qq) {
      const int e = lane + 64 * qq;
      vals[qq] = -INFINITY;
      if (e < E) {
        vals[qq] = rr * lg[tl2][e] + (bias ? bias[e] : 0.f);
        if (ex.noise) vals[qq] += ex.noise_std * ex.noise[int64_t(tt) * E + e];
        if (logits) logits[int64_t(tt) * E + e] = vals[qq];
      }
    }
    if (k <= 64) {
      wave_select_gates<QV>(vals, E, k, renorm, tt, ids, wout, cand_s[wid], selv_s[wid],
                            seli_s[wid], stats ? pacc_s[wid] : nullptr,
                            stats ? gacc_s[wid] : nullptr, stats ? cacc_s[wid] : nullptr);
    } else {
      float sv[QV];
      int si[QV];
      wave_topk<QV, QV>(vals, E, k, sv, si);
      write_gates<QV, QV>(sv, si, vals, E, k, renorm, tt, ids, wout);
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (stats) {
    // the workgroup's partial sums: waves combined in a fixed order
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 64 * NW) {
      float sp = 0.f, sg = 0.f;
      int sc = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sp += pacc_s[w][e];
        sg += gacc_s[w][e];
        sc += cacc_s[w][e];
      }
      ex.part_p[int64_t(blockIdx.x) * E + e] = sp;
      ex.part_g[int64_t(blockIdx.x) * E + e] = sg;
      ex.part_c[int64_t(blockIdx.x) * E + e] = sc;
    }
  }
}

// ---------------------------------------------------------------- dense router, fp32

__global__ void k_router_logits_f32(const float* __restrict__ x, int T, int d,
                                    const float* __restrict__ wr, const float* __restrict__ bias,
                                    int E, const float* __restrict__ r_in, float eps,
                                    float* __restrict__ r_out, float* __restrict__ lg) {
  const int64_t g = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (g >= int64_t(T) * E) return;
  const int t = int(g / E), e = int(g % E);
  const float* xr = x + int64_t(t) * d;
  const float* wrow = wr + int64_t(e) * d;
  float acc = 0.f, ss = 0.f;
  for (int i = 0; i < d; ++i) {
    acc = fmaf(xr[i], wrow[i], acc);
    ss = fmaf(xr[i], xr[i], ss);
  }
  const float rr = r_in ? r_in[t] : 1.0f / sqrtf(ss / float(d) + eps);
  if (!r_in && r_out && e == 0) r_out[t] = rr;
  lg[g] = rr * acc + (bias ? bias[e] : 0.f);
}

__global__ void __launch_bounds__(256) k_topk_rows(float* __restrict__ lg, int T, int E, int k,
                                                   int renorm, int32_t* __restrict__ ids,
                                                   float* __restrict__ wout, RouterExtras ex) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __shared__ uint32_t cand_s[4][64];
  __shared__ float selv_s[4][64];
  __shared__ int seli_s[4][64];
  __shared__ float pacc_s[4][256];
  __shared__ float gacc_s[4][256];
  __shared__ int cacc_s[4][256];
  const bool stats = ex.part_p != nullptr;
  const int t = blockIdx.x * 4 + wid;
  if (stats)
    for (int e = lane; e < E; e += 64) {
      pacc_s[wid][e] = gacc_s[wid][e] = 0.f;
      cacc_s[wid][e] = 0;
    }
  if (t < T) {
    float vals[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      vals[q] = -INFINITY;
      if (e < E) {
        vals[q] = lg[int64_t(t) * E + e];
        if (ex.noise) {
          vals[q] += ex.noise_std * ex.noise[int64_t(t) * E + e];
          lg[int64_t(t) * E + e] = vals[q];
        }
      }
    }
    if (k <= 64) {
      wave_select_gates<4>(vals, E, k, renorm, t, ids, wout, cand_s[wid], selv_s[wid],
                           seli_s[wid], stats ? pacc_s[wid] : nullptr,
                           stats ? gacc_s[wid] : nullptr, stats ? cacc_s[wid] : nullptr);
    } else {
      float sv[4];
      int si[4];
      wave_topk<4, 4>(vals, E, k, sv, si);
      write_gates<4, 4>(sv, si, vals, E, k, renorm, t, ids, wout);
    }
  }
  if (stats) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
      float sp = 0.f, sg = 0.f;
      int sc = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        sp += pacc_s[w][e];
        sg += gacc_s[w][e];
        sc += cacc_s[w][e];
      }
      ex.part_p[int64_t(blockIdx.x) * E + e] = sp;
      ex.part_g[int64_t(blockIdx.x) * E + e] = sg;
      ex.part_c[int64_t(blockIdx.x) * E + e] = sc;
    }
  }
}

// Routing statistics from the per-workgroup partial sums.  k_router_sums:
// one workgroup per expert; thread i adds the partial rows i, i + 256, ...
// and a fixed-shape tree combines the 256 sums, so the order never varies.
__global__ void __launch_bounds__(256) k_router_sums(const float* __restrict__ part_p,
                                                     const float* __restrict__ part_g,
                                                     const int* __restrict__ part_c, int nblk,
                                                     int E, float* __restrict__ sum_p,
                                                     float* __restrict__ sum_g,
                                                     long long* __restrict__ sum_c) {
  __shared__ float sp[256], sg[256];
  __shared__ long long sc[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  float ap = 0.f, ag = 0.f;
  long long ac = 0;
  for (int b = tid; b < nblk; b += 256) {
    ap += part_p[int64_t(b) * E + e];
    ag += part_g[int64_t(b) * E + e];
    ac += part_c[int64_t(b) * E + e];
  }
  sp[tid] = ap;
  sg[tid] = ag;
  sc[tid] = ac;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) {
      sp[tid] += sp[tid + h];
      sg[tid] += sg[tid + h];
      sc[tid] += sc[tid + h];
    }
    __syncthreads();
  }
  if (tid == 0) {
    sum_p[e] = sp[0];
    sum_g[e] = sg[0];
    sum_c[e] = sc[0];
  }
}

// The squared coefficient of variation (population variance / mean^2) of the
// three per-expert sums, in float64 (one workgroup, three threads).
__global__ void __launch_bounds__(64) k_router_cv2(const float* __restrict__ sum_p,
                                                   const float* __restrict__ sum_g,
                                                   const long long* __restrict__ sum_c, int E,
                                                   float* __restrict__ prob_sum,
                                                   float* __restrict__ gate_sum,
                                                   float* __restrict__ aux) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 64) {
    if (prob_sum) prob_sum[e] = sum_p[e];
    if (gate_sum) gate_sum[e] = sum_g[e];
  }
  if (tid < 3 && aux) {
    auto val = [&](int i) {
      return tid == 0 ? double(sum_p[i]) : tid == 1 ? double(sum_g[i]) : double(sum_c[i]);
    };
    double s1 = 0.0;
    for (int i = 0; i < E; ++i) s1 += val(i);
    const double mean = s1 / E;
    double s2 = 0.0;
    for (int i = 0; i < E; ++i) {
      const double v = val(i) - mean;
      s2 += v * v;
    }
    aux[tid] = mean != 0.0 ? float((s2 / E) / (mean * mean)) : __int_as_float(0x7fc00000);
  }
}

// ---------------------------------------------------------------- Cartesian two-stage top-k

// One wave per token.  scores row = [s1 (Nr) | s2 (Nc)] fp32; lane l holds
// elements l + 64 q.  Stage 1 selects the k best rows of s1 and the k best
// columns of s2 (score descending, index ascending); stage 2 selects the k
// best of the k * k pair sums (sum descending, flat id row * Nc + col
// ascending), which contain the k best pairs of the whole grid.  Each
// selection finds the k-th largest key, keeps everything above it and the
// needed number of ties at it in index order, and compacts the winners
// into LDS; the final k are placed by rank.  Q = ceil(max(Nr, Nc, k*k)/64).
template <int Q>
__global__ void __launch_bounds__(256) k_cartesian_topk(const float* __restrict__ scores, int T,
                                                        int Nr, int Nc, int k, int renorm,
                                                        int32_t* __restrict__ ids,
                                                        float* __restrict__ wout) {
  __shared__ float sel_v[4][2][64];
  __shared__ int sel_i[4][2][64];
  __shared__ uint32_t cand_s[4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wid;
  if (t >= T) return;
  const float* row = scores + int64_t(t) * (Nr + Nc);
  float m[2] = {-INFINITY, -INFINITY}, z[2] = {0.f, 0.f};

  // stage 1: list 0 = rows of s1, list 1 = columns of s2
#pragma unroll
  for (int list = 0; list < 2; ++list) {
    const int n = list == 0 ? Nr : Nc;
    const float* src = row + (list == 0 ? 0 : Nr);
    float v[Q];
    uint32_t u[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = lane + 64 * q;
      v[q] = i < n ? src[i] : -INFINITY;
      u[q] = i < n ? score_key(v[q]) : 0u;
    }
    if (!renorm) {
      float mx = -INFINITY;
#pragma unroll
      for (int q = 0; q < Q; ++q) mx = fmaxf(mx, v[q]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      float zz = 0.f;
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (lane + 64 * q < n) zz += expf(v[q] - mx);
      m[list] = mx;
      z[list] = wave_sum(zz);
    }
    const uint32_t th = kth_largest_key_fast<Q>(u, k, cand_s[wid]);
    int need = k;
#pragma unroll
    for (int q = 0; q < Q; ++q) need -= __popcll(__ballot(u[q] > th));
    int base = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      // ties at the threshold go to the lowest indices: q ascending, then lane
      const uint64_t eq = __ballot(u[q] == th);
      const bool take_eq = u[q] == th && rank_below(eq) < need;
      need -= min(need, __popcll(eq));
      const bool sel = u[q] > th || take_eq;
      const uint64_t sm = __ballot(sel);
      if (sel) {
        const int p = base + rank_below(sm);
        sel_v[wid][list][p] = v[q];
        sel_i[wid][list][p] = lane + 64 * q;
      }
      base += __popcll(sm);
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // stage 2: candidate c = a * k + b pairs row choice a with column choice b
  // (a, b) of c = lane + 64 q advance by (64 / k, 64 % k) per q with one
  // carry, instead of a division per candidate
  const int nc = k * k;
  const int da = 64 / k, db = 64 - da * k;
  int a = lane / k, b = lane - (lane / k) * k;
  float cv[Q];
  int cid[Q];
  uint32_t cu[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = lane + 64 * q;
    if (c < nc) {
      cv[q] = sel_v[wid][0][a] + sel_v[wid][1][b];
      cid[q] = sel_i[wid][0][a] * Nc + sel_i[wid][1][b];
      cu[q] = score_key(cv[q]);
    } else {
      cv[q] = -INFINITY;
      cid[q] = 0x7fffffff;
      cu[q] = 0u;
    }
    a += da;
    b += db;
    if (b >= k) {
      b -= k;
      ++a;
    }
  }
  const uint32_t th = kth_largest_key_fast<Q>(cu, k, cand_s[wid]);
  int need = k;
  bool sel[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    sel[q] = cu[q] > th;
    need -= __popcll(__ballot(sel[q]));
  }
  // ties at the threshold go to the lowest flat ids (exact fp32 ties only)
  while (need > 0) {
    int best = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (cu[q] == th && !sel[q]) best = min(best, cid[q]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o, 64));
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (cu[q] == th && !sel[q] && cid[q] == best) sel[q] = true;
    --need;
  }
  // compact the k winners to lanes 0 .. k-1 (through LDS list 0)
  __builtin_amdgcn_wave_barrier();
  int base = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint64_t sm = __ballot(sel[q]);
    if (sel[q]) {
      const int p = base + rank_below(sm);
      sel_v[wid][0][p] = cv[q];
      sel_i[wid][0][p] = cid[q];
    }
    base += __popcll(sm);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const bool mine = lane < k;
  const float sv = mine ? sel_v[wid][0][lane] : -INFINITY;
  const int si = mine ? sel_i[wid][0][lane] : 0x7fffffff;
  const uint32_t su = mine ? score_key(sv) : 0u;
  // slot = rank among the k winners (sum descending, flat id ascending)
  int rank = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t uj = __builtin_amdgcn_readlane(su, j);
    const int ij = __builtin_amdgcn_readlane(si, j);
    rank += (uj > su || (uj == su && ij < si)) ? 1 : 0;
  }
  // the best sum is the one of rank 0
  const uint64_t top = __ballot(mine && rank == 0);
  const float mx = __shfl(sv, int(__builtin_ctzll(top)), 64);
  if (renorm) {
    const float e = mine ? expf(sv - mx) : 0.f;
    const float dd = wave_sum(e);
    if (!mine) return;
    ids[int64_t(t) * k + rank] = si;
    wout[int64_t(t) * k + rank] = e / dd;
  } else {
    if (!mine) return;
    // full softmax over the grid: sum_ij exp(s1_i + s2_j) = (sum_i e^s1_i)(sum_j e^s2_j)
    ids[int64_t(t) * k + rank] = si;
    const float s1 = row[si / Nc], s2 = row[Nr + si % Nc];
    wout[int64_t(t) * k + rank] = expf(s1 - m[0]) * expf(s2 - m[1]) / (z[0] * z[1]);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, int dtype, int64_t T, int64_t d, const void* gamma,
                          float eps, float* r, void* xg, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 g(unsigned((T + 3) / 4));
  if (dtype == 0)
    hipLaunchKernelGGL(k_rmsnorm<float>, g, dim3(256), 0, s, static_cast<const float*>(x), T, d,
                       static_cast<const float*>(gamma), eps, r, static_cast<float*>(xg));
  else
    hipLaunchKernelGGL(k_rmsnorm<uint16_t>, g, dim3(256), 0, s, static_cast<const uint16_t*>(x), T,
                       d, static_cast<const uint16_t*>(gamma), eps, r, static_cast<uint16_t*>(xg));
  return hipGetLastError();
}

int64_t router_dense_blocks(int dtype, int64_t T) {
  return dtype == 0 ? (T + 3) / 4 : (T + kRouterTok - 1) / kRouterTok;
}

hipError_t launch_router_dense(const void* x, int dtype, int64_t T, int64_t d, const void* wr_t,
                               const float* bias, int64_t E, const float* r_in, float eps,
                               float* r_out, int k, int renorm, int32_t* ids, float* w,
                               float* logits, const RouterExtras& ex, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 0) {
    // fp32: logits into the caller's buffer (required), then top-k per row
    const int64_t n = T * E;
    hipLaunchKernelGGL(k_router_logits_f32, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(x), int(T), int(d),
                       static_cast<const float*>(wr_t), bias, int(E), r_in, eps, r_out, logits);
    hipLaunchKernelGGL(k_topk_rows, dim3(unsigned((T + 3) / 4)), dim3(256), 0, s, logits, int(T),
                       int(E), k, renorm, ids, w, ex);
  } else {
    const dim3 g(unsigned((T + kRouterTok - 1) / kRouterTok));
    const int nb = int((E + 15) / 16);
    // waves per workgroup: each wave's K range a multiple of 32; with more
    // than 32 experts 8 waves, whose partial logits still fit the one-pass
    // reduction in LDS
    const int nw = d % (16 * 32) == 0 && nb <= 2 ? 16 : d % (8 * 32) == 0 ? 8 : 4;
#define MOE_ROUTER_CASE(NBV, NWV)                                                              \
    hipLaunchKernelGGL((k_router_bf16<NBV, NWV>), g, dim3(64 * NWV), 0, s,                       \
                       static_cast<const uint16_t*>(x), int(T), int(d),                         \
                       static_cast<const uint16_t*>(wr_t), bias, int(E), r_in, eps, r_out, k,   \
                       renorm, ids, w, logits, ex)
#define MOE_ROUTER_NB(NWV)                                                                     \
    if (nb <= 1) MOE_ROUTER_CASE(1, NWV);                                                      \
    else if (nb <= 2) MOE_ROUTER_CASE(2, NWV);                                                 \
    else if (nb <= 4) MOE_ROUTER_CASE(4, NWV);                                                 \
    else if (nb <= 8) MOE_ROUTER_CASE(8, NWV);                                                 \
    else MOE_ROUTER_CASE(16, NWV);
    if (nw == 16) {
      MOE_ROUTER_NB(16)
    } else if (nw == 8) {
      MOE_ROUTER_NB(8)
    } else {
      MOE_ROUTER_NB(4)
    }
#undef MOE_ROUTER_NB
#undef MOE_ROUTER_CASE
  }
  if (ex.part_p) {
    hipLaunchKernelGGL(k_router_sums, dim3(unsigned(E)), dim3(256), 0, s, ex.part_p, ex.part_g,
                       ex.part_c, int(router_dense_blocks(dtype, T)), int(E), ex.sum_p, ex.sum_g,
                       ex.sum_c);
    hipLaunchKernelGGL(k_router_cv2, dim3(1), dim3(64), 0, s, ex.sum_p, ex.sum_g, ex.sum_c,
                       int(E), ex.prob_sum, ex.gate_sum, ex.aux);
  }
  return hipGetLastError();
}

hipError_t launch_cartesian_topk(const float* scores, int64_t T, int64_t Nr, int64_t Nc, int k,
                                 int renorm, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t need = std::max<int64_t>(std::max<int64_t>(Nr, Nc), int64_t(k) * k);
  const dim3 g(unsigned((T + 3) / 4));
  if (need <= 64 * 4)
    hipLaunchKernelGGL(k_cartesian_topk<4>, g, dim3(256), 0, s, scores, int(T), int(Nr), int(Nc),
                       k, renorm, ids, w);
  else if (need <= 64 * 16)
    hipLaunchKernelGGL(k_cartesian_topk<16>, g, dim3(256), 0, s, scores, int(T), int(Nr),
                       int(Nc), k, renorm, ids, w);
  else if (need <= 64 * 32)
    hipLaunchKernelGGL(k_cartesian_topk<32>, g, dim3(256), 0, s, scores, int(T), int(Nr),
                       int(Nc), k, renorm, ids, w);
  else
    hipLaunchKernelGGL(k_cartesian_topk<64>, g, dim3(256), 0, s, scores, int(T), int(Nr),
                       int(Nc), k, renorm, ids, w);
  return hipGetLastError();
}

}  // namespace moe
