// Backward pass of the MoE layer: the kernels around the expert GEMMs.
//
// CODA sparse-MoE thread: the RMSNorm backward is fused into the backward of
// the linear that consumed the normed input, and needs the saved statistic r
// (the reason r is applied in epilogues).  Here the per-slot gradients of the
// normed input are summed back to token order in one pass that also applies
// the RMSNorm backward with r, so no normed activation is ever stored.
//
// The weight gradients are GEMMs over the rows of each expert (K = rows).
// Their operands are made K-contiguous by a gather-transpose that also
// applies the row's factor (gate or r) and zero-fills each expert's rows up
// to a multiple of 64 (the GEMM's K stage): the role the sparse transpose of
// the "Variable-size experts" nanoMOE notes plays for their block-sparse
// backward.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

__device__ __forceinline__ int pad64(int n) { return (n + 63) & ~63; }

// ---------------------------------------------------------------- gather-transpose

// out[base_e + m, j] = scale(row) * src[srow(row), m] for row = seg0_e + j,
// j < cnt_e, and 0 for cnt_e <= j < pad64(cnt_e); m < width_e.  A block moves
// a 64 (j) x 64 (m) tile through LDS.
__global__ void __launch_bounds__(256) k_gather_t(GatherTArgs a) {
  __shared__ uint16_t tile[64][64 + 2];
  const int e = blockIdx.z;
  const int seg0 = a.offsets ? a.offsets[e] : 0;
  const int cnt = a.offsets ? a.offsets[e + 1] - seg0 : a.dense_rows;
  const int j0 = int(blockIdx.y) * 64;
  if (j0 >= pad64(cnt)) return;
  int width, base;
  if (a.wfix > 0) {
    width = a.wfix;
    base = e * a.wfix;
  } else {
    width = a.wmul * (a.foff[e + 1] - a.foff[e]);
    base = a.wmul * a.foff[e];
  }
  const int m0 = int(blockIdx.x) * 64;
  if (m0 >= width) return;
  const int t = threadIdx.x;
  {
    const int jj = t >> 2, cq = (t & 3) * 16;
    const int j = j0 + jj;
    int srow = -1;
    float sc = 1.f;
    if (j < cnt) {
      const int row = seg0 + j;
      srow = a.rowmap ? a.rowmap[row] : row;
      if (a.rscale) sc = a.rscale[row];
    }
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (srow >= 0) {
      const uint4* p = reinterpret_cast<const uint4*>(a.src + int64_t(srow) * a.lds + m0 + cq);
      v0 = p[0];
      v1 = p[1];
    }
    float f[16];
    unpack16(v0, f, (const uint16_t*)nullptr);
    unpack16(v1, f + 8, (const uint16_t*)nullptr);
#pragma unroll
    for (int q = 0; q < 16; ++q) tile[jj][cq + q] = a.rscale ? f2bf(sc * f[q]) : f2bf(f[q]);
  }
  __syncthreads();
  {
    const int m = t >> 2, jq = (t & 3) * 16;
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      w[q] = uint32_t(tile[jq + 2 * q][m]) | (uint32_t(tile[jq + 2 * q + 1][m]) << 16);
    uint4* o = reinterpret_cast<uint4*>(a.out + int64_t(base + m0 + m) * a.ldo + j0 + jq);
    o[0] = make_uint4(w[0], w[1], w[2], w[3]);
    o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// ---------------------------------------------------------------- activation backward

// One block per (64 rows of an expert segment, 64 hidden units).  From the
// second linear's backward product t = dout_row . w2^T (ungated, bf16), the
// gate g and r of the row and the saved h and pre-activations a (and u):
//   dh = g t;  GELU: da = dh act'(a);  SwiGLU: da = dh u silu'(a), du = dh silu(a)
// written row-major in the packed order (dpre, the dxhat GEMM's operand) and
// transposed per segment (dpreT, and hT from h: the weight gradients'
// K-contiguous operands, zero past the segment's rows up to a multiple of
// 64), with the row's sums over the block's units of t * h (the gate's
// gradient) and (a da + u du) / r (the statistic's) in part[row, 2 blk].
__global__ void __launch_bounds__(256) k_act_bwd(ActBwdArgs a) {
  __shared__ uint16_t th[64][64 + 2];
  __shared__ uint16_t tda[64][64 + 2];
  __shared__ uint16_t tdu[64][64 + 2];
  const int e = blockIdx.z;
  const int seg0 = a.offsets ? a.offsets[e] : 0;
  const int cnt = a.offsets ? a.offsets[e + 1] - seg0 : a.dense_rows;
  const int j0 = int(blockIdx.y) * 64;
  if (j0 >= pad64(cnt)) return;
  const int fe = a.foff[e + 1] - a.foff[e];
  const int f0 = int(blockIdx.x) * 64;
  if (f0 >= fe) return;
  const bool swi = a.swiglu != 0;
  const int t = threadIdx.x;
  {
    const int jj = t >> 2, cq = (t & 3) * 16;
    const int j = j0 + jj;
    const int row = seg0 + j;
    const bool live = j < cnt;
    const int f = f0 + cq;                       // first of this thread's 16 units
    const int pk = swi ? (f / 32) * 64 + (f % 32) : f;
    float tv[16], hv[16], av[16], uv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) tv[q] = hv[q] = av[q] = uv[q] = 0.f;
    float gate = 0.f, rr = 0.f;
    if (live) {
      gate = a.row_w ? a.row_w[row] : 1.f;
      rr = a.row_r[row];
      const uint4* pt = reinterpret_cast<const uint4*>(a.t + int64_t(row) * a.ldt + f);
      const uint4* ph = reinterpret_cast<const uint4*>(a.h + int64_t(row) * a.ldh + f);
      const uint4* pa = reinterpret_cast<const uint4*>(a.pre + int64_t(row) * a.ldpre + pk);
      const uint4 t0 = pt[0], t1 = pt[1], h0 = ph[0], h1 = ph[1], a0 = pa[0], a1 = pa[1];
      unpack16(t0, tv, (const uint16_t*)nullptr);
      unpack16(t1, tv + 8, (const uint16_t*)nullptr);
      unpack16(h0, hv, (const uint16_t*)nullptr);
      unpack16(h1, hv + 8, (const uint16_t*)nullptr);
      unpack16(a0, av, (const uint16_t*)nullptr);
      unpack16(a1, av + 8, (const uint16_t*)nullptr);
      if (swi) {
        const uint4* pu = reinterpret_cast<const uint4*>(a.pre + int64_t(row) * a.ldpre + pk + 32);
        const uint4 u0 = pu[0], u1 = pu[1];
        unpack16(u0, uv, (const uint16_t*)nullptr);
        unpack16(u1, uv + 8, (const uint16_t*)nullptr);
      }
    }
    float da[16], du[16], sg = 0.f, sr = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      sg += tv[q] * hv[q];
      const float dh = gate * tv[q];
      if (swi) {
        const float sgm = sigmoidf(av[q]);
        da[q] = dh * uv[q] * sgm * (1.f + av[q] * (1.f - sgm));
        du[q] = dh * av[q] * sgm;
        sr += av[q] * da[q] + uv[q] * du[q];
      } else {
        da[q] = dh * (a.act == 1 ? gelu_tanh_grad(av[q]) : gelu_erf_grad(av[q]));
        du[q] = 0.f;
        sr += av[q] * da[q];
      }
    }
    // the four threads of a row are adjacent lanes: sum them in a fixed order
    sg += __shfl_xor(sg, 1, 64);
    sr += __shfl_xor(sr, 1, 64);
    sg += __shfl_xor(sg, 2, 64);
    sr += __shfl_xor(sr, 2, 64);
    if (live) {
      uint4* pd = reinterpret_cast<uint4*>(a.dpre + int64_t(row) * a.lddp + pk);
      pd[0] = pack16(da, (const uint16_t*)nullptr);
      pd[1] = pack16(da + 8, (const uint16_t*)nullptr);
      if (swi) {
        pd = reinterpret_cast<uint4*>(a.dpre + int64_t(row) * a.lddp + pk + 32);
        pd[0] = pack16(du, (const uint16_t*)nullptr);
        pd[1] = pack16(du + 8, (const uint16_t*)nullptr);
      }
      if (cq == 0) {
        float* pp = a.part + int64_t(row) * a.ldpart + 2 * (f0 / 64);
        pp[0] = sg;
        pp[1] = rr > 0.f ? sr / rr : 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      th[jj][cq + q] = f2bf(hv[q]);
      tda[jj][cq + q] = f2bf(da[q]);
      tdu[jj][cq + q] = f2bf(du[q]);
    }
  }
  __syncthreads();
  {
    // transposed stores: unit m (64) x 16 rows per thread; SwiGLU writes the
    // gate and up rows of the packed order
    const int m = t >> 2, jq = (t & 3) * 16;
    const int fu = f0 + m;
    const int pku = swi ? (fu / 32) * 64 + (fu % 32) : fu;
    auto put = [&](uint16_t (*tile)[66], uint16_t* out, int64_t orow) {
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q] = uint32_t(tile[jq + 2 * q][m]) | (uint32_t(tile[jq + 2 * q + 1][m]) << 16);
      uint4* o = reinterpret_cast<uint4*>(out + orow * a.ldo + j0 + jq);
      o[0] = make_uint4(w[0], w[1], w[2], w[3]);
      o[1] = make_uint4(w[4], w[5], w[6], w[7]);
    };
    put(th, a.hT, int64_t(a.foff[e]) + fu);
    const int64_t pbase = int64_t(swi ? 2 : 1) * a.foff[e];
    put(tda, a.dpreT, pbase + pku);
    if (swi) put(tdu, a.dpreT, pbase + pku + 32);
  }
}

// ---------------------------------------------------------------- weight-gradient tile plan

// Tiles of Y[xrow, c] = sum_j X[xrow, j] W[wbase_e + c, j] over each
// expert's K = pad64(rows_e): X rows of expert e are xb_e .. xb_e + xr_e - 1
// (xr_e = xmul * f_e at xmul * foff[e], or xfix rows at 0), c covers d in
// blocks of the tile edge, W rows start at e * wstride.
constexpr int kWgPlanMax = 4096;

__global__ void __launch_bounds__(1024) k_plan_wgrad(WgradPlanArgs p) {
  __shared__ int base_s[kWgPlanMax + 1];
  __shared__ long long sh[33];
  const int nunits = p.offsets ? p.E : 1;
  const int bt = p.tile;                       // tile edge (rows and columns)
  const int nf = p.d / bt;
  const int per = (nunits + blockDim.x - 1) / blockDim.x;
  const int lo = min(nunits, int(threadIdx.x) * per), hi = min(nunits, lo + per);
  auto xr_of = [&](int u) { return p.xfix > 0 ? p.xfix : p.xmul * (p.foff[u + 1] - p.foff[u]); };
  long long local = 0;
  for (int u = lo; u < hi; ++u) {
    const int c = ((xr_of(u) + bt - 1) / bt) * nf;
    base_s[u] = c;
    local += c;
  }
  long long total;
  {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    long long incl = local;
    for (int o = 1; o < 64; o <<= 1) {
      const long long v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
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
    total = sh[32];
    for (int u = lo; u < hi; ++u) {
      const int c = base_s[u];
      base_s[u] = int(b);
      b += c;
    }
    if (threadIdx.x == 0) base_s[nunits] = int(total);
  }
  __syncthreads();
  const int ntot = int(min<long long>(total, p.max_tiles));
  if (threadIdx.x == 0) *p.ntiles = ntot;
  for (int idx = threadIdx.x; idx < ntot; idx += blockDim.x) {
    int u = 0;
    {
      int l = 0, h = nunits + 1;            // last u with base_s[u] <= idx
      while (l < h) {
        const int mid = (l + h) >> 1;
        if (base_s[mid] <= idx) l = mid + 1;
        else h = mid;
      }
      u = l - 1;
    }
    const int n = idx - base_s[u];
    const int xr = xr_of(u);
    const int xb = p.xfix > 0 ? 0 : p.xmul * p.foff[u];
    const int mb = n / nf, cb = n - mb * nf;
    const int rows = p.offsets ? p.offsets[u + 1] - p.offsets[u] : p.dense_rows;
    Tile t{};
    t.expert = u;
    t.spare = 0;
    t.row0 = xb + mb * bt;
    t.row_end = xb + xr;
    t.wrow0 = u * p.wstride + cb * bt;
    t.kofs = 0;
    t.klen = pad64(rows);
    t.ocol0 = cb * bt;
    p.tiles[idx] = t;
  }
}

// ---------------------------------------------------------------- reductions

// dg_row[row] / dr_row[row]: sums over the row's 64-unit blocks of the
// activation backward's partials (fixed order).  Rows of no expert get 0.
__global__ void __launch_bounds__(256) k_reduce_part(const float* __restrict__ part, int64_t ldpart,
                                                     int64_t rows, const int32_t* __restrict__ row_expert,
                                                     const int32_t* __restrict__ foff, int dense_nft,
                                                     float* __restrict__ dg_row,
                                                     float* __restrict__ dr_row) {
  const int64_t row = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (row >= rows) return;
  int nft = dense_nft;
  if (row_expert) {
    const int e = row_expert[row];
    nft = e < 0 ? 0 : (foff[e + 1] - foff[e] + 63) / 64;
  }
  float sg = 0.f, sr = 0.f;
  for (int f = 0; f < nft; ++f) {
    sg += part[row * ldpart + 2 * f];
    sr += part[row * ldpart + 2 * f + 1];
  }
  if (dg_row) dg_row[row] = sg;
  dr_row[row] = sr;
}

// out[c] = sum over i < n of in[i * ld + c], in order.
__global__ void __launch_bounds__(256) k_colsum(const float* __restrict__ in, int64_t n, int64_t ld,
                                                int64_t cols, float* __restrict__ out) {
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (c >= cols) return;
  float s = 0.f;
  for (int64_t i = 0; i < n; ++i) s += in[i * ld + c];
  out[c] = s;
}

// ---------------------------------------------------------------- router backward

// One wave per token t < Tpad.  From the gate gradients dg (the slot's row
// sum, 0 for a dropped slot) and the saved logits l:
//   renorm = 1 (softmax over the k selected):  dl[sel_j] = g_j (dg_j - S)
//   renorm = 0 (full-softmax gates):            dl[e] = P_e (sum_{sel_j = e} dg_j - S)
// with S = sum_j g_j dg_j.  Writes dl [T, E] (fp32), dlT [E, ldt] (bf16, the
// weight-gradient operand; zero for t >= T) and the router's share of the
// statistic's gradient, dr[t] = sum_e ((l_e - b_e) / r) dl_e.
__global__ void __launch_bounds__(256) k_router_bwd(RouterBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = int(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.Tpad) return;
  const int E = a.E, k = a.k;
  if (t >= a.T) {
    for (int e = lane; e < E; e += 64) a.dlT[int64_t(e) * a.ldt + t] = 0;
    return;
  }
  const int32_t* ids = a.ids + int64_t(t) * k;
  const float* g = a.w + int64_t(t) * k;
  const int32_t* pos = a.pos + int64_t(t) * k;
  // S = sum_j g_j dg_j
  float s = 0.f;
  for (int j = lane; j < k; j += 64) {
    const int p = pos[j];
    const float dg = p >= 0 ? a.dg_row[p] : 0.f;
    s += g[j] * dg;
  }
  s = wave_sum(s);
  const float* l = a.logits + int64_t(t) * E;
  float m = -INFINITY, z = 0.f;
  if (!a.renorm) {
    for (int e = lane; e < E; e += 64) m = fmaxf(m, l[e]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    for (int e = lane; e < E; e += 64) z += expf(l[e] - m);
    z = wave_sum(z);
  }
  const float r = a.r[t];
  float drp = 0.f;
  for (int e = lane; e < E; e += 64) {
    float sdg = 0.f, gsel = 0.f;
    bool sel = false;
    for (int j = 0; j < k; ++j) {
      if (ids[j] == e) {
        const int p = pos[j];
        sdg += p >= 0 ? a.dg_row[p] : 0.f;
        gsel = g[j];
        sel = true;
      }
    }
    float dl;
    if (a.renorm) dl = sel ? gsel * (sdg - s) : 0.f;
    else dl = (expf(l[e] - m) / z) * (sdg - s);
    a.dl[int64_t(t) * E + e] = dl;
    a.dlT[int64_t(e) * a.ldt + t] = f2bf(dl);
    const float b = a.bias ? a.bias[e] : 0.f;
    if (r > 0.f) drp += (l[e] - b) / r * dl;
  }
  drp = wave_sum(drp);
  if (lane == 0) a.dr[t] = drp;
}

// ---------------------------------------------------------------- token backward

// One block per TB tokens.  For token t, with its kept slots' rows p_j:
//   dr_t   = sum_j dr_row[p_j] + dr_shared[t] + dr_router[t]
//   dxh[c] = sum_j dxperm[p_j, c] + dxs[t, c] + r_t sum_e dl[t, e] wr[e, c]
// (dxperm summed over its K-split planes)
//   dx[c]  = dout[t, c] (residual) + gamma[c] dxh[c] - (r_t^3 / d) dr_t x[t, c]
// (the RMSNorm backward with the saved r), and the block's partial of
// dgamma[c] = sum_t dxh[c] x[t, c].  Each thread owns 8 consecutive columns.
constexpr int kTokB = 8;

__global__ void __launch_bounds__(256) k_bwd_token(TokenBwdArgs a) {
  const int t0 = int(blockIdx.x) * kTokB;
  const int64_t d = a.d;
  for (int64_t c0 = int64_t(threadIdx.x) * 8; c0 < d; c0 += 256 * 8) {
    float gam[8], gacc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      gam[q] = 1.f;
      gacc[q] = 0.f;
    }
    if (a.gamma) {
      float tmp[8];
      unpack16(*reinterpret_cast<const uint4*>(a.gamma + c0), tmp, (const uint16_t*)nullptr);
#pragma unroll
      for (int q = 0; q < 8; ++q) gam[q] = tmp[q];
    }
    for (int t = t0; t < min(t0 + kTokB, int(a.T)); ++t) {
      const float r = a.r[t];
      float dr = a.dr_router[t] + (a.dr_shared ? a.dr_shared[t] : 0.f);
      float dxh[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) dxh[q] = 0.f;
      for (int j = 0; j < a.k; ++j) {
        const int p = a.pos[int64_t(t) * a.k + j];
        if (p < 0) continue;
        dr += a.dr_row[p];
        for (int sp = 0; sp < a.ksplit; ++sp) {
          const float4* s =
              reinterpret_cast<const float4*>(a.dxperm + sp * a.plane + int64_t(p) * d + c0);
          const float4 u = s[0], v = s[1];
          dxh[0] += u.x; dxh[1] += u.y; dxh[2] += u.z; dxh[3] += u.w;
          dxh[4] += v.x; dxh[5] += v.y; dxh[6] += v.z; dxh[7] += v.w;
        }
      }
      if (a.dxs) {
        const float4* s = reinterpret_cast<const float4*>(a.dxs + int64_t(t) * d + c0);
        const float4 u = s[0], v = s[1];
        dxh[0] += u.x; dxh[1] += u.y; dxh[2] += u.z; dxh[3] += u.w;
        dxh[4] += v.x; dxh[5] += v.y; dxh[6] += v.z; dxh[7] += v.w;
      }
      for (int e = 0; e < a.E; ++e) {
        const float de = a.dl[int64_t(t) * a.E + e];
        if (de == 0.f) continue;                 // uniform over the block
        float wv[8];
        unpack16(*reinterpret_cast<const uint4*>(a.wr + int64_t(e) * d + c0), wv,
                 (const uint16_t*)nullptr);
        const float f = r * de;
#pragma unroll
        for (int q = 0; q < 8; ++q) dxh[q] += f * wv[q];
      }
      float xv[8], gv[8];
      unpack16(*reinterpret_cast<const uint4*>(a.x + int64_t(t) * d + c0), xv,
               (const uint16_t*)nullptr);
      unpack16(*reinterpret_cast<const uint4*>(a.dout + int64_t(t) * d + c0), gv,
               (const uint16_t*)nullptr);
      const float cr = r * r * r / float(d) * dr;
      float o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        o[q] = (a.residual ? gv[q] : 0.f) + gam[q] * dxh[q] - cr * xv[q];
        gacc[q] += dxh[q] * xv[q];
      }
      *reinterpret_cast<uint4*>(a.dx + int64_t(t) * d + c0) = pack16(o, (const uint16_t*)nullptr);
    }
    if (a.dgamma_part) {
      float4* gp = reinterpret_cast<float4*>(a.dgamma_part + int64_t(blockIdx.x) * d + c0);
      gp[0] = make_float4(gacc[0], gacc[1], gacc[2], gacc[3]);
      gp[1] = make_float4(gacc[4], gacc[5], gacc[6], gacc[7]);
    }
  }
}

}  // namespace

int token_bwd_blocks(int64_t T) { return int((T + kTokB - 1) / kTokB); }

hipError_t launch_gather_t(const GatherTArgs& a, int max_width, int max_rows, int units,
                           hipStream_t s) {
  if (max_width <= 0 || max_rows <= 0 || units <= 0) return hipSuccess;
  const dim3 g(unsigned((max_width + 63) / 64), unsigned((max_rows + 63) / 64), unsigned(units));
  hipLaunchKernelGGL(k_gather_t, g, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_act_bwd(const ActBwdArgs& a, int max_units, int max_rows, int units,
                          hipStream_t s) {
  if (max_units <= 0 || max_rows <= 0 || units <= 0) return hipSuccess;
  const dim3 g(unsigned((max_units + 63) / 64), unsigned((max_rows + 63) / 64), unsigned(units));
  hipLaunchKernelGGL(k_act_bwd, g, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_plan_wgrad(const WgradPlanArgs& p, hipStream_t s) {
  if ((p.offsets ? p.E : 1) > kWgPlanMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_plan_wgrad, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_reduce_part(const float* part, int64_t ldpart, int64_t rows,
                              const int32_t* row_expert, const int32_t* foff, int dense_nft,
                              float* dg_row, float* dr_row, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_reduce_part, dim3(unsigned((rows + 255) / 256)), dim3(256), 0, s, part,
                     ldpart, rows, row_expert, foff, dense_nft, dg_row, dr_row);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* in, int64_t n, int64_t ld, int64_t cols, float* out,
                         hipStream_t s) {
  if (cols <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_colsum, dim3(unsigned((cols + 255) / 256)), dim3(256), 0, s, in, n, ld, cols,
                     out);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const RouterBwdArgs& a, hipStream_t s) {
  if (a.Tpad <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_router_bwd, dim3(unsigned((a.Tpad + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_token_bwd(const TokenBwdArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_token, dim3(unsigned(token_bwd_blocks(a.T))), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
