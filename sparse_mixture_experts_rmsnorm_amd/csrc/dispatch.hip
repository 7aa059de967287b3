// Capacity rule + dispatch: histogram, prefix sum and a stable permutation of
// the (token, slot) assignments into expert-contiguous rows.
//
// The expert-capacity entry of the "Mixture of Experts (MoE)" glossary fixes
// the per-expert limit; overflow slots are dropped.  Within an expert the
// rows keep token order (the OmniMoE summary, 2.2, sorts tasks by token id
// inside each expert group), which also decides which slots overflow.  The
// permuted rows carry the RMSNorm statistic r and the gate (the CODA thread:
// the r-scale must travel with the dispatched tokens).
//
// Determinism without ordering atomics: the slot list is cut into chunks of
// kChunkTokens tokens.  Pass 1 counts per (chunk, expert) (LDS atomics, which
// only count), pass 2 turns the counts into per-(chunk, expert) bases and the
// expert offsets, pass 3 ranks every slot inside its chunk with wavefront
// ballots -- lanes holding the same expert id find each other bit by bit, a
// lane's rank is the popcount of its peers below it, and per-wave totals are
// combined in wave order -- so the permutation is a stable counting sort.
//
// Very large expert counts (the 2^20 atomic experts of OmniMoE) use the same
// ballot ranking as the scatter of a two-pass LSD radix sort of the slots by
// expert id; offsets then come from a lower-bound search of the sorted keys.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kChunkTokens = 256;   // dense path: tokens per chunk
constexpr int kThreads = 256;       // 4 waves
constexpr int kRadixChunk = 2048;   // radix path: slots per chunk
constexpr int kDenseMaxE = 2048;

// stats layout: [0] rows, [1] dropped, [2] max_load, [3] errors
__device__ __forceinline__ uint64_t match_peers(int key, bool ok, int nbits) {
  uint64_t peers = __ballot(ok);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = ok && ((key >> b) & 1);
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__global__ void k_fill_rows(int64_t rows_max, int32_t* row_token, float* row_r, float* row_w,
                            int32_t* row_expert) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < rows_max;
       i += int64_t(gridDim.x) * blockDim.x) {
    row_token[i] = -1;
    row_r[i] = 0.f;
    row_w[i] = 0.f;
    if (row_expert) row_expert[i] = -1;
  }
}

// ---------------------------------------------------------------- dense path

// Pass 1: per-chunk expert histogram.
__global__ void __launch_bounds__(kThreads) k_count(const int32_t* __restrict__ ids, int T, int k,
                                                    int E, int32_t* __restrict__ cc,
                                                    int32_t* __restrict__ cerr, int nchunks,
                                                    int64_t rows_max, int32_t* __restrict__ row_token,
                                                    float* __restrict__ row_r,
                                                    float* __restrict__ row_w,
                                                    int32_t* __restrict__ row_expert) {
  extern __shared__ int hist[];
  __shared__ int err_s;
  const int c = blockIdx.x;
  if (c >= nchunks) {
    // the remaining blocks reset the per-row metadata
    const int64_t nb = gridDim.x - nchunks;
    for (int64_t i = (c - nchunks) * int64_t(kThreads) + threadIdx.x; i < rows_max;
         i += nb * kThreads) {
      row_token[i] = -1;
      row_r[i] = 0.f;
      row_w[i] = 0.f;
      if (row_expert) row_expert[i] = -1;
    }
    return;
  }
  for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
  if (threadIdx.x == 0) err_s = 0;
  __syncthreads();
  const int t0 = c * kChunkTokens;
  const int n = min(kChunkTokens, T - t0) * k;
  int err = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int e = ids[int64_t(t0) * k + i];
    if (unsigned(e) < unsigned(E)) atomicAdd(&hist[e], 1);
    else ++err;
  }
  if (err) atomicAdd(&err_s, err);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) cc[int64_t(c) * E + e] = hist[e];
  if (threadIdx.x == 0) cerr[c] = err_s;
}

// Block-wide exclusive scan, one value per thread (blockDim a multiple of 64,
// at most 1024).  sh needs 33 ints.
__device__ long long block_exscan(long long v, long long* total, long long* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  long long incl = v;
#pragma unroll
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
  const long long res = sh[wid] + incl - v;
  *total = sh[32];
  __syncthreads();
  return res;
}

// Pass 2: chunk bases, expert counts, capacity, padded offsets, statistics.
__global__ void __launch_bounds__(1024) k_scan(int32_t* __restrict__ cc,
                                               const int32_t* __restrict__ cerr, int nchunks,
                                               int E, int cap, int pad,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ stats) {
  __shared__ long long sh[33];
  __shared__ int padded_s[kDenseMaxE];
  long long dropped = 0, errs = 0;
  int maxl = 0;
  // one wave per expert: the expert's column of chunk counts is scanned 64
  // chunks at a time (a shuffle scan per round), in place, to exclusive
  // per-chunk bases
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int e = wv; e < E; e += nw) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const int c = c0 + lane;
      const int v = c < nchunks ? cc[int64_t(c) * E + e] : 0;
      int inc = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
      }
      if (c < nchunks) cc[int64_t(c) * E + e] = run + inc - v;
      run += __shfl(inc, 63, 64);
    }
    if (lane == 0) {
      counts[e] = run;
      const int kept = min(run, cap);
      padded_s[e] = (kept + pad - 1) / pad * pad;
      dropped += run - kept;
      maxl = max(maxl, run);
    }
  }
  for (int c = threadIdx.x; c < nchunks; c += blockDim.x) errs += cerr[c];
  __syncthreads();
  // exclusive scan of padded_s: each thread owns a contiguous run
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int lo = min(E, int(threadIdx.x) * per), hi = min(E, lo + per);
  long long local = 0;
  for (int e = lo; e < hi; ++e) local += padded_s[e];
  long long total;
  long long base = block_exscan(local, &total, sh);
  for (int e = lo; e < hi; ++e) {
    offsets[e] = int(base);
    base += padded_s[e];
  }
  if (threadIdx.x == 0) offsets[E] = int(total);
  // statistics
  long long tot;
  block_exscan(dropped, &tot, sh);
  const long long all_dropped = tot;
  block_exscan(errs, &tot, sh);
  const long long all_errs = tot;
  // max via shuffles + LDS
  int m = maxl;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
  __shared__ int mx[16];
  if ((threadIdx.x & 63) == 0) mx[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0 && stats) {
    int mm = 0;
    for (int w = 0; w < int(blockDim.x >> 6); ++w) mm = max(mm, mx[w]);
    stats[0] = int(total);
    stats[1] = int(all_dropped);
    stats[2] = mm;
    stats[3] = int(all_errs);
  }
}

// Pass 3: stable rank inside the chunk, capacity test, row metadata.
__global__ void __launch_bounds__(kThreads) k_rank(
    const int32_t* __restrict__ ids, const float* __restrict__ w, const float* __restrict__ r,
    int T, int k, int E, int nbits, int cap, const int32_t* __restrict__ cc,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ pos,
    int32_t* __restrict__ row_token, float* __restrict__ row_r, float* __restrict__ row_w,
    int32_t* __restrict__ row_expert) {
  extern __shared__ int sm[];
  int* running = sm;          // [E]
  int* wtag = sm + E;         // [4][E]: (batch + 1) << 8 | count
  const int c = blockIdx.x;
  const int wid = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += kThreads) {
    running[e] = cc[int64_t(c) * E + e];
    wtag[e] = wtag[E + e] = wtag[2 * E + e] = wtag[3 * E + e] = 0;
  }
  __syncthreads();
  const int t0 = c * kChunkTokens;
  const int n = min(kChunkTokens, T - t0) * k;
  const int64_t base_flat = int64_t(t0) * k;
  for (int b = 0; b * kThreads < n; ++b) {
    const int i = b * kThreads + threadIdx.x;
    const bool valid = i < n;
    int e = valid ? ids[base_flat + i] : -1;
    if (unsigned(e) >= unsigned(E)) e = -1;
    const bool ok = e >= 0;
    const uint64_t peers = match_peers(e, ok, nbits);
    const int lr = rank_below(peers);
    const int tag = b + 1;
    if (ok && lr == 0) wtag[wid * E + e] = (tag << 8) | __popcll(peers);
    __syncthreads();
    if (valid) {
      const int64_t flat = base_flat + i;
      int p = -1;
      if (ok) {
        int rank = running[e] + lr;
        for (int w2 = 0; w2 < wid; ++w2) {
          const int v = wtag[w2 * E + e];
          if ((v >> 8) == tag) rank += v & 255;
        }
        if (rank < cap) {
          p = offsets[e] + rank;
          const int t = int(flat / k);
          row_token[p] = t;
          row_r[p] = r[t];
          row_w[p] = w[flat];
          if (row_expert) row_expert[p] = e;
        }
      }
      pos[flat] = p;
    }
    __syncthreads();
    if (ok && lr == 0) {
      bool last = true;
      for (int w2 = wid + 1; w2 < 4; ++w2)
        if ((wtag[w2 * E + e] >> 8) == tag) last = false;
      if (last) {
        int tot = 0;
        for (int w2 = 0; w2 <= wid; ++w2) {
          const int v = wtag[w2 * E + e];
          if ((v >> 8) == tag) tot += v & 255;
        }
        running[e] += tot;
      }
    }
    __syncthreads();
  }
}

// Passes 2 and 3 in one launch, for layers whose chunk counts are few
// (nch * E <= kFusedScanMax): every block reads the whole (chunk, expert)
// count table itself -- its chunk's bases, the expert totals, the capacity
// test and the padded offsets -- so no separate scan launch sits between the
// count and the rank.  Block 0 writes counts, offsets and the statistics.
// With GATHER (rows of 2 KB and more) the chunk is ranked by `workers`
// blocks, all of which compute the same ranks; worker 0 writes the slot
// metadata and each worker copies its share of the chunk's kept rows into
// x_perm (token row t to row p), so the gather runs in the same launch; the
// last chunk's workers also zero the padding rows.
constexpr int kFusedScanMax = 1 << 15;

template <bool GATHER, typename T>
__global__ void __launch_bounds__(kThreads) k_rank_fused(
    const int32_t* __restrict__ ids, const float* __restrict__ w, const float* __restrict__ r,
    int Tn, int k, int E, int nbits, int cap, int pad, int nch, int workers,
    const int32_t* __restrict__ cc, const int32_t* __restrict__ cerr,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ stats,
    int32_t* __restrict__ pos, int32_t* __restrict__ row_token, float* __restrict__ row_r,
    float* __restrict__ row_w, int32_t* __restrict__ row_expert, const T* __restrict__ x,
    int64_t d, T* __restrict__ x_perm) {
  extern __shared__ int sm[];
  int* running = sm;              // [E] slots of this expert in earlier chunks, then running
  int* wtag = sm + E;             // [4][E]: (batch + 1) << 8 | count
  int* offs = sm + 5 * E;         // [E + 1] padded expert offsets
  int* tot_s = sm + 6 * E + 1;    // [E] slots of this expert in all chunks
  int* slot_p = sm + 7 * E + 1;   // [chunk slots] row of each slot (GATHER)
  __shared__ long long sh[33];
  const int c = int(blockIdx.x) / workers, wk = int(blockIdx.x) - c * workers;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  for (int e = tid; e < E; e += kThreads) {
    running[e] = 0;
    tot_s[e] = 0;
    wtag[e] = wtag[E + e] = wtag[2 * E + e] = wtag[3 * E + e] = 0;
  }
  __syncthreads();
  // 1. per expert, the slots of the chunks before this one and of all chunks:
  //    G threads per expert, each summing every G-th chunk (integer sums, so
  //    the LDS atomics give the same totals in any order)
  {
    const int G = E >= kThreads ? 1 : kThreads / E;
    for (int idx = tid; idx < E * G; idx += kThreads) {
      const int e = idx % E, g = idx / E;
      int before = 0, all = 0;
      for (int c2 = g; c2 < nch; c2 += G) {
        const int v = cc[int64_t(c2) * E + e];
        all += v;
        before += c2 < c ? v : 0;
      }
      if (before) atomicAdd(&running[e], before);
      if (all) atomicAdd(&tot_s[e], all);
    }
  }
  __syncthreads();
  // 2. capacity and padded offsets (each thread owns a contiguous run of experts)
  const int per = (E + kThreads - 1) / kThreads;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  long long local = 0, dropped = 0;
  int maxl = 0;
  for (int e = lo; e < hi; ++e) {
    const int kept = min(tot_s[e], cap);
    local += (kept + pad - 1) / pad * pad;
    dropped += tot_s[e] - kept;
    maxl = max(maxl, tot_s[e]);
  }
  long long total;
  long long base = block_exscan(local, &total, sh);
  for (int e = lo; e < hi; ++e) {
    offs[e] = int(base);
    base += (min(tot_s[e], cap) + pad - 1) / pad * pad;
  }
  if (tid == 0) offs[E] = int(total);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += kThreads) {
      offsets[e] = offs[e];
      if (e < E) counts[e] = tot_s[e];
    }
    long long errs = 0;
    for (int c2 = tid; c2 < nch; c2 += kThreads) errs += cerr[c2];
    long long tot;
    block_exscan(dropped, &tot, sh);
    const long long all_dropped = tot;
    block_exscan(errs, &tot, sh);
    const long long all_errs = tot;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) maxl = max(maxl, __shfl_xor(maxl, o, 64));
    __shared__ int mx[kThreads / 64];
    if (lane == 0) mx[wid] = maxl;
    __syncthreads();
    if (tid == 0 && stats) {
      int mm = 0;
      for (int w2 = 0; w2 < kThreads / 64; ++w2) mm = max(mm, mx[w2]);
      stats[0] = int(total);
      stats[1] = int(all_dropped);
      stats[2] = mm;
      stats[3] = int(all_errs);
    }
  }
  // 3. stable rank inside the chunk (as k_rank), capacity test, row metadata
  const int t0 = c * kChunkTokens;
  const int n = min(kChunkTokens, Tn - t0) * k;
  const int64_t base_flat = int64_t(t0) * k;
  const bool meta = wk == 0;
  for (int b = 0; b * kThreads < n; ++b) {
    const int i = b * kThreads + tid;
    const bool valid = i < n;
    int e = valid ? ids[base_flat + i] : -1;
    if (unsigned(e) >= unsigned(E)) e = -1;
    const bool ok = e >= 0;
    const uint64_t peers = match_peers(e, ok, nbits);
    const int lr = rank_below(peers);
    const int tag = b + 1;
    if (ok && lr == 0) wtag[wid * E + e] = (tag << 8) | __popcll(peers);
    __syncthreads();
    if (valid) {
      const int64_t flat = base_flat + i;
      int p = -1;
      if (ok) {
        int rank = running[e] + lr;
        for (int w2 = 0; w2 < wid; ++w2) {
          const int v = wtag[w2 * E + e];
          if ((v >> 8) == tag) rank += v & 255;
        }
        if (rank < cap) {
          p = offs[e] + rank;
          if (meta) {
            const int t = int(flat / k);
            row_token[p] = t;
            row_r[p] = r[t];
            row_w[p] = w[flat];
            if (row_expert) row_expert[p] = e;
          }
        }
      }
      if (meta) pos[flat] = p;
      if (GATHER) slot_p[i] = p;
    }
    __syncthreads();
    if (ok && lr == 0) {
      bool last = true;
      for (int w2 = wid + 1; w2 < 4; ++w2)
        if ((wtag[w2 * E + e] >> 8) == tag) last = false;
      if (last) {
        int tot = 0;
        for (int w2 = 0; w2 <= wid; ++w2) {
          const int v = wtag[w2 * E + e];
          if ((v >> 8) == tag) tot += v & 255;
        }
        running[e] += tot;
      }
    }
    __syncthreads();
  }
  if constexpr (GATHER) {
    // 4. this worker's share of the chunk's slots: one row per wave at a time,
    //    each lane's loads issued before its stores
    const int64_t nvec = d / Vec16<T>::N;
    const u32x4* __restrict__ xs = reinterpret_cast<const u32x4*>(x);
    u32x4* __restrict__ xp = reinterpret_cast<u32x4*>(x_perm);
    auto copy_row = [&](int64_t src_row, int64_t dst_row) {
      for (int64_t v0 = 0; v0 < nvec; v0 += 64 * 8) {
        u32x4 buf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t v = v0 + u * 64 + lane;
          buf[u] = (v < nvec && src_row >= 0) ? xs[src_row * nvec + v] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t v = v0 + u * 64 + lane;
          if (v < nvec) xp[dst_row * nvec + v] = buf[u];
        }
      }
    };
    const int i0 = int(int64_t(n) * wk / workers), i1 = int(int64_t(n) * (wk + 1) / workers);
    for (int i = i0 + wid; i < i1; i += kThreads / 64) {
      const int p = slot_p[i];
      if (p >= 0) copy_row((base_flat + i) / k, p);
    }
    // padding rows of every expert, zeroed by the last chunk's workers
    if (c == nch - 1) {
      for (int e = wk; e < E; e += workers) {
        const int kept = min(tot_s[e], cap);
        for (int row = offs[e] + kept + wid; row < offs[e + 1]; row += kThreads / 64)
          copy_row(-1, row);
      }
    }
  }
}

// Row gather: x_perm[row] = x[row_token[row]] (zeros on padding rows).  A
// wave copies one row; each lane moves up to 8 16-byte chunks, all loads
// issued before the stores.
template <typename T>
__global__ void __launch_bounds__(kThreads) k_gather(const T* __restrict__ x, int64_t d,
                                                     const int32_t* __restrict__ rows_used,
                                                     const int32_t* __restrict__ row_token,
                                                     T* __restrict__ x_perm) {
  const int rows = *rows_used;
  const int64_t nvec = d / Vec16<T>::N;
  const u32x4* __restrict__ xs = reinterpret_cast<const u32x4*>(x);
  u32x4* __restrict__ xp = reinterpret_cast<u32x4*>(x_perm);
  const int lane = threadIdx.x & 63;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += gridDim.x * 4) {
    const int t = row_token[row];
    const u32x4* src = xs + int64_t(t < 0 ? 0 : t) * nvec;
    u32x4* dst = xp + int64_t(row) * nvec;
    for (int64_t v0 = 0; v0 < nvec; v0 += 64 * 8) {
      u32x4 buf[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        buf[u] = (v < nvec && t >= 0) ? src[v] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        if (v < nvec) dst[v] = buf[u];
      }
    }
  }
}

// ---------------------------------------------------------------- radix path

// Keys = expert id, or E for an invalid id (sorts last).
__global__ void k_radix_prep(const int32_t* __restrict__ ids, int64_t N, int E,
                             int32_t* __restrict__ keys) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < N;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int e = ids[i];
    keys[i] = unsigned(e) < unsigned(E) ? e : E;
  }
}

__global__ void __launch_bounds__(kThreads) k_radix_count(const int32_t* __restrict__ keys,
                                                          int64_t N, int shift, int bits,
                                                          int nch, int32_t* __restrict__ cc) {
  extern __shared__ int hist[];
  const int nb = 1 << bits;
  const int c = blockIdx.x;
  for (int b = threadIdx.x; b < nb; b += kThreads) hist[b] = 0;
  __syncthreads();
  const int64_t i0 = int64_t(c) * kRadixChunk;
  const int n = int(min<int64_t>(kRadixChunk, N - i0));
  for (int i = threadIdx.x; i < n; i += kThreads)
    atomicAdd(&hist[(keys[i0 + i] >> shift) & (nb - 1)], 1);
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += kThreads) cc[int64_t(b) * nch + c] = hist[b];
}

// Exclusive scan of n ints in place: block partial sums, a scan of the block
// sums, then each block scans its run and adds its prefix.
constexpr int kScanPerThread = 16;
constexpr int kScanBlock = 256 * kScanPerThread;

__global__ void __launch_bounds__(256) k_scan_partial(const int32_t* __restrict__ v, int64_t n,
                                                      int32_t* __restrict__ part) {
  __shared__ long long sh[33];
  const int64_t lo = int64_t(blockIdx.x) * kScanBlock + threadIdx.x * kScanPerThread;
  long long local = 0;
  for (int i = 0; i < kScanPerThread; ++i)
    if (lo + i < n) local += v[lo + i];
  long long total;
  block_exscan(local, &total, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = int(total);
}

__global__ void __launch_bounds__(1024) k_scan_top(int32_t* __restrict__ part, int nb) {
  __shared__ long long sh[33];
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int lo = min(nb, int(threadIdx.x) * per), hi = min(nb, lo + per);
  long long local = 0;
  for (int i = lo; i < hi; ++i) local += part[i];
  long long total;
  long long base = block_exscan(local, &total, sh);
  for (int i = lo; i < hi; ++i) {
    const int x = part[i];
    part[i] = int(base);
    base += x;
  }
}

__global__ void __launch_bounds__(256) k_scan_final(int32_t* __restrict__ v, int64_t n,
                                                    const int32_t* __restrict__ part) {
  __shared__ long long sh[33];
  const int64_t lo = int64_t(blockIdx.x) * kScanBlock + threadIdx.x * kScanPerThread;
  int x[kScanPerThread];
  long long local = 0;
#pragma unroll
  for (int i = 0; i < kScanPerThread; ++i) {
    x[i] = lo + i < n ? v[lo + i] : 0;
    local += x[i];
  }
  long long total;
  long long base = block_exscan(local, &total, sh) + part[blockIdx.x];
#pragma unroll
  for (int i = 0; i < kScanPerThread; ++i) {
    if (lo + i < n) v[lo + i] = int(base);
    base += x[i];
  }
}

__global__ void __launch_bounds__(kThreads) k_radix_scatter(
    const int32_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in, int64_t N,
    int shift, int bits, int nch, const int32_t* __restrict__ cc,
    int32_t* __restrict__ keys_out, int32_t* __restrict__ vals_out) {
  extern __shared__ int sm[];
  const int nb = 1 << bits;
  int* running = sm;
  int* wtag = sm + nb;
  const int c = blockIdx.x;
  const int wid = threadIdx.x >> 6;
  for (int b = threadIdx.x; b < nb; b += kThreads) {
    running[b] = cc[int64_t(b) * nch + c];
    wtag[b] = wtag[nb + b] = wtag[2 * nb + b] = wtag[3 * nb + b] = 0;
  }
  __syncthreads();
  const int64_t i0 = int64_t(c) * kRadixChunk;
  const int n = int(min<int64_t>(kRadixChunk, N - i0));
  for (int b = 0; b * kThreads < n; ++b) {
    const int i = b * kThreads + threadIdx.x;
    const bool ok = i < n;
    const int key = ok ? keys_in[i0 + i] : 0;
    const int dig = (key >> shift) & (nb - 1);
    const uint64_t peers = match_peers(dig, ok, bits);
    const int lr = rank_below(peers);
    const int tag = b + 1;
    if (ok && lr == 0) wtag[wid * nb + dig] = (tag << 8) | __popcll(peers);
    __syncthreads();
    if (ok) {
      int dst = running[dig] + lr;
      for (int w2 = 0; w2 < wid; ++w2) {
        const int v = wtag[w2 * nb + dig];
        if ((v >> 8) == tag) dst += v & 255;
      }
      keys_out[dst] = key;
      vals_out[dst] = vals_in ? vals_in[i0 + i] : int(i0 + i);
    }
    __syncthreads();
    if (ok && lr == 0) {
      bool last = true;
      for (int w2 = wid + 1; w2 < 4; ++w2)
        if ((wtag[w2 * nb + dig] >> 8) == tag) last = false;
      if (last) {
        int tot = 0;
        for (int w2 = 0; w2 <= wid; ++w2) {
          const int v = wtag[w2 * nb + dig];
          if ((v >> 8) == tag) tot += v & 255;
        }
        running[dig] += tot;
      }
    }
    __syncthreads();
  }
}

// offsets[e] = first sorted slot with key >= e, for every e in [0, E]:
// slot i fills the experts in (key[i-1], key[i]] (the gap before its key),
// slot N fills the tail; every e is written exactly once.
__global__ void k_radix_offsets(const int32_t* __restrict__ keys, int N, int E,
                                int32_t* __restrict__ offsets) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i <= N;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int prev = i == 0 ? -1 : min(keys[i - 1], E);
    const int cur = i == N ? E : min(keys[i], E);
    for (int e = prev + 1; e <= cur; ++e) offsets[e] = int(i);
  }
}

// counts[e] = offsets[e+1] - offsets[e]; statistics of the radix path.
__global__ void k_radix_counts(const int32_t* __restrict__ offsets, int N, int E,
                               int32_t* __restrict__ counts, int32_t* __restrict__ stats) {
  int mx = 0;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < E;
       e += int64_t(gridDim.x) * blockDim.x) {
    const int c = offsets[e + 1] - offsets[e];
    counts[e] = c;
    mx = max(mx, c);
  }
  if (stats) {
    // one atomic per workgroup: same-address atomics serialise in L2
    __shared__ int wmax[4];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      mx = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
      if (mx > 0) atomicMax(&stats[2], mx);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      const int rows = offsets[E];
      stats[0] = rows;
      stats[1] = 0;
      stats[3] = N - rows;
    }
  }
}

__global__ void k_zero_stat(int32_t* stats) {
  if (threadIdx.x == 0) stats[2] = 0;
}

__global__ void k_radix_rows(const int32_t* __restrict__ keys, const int32_t* __restrict__ vals,
                             int64_t N, int E, int k, const float* __restrict__ w,
                             const float* __restrict__ r, int32_t* __restrict__ pos,
                             int32_t* __restrict__ row_token, float* __restrict__ row_r,
                             float* __restrict__ row_w, int32_t* __restrict__ row_expert) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < N;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int key = keys[i];
    const int flat = vals[i];
    if (key >= E) {
      pos[flat] = -1;
      continue;
    }
    const int t = flat / k;
    pos[flat] = int(i);
    row_token[i] = t;
    row_r[i] = r[t];
    row_w[i] = w[flat];
    if (row_expert) row_expert[i] = key;
  }
}

void scan_inplace(int32_t* v, int64_t n, int32_t* part, hipStream_t s) {
  const int nb = int((n + kScanBlock - 1) / kScanBlock);
  hipLaunchKernelGGL(k_scan_partial, dim3(nb), dim3(256), 0, s, v, n, part);
  hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(1024), 0, s, part, nb);
  hipLaunchKernelGGL(k_scan_final, dim3(nb), dim3(256), 0, s, v, n, part);
}

int ceil_log2(int64_t v) {
  int b = 0;
  while ((int64_t(1) << b) < v) ++b;
  return b;
}

}  // namespace

size_t dispatch_ws_bytes(int64_t T, int k, int64_t E) {
  if (E <= kDenseMaxE) {
    const int64_t nch = (T + kChunkTokens - 1) / kChunkTokens;
    return size_t(nch * E + nch + 64) * sizeof(int32_t);
  }
  const int64_t N = T * k;
  const int64_t nch = (N + kRadixChunk - 1) / kRadixChunk;
  const int B = ceil_log2(E + 1);
  const int b1 = (B + 1) / 2;
  const int64_t nscan = (int64_t(1) << b1) * nch;
  return size_t(4 * N + nscan + nscan / kScanBlock + 64) * sizeof(int32_t);
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const int T = int(a.T), k = a.k, E = int(a.E);
  int32_t* stats = reinterpret_cast<int32_t*>(a.stats);
  const int64_t fill_blocks = std::min<int64_t>(1024, (a.rows_max + 255) / 256);
  bool gathered = false;   // the rank launch also wrote x_perm
  if (E <= kDenseMaxE) {
    const int nch = (T + kChunkTokens - 1) / kChunkTokens;
    int32_t* cc = reinterpret_cast<int32_t*>(a.ws);
    int32_t* cerr = cc + int64_t(nch) * E;
    if (nch + fill_blocks > 0)
      hipLaunchKernelGGL(k_count, dim3(unsigned(nch + fill_blocks)), dim3(kThreads),
                         E * sizeof(int), s, a.ids, T, k, E, cc, cerr, nch, a.rows_max,
                         a.row_token, a.row_r, a.row_w, a.row_expert);
    const int cap = int(std::min<int64_t>(a.cap, int64_t(1) << 30));
    const int nbits = ceil_log2(E);
    const int chunk_slots = std::min(kChunkTokens, std::max(T, 1)) * k;
    // the row gather joins the rank launch for rows of 2 KB and more; shorter
    // rows copy faster with the separate gather kernel's one row per wave
    // (measured: 1.5 KB rows 19.6 us against 26 us fused, 8 KB rows 22.9
    // against 30 us)
    const bool fuse_gather = a.x_perm && a.d * (a.dtype == 0 ? 4 : 2) >= 2048;
    const size_t smem_fused = size_t(7 * E + 1 + (fuse_gather ? chunk_slots : 0)) * sizeof(int);
    if (int64_t(nch) * E <= kFusedScanMax && smem_fused <= 60 * 1024) {
      // workers per chunk: about 1024 blocks in all (each repeats its chunk's
      // rank before copying its share of the rows)
      const int workers = fuse_gather ? std::max(1, std::min(64, 1024 / std::max(nch, 1))) : 1;
      const dim3 g(unsigned(std::max(nch, 1) * workers));
#define MOE_RANK_FUSED(G, TY)                                                                  \
  hipLaunchKernelGGL((k_rank_fused<G, TY>), g, dim3(kThreads), smem_fused, s, a.ids, a.w, a.r, T, \
                     k, E, nbits, cap, a.pad, nch, workers, cc, cerr, a.counts, a.offsets,     \
                     stats, a.pos, a.row_token, a.row_r, a.row_w, a.row_expert,               \
                     static_cast<const TY*>(a.x), a.d, static_cast<TY*>(a.x_perm))
      if (!fuse_gather) MOE_RANK_FUSED(false, uint16_t);
      else if (a.dtype == 0) MOE_RANK_FUSED(true, float);
      else MOE_RANK_FUSED(true, uint16_t);
#undef MOE_RANK_FUSED
      gathered = fuse_gather;
    } else {
      hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, cc, cerr, nch, E, cap, a.pad,
                         a.counts, a.offsets, stats);
      if (nch > 0)
        hipLaunchKernelGGL(k_rank, dim3(nch), dim3(kThreads), 5 * E * sizeof(int), s, a.ids,
                           a.w, a.r, T, k, E, nbits, cap, cc, a.offsets, a.pos, a.row_token,
                           a.row_r, a.row_w, a.row_expert);
    }
  } else {
    // two-pass LSD radix sort of the slots by expert id (keys < 2^B, E = sentinel)
    const int64_t N = int64_t(T) * k;
    const int nch = int((N + kRadixChunk - 1) / kRadixChunk);
    const int B = ceil_log2(int64_t(E) + 1);
    const int b1 = (B + 1) / 2, b2 = B - b1;
    int32_t* keys0 = reinterpret_cast<int32_t*>(a.ws);
    int32_t* vals0 = keys0 + N;
    int32_t* keys1 = vals0 + N;
    int32_t* vals1 = keys1 + N;
    int32_t* cc = vals1 + N;
    int32_t* part = cc + (int64_t(nch) << b1);
    if (fill_blocks > 0)
      hipLaunchKernelGGL(k_fill_rows, dim3(unsigned(fill_blocks)), dim3(256), 0, s, a.rows_max,
                         a.row_token, a.row_r, a.row_w, a.row_expert);
    if (N > 0) {
      const unsigned g = unsigned(std::min<int64_t>(4096, (N + 255) / 256));
      hipLaunchKernelGGL(k_radix_prep, dim3(g), dim3(256), 0, s, a.ids, N, E, keys1);
      // pass 1: low b1 bits, keys1 -> keys0 / vals0
      hipLaunchKernelGGL(k_radix_count, dim3(nch), dim3(kThreads), (1 << b1) * sizeof(int), s,
                         keys1, N, 0, b1, nch, cc);
      scan_inplace(cc, int64_t(nch) << b1, part, s);
      hipLaunchKernelGGL(k_radix_scatter, dim3(nch), dim3(kThreads), 5 * (1 << b1) * sizeof(int),
                         s, keys1, (const int32_t*)nullptr, N, 0, b1, nch, cc, keys0, vals0);
      // pass 2: high b2 bits, keys0 -> keys1 / vals1
      hipLaunchKernelGGL(k_radix_count, dim3(nch), dim3(kThreads), (1 << b2) * sizeof(int), s,
                         keys0, N, b1, b2, nch, cc);
      scan_inplace(cc, int64_t(nch) << b2, part, s);
      hipLaunchKernelGGL(k_radix_scatter, dim3(nch), dim3(kThreads), 5 * (1 << b2) * sizeof(int),
                         s, keys0, vals0, N, b1, b2, nch, cc, keys1, vals1);
    }
    if (stats) hipLaunchKernelGGL(k_zero_stat, dim3(1), dim3(64), 0, s, stats);
    hipLaunchKernelGGL(k_radix_offsets, dim3(unsigned(std::min<int64_t>(4096, (N + 1 + 255) / 256))),
                       dim3(256), 0, s, keys1, int(N), E, a.offsets);
    hipLaunchKernelGGL(k_radix_counts, dim3(unsigned(std::min<int64_t>(256, (E + 255) / 256))),
                       dim3(256), 0, s, a.offsets, int(N), E, a.counts, stats);
    if (N > 0) {
      const unsigned g = unsigned(std::min<int64_t>(4096, (N + 255) / 256));
      hipLaunchKernelGGL(k_radix_rows, dim3(g), dim3(256), 0, s, keys1, vals1, N, E, k, a.w,
                         a.r, a.pos, a.row_token, a.row_r, a.row_w, a.row_expert);
    }
  }
  if (a.x_perm && !gathered) {
    const unsigned g = unsigned(std::max<int64_t>(1, std::min<int64_t>(8192, (a.rows_max + 3) / 4)));
    if (a.dtype == 0)
      hipLaunchKernelGGL(k_gather<float>, dim3(g), dim3(kThreads), 0, s,
                         static_cast<const float*>(a.x), a.d, a.offsets + E, a.row_token,
                         static_cast<float*>(a.x_perm));
    else
      hipLaunchKernelGGL(k_gather<uint16_t>, dim3(g), dim3(kThreads), 0, s,
                         static_cast<const uint16_t*>(a.x), a.d, a.offsets + E, a.row_token,
                         static_cast<uint16_t*>(a.x_perm));
  }
  return hipGetLastError();
}

}  // namespace moe
