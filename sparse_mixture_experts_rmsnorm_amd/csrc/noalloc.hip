// Allocation-free dispatch for callers that cannot allocate device memory.
//
// moe_dispatch_noalloc is moe_dispatch (the histogram, prefix sum and stable
// permutation of the expert-capacity rule) with its workspace taken from a
// file-scope device array instead of a caller-supplied buffer.  Each GPU the
// library runs on holds its own copy of the array, MOE_NOALLOC_SCRATCH_BYTES
// bytes, until the process ends.  Its device address is looked up once per
// device, on the entry point's first call with that device current; host
// code uses only that address, never the array's name (which on the host is
// a stand-in, not a device address).
//
// Every call on one GPU shares that GPU's array.  The dispatch kernels write
// every scratch word they later read within the same call (per-chunk
// histograms, error counts, radix keys and scan partials), so nothing needs
// clearing between calls, but two calls that overlap on one GPU (different
// streams, no ordering between them) race on the array.
#include <mutex>

#include "common.h"
#include "internal.h"
#include "moe.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on first use.
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return moe::report_error(MOE_EHIP, "moe_dispatch_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return moe::report_error(MOE_EUNSUPPORTED, "moe_dispatch_noalloc: device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return moe::report_error(MOE_EHIP,
                               "moe_dispatch_noalloc: hipGetSymbolAddress of the scratch failed");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_dispatch_noalloc(const int32_t* ids, const float* w, const float* r,
                                    const void* x, int dtype, int64_t T, int64_t d, int64_t E,
                                    int k, int64_t capacity, int pad, int64_t rows_max,
                                    int32_t* counts, int32_t* offsets, int32_t* pos,
                                    int32_t* row_token, float* row_r, float* row_w,
                                    int32_t* row_expert, void* x_perm, moe_stats* stats,
                                    hipStream_t stream) {
  const size_t need = moe_dispatch_workspace_size(T, k, E);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "moe_dispatch_noalloc: T=%lld, k=%d, E=%lld needs %zu bytes of scratch, more than "
             "the %zu bytes of the static scratch (use moe_dispatch with a workspace)",
             (long long)T, k, (long long)E, need, kScratchBytes);
    return moe::report_error(MOE_EWORKSPACE, msg);
  }
  void* ws = nullptr;
  const int rc = current_scratch(&ws);
  if (rc != MOE_OK) return rc;
  // the same host checks and kernels as moe_dispatch, on the static scratch
  return moe_dispatch(ids, w, r, x, dtype, T, d, E, k, capacity, pad, rows_max, counts, offsets,
                      pos, row_token, row_r, row_w, row_expert, x_perm, stats, ws, kScratchBytes,
                      stream);
}
