// kvc_score_centroid_noalloc: the centroid score (kvc_score_centroid) for callers
// that cannot allocate device memory (code under stream capture, tight serving
// loops, harnesses that forbid allocation).  Its scratch is a file-scope device
// array of kNoallocScratchBytes; its address on the current device is looked up
// once per device with hipGetSymbolAddress and kept, and the same kernels as the
// workspace entry point receive that address as their workspace.  Every call on a
// device shares that device's array, which keeps the last call's contents (each
// call clears what must start at zero with a kernel before it is read), so calls
// that overlap on one device race.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr size_t kNoallocScratchBytes = static_cast<size_t>(KVC_NOALLOC_SCRATCH_BYTES);

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::atomic<void *> scratch_by_dev[64];

// Device address of `scratch` on the current device (host code never passes the
// array's name itself to a kernel: on the host it is a stand-in, not a device address).
kvc_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return KVC_ERR_HIP;
    void *p = scratch_by_dev[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVC_ERR_HIP;
        scratch_by_dev[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return KVC_OK;
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_score_centroid_noalloc(const uint16_t *K, int64_t G, int64_t S, int32_t D,
                                                 int64_t W, int32_t metric, float *scores,
                                                 float *centroids, hipStream_t stream) {
    using namespace kvc;
    if (G < 0 || S < 1 || W < 1 || D <= 0) return KVC_ERR_INVALID_ARGUMENT;
    if (metric != KVC_METRIC_L2 && metric != KVC_METRIC_COSINE) return KVC_ERR_INVALID_ARGUMENT;
    if (G == 0) return KVC_OK;
    if (score_workspace_bytes(G, S, W) > kNoallocScratchBytes) return KVC_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    const kvc_status st = scratch_address(&ws);
    if (st != KVC_OK) return st;
    return score_centroid_impl(K, G, S, D, W, metric, scores, centroids, ws, kNoallocScratchBytes, stream);
}
