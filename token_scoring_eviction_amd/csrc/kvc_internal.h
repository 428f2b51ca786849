// Internal helpers shared by the libkvc HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "kvc.h"

namespace kvc {

constexpr int kHeadDim = 128;        // the only head dimension built
constexpr size_t kWsAlign = 256;     // sub-buffer alignment inside a workspace

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Carves consecutive aligned sub-buffers out of a caller-provided workspace.
struct WsCursor {
    char *base;
    size_t off = 0;
    explicit WsCursor(void *p) : base(static_cast<char *>(p)) {}
    template <class T>
    T *take(size_t count) {
        off = align_up(off, kWsAlign);
        T *p = reinterpret_cast<T *>(base + off);
        off += count * sizeof(T);
        return p;
    }
};

// Same layout arithmetic without a base pointer, for kvc_workspace_bytes.
struct WsSizer {
    size_t off = 0;
    template <class T>
    void take(size_t count) {
        off = align_up(off, kWsAlign);
        off += count * sizeof(T);
    }
    size_t bytes() const { return off; }
};

// Workspaces that report failures found by the kernels themselves (expired
// in-kernel waits, invalid device-side budgets) start with this header; its first
// word holds kStatus* bits, cleared by each call before its kernels run and read
// by kvc_workspace_status.
constexpr size_t kStatusBytes = 256;
constexpr uint32_t kStatusBadBudget = 2u;  // a per-slice budget outside its bounds
constexpr uint32_t kStatusRepair = 4u;     // a centroid wait ran past its limit; the call's
                                           // repair launch recomputed those teams (not a failure)

// Process-wide options set by kvc_set_option (tests and measurements choose a
// kernel path with them; the defaults select the production paths).
struct Options {
    std::atomic<int64_t> score_path{0};   // 0 automatic, 1 single-read kernel, 2 three launches
    std::atomic<int64_t> spin_limit{-1};  // polls of a centroid wait; -1: the built-in limit
    std::atomic<int64_t> gather_path{0};  // 0 wide gather launch, 1 in-workgroup copy
};
Options &options();

// Centroid scoring (kvc_score_centroid) with the caller's workspace of ws_bytes; and
// the workspace it needs (0 for invalid shapes).
kvc_status score_centroid_impl(const uint16_t *K, int64_t G, int64_t S, int32_t D, int64_t W, int metric,
                               float *scores, float *centroids, void *ws, size_t ws_bytes,
                               hipStream_t stream);
size_t score_workspace_bytes(int64_t G, int64_t S, int64_t W);

inline kvc_status launch_status() {
    return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// Per-device values cached by host code are atomics: host threads that call the
// library at once may both fill an entry, which is harmless (they compute the same
// value), and no access races.

// Lets `kernel` take up to 160 KB of dynamic LDS on the current device (the
// default cap is 64 KB); done once per device, `done` is the caller's per-kernel flag array.
inline kvc_status allow_large_lds(const void *kernel, std::atomic<bool> (&done)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return KVC_ERR_HIP;
    if (!done[dev].load(std::memory_order_acquire)) {
        if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
            return KVC_ERR_HIP;
        done[dev].store(true, std::memory_order_release);
    }
    return KVC_OK;
}

// Compute units of the current device (cached per device; 0 if it cannot be queried).
inline int device_cu_count() {
    static std::atomic<int> cus_by_dev[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int cus = cus_by_dev[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cus_by_dev[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// ------------------------------------------------------------ device helpers

// Exact bf16 -> fp32 widening of the two halves of a packed 32-bit word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Streaming 16-byte loads and stores (the non-temporal hint of the vector memory
// instructions) for data touched once: on MI355X a 1 GiB copy moves 5.9-6.1 TB/s with
// them and 5.2-5.4 TB/s without, a read-only stream 6.1-6.7 against 5.6-6.0 TB/s.
// Only where each instruction covers whole 128-byte lines (16 lanes x 16 bytes of a
// row): the lines are not kept, so an access pattern that takes a line in pieces over
// several instructions fetches it again (the projection kernel's key loads, 32 bytes
// of a row per instruction, went 7.4 -> 8.6 ms) and partial-line stores reach HBM
// unmerged.  Data read again soon (scores, partial sums) keeps plain accesses.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    const u32x4_nt t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st_stream(uint4 *p, const uint4 &v) {
    const u32x4_nt t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_nt *>(p));
}
__device__ __forceinline__ float4 ld_stream(const float4 *p) {
    const uint4 u = ld_stream(reinterpret_cast<const uint4 *>(p));
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}
__device__ __forceinline__ void st_stream(float4 *p, const float4 &v) {
    st_stream(reinterpret_cast<uint4 *>(p),
              make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)));
}

// Order-preserving map of an fp32 value to an unsigned key: a > b <=> key(a) > key(b).
// -0.0 is folded onto +0.0 so that the two compare equal, as in IEEE arithmetic.
// A NaN (inputs are finite, but a scoring wait that expired leaves NaN scores) maps
// to 0, below every other key (-inf maps to 0x007fffff), so it is never kept ahead
// of a number.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace kvc
