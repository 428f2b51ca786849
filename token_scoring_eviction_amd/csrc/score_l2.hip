// ManifoldKV scoring: Euclidean distance of every key to the centroid of the
// slice ("ManifoldKV: Training-Free KV Cache Compression via Euclidean Outlier
// Detection", abstract) or of its contiguous window (WindowedManifoldKV, same
// abstract).  The global score is the windowed score with one window.  The
// same kernels also give the cosine dissimilarity 1 - cos(k, mu) of the
// cosine-to-centroid baseline that abstract compares against, evaluated as
// ||k/||k|| - mu/||mu||||^2 / 2 so that nearly parallel keys keep their
// relative accuracy.
//
// Fused path (used whenever a window's tiles fit on the GPU at once): one
// launch of a persistent grid reads every key exactly once.
//   - A window (the whole slice for the global score) is a team of 256-token
//     tiles; the grid is a multiple of the team size, sized to the workgroups the
//     GPU holds at once, so a team's tiles run in the same round.  Each workgroup
//     keeps its tile in registers (16 rows x 8 channels per thread, 16-byte
//     coalesced loads).
//   - Each workgroup publishes its tile's fp32 column sums with coherent stores
//     and goes on without waiting for them.  An aggregator of the team (one per
//     32 tiles, rounded up to a power of two, each owning a block of channels;
//     the roles rotate over the team's workgroups) polls its channels of the
//     team's partial words until all are written -- they are set before the
//     launch to a pattern no sum can take -- adds them in a fixed order of tile
//     groups (deterministic), divides by the window length and publishes its
//     centroid words; the members poll those.
//   - Every workgroup then scores its rows from registers.  Two tiles are in
//     flight per workgroup: every load of the next tile is issued before the
//     workgroup waits for the current tile's centroid, and the next tile's
//     partial is published right after the current tile is scored.
//   - Every wait is bounded.  One that runs past its limit (possible only when a
//     team's workgroups are not all resident, e.g. another kernel holds part of
//     the GPU) flags the team; a repair launch queued right after recomputes the
//     flagged teams' centroids and scores from the keys, with the same bits, and
//     returns at once when nothing is flagged.  So the launch needs no
//     co-residency guarantee and is an ordinary launch.
//
// Fallback path, three launches on the caller's stream:
//   1. centroid_partial: column sums of bf16 keys over fixed 256-token chunks
//      (coalesced 16-byte loads, fp32 accumulation, one LDS reduction);
//   2. centroid_final: per window, the chunk partials added in chunk order
//      (deterministic, no float atomics) and divided by the window's length;
//   3. l2_distance: 16 lanes per key row, each lane 8 channels, a 16-lane
//      butterfly for the squared norm, fp32 sqrt.
#include <type_traits>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kChunk = 256;   // tokens per centroid partial
constexpr int kThreads = 256;

constexpr int kMetricL2 = KVC_METRIC_L2;
constexpr int kMetricCosine = KVC_METRIC_COSINE;

struct WinGeom {
    int64_t G, S, W, nwin, nchunk;  // nchunk: chunks per window
    int metric;                     // kvc_metric
};

__global__ __launch_bounds__(kThreads) void centroid_partial(const uint16_t *__restrict__ K,
                                                             WinGeom geo,
                                                             float *__restrict__ partial) {
    // one block per (slice, window, chunk)
    const int64_t item = blockIdx.x;
    const int64_t c = item % geo.nchunk;
    const int64_t gw = item / geo.nchunk;
    const int64_t w = gw % geo.nwin;
    const int64_t g = gw / geo.nwin;
    const int64_t w0 = w * geo.W;
    const int64_t w1 = min(w0 + geo.W, geo.S);
    const int64_t t0 = w0 + c * kChunk;
    const int64_t t1 = min(t0 + kChunk, w1);

    const int lane16 = threadIdx.x & 15;  // channel group: channels lane16*8 .. +8
    const int row = threadIdx.x >> 4;     // 0..15
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint4 *base = reinterpret_cast<const uint4 *>(K + (g * geo.S) * kHeadDim) + lane16;
    for (int64_t t = t0 + row; t < t1; t += 16) {
        uint4 v = base[t * (kHeadDim / 8)];
        acc[0] += bf16_lo(v.x);
        acc[1] += bf16_hi(v.x);
        acc[2] += bf16_lo(v.y);
        acc[3] += bf16_hi(v.y);
        acc[4] += bf16_lo(v.z);
        acc[5] += bf16_hi(v.z);
        acc[6] += bf16_lo(v.w);
        acc[7] += bf16_hi(v.w);
    }
    __shared__ float red[16][kHeadDim + 4];
#pragma unroll
    for (int j = 0; j < 8; ++j) red[row][lane16 * 8 + j] = acc[j];
    __syncthreads();
    if (threadIdx.x < kHeadDim) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) s += red[r][threadIdx.x];
        partial[item * kHeadDim + threadIdx.x] = s;
    }
}

__global__ __launch_bounds__(kHeadDim) void centroid_final(const float *__restrict__ partial,
                                                           WinGeom geo, float *__restrict__ mu,
                                                           float *__restrict__ mu_user,
                                                           uint32_t *__restrict__ status) {
    const int64_t gw = blockIdx.x;  // (slice, window)
    if (gw == 0 && threadIdx.x == 0) *status = 0u;  // this path has no wait that can expire
    const int64_t w = gw % geo.nwin;
    const int64_t w0 = w * geo.W;
    const int64_t len = min(w0 + geo.W, geo.S) - w0;
    const float *p = partial + gw * geo.nchunk * kHeadDim + threadIdx.x;
    float s = 0.f;
    for (int64_t c = 0; c < geo.nchunk; ++c) s += p[c * kHeadDim];
    const float m = s / static_cast<float>(len);
    mu[gw * kHeadDim + threadIdx.x] = m;
    if (mu_user) mu_user[gw * kHeadDim + threadIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void l2_distance(const uint16_t *__restrict__ K,
                                                        const float *__restrict__ mu, WinGeom geo,
                                                        float *__restrict__ scores) {
    const int64_t tok = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + (threadIdx.x >> 4);
    const int lane16 = threadIdx.x & 15;
    const bool valid = tok < geo.G * geo.S;
    float part = 0.f;
    if (valid) {
        const int64_t g = tok / geo.S;
        const int64_t t = tok - g * geo.S;
        const int64_t w = t / geo.W;
        const uint4 v = reinterpret_cast<const uint4 *>(K + tok * kHeadDim)[lane16];
        const float4 *m4 =
            reinterpret_cast<const float4 *>(mu + (g * geo.nwin + w) * kHeadDim + lane16 * 8);
        const float4 ma = m4[0], mb = m4[1];
        float d;
        d = bf16_lo(v.x) - ma.x; part += d * d;
        d = bf16_hi(v.x) - ma.y; part += d * d;
        d = bf16_lo(v.y) - ma.z; part += d * d;
        d = bf16_hi(v.y) - ma.w; part += d * d;
        d = bf16_lo(v.z) - mb.x; part += d * d;
        d = bf16_hi(v.z) - mb.y; part += d * d;
        d = bf16_lo(v.w) - mb.z; part += d * d;
        d = bf16_hi(v.w) - mb.w; part += d * d;
    }
    part += __shfl_xor(part, 8, 16);
    part += __shfl_xor(part, 4, 16);
    part += __shfl_xor(part, 2, 16);
    part += __shfl_xor(part, 1, 16);
    if (valid && lane16 == 0) scores[tok] = sqrtf(part);
}

// a*b - c*d with both products rounded on their own: never contracted into a
// fused multiply-add, so equal operands cancel exactly.
__device__ __forceinline__ float diff_of_products(float a, float b, float c, float d) {
#pragma clang fp contract(off)
    return a * b - c * d;
}

// 1 - cos(k_t, mu) as ||k_t/||k_t|| - mu/||mu||||^2 / 2; 1 where k_t or mu is
// zero.  16 lanes per key row.
__global__ __launch_bounds__(kThreads) void cosine_distance(const uint16_t *__restrict__ K,
                                                            const float *__restrict__ mu_dir,
                                                            WinGeom geo, float *__restrict__ scores) {
    const int64_t tok = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + (threadIdx.x >> 4);
    const int lane16 = threadIdx.x & 15;
    const bool valid = tok < geo.G * geo.S;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (valid) {
        const int64_t g = tok / geo.S;
        const int64_t t = tok - g * geo.S;
        const int64_t w = t / geo.W;
        const uint4 v = reinterpret_cast<const uint4 *>(K + tok * kHeadDim)[lane16];
        x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
        x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
        const float4 *m4 =
            reinterpret_cast<const float4 *>(mu_dir + (g * geo.nwin + w) * kHeadDim + lane16 * 8);
        const float4 ma = m4[0], mb = m4[1];
        m[0] = ma.x; m[1] = ma.y; m[2] = ma.z; m[3] = ma.w;
        m[4] = mb.x; m[5] = mb.y; m[6] = mb.z; m[7] = mb.w;
    }
    auto sum16 = [](float a) {
        a += __shfl_xor(a, 8, 16);
        a += __shfl_xor(a, 4, 16);
        a += __shfl_xor(a, 2, 16);
        a += __shfl_xor(a, 1, 16);
        return a;
    };
    // both norms with the same lane split and butterfly, so k = mu scores exactly 0
    float kk = 0.f, mm = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        kk += x[j] * x[j];
        mm += m[j] * m[j];
    }
    kk = sum16(kk);
    mm = sum16(mm);
    const float inv = kk > 0.f ? 1.f / sqrtf(kk) : 0.f;
    const float inv_m = mm > 0.f ? 1.f / sqrtf(mm) : 0.f;
    float e = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float d = diff_of_products(x[j], inv, m[j], inv_m);
        e += d * d;
    }
    e = sum16(e);
    if (valid && lane16 == 0) scores[tok] = (kk > 0.f && mm > 0.f) ? 0.5f * e : 1.f;
}

// ----------------------------------------------------------- fused path

#ifndef KVC_FUSE_ROWS
#define KVC_FUSE_ROWS 16
#endif
#ifndef KVC_FUSE_MINBLOCKS
#define KVC_FUSE_MINBLOCKS 3
#endif
#ifndef KVC_FUSE_THREADS
#define KVC_FUSE_THREADS 256
#endif
constexpr int kFuseThreads = KVC_FUSE_THREADS;                // a multiple of 64
constexpr int kRowGroups = kFuseThreads / 16;                 // 16 lanes per key row
constexpr int kFuseRows = KVC_FUSE_ROWS;                      // rows per thread (8 or 16)
constexpr int kFuseTile = kRowGroups * kFuseRows;             // tokens per tile
constexpr int kMemberGroups = kFuseThreads / 32;              // member groups per aggregator with
                                                              // all 32 channel groups of 4
// Tiles a gathering thread requests per poll: 4 for teams of up to kDeepTeam tiles,
// 8 above (fewer aggregators for large teams).  Scoring call, depth 4 vs 8 on one
// box: 256 x 16384 0.238-0.240 vs 0.244-0.249 ms, 256 x 32768 0.445 vs 0.458 ms,
// 256 x 65536 tied at 0.94 ms, 256 x 98304 1.63-1.64 vs 1.54-1.56 ms, 256 x 131072
// 2.50 vs 2.37-2.40 ms.  (Depth 2: 0.240 ms and 0.452 ms at the first two.)
constexpr int kGatherDepthSmall = 4, kGatherDepthLarge = 8;
constexpr int64_t kDeepTeam = 256;
constexpr int kMaxAggShift = 5;                               // at most 32 aggregators per team
static_assert(kFuseThreads % 64 == 0 && kMemberGroups <= kRowGroups, "fused tile shape");
static_assert(kRowGroups * (kHeadDim + 4) >= (kMemberGroups << kMaxAggShift) * ((kHeadDim >> kMaxAggShift) + 4),
              "the gather's group sums fit the reduction buffer");
// Polls of a centroid wait before it gives up and leaves the team to the repair
// launch: ~28 ms with the back-off, far above a wait among resident workgroups (~10 us).
constexpr uint32_t kSpinLimit = 1u << 16;
constexpr int64_t kRepairGrid = 256;  // workgroups of the repair launch
constexpr int64_t kEarlyMembers = 32;  // teams of this many tiles or more publish early

struct FuseGeom {
    int64_t G, S, W, nwin;
    int metric;       // kvc_metric
    int64_t members;  // tiles per window
    int64_t teams;    // G * nwin
    int64_t tiles;    // teams * members
    int agg_shift;    // log2 of the aggregators per team (each owns 128 >> agg_shift channels)
    int64_t per;      // members per member group: kMemberGroups << agg_shift groups per team
    int depth;        // tiles per gathering poll (kGatherDepthSmall or kGatherDepthLarge)
    uint32_t spin_limit;  // polls of a centroid wait before it gives up (kSpinLimit)
};

__device__ __forceinline__ void widen8(const uint4 &v, float *x) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// DPP lane exchanges inside a row of 16 lanes (gfx9 encodings): partner = lane ^ m
// for m = 15 (row_mirror), 7 (row_half_mirror), 3 and 1 (quad_perm).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppXor15 = 0x140, kDppXor7 = 0x141, kDppXor3 = 0x1b, kDppXor1 = 0xb1;

// One butterfly step over n values: pairs (v[j], v[j + n/2]); the lane whose
// `bit` is set keeps the upper half.  After it, v[0..n/2) hold the kept rows
// summed over the lane and its partner.
template <int kCtrl, int n>
__device__ __forceinline__ void fold_step(float *v, bool upper) {
#pragma unroll
    for (int j = 0; j < n / 2; ++j) {
        const float send = upper ? v[j] : v[j + n / 2];
        const float keep = upper ? v[j + n / 2] : v[j];
        v[j] = keep + dpp_f<kCtrl>(send);
    }
}

// Transpose-reduce across the 16 lanes of a row group: on entry lane i holds
// n per-row partials v[0..n); on exit v[0] holds the 16-lane total of row
// i (n = 16) or of row i >> 1 (n = 8; lanes i and i ^ 1 hold the same total).
template <int n>
__device__ __forceinline__ void row_transpose_reduce(float *v, int lane16) {
    if (n == 16) {
        fold_step<kDppXor15, 16>(v, lane16 & 8);
        fold_step<kDppXor7, 8>(v, lane16 & 4);
        fold_step<kDppXor3, 4>(v, lane16 & 2);
        fold_step<kDppXor1, 2>(v, lane16 & 1);
    } else {
        fold_step<kDppXor15, 8>(v, lane16 & 8);
        fold_step<kDppXor7, 4>(v, lane16 & 4);
        fold_step<kDppXor3, 2>(v, lane16 & 2);
        v[0] += dpp_f<kDppXor1>(v[0]);
    }
}

// Lane r's value in every lane of its row group of 16 (a swizzle in bitmask mode:
// lane' = (lane & 0x10) | r within each 32 lanes).
template <int r>
__device__ __forceinline__ float row_bcast(float a) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(a), 0x10 | (r << 5)));
}

// f(integral_constant<int, r>) for r = R .. N-1, in order.
template <int R, int N, class F>
__device__ __forceinline__ void for_rows(F &&f) {
    if constexpr (R < N) {
        f(std::integral_constant<int, R>());
        for_rows<R + 1, N>(f);
    }
}

// Sum over the 16 lanes of a row group, the same bits in every lane (each
// butterfly step adds a commuted pair).
__device__ __forceinline__ float sum16(float a) {
    a += dpp_f<kDppXor15>(a);
    a += dpp_f<kDppXor7>(a);
    a += dpp_f<kDppXor3>(a);
    a += dpp_f<kDppXor1>(a);
    return a;
}

// Per-lane arithmetic of a key row (its 128 channels spread over the 16 lanes of a
// row group, 8 per lane), shared by the scoring kernel and its repair launch so that
// both give the same bits.  lane_d2: the lane's part of ||k - mu||^2.  row_cos: the
// row's cosine score ||k/||k|| - mu/||mu||||^2 / 2 (1 where k or mu is zero) in every
// lane of the row group, with ||mu||^2 (mm) formed by the same lane split and
// butterfly as each key's ||k||^2, so that a key equal to the centroid scores 0.
__device__ __forceinline__ float lane_d2(const uint4 &w, const float *m) {
    float x[8];
    widen8(w, x);
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float d = x[j] - m[j];
        acc += d * d;
    }
    return acc;
}
// The lane's part of ||k||^2 and, given the row's 1 / ||k||, of ||k/||k|| - mu/||mu||||^2.
__device__ __forceinline__ float lane_kk(const uint4 &w) {
    float x[8];
    widen8(w, x);
    float kk = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) kk += x[j] * x[j];
    return kk;
}
__device__ __forceinline__ float lane_e(const uint4 &w, float inv, const float *m, float inv_m) {
    float x[8];
    widen8(w, x);
    float e = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float d = diff_of_products(x[j], inv, m[j], inv_m);
        e += d * d;
    }
    return e;
}
__device__ __forceinline__ float inv_norm(float kk) { return kk > 0.f ? 1.f / sqrtf(kk) : 0.f; }
__device__ __forceinline__ float cos_score(float kk, float e, float mm) {
    return (kk > 0.f && mm > 0.f) ? 0.5f * e : 1.f;
}
__device__ __forceinline__ float row_cos(const uint4 &w, const float *m, float mm, float inv_m) {
    const float kk = sum16(lane_kk(w));
    return cos_score(kk, sum16(lane_e(w, inv_norm(kk), m, inv_m)), mm);
}
// ||mu||^2 over the row group's lanes (channels lane16*8 .. +8 in m) and 1/||mu||.
__device__ __forceinline__ void centroid_norm(const float *m, float &mm, float &inv_m) {
    mm = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) mm += m[j] * m[j];
    mm = sum16(mm);
    inv_m = mm > 0.f ? 1.f / sqrtf(mm) : 0.f;
}

constexpr int kZeroThreads = 256;
// Words [0, n_zero) of p become 0, words [n_zero, n) become `value`.
__global__ __launch_bounds__(kZeroThreads) void fill_words(uint32_t *p, int64_t n_zero, int64_t n,
                                                           uint32_t value) {
    // 16-byte stores over whole groups of 4 words (p is 16-byte aligned), then the tail
    const int64_t n4 = n / 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (int64_t i = first; i < n4; i += stride) {
        const int64_t w = 4 * i;
        reinterpret_cast<uint4 *>(p)[i] = make_uint4(w < n_zero ? 0u : value, w + 1 < n_zero ? 0u : value,
                                                     w + 2 < n_zero ? 0u : value, w + 3 < n_zero ? 0u : value);
    }
    for (int64_t i = 4 * n4 + first; i < n; i += stride) p[i] = i < n_zero ? 0u : value;
}

// Exchange words (tile partials and published centroids) are 32-bit fp32 bit
// patterns, set to kPending before the launch.  kPending and kFailed are NaNs whose
// low 16 bits are set: widened bf16 keys have those bits clear, and sums and
// quotients of them either keep a NaN operand's payload or produce the default NaN,
// so no computed value equals either pattern.
constexpr uint32_t kPending = 0x7fffffffu;  // not written yet
constexpr uint32_t kFailed = 0xffffffffu;   // the team's gather gave up; the repair launch
                                            // recomputes the team

template <int kMetric, bool kEarly, int kGatherDepth>
__global__ __launch_bounds__(kFuseThreads, KVC_FUSE_MINBLOCKS) void l2_fused(const uint16_t *__restrict__ K, FuseGeom geo,
                                                         uint32_t *partial, uint32_t *mu_pub,
                                                         uint32_t *repair, uint32_t *status,
                                                         float *__restrict__ scores,
                                                         float *__restrict__ mu_user) {
    const int tid = threadIdx.x;
    const int lane16 = tid & 15;
    const int rowg = tid >> 4;  // 0 .. kRowGroups-1
    __shared__ float red[kRowGroups][kHeadDim + 4];
    __shared__ float mu_s[kHeadDim];

    struct TileGeo {
        int64_t team, member, g, w0, w1, t0;
    };
    auto geo_of = [&](int64_t tile) {
        TileGeo t;
        t.team = tile / geo.members;
        t.member = tile - t.team * geo.members;
        t.g = t.team / geo.nwin;
        const int64_t w = t.team - t.g * geo.nwin;
        t.w0 = w * geo.W;
        t.w1 = min(t.w0 + geo.W, geo.S);
        t.t0 = t.w0 + t.member * kFuseTile + rowg;  // this thread's first row
        return t;
    };
    auto load_tile = [&](const TileGeo &t, uint4 *v) {
        const uint4 *base = reinterpret_cast<const uint4 *>(K + t.g * geo.S * kHeadDim) + lane16;
#pragma unroll
        for (int r = 0; r < kFuseRows; ++r) {
            const int64_t row = t.t0 + static_cast<int64_t>(kRowGroups) * r;
            // keys are read once (streaming loads)
            v[r] = row < t.w1 ? ld_stream(base + row * (kHeadDim / 8)) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    bool agg_ok = false;  // the last gather's outcome (its centroid is in mu_s)
    // A wait that ran past its limit marks its team for the repair launch that follows
    // this kernel on the stream, which recomputes the team's centroid and scores from
    // the keys (the tile's scores are NaN until then).
    auto flag_repair = [&](const TileGeo &t) {
        if (tid == 0) {
            __hip_atomic_store(repair + t.team, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            atomicOr(status, kStatusRepair);
        }
    };
    auto nap_for = [](int &nap) {
        // back-off: a team polls the same few lines; hammering them costs the data
        // loads bandwidth on those memory channels
        if (nap <= 1) __builtin_amdgcn_s_sleep(1);
        else if (nap <= 4) __builtin_amdgcn_s_sleep(4);
        else __builtin_amdgcn_s_sleep(16);
        nap = nap < 16 ? nap * 2 : 16;
    };
    // A team has A = 1 << agg_shift aggregators (one while the team has at most 32
    // tiles): members (team + a * members / A) mod members, a = 0 .. A-1, so the roles
    // rotate over the team's workgroups from round to round.  Returns a, or -1.
    auto agg_of = [&](const TileGeo &t) -> int {
        const int64_t d = (t.member - t.team % geo.members + geo.members) % geo.members;
        const int64_t step = geo.members >> geo.agg_shift;
        if (d % step != 0) return -1;
        const int64_t a = d / step;
        return a < (1 << geo.agg_shift) ? static_cast<int>(a) : -1;
    };
    // Aggregator a owns channels [a, a + 1) * 128 / A of the centroid.  It polls those
    // channels of the team's partials until every word is written and adds them in
    // tile order: the team's tiles fall into kMemberGroups * A member groups of `per`
    // consecutive tiles (per <= kGatherDepth, so each thread requests its whole group
    // in one poll), a group's tiles are added in order, then the groups in order.  It divides
    // by the window's length and publishes its channels.  The wait is bounded: past
    // the limit it publishes kFailed in its channels, flags the team for the repair
    // launch and returns false.  Its channels of the centroid are left in mu_s (all of
    // it when A = 1, for the aggregator's own scoring of the tile).
    auto gather_mu = [&](const TileGeo &t, int a) -> bool {
        const int sh = geo.agg_shift;
        const int chans = kHeadDim >> sh;      // this aggregator's channels
        const int stride = chans + 4;          // of a member group's row in red
        const int cg = tid & ((32 >> sh) - 1);  // channel group of 4
        const int mg = tid >> (5 - sh);         // member group, 0 .. kMemberGroups * A - 1
        const int64_t m0 = mg * geo.per, m1 = min(geo.members, m0 + geo.per);
        const uint64_t *p =
            reinterpret_cast<const uint64_t *>(partial + t.team * geo.members * kHeadDim + a * chans) + cg * 2;
        float sx = 0.f, sy = 0.f, sz = 0.f, sw = 0.f;
        bool failed = false;
        uint32_t spins = 0;
        // Polls members [m, m + n) until all their words are written, then adds them in
        // order.  Each poll loads only the words not yet seen written (a written
        // partial never changes).
        auto take = [&](int64_t m, auto n_const) {
            constexpr int n = decltype(n_const)::value;
            uint64_t x[n][2];
            uint32_t pending = (1u << (2 * n)) - 1u;
            int nap = 1;
            for (;;) {
#pragma unroll
                for (int u = 0; u < n; ++u)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        if (pending & (1u << (2 * u + c)))
                            x[u][c] = __hip_atomic_load(p + (m + u) * (kHeadDim / 2) + c, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                for (int u = 0; u < n; ++u)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        if (static_cast<uint32_t>(x[u][c]) != kPending &&
                            static_cast<uint32_t>(x[u][c] >> 32) != kPending)
                            pending &= ~(1u << (2 * u + c));
                if (!pending) break;
                if (++spins > geo.spin_limit) {
                    failed = true;
                    return;
                }
                nap_for(nap);
            }
#pragma unroll
            for (int u = 0; u < n; ++u) {
                sx += __uint_as_float(static_cast<uint32_t>(x[u][0]));
                sy += __uint_as_float(static_cast<uint32_t>(x[u][0] >> 32));
                sz += __uint_as_float(static_cast<uint32_t>(x[u][1]));
                sw += __uint_as_float(static_cast<uint32_t>(x[u][1] >> 32));
            }
        };
        // chunks of 8, 4, 2, 1 members: a group of 8 or of a power of two below 8 is
        // requested in one poll
        static_assert(kGatherDepth == 8 || kGatherDepth == 4, "gather depth");
        int64_t m = m0;
        if constexpr (kGatherDepth == 8) {
            for (; m + 8 <= m1 && !failed; m += 8) take(m, std::integral_constant<int, 8>());
            if (m + 4 <= m1 && !failed) { take(m, std::integral_constant<int, 4>()); m += 4; }
        } else {
            for (; m + 4 <= m1 && !failed; m += 4) take(m, std::integral_constant<int, 4>());
        }
        if (m + 2 <= m1 && !failed) { take(m, std::integral_constant<int, 2>()); m += 2; }
        if (m < m1 && !failed) take(m, std::integral_constant<int, 1>());
        float *rf = &red[0][0];
        rf[mg * stride + cg * 4 + 0] = sx;
        rf[mg * stride + cg * 4 + 1] = sy;
        rf[mg * stride + cg * 4 + 2] = sz;
        rf[mg * stride + cg * 4 + 3] = sw;
        const bool any_failed = __syncthreads_or(failed);
        if (tid < chans) {
            uint32_t w = kFailed;
            float mu = __int_as_float(0x7fc00000);
            if (!any_failed) {
                float sum = 0.f;
                for (int q = 0; q < (kMemberGroups << sh); ++q) sum += rf[q * stride + tid];
                mu = sum / static_cast<float>(t.w1 - t.w0);
                w = __float_as_uint(mu);
            }
            const int ch = a * chans + tid;
            if (mu_user) mu_user[t.team * kHeadDim + ch] = mu;
            __hip_atomic_store(mu_pub + t.team * kHeadDim + ch, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            mu_s[ch] = __uint_as_float(w);
        }
        if (any_failed) flag_repair(t);
        __syncthreads();  // red and mu_s
        return !any_failed;
    };
    // Column sums of the tile -> the tile's partial words (32-bit coherent stores,
    // nothing waited for).  A team's aggregator then gathers its channels of the
    // centroid, while it holds only this tile.
    // Cosine metric: the tile's ||k||^2 of row lane16 (its 16 rows by one
    // transpose-reduce) is formed before the tile's centroid arrives and carried with
    // the tile to its scoring.  With the small teams' order it is formed in publish, in
    // the shadow of the next centroid wait (windowed scoring call at 256 x 65536, W
    // 4096: 1.082 -> 0.993 ms).  In the early-publish order publish runs while two
    // tiles are held (formed there: 0.297 -> 0.307 ms, more spills), so it is formed at
    // the end of the iteration, when only the next tile is held (256 x 16384: 0.293 ->
    // 0.276 ms, 25 -> 8 registers spilled).
    constexpr bool kNorms = kMetric == kMetricCosine && kFuseRows == 16 && !kEarly;
    constexpr bool kNormsEnd = kMetric == kMetricCosine && kFuseRows == 16 && kEarly;
    float kk_pub = 0.f;
    auto publish = [&](int64_t tile, const TileGeo &t, const uint4 *v) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float part[kFuseRows];  // cosine: each row's lane part of ||k||^2 (lane_kk's sum)
#pragma unroll
        for (int r = 0; r < kFuseRows; ++r) {
            float x[8];
            widen8(v[r], x);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += x[j];
            if constexpr (kNorms) {
                float kk = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) kk += x[j] * x[j];
                part[r] = kk;
            }
        }
        if constexpr (kNorms) {
            row_transpose_reduce<kFuseRows>(part, lane16);
            kk_pub = part[0];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) red[rowg][lane16 * 8 + j] = acc[j];
        __syncthreads();
        if (tid < kHeadDim) {
            float sum = 0.f;
#pragma unroll
            for (int r = 0; r < kRowGroups; ++r) sum += red[r][tid];
            __hip_atomic_store(partial + tile * kHeadDim + tid, __float_as_uint(sum), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();  // red is reused
        if constexpr (!kEarly) {
            const int a = agg_of(t);
            if (a >= 0) agg_ok = gather_mu(t, a);
        }
    };
    // The other members, and every member when a team has several aggregators, poll
    // the published centroid (bounded like the gather).
    auto poll_mu = [&](const TileGeo &t) -> bool {
        uint32_t spins = 0;
        int nap = 1;
        for (;;) {
            bool ready = true;
            if (tid < kHeadDim) {
                const uint32_t w = __hip_atomic_load(mu_pub + t.team * kHeadDim + tid, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                ready = w != kPending;
                mu_s[tid] = __uint_as_float(w);
            }
            if (__syncthreads_and(ready)) break;
            if (++spins > geo.spin_limit) {
                flag_repair(t);
                return false;
            }
            nap_for(nap);
        }
        return !__syncthreads_or(tid < kHeadDim && __float_as_uint(mu_s[tid]) == kFailed);
    };
    auto fetch_mu = [&](const TileGeo &t) -> bool {
        return geo.agg_shift == 0 && agg_of(t) == 0 ? agg_ok : poll_mu(t);
    };

    // Scores tile `t` (held in v) once its team's centroid is published.  Without a
    // centroid (a wait that gave up: the team is flagged) the tile's scores are
    // written as quiet NaN, which the repair launch then overwrites.
    auto score_tile = [&](const TileGeo &t, const uint4 *v, bool ok, float kk_row) {
        const float nan = __int_as_float(0x7fc00000);
        float m[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) m[j] = mu_s[lane16 * 8 + j];
        if (kMetric == kMetricCosine && kFuseRows == 16) {
            // The 16 rows' ||k||^2 by one transpose-reduce (lane r holds row r's;
            // formed before the centroid wait and carried in kk_row), 1 / ||k||
            // formed once per row in its lane and broadcast to the row group, then
            // the 16 rows' ||k/||k|| - mu/||mu||||^2 by a second transpose-reduce.
            // The same pairings and per-row arithmetic as row_cos: the same bits.
            float mm, inv_m;
            centroid_norm(m, mm, inv_m);
            float part[kFuseRows];
            float kk = kk_row;
            if constexpr (!kNorms && !kNormsEnd) {
#pragma unroll
                for (int r = 0; r < kFuseRows; ++r) part[r] = lane_kk(v[r]);
                row_transpose_reduce<kFuseRows>(part, lane16);
                kk = part[0];
            }
            const float inv_mine = inv_norm(kk);
            for_rows<0, kFuseRows>([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                // widened again rather than kept from the first pass (128 more live
                // registers otherwise): the empty asm hides that the bits are the same
                uint4 w = v[r];
                asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
                part[r] = lane_e(w, row_bcast<r>(inv_mine), m, inv_m);
            });
            row_transpose_reduce<kFuseRows>(part, lane16);
            const int64_t row = t.t0 + static_cast<int64_t>(kRowGroups) * lane16;
            if (row < t.w1) scores[t.g * geo.S + row] = ok ? cos_score(kk, part[0], mm) : nan;
        } else if (kMetric == kMetricCosine) {
            float mm, inv_m;
            centroid_norm(m, mm, inv_m);
            float mine = 0.f;
#pragma unroll
            for (int r = 0; r < kFuseRows; ++r) {
                const float c = row_cos(v[r], m, mm, inv_m);
                if (lane16 == r) mine = c;
            }
            const int64_t row = t.t0 + static_cast<int64_t>(kRowGroups) * lane16;
            if (lane16 < kFuseRows && row < t.w1) scores[t.g * geo.S + row] = ok ? mine : nan;
        } else {
            // the 16 rows' lane parts reduced across the row group at once (DPP
            // transpose-reduce, the same pairing as a 16-lane butterfly per row)
            float d2[kFuseRows];
#pragma unroll
            for (int r = 0; r < kFuseRows; ++r) d2[r] = lane_d2(v[r], m);
            row_transpose_reduce<kFuseRows>(d2, lane16);
            const int r = kFuseRows == 16 ? lane16 : (lane16 >> 1);
            const int64_t row = t.t0 + static_cast<int64_t>(kRowGroups) * r;
            if ((kFuseRows == 16 || (lane16 & 1) == 0) && row < t.w1)
                scores[t.g * geo.S + row] = ok ? sqrtf(d2[0]) : nan;
        }
        __syncthreads();  // mu_s is rewritten by the next fetch
    };

    const int64_t step = gridDim.x;
    int64_t tile = blockIdx.x;
    // Two tiles per workgroup (the current one and the next).
    uint4 v[kFuseRows], vn[kFuseRows];
    if constexpr (kEarly) {
        // Large teams: a tile's partial is published as soon as its keys are in, before
        // the workgroup waits for the current tile's centroid, and the aggregator
        // gathers after scoring (holding one tile).  Rounds overlap: the next
        // centroid no longer waits for the current one to be scored first
        // (scoring call at 256 x 16384: 0.248 -> 0.239 ms; with 16-tile teams,
        // 256 x 65536 in 4096-token windows, 0.893 -> 0.934 ms, so smaller teams
        // keep the order below).
        float kk_cur = 0.f;  // the current tile's row norms (cosine)
        auto norms_of = [&](const uint4 *w) -> float {
            float part[kFuseRows];
#pragma unroll
            for (int r = 0; r < kFuseRows; ++r) part[r] = lane_kk(w[r]);
            row_transpose_reduce<kFuseRows>(part, lane16);
            return part[0];
        };
        if (tile < geo.tiles) {
            const TileGeo t = geo_of(tile);
            load_tile(t, v);
            publish(tile, t, v);
            kk_cur = kk_pub;
            if constexpr (kNormsEnd) kk_cur = norms_of(v);
            const int a = agg_of(t);
            if (a >= 0) agg_ok = gather_mu(t, a);
        }
        for (; tile < geo.tiles; tile += step) {
            const TileGeo t = geo_of(tile);
            const int64_t next = tile + step;
            TileGeo tn;
            if (next < geo.tiles) {
                tn = geo_of(next);
                load_tile(tn, vn);
                publish(next, tn, vn);
            }
            const bool ok = fetch_mu(t);
            score_tile(t, v, ok, kk_cur);
            if (next < geo.tiles) {
                const int a = agg_of(tn);
                if (a >= 0) agg_ok = gather_mu(tn, a);
            }
#pragma unroll
            for (int r = 0; r < kFuseRows; ++r) v[r] = vn[r];
            kk_cur = kk_pub;
            if constexpr (kNormsEnd)
                if (next < geo.tiles) kk_cur = norms_of(v);
        }
    } else {
        // While tile `tile` waits for its team's centroid and is scored, every load of
        // the next tile is already in flight; its partial is published right after
        // (the aggregator gathers in publish).  Requesting half of the next tile
        // before the wait and half after it: 0.273 vs 0.267 ms per scoring call at
        // 256 x 16384.
        float kk_cur = 0.f;  // the current tile's row norms (cosine)
        if (tile < geo.tiles) {
            const TileGeo t = geo_of(tile);
            load_tile(t, v);
            publish(tile, t, v);
            kk_cur = kk_pub;
        }
        for (; tile < geo.tiles; tile += step) {
            const TileGeo t = geo_of(tile);
            const int64_t next = tile + step;
            TileGeo tn;
            if (next < geo.tiles) {
                tn = geo_of(next);
                load_tile(tn, vn);
            }
            const bool ok = fetch_mu(t);
            score_tile(t, v, ok, kk_cur);
            if (next < geo.tiles) publish(next, tn, vn);
#pragma unroll
            for (int r = 0; r < kFuseRows; ++r) v[r] = vn[r];
            kk_cur = kk_pub;
        }
    }
}

// Repair launch, queued right after l2_fused on the same stream.  When no centroid
// wait of that launch ran past its limit (the status bit is clear) every workgroup
// returns at once.  Otherwise each flagged team's centroid is computed from its
// keys -- every member tile's column sums formed as l2_fused's publish forms them,
// added in its aggregator's order -- and every tile of the team is scored from its
// keys read again, with the scoring kernel's per-row arithmetic.  The results are
// the bits l2_fused produces when its waits succeed.  With this launch the fused
// path needs no co-residency guarantee: a team whose workgroups are not all
// resident at once only costs a second read of its keys.
template <int kMetric>
__global__ __launch_bounds__(kFuseThreads) void l2_repair(const uint16_t *__restrict__ K, FuseGeom geo,
                                                          const uint32_t *__restrict__ repair,
                                                          const uint32_t *__restrict__ status,
                                                          float *__restrict__ scores,
                                                          float *__restrict__ mu_user) {
    if ((*status & kStatusRepair) == 0u) return;
    const int tid = threadIdx.x;
    const int lane16 = tid & 15;
    const int rowg = tid >> 4;
    __shared__ float red[kRowGroups][kHeadDim + 4];
    __shared__ float mu_s[kHeadDim];
    for (int64_t team = blockIdx.x; team < geo.teams; team += gridDim.x) {
        if (repair[team] == 0u) continue;
        const int64_t g = team / geo.nwin;
        const int64_t w0 = (team - g * geo.nwin) * geo.W;
        const int64_t w1 = min(w0 + geo.W, geo.S);
        const uint4 *base = reinterpret_cast<const uint4 *>(K + g * geo.S * kHeadDim) + lane16;
        // the centroid: tile column sums (rows t0 + 16 r of the thread's row group,
        // then the 16 row groups in order), member groups of `per` tiles added in
        // order, then the groups in order
        float total = 0.f, group = 0.f;
        for (int64_t j = 0; j < geo.members; ++j) {
            const int64_t t0 = w0 + j * kFuseTile + rowg;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < kFuseRows; ++r) {
                const int64_t row = t0 + static_cast<int64_t>(kRowGroups) * r;
                const uint4 w = row < w1 ? ld_stream(base + row * (kHeadDim / 8)) : make_uint4(0u, 0u, 0u, 0u);
                float x[8];
                widen8(w, x);
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c] += x[c];
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) red[rowg][lane16 * 8 + c] = acc[c];
            __syncthreads();
            if (tid < kHeadDim) {
                float sum = 0.f;
#pragma unroll
                for (int r = 0; r < kRowGroups; ++r) sum += red[r][tid];
                group += sum;
                if ((j + 1) % geo.per == 0 || j + 1 == geo.members) {
                    total += group;
                    group = 0.f;
                }
            }
            __syncthreads();  // red is reused
        }
        if (tid < kHeadDim) {
            const float mu = total / static_cast<float>(w1 - w0);
            mu_s[tid] = mu;
            if (mu_user) mu_user[team * kHeadDim + tid] = mu;
        }
        __syncthreads();
        float m[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) m[c] = mu_s[lane16 * 8 + c];
        float mm = 0.f, inv_m = 0.f;
        if (kMetric == kMetricCosine) centroid_norm(m, mm, inv_m);
        // every tile of the team: lane r of a row group keeps row r's score; a row's
        // lane parts are added by a 16-lane butterfly, the pairing of the scoring
        // kernel's transpose-reduce
        for (int64_t j = 0; j < geo.members; ++j) {
            const int64_t t0 = w0 + j * kFuseTile + rowg;
            float mine = 0.f;
#pragma unroll
            for (int r = 0; r < kFuseRows; ++r) {
                const int64_t row = t0 + static_cast<int64_t>(kRowGroups) * r;
                const uint4 w = row < w1 ? ld_stream(base + row * (kHeadDim / 8)) : make_uint4(0u, 0u, 0u, 0u);
                const float c = kMetric == kMetricCosine ? row_cos(w, m, mm, inv_m) : sqrtf(sum16(lane_d2(w, m)));
                if (lane16 == r) mine = c;
            }
            const int64_t row = t0 + static_cast<int64_t>(kRowGroups) * lane16;
            if (lane16 < kFuseRows && row < w1) scores[g * geo.S + row] = mine;
        }
        __syncthreads();  // mu_s is rewritten for the next team
    }
}

FuseGeom make_fuse_geom(int64_t G, int64_t S, int64_t W, int metric = kMetricL2) {
    FuseGeom f;
    f.metric = metric;
    f.G = G;
    f.S = S;
    f.W = W < S ? W : S;
    f.nwin = (S + f.W - 1) / f.W;
    f.members = (f.W + kFuseTile - 1) / kFuseTile;
    f.teams = G * f.nwin;
    f.tiles = f.teams * f.members;
    // one aggregator per kMemberGroups * depth tiles of a team, rounded up to a power
    // of two: each gathering thread then polls at most `depth` tiles, in one request
    // (a 64-tile team has 2 aggregators, a 512-tile team 8)
    f.depth = f.members > kDeepTeam ? kGatherDepthLarge : kGatherDepthSmall;
    int sh = 0;
    while (sh < kMaxAggShift && f.members > (static_cast<int64_t>(kMemberGroups * f.depth) << sh)) ++sh;
    f.agg_shift = sh;
    f.per = (f.members + (kMemberGroups << sh) - 1) / (kMemberGroups << sh);
    f.spin_limit = kSpinLimit;
    return f;
}

// Status header, published centroid words, then the tile partials: one contiguous
// range that a single launch prepares.
template <class Ws>
void fused_ws_layout(Ws &ws, const FuseGeom &f) {
    ws.template take<uint32_t>(kStatusBytes / 4);                          // status header
    ws.template take<uint32_t>(static_cast<size_t>(f.teams));              // repair flags
    ws.template take<uint32_t>(static_cast<size_t>(f.teams) * kHeadDim);   // published centroids
    ws.template take<uint32_t>(static_cast<size_t>(f.tiles) * kHeadDim);   // tile partials
}

// Co-resident workgroups of a fused-kernel instance on the current device (0 if unknown).
int64_t fused_capacity(const void *kernel) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kFuseThreads, 0) != hipSuccess)
        return 0;
    return static_cast<int64_t>(cus) * per_cu;
}

WinGeom make_geom(int64_t G, int64_t S, int64_t W, int metric = kMetricL2) {
    WinGeom geo;
    geo.metric = metric;
    geo.G = G;
    geo.S = S;
    geo.W = W < S ? W : S;
    geo.nwin = (S + geo.W - 1) / geo.W;
    geo.nchunk = (geo.W + kChunk - 1) / kChunk;
    return geo;
}

template <class Ws>
void score_ws_layout(Ws &ws, const WinGeom &geo) {
    ws.template take<uint32_t>(kStatusBytes / 4);  // status header
    ws.template take<float>(static_cast<size_t>(geo.G * geo.nwin * geo.nchunk) * kHeadDim);
    ws.template take<float>(static_cast<size_t>(geo.G * geo.nwin) * kHeadDim);
}

size_t score_bytes(int64_t G, int64_t S, int64_t W) {
    WsSizer a, b;
    score_ws_layout(a, make_geom(G, S, W));
    fused_ws_layout(b, make_fuse_geom(G, S, W));
    return a.bytes() > b.bytes() ? a.bytes() : b.bytes();
}

// Caches smaller than this take the three-launch path (its second read of K comes
// from the caches, and it has no team exchange to wait for).  Measured on MI355X,
// scoring call three-launch vs single-read: 8 MB of keys 16.6 vs 17.4 us, 17 MB 28.3
// vs 17.1, 67 MB 42.1 vs 24.4, 134 MB 64.0 vs 39.7, 268 MB 112.0 vs 67.9, 1 GB 449.9
// vs 240.9 us.
constexpr int64_t kSmallCacheBytes = 12ll << 20;

// The option KVC_OPTION_SCORE_PATH overrides the choice (1: the single-read kernel,
// 2: the three-launch path), so that tests and measurements can compare both.
// Returns true for the three-launch path.
bool take_unfused(int64_t G, int64_t S) {
    const int64_t path = options().score_path.load(std::memory_order_relaxed);
    if (path == 1) return false;
    if (path == 2) return true;
    return G * S * kHeadDim * 2 < kSmallCacheBytes;
}

kvc_status score_windowed_impl(const uint16_t *K, int64_t G, int64_t S, int32_t D, int64_t W,
                               int metric, float *scores, float *centroids, void *ws,
                               size_t ws_bytes, hipStream_t stream) {
    if (G < 0 || S < 1 || W < 1 || D <= 0) return KVC_ERR_INVALID_ARGUMENT;
    if (metric != kMetricL2 && metric != kMetricCosine) return KVC_ERR_INVALID_ARGUMENT;
    if (D != kHeadDim) return KVC_ERR_UNSUPPORTED;
    if (S > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    if (G == 0) return KVC_OK;
    if (!K || !scores || !ws) return KVC_ERR_INVALID_ARGUMENT;
    if (!aligned(K, 16) || !aligned(scores, 4) || !aligned(ws, kWsAlign) ||
        (centroids && !aligned(centroids, 4)))
        return KVC_ERR_INVALID_ARGUMENT;
    if (ws_bytes < score_bytes(G, S, W)) return KVC_ERR_WORKSPACE_TOO_SMALL;

    const FuseGeom f = make_fuse_geom(G, S, W, metric);
    // occupancy of the single-read kernel (both loop orders compile to the same budget)
    const void *fused = metric == kMetricCosine
                            ? reinterpret_cast<const void *>(&l2_fused<kMetricCosine, false, kGatherDepthSmall>)
                            : reinterpret_cast<const void *>(&l2_fused<kMetricL2, false, kGatherDepthSmall>);
    static std::atomic<int64_t> capacity_by_dev[2][64];  // capacity + 1; 0: not queried yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return KVC_ERR_HIP;
    int64_t cap1 = capacity_by_dev[metric][dev].load(std::memory_order_relaxed);
    if (cap1 == 0) {
        cap1 = fused_capacity(fused) + 1;
        capacity_by_dev[metric][dev].store(cap1, std::memory_order_relaxed);
    }
    const int64_t capacity = cap1 - 1;
    if (capacity >= f.members && f.tiles <= INT32_MAX && !take_unfused(G, S)) {
        WsCursor cur(ws);
        uint32_t *status = cur.take<uint32_t>(kStatusBytes / 4);
        uint32_t *repair = cur.take<uint32_t>(static_cast<size_t>(f.teams));
        uint32_t *mu_pub = cur.take<uint32_t>(static_cast<size_t>(f.teams) * kHeadDim);
        uint32_t *partial = cur.take<uint32_t>(static_cast<size_t>(f.tiles) * kHeadDim);
        // the status word and the repair flags cleared, the centroid and partial words
        // set to kPending, in one launch (they are adjacent in the workspace; a kernel,
        // not a memset, so the sequence can be captured in a graph)
        const int64_t n_zero = (repair + f.teams) - status;
        const int64_t n_clear = (partial + f.tiles * kHeadDim) - status;
        const int64_t zb = (n_clear / 4 + kZeroThreads - 1) / kZeroThreads + 1;
        hipLaunchKernelGGL(fill_words, dim3(static_cast<unsigned>(zb < 2048 ? zb : 2048)), dim3(kZeroThreads), 0,
                           stream, status, n_zero, n_clear, kPending);
        FuseGeom fa = f;
        // KVC_OPTION_SCORE_SPIN_LIMIT shortens the waits, so that a test can force the
        // repair path from the host
        const int64_t lim = options().spin_limit.load(std::memory_order_relaxed);
        fa.spin_limit = lim >= 0 ? static_cast<uint32_t>(lim) : kSpinLimit;
        float *mu_user = centroids;
        int64_t grid = capacity / f.members * f.members;
        if (grid > f.tiles) grid = f.tiles;
        // Plain launches: no co-residency is needed (a team whose waits run long is
        // recomputed by the repair launch), and a cooperative launch costs ~16 us more
        // per call (scoring call at 256 x 16384: 0.264 vs 0.248 ms).
        const int64_t rgrid = f.teams < kRepairGrid ? f.teams : kRepairGrid;
        const bool early = f.members >= kEarlyMembers;
        // the teams' order (early publish or not) and gather depth pick the instance
        auto fused_kernel = [&](auto metric_c) -> decltype(&l2_fused<kMetricL2, false, kGatherDepthSmall>) {
            constexpr int kM = decltype(metric_c)::value;
            if (!early) return &l2_fused<kM, false, kGatherDepthSmall>;
            return f.depth == kGatherDepthLarge ? &l2_fused<kM, true, kGatherDepthLarge>
                                                : &l2_fused<kM, true, kGatherDepthSmall>;
        };
        if (metric == kMetricCosine) {
            hipLaunchKernelGGL(fused_kernel(std::integral_constant<int, kMetricCosine>()),
                               dim3(static_cast<unsigned>(grid)), dim3(kFuseThreads), 0, stream, K, fa, partial,
                               mu_pub, repair, status, scores, mu_user);
            hipLaunchKernelGGL(l2_repair<kMetricCosine>, dim3(static_cast<unsigned>(rgrid)), dim3(kFuseThreads), 0,
                               stream, K, fa, repair, status, scores, mu_user);
        } else {
            hipLaunchKernelGGL(fused_kernel(std::integral_constant<int, kMetricL2>()),
                               dim3(static_cast<unsigned>(grid)), dim3(kFuseThreads), 0, stream, K, fa, partial,
                               mu_pub, repair, status, scores, mu_user);
            hipLaunchKernelGGL(l2_repair<kMetricL2>, dim3(static_cast<unsigned>(rgrid)), dim3(kFuseThreads), 0,
                               stream, K, fa, repair, status, scores, mu_user);
        }
        return launch_status();
    }

    const WinGeom geo = make_geom(G, S, W, metric);
    WsCursor cur(ws);
    uint32_t *status = cur.take<uint32_t>(kStatusBytes / 4);
    float *partial = cur.take<float>(static_cast<size_t>(geo.G * geo.nwin * geo.nchunk) * kHeadDim);
    float *mu = cur.take<float>(static_cast<size_t>(geo.G * geo.nwin) * kHeadDim);

    const int64_t nitems = geo.G * geo.nwin * geo.nchunk;
    if (nitems > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(centroid_partial, dim3(static_cast<unsigned>(nitems)), dim3(kThreads), 0,
                       stream, K, geo, partial);
    hipLaunchKernelGGL(centroid_final, dim3(static_cast<unsigned>(geo.G * geo.nwin)),
                       dim3(kHeadDim), 0, stream, partial, geo, mu, centroids, status);
    const int64_t nblk = (geo.G * geo.S + (kThreads / 16) - 1) / (kThreads / 16);
    if (nblk > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    if (metric == kMetricCosine)
        hipLaunchKernelGGL(cosine_distance, dim3(static_cast<unsigned>(nblk)), dim3(kThreads), 0, stream,
                           K, mu, geo, scores);
    else
        hipLaunchKernelGGL(l2_distance, dim3(static_cast<unsigned>(nblk)), dim3(kThreads), 0, stream, K,
                           mu, geo, scores);
    return launch_status();
}

}  // namespace

size_t score_workspace_bytes(int64_t G, int64_t S, int64_t W) {
    if (G < 0 || S < 1 || W < 1) return 0;
    return score_bytes(G, S, W);
}

kvc_status score_centroid_impl(const uint16_t *K, int64_t G, int64_t S, int32_t D, int64_t W, int metric,
                               float *scores, float *centroids, void *ws, size_t ws_bytes,
                               hipStream_t stream) {
    return score_windowed_impl(K, G, S, D, W, metric, scores, centroids, ws, ws_bytes, stream);
}

}  // namespace kvc

extern "C" kvc_status kvc_score_l2(const uint16_t *K, int64_t G, int64_t S, int32_t D, float *scores,
                                   float *centroid, void *ws, size_t ws_bytes, hipStream_t stream) {
    return kvc::score_windowed_impl(K, G, S, D, S, KVC_METRIC_L2, scores, centroid, ws, ws_bytes,
                                    stream);
}

extern "C" kvc_status kvc_score_l2_windowed(const uint16_t *K, int64_t G, int64_t S, int32_t D,
                                            int64_t W, float *scores, float *centroids, void *ws,
                                            size_t ws_bytes, hipStream_t stream) {
    return kvc::score_windowed_impl(K, G, S, D, W, KVC_METRIC_L2, scores, centroids, ws, ws_bytes,
                                    stream);
}

extern "C" kvc_status kvc_score_centroid(const uint16_t *K, int64_t G, int64_t S, int32_t D, int64_t W,
                                         int32_t metric, float *scores, float *centroids, void *ws,
                                         size_t ws_bytes, hipStream_t stream) {
    return kvc::score_windowed_impl(K, G, S, D, W, metric, scores, centroids, ws, ws_bytes, stream);
}
