// ManifoldKV scoring: Euclidean distance of every key to the centroid of the
// slice ("ManifoldKV: Training-Free KV Cache Compression via Euclidean Outlier
// Detection", abstract) or of its contiguous window (WindowedManifoldKV, same
// abstract).  The global score is the windowed score with one window.
//
// Three launches on the caller's stream:
//   1. centroid_partial: column sums of bf16 keys over fixed 256-token chunks
//      (coalesced 16-byte loads, fp32 accumulation, one LDS reduction);
//   2. centroid_final: per window, the chunk partials added in chunk order
//      (deterministic, no float atomics) and divided by the window's length;
//   3. l2_distance: 16 lanes per key row, each lane 8 channels, a 16-lane
//      butterfly for the squared norm, fp32 sqrt.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kChunk = 256;   // tokens per centroid partial
constexpr int kThreads = 256;

struct WinGeom {
    int64_t G, S, W, nwin, nchunk;  // nchunk: chunks per window
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
                                                           float *__restrict__ mu_user) {
    const int64_t gw = blockIdx.x;  // (slice, window)
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

WinGeom make_geom(int64_t G, int64_t S, int64_t W) {
    WinGeom geo;
    geo.G = G;
    geo.S = S;
    geo.W = W < S ? W : S;
    geo.nwin = (S + geo.W - 1) / geo.W;
    geo.nchunk = (geo.W + kChunk - 1) / kChunk;
    return geo;
}

template <class Ws>
void score_ws_layout(Ws &ws, const WinGeom &geo) {
    ws.template take<float>(static_cast<size_t>(geo.G * geo.nwin * geo.nchunk) * kHeadDim);
    ws.template take<float>(static_cast<size_t>(geo.G * geo.nwin) * kHeadDim);
}

kvc_status score_windowed_impl(const uint16_t *K, int64_t G, int64_t S, int32_t D, int64_t W,
                               float *scores, float *centroids, void *ws, size_t ws_bytes,
                               hipStream_t stream) {
    if (G < 0 || S < 1 || W < 1 || D <= 0) return KVC_ERR_INVALID_ARGUMENT;
    if (D != kHeadDim) return KVC_ERR_UNSUPPORTED;
    if (S > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    if (G == 0) return KVC_OK;
    if (!K || !scores || !ws) return KVC_ERR_INVALID_ARGUMENT;
    if (!aligned(K, 16) || !aligned(scores, 4) || !aligned(ws, kWsAlign) ||
        (centroids && !aligned(centroids, 4)))
        return KVC_ERR_INVALID_ARGUMENT;
    const WinGeom geo = make_geom(G, S, W);
    WsSizer sz;
    score_ws_layout(sz, geo);
    if (ws_bytes < sz.bytes()) return KVC_ERR_WORKSPACE_TOO_SMALL;
    WsCursor cur(ws);
    float *partial = cur.take<float>(static_cast<size_t>(geo.G * geo.nwin * geo.nchunk) * kHeadDim);
    float *mu = cur.take<float>(static_cast<size_t>(geo.G * geo.nwin) * kHeadDim);

    const int64_t nitems = geo.G * geo.nwin * geo.nchunk;
    if (nitems > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(centroid_partial, dim3(static_cast<unsigned>(nitems)), dim3(kThreads), 0,
                       stream, K, geo, partial);
    hipLaunchKernelGGL(centroid_final, dim3(static_cast<unsigned>(geo.G * geo.nwin)),
                       dim3(kHeadDim), 0, stream, partial, geo, mu, centroids);
    const int64_t nblk = (geo.G * geo.S + (kThreads / 16) - 1) / (kThreads / 16);
    if (nblk > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(l2_distance, dim3(static_cast<unsigned>(nblk)), dim3(kThreads), 0, stream, K,
                       mu, geo, scores);
    return launch_status();
}

}  // namespace

size_t score_workspace_bytes(int64_t G, int64_t S, int64_t W) {
    if (G < 0 || S < 1 || W < 1) return 0;
    WsSizer sz;
    score_ws_layout(sz, make_geom(G, S, W));
    return sz.bytes();
}

}  // namespace kvc

extern "C" kvc_status kvc_score_l2(const uint16_t *K, int64_t G, int64_t S, int32_t D, float *scores,
                                   float *centroid, void *ws, size_t ws_bytes, hipStream_t stream) {
    return kvc::score_windowed_impl(K, G, S, D, S, scores, centroid, ws, ws_bytes, stream);
}

extern "C" kvc_status kvc_score_l2_windowed(const uint16_t *K, int64_t G, int64_t S, int32_t D,
                                            int64_t W, float *scores, float *centroids, void *ws,
                                            size_t ws_bytes, hipStream_t stream) {
    return kvc::score_windowed_impl(K, G, S, D, W, scores, centroids, ws, ws_bytes, stream);
}
