// RefineKV cluster summaries and risk scores ("RefineKV" project page:
// "Summarize" -- contiguous clusters with cached mean keys, mean values and
// metadata -- and "Select" with the Figure 2 risk formula
//   RC = 2 p_C Vmax [ (cosh d_C - 1) / Dn + tanh(d_C / 2) ],  Dn = sum_C' p_C' cosh d_C').
// The page names p_C (the cluster's approximate share of attention mass) and d_C
// (a bound on the deviation of its keys' logits from the representative's) without
// formulas; here
//   p_C = n_C exp(z_C) / sum_C' n_C' exp(z_C'),  z_C = q . mu_C / sqrt(D),
//   d_C = ||q|| radius_C / sqrt(D)  (Cauchy-Schwarz on q . (k - mu_C)),
//   Vmax = the largest value norm of the slice.
//
// cluster_summary_kernel: one wave per cluster, four 256-byte rows per 16-byte load
//   (16 lanes per row, 8 channels per lane), up to 16 (c <= 16) or 32 rows of K and V
//   in flight at once; per-lane sums in token order, the four row slots added in a
//   fixed order, 16-lane sums for the row norms; the first chunk's key rows stay in
//   registers for the radius pass, later ones are read again.
// risk_partial_kernel + risk_final_kernel: the slice's clusters are spread over
//   many workgroups (a single workgroup per slice left the mean-key stream
//   latency-bound).  The partial pass computes the logits z (16 lanes per cluster,
//   8 channels each) into the RC rows and, per chunk of clusters, the maxima and
//   the rescaled sums of the softmax and of the normaliser; the final pass merges
//   the chunk records in chunk order (deterministic) and turns each logit into RC.
//   The normaliser's terms are shifted by their largest exponent max_C (z_C + d_C),
//   so no cosh overflows fp32 however far apart a cluster's keys lie.
#include <math.h>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kSumWaves = 1;             // clusters per summary workgroup (one wave: 3.39 -> 3.15 ms for 32-key clusters at 256 x 131072)
constexpr int kRiskThreads = 256;        // both risk passes
constexpr int kMaxRiskQueries = 8;
constexpr int kRiskBatch = 2;            // clusters per 16-lane row loaded before any is used
constexpr int kRiskPerRow = 8;           // clusters per 16-lane row in a partial-pass workgroup
constexpr int kRiskChunk = 16 * kRiskPerRow;     // clusters per partial-pass workgroup
constexpr int kRiskFinalChunk = 2048;    // clusters per final-pass workgroup
constexpr int kPartStride = kMaxRiskQueries + 1;  // float4 records per (slice, chunk)

// Exchanges inside a row of 16 lanes (DPP, gfx9 encodings): partner = lane ^ m for
// m = 15 (row_mirror), 7 (row_half_mirror), 3 and 1 (quad_perm).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}
// Sum over a row of 16 lanes; every lane of the row gets the same bits.
__device__ __forceinline__ float sum16(float a) {
    a += dpp_f<0x140>(a);
    a += dpp_f<0x141>(a);
    a += dpp_f<0x1b>(a);
    a += dpp_f<0xb1>(a);
    return a;
}

__device__ __forceinline__ void widen8(const uint4 &v, float *x) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// One wave per cluster.  Lane (slot, l) = (lane / 16, lane % 16) holds channels
// 8l .. 8l + 7 of the rows t0 + slot, t0 + slot + 4, ...: one 16-byte load per lane
// covers four 256-byte rows.  NR loads of K and of V (4 NR rows) are in flight per
// chunk; the first chunk's key rows stay in registers for the radius pass (later
// chunks are read again).  Channel sums run over a lane's rows in token order and
// the four slots are then added in a fixed order ((0 + 1) + (2 + 3)); row norms
// are 16-lane sums.
template <int NR>
__global__ __launch_bounds__(64 * kSumWaves) void cluster_summary_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, int64_t G, int64_t S, int64_t c,
    int64_t nC, float *__restrict__ mu_k, float *__restrict__ mu_v, float *__restrict__ radius,
    float *__restrict__ vnorm) {
    const int64_t cl = static_cast<int64_t>(blockIdx.x) * kSumWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, slot = lane >> 4, l16 = lane & 15;
    if (cl >= G * nC) return;  // whole waves leave together
    const int64_t g = cl / nC, j = cl - g * nC;
    const int64_t t0 = j * c, t1 = min(t0 + c, S);
    const uint4 *kr = reinterpret_cast<const uint4 *>(K + (g * S) * kHeadDim) + l16;
    const uint4 *vr = reinterpret_cast<const uint4 *>(V + (g * S) * kHeadDim) + l16;
    float sk[8], sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
    float vmax2 = 0.f;
    uint4 kw[NR];
    for (int64_t base = t0; base < t1; base += 4 * NR) {
        uint4 kc[NR], vc[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t t = base + 4 * i + slot;
            kc[i] = vc[i] = make_uint4(0u, 0u, 0u, 0u);
            if (t < t1) {  // rows past the cluster are not read
                // whole rows per 16 lanes: V is read once (streaming), and so are the
                // keys of the first chunk (later chunks are read again for the radius)
                kc[i] = base == t0 ? ld_stream(kr + t * (kHeadDim / 8)) : kr[t * (kHeadDim / 8)];
                vc[i] = ld_stream(vr + t * (kHeadDim / 8));
            }
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            // rows past the cluster are zeros: they add nothing, and their norm is 0
            float x[8], y[8];
            widen8(kc[i], x);
            widen8(vc[i], y);
            float n2 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sk[e] += x[e];
                sv[e] += y[e];
                n2 += y[e] * y[e];
            }
            vmax2 = fmaxf(vmax2, sum16(n2));
        }
        if (base == t0) {
#pragma unroll
            for (int i = 0; i < NR; ++i) kw[i] = kc[i];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        sk[e] += __shfl_xor(sk[e], 16, 64);
        sk[e] += __shfl_xor(sk[e], 32, 64);
        sv[e] += __shfl_xor(sv[e], 16, 64);
        sv[e] += __shfl_xor(sv[e], 32, 64);
    }
    vmax2 = fmaxf(vmax2, __shfl_xor(vmax2, 16, 64));
    vmax2 = fmaxf(vmax2, __shfl_xor(vmax2, 32, 64));
    const float n = static_cast<float>(t1 - t0);
    float m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = sk[e] / n;
    float rmax2 = 0.f;
    for (int64_t base = t0; base < t1; base += 4 * NR) {
        uint4 kc[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t t = base + 4 * i + slot;
            const bool ok = t < t1;
            if (base == t0) {
                kc[i] = kw[i];
            } else {
                const uint4 a = kr[(ok ? t : t0) * (kHeadDim / 8)];
                kc[i] = ok ? a : make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            float x[8];
            widen8(kc[i], x);
            float d2 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = x[e] - m[e];
                d2 += d * d;
            }
            d2 = sum16(d2);
            if (base + 4 * i + slot < t1) rmax2 = fmaxf(rmax2, d2);  // uniform within a row
        }
    }
    rmax2 = fmaxf(rmax2, __shfl_xor(rmax2, 16, 64));
    rmax2 = fmaxf(rmax2, __shfl_xor(rmax2, 32, 64));
    if (slot == 0) {
        float4 *mk = reinterpret_cast<float4 *>(mu_k + cl * kHeadDim + 8 * l16);
        float4 *mv = reinterpret_cast<float4 *>(mu_v + cl * kHeadDim + 8 * l16);
        mk[0] = make_float4(m[0], m[1], m[2], m[3]);
        mk[1] = make_float4(m[4], m[5], m[6], m[7]);
        mv[0] = make_float4(sv[0] / n, sv[1] / n, sv[2] / n, sv[3] / n);
        mv[1] = make_float4(sv[4] / n, sv[5] / n, sv[6] / n, sv[7] / n);
    }
    if (lane == 0) {
        radius[cl] = sqrtf(rmax2);
        vnorm[cl] = sqrtf(vmax2);
    }
}

// ||q|| of one query row over a row of 16 lanes, 8 channels per lane; every lane
// of the row gets the same bits, and both risk kernels compute it this way.
__device__ __forceinline__ float query_norm(const uint16_t *qrow, int lane16) {
    float x[8];
    widen8(reinterpret_cast<const uint4 *>(qrow)[lane16], x);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += x[e] * x[e];
    return sqrtf(sum16(s));
}

__device__ __forceinline__ float cluster_size(int64_t j, int64_t c, int64_t S) {
    return static_cast<float>(min((j + 1) * c, S) - j * c);
}

// Partial pass: one workgroup per (slice, chunk of kRiskChunk clusters).  A 16-lane
// row takes clusters grp, grp + 16, ... of the chunk (kRiskBatch loaded before any
// is used); lane i of the row keeps query i's logit z and deviation d of each.
// The logits go to the RC rows (read back by the final pass); the chunk's record
// holds, per query, {zmax_c, zdmax_c, psum_c, dsum_c} with
//   psum_c = sum_C n_C e^{z_C - zmax_c},
//   dsum_c = sum_C n_C (e^{z_C + d_C - zdmax_c} + e^{z_C - d_C - zdmax_c}) / 2,
// zdmax_c = max_C (z_C + d_C) (so no exponent is positive), and the chunk's
// largest value norm.  Rows of the chunk are added in row order.
__global__ __launch_bounds__(kRiskThreads) void risk_partial_kernel(
    const float *__restrict__ mu_k, const float *__restrict__ radius, const float *__restrict__ vnorm,
    int64_t S, int64_t c, int64_t nC, int64_t nchunk, const uint16_t *__restrict__ Q, int nq,
    float *__restrict__ rc, float4 *__restrict__ part) {
    __shared__ float qs[kMaxRiskQueries][kHeadDim];
    __shared__ float red[4][16][kMaxRiskQueries];
    __shared__ float vred[kRiskThreads / 64];
    const int64_t g = blockIdx.x / nchunk, ch = blockIdx.x - g * nchunk;
    const int tid = threadIdx.x, lane16 = tid & 15, grp = tid >> 4;
    const float rs = 1.f / sqrtf(static_cast<float>(kHeadDim));
    const uint16_t *Qg = Q + g * nq * kHeadDim;
    for (int i = tid; i < nq * kHeadDim; i += kRiskThreads)
        qs[i / kHeadDim][i % kHeadDim] = __uint_as_float(static_cast<uint32_t>(Qg[i]) << 16);
    float qn = 0.f;  // ||q|| of this lane's query
    for (int i = 0; i < nq; ++i) {
        const float n = query_norm(Qg + i * kHeadDim, lane16);
        if (lane16 == i) qn = n;
    }
    __syncthreads();  // qs
    const int64_t j0 = ch * kRiskChunk + grp;
    float zr[kRiskPerRow], dr[kRiskPerRow];
    float zmax = -INFINITY, zdmax = -INFINITY, vm = 0.f;
#pragma unroll
    for (int bt = 0; bt < kRiskPerRow / kRiskBatch; ++bt) {
        float4 a[kRiskBatch], b[kRiskBatch];
        float rd[kRiskBatch];
#pragma unroll
        for (int u = 0; u < kRiskBatch; ++u) {
            const int64_t j = j0 + 16 * (bt * kRiskBatch + u);
            const int64_t js = j < nC ? j : nC - 1;  // never past the slice's clusters
            // lane l16 holds channels 4 l16 .. + 3 and 64 + 4 l16 .. + 3: each load covers
            // 256 contiguous bytes of the mean key (streaming: read once)
            const float4 *m4 = reinterpret_cast<const float4 *>(mu_k + (g * nC + js) * kHeadDim) + lane16;
            a[u] = ld_stream(m4);
            b[u] = ld_stream(m4 + 16);
            rd[u] = radius[g * nC + js];
            vm = fmaxf(vm, vnorm[g * nC + js]);  // a repeated cluster leaves the maximum as it is
        }
#pragma unroll
        for (int u = 0; u < kRiskBatch; ++u) {
            const int k = bt * kRiskBatch + u;
            const int64_t j = j0 + 16 * k;
            float zi = 0.f;
            for (int i = 0; i < nq; ++i) {
                const float *q = &qs[i][lane16 * 4], *q2 = q + 64;
                const float z = a[u].x * q[0] + a[u].y * q[1] + a[u].z * q[2] + a[u].w * q[3] + b[u].x * q2[0] +
                                b[u].y * q2[1] + b[u].z * q2[2] + b[u].w * q2[3];
                const float zs = sum16(z) * rs;
                zi = lane16 == i ? zs : zi;
            }
            const float dl = qn * rd[u] * rs;
            zr[k] = zi;
            dr[k] = dl;
            if (j < nC && lane16 < nq) {
                rc[(g * nq + lane16) * nC + j] = zi;
                zmax = fmaxf(zmax, zi);
                zdmax = fmaxf(zdmax, zi + dl);
            }
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) vm = fmaxf(vm, __shfl_xor(vm, d, 64));
    if ((tid & 63) == 0) vred[tid >> 6] = vm;
    if (lane16 < kMaxRiskQueries) {
        red[0][grp][lane16] = zmax;
        red[1][grp][lane16] = zdmax;
    }
    __syncthreads();
    float cz = -INFINITY, czd = -INFINITY, ps = 0.f, ds = 0.f;
    if (lane16 < nq) {
        for (int r = 0; r < 16; ++r) {
            cz = fmaxf(cz, red[0][r][lane16]);
            czd = fmaxf(czd, red[1][r][lane16]);
        }
#pragma unroll
        for (int k = 0; k < kRiskPerRow; ++k) {
            const int64_t j = j0 + 16 * k;
            if (j < nC) {
                const float n = cluster_size(j, c, S);
                ps += n * expf(zr[k] - cz);
                ds += n * 0.5f * (expf(zr[k] + dr[k] - czd) + expf(zr[k] - dr[k] - czd));
            }
        }
        red[2][grp][lane16] = ps;
        red[3][grp][lane16] = ds;
    }
    __syncthreads();
    float4 *rec = part + (g * nchunk + ch) * kPartStride;
    if (tid < nq) {  // row 0, lane i: cz, czd are query i's chunk maxima
        float P = 0.f, D = 0.f;
        for (int r = 0; r < 16; ++r) {
            P += red[2][r][tid];
            D += red[3][r][tid];
        }
        rec[tid] = make_float4(cz, czd, P, D);
    }
    if (tid == 0) {
        float v = vred[0];
        for (int w = 1; w < kRiskThreads / 64; ++w) v = fmaxf(v, vred[w]);
        rec[kMaxRiskQueries] = make_float4(v, 0.f, 0.f, 0.f);
    }
}

// Final pass: one workgroup per (slice, kRiskFinalChunk clusters).  The slice's
// chunk records are merged (maxima, then the sums rescaled to the common maxima:
// 32 lanes per query, chunks c = lane, lane + 32, ... in order, then a 32-lane
// butterfly, so every workgroup of the slice holds the same bits); then
//   RC = 2 Vmax [ n e^{z + d - zdmax} expm1(-d)^2 / (2 dsum) + p tanh(d / 2) ],
//   p = n e^{z - zmax} / psum,
// the first term being p (cosh d - 1) / Dn with cosh d - 1 = e^d expm1(-d)^2 / 2
// and Dn = e^{zdmax - zmax} dsum / psum: no exponent is positive, nothing cancels.
__global__ __launch_bounds__(kRiskThreads) void risk_final_kernel(
    const float *__restrict__ radius, int64_t S, int64_t c, int64_t nC, int64_t nchunk, int64_t nfin,
    const uint16_t *__restrict__ Q, int nq, const float4 *__restrict__ part, float *__restrict__ rc) {
    __shared__ float4 merged[kMaxRiskQueries];
    __shared__ float vmax_s;
    const int64_t g = blockIdx.x / nfin, fc = blockIdx.x - g * nfin;
    const int tid = threadIdx.x, lane16 = tid & 15;
    const float rs = 1.f / sqrtf(static_cast<float>(kHeadDim));
    const uint16_t *Qg = Q + g * nq * kHeadDim;
    float qn[kMaxRiskQueries];
#pragma unroll
    for (int i = 0; i < kMaxRiskQueries; ++i) qn[i] = i < nq ? query_norm(Qg + i * kHeadDim, lane16) : 0.f;
    {
        const int mi = tid >> 5, sl = tid & 31;  // query, lane within its 32
        const float4 *pg = part + g * nchunk * kPartStride;
        float m = -INFINITY, md = -INFINITY, vm = 0.f, P = 0.f, D = 0.f;
        if (mi < nq) {
            for (int64_t k = sl; k < nchunk; k += 32) {
                const float4 r = pg[k * kPartStride + mi];
                m = fmaxf(m, r.x);
                md = fmaxf(md, r.y);
            }
        }
        if (mi == 0)
            for (int64_t k = sl; k < nchunk; k += 32) vm = fmaxf(vm, pg[k * kPartStride + kMaxRiskQueries].x);
#pragma unroll
        for (int d = 16; d >= 1; d >>= 1) {
            m = fmaxf(m, __shfl_xor(m, d, 32));
            md = fmaxf(md, __shfl_xor(md, d, 32));
            vm = fmaxf(vm, __shfl_xor(vm, d, 32));
        }
        if (mi < nq) {
            for (int64_t k = sl; k < nchunk; k += 32) {
                const float4 r = pg[k * kPartStride + mi];
                P += r.z * expf(r.x - m);
                D += r.w * expf(r.y - md);
            }
        }
#pragma unroll
        for (int d = 16; d >= 1; d >>= 1) {
            P += __shfl_xor(P, d, 32);
            D += __shfl_xor(D, d, 32);
        }
        if (sl == 0 && mi < nq) merged[mi] = make_float4(m, md, P, D);
        if (tid == 0) vmax_s = vm;
    }
    __syncthreads();
    const float vmax = vmax_s;
    const int64_t j1 = min((fc + 1) * kRiskFinalChunk, nC);
    for (int64_t j = fc * kRiskFinalChunk + tid; j < j1; j += kRiskThreads) {
        const float n = cluster_size(j, c, S);
        const float r = radius[g * nC + j];
#pragma unroll
        for (int i = 0; i < kMaxRiskQueries; ++i) {
            if (i >= nq) break;
            const float4 M = merged[i];
            float *o = rc + (g * nq + i) * nC + j;
            const float z = *o, dl = qn[i] * r * rs;
            const float p = n * expf(z - M.x) / M.z;
            const float em = expm1f(-dl);
            const float dev = n * expf(z + dl - M.y) * em * em / (2.f * M.w);
            *o = 2.f * vmax * (dev + p * tanhf(0.5f * dl));
        }
    }
}

}  // namespace

// Chunk records of the risk passes: kPartStride float4 per (slice, chunk).
size_t risk_bytes(int64_t G, int64_t S, int64_t c) {
    if (G < 0 || S < 1 || c < 1) return 0;
    const int64_t nC = (S + c - 1) / c;
    const int64_t nchunk = (nC + kRiskChunk - 1) / kRiskChunk;
    return static_cast<size_t>(G * nchunk) * kPartStride * sizeof(float4);
}

}  // namespace kvc

extern "C" kvc_status kvc_cluster_summaries(const uint16_t *K, const uint16_t *V, int64_t G, int64_t S,
                                            int32_t D, int64_t c, float *mu_k, float *mu_v,
                                            float *radius, float *vnorm, hipStream_t stream) {
    using namespace kvc;
    if (G < 0 || S < 1 || c < 1 || D <= 0) return KVC_ERR_INVALID_ARGUMENT;
    if (D != kHeadDim) return KVC_ERR_UNSUPPORTED;
    if (G == 0) return KVC_OK;
    if (!K || !V || !mu_k || !mu_v || !radius || !vnorm) return KVC_ERR_INVALID_ARGUMENT;
    if (!aligned(K, 16) || !aligned(V, 16) || !aligned(mu_k, 16) || !aligned(mu_v, 16) ||
        !aligned(radius, 4) || !aligned(vnorm, 4))
        return KVC_ERR_INVALID_ARGUMENT;
    const int64_t nC = (S + c - 1) / c;
    const int64_t blocks = (G * nC + kSumWaves - 1) / kSumWaves;
    if (blocks > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    // rows per chunk (in flight together, the first chunk kept for the radius pass)
    if (c <= 12)
        hipLaunchKernelGGL(cluster_summary_kernel<3>, dim3(static_cast<unsigned>(blocks)), dim3(64 * kSumWaves),
                           0, stream, K, V, G, S, c, nC, mu_k, mu_v, radius, vnorm);
    else if (c <= 16)
        hipLaunchKernelGGL(cluster_summary_kernel<4>, dim3(static_cast<unsigned>(blocks)), dim3(64 * kSumWaves),
                           0, stream, K, V, G, S, c, nC, mu_k, mu_v, radius, vnorm);
    else
        hipLaunchKernelGGL(cluster_summary_kernel<8>, dim3(static_cast<unsigned>(blocks)), dim3(64 * kSumWaves),
                           0, stream, K, V, G, S, c, nC, mu_k, mu_v, radius, vnorm);
    return launch_status();
}

extern "C" kvc_status kvc_refine_risk(const float *mu_k, const float *radius, const float *vnorm,
                                      int64_t G, int64_t S, int64_t c, int32_t D, const uint16_t *Q,
                                      int32_t nq, float *rc, void *ws, size_t ws_bytes,
                                      hipStream_t stream) {
    using namespace kvc;
    if (G < 0 || S < 1 || c < 1 || D <= 0 || nq < 0) return KVC_ERR_INVALID_ARGUMENT;
    if (D != kHeadDim || nq > kMaxRiskQueries) return KVC_ERR_UNSUPPORTED;
    if (G == 0 || nq == 0) return KVC_OK;
    if (!mu_k || !radius || !vnorm || !Q || !rc || !ws) return KVC_ERR_INVALID_ARGUMENT;
    if (!aligned(mu_k, 16) || !aligned(radius, 4) || !aligned(vnorm, 4) || !aligned(Q, 16) ||
        !aligned(rc, 4) || !aligned(ws, 16))
        return KVC_ERR_INVALID_ARGUMENT;
    if (ws_bytes < risk_bytes(G, S, c)) return KVC_ERR_WORKSPACE_TOO_SMALL;
    const int64_t nC = (S + c - 1) / c;
    const int64_t nchunk = (nC + kRiskChunk - 1) / kRiskChunk;
    const int64_t nfin = (nC + kRiskFinalChunk - 1) / kRiskFinalChunk;
    if (G * nchunk > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    float4 *part = static_cast<float4 *>(ws);
    hipLaunchKernelGGL(risk_partial_kernel, dim3(static_cast<unsigned>(G * nchunk)), dim3(kRiskThreads), 0,
                       stream, mu_k, radius, vnorm, S, c, nC, nchunk, Q, nq, rc, part);
    hipLaunchKernelGGL(risk_final_kernel, dim3(static_cast<unsigned>(G * nfin)), dim3(kRiskThreads), 0, stream,
                       radius, S, c, nC, nchunk, nfin, Q, nq, part, rc);
    return launch_status();
}
