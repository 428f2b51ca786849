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
// refine_risk_kernel: one 1024-thread workgroup per slice and its queries; 16
//   lanes per cluster (8 channels each) for the logits z, written into the RC
//   buffer and read back for the normalisation passes; block reductions in a
//   fixed order (deterministic).  The normaliser's terms are shifted by their
//   largest exponent max_C (z_C + d_C), so no cosh overflows fp32 however far
//   apart a cluster's keys lie.
#include <math.h>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kSumWaves = 4;       // clusters per summary workgroup
constexpr int kRiskThreads = 1024;
constexpr int kMaxRiskQueries = 8;
constexpr int kRiskUnroll = 4;     // clusters in flight per 16-lane group in the logit pass

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
            const bool ok = t < t1;
            const int64_t ts = ok ? t : t0;  // rows past the cluster are never read
            const uint4 a = kr[ts * (kHeadDim / 8)], b = vr[ts * (kHeadDim / 8)];
            kc[i] = ok ? a : make_uint4(0u, 0u, 0u, 0u);
            vc[i] = ok ? b : make_uint4(0u, 0u, 0u, 0u);
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

// Block-wide reduction over 1024 threads in a fixed order (op: 0 sum, 1 max).
template <int kOp>
__device__ __forceinline__ float block_reduce(float x, float *scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const float y = __shfl_xor(x, d, 64);
        x = kOp == 0 ? x + y : fmaxf(x, y);
    }
    __syncthreads();  // scratch is free
    if (lane == 0) scratch[wave] = x;
    __syncthreads();
    float r = kOp == 0 ? 0.f : -INFINITY;
    for (int w = 0; w < kRiskThreads / 64; ++w) r = kOp == 0 ? r + scratch[w] : fmaxf(r, scratch[w]);
    return r;
}

__global__ __launch_bounds__(kRiskThreads) void refine_risk_kernel(
    const float *__restrict__ mu_k, const float *__restrict__ radius, const float *__restrict__ vnorm,
    int64_t S, int64_t c, int64_t nC, const uint16_t *__restrict__ Q, int nq, float *__restrict__ rc) {
    __shared__ float qs[kMaxRiskQueries][kHeadDim];
    __shared__ float scratch[kRiskThreads / 64];
    const int64_t g = blockIdx.x;
    const int tid = threadIdx.x, lane16 = tid & 15, grp = tid >> 4;  // 64 groups of 16 lanes
    const float rs = 1.f / sqrtf(static_cast<float>(kHeadDim));
    for (int i = tid; i < nq * kHeadDim; i += kRiskThreads) {
        const uint16_t h = Q[(g * nq) * kHeadDim + i];
        qs[i / kHeadDim][i % kHeadDim] = __uint_as_float(static_cast<uint32_t>(h) << 16);
    }
    __syncthreads();
    float qn[kMaxRiskQueries];
    for (int i = 0; i < nq; ++i) {
        float s = 0.f;
        for (int d = 0; d < kHeadDim; ++d) s += qs[i][d] * qs[i][d];
        qn[i] = sqrtf(s);  // the same bits in every thread
    }
    float *rcg = rc + g * nq * nC;
    // pass 1: logits z into the output rows; running maxima; the slice's value bound
    // zdmax = max_C (z_C + d_C), the largest exponent of n_C e^{z_C} cosh d_C
    float zmax[kMaxRiskQueries], zdmax[kMaxRiskQueries], vm = 0.f;
    for (int i = 0; i < kMaxRiskQueries; ++i) zmax[i] = zdmax[i] = -INFINITY;
    // kRiskUnroll clusters per 16-lane group are loaded before any is used
    constexpr int kGroups = kRiskThreads / 16;
    for (int64_t j0 = grp; j0 < nC; j0 += kRiskUnroll * kGroups) {
        float4 a[kRiskUnroll], b[kRiskUnroll];
        float vn[kRiskUnroll], rd[kRiskUnroll];
#pragma unroll
        for (int u = 0; u < kRiskUnroll; ++u) {
            const int64_t j = j0 + u * kGroups;
            const int64_t js = j < nC ? j : j0;  // never past the slice's clusters
            const float4 *m4 = reinterpret_cast<const float4 *>(mu_k + (g * nC + js) * kHeadDim + lane16 * 8);
            a[u] = m4[0];
            b[u] = m4[1];
            vn[u] = vnorm[g * nC + js];
            rd[u] = radius[g * nC + js];
        }
#pragma unroll
        for (int u = 0; u < kRiskUnroll; ++u) {
            const int64_t j = j0 + u * kGroups;
            if (j >= nC) break;  // uniform within the 16-lane group
            for (int i = 0; i < nq; ++i) {
                const float *q = &qs[i][lane16 * 8];
                float z = a[u].x * q[0] + a[u].y * q[1] + a[u].z * q[2] + a[u].w * q[3] + b[u].x * q[4] +
                          b[u].y * q[5] + b[u].z * q[6] + b[u].w * q[7];
                z += __shfl_xor(z, 8, 16);
                z += __shfl_xor(z, 4, 16);
                z += __shfl_xor(z, 2, 16);
                z += __shfl_xor(z, 1, 16);
                z *= rs;
                zmax[i] = fmaxf(zmax[i], z);
                zdmax[i] = fmaxf(zdmax[i], z + qn[i] * rd[u] * rs);
                if (lane16 == i) rcg[i * nC + j] = z;
            }
            vm = fmaxf(vm, vn[u]);
        }
    }
    const float vmax = block_reduce<1>(vm, scratch);
    for (int i = 0; i < nq; ++i) {
        zmax[i] = block_reduce<1>(zmax[i], scratch);
        zdmax[i] = block_reduce<1>(zdmax[i], scratch);
    }
    __syncthreads();  // the logits written by other threads are visible
    // pass 2: masses n_C e^{z - zmax} and their sum psum; the normaliser as
    // dsum = sum_C n_C e^{z_C - zdmax} cosh d_C, every exponent <= 0 (cosh d overflows
    // fp32 past d ~ 89; here the largest term is >= n_C / 2 and none overflows), so
    // Dn = e^{zdmax - zmax} dsum / psum
    float psum[kMaxRiskQueries], dsum[kMaxRiskQueries];
    for (int i = 0; i < nq; ++i) {
        psum[i] = 0.f;
        dsum[i] = 0.f;
    }
    for (int64_t j = tid; j < nC; j += kRiskThreads) {
        const float n = static_cast<float>(min((j + 1) * c, S) - j * c);
        const float r = radius[g * nC + j];
        for (int i = 0; i < nq; ++i) {
            const float z = rcg[i * nC + j], dl = qn[i] * r * rs;
            psum[i] += n * expf(z - zmax[i]);
            dsum[i] += n * 0.5f * (expf(z + dl - zdmax[i]) + expf(z - dl - zdmax[i]));
        }
    }
    for (int i = 0; i < nq; ++i) {
        psum[i] = block_reduce<0>(psum[i], scratch);
        dsum[i] = block_reduce<0>(dsum[i], scratch);
    }
    // pass 3: RC = 2 p Vmax [ (cosh d - 1) / Dn + tanh(d / 2) ]; with cosh d - 1 =
    // 2 sinh^2(d / 2) = e^d expm1(-d)^2 / 2 the first term is
    // n e^{z + d - zdmax} expm1(-d)^2 / (2 dsum): an exponent <= 0 and no cancellation
    for (int64_t j = tid; j < nC; j += kRiskThreads) {
        const float n = static_cast<float>(min((j + 1) * c, S) - j * c);
        const float r = radius[g * nC + j];
        for (int i = 0; i < nq; ++i) {
            const float z = rcg[i * nC + j], dl = qn[i] * r * rs;
            const float p = n * expf(z - zmax[i]) / psum[i];
            const float em = expm1f(-dl);
            const float dev = n * expf(z + dl - zdmax[i]) * em * em / (2.f * dsum[i]);
            rcg[i * nC + j] = 2.f * vmax * (dev + p * tanhf(0.5f * dl));
        }
    }
}

}  // namespace
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
                                      int32_t nq, float *rc, hipStream_t stream) {
    using namespace kvc;
    if (G < 0 || S < 1 || c < 1 || D <= 0 || nq < 0) return KVC_ERR_INVALID_ARGUMENT;
    if (D != kHeadDim || nq > kMaxRiskQueries) return KVC_ERR_UNSUPPORTED;
    if (G == 0 || nq == 0) return KVC_OK;
    if (!mu_k || !radius || !vnorm || !Q || !rc) return KVC_ERR_INVALID_ARGUMENT;
    if (!aligned(mu_k, 16) || !aligned(radius, 4) || !aligned(vnorm, 4) || !aligned(Q, 2) ||
        !aligned(rc, 4))
        return KVC_ERR_INVALID_ARGUMENT;
    if (G > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    const int64_t nC = (S + c - 1) / c;
    hipLaunchKernelGGL(refine_risk_kernel, dim3(static_cast<unsigned>(G)), dim3(kRiskThreads), 0, stream,
                       mu_k, radius, vnorm, S, c, nC, Q, nq, rc);
    return launch_status();
}
