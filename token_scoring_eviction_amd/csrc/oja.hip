// Oja basis update with pooling and QR ("OjaKV: Context-Aware Online Low-Rank
// KV Cache Compression": the Oja rule U <- U + eta (x x^T U - U U^T x x^T U) in
// "how it works"; the pooled prefill update with the empirical covariance, the
// buffered decode update and the QR re-orthonormalisation in method details).
//
//   pool_kernel        X bf16 [slice][N][128] -> Xp fp32 [slice][ceil(N/p)][128]
//                      (mean over each window of p tokens; short tail window)
//   cov_partial_kernel per (layer, kv head) and chunk of pooled rows (rows of
//                      all sequences of the batch): sum of x x^T in fp32,
//                      8x8 register tiles over LDS-staged rows
//   oja_step_qr_*      per (layer, kv head), fp64 arithmetic: C = sum of
//                      partials / n in chunk order; CU = C U; M = U^T CU;
//                      U' = U + eta (CU - U M); then a QR with a positive
//                      diagonal, U <- fp32(Q).  R <= 64 (oja_step_qr_lds_kernel)
//                      runs entirely in LDS with the products on the fp64
//                      matrix cores and Cholesky QR applied twice (the Gram
//                      matrix factored by rows on one wave); R = 96 and 128
//                      (oja_step_qr_kernel) keep C, CU, M in the workspace and
//                      use classical Gram-Schmidt applied twice per column.
#include <cmath>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kCovStage = 64;  // pooled rows staged in LDS per step

constexpr int kPoolThreads = 64;  // one wave, four pooled rows per workgroup
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const uint16_t *__restrict__ X, int64_t rows,
                                                   int64_t N, int64_t S_stride, int p, int64_t np,
                                                   float *__restrict__ Xp) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * (kPoolThreads / 16) + (threadIdx.x >> 4);
    const int lane16 = threadIdx.x & 15;
    if (r >= rows) return;
    const int64_t slice = r / np, i = r % np;
    const int64_t t0 = i * p, t1 = min(t0 + p, N);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint4 *src = reinterpret_cast<const uint4 *>(X + slice * S_stride * kHeadDim) + lane16;
    for (int64_t t = t0; t < t1; ++t) {
        const uint4 v = ld_stream(src + t * (kHeadDim / 8));  // whole rows, read once
        acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x);
        acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
        acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z);
        acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
    }
    const float cnt = static_cast<float>(t1 - t0);
    float4 *dst = reinterpret_cast<float4 *>(Xp + r * kHeadDim + lane16 * 8);
    dst[0] = make_float4(acc[0] / cnt, acc[1] / cnt, acc[2] / cnt, acc[3] / cnt);
    dst[1] = make_float4(acc[4] / cnt, acc[5] / cnt, acc[6] / cnt, acc[7] / cnt);
}

__global__ __launch_bounds__(256) void cov_partial_kernel(const float *__restrict__ Xp, int64_t B,
                                                          int64_t Hkv, int64_t np,
                                                          int64_t rows_per_chunk, int64_t nchunk,
                                                          float *__restrict__ Cpart) {
    const int64_t lh = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const int64_t l = lh / Hkv, h = lh % Hkv;
    const int64_t n = B * np;
    const int64_t m0 = chunk * rows_per_chunk, m1 = min(m0 + rows_per_chunk, n);
    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
    __shared__ float xs[kCovStage][kHeadDim + 4];
    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    for (int64_t mb = m0; mb < m1; mb += kCovStage) {
        for (int e = threadIdx.x; e < kCovStage * (kHeadDim / 4); e += blockDim.x) {
            const int rr = e / (kHeadDim / 4), c4 = e % (kHeadDim / 4);
            const int64_t m = mb + rr;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m < m1) {
                const int64_t b = m / np, i = m % np;
                const int64_t row = ((l * B + b) * Hkv + h) * np + i;
                v = reinterpret_cast<const float4 *>(Xp + row * kHeadDim)[c4];
            }
            xs[rr][c4 * 4 + 0] = v.x;
            xs[rr][c4 * 4 + 1] = v.y;
            xs[rr][c4 * 4 + 2] = v.z;
            xs[rr][c4 * 4 + 3] = v.w;
        }
        __syncthreads();
        for (int m = 0; m < kCovStage; ++m) {
            float xa[8], xc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xa[i] = xs[m][ty * 8 + i];
                xc[i] = xs[m][tx * 8 + i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] += xa[i] * xc[j];
        }
        __syncthreads();
    }
    float *dst = Cpart + (lh * nchunk + chunk) * (kHeadDim * kHeadDim);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[(ty * 8 + i) * kHeadDim + tx * 8 + j] = acc[i][j];
}

__device__ __forceinline__ double block_sum_128(double v, double *red) {
    // sum over threads 0..127 (others pass 0); result broadcast to all threads
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if ((threadIdx.x & 63) == 0 && threadIdx.x < 128) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const double s = red[0] + red[1];
    __syncthreads();
    return s;
}

__global__ __launch_bounds__(256) void oja_step_qr_kernel(float *__restrict__ U,
                                                          const float *__restrict__ Cpart,
                                                          int64_t nchunk, int64_t n, int R,
                                                          double eta, double *__restrict__ C64,
                                                          double *__restrict__ CU64,
                                                          double *__restrict__ M64) {
    extern __shared__ double lds[];
    const int ld = R + 1;
    double *Ul = lds;                     // [128][R+1]: U, then Q
    double *vs = Ul + kHeadDim * ld;      // [128]
    double *ds = vs + kHeadDim;           // [128]
    double *red = ds + kHeadDim;          // [2]
    const int64_t lh = blockIdx.x;
    const int tid = threadIdx.x;
    float *Ug = U + lh * kHeadDim * R;
    double *Cg = C64 + lh * kHeadDim * kHeadDim;
    double *CUg = CU64 + lh * kHeadDim * R;
    double *Mg = M64 + lh * R * R;
    const int DD = kHeadDim * kHeadDim;

    for (int e = tid; e < DD; e += blockDim.x) {
        double s = 0.0;
        for (int64_t ch = 0; ch < nchunk; ++ch) s += static_cast<double>(Cpart[(lh * nchunk + ch) * DD + e]);
        Cg[e] = s / static_cast<double>(n);
    }
    for (int e = tid; e < kHeadDim * R; e += blockDim.x) Ul[(e / R) * ld + e % R] = static_cast<double>(Ug[e]);
    __syncthreads();
    // CU = C U
    for (int e = tid; e < kHeadDim * R; e += blockDim.x) {
        const int a = e / R, j = e % R;
        double s = 0.0;
        for (int c = 0; c < kHeadDim; ++c) s += Cg[a * kHeadDim + c] * Ul[c * ld + j];
        CUg[e] = s;
    }
    __syncthreads();
    // M = U^T (C U)
    for (int e = tid; e < R * R; e += blockDim.x) {
        const int i = e / R, j = e % R;
        double s = 0.0;
        for (int a = 0; a < kHeadDim; ++a) s += Ul[a * ld + i] * CUg[a * R + j];
        Mg[e] = s;
    }
    __syncthreads();
    // U' = U + eta (CU - U M), written over CU
    for (int e = tid; e < kHeadDim * R; e += blockDim.x) {
        const int a = e / R, j = e % R;
        double s = 0.0;
        for (int i = 0; i < R; ++i) s += Ul[a * ld + i] * Mg[i * R + j];
        CUg[e] = Ul[a * ld + j] + eta * (CUg[e] - s);
    }
    __syncthreads();
    // QR of U' by Gram-Schmidt, twice per column; Q overwrites Ul column by column
    for (int j = 0; j < R; ++j) {
        double v = tid < kHeadDim ? CUg[tid * R + j] : 0.0;
        for (int pass = 0; pass < 2; ++pass) {
            if (tid < kHeadDim) vs[tid] = v;
            __syncthreads();
            if (tid < j) {
                double d = 0.0;
                for (int a = 0; a < kHeadDim; ++a) d += Ul[a * ld + tid] * vs[a];
                ds[tid] = d;
            }
            __syncthreads();
            if (tid < kHeadDim) {
                double s = 0.0;
                for (int i = 0; i < j; ++i) s += ds[i] * Ul[tid * ld + i];
                v -= s;
            }
            __syncthreads();
        }
        const double nrm2 = block_sum_128(tid < kHeadDim ? v * v : 0.0, red);
        if (tid < kHeadDim) Ul[tid * ld + j] = v / sqrt(nrm2);
        __syncthreads();
    }
    for (int e = tid; e < kHeadDim * R; e += blockDim.x) Ug[e] = static_cast<float>(Ul[(e / R) * ld + e % R]);
}

// fp64 matrix cores, v_mfma_f64_16x16x4f64: A[i][k] comes from lane i + 16k, B[k][j]
// from lane j + 16k, and element r of lane l receives D[l / 16 + 4r][l % 16].
typedef double f64x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// X^T Y for two [128][R] fp64 matrices in LDS (row strides ldx, ldy) into out [R][ldo],
// on the matrix cores: the (R/16)^2 16 x 16 blocks are shared by the four waves,
// each summed over the 128 rows in 32 steps of 4.  Every element of the result is
// the same sequence of fp64 products in the same order wherever its block sits.
template <int R, typename OutT>
__device__ __forceinline__ void gram128(const double *X, int ldx, const double *Y, int ldy, OutT *out, int ldo) {
    constexpr int NB = R / 16, kPer = NB * NB / 4;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, kq = lane >> 4;
    f64x4 acc[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) acc[t] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int k0 = 0; k0 < kHeadDim; k0 += 4) {
        double a[kPer], b[kPer];
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int blk = wave * kPer + t, ib = blk / NB, jb = blk % NB;
            a[t] = X[(k0 + kq) * ldx + 16 * ib + l16];
            b[t] = Y[(k0 + kq) * ldy + 16 * jb + l16];
        }
#pragma unroll
        for (int t = 0; t < kPer; ++t) acc[t] = mfma_f64(a[t], b[t], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
        const int blk = wave * kPer + t, ib = blk / NB, jb = blk % NB;
#pragma unroll
        for (int r = 0; r < 4; ++r) out[(16 * ib + kq + 4 * r) * ldo + 16 * jb + l16] = static_cast<OutT>(acc[t][r]);
    }
}

// Cholesky QR of W [128][R] (fp64, LDS, row-major) applied twice: G = W^T W =
// R_^T R_ with R_ upper triangular and a positive diagonal, then W <- W R_^{-1}.
// One pass leaves an orthogonality error of about cond(W)^2 eps; the second
// pass, on a W that is already orthonormal to that level, brings it to eps.  The
// Q factor with a positive diagonal of R is unique, so this is the same Q as any
// other QR with that convention.  256 threads; G [R][R+1] is scratch.
template <int R>
__device__ void cholesky_qr2(double *W, double *G) {
    constexpr int ldg = R + 1;
    const int tid = threadIdx.x;
    for (int pass = 0; pass < 2; ++pass) {
        gram128<R>(W, R, W, R, G, ldg);  // G = W^T W (only the upper triangle is read)
        __syncthreads();
        // Cholesky factor by rows, on one wave (no workgroup barriers): lane j keeps
        // column j of R_ in registers; at step k every lane forms
        //   v_j = G_kj - sum_{i<k} R_ik R_ij
        // (R_ik read from the rows already stored), R_kk = sqrt(v_k) comes from lane k,
        // and R_kj = v_j / R_kk overwrites G_kj.  (Right-looking on the whole
        // workgroup, with a barrier per step, this took 45 us of a 0.37 ms call;
        // right-looking on one wave, with every lane's trailing column in registers,
        // it spilled.)
        if (tid < 64) {
            const int j = tid;
            double col[R];
#pragma unroll
            for (int i = 0; i < R; ++i) col[i] = 0.0;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                double s0 = 0.0, s1 = 0.0;
#pragma unroll
                for (int i = 0; i < k; ++i) {
                    const double rik = G[i * ldg + k];
                    if (i & 1) s1 = fma(rik, col[i], s1);
                    else s0 = fma(rik, col[i], s0);
                }
                const double v = (j < R ? G[k * ldg + (j < R ? j : 0)] : 0.0) - (s0 + s1);
                const double rkk = sqrt(__shfl(v, k, 64));
                const double rkj = j == k ? rkk : v / rkk;
                if (j >= k && j < R) {
                    col[k] = rkj;
                    G[k * ldg + j] = rkj;
                }
                // row k is read back by the next steps of this wave
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
        __syncthreads();
        // W <- W R_^{-1}: one row per thread, forward substitution in registers
        if (tid < kHeadDim) {
            double x[R];
#pragma unroll
            for (int j = 0; j < R; ++j) x[j] = W[tid * R + j];
#pragma unroll
            for (int j = 0; j < R; ++j) {
                double s0 = x[j], s1 = 0.0;
#pragma unroll
                for (int i = 0; i < j; ++i) {
                    if (i & 1) s1 = fma(-x[i], G[i * ldg + j], s1);
                    else s0 = fma(-x[i], G[i * ldg + j], s0);
                }
                x[j] = (s0 + s1) / G[j * ldg + j];
            }
#pragma unroll
            for (int j = 0; j < R; ++j) W[tid * R + j] = x[j];
        }
        __syncthreads();
    }
}

// Fast path for R <= 64: everything per head stays in LDS, and the products
// (CU, U^T CU, U M and the Gram matrices of the QR) run on the fp64 matrix cores.
//   Ud [128][R+1] fp64: U, later the Gram matrix of the QR;  Wd [128][R] fp64: C
//   column chunks, then CU, then U', then Q;  Mf [R][R+1] fp32: U^T C U.
// (With fp64 vector FMAs, one row and half the columns of CU and U' per thread,
// and a workgroup-wide right-looking Cholesky, a call took 0.37 ms at 256 heads.)
constexpr int kCChunk = 16;  // C columns staged per step

template <int R>
__global__ __launch_bounds__(256) void oja_step_qr_lds_kernel(float *__restrict__ U,
                                                              const float *__restrict__ Cpart,
                                                              int64_t nchunk, int64_t n, double eta) {
    extern __shared__ double lds[];
    const int ld = R + 1;
    double *Ud = lds;                                  // [128][R+1]
    double *Wd = Ud + kHeadDim * ld;                   // [128][R] (>= [128][kCChunk])
    float *Mf = reinterpret_cast<float *>(Wd + kHeadDim * R);  // [R][R+1]
    const int64_t lh = blockIdx.x;
    const int tid = threadIdx.x;
    float *Ug = U + lh * kHeadDim * R;
    const int DD = kHeadDim * kHeadDim;
    const double inv_n = 1.0 / static_cast<double>(n);

    for (int e = tid; e < kHeadDim * R; e += blockDim.x) Ud[(e / R) * ld + e % R] = static_cast<double>(Ug[e]);
    // CU = C U on the matrix cores: wave w takes row blocks 2w and 2w + 1 and every
    // column block; C is staged kCChunk columns at a time (row stride kCChunk + 1),
    // the chunk partials of each entry added in chunk order
    constexpr int NB = R / 16, kCs = kCChunk + 1;
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, kq = lane >> 4;
    f64x4 cu[2][NB];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) cu[hh][cb] = f64x4{0.0, 0.0, 0.0, 0.0};
    for (int c0 = 0; c0 < kHeadDim; c0 += kCChunk) {
        __syncthreads();
        for (int e = tid; e < kHeadDim * kCChunk; e += blockDim.x) {
            const int r = e / kCChunk, c = c0 + e % kCChunk;
            double sum = 0.0;
            for (int64_t ch = 0; ch < nchunk; ++ch)
                sum += static_cast<double>(Cpart[(lh * nchunk + ch) * DD + r * kHeadDim + c]);
            Wd[r * kCs + e % kCChunk] = sum * inv_n;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kCChunk; kk += 4) {
            double av[2], bv[NB];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) av[hh] = Wd[(16 * (2 * wave + hh) + l16) * kCs + kk + kq];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) bv[cb] = Ud[(c0 + kk + kq) * ld + 16 * cb + l16];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) cu[hh][cb] = mfma_f64(av[hh], bv[cb], cu[hh][cb]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Wd[(16 * (2 * wave + hh) + kq + 4 * r) * R + 16 * cb + l16] = cu[hh][cb][r];
    __syncthreads();
    // M = U^T (C U), kept in fp32
    gram128<R>(Ud, ld, Wd, R, Mf, ld);
    __syncthreads();
    // U' = U + eta (CU - U M): U M on the matrix cores in the blocks of CU; each lane
    // updates the entries of Wd that its accumulators hold
    {
        f64x4 um[2][NB];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) um[hh][cb] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int k0 = 0; k0 < R; k0 += 4) {
            double av[2], bv[NB];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) av[hh] = Ud[(16 * (2 * wave + hh) + l16) * ld + k0 + kq];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) bv[cb] = static_cast<double>(Mf[(k0 + kq) * ld + 16 * cb + l16]);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) um[hh][cb] = mfma_f64(av[hh], bv[cb], um[hh][cb]);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * (2 * wave + hh) + kq + 4 * r, col = 16 * cb + l16;
                    Wd[row * R + col] = Ud[row * ld + col] + eta * (Wd[row * R + col] - um[hh][cb][r]);
                }
    }
    __syncthreads();
    // QR of U' (in Wd) by Cholesky QR twice; U is no longer needed, so its
    // storage holds the Gram matrix
    cholesky_qr2<R>(Wd, Ud);
    for (int e = tid; e < kHeadDim * R; e += blockDim.x) Ug[e] = static_cast<float>(Wd[e]);
}

size_t oja_lds_bytes(int R) {
    const size_t ld = R + 1;
    return (kHeadDim * ld + kHeadDim * R) * sizeof(double) + R * ld * sizeof(float);
}

struct OjaGeom {
    int64_t G, LH, N, S_stride, np, n, nchunk, rows_per_chunk;
};

OjaGeom make_oja_geom(const kvc_dims *d, int64_t pool) {
    OjaGeom o;
    o.G = d->L * d->B * d->H_kv;
    o.LH = d->L * d->H_kv;
    o.N = d->S;
    o.S_stride = d->S_stride ? d->S_stride : d->S;
    o.np = (d->S + pool - 1) / pool;
    o.n = d->B * o.np;
    int64_t want = o.LH > 0 ? (1024 + o.LH - 1) / o.LH : 1;  // chunks per head
    int64_t maxc = (o.n + kCovStage - 1) / kCovStage;
    if (want > maxc) want = maxc;
    if (want < 1) want = 1;
    o.rows_per_chunk = (o.n + want - 1) / want;
    o.rows_per_chunk = (o.rows_per_chunk + kCovStage - 1) / kCovStage * kCovStage;
    o.nchunk = (o.n + o.rows_per_chunk - 1) / o.rows_per_chunk;
    return o;
}

template <class Ws>
void oja_ws_layout(Ws &ws, const OjaGeom &o, int64_t R) {
    ws.template take<float>(static_cast<size_t>(o.G * o.np * kHeadDim));
    ws.template take<float>(static_cast<size_t>(o.LH * o.nchunk * kHeadDim * kHeadDim));
    ws.template take<double>(static_cast<size_t>(o.LH * kHeadDim * kHeadDim));
    ws.template take<double>(static_cast<size_t>(o.LH * kHeadDim * R));
    ws.template take<double>(static_cast<size_t>(o.LH * R * R));
}

kvc_status check_oja(const kvc_dims *d, int64_t pool) {
    if (!d || pool < 1) return KVC_ERR_INVALID_ARGUMENT;
    if (d->L < 0 || d->B <= 0 || d->H_kv <= 0 || d->S <= 0 || d->D <= 0 || d->R <= 0 || d->R > d->D)
        return KVC_ERR_INVALID_ARGUMENT;
    if (d->S_stride != 0 && d->S_stride < d->S) return KVC_ERR_INVALID_ARGUMENT;
    if (d->D != kHeadDim || !(d->R == 32 || d->R == 64 || d->R == 96 || d->R == 128))
        return KVC_ERR_UNSUPPORTED;
    if (d->S > INT32_MAX || pool > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    return KVC_OK;
}

}  // namespace

size_t oja_workspace_bytes(const kvc_dims *d, int64_t pool) {
    if (check_oja(d, pool) != KVC_OK) return 0;
    WsSizer sz;
    oja_ws_layout(sz, make_oja_geom(d, pool), d->R);
    return sz.bytes();
}

}  // namespace kvc

extern "C" kvc_status kvc_oja_update(const kvc_dims *d, float *U, const uint16_t *X, int32_t pool,
                                     float eta, void *ws, size_t ws_bytes, hipStream_t stream) {
    using namespace kvc;
    kvc_status st = check_oja(d, pool);
    if (st != KVC_OK) return st;
    if (!std::isfinite(eta)) return KVC_ERR_INVALID_ARGUMENT;
    const OjaGeom o = make_oja_geom(d, pool);
    if (o.G == 0) return KVC_OK;
    if (!U || !X || !ws || !aligned(U, 16) || !aligned(X, 16) || !aligned(ws, kWsAlign))
        return KVC_ERR_INVALID_ARGUMENT;
    WsSizer sz;
    oja_ws_layout(sz, o, d->R);
    if (ws_bytes < sz.bytes()) return KVC_ERR_WORKSPACE_TOO_SMALL;
    WsCursor cur(ws);
    float *Xp = cur.take<float>(static_cast<size_t>(o.G * o.np * kHeadDim));
    float *Cpart = cur.take<float>(static_cast<size_t>(o.LH * o.nchunk * kHeadDim * kHeadDim));
    double *C64 = cur.take<double>(static_cast<size_t>(o.LH * kHeadDim * kHeadDim));
    double *CU64 = cur.take<double>(static_cast<size_t>(o.LH * kHeadDim * d->R));
    double *M64 = cur.take<double>(static_cast<size_t>(o.LH * d->R * d->R));

    const int64_t rows = o.G * o.np;
    const int64_t pb = (rows + kPoolThreads / 16 - 1) / (kPoolThreads / 16);
    if (pb > INT32_MAX || o.LH * o.nchunk > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(pool_kernel, dim3(static_cast<unsigned>(pb)), dim3(kPoolThreads), 0, stream, X, rows,
                       o.N, o.S_stride, pool, o.np, Xp);
    hipLaunchKernelGGL(cov_partial_kernel, dim3(static_cast<unsigned>(o.LH * o.nchunk)), dim3(256), 0,
                       stream, Xp, d->B, d->H_kv, o.np, o.rows_per_chunk, o.nchunk, Cpart);
    if (d->R <= 64) {
        static std::atomic<bool> lds_ok[2][64];
        const void *fn = d->R == 32 ? reinterpret_cast<const void *>(&oja_step_qr_lds_kernel<32>)
                                    : reinterpret_cast<const void *>(&oja_step_qr_lds_kernel<64>);
        if (allow_large_lds(fn, lds_ok[d->R == 32 ? 0 : 1]) != KVC_OK) return KVC_ERR_HIP;
        const size_t lds = oja_lds_bytes(static_cast<int>(d->R));
        if (d->R == 32)
            hipLaunchKernelGGL(oja_step_qr_lds_kernel<32>, dim3(static_cast<unsigned>(o.LH)), dim3(256), lds,
                               stream, U, Cpart, o.nchunk, o.n, static_cast<double>(eta));
        else
            hipLaunchKernelGGL(oja_step_qr_lds_kernel<64>, dim3(static_cast<unsigned>(o.LH)), dim3(256), lds,
                               stream, U, Cpart, o.nchunk, o.n, static_cast<double>(eta));
        return launch_status();
    }
    const size_t lds = (static_cast<size_t>(kHeadDim) * (d->R + 1) + 2 * kHeadDim + 2) * sizeof(double);
    static std::atomic<bool> lds_ok[64];
    if (allow_large_lds(reinterpret_cast<const void *>(&oja_step_qr_kernel), lds_ok) != KVC_OK)
        return KVC_ERR_HIP;
    hipLaunchKernelGGL(oja_step_qr_kernel, dim3(static_cast<unsigned>(o.LH)), dim3(256), lds, stream, U,
                       Cpart, o.nchunk, o.n, static_cast<int>(d->R), static_cast<double>(eta), C64,
                       CU64, M64);
    return launch_status();
}
