// OjaKV hybrid low-rank path on MFMA ("OjaKV: Context-Aware Online Low-Rank KV
// Cache Compression", background on low-rank attention and method details):
//   compress:     K~ = K U_k, V~ = V U_v, and the query-weighted error score
//                 err_t = 1/|W| sum_q |q^T r_t| / sqrt(D), r_t = k_t - U U^T k_t;
//   reconstruct:  X^ = X~ U^T, then the full-rank anchor rows put back.
//
// Precision.  K, V and Q are bf16 and enter the bf16 MFMA exactly.  fp32
// operands (U, X~, the folded query matrix) are split as x = hi + lo with hi,
// lo bf16 (|x - hi - lo| <= 2^-17 |x|) and every product is accumulated in
// fp32 by v_mfma_f32_32x32x16_bf16, so the result carries ~2^-16 relative
// error instead of the 2^-8 of a plain bf16 rounding.
//
// Error score without materialising r_t.  Because (I - U U^T) is symmetric,
// q^T r_t = ((I - U U^T) q)^T k_t for any U.  A per-slice prep kernel forms
// Q'' = (Q_win (I - U U^T)) / (|W| sqrt(D)) once in fp64 and stores its hi/lo
// MFMA fragments; the streaming kernel then needs one contraction per token,
// err_t = sum_q |Q''_q . k_t|, fused with the projection on the same key tile.
//
// MFMA tiling (32x32x16, wave64): a wave owns 64 tokens (two 32-token column
// blocks) per step.  Key rows are the B operand: lane i loads 16 bytes of token
// (i % 32) at channel 16s + 8(i / 32) for k-step s, so each lane reads whole
// 256-byte rows over the 8 k-steps.  The A operands (U^T and Q'' fragments,
// hi and lo) sit in LDS as [fragment][lane][16 bytes], read conflict-free.
// Accumulator lane i, register r holds row 8(r/4) + 4(i/32) + r%4, column i%32,
// so four consecutive output features go out as one 16-byte store.
//
// Rank order of the reconstruction.  A sum over the rank may take the ranks in
// any order as long as both operands agree.  Reconstruction k-step ks gives
// operand element e of lane half h the rank 16ks + 8(e/4) + 4h + e%4: exactly the
// ranks that a projection accumulator lane already holds in registers 8(ks%2)..+7
// of its rank block, so the fused kernel feeds X~ to the reconstruction straight
// from the projection's accumulators, and the stand-alone reconstruction (which
// loads X~ in the same order) gives bit-identical X^.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFragBytes = 64 * 16;  // one MFMA operand fragment: 64 lanes x 8 bf16


__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// x (8 fp32) -> hi, lo (8 bf16 each, packed little-endian in 4 dwords)
__device__ __forceinline__ void split8(const float *x, u32x4 &hi, u32x4 &lo) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = f32_to_bf16_rne(x[e]);
        l[e] = f32_to_bf16_rne(x[e] - __uint_as_float(h[e] << 16));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        hi[q] = h[2 * q] | (h[2 * q + 1] << 16);
        lo[q] = l[2 * q] | (l[2 * q + 1] << 16);
    }
}

// rank carried by operand element e of lane half h at reconstruction k-step ks
__host__ __device__ constexpr int recon_rank(int ks, int h, int e) {
    return 16 * ks + 8 * (e >> 2) + 4 * h + (e & 3);
}

// Reconstruction B operand: U[c][rank] for channel block cb, hi/lo bf16 split,
// stored as [cb][ks][hi|lo][lane] fragments (lane = channel cb*32 + lane%32, half lane/32).
template <int R>
__device__ void stage_recon_u(const float *__restrict__ U, u32x4 *frag) {
    constexpr int KS = R / 16;
    for (int p = threadIdx.x; p < 4 * KS * 64; p += blockDim.x) {
        const int lane = p & 63, fs = p >> 6, ks = fs % KS, cb = fs / KS;
        const int c = cb * 32 + (lane & 31), h = lane >> 5;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = U[c * R + recon_rank(ks, h, e)];
        u32x4 hi, lo;
        split8(x, hi, lo);
        frag[((cb * KS + ks) * 2 + 0) * 64 + lane] = hi;
        frag[((cb * KS + ks) * 2 + 1) * 64 + lane] = lo;
    }
}

// One reconstruction k-step: X~ fragment x (token rows) times U fragment u
// (channel columns), D[token][channel].
__device__ __forceinline__ f32x16 recon_mfma(u32x4 x, u32x4 u, f32x16 c) { return mfma32x32x16(x, u, c); }

// Stores a 32-token x 32-channel block of X^ (tokens t0.., channels cb*32..):
// lane (col, khalf) holds channel cb*32 + col of tokens 8(j/4) + 4khalf + j%4, so
// each fp32 store covers two 128-byte row segments; bf16 pairs go out from the
// even lane.  (The transposed block, 16-byte pieces of 32 rows per store, was
// measured 20% slower for fp32 and 36% slower for bf16.)
template <typename OutT>
__device__ __forceinline__ void recon_store(OutT *xh, int64_t t0, int64_t t_end, int cb, int col, int khalf,
                                            const f32x16 &acc) {
    constexpr bool kBf16 = sizeof(OutT) == 2;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int64_t tj = t0 + (j >> 2) * 8 + khalf * 4 + (j & 3);
        if constexpr (kBf16) {
            const float nb = __shfl_xor(acc[j], 1);  // channel col ^ 1, same token
            if (!(col & 1) && tj < t_end)
                *reinterpret_cast<uint32_t *>(xh + tj * kHeadDim + cb * 32 + col) =
                    f32_to_bf16_rne(acc[j]) | (f32_to_bf16_rne(nb) << 16);
        } else {
            // 32 lanes write one whole 128-byte line of a row: streaming store
            if (tj < t_end) __builtin_nontemporal_store(acc[j], xh + tj * kHeadDim + cb * 32 + col);
        }
    }
}

// Whole-row stores of bf16 X^ through a per-wave LDS tile of ROWS rows x 256
// bytes.  The reconstruction block is taken transposed, D[channel][token] (lane
// (col, khalf) holds channels cb*32 + 8q + 4khalf .. +3 of token col), rounded to
// bf16 quads and written into the tile; the rows then leave as 16-byte pieces, 16
// lanes per 256-byte row and four rows per store.  Chunk c of row r sits at chunk
// position (c ^ r) mod 16, so both the column writes and the row reads spread over
// the banks without padding.  (Stored straight from the untransposed block, bf16
// rows go out in 64-byte halves of a cache line: 3.8 ms instead of 2.6 ms for
// 256 slices x 131072 tokens.)
template <int ROWS>
struct Bf16RowTile {
    static constexpr int kBytes = ROWS * 256;
    __device__ static int at(int r, int byte) { return r * 256 + ((((byte >> 4) ^ r) & 15) << 4) + (byte & 15); }
    // tokens row0 .. row0 + ROWS - 1 of channel block cb into the tile
    __device__ static void put(uint8_t *tile, int lane, int cb, int row0, const f32x16 &acc) {
        const int col = lane & 31, khalf = lane >> 5;
        const int r = col - row0;
        if (r < 0 || r >= ROWS) return;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint2 *>(tile + at(r, (cb * 32 + 8 * q + 4 * khalf) * 2)) =
                make_uint2(f32_to_bf16_rne(acc[4 * q]) | (f32_to_bf16_rne(acc[4 * q + 1]) << 16),
                           f32_to_bf16_rne(acc[4 * q + 2]) | (f32_to_bf16_rne(acc[4 * q + 3]) << 16));
    }
    // tile rows r -> X^ rows t0 + r (those below t_end); the wave's tile is free again after it
    __device__ static void flush(uint16_t *xh, int64_t t0, int64_t t_end, int lane, const uint8_t *tile) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int part = 0; part < ROWS / 4; ++part) {
            const int r = (lane >> 4) + 4 * part, c = lane & 15;
            const uint4 v = *reinterpret_cast<const uint4 *>(tile + r * 256 + (((c ^ r) & 15) << 4));
            const int64_t tok = t0 + r;
            if (tok < t_end) st_stream(reinterpret_cast<uint4 *>(xh + tok * kHeadDim + c * 8), v);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
};

struct Slices {
    int64_t B, Hkv, S, S_stride;
    int64_t nsplit;     // blocks per slice
    int64_t per_split;  // tokens per block (multiple of 64)
};

// ------------------------------------------------------------ compress prep

constexpr int kQParts = 3;  // bf16 terms per folded-query element (at most)

// Terms used for the folded query: three for small windows (a single |q . r_t|
// can cancel far below ||q|| ||r_t||: two terms missed the score tolerance at a
// one-query window), two once the score averages >= 32 products.
inline int query_terms(int64_t nq) { return nq < 32 ? 3 : 2; }

// Folded, scaled query fragments of one slice:
//   Q''[q][c] = scale * (Q[q][c] - sum_j T[q][j] U[c][j]),  T = Q U
// in fp64, split into three bf16 terms, as A-operand fragments
// [qb][s][term][lane].  Three terms keep the score's error at the level of
// the fp32 accumulation even when |q . r_t| cancels far below ||q|| ||r_t||.
constexpr int kPrepJ = 64;                  // basis columns per chunk of the prep
constexpr int kPrepQStride = kHeadDim + 2;  // bf16 row stride of the staged window
constexpr int kPrepStride = kPrepJ + 1;     // row stride of T and of the U chunk (in elements)
constexpr size_t kPrepLds = static_cast<size_t>(kHeadDim) * kPrepStride * sizeof(double) +
                            static_cast<size_t>(kHeadDim) * kPrepStride * sizeof(float) +
                            static_cast<size_t>(kHeadDim) * kPrepQStride * sizeof(uint16_t);

// fp64 matrix cores, v_mfma_f64_16x16x4f64: A[i][k] comes from lane i + 16k, B[k][j]
// from lane j + 16k, and element r of lane l receives D[l / 16 + 4r][l % 16].
typedef double f64x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// One workgroup of eight waves (two per SIMD) per slice; U is taken in chunks of 64
// columns and the window in NRB = 2 nqb 16-row blocks (rows past nq zero):
//   phase 1  T[q][j] = sum_c Q[q][c] U[c][j]    wave w: columns 16 (w % 4) .. + 15 of the
//                                               chunk, row blocks of half w / 4
//   phase 2  P[q][c] += sum_j T[q][j] U[c][j]   wave w: channels 16w .. 16w + 15, accumulated
//                                               over the chunks in registers
// then Q''[q][c] = scale * (Q[q][c] - P[q][c]), split into bf16 terms and stored
// two channels per 32-bit word in fragment order.  Every product is fp64 on the
// matrix cores (bf16 x fp32 products are exact in fp64); T goes through LDS in fp64.
// With fp64 FMAs on the vector units (a 4 x 4 register tile per thread, operands
// converted from LDS at every use) the same work took 0.34-0.37 ms at 1024 slices.
constexpr int kPrepThreads = 512;
template <int NRB>  // 16-row blocks of the window: 2 nqb (rows past nq are zero)
__global__ __launch_bounds__(kPrepThreads) void prep_query_kernel(const uint16_t *__restrict__ Q,
                                                                  const float *__restrict__ Uk, int64_t B,
                                                                  int64_t Hkv, int64_t Hq, int64_t Wq, int R,
                                                                  int nq, int nqb, int nterm, double scale,
                                                                  u32x4 *__restrict__ qfrag) {
    extern __shared__ double lds_prep[];
    double *Ts = lds_prep;                                                     // [128][65]
    float *Uc = reinterpret_cast<float *>(Ts + kHeadDim * kPrepStride);        // [128][65]
    uint16_t *Qs = reinterpret_cast<uint16_t *>(Uc + kHeadDim * kPrepStride);  // [128][130]
    const int tid = threadIdx.x;
    const int64_t slice = blockIdx.x;
    const int64_t h = slice % Hkv;
    const int64_t lb = slice / Hkv;  // l*B + b
    const int64_t l = lb / B;
    const int64_t grp = Hq / Hkv;
    const float *U = Uk + (l * Hkv + h) * kHeadDim * R;
    // window rows q = (group head) * Wq + (query); the group's heads are contiguous in Q
    const uint16_t *Qg = Q + ((lb * Hq + h * grp) * Wq) * kHeadDim;
    // staging: every thread issues all its 16-byte loads before storing any to LDS
    // (one 4-byte load at a time per thread left the prep waiting on memory latency)
    constexpr int kStageLoads = kHeadDim * kHeadDim / 8 / kPrepThreads;  // 16-byte pieces per thread
    {
        uint4 v[kStageLoads];
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int i = tid + u * kPrepThreads, q = i >> 4, c8 = i & 15;  // rows past nq are zero
            v[u] = q < nq ? reinterpret_cast<const uint4 *>(Qg + q * kHeadDim)[c8] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int i = tid + u * kPrepThreads, q = i >> 4, c8 = i & 15;
            uint32_t *row = reinterpret_cast<uint32_t *>(Qs + q * kPrepQStride) + 4 * c8;
            row[0] = v[u].x;
            row[1] = v[u].y;
            row[2] = v[u].z;
            row[3] = v[u].w;
        }
    }
    auto qval = [&](int q, int c) {
        return static_cast<double>(__uint_as_float(static_cast<uint32_t>(Qs[q * kPrepQStride + c]) << 16));
    };
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, kq = lane >> 4;
    constexpr int RB1 = NRB / 2;  // row blocks per wave in phase 1
    const int jb = wave & 3, r0 = (wave >> 2) * RB1;
    f64x4 pacc[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) pacc[rb] = f64x4{0.0, 0.0, 0.0, 0.0};

    for (int j0 = 0; j0 < R; j0 += kPrepJ) {
        const int jn = min(kPrepJ, R - j0);  // 32 or 64
        __syncthreads();                     // previous chunk's readers are done
        {
            const int n4 = jn / 4;  // 16-byte pieces per U row in the chunk
            float4 v[kStageLoads];
#pragma unroll
            for (int u = 0; u < kStageLoads; ++u) {
                const int i = tid + u * kPrepThreads, c = i / n4, j4 = i % n4;
                if (c < kHeadDim) v[u] = reinterpret_cast<const float4 *>(U + c * R + j0)[j4];
            }
#pragma unroll
            for (int u = 0; u < kStageLoads; ++u) {
                const int i = tid + u * kPrepThreads, c = i / n4, j4 = i % n4;
                if (c < kHeadDim) {
                    float *row = Uc + c * kPrepStride + 4 * j4;
                    row[0] = v[u].x;
                    row[1] = v[u].y;
                    row[2] = v[u].z;
                    row[3] = v[u].w;
                }
            }
        }
        __syncthreads();
        if (16 * jb < jn) {
            f64x4 tacc[RB1];
#pragma unroll
            for (int rb = 0; rb < RB1; ++rb) tacc[rb] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
            for (int c0 = 0; c0 < kHeadDim; c0 += 4) {
                const double b = static_cast<double>(Uc[(c0 + kq) * kPrepStride + 16 * jb + l16]);
                double a[RB1];
#pragma unroll
                for (int rb = 0; rb < RB1; ++rb) a[rb] = qval(16 * (r0 + rb) + l16, c0 + kq);
#pragma unroll
                for (int rb = 0; rb < RB1; ++rb) tacc[rb] = mfma_f64(a[rb], b, tacc[rb]);
            }
#pragma unroll
            for (int rb = 0; rb < RB1; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Ts[(16 * (r0 + rb) + kq + 4 * r) * kPrepStride + 16 * jb + l16] = tacc[rb][r];
        }
        __syncthreads();
#pragma unroll 2
        for (int j = 0; j < jn; j += 4) {
            double a[NRB];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) a[rb] = Ts[(16 * rb + l16) * kPrepStride + j + kq];
            const double b = static_cast<double>(Uc[(16 * wave + l16) * kPrepStride + j + kq]);
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) pacc[rb] = mfma_f64(a[rb], b, pacc[rb]);
        }
    }
    // Q'' in fragment order: lane (q % 32) + 32 * ((c / 8) % 2) of fragment (q / 32, c / 16)
    // holds channels 8 (c / 8) .. + 7 of query q (bf16 pairs per 32-bit word); queries
    // nq .. 32 nqb - 1 are zero.  Lanes l16 and l16 ^ 1 hold channels c and c ^ 1.
    uint32_t *out = reinterpret_cast<uint32_t *>(qfrag + slice * static_cast<int64_t>(nqb) * 8 * nterm * 64);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int q = 16 * rb + kq + 4 * r, c = 16 * wave + l16;
                double rest = q < nq ? scale * (qval(q, c) - pacc[rb][r]) : 0.0;
                uint32_t t[kQParts];
#pragma unroll
                for (int p = 0; p < kQParts; ++p) {
                    t[p] = f32_to_bf16_rne(static_cast<float>(rest));
                    rest -= static_cast<double>(__uint_as_float(t[p] << 16));
                }
                const int64_t word = (((q >> 5) * 8 + (c >> 4)) * nterm) * 64 + (q & 31) + 32 * ((c >> 3) & 1);
                for (int p = 0; p < nterm; ++p) {
                    const uint32_t nb = __shfl_xor(t[p], 1, 64);
                    if (!(l16 & 1)) out[(word + p * 64) * 4 + ((c & 7) >> 1)] = t[p] | (nb << 16);
                }
            }
    }
}

// --------------------------------------------------------------- compress

// One block per (slice, token range).  Each wave takes 32*HB tokens per step
// (HB column blocks of 32 tokens share every A fragment read from LDS).
// LDS: U^T fragments [rb][s][hi|lo] (NRB*16 KB), with kRebuild the
// reconstruction's U fragments [cb][ks][hi|lo] (NRB*16 KB), then Q'' fragments
// [qb][s][term] (nqb*8*nterm KB).  HB = 1 runs 16 waves per block (4 per SIMD),
// HB = 2 runs 8 waves with twice the reuse of each fragment.
//
// kRebuild also writes X^ = X~ U^T for every token (no anchors): the step's X~
// accumulators, split hi/lo (fp32 storage) or rounded to the stored bf16, are the
// A operand of the reconstruction in the rank order of recon_rank, so X~ is
// never read back from memory.
template <int NRB, int HB, bool kRowStores, bool kRebuild, typename OutT, int kStageRows = 0>
__global__ __launch_bounds__(HB == 1 ? 1024 : 512) void project_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ Ubase, const u32x4 *__restrict__ qfrag,
    int nqb, int nterm, Slices sl, OutT *__restrict__ Xt, float *__restrict__ err,
    OutT *__restrict__ Xh) {
    // OutT float: fp32 K~ rows; OutT uint16_t: bf16 K~ rows (round to nearest even)
    static_assert(!(kRowStores && kRebuild), "the fused reconstruction needs rank-major accumulators");
    constexpr bool kBf16 = sizeof(OutT) == 2;
    constexpr int R = 32 * NRB;
    constexpr int KS = R / 16;  // reconstruction k-steps
    constexpr int TOK = 32 * HB;
#ifndef KVC_FUSED_LATE_PREFETCH
#define KVC_FUSED_LATE_PREFETCH 0
#endif
    // The fused kernel's next keys: requested at the start of a step for fp32 storage
    // (256 VGPRs, 2 spilled; the loop's fused pass at S = 131072, five A/B pairs on two
    // boxes: 13.30-14.20 against 13.63-14.10 ms, mean 13.67 against 14.00, the early
    // request faster in four; requested after the projection it needs 194 VGPRs),
    // after the projection for bf16 storage (requested early its variants spill 11
    // and 26).  The same bits either way.
    constexpr bool kLatePrefetch = kRebuild && (kBf16 || KVC_FUSED_LATE_PREFETCH);
    extern __shared__ u32x4 lds[];
    u32x4 *ufr = lds;
    u32x4 *rfr = lds + NRB * 16 * 64;                            // reconstruction fragments
    u32x4 *qfr = lds + NRB * 16 * 64 * (kRebuild ? 2 : 1);       // after the U fragments

    const int64_t slice = blockIdx.x / sl.nsplit;
    const int64_t split = blockIdx.x % sl.nsplit;
    const int64_t h = slice % sl.Hkv;
    const int64_t l = slice / (sl.Hkv * sl.B);
    const float *U = Ubase + (l * sl.Hkv + h) * kHeadDim * R;

    for (int p = threadIdx.x; p < NRB * 8 * 64; p += blockDim.x) {
        const int lane = p & 63, fs = p >> 6, s = fs & 7, rb = fs >> 3;
        const int j = rb * 32 + (lane & 31);
        const int c0 = 16 * s + (lane >> 5) * 8;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = U[(c0 + e) * R + j];
        u32x4 hi, lo;
        split8(x, hi, lo);
        ufr[((rb * 8 + s) * 2 + 0) * 64 + lane] = hi;
        ufr[((rb * 8 + s) * 2 + 1) * 64 + lane] = lo;
    }
    if constexpr (kRebuild) stage_recon_u<R>(U, rfr);
    if (nqb > 0) {
        const int nq4 = nqb * 8 * nterm * 64;
        const u32x4 *src = qfrag + slice * static_cast<int64_t>(nq4);
        for (int p = threadIdx.x; p < nq4; p += blockDim.x) qfr[p] = src[p];
    }
    __syncthreads();

    const int64_t t_begin = split * sl.per_split;
    const int64_t t_end = min(sl.S, t_begin + sl.per_split);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, khalf = lane >> 5;
    const u32x4 *xrows = reinterpret_cast<const u32x4 *>(X + slice * sl.S_stride * kHeadDim);
    OutT *xt = Xt + slice * sl.S_stride * R;
    // Projection-only launches (no error score) write K~ rows in full 128-byte
    // segments; with the score fused, register pressure favours 16-byte pieces.
    constexpr bool row_stores = kRowStores;

    // key tile of a wave step: lane (col, khalf) holds 16 bytes of token t0+32hb+col
    // at channel 16s + 8khalf, s = 0..7 (B operand of the k-steps)
    auto load_b = [&](int64_t t0, u32x4 (&b)[HB][8]) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int64_t tok = t0 + hb * 32 + col;
            const bool ok = tok < t_end;
            const u32x4 *row = xrows + (ok ? tok : 0) * 16;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                b[hb][s] = row[2 * s + khalf];
                if (!ok) b[hb][s] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // error score of the step's tokens: err_t = sum over the folded queries of |Q''_q . k_t|
    // (the term count is a compile-time constant in each branch, so the fragment
    // loads of a step are issued together; with a run-time bound every pair of
    // MFMAs waited on its own LDS read: K side 3.80 -> 3.71 ms at 1024 x 32768)
    auto score_step = [&](int64_t t0, const u32x4 (&b)[HB][8]) {
        float e[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) e[hb] = 0.f;
        auto terms = [&](auto nt) {
            const int NT = nt;
#pragma unroll 1
            for (int qb = 0; qb < nqb; ++qb) {
                f32x16 a[HB];
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) a[hb] = f32x16{};
#pragma unroll
                for (int s = 0; s < 8; ++s) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const u32x4 f = qfr[((qb * 8 + s) * NT + t) * 64 + lane];
#pragma unroll
                        for (int hb = 0; hb < HB; ++hb) a[hb] = mfma32x32x16(f, b[hb][s], a[hb]);
                    }
                }
#pragma unroll
                for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) e[hb] += fabsf(a[hb][r]);
            }
        };
        // (the bf16 fused variant with the 16-row tile would spill with the two
        // specialised copies; it keeps the run-time loop)
        if constexpr (kBf16 && kRebuild && kStageRows == 16) {
            terms(nterm);
        } else {
            if (nterm == 2) terms(std::integral_constant<int, 2>{});
            else terms(std::integral_constant<int, 3>{});
        }
        float *er = err + slice * sl.S_stride;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            e[hb] += __shfl_xor(e[hb], 32);
            if (khalf == 0 && t0 + hb * 32 + col < t_end) er[t0 + hb * 32 + col] = e[hb];
        }
    };
    const int64_t wstep = (blockDim.x / 64) * TOK;
    // Score launches without the fused reconstruction keep two steps of keys in
    // flight at ranks 64 and 96 (254 / 250 VGPRs, no spills; the other ranks would
    // spill): the error-score MFMAs otherwise leave the memory pipe idle (K side
    // 4.1-4.4 -> 3.95-4.05 ms at 1024 slices x 32768, r = 64).
    // bf16 compression without the reconstruction: the step's 64 K~ rows go through
    // a per-wave tile of 64 rows x 2R bytes and leave whole (16-byte chunk c of row
    // r at position c ^ r); stored as 8-byte pieces they were 16-byte segments
    constexpr bool kStageKt = kBf16 && !kRebuild && kStageRows == 64;
    // fp32 compression with the score: one 32-token column block at a time, its K~
    // rows (4R bytes) through a per-wave tile of 32 rows and out whole
    constexpr bool kStageKtF = !kBf16 && !kRebuild && kStageRows == 32;
    constexpr int kFRowB = 4 * R, kFChunks = R / 4;
    constexpr bool kDepth2 = !kRebuild && !kRowStores && !kStageKt && !kStageKtF && (NRB == 2 || NRB == 3);

    constexpr int kKtRowB = 2 * R, kKtChunks = R / 8;
    auto kt_at = [](int r, int byte) {
        return r * kKtRowB + ((((byte >> 4) ^ r) & (kKtChunks - 1)) << 4) + (byte & 15);
    };
    uint8_t *kt_tile = reinterpret_cast<uint8_t *>(qfr + nqb * 8 * nterm * 64) + wave * 64 * kKtRowB;
    u32x4 b[HB][8], bn[HB][8], bnn[kDepth2 ? HB : 1][8];
    // X~ of the step as reconstruction operands: [k-step][hb][hi|lo]
    u32x4 xf[kRebuild ? KS : 1][HB][2];
    if (t_begin + wave * TOK < t_end) load_b(t_begin + wave * TOK, b);
    if (kDepth2 && t_begin + wave * TOK + wstep < t_end) load_b(t_begin + wave * TOK + wstep, bn);
    for (int64_t t0 = t_begin + wave * TOK; t0 < t_end; t0 += wstep) {
        // the next step's keys are requested before this step's contractions (fused:
        // once the projection is done, which keeps fewer registers live)
        if constexpr (kDepth2) {
            if (t0 + 2 * wstep < t_end) load_b(t0 + 2 * wstep, bnn);
        } else {
            if (!kLatePrefetch && t0 + wstep < t_end) load_b(t0 + wstep, bn);
        }
        // fused: the score first, so that the keys are dead once the projection
        // has built the X~ fragments (fewer registers live at once)
        if (kRebuild && nqb > 0) score_step(t0, b);
        if constexpr (kStageKtF) {
            uint8_t *tile = reinterpret_cast<uint8_t *>(qfr + nqb * 8 * nterm * 64) + wave * 32 * kFRowB;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
#pragma unroll 1
                for (int rb = 0; rb < NRB; ++rb) {
                    f32x16 acc = {};
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const u32x4 fh = ufr[((rb * 8 + s) * 2 + 0) * 64 + lane];
                        const u32x4 fl = ufr[((rb * 8 + s) * 2 + 1) * 64 + lane];
                        acc = mfma32x32x16(fh, b[hb][s], acc);  // same products and order as below
                        acc = mfma32x32x16(fl, b[hb][s], acc);
                    }
                    // lane (col, khalf): ranks rb*32 + 8q + 4khalf .. +3 of token col
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int byte = (rb * 32 + 8 * q + 4 * khalf) * 4;
                        *reinterpret_cast<float4 *>(tile + col * kFRowB + ((((byte >> 4) ^ col) & (kFChunks - 1)) << 4)) =
                            make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int part = 0; part < kFChunks / 2; ++part) {
                    const int r = lane / kFChunks + (64 / kFChunks) * part, c = lane % kFChunks;
                    const float4 v =
                        *reinterpret_cast<const float4 *>(tile + r * kFRowB + (((c ^ r) & (kFChunks - 1)) << 4));
                    const int64_t tok = t0 + hb * 32 + r;
                    if (tok < t_end) st_stream(reinterpret_cast<float4 *>(xt + tok * R + c * 4), v);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
#pragma unroll 1
        for (int rb = 0; rb < (kStageKtF ? 0 : NRB); ++rb) {
            f32x16 a[HB];
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) a[hb] = f32x16{};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const u32x4 fh = ufr[((rb * 8 + s) * 2 + 0) * 64 + lane];
                const u32x4 fl = ufr[((rb * 8 + s) * 2 + 1) * 64 + lane];
                if constexpr (row_stores) {
                    // keys as the A operand (same registers): D[token][rank]
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) a[hb] = mfma32x32x16(b[hb][s], fh, a[hb]);
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) a[hb] = mfma32x32x16(b[hb][s], fl, a[hb]);
                } else {
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) a[hb] = mfma32x32x16(fh, b[hb][s], a[hb]);
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) a[hb] = mfma32x32x16(fl, b[hb][s], a[hb]);
                }
            }
            if constexpr (row_stores) {
                // lane (col, khalf) holds rank rb*32+col of tokens 8(j/4) + 4khalf + j%4:
                // each store writes two 128-byte (fp32) or 64-byte (bf16 pairs) row segments
#pragma unroll
                for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int64_t tok = t0 + hb * 32 + (j >> 2) * 8 + khalf * 4 + (j & 3);
                        if constexpr (kBf16) {
                            const float nb = __shfl_xor(a[hb][j], 1);  // rank col ^ 1, same token
                            if (!(col & 1) && tok < t_end)
                                *reinterpret_cast<uint32_t *>(xt + tok * R + rb * 32 + col) =
                                    f32_to_bf16_rne(a[hb][j]) | (f32_to_bf16_rne(nb) << 16);
                        } else {
                            if (tok < t_end) xt[tok * R + rb * 32 + col] = a[hb][j];
                        }
                    }
            } else {
                if constexpr (kStageKt) {
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<uint2 *>(kt_tile +
                                                       kt_at(hb * 32 + col, (rb * 32 + 8 * q + 4 * khalf) * 2)) =
                                make_uint2(f32_to_bf16_rne(a[hb][4 * q]) | (f32_to_bf16_rne(a[hb][4 * q + 1]) << 16),
                                           f32_to_bf16_rne(a[hb][4 * q + 2]) | (f32_to_bf16_rne(a[hb][4 * q + 3]) << 16));
                }
                if constexpr (kRebuild) {
                    // registers 8sp..8sp+7 hold ranks recon_rank(2rb + sp, khalf, 0..7);
                    // the loop stays rolled (fewer live fragments), so the rank block
                    // picks its registers by a uniform branch
                    auto keep = [&](auto rbc) {
                        constexpr int kb = decltype(rbc)::value;
#pragma unroll
                        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                            for (int sp = 0; sp < 2; ++sp) {
                                float x[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e) x[e] = a[hb][8 * sp + e];
                                split8(x, xf[2 * kb + sp][hb][0], xf[2 * kb + sp][hb][1]);
                            }
                    };
                    if (rb == 0) keep(std::integral_constant<int, 0>{});
                    if constexpr (NRB > 1) {
                        if (rb == 1) keep(std::integral_constant<int, 1>{});
                    }
                }
                // lane (col, khalf) holds ranks rb*32 + 8q + 4khalf .. +4 of token col
                // (staged bf16 launches write whole K~ rows from a tile instead)
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
                    const int64_t tok = t0 + hb * 32 + col;
                    constexpr bool kPieces = kStageRows == 0 || (kStageRows == 16 && kRebuild);
                    if (kPieces && tok < t_end) {
                        OutT *dst = xt + tok * R + rb * 32 + khalf * 4;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if constexpr (kBf16) {
                                *reinterpret_cast<uint2 *>(dst + q * 8) = make_uint2(
                                    f32_to_bf16_rne(a[hb][4 * q]) | (f32_to_bf16_rne(a[hb][4 * q + 1]) << 16),
                                    f32_to_bf16_rne(a[hb][4 * q + 2]) | (f32_to_bf16_rne(a[hb][4 * q + 3]) << 16));
                            } else {
                                *reinterpret_cast<float4 *>(dst + q * 8) = make_float4(
                                    a[hb][4 * q], a[hb][4 * q + 1], a[hb][4 * q + 2], a[hb][4 * q + 3]);
                            }
                        }
                    }
                }
            }
        }
        if constexpr (kStageKt) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int part = 0; part < kKtChunks; ++part) {
                const int r = lane / kKtChunks + (64 / kKtChunks) * part, c = lane % kKtChunks;
                const uint4 v =
                    *reinterpret_cast<const uint4 *>(kt_tile + r * kKtRowB + (((c ^ r) & (kKtChunks - 1)) << 4));
                const int64_t tok = t0 + r;  // row hb*32 + col is token t0 + hb*32 + col
                if (tok < t_end) st_stream(reinterpret_cast<uint4 *>(xt + tok * R + c * 8), v);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (!kRebuild && nqb > 0) score_step(t0, b);
        if constexpr (kBf16 && kStageRows == 32) {
            // bf16 K~ of each 32-token column block from its fragments (the stored
            // values exactly: ranks recon_rank(ks, khalf, 0..7) of token col) through
            // the wave's tile as whole 2R-byte rows; chunk c of row r sits at c ^ r
            constexpr int kRowB = 2 * R, kChunks = R / 8;
            uint8_t *tile = reinterpret_cast<uint8_t *>(qfr + nqb * 8 * nterm * 64) + wave * Bf16RowTile<32>::kBytes;
            auto at = [](int r, int byte) {
                return r * kRowB + ((((byte >> 4) ^ r) & (kChunks - 1)) << 4) + (byte & 15);
            };
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const u32x4 f = xf[ks][hb][0];
                    *reinterpret_cast<uint2 *>(tile + at(col, (16 * ks + 4 * khalf) * 2)) = make_uint2(f[0], f[1]);
                    *reinterpret_cast<uint2 *>(tile + at(col, (16 * ks + 8 + 4 * khalf) * 2)) = make_uint2(f[2], f[3]);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int part = 0; part < 32 * kChunks / 64; ++part) {
                    const int r = lane / kChunks + (64 / kChunks) * part, c = lane % kChunks;
                    const uint4 v = *reinterpret_cast<const uint4 *>(tile + r * kRowB + (((c ^ r) & (kChunks - 1)) << 4));
                    const int64_t tok = t0 + hb * 32 + r;
                    if (tok < t_end) st_stream(reinterpret_cast<uint4 *>(xt + tok * R + c * 8), v);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
        // (a scheduling fence keeps the prefetch's registers out of the phases above)
        if constexpr (kLatePrefetch) __builtin_amdgcn_sched_barrier(0);
        if (kLatePrefetch && t0 + wstep < t_end) load_b(t0 + wstep, bn);
        if constexpr (kRebuild) {
            // X^[t][c] for channel block cb: hi*hi + hi*lo + lo*hi (fp32 X~), or the
            // stored bf16 X~ times U hi and lo
            OutT *xh = Xh + slice * sl.S_stride * kHeadDim;
            if constexpr (kBf16 && kStageRows == 32) {
                // bf16: each 32-token column block, transposed, leaves as whole rows
                // through the wave's 32-row tile (after the Q'' fragments)
                uint8_t *tile = reinterpret_cast<uint8_t *>(qfr + nqb * 8 * nterm * 64) +
                                wave * Bf16RowTile<32>::kBytes;
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
#pragma unroll 1
                    for (int cb = 0; cb < 4; ++cb) {
                        f32x16 acc = {};
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            const u32x4 uh = rfr[((cb * KS + ks) * 2 + 0) * 64 + lane];
                            const u32x4 ul = rfr[((cb * KS + ks) * 2 + 1) * 64 + lane];
                            acc = mfma32x32x16(uh, xf[ks][hb][0], acc);  // D[channel][token]
                            acc = mfma32x32x16(ul, xf[ks][hb][0], acc);
                        }
                        Bf16RowTile<32>::put(tile, lane, cb, 0, acc);
                    }
                    Bf16RowTile<32>::flush(xh, t0 + hb * 32, t_end, lane, tile);
                }
            } else if constexpr (kBf16) {
                // where LDS is short (the score's fragments): a 16-row tile, the four
                // channel blocks of a column block held in registers, 16 tokens at a
                // time (computing each block once per half instead was slower: the
                // K side at r = 64 went 5.97 -> 6.25 ms)
                uint8_t *tile = reinterpret_cast<uint8_t *>(qfr + nqb * 8 * nterm * 64) +
                                wave * Bf16RowTile<16>::kBytes;
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
                    f32x16 acc[4];
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) {
                        acc[cb] = f32x16{};
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            const u32x4 uh = rfr[((cb * KS + ks) * 2 + 0) * 64 + lane];
                            const u32x4 ul = rfr[((cb * KS + ks) * 2 + 1) * 64 + lane];
                            acc[cb] = mfma32x32x16(uh, xf[ks][hb][0], acc[cb]);  // D[channel][token]
                            acc[cb] = mfma32x32x16(ul, xf[ks][hb][0], acc[cb]);
                        }
                    }
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
#pragma unroll
                        for (int cb = 0; cb < 4; ++cb) Bf16RowTile<16>::put(tile, lane, cb, 16 * half, acc[cb]);
                        Bf16RowTile<16>::flush(xh, t0 + hb * 32 + 16 * half, t_end, lane, tile);
                    }
                }
            } else {
#pragma unroll 1
            for (int cb = 0; cb < 4; ++cb) {
                f32x16 acc[HB];
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const u32x4 uh = rfr[((cb * KS + ks) * 2 + 0) * 64 + lane];
                    const u32x4 ul = rfr[((cb * KS + ks) * 2 + 1) * 64 + lane];
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) {
                        acc[hb] = recon_mfma(xf[ks][hb][0], uh, acc[hb]);
                        acc[hb] = recon_mfma(xf[ks][hb][0], ul, acc[hb]);
                        if constexpr (!kBf16) acc[hb] = recon_mfma(xf[ks][hb][1], uh, acc[hb]);
                    }
                }
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) recon_store(xh, t0 + hb * 32, t_end, cb, col, khalf, acc[hb]);
            }
            }
        }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                b[hb][s] = bn[hb][s];
                if constexpr (kDepth2) bn[hb][s] = bnn[hb][s];
            }
    }
}

// ------------------------------------------------------------- reconstruct

// One block per (slice, token range); 4 waves; each wave 32 tokens per step.
// X^[t][c] = sum_j X~[t][j] U[c][j]: A = X~ split hi/lo in registers, B = U
// (channel columns, hi/lo in LDS), ranks in the reconstruction order;
// hi*hi + hi*lo + lo*hi.
template <int NRB>
__global__ __launch_bounds__(256) void reconstruct_kernel(const float *__restrict__ Xt,
                                                          const float *__restrict__ Ubase,
                                                          Slices sl, float *__restrict__ Xh) {
    constexpr int R = 32 * NRB;
    constexpr int KS = R / 16;  // k-steps
    __shared__ u32x4 ufr[4 * KS * 2 * 64];

    const int64_t slice = blockIdx.x / sl.nsplit;
    const int64_t split = blockIdx.x % sl.nsplit;
    const int64_t h = slice % sl.Hkv;
    const int64_t l = slice / (sl.Hkv * sl.B);
    const float *U = Ubase + (l * sl.Hkv + h) * kHeadDim * R;

    stage_recon_u<R>(U, ufr);
    __syncthreads();

    const int64_t t_begin = split * sl.per_split;
    const int64_t t_end = min(sl.S, t_begin + sl.per_split);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, khalf = lane >> 5;
    const float *xt = Xt + slice * sl.S_stride * R;
    float *xh = Xh + slice * sl.S_stride * kHeadDim;

    // X~ rows of a wave step: lane (col, khalf) holds ranks recon_rank(s, khalf, 0..7)
    // of token t0 + col (two 16-byte pieces), split hi/lo once the step's data is in hand
    const int64_t wstep = (blockDim.x / 64) * 32;
    float4 xc[2 * KS], xn[2 * KS];
#define KVC_LOAD_X(T0, DST)                                                                      \
    do {                                                                                          \
        const int64_t tok_ = (T0) + col;                                                          \
        const bool ok_ = tok_ < t_end;                                                            \
        const float4 *src_ = reinterpret_cast<const float4 *>(xt + (ok_ ? tok_ : 0) * R + khalf * 4); \
        _Pragma("unroll") for (int s_ = 0; s_ < 2 * KS; ++s_) {                                   \
            DST[s_] = src_[(s_ >> 1) * 4 + (s_ & 1) * 2];                                         \
            if (!ok_) DST[s_] = make_float4(0.f, 0.f, 0.f, 0.f);                                  \
        }                                                                                         \
    } while (0)
    if (t_begin + wave * 32 < t_end) KVC_LOAD_X(t_begin + wave * 32, xc);
    for (int64_t t0 = t_begin + wave * 32; t0 < t_end; t0 += wstep) {
        if (t0 + wstep < t_end) KVC_LOAD_X(t0 + wstep, xn);  // next step in flight
        u32x4 bh[KS], bl[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float x[8];
            x[0] = xc[2 * s].x; x[1] = xc[2 * s].y; x[2] = xc[2 * s].z; x[3] = xc[2 * s].w;
            x[4] = xc[2 * s + 1].x; x[5] = xc[2 * s + 1].y; x[6] = xc[2 * s + 1].z; x[7] = xc[2 * s + 1].w;
            split8(x, bh[s], bl[s]);
        }
#pragma unroll 1
        for (int cb = 0; cb < 4; ++cb) {
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 ah = ufr[((cb * KS + s) * 2 + 0) * 64 + lane];
                const u32x4 al = ufr[((cb * KS + s) * 2 + 1) * 64 + lane];
                acc = recon_mfma(bh[s], ah, acc);
                acc = recon_mfma(bh[s], al, acc);
                acc = recon_mfma(bl[s], ah, acc);
            }
            recon_store(xh, t0, t_end, cb, col, khalf, acc);
        }
#pragma unroll
        for (int s = 0; s < 2 * KS; ++s) xc[s] = xn[s];
    }
#undef KVC_LOAD_X
}

// bf16 storage of the compressed cache: X~ bf16 rows are the MFMA operand as they
// are (exact, no split), U hi/lo from LDS (two products), X^ rounded to bf16
// (nearest even).  Same tiling as reconstruct_kernel, with the block taken
// transposed and a wave step's 32 rows stored whole through Bf16RowTile.
template <int NRB>
__global__ __launch_bounds__(256) void reconstruct_bf16_kernel(const uint16_t *__restrict__ Xt,
                                                               const float *__restrict__ Ubase,
                                                               Slices sl, uint16_t *__restrict__ Xh) {
    constexpr int R = 32 * NRB;
    constexpr int KS = R / 16;  // k-steps
    __shared__ u32x4 ufr[4 * KS * 2 * 64];
    __shared__ __attribute__((aligned(16))) uint8_t stile[4][Bf16RowTile<32>::kBytes];

    const int64_t slice = blockIdx.x / sl.nsplit;
    const int64_t split = blockIdx.x % sl.nsplit;
    const int64_t h = slice % sl.Hkv;
    const int64_t l = slice / (sl.Hkv * sl.B);
    const float *U = Ubase + (l * sl.Hkv + h) * kHeadDim * R;

    stage_recon_u<R>(U, ufr);
    __syncthreads();

    const int64_t t_begin = split * sl.per_split;
    const int64_t t_end = min(sl.S, t_begin + sl.per_split);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, khalf = lane >> 5;
    const uint16_t *xt = Xt + slice * sl.S_stride * R;
    uint16_t *xh = Xh + slice * sl.S_stride * kHeadDim;

    // lane (col, khalf) holds ranks recon_rank(s, khalf, 0..7) of token t0 + col: two 8-byte loads per k-step
    const int64_t wstep = (blockDim.x / 64) * 32;
    u32x4 xc[KS], xn[KS];
#define KVC_LOAD_XB(T0, DST)                                                                     \
    do {                                                                                          \
        const int64_t tok_ = (T0) + col;                                                          \
        const bool ok_ = tok_ < t_end;                                                            \
        const uint2 *src_ = reinterpret_cast<const uint2 *>(xt + (ok_ ? tok_ : 0) * R + khalf * 4); \
        _Pragma("unroll") for (int s_ = 0; s_ < KS; ++s_) {                                       \
            const uint2 p0_ = src_[4 * s_], p1_ = src_[4 * s_ + 2];                               \
            DST[s_] = u32x4{p0_.x, p0_.y, p1_.x, p1_.y};                                          \
            if (!ok_) DST[s_] = u32x4{0u, 0u, 0u, 0u};                                            \
        }                                                                                         \
    } while (0)
    if (t_begin + wave * 32 < t_end) KVC_LOAD_XB(t_begin + wave * 32, xc);
    for (int64_t t0 = t_begin + wave * 32; t0 < t_end; t0 += wstep) {
        if (t0 + wstep < t_end) KVC_LOAD_XB(t0 + wstep, xn);  // next step in flight
#pragma unroll 1
        for (int cb = 0; cb < 4; ++cb) {
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 ah = ufr[((cb * KS + s) * 2 + 0) * 64 + lane];
                const u32x4 al = ufr[((cb * KS + s) * 2 + 1) * 64 + lane];
                acc = mfma32x32x16(ah, xc[s], acc);  // D[channel][token]: same products and order
                acc = mfma32x32x16(al, xc[s], acc);
            }
            Bf16RowTile<32>::put(stile[wave], lane, cb, 0, acc);
        }
        Bf16RowTile<32>::flush(xh, t0, t_end, lane, stile[wave]);
#pragma unroll
        for (int s = 0; s < KS; ++s) xc[s] = xn[s];
    }
#undef KVC_LOAD_XB
}

// Row kernels (anchor rows): one wave per workgroup, 16 lanes per 256-byte row; many
// small workgroups move rows fastest (as measured for the compaction gather).
constexpr int kRowThreads = 64;
constexpr int kRowsPerBlock = kRowThreads / 16;

// Anchor rows of a bf16 X^: a bit-exact copy, 16 lanes per row.
__global__ __launch_bounds__(kRowThreads) void anchor_copy_bf16_kernel(const int32_t *__restrict__ idx,
                                                               const uint16_t *__restrict__ rows,
                                                               int64_t k, int64_t blocks_per_slice,
                                                               int64_t S, int64_t S_stride,
                                                               uint16_t *__restrict__ Xh) {
    const int64_t g = blockIdx.x / blocks_per_slice;
    const int64_t i = (blockIdx.x % blocks_per_slice) * kRowsPerBlock + (threadIdx.x >> 4);
    const int lane16 = threadIdx.x & 15;
    if (i >= k) return;
    const int64_t t = idx[g * k + i];
    if (t < 0 || t >= S) return;  // documented precondition; never write outside the slice
    // whole rows per 16 lanes, touched once: streaming load and store
    st_stream(reinterpret_cast<uint4 *>(Xh + (g * S_stride + t) * kHeadDim) + lane16,
              ld_stream(reinterpret_cast<const uint4 *>(rows + (g * k + i) * kHeadDim) + lane16));
}

// Anchor rows back into X^: 16 lanes per row, bf16 widened exactly.
__global__ __launch_bounds__(kRowThreads) void anchor_scatter_kernel(const int32_t *__restrict__ idx,
                                                             const uint16_t *__restrict__ rows,
                                                             int64_t k, int64_t blocks_per_slice,
                                                             int64_t S, int64_t S_stride,
                                                             float *__restrict__ Xh) {
    const int64_t g = blockIdx.x / blocks_per_slice;
    const int64_t i = (blockIdx.x % blocks_per_slice) * kRowsPerBlock + (threadIdx.x >> 4);
    const int lane16 = threadIdx.x & 15;
    if (i >= k) return;
    const int64_t t = idx[g * k + i];
    if (t < 0 || t >= S) return;  // documented precondition; never write outside the slice
    // lane l16 takes channels 4 l16 .. + 3 and 64 + 4 l16 .. + 3, so each load covers a
    // contiguous 128-byte line of the bf16 row and each store 256 contiguous bytes of the
    // fp32 row (streaming: the rows are touched once)
    const uint2 *src = reinterpret_cast<const uint2 *>(rows + (g * k + i) * kHeadDim);
    const uint2 v0 = src[lane16], v1 = src[16 + lane16];
    float4 *dst = reinterpret_cast<float4 *>(Xh + (g * S_stride + t) * kHeadDim);
    st_stream(dst + lane16, make_float4(bf16_lo(v0.x), bf16_hi(v0.x), bf16_lo(v0.y), bf16_hi(v0.y)));
    st_stream(dst + 16 + lane16, make_float4(bf16_lo(v1.x), bf16_hi(v1.x), bf16_lo(v1.y), bf16_hi(v1.y)));
}

// ------------------------------------------------------------------- host

bool rank_ok(int64_t R) { return R == 32 || R == 64 || R == 96 || R == 128; }

kvc_status check_dims(const kvc_dims *d, bool need_q) {
    if (!d) return KVC_ERR_INVALID_ARGUMENT;
    if (d->L < 0 || d->B < 0 || d->H_kv <= 0 || d->S < 0 || d->D <= 0 || d->R <= 0)
        return KVC_ERR_INVALID_ARGUMENT;
    if (d->S_stride != 0 && d->S_stride < d->S) return KVC_ERR_INVALID_ARGUMENT;
    if (need_q && (d->H_q <= 0 || d->W_q <= 0 || d->H_q % d->H_kv != 0))
        return KVC_ERR_INVALID_ARGUMENT;
    if (d->R > d->D) return KVC_ERR_INVALID_ARGUMENT;
    if (d->D != kHeadDim || !rank_ok(d->R)) return KVC_ERR_UNSUPPORTED;
    if (need_q && (d->H_q / d->H_kv) * d->W_q > 128) return KVC_ERR_UNSUPPORTED;
    if (d->S > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    return KVC_OK;
}

int64_t stride_of(const kvc_dims *d) { return d->S_stride ? d->S_stride : d->S; }

Slices make_slices(const kvc_dims *d, int64_t tokens_per_step) {
    Slices sl;
    sl.B = d->B;
    sl.Hkv = d->H_kv;
    sl.S = d->S;
    sl.S_stride = stride_of(d);
    const int64_t G = d->L * d->B * d->H_kv;
    // aim at >= 1024 blocks in flight, never below one step of tokens per block
    int64_t nsplit = G > 0 ? (1024 + G - 1) / G : 1;
    const int64_t max_split = (d->S + tokens_per_step - 1) / tokens_per_step;
    if (nsplit > max_split) nsplit = max_split;
    if (nsplit < 1) nsplit = 1;
    int64_t per = (d->S + nsplit - 1) / nsplit;
    per = (per + 63) / 64 * 64;
    sl.nsplit = nsplit;
    sl.per_split = per > 0 ? per : 64;
    return sl;
}

template <class Ws>
void compress_ws_layout(Ws &ws, const kvc_dims *d, bool with_q) {
    if (with_q) {
        const int64_t G = d->L * d->B * d->H_kv;
        const int64_t nq = (d->H_q / d->H_kv) * d->W_q;
        const int64_t nqb = (nq + 31) / 32;
        ws.template take<u32x4>(static_cast<size_t>(G * nqb * 8 * query_terms(nq) * 64));
    }
}

#ifndef KVC_PROJECT_HB
#define KVC_PROJECT_HB 2
#endif
// LDS of a projection launch; the fused bf16 reconstruction adds a staging tile
// of stage_rows x 256 bytes per wave after the fragments
constexpr int kProjectWaves = KVC_PROJECT_HB == 1 ? 16 : 8;
size_t project_lds(int NRB, bool rebuild, int nqb, int nterm, int stage_rows) {
    // rebuild: stage_rows x 256-byte rows of X^; otherwise (bf16 K~ staging, 64):
    // 64 rows x 2R bytes
    // (bf16 K~ staging: 64 rows x 2R bytes; fp32 K~ staging: 32 rows x 4R bytes)
    const size_t per_wave = rebuild ? static_cast<size_t>(stage_rows) * 256
                                    : static_cast<size_t>(stage_rows) * (stage_rows == 64 ? 2 : 4) * 32 * NRB;
    return static_cast<size_t>(NRB * 16 * (rebuild ? 2 : 1) + nqb * 8 * nterm) * kFragBytes +
           static_cast<size_t>(kProjectWaves) * per_wave;
}

// The fused reconstruction keeps all of a step's X~ fragments in registers
// (ranks <= 64) and both U fragment sets in LDS; bf16 also needs a staging tile
// of at least 16 rows per wave.
constexpr size_t kMaxLds = 160 * 1024;
bool rebuild_fusable(int64_t R, int nqb, int nterm, bool bf16) {
    return R <= 64 && project_lds(static_cast<int>(R / 32), true, nqb, nterm, bf16 ? 16 : 0) <= kMaxLds;
}

template <int NRB, bool kRowStores, bool kRebuild, typename OutT, int kStageRows = 0>
kvc_status launch_project_variant(const uint16_t *X, const float *U, const u32x4 *qfrag, int nqb,
                                  int nterm, const Slices &sl, int64_t G, OutT *Xt, float *err,
                                  OutT *Xh, hipStream_t stream) {
    constexpr int HB = KVC_PROJECT_HB;
    const size_t lds = project_lds(NRB, kRebuild, nqb, nterm, kStageRows);
    static std::atomic<bool> lds_ok[64];
    if (allow_large_lds(
            reinterpret_cast<const void *>(&project_kernel<NRB, HB, kRowStores, kRebuild, OutT, kStageRows>),
            lds_ok) != KVC_OK)
        return KVC_ERR_HIP;
    const int64_t blocks = G * sl.nsplit;
    if (blocks > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((project_kernel<NRB, HB, kRowStores, kRebuild, OutT, kStageRows>),
                       dim3(static_cast<unsigned>(blocks)), dim3(HB == 1 ? 1024 : 512), lds, stream, X, U, qfrag,
                       nqb, nterm, sl, Xt, err, Xh);
    return launch_status();
}

// Xh != nullptr: fused reconstruction (only called when rebuild_fusable); bf16
// stages whole rows through a 32-row tile per wave where LDS allows, else 16 rows
template <int NRB, typename OutT>
kvc_status launch_project(const uint16_t *X, const float *U, const u32x4 *qfrag, int nqb,
                          int nterm, const Slices &sl, int64_t G, OutT *Xt, float *err,
                          OutT *Xh, hipStream_t stream) {
    if constexpr (NRB <= 2) {
        if (Xh) {
            if constexpr (sizeof(OutT) == 2) {
                // rank 32 fits the 32-row tile at every window size (<= 160 KB)
                if (NRB == 1 || project_lds(NRB, true, nqb, nterm, 32) <= kMaxLds)
                    return launch_project_variant<NRB, false, true, OutT, 32>(X, U, qfrag, nqb, nterm, sl, G, Xt,
                                                                              err, Xh, stream);
                if constexpr (NRB == 2)
                    return launch_project_variant<NRB, false, true, OutT, 16>(X, U, qfrag, nqb, nterm, sl, G, Xt,
                                                                              err, Xh, stream);
                return KVC_ERR_UNSUPPORTED;
            } else {
                return launch_project_variant<NRB, false, true>(X, U, qfrag, nqb, nterm, sl, G, Xt, err, Xh,
                                                                stream);
            }
        }
    } else {
        if (Xh) return KVC_ERR_UNSUPPORTED;
    }
    if constexpr (sizeof(OutT) == 2 && NRB <= 2) {
        // bf16 K~ rows staged whole where the tile fits (both sides at ranks <= 64)
        if (project_lds(NRB, false, nqb, nterm, 64) <= kMaxLds)
            return launch_project_variant<NRB, false, false, OutT, 64>(X, U, qfrag, nqb, nterm, sl, G, Xt, err, Xh,
                                                                       stream);
    }
    if constexpr (sizeof(OutT) == 4 && NRB <= 2) {
        // fp32 score launches: K~ rows staged whole, one column block at a time
        // (3.9-4.3 -> 3.75 ms at 1024 slices x 32768; the V side's 128-byte row
        // segments gain nothing from it)
        if (nqb > 0 && project_lds(NRB, false, nqb, nterm, 32) <= kMaxLds)
            return launch_project_variant<NRB, false, false, OutT, 32>(X, U, qfrag, nqb, nterm, sl, G, Xt, err, Xh,
                                                                       stream);
    }
    return nqb > 0
               ? launch_project_variant<NRB, false, false>(X, U, qfrag, nqb, nterm, sl, G, Xt, err, Xh, stream)
               : launch_project_variant<NRB, true, false>(X, U, qfrag, nqb, nterm, sl, G, Xt, err, Xh, stream);
}

template <typename OutT>
kvc_status project_dispatch(int64_t R, const uint16_t *X, const float *U, const u32x4 *qfrag,
                            int nqb, int nterm, const Slices &sl, int64_t G, OutT *Xt, float *err,
                            OutT *Xh, hipStream_t stream) {
    switch (R) {
        case 32: return launch_project<1>(X, U, qfrag, nqb, nterm, sl, G, Xt, err, Xh, stream);
        case 64: return launch_project<2>(X, U, qfrag, nqb, nterm, sl, G, Xt, err, Xh, stream);
        case 96: return launch_project<3>(X, U, qfrag, nqb, nterm, sl, G, Xt, err, Xh, stream);
        case 128: return launch_project<4>(X, U, qfrag, nqb, nterm, sl, G, Xt, err, Xh, stream);
    }
    return KVC_ERR_UNSUPPORTED;
}

template <int NRB>
kvc_status launch_reconstruct(const float *Xt, const float *U, const Slices &sl, int64_t G,
                              float *Xh, hipStream_t stream) {
    const int64_t blocks = G * sl.nsplit;
    if (blocks > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(reconstruct_kernel<NRB>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, Xt, U, sl, Xh);
    return launch_status();
}

template <int NRB>
kvc_status launch_reconstruct(const uint16_t *Xt, const float *U, const Slices &sl, int64_t G,
                              uint16_t *Xh, hipStream_t stream) {
    const int64_t blocks = G * sl.nsplit;
    if (blocks > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(reconstruct_bf16_kernel<NRB>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, Xt, U, sl, Xh);
    return launch_status();
}

// X^ = X~ U^T for every token (OutT float: fp32 rows; uint16_t: bf16 rows)
template <typename OutT>
kvc_status reconstruct_dispatch(const kvc_dims *d, const OutT *Xt, const float *U, int64_t G, OutT *Xh,
                                hipStream_t stream) {
    const Slices sl = make_slices(d, 128);
    switch (d->R) {
        case 32: return launch_reconstruct<1>(Xt, U, sl, G, Xh, stream);
        case 64: return launch_reconstruct<2>(Xt, U, sl, G, Xh, stream);
        case 96: return launch_reconstruct<3>(Xt, U, sl, G, Xh, stream);
        case 128: return launch_reconstruct<4>(Xt, U, sl, G, Xh, stream);
    }
    return KVC_ERR_UNSUPPORTED;
}

// Anchor rows into X^ (fp32: widened exactly; bf16: copied).  Bounds were
// checked by the caller; out-of-slice indices are skipped by the kernels.
kvc_status launch_anchors(const int32_t *idx, const uint16_t *rows, int64_t k, int64_t G, int64_t S,
                          int64_t S_stride, float *Xh, hipStream_t stream) {
    const int64_t bps = (k + kRowsPerBlock - 1) / kRowsPerBlock;
    if (G * bps > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(anchor_scatter_kernel, dim3(static_cast<unsigned>(G * bps)), dim3(kRowThreads), 0, stream,
                       idx, rows, k, bps, S, S_stride, Xh);
    return launch_status();
}

kvc_status launch_anchors(const int32_t *idx, const uint16_t *rows, int64_t k, int64_t G, int64_t S,
                          int64_t S_stride, uint16_t *Xh, hipStream_t stream) {
    const int64_t bps = (k + kRowsPerBlock - 1) / kRowsPerBlock;
    if (G * bps > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(anchor_copy_bf16_kernel, dim3(static_cast<unsigned>(G * bps)), dim3(kRowThreads), 0, stream,
                       idx, rows, k, bps, S, S_stride, Xh);
    return launch_status();
}

}  // namespace

size_t compress_workspace_bytes(const kvc_dims *d) {
    if (!d || check_dims(d, false) != KVC_OK) return 0;
    const bool with_q = d->H_q > 0 && d->W_q > 0 && d->H_q % d->H_kv == 0 &&
                        (d->H_q / d->H_kv) * d->W_q <= 128;
    WsSizer sz;
    compress_ws_layout(sz, d, with_q);
    return sz.bytes();
}

size_t reconstruct_workspace_bytes(const kvc_dims *) { return 0; }

}  // namespace kvc

namespace kvc {
namespace {

// K_hat == nullptr: compression only.  Otherwise X^ = X~ U^T is also written for
// every token of K (and of V when given), fused into the projection where it fits
// (ranks <= 64), else by the stand-alone reconstruction; both give the same bits.
template <typename OutT>
kvc_status compress_impl(const kvc_dims *d, const uint16_t *K, const uint16_t *V,
                         const uint16_t *Q_win, const float *U_k, const float *U_v, OutT *K_tilde,
                         OutT *V_tilde, float *err, OutT *K_hat, OutT *V_hat, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
    const bool with_q = Q_win != nullptr;
    kvc_status st = check_dims(d, with_q);
    if (st != KVC_OK) return st;
    if ((Q_win == nullptr) != (err == nullptr)) return KVC_ERR_INVALID_ARGUMENT;
    if ((V == nullptr) != (V_tilde == nullptr) || (V && !U_v)) return KVC_ERR_INVALID_ARGUMENT;
    if (!K_hat && V_hat) return KVC_ERR_INVALID_ARGUMENT;
    if (K_hat && (V == nullptr) != (V_hat == nullptr)) return KVC_ERR_INVALID_ARGUMENT;
    const int64_t G = d->L * d->B * d->H_kv;
    if (G == 0 || d->S == 0) return KVC_OK;
    if (!K || !U_k || !K_tilde) return KVC_ERR_INVALID_ARGUMENT;
    if (!aligned(K, 16) || !aligned(U_k, 16) || !aligned(K_tilde, 16) ||
        (V && (!aligned(V, 16) || !aligned(U_v, 16) || !aligned(V_tilde, 16))) ||
        (with_q && (!aligned(Q_win, 16) || !aligned(err, 4))) ||
        (K_hat && !aligned(K_hat, 16)) || (V_hat && !aligned(V_hat, 16)))
        return KVC_ERR_INVALID_ARGUMENT;
    WsSizer sz;
    compress_ws_layout(sz, d, with_q);
    if (sz.bytes() > 0 && (!ws || !aligned(ws, kWsAlign))) return KVC_ERR_INVALID_ARGUMENT;
    if (ws_bytes < sz.bytes()) return KVC_ERR_WORKSPACE_TOO_SMALL;

    const Slices sl = make_slices(d, 512);
    int nqb = 0, nterm = 0;
    u32x4 *qfrag = nullptr;
    if (with_q) {
        WsCursor cur(ws);
        const int64_t nq = (d->H_q / d->H_kv) * d->W_q;
        nqb = static_cast<int>((nq + 31) / 32);
        nterm = query_terms(nq);
        qfrag = cur.take<u32x4>(static_cast<size_t>(G * nqb * 8 * nterm * 64));
        const double scale = 1.0 / (static_cast<double>(nq) * sqrt(static_cast<double>(d->D)));
        if (G > INT32_MAX) return KVC_ERR_UNSUPPORTED;
        static std::atomic<bool> lds_ok[4][64];
        auto prep = [&](auto kernel, std::atomic<bool>(&ok)[64]) -> kvc_status {
            if (allow_large_lds(reinterpret_cast<const void *>(kernel), ok) != KVC_OK) return KVC_ERR_HIP;
            hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(G)), dim3(kPrepThreads), kPrepLds, stream,
                               Q_win, U_k, d->B, d->H_kv, d->H_q, d->W_q, static_cast<int>(d->R),
                               static_cast<int>(nq), nqb, nterm, scale, qfrag);
            return launch_status();
        };
        switch (nqb) {  // nq <= 128 was checked
            case 1: st = prep(&prep_query_kernel<2>, lds_ok[0]); break;
            case 2: st = prep(&prep_query_kernel<4>, lds_ok[1]); break;
            case 3: st = prep(&prep_query_kernel<6>, lds_ok[2]); break;
            default: st = prep(&prep_query_kernel<8>, lds_ok[3]); break;
        }
        if (st != KVC_OK) return st;
    }
    // one side (K with its error score, or V): projection, then X^ fused or separate
    auto side = [&](const uint16_t *X, const float *U, const u32x4 *qf, int nb, int nt, OutT *Xt,
                    float *e, OutT *Xh) -> kvc_status {
        if (Xh && !rebuild_fusable(d->R, nb, nt, sizeof(OutT) == 2)) {
            const kvc_status s1 =
                project_dispatch(d->R, X, U, qf, nb, nt, sl, G, Xt, e, static_cast<OutT *>(nullptr), stream);
            if (s1 != KVC_OK) return s1;
            return reconstruct_dispatch(d, static_cast<const OutT *>(Xt), U, G, Xh, stream);
        }
        return project_dispatch(d->R, X, U, qf, nb, nt, sl, G, Xt, e, Xh, stream);
    };
    st = side(K, U_k, qfrag, nqb, nterm, K_tilde, err, K_hat);
    if (st != KVC_OK) return st;
    if (V) st = side(V, U_v, nullptr, 0, 0, V_tilde, nullptr, V_hat);
    return st;
}

template <typename OutT>
kvc_status reconstruct_impl(const kvc_dims *d, const OutT *X_tilde, const float *U, const int32_t *anchor_idx,
                            const uint16_t *anchor_rows, int64_t k, OutT *X_hat, hipStream_t stream) {
    kvc_status st = check_dims(d, false);
    if (st != KVC_OK) return st;
    if (k < 0 || k > d->S) return KVC_ERR_INVALID_ARGUMENT;
    if ((k > 0) && (!anchor_idx || !anchor_rows)) return KVC_ERR_INVALID_ARGUMENT;
    const int64_t G = d->L * d->B * d->H_kv;
    if (G == 0 || d->S == 0) return KVC_OK;
    if (!X_tilde || !U || !X_hat || !aligned(X_tilde, 16) || !aligned(U, 16) || !aligned(X_hat, 16))
        return KVC_ERR_INVALID_ARGUMENT;
    if (k > 0 && (!aligned(anchor_idx, 4) || !aligned(anchor_rows, 16)))
        return KVC_ERR_INVALID_ARGUMENT;
    st = reconstruct_dispatch(d, X_tilde, U, G, X_hat, stream);
    if (st != KVC_OK || k == 0) return st;
    return launch_anchors(anchor_idx, anchor_rows, k, G, d->S, stride_of(d), X_hat, stream);
}

template <typename OutT>
kvc_status place_anchors_impl(const kvc_dims *d, const int32_t *anchor_idx, const uint16_t *anchor_rows,
                              int64_t k, OutT *X_hat, hipStream_t stream) {
    if (!d) return KVC_ERR_INVALID_ARGUMENT;
    if (d->L < 0 || d->B < 0 || d->H_kv <= 0 || d->S < 0 || d->D <= 0) return KVC_ERR_INVALID_ARGUMENT;
    if (d->S_stride != 0 && d->S_stride < d->S) return KVC_ERR_INVALID_ARGUMENT;
    if (d->D != kHeadDim) return KVC_ERR_UNSUPPORTED;
    if (k < 0 || k > d->S) return KVC_ERR_INVALID_ARGUMENT;
    const int64_t G = d->L * d->B * d->H_kv;
    if (G == 0 || d->S == 0 || k == 0) return KVC_OK;
    if (!anchor_idx || !anchor_rows || !X_hat || !aligned(anchor_idx, 4) || !aligned(anchor_rows, 16) ||
        !aligned(X_hat, 16))
        return KVC_ERR_INVALID_ARGUMENT;
    return launch_anchors(anchor_idx, anchor_rows, k, G, d->S, stride_of(d), X_hat, stream);
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_lowrank_compress(const kvc_dims *d, const uint16_t *K, const uint16_t *V,
                                           const uint16_t *Q_win, const float *U_k,
                                           const float *U_v, float *K_tilde, float *V_tilde,
                                           float *err, void *ws, size_t ws_bytes,
                                           hipStream_t stream) {
    return kvc::compress_impl(d, K, V, Q_win, U_k, U_v, K_tilde, V_tilde, err, static_cast<float *>(nullptr),
                              static_cast<float *>(nullptr), ws, ws_bytes, stream);
}

extern "C" kvc_status kvc_lowrank_compress_bf16(const kvc_dims *d, const uint16_t *K, const uint16_t *V,
                                                const uint16_t *Q_win, const float *U_k,
                                                const float *U_v, uint16_t *K_tilde,
                                                uint16_t *V_tilde, float *err, void *ws,
                                                size_t ws_bytes, hipStream_t stream) {
    return kvc::compress_impl(d, K, V, Q_win, U_k, U_v, K_tilde, V_tilde, err, static_cast<uint16_t *>(nullptr),
                              static_cast<uint16_t *>(nullptr), ws, ws_bytes, stream);
}

extern "C" kvc_status kvc_lowrank_compress_reconstruct(const kvc_dims *d, const uint16_t *K,
                                                       const uint16_t *V, const uint16_t *Q_win,
                                                       const float *U_k, const float *U_v, float *K_tilde,
                                                       float *V_tilde, float *err, float *K_hat,
                                                       float *V_hat, void *ws, size_t ws_bytes,
                                                       hipStream_t stream) {
    if (!K_hat) return KVC_ERR_INVALID_ARGUMENT;
    return kvc::compress_impl(d, K, V, Q_win, U_k, U_v, K_tilde, V_tilde, err, K_hat, V_hat, ws, ws_bytes,
                              stream);
}

extern "C" kvc_status kvc_lowrank_compress_reconstruct_bf16(const kvc_dims *d, const uint16_t *K,
                                                            const uint16_t *V, const uint16_t *Q_win,
                                                            const float *U_k, const float *U_v,
                                                            uint16_t *K_tilde, uint16_t *V_tilde, float *err,
                                                            uint16_t *K_hat, uint16_t *V_hat, void *ws,
                                                            size_t ws_bytes, hipStream_t stream) {
    if (!K_hat) return KVC_ERR_INVALID_ARGUMENT;
    return kvc::compress_impl(d, K, V, Q_win, U_k, U_v, K_tilde, V_tilde, err, K_hat, V_hat, ws, ws_bytes,
                              stream);
}

extern "C" kvc_status kvc_reconstruct(const kvc_dims *d, const float *X_tilde, const float *U,
                                      const int32_t *anchor_idx, const uint16_t *anchor_rows,
                                      int64_t k, float *X_hat, void *ws, size_t ws_bytes,
                                      hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    return kvc::reconstruct_impl(d, X_tilde, U, anchor_idx, anchor_rows, k, X_hat, stream);
}

extern "C" kvc_status kvc_reconstruct_bf16(const kvc_dims *d, const uint16_t *X_tilde, const float *U,
                                           const int32_t *anchor_idx, const uint16_t *anchor_rows,
                                           int64_t k, uint16_t *X_hat, void *ws, size_t ws_bytes,
                                           hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    return kvc::reconstruct_impl(d, X_tilde, U, anchor_idx, anchor_rows, k, X_hat, stream);
}

extern "C" kvc_status kvc_place_anchors(const kvc_dims *d, const int32_t *anchor_idx,
                                        const uint16_t *anchor_rows, int64_t k, float *X_hat,
                                        hipStream_t stream) {
    return kvc::place_anchors_impl(d, anchor_idx, anchor_rows, k, X_hat, stream);
}

extern "C" kvc_status kvc_place_anchors_bf16(const kvc_dims *d, const int32_t *anchor_idx,
                                             const uint16_t *anchor_rows, int64_t k, uint16_t *X_hat,
                                             hipStream_t stream) {
    return kvc::place_anchors_impl(d, anchor_idx, anchor_rows, k, X_hat, stream);
}
