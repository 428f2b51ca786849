// Retention and compaction: per slice, the k largest fp32 scores (equal
// scores: lower token index first), their indices in ascending order, and a
// bit-exact gather of the retained K and V rows.  ManifoldKV keeps the keys
// farthest from the centroid ("ManifoldKV ...", abstract and lay summary);
// OjaKV keeps the top-k error-score tokens at full rank ("OjaKV ...", method
// details).
//
// select_compact: one 1024-thread workgroup per slice.
//   - scores are mapped to order-preserving 32-bit keys;
//   - radix select, 8 bits per pass from the top: per-wave LDS histograms of
//     the keys that still match the prefix, then a 256-bin suffix scan finds
//     the digit holding the k-th largest key; after 4 passes the threshold
//     key T is exact and `need` = how many keys equal to T are kept.  The
//     passes stop early when the chosen bin holds exactly the keys still
//     needed: all of them are kept, and the lower digits cannot change the set;
//   - slices of up to 16 x 4096 scores are read once: each thread keeps its
//     keys in registers for the four passes and the ordered pass (longer
//     slices read the scores again at every pass);
//   - one ordered pass in 4096-key tiles: a packed (greater, equal) count
//     scan gives every kept key its output slot, equal keys taken lowest
//     index first until `need` are taken.
// gather_rows: 16 lanes per 256-byte row, 16-byte loads and stores.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kPerThread = 4;
constexpr int kTile = kSelThreads * kPerThread;

// Inclusive scan over the 1024 threads of the block; returns the exclusive
// prefix and writes the block total to *total.  `wtot` holds kSelWaves words.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wtot,
                                                         uint32_t *total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wtot[wave] = x;
    __syncthreads();
    if (wave == 0) {
        uint32_t w = lane < kSelWaves ? wtot[lane] : 0u;
#pragma unroll
        for (int d = 1; d < kSelWaves; d <<= 1) {
            uint32_t y = __shfl_up(w, d, 64);
            if (lane >= d) w += y;
        }
        if (lane < kSelWaves) wtot[kSelWaves + lane] = w;  // inclusive wave prefix
    }
    __syncthreads();
    const uint32_t wave_excl = wave ? wtot[kSelWaves + wave - 1] : 0u;
    *total = wtot[2 * kSelWaves - 1];
    const uint32_t excl = wave_excl + x - v;
    __syncthreads();  // wtot may be reused by the caller's next scan
    return excl;
}

// Longest slice whose keys are held in registers: 16 tiles of 4096 keys, 64 keys
// (64 VGPRs) per thread.
constexpr int kMaxHeldTiles = 16;

// kg / koff (device, nullable): per-slice budget and output offset (packed
// outputs); otherwise every slice keeps k and its outputs start at g * k.
// NT > 0: key t * kTile + 4 * thread + j (t < NT) is read once into held[t][j] and
// every pass reads it there; without kTail the slice holds at most NT * kTile
// scores, with kTail the scores past NT * kTile are read again at every pass.
// NT == 0: each pass reads all the scores again.
template <int NT, bool kTail = false>
__global__ __launch_bounds__(kSelThreads) void select_compact(const float *__restrict__ scores,
                                                              int64_t S, int64_t s_stride,
                                                              int64_t k_all,
                                                              const int64_t *__restrict__ kg,
                                                              const int64_t *__restrict__ koff,
                                                              int32_t *__restrict__ idx_out,
                                                              const uint16_t *__restrict__ K,
                                                              const uint16_t *__restrict__ V,
                                                              uint16_t *__restrict__ K_out,
                                                              uint16_t *__restrict__ V_out) {
    const int64_t g = blockIdx.x;
    const int64_t k = kg ? kg[g] : k_all;
    const int64_t base = koff ? koff[g] : g * k_all;
    if (k <= 0 || k > S) return;  // budgets were validated (host or device); uniform per block
    const float *s = scores + g * s_stride;
    int32_t *out = idx_out + base;

    __shared__ uint32_t hist[kSelWaves][256];
    __shared__ uint32_t suffix[257];
    __shared__ uint32_t sel[3];
    __shared__ uint32_t wtot[2 * kSelWaves];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    uint32_t prefix = 0, mask = 0;
    uint32_t remaining = static_cast<uint32_t>(k);
    // 16-byte loads when the slice's scores are 16-byte aligned (uniform per block)
    const bool vec = (reinterpret_cast<uintptr_t>(s) & 15u) == 0;
    const int64_t S4 = vec ? S / 4 * 4 : 0;

    uint32_t held[NT > 0 ? NT : 1][kPerThread];
    constexpr int64_t kTail0 = static_cast<int64_t>(NT) * kTile;  // first score not held
    if constexpr (NT > 0) {
        // every thread's loads in flight at once
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int64_t i0 = static_cast<int64_t>(t) * kTile + static_cast<int64_t>(threadIdx.x) * kPerThread;
            if (vec && i0 + kPerThread <= S) {
                const float4 x = *reinterpret_cast<const float4 *>(s + i0);
                held[t][0] = order_key(x.x);
                held[t][1] = order_key(x.y);
                held[t][2] = order_key(x.z);
                held[t][3] = order_key(x.w);
            } else {
#pragma unroll
                for (int j = 0; j < kPerThread; ++j) held[t][j] = i0 + j < S ? order_key(s[i0 + j]) : 0u;
            }
        }
    }

    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = threadIdx.x; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0u;
        __syncthreads();
        // Keys that match the prefix add to their digit's bin.  In the first pass the
        // digit is the top byte -- the sign and exponent -- so most keys share a few
        // digits and 64 atomics on one LDS address would serialise: the lanes holding
        // the digit of the wave's first matching lane add with one atomic and the
        // others one each.  The later passes' digits are mantissa bits, spread over
        // many bins, and every key adds its own atomic: the ballots of an aggregation
        // round cost more than the conflicts they save there (one round in every pass
        // -> in the first pass only: 21.4 -> 19.9 us at 256 x 16384, 72.4 -> 65.6 us at
        // 256 x 65536, 164 -> 153 us for 1024 x 32768 error scores; two or more rounds
        // in the first pass: 47 us at 256 x 16384).  The bin counts are the same either way.
        auto count = [&](uint32_t key, bool valid) {
            const bool m = valid && (key & mask) == prefix;
            const uint32_t dig = (key >> shift) & 255u;
            if (pass > 0) {
                if (m) atomicAdd(&hist[wave][dig], 1u);
                return;
            }
            const uint64_t act = __ballot(m);
            if (act == 0) return;  // uniform across the wave
            const int first = __ffsll(static_cast<unsigned long long>(act)) - 1;
            const uint32_t d0 = __shfl(dig, first, 64);
            const bool same = m && dig == d0;
            const uint64_t agg = __ballot(same);
            if (lane == first) atomicAdd(&hist[wave][d0], static_cast<uint32_t>(__popcll(agg)));
            else if (m && !same) atomicAdd(&hist[wave][dig], 1u);
        };
        if constexpr (NT > 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int j = 0; j < kPerThread; ++j)
                    count(held[t][j], static_cast<int64_t>(t) * kTile + static_cast<int64_t>(threadIdx.x) * kPerThread + j < S);
        }
        if constexpr (NT == 0 || kTail) {
            // the scores past the held ones: four 16-byte loads per thread in flight per step
            constexpr int64_t kStep = static_cast<int64_t>(kSelThreads) * 4;
            for (int64_t i = kTail0 + static_cast<int64_t>(threadIdx.x) * 4; i < S4; i += 4 * kStep) {
                float4 x[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (i + u * kStep < S4) x[u] = *reinterpret_cast<const float4 *>(s + i + u * kStep);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (i + u * kStep < S4) {
                        count(order_key(x[u].x), true);
                        count(order_key(x[u].y), true);
                        count(order_key(x[u].z), true);
                        count(order_key(x[u].w), true);
                    }
            }
            for (int64_t i = S4 + threadIdx.x; i < S; i += kSelThreads) count(order_key(s[i]), true);
        }
        __syncthreads();
        // suffix sums over bins, suffix[b] = count of matching keys with digit >= b:
        // a 64-lane suffix scan per wave over its 64 bins, then the waves above added
        uint32_t c = 0;
        if (threadIdx.x < 256) {
#pragma unroll
            for (int w = 0; w < kSelWaves; ++w) c += hist[w][threadIdx.x];
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t y = __shfl_down(c, d, 64);
                if (lane + d < 64) c += y;
            }
            if (lane == 0) wtot[wave] = c;  // total of the wave's 64 bins
        }
        __syncthreads();
        if (threadIdx.x < 256) {
            for (int w = wave + 1; w < 4; ++w) c += wtot[w];
            suffix[threadIdx.x] = c;
        }
        if (threadIdx.x == 0) suffix[256] = 0u;
        __syncthreads();
        if (threadIdx.x < 256) {
            const uint32_t here = suffix[threadIdx.x], above = suffix[threadIdx.x + 1];
            if (here >= remaining && above < remaining) {
                sel[0] = threadIdx.x;
                sel[1] = above;
                sel[2] = here - above;  // keys in the chosen bin
            }
        }
        __syncthreads();
        const uint32_t digit = sel[0];
        remaining -= sel[1];
        prefix |= digit << shift;
        mask |= 255u << shift;
        const bool whole_bin = sel[2] == remaining;
        __syncthreads();
        // every key of the chosen bin is kept: the lower digits cannot change the set
        // (the k-th largest key is the bin's smallest, and keys equal to it share the
        // bin), so the passes left are skipped (uniform across the block)
        if (whole_bin) break;
    }
    // The kept keys are those whose masked key is above the prefix, and of the keys
    // whose masked key equals it the first `need` in index order (all of them when
    // the passes stopped at a whole bin).  With all four passes the mask covers the
    // whole key and the prefix is the key of the k-th largest score.
    const uint32_t T = prefix;
    const uint32_t need = remaining;  // keys at the prefix that are kept (>= 1)

    uint32_t out_pos = 0;  // kept so far (uniform across the block)
    uint32_t eq_seen = 0;  // keys equal to T seen so far
    // one 4096-key tile of the ordered pass, keys[j] = key of index base + 4 * thread + j
    auto ordered_tile = [&](int64_t base, const uint32_t (&keys)[kPerThread]) {
        const int64_t i0 = base + static_cast<int64_t>(threadIdx.x) * kPerThread;
        uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t i = i0 + j;
            n_gt += (i < S && (keys[j] & mask) > T);
            n_eq += (i < S && (keys[j] & mask) == T);
        }
        uint32_t tot;
        const uint32_t excl = block_exclusive_scan((n_gt << 16) | n_eq, wtot, &tot);
        const uint32_t gt_before = excl >> 16, eq_before = excl & 0xffffu;
        const uint32_t tile_gt = tot >> 16, tile_eq = tot & 0xffffu;
        uint32_t pos = out_pos + gt_before + (min(eq_seen + eq_before, need) - min(eq_seen, need));
        uint32_t eq_rank = eq_seen + eq_before;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t i = i0 + j;
            if (i >= S) break;
            // pos < k holds by construction (exactly k keys are kept); the
            // test only keeps a write inside the slice's output row regardless
            if ((keys[j] & mask) > T) {
                if (pos < k) out[pos] = static_cast<int32_t>(i);
                ++pos;
            } else if ((keys[j] & mask) == T) {
                if (eq_rank < need) {
                    if (pos < k) out[pos] = static_cast<int32_t>(i);
                    ++pos;
                }
                ++eq_rank;
            }
        }
        out_pos += tile_gt + (min(eq_seen + tile_eq, need) - min(eq_seen, need));
        eq_seen += tile_eq;
    };
    if constexpr (NT > 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (static_cast<int64_t>(t) * kTile >= S) break;  // uniform across the block
            ordered_tile(static_cast<int64_t>(t) * kTile, held[t]);
        }
    }
    if constexpr (NT == 0 || kTail) {
        for (int64_t base = kTail0; base < S; base += kTile) {
            const int64_t i0 = base + static_cast<int64_t>(threadIdx.x) * kPerThread;
            uint32_t keys[kPerThread];
            if (vec && i0 + kPerThread <= S) {
                const float4 x = *reinterpret_cast<const float4 *>(s + i0);
                keys[0] = order_key(x.x);
                keys[1] = order_key(x.y);
                keys[2] = order_key(x.z);
                keys[3] = order_key(x.w);
            } else {
#pragma unroll
                for (int j = 0; j < kPerThread; ++j) keys[j] = i0 + j < S ? order_key(s[i0 + j]) : 0u;
            }
            ordered_tile(base, keys);
        }
    }
    if (!K && !V) return;
    // Compaction of the slice's rows by the same workgroup, as soon as its
    // indices exist: 16 lanes per 256-byte row, 4 rows per thread in flight.
    __syncthreads();  // this workgroup's index writes are visible to it
    const int lane16 = threadIdx.x & 15;
    const int rsub = threadIdx.x >> 4;  // 0..63
    const uint4 *Ks = K ? reinterpret_cast<const uint4 *>(K + g * s_stride * kHeadDim) : nullptr;
    const uint4 *Vs = V ? reinterpret_cast<const uint4 *>(V + g * s_stride * kHeadDim) : nullptr;
    uint4 *Ko = K_out ? reinterpret_cast<uint4 *>(K_out + base * kHeadDim) : nullptr;
    uint4 *Vo = V_out ? reinterpret_cast<uint4 *>(V_out + base * kHeadDim) : nullptr;
    constexpr int kRowsPerPass = kSelThreads / 16;  // 64
    constexpr int kUnroll = 4;  // rows per thread in flight (fetch(0..3) below)
    for (int64_t i0 = 0; i0 < k; i0 += kRowsPerPass * kUnroll) {
        int64_t src0, src1, src2, src3;
        bool ok0, ok1, ok2, ok3;
        auto fetch = [&](int u, int64_t &src, bool &ok) {
            const int64_t i = i0 + u * kRowsPerPass + rsub;
            const int64_t t = i < k ? out[i] : -1;
            ok = t >= 0 && t < S;  // never read outside the slice
            src = ok ? t : 0;
        };
        fetch(0, src0, ok0);
        fetch(1, src1, ok1);
        fetch(2, src2, ok2);
        fetch(3, src3, ok3);
        // rows are read and written once: streaming loads and stores
        if (Ks) {
            const uint4 a0 = ld_stream(Ks + src0 * 16 + lane16), a1 = ld_stream(Ks + src1 * 16 + lane16);
            const uint4 a2 = ld_stream(Ks + src2 * 16 + lane16), a3 = ld_stream(Ks + src3 * 16 + lane16);
            if (ok0) st_stream(Ko + (i0 + 0 * kRowsPerPass + rsub) * 16 + lane16, a0);
            if (ok1) st_stream(Ko + (i0 + 1 * kRowsPerPass + rsub) * 16 + lane16, a1);
            if (ok2) st_stream(Ko + (i0 + 2 * kRowsPerPass + rsub) * 16 + lane16, a2);
            if (ok3) st_stream(Ko + (i0 + 3 * kRowsPerPass + rsub) * 16 + lane16, a3);
        }
        if (Vs) {
            const uint4 b0 = ld_stream(Vs + src0 * 16 + lane16), b1 = ld_stream(Vs + src1 * 16 + lane16);
            const uint4 b2 = ld_stream(Vs + src2 * 16 + lane16), b3 = ld_stream(Vs + src3 * 16 + lane16);
            if (ok0) st_stream(Vo + (i0 + 0 * kRowsPerPass + rsub) * 16 + lane16, b0);
            if (ok1) st_stream(Vo + (i0 + 1 * kRowsPerPass + rsub) * 16 + lane16, b1);
            if (ok2) st_stream(Vo + (i0 + 2 * kRowsPerPass + rsub) * 16 + lane16, b2);
            if (ok3) st_stream(Vo + (i0 + 3 * kRowsPerPass + rsub) * 16 + lane16, b3);
        }
    }
}

// one wave per workgroup, one row per 16 lanes: many small workgroups move the rows
// fastest (256 x 16384, keep 8192: 0.369 ms with 64 threads, 0.377-0.382 with 256 and
// one row per thread, 0.410-0.414 with 256 and four rows per thread)
constexpr int kGatherThreads = 64;
constexpr int kGatherRows = 4;  // rows per workgroup

// kg / koff as for select_compact (nullable: k_all rows per slice at g * k_all).
__global__ __launch_bounds__(kGatherThreads) void gather_rows(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, int64_t S, int64_t s_stride,
    const int32_t *__restrict__ idx_all, int64_t k_all, const int64_t *__restrict__ kg,
    const int64_t *__restrict__ koff, int64_t blocks_per_slice, uint16_t *__restrict__ K_out,
    uint16_t *__restrict__ V_out) {
    // slices in reverse order: the scoring kernel reads the last slices' keys last, so
    // part of them is still in the last-level cache when the copy starts (windowed
    // step at 256 x 65536: 3.045 -> 3.005 ms; global step unchanged)
    const int64_t g = (gridDim.x / blocks_per_slice) - 1 - blockIdx.x / blocks_per_slice;
    const int64_t k = kg ? kg[g] : k_all;
    const int64_t base = koff ? koff[g] : g * k_all;
    const int32_t *idx = idx_all + base;
    const int lane16 = threadIdx.x & 15;
    const int rsub = threadIdx.x >> 4;  // row of the pass
    constexpr int kPass = kGatherThreads / 16;  // rows per pass of the workgroup
    constexpr int kRows = kGatherRows / kPass;  // rows per thread
    const uint4 *Ks = reinterpret_cast<const uint4 *>(K), *Vs = reinterpret_cast<const uint4 *>(V);
    // Block b of a slice copies rows [4 b, 4 b + 4), then, with per-slice budgets
    // (the grid sized for the mean budget), the blocks b + blocks_per_slice, ... that
    // the slice's budget reaches: as many workgroups as with one budget, and none
    // launched only to find nothing to copy (a grid sized for the largest budget left
    // half its one-wave workgroups empty: 366.6 against 342.5 us at 256 x 16384 with
    // budgets from 3976 to 15906 rows; block j of every slice before block j + 1
    // instead: 0.48 ms, the copy's reads no longer walking a slice in order).
    for (int64_t r0 = (blockIdx.x % blocks_per_slice) * kGatherRows; r0 < k;
         r0 += blocks_per_slice * kGatherRows) {
        // all indices, then all row loads, then the stores: a thread keeps 2 kRows
        // 16-byte loads in flight (issued one row at a time, each waited on its index
        // and its load)
        int64_t src[kRows], dst[kRows];
        bool ok[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int64_t i = r0 + r * kPass + rsub;
            const int64_t t = i < k ? idx[i] : -1;
            ok[r] = t >= 0 && t < S;  // indices come from select_compact; never read outside
            src[r] = (g * s_stride + (ok[r] ? t : 0)) * (kHeadDim / 8) + lane16;
            dst[r] = (base + i) * (kHeadDim / 8) + lane16;
        }
        uint4 kv[kRows], vv[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            if (K) kv[r] = ld_stream(Ks + src[r]);
            if (V) vv[r] = ld_stream(Vs + src[r]);
        }
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            if (!ok[r]) continue;
            if (K) st_stream(reinterpret_cast<uint4 *>(K_out) + dst[r], kv[r]);
            if (V) st_stream(reinterpret_cast<uint4 *>(V_out) + dst[r], vv[r]);
        }
    }
}

// The kept rows are copied by the separate wide launch: with one row per thread and
// many small workgroups it moves them faster than the selecting workgroups can
// (256 x 16384, keep 8192: 0.385 against 0.419 ms for select + copy; 1024 x 32768,
// keep 1639: 0.467 against 0.484 ms).  The option KVC_OPTION_GATHER_PATH = 1 selects
// the in-workgroup copy instead.
bool fused_gather() { return options().gather_path.load(std::memory_order_relaxed) == 1; }

// Per-slice budgets of kvc_topk_compact_ragged, checked and packed on the device:
// one workgroup reads the caller's budgets k[g], keeps a budget only if it lies in
// [0, k_max] and its rows fit before k_total (else the slice keeps nothing and the
// status word says so), and writes each slice's effective budget and output offset
// (an exclusive scan in slice order) to the workspace.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void ragged_offsets(const int64_t *__restrict__ k, int64_t G,
                                                               int64_t k_max, int64_t k_total,
                                                               uint32_t *__restrict__ status,
                                                               int64_t *__restrict__ keff,
                                                               int64_t *__restrict__ koff) {
    __shared__ int64_t wsum[kScanThreads / 64];
    __shared__ uint32_t bad;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) bad = 0u;
    __syncthreads();
    int64_t carry = 0;  // rows packed by the slices before this chunk (uniform)
    for (int64_t g0 = 0; g0 < G; g0 += kScanThreads) {
        const int64_t g = g0 + threadIdx.x;
        int64_t v = g < G ? k[g] : 0;
        if (v < 0 || v > k_max) {
            bad = 1u;
            v = 0;
        }
        // inclusive scan of the chunk: within each wave, then across the waves
        int64_t x = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int64_t before = 0, chunk = 0;
        for (int w = 0; w < kScanThreads / 64; ++w) {
            if (w < wave) before += wsum[w];
            chunk += wsum[w];
        }
        int64_t off = carry + before + x - v;
        if (off + v > k_total) {  // outputs sized for fewer rows: this slice keeps none
            bad = 1u;
            v = 0;
        }
        if (g < G) {
            keff[g] = v;
            koff[g] = off < k_total ? off : k_total;
        }
        carry += chunk;
        __syncthreads();  // wsum is rewritten by the next chunk
    }
    __syncthreads();
    if (threadIdx.x == 0) *status = bad ? kStatusBadBudget : 0u;
}

// select_compact for a slice length S: the register-held instance with the fewest
// tiles that covers S, else the instance that holds the first 12 tiles (49152
// scores; holding 14 or 16 next to the tail's loads spilled) and reads the rest at
// every pass (the decode loop's 131072 + 32j scores: 172 us per call when every
// score was read at each of the five passes).
void launch_select(int64_t G, int64_t S, hipStream_t stream, const float *scores, int64_t s_stride,
                   int64_t k_all, const int64_t *kg, const int64_t *koff, int32_t *idx_out,
                   const uint16_t *K, const uint16_t *V, uint16_t *K_out, uint16_t *V_out) {
    const dim3 grid(static_cast<unsigned>(G)), block(kSelThreads);
#define KVC_SELECT(nt)                                                                            \
    hipLaunchKernelGGL(select_compact<nt>, grid, block, 0, stream, scores, S, s_stride, k_all, kg, \
                       koff, idx_out, K, V, K_out, V_out)
    if (S <= 1 * kTile) KVC_SELECT(1);
    else if (S <= 2 * kTile) KVC_SELECT(2);
    else if (S <= 4 * kTile) KVC_SELECT(4);
    else if (S <= 8 * kTile) KVC_SELECT(8);
    else if (S <= kMaxHeldTiles * kTile) KVC_SELECT(kMaxHeldTiles);
    else
        hipLaunchKernelGGL((select_compact<12, true>), grid, block, 0, stream, scores, S, s_stride, k_all,
                           kg, koff, idx_out, K, V, K_out, V_out);
#undef KVC_SELECT
}

}  // namespace

size_t topk_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

// Status header, then the per-slice effective budgets and output offsets of
// kvc_topk_compact_ragged.
template <class Ws>
void ragged_ws_layout(Ws &ws, int64_t G) {
    ws.template take<uint32_t>(kStatusBytes / 4);
    ws.template take<int64_t>(static_cast<size_t>(G));
    ws.template take<int64_t>(static_cast<size_t>(G));
}

size_t topk_ragged_workspace_bytes(int64_t G) {
    if (G <= 0) return 0;
    WsSizer z;
    ragged_ws_layout(z, G);
    return z.bytes();
}

}  // namespace kvc

extern "C" kvc_status kvc_topk_compact(const float *scores, int64_t G, int64_t S, int64_t s_stride,
                                       int64_t k, const uint16_t *K, const uint16_t *V, int32_t D,
                                       int32_t *idx_out, uint16_t *K_out, uint16_t *V_out,
                                       void *ws, size_t ws_bytes, hipStream_t stream) {
    using namespace kvc;
    (void)ws;
    (void)ws_bytes;
    if (G < 0 || S < 0 || k < 0 || k > S || s_stride < S) return KVC_ERR_INVALID_ARGUMENT;
    if (G == 0 || k == 0) return KVC_OK;  // nothing to write: the outputs may be NULL
    if ((K == nullptr) != (K_out == nullptr) || (V == nullptr) != (V_out == nullptr))
        return KVC_ERR_INVALID_ARGUMENT;
    if ((K || V) && D != kHeadDim) return D <= 0 ? KVC_ERR_INVALID_ARGUMENT : KVC_ERR_UNSUPPORTED;
    if (S > INT32_MAX || G > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    if (!scores || !idx_out || !aligned(scores, 4) || !aligned(idx_out, 4))
        return KVC_ERR_INVALID_ARGUMENT;
    if ((K && (!aligned(K, 16) || !aligned(K_out, 16))) || (V && (!aligned(V, 16) || !aligned(V_out, 16))))
        return KVC_ERR_INVALID_ARGUMENT;
    // the selecting workgroup also copies its slice's rows when the copy is small
    // (k <= 8192 rows per slice) and there are enough slices to occupy every compute
    // unit; otherwise the copy goes to a wide gather launch
    if ((K || V) && k <= 8192 && G >= device_cu_count() && fused_gather()) {
        launch_select(G, S, stream, scores, s_stride, k, nullptr, nullptr, idx_out, K, V, K_out, V_out);
        return launch_status();
    }
    launch_select(G, S, stream, scores, s_stride, k, nullptr, nullptr, idx_out, nullptr, nullptr, nullptr,
                  nullptr);
    if (K || V) {
        const int64_t bps = (k + kGatherRows - 1) / kGatherRows;
        if (G * bps > INT32_MAX) return KVC_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(gather_rows, dim3(static_cast<unsigned>(G * bps)), dim3(kGatherThreads), 0,
                           stream, K, V, S, s_stride, idx_out, k, nullptr, nullptr, bps, K_out, V_out);
    }
    return launch_status();
}

extern "C" kvc_status kvc_topk_compact_ragged(const float *scores, int64_t G, int64_t S,
                                              int64_t s_stride, const int64_t *k, int64_t k_max,
                                              int64_t k_total, const uint16_t *K, const uint16_t *V,
                                              int32_t D, int32_t *idx_out, uint16_t *K_out,
                                              uint16_t *V_out, void *ws, size_t ws_bytes,
                                              hipStream_t stream) {
    using namespace kvc;
    if (G < 0 || S < 0 || s_stride < S || k_max < 0 || k_max > S || k_total < 0)
        return KVC_ERR_INVALID_ARGUMENT;
    // with k_total == 0 no row is written: the row outputs may then be NULL
    if (k_total > 0 && ((K == nullptr) != (K_out == nullptr) || (V == nullptr) != (V_out == nullptr)))
        return KVC_ERR_INVALID_ARGUMENT;
    if (k_total > 0 && (K || V) && D != kHeadDim) return D <= 0 ? KVC_ERR_INVALID_ARGUMENT : KVC_ERR_UNSUPPORTED;
    if (S > INT32_MAX || G > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    if (G == 0) return KVC_OK;
    if (!k || !aligned(k, 8) || !ws || !aligned(ws, kWsAlign)) return KVC_ERR_INVALID_ARGUMENT;
    if (ws_bytes < topk_ragged_workspace_bytes(G)) return KVC_ERR_WORKSPACE_TOO_SMALL;
    if (k_total > 0 && (!scores || !idx_out || !aligned(scores, 4) || !aligned(idx_out, 4)))
        return KVC_ERR_INVALID_ARGUMENT;
    if (k_total > 0 &&
        ((K && (!aligned(K, 16) || !aligned(K_out, 16))) || (V && (!aligned(V, 16) || !aligned(V_out, 16)))))
        return KVC_ERR_INVALID_ARGUMENT;
    WsCursor cur(ws);
    uint32_t *status = cur.take<uint32_t>(kStatusBytes / 4);
    int64_t *kg = cur.take<int64_t>(static_cast<size_t>(G));
    int64_t *koff = cur.take<int64_t>(static_cast<size_t>(G));
    // the budgets are checked and packed by a kernel on the stream (no host copy)
    hipLaunchKernelGGL(ragged_offsets, dim3(1), dim3(kScanThreads), 0, stream, k, G, k_max, k_total,
                       status, kg, koff);
    if (k_max == 0 || k_total == 0) return launch_status();
    if ((K || V) && k_max <= 8192 && G >= device_cu_count() && fused_gather()) {
        launch_select(G, S, stream, scores, s_stride, int64_t{0}, kg, koff, idx_out, K, V, K_out, V_out);
        return launch_status();
    }
    launch_select(G, S, stream, scores, s_stride, int64_t{0}, kg, koff, idx_out, nullptr, nullptr, nullptr,
                  nullptr);
    if (K || V) {
        // blocks for the mean budget (the packed outputs hold k_total rows); a slice
        // with more rows loops over its further blocks
        const int64_t mean = (k_total + G - 1) / G;
        const int64_t rows = mean < k_max ? mean : k_max;
        const int64_t bps = (rows + kGatherRows - 1) / kGatherRows;
        if (G * bps > INT32_MAX) return KVC_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(gather_rows, dim3(static_cast<unsigned>(G * bps)), dim3(kGatherThreads), 0,
                           stream, K, V, S, s_stride, idx_out, int64_t{0}, kg, koff, bps, K_out, V_out);
    }
    return launch_status();
}
