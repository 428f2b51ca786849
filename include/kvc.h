/*
 * kvc.h -- C ABI of libkvc: KV-cache token scoring, eviction/compaction and
 * hybrid low-rank compression on AMD Instinct MI355X (gfx950).
 *
 * Methods (cited by page title and section):
 *   [MKV] "ManifoldKV: Training-Free KV Cache Compression via Euclidean
 *         Outlier Detection" (ICML 2026 poster page), abstract.
 *   [OJA] "OjaKV: Context-Aware Online Low-Rank KV Cache Compression"
 *         (papercache deep-notes page): "how it works" equations, background
 *         on low-rank attention, method details, appendix A.1 (Algorithm 1).
 *   [RKV] "RippleKV: Cross-Layer KV Cache Allocation via Perturbation
 *         Propagation" (explainer page), sensitivity-guided budget allocation.
 *   [RFK] "RefineKV" (project page): "Summarize", "Select", the Figure 2 risk
 *         formula.
 *
 * Common conventions
 *   - Every tensor pointer is a DEVICE pointer to dense row-major memory.
 *     bf16 tensors are passed as uint16_t bit patterns.  Pointers to bf16 and
 *     fp32 tensors must be 16-byte aligned.
 *   - A "slice" is one (layer, batch, kv head).  Per-token tensors are laid
 *     out [slice][token][...]; G = number of slices.  Where a `s_stride`
 *     appears, consecutive slices are s_stride tokens apart (s_stride >= S)
 *     so that a cache with spare capacity can be processed in place.
 *   - Ownership: the caller allocates every buffer, including the workspace
 *     `ws` of at least kvc_workspace_bytes(...) bytes (256-byte aligned).  The
 *     library never allocates or frees device memory and keeps no pointer
 *     after the call returns.  Buffers must stay valid until the work queued
 *     on `stream` has completed.  Inputs and outputs must not overlap, except
 *     where a parameter is documented in/out.
 *   - Execution: arguments are validated synchronously; on any error nothing
 *     is launched and the status is returned.  Otherwise the work is queued on
 *     `stream` (0 = the null stream) and the call returns without waiting.
 *     Results are deterministic: the same inputs give the same bits on every
 *     run.  Two calls that share a workspace must not run concurrently.
 *   - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 *   - Supported shapes: head dimension D = 128; low rank R in {32, 64, 96,
 *     128}; at most 128 queries per error-score window (g * W_q <= 128);
 *     S, k and window counts below 2^31.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 5

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, negative or inconsistent size */
    KVC_ERR_UNSUPPORTED = 2,        /* valid but not built: D != 128, R not in {32,64,96,128}, ... */
    KVC_ERR_WORKSPACE_TOO_SMALL = 3,/* ws_bytes < kvc_workspace_bytes(...) */
    KVC_ERR_HIP = 4,                /* a HIP runtime call or kernel launch failed */
    KVC_ERR_WAIT_EXPIRED = 5,       /* no longer reported (a centroid wait that gives up is
                                       repaired within the call); kept so codes stay stable */
    KVC_STATUS_MAX_ENUM = 0x7fffffff /* not a status: makes every int32 value a valid
                                        kvc_status, so callers may pass any code */
} kvc_status;

/* Process-wide options for tests and measurements (kvc_set_option).  The
 * defaults select the production kernel paths; every path computes the same
 * results. */
typedef enum kvc_option {
    KVC_OPTION_SCORE_PATH = 0,       /* centroid scores: 0 automatic (default), 1 the single-read
                                        kernel where a window's tiles fit the GPU at once, 2 the
                                        three-launch path */
    KVC_OPTION_SCORE_SPIN_LIMIT = 1, /* polls of a centroid wait before it gives up and leaves its
                                        team to the call's repair launch: -1 the built-in limit
                                        (default), 0 .. 2^32-1 (0: the first poll that finds no
                                        centroid gives up; lets a test force the repair path) */
    KVC_OPTION_GATHER_PATH = 2,      /* kept-row copy: 0 a separate wide gather launch (default),
                                        1 the selecting workgroup copies its slice's rows when
                                        k <= 8192 and there are at least as many slices as CUs */
    KVC_OPTION_MAX_ENUM = 0x7fffffff /* not an option: every int32 value is a valid kvc_option */
} kvc_option;

typedef enum kvc_op {
    KVC_OP_SCORE_L2 = 0,
    KVC_OP_SCORE_L2_WINDOWED = 1,
    KVC_OP_TOPK_COMPACT = 2,
    KVC_OP_LOWRANK_COMPRESS = 3,
    KVC_OP_OJA_UPDATE = 4,
    KVC_OP_RECONSTRUCT = 5,
    KVC_OP_SCORE_CENTROID = 6,
    KVC_OP_TOPK_RAGGED = 7,
    KVC_OP_REFINE_RISK = 8,
    KVC_OP_MAX_ENUM = 0x7fffffff    /* not an op: every int32 value is a valid kvc_op */
} kvc_op;

/* Score of a key against its (global or window) centroid mu, for
 * kvc_score_centroid. */
typedef enum kvc_metric {
    KVC_METRIC_L2 = 0,     /* || k_t - mu ||_2: ManifoldKV ([MKV] abstract) */
    KVC_METRIC_COSINE = 1, /* 1 - cos(k_t, mu): the cosine-to-centroid baseline the [MKV]
                              abstract compares against (scale-invariant); taken as 1 where
                              k_t or mu is the zero vector */
    KVC_METRIC_MAX_ENUM = 0x7fffffff
} kvc_metric;

/* Shapes of a multi-layer KV cache.
 *   L layers, B sequences, H_kv key/value heads, H_q query heads (a multiple of
 *   H_kv; kv head h serves query heads h*g .. h*g+g-1 with g = H_q/H_kv),
 *   S valid tokens per slice, S_stride allocated tokens per slice (0 -> S),
 *   D head dimension, R low rank, W_q recent queries per query head. */
typedef struct kvc_dims {
    int64_t L, B, H_kv, H_q, S, S_stride, D, R, W_q;
} kvc_dims;

/* ABI version of the loaded library (KVC_ABI_VERSION). */
int kvc_abi_version(void);

/* Sets a kvc_option for every later call in the process (calls already queued
 * are not affected).  A value outside the option's range, or an unknown
 * option: KVC_ERR_INVALID_ARGUMENT, and nothing changes. */
kvc_status kvc_set_option(kvc_option opt, int64_t value);

/* Failures that only the kernels can see, recorded in the status header at the
 * start of `ws` by the last call that used this workspace (kvc_score_l2,
 * kvc_score_l2_windowed, kvc_score_centroid, kvc_topk_compact_ragged; each of
 * them clears it before its kernels run).  Waits for `stream` to finish, then
 * reads the header: KVC_OK; KVC_ERR_INVALID_ARGUMENT when a device-side budget
 * of kvc_topk_compact_ragged was out of bounds (that slice kept nothing);
 * KVC_ERR_HIP when the wait or the read failed.  The scoring calls have no
 * failure to report (a centroid wait that gives up is repaired within the
 * call), so for them it returns KVC_OK.  ws must be a workspace of one of those
 * calls, 256-byte aligned. */
kvc_status kvc_workspace_status(const void *ws, hipStream_t stream);

/* Static, human-readable text for a status code. */
const char *kvc_status_str(kvc_status s);

/* Workspace bytes needed by one call of `op`.
 *   SCORE_L2, SCORE_L2_WINDOWED, SCORE_CENTROID: G = L*B*H_kv slices of S
 *     tokens; W = window (ignored for SCORE_L2).
 *   TOPK_COMPACT: G = L*B*H_kv slices of S tokens; k = tokens kept.
 *   TOPK_RAGGED: G = L*B*H_kv slices (a 256-byte status header + 16 bytes per slice).
 *   REFINE_RISK: G = L*B*H_kv slices of S tokens; k = cluster size c
 *     (144 bytes per 128 clusters of a slice).
 *   LOWRANK_COMPRESS, OJA_UPDATE, RECONSTRUCT: shapes from `d`; for OJA_UPDATE
 *     d->S is the token count N and W is the pooling window.  The bf16-storage
 *     variants need what LOWRANK_COMPRESS and RECONSTRUCT need.
 * 0 means the call needs no workspace (ws may then be NULL); invalid shapes
 * also give 0 and are reported by the call itself. */
size_t kvc_workspace_bytes(kvc_op op, const kvc_dims *d, int64_t k, int64_t W);

/* Global ManifoldKV score ([MKV] abstract): for every slice g and token t,
 *   mu_g       = (1/S) sum_t K[g][t][:]           (the key centroid)
 *   scores[g][t] = || K[g][t][:] - mu_g ||_2      (Euclidean distance)
 * K: bf16 [G][S][D].  scores: fp32 [G][S].  centroid: fp32 [G][D] or NULL.
 * Accumulation is fp32.  G >= 0, S >= 1 (G = 0 is a no-op).
 * Large caches are scored by one persistent launch whose workgroups exchange
 * each window's centroid; every wait in it is bounded.  A wait that runs past
 * its limit (a team's workgroups not all resident, e.g. while another kernel
 * holds part of the GPU) flags its window, and a repair launch queued in the
 * same call recomputes the flagged windows from the keys with the same bits, so
 * the results never depend on residency.  Results are deterministic. */
kvc_status kvc_score_l2(const uint16_t *K, int64_t G, int64_t S, int32_t D, float *scores,
                        float *centroid, void *ws, size_t ws_bytes, hipStream_t stream);

/* WindowedManifoldKV score ([MKV] abstract): as kvc_score_l2, but token t is
 * scored against the centroid of its contiguous window j = floor(t/W), the
 * mean over tokens [jW, min((j+1)W, S)) (a short last window is averaged over
 * the tokens it holds).  W >= S reproduces kvc_score_l2.
 * centroids: fp32 [G][ceil(S/W)][D] or NULL.  W >= 1. */
kvc_status kvc_score_l2_windowed(const uint16_t *K, int64_t G, int64_t S, int32_t D, int64_t W,
                                 float *scores, float *centroids, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Centroid score with a choice of metric: as kvc_score_l2_windowed (windows
 * of W tokens; W >= S is the global centroid), with scores[g][t] =
 * metric(K[g][t][:], mu) for `metric` a kvc_metric.  KVC_METRIC_L2 gives the
 * same bits as kvc_score_l2(_windowed).  For KVC_METRIC_COSINE the score is
 * evaluated as ||k/||k|| - mu/||mu||||^2 / 2 (equal to 1 - cos), which keeps
 * its relative accuracy for keys nearly parallel to mu; it lies in [0, 2].
 * centroids: fp32 [G][ceil(S/W)][D] or NULL (always the mean, not its
 * direction).  Unknown metric: KVC_ERR_INVALID_ARGUMENT. */
kvc_status kvc_score_centroid(const uint16_t *K, int64_t G, int64_t S, int32_t D, int64_t W,
                              int32_t metric, float *scores, float *centroids, void *ws,
                              size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): kvc_score_centroid
 * with no workspace argument.  Its scratch is a device array of
 * KVC_NOALLOC_SCRATCH_BYTES inside the library, one per device, held until the
 * process ends; the call allocates nothing.  It accepts the shapes whose
 * kvc_workspace_bytes(KVC_OP_SCORE_CENTROID, ...) fits that size (e.g. 256
 * slices of 65536 tokens with 4096-token windows; 2 bytes per token plus a few
 * KiB per window) and returns KVC_ERR_WORKSPACE_TOO_SMALL for larger ones,
 * before launching anything.  Results are bit-identical to kvc_score_centroid.
 * Every call on a device shares that device's scratch, so calls that may overlap
 * on one device (different streams or threads) race; calls queued in order on
 * one stream do not. */
#define KVC_NOALLOC_SCRATCH_BYTES (48ull << 20)
kvc_status kvc_score_centroid_noalloc(const uint16_t *K, int64_t G, int64_t S, int32_t D, int64_t W,
                                      int32_t metric, float *scores, float *centroids,
                                      hipStream_t stream);

/* Retention and compaction ([MKV] abstract: the keys farthest from the
 * centroid are retained; [OJA] method details: the top-k error scores are kept
 * at full rank).  For each slice g, selects the k largest scores[g][0..S)
 * (equal scores: the lower token index wins; +0.0 == -0.0), writes their token
 * indices in ascending order to idx_out[g][0..k), and, when K / V are given,
 * copies the selected rows bit for bit: K_out[g][i][:] = K[g][idx_out[g][i]][:].
 *   scores: fp32, slice stride s_stride floats (s_stride >= S)
 *   K, V:   bf16, slice stride s_stride rows of D, or NULL
 *   idx_out: int32 [G][k];  K_out, V_out: bf16 [G][k][D] (NULL iff K / V NULL)
 * 0 <= k <= S.  With k == 0 (or G == 0) nothing is written and every output may
 * be NULL. */
kvc_status kvc_topk_compact(const float *scores, int64_t G, int64_t S, int64_t s_stride, int64_t k,
                            const uint16_t *K, const uint16_t *V, int32_t D, int32_t *idx_out,
                            uint16_t *K_out, uint16_t *V_out, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* RippleKV budget allocation ([RKV] "RippleKV: Cross-Layer KV Cache Allocation
 * via Perturbation Propagation", sensitivity-guided budget allocation).  HOST
 * function, host pointers.  For layers l = 0..L-1 with sensitivities s_l:
 *   s^_l = (s_l - min s) / (max s - min s)    (0 for all when they are equal),
 *   w_l  = r^{s^_l} clipped to [1/gamma, gamma],
 *   k_l  proportional to w_l with sum_l k_l = B.
 * A share above S is pinned at S and the remaining budget shared again by the
 * other layers; whole tokens are the floors plus one for the largest fractional
 * parts (equal parts: the lower layer first).  Requires r > 0, gamma >= 1,
 * 0 <= B <= L * S.  k_out: int64 [L]. */
kvc_status kvc_layer_budgets(const double *sensitivity, int64_t L, double r, double gamma,
                             int64_t B, int64_t S, int64_t *k_out);

/* Retention and compaction with a budget per slice (e.g. RippleKV's layer
 * budgets, every slice of layer l keeping k_l): as kvc_topk_compact with slice
 * g keeping k[g] tokens.  k is a DEVICE array int64 [G] (8-byte aligned), read
 * by the call's kernels on `stream`.  Outputs are packed in slice order: slice
 * g's indices are idx_out[o_g .. o_g + k[g]) with o_g = k[0] + ... + k[g-1],
 * and its rows K_out[o_g + i][:] (likewise V_out).
 *   k_max:   host bound on every budget, 0 <= k_max <= S (sizes the row copy)
 *   k_total: capacity of the packed outputs in rows: idx_out int32 [k_total],
 *            K_out, V_out bf16 [k_total][D] (any of them may be NULL when
 *            k_total == 0: no row is written)
 * The budgets are checked on the device: a slice whose budget is negative or
 * above k_max, or whose rows would end past k_total, keeps nothing, no output
 * is written outside [0, k_total), and kvc_workspace_status on this workspace
 * reports KVC_ERR_INVALID_ARGUMENT.  The workspace (kvc_workspace_bytes(
 * KVC_OP_TOPK_RAGGED, ...)) holds the status header, the checked budgets and
 * the offsets. */
kvc_status kvc_topk_compact_ragged(const float *scores, int64_t G, int64_t S, int64_t s_stride,
                                   const int64_t *k, int64_t k_max, int64_t k_total, const uint16_t *K,
                                   const uint16_t *V, int32_t D, int32_t *idx_out, uint16_t *K_out,
                                   uint16_t *V_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* RefineKV cluster summaries ([RFK] "Summarize": contiguous clusters with
 * cached mean keys, mean values and metadata).  For slice g and cluster
 * j = tokens [jc, min((j+1)c, S)), nC = ceil(S/c):
 *   mu_k[g][j][:] = mean key, mu_v[g][j][:] = mean value   (fp32 [G][nC][D]),
 *   radius[g][j]  = max_t ||k_t - mu_k[g][j]||_2            (fp32 [G][nC]),
 *   vnorm[g][j]   = max_t ||v_t||_2                          (fp32 [G][nC]).
 * K, V: bf16 [G][S][D].  fp32 accumulation in token order.  c >= 1. */
kvc_status kvc_cluster_summaries(const uint16_t *K, const uint16_t *V, int64_t G, int64_t S,
                                 int32_t D, int64_t c, float *mu_k, float *mu_v, float *radius,
                                 float *vnorm, hipStream_t stream);

/* RefineKV risk score of every cluster for each query ([RFK] "Select": global
 * importance x local distortion, with the Figure 2 formula)
 *   RC = 2 p_C Vmax [ (cosh d_C - 1) / Dn + tanh(d_C / 2) ],  Dn = sum_C' p_C' cosh d_C',
 * where (readings: the page names these quantities without formulas)
 *   p_C  = n_C exp(z_C) / sum_C' n_C' exp(z_C'),  z_C = q . mu_k[C] / sqrt(D),
 *   d_C  = ||q|| radius[C] / sqrt(D)   (bounds |q.k - q.mu_C| / sqrt(D) for k in C),
 *   Vmax = max_C vnorm[C] over the slice.
 * Summaries as from kvc_cluster_summaries (same S and c); Q: bf16 [G][nq][D],
 * 16-byte aligned (the queries served by slice g, nq <= 8); rc: fp32 [G][nq][nC].
 * ws: kvc_workspace_bytes(KVC_OP_REFINE_RISK, d, c, 0) bytes, 16-byte aligned,
 * for per-chunk softmax records.  Evaluated without overflow for any finite d_C
 * (terms rescaled by the largest exponent).  A cluster with RC > tau would be
 * expanded to its exact entries (not done here). */
kvc_status kvc_refine_risk(const float *mu_k, const float *radius, const float *vnorm, int64_t G,
                           int64_t S, int64_t c, int32_t D, const uint16_t *Q, int32_t nq, float *rc,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* Hybrid low-rank compression ([OJA] background: K~ = K U_k, V~ = V U_v;
 * method details: residual r_t = k_t - U_k U_k^T k_t and query-weighted error
 *   err_t = 1/|W_t| sum_{h, q in W_t} | q_{h,q}^T r_t / sqrt(D) |,
 * the window W_t being the W_q recent queries of the g query heads of the
 * slice's kv head, |W_t| = g*W_q).
 *   K, V:   bf16 [L][B][H_kv][S_stride][D]     (V may be NULL)
 *   Q_win:  bf16 [L][B][H_q][W_q][D]           (NULL: no error score)
 *   U_k, U_v: fp32 [L][H_kv][D][R], one basis per (layer, kv head), shared by
 *           the batch; any matrix is accepted (orthonormality is not checked)
 *   K_tilde, V_tilde: fp32 [L][B][H_kv][S_stride][R]  (V_tilde NULL iff V NULL)
 *   err:    fp32 [L][B][H_kv][S_stride]        (NULL iff Q_win NULL)
 * Rows t >= S of the outputs are not written. */
kvc_status kvc_lowrank_compress(const kvc_dims *d, const uint16_t *K, const uint16_t *V,
                                const uint16_t *Q_win, const float *U_k, const float *U_v,
                                float *K_tilde, float *V_tilde, float *err, void *ws,
                                size_t ws_bytes, hipStream_t stream);

/* bf16 storage of the compressed cache ([OJA] efficiency analysis: the memory
 * saving comes from storing K~ and V~ instead of K and V): as
 * kvc_lowrank_compress, with K~ and V~ written as bf16, the round-to-nearest-even
 * of the same fp32 result; err stays fp32.
 *   K_tilde, V_tilde: bf16 [L][B][H_kv][S_stride][R] */
kvc_status kvc_lowrank_compress_bf16(const kvc_dims *d, const uint16_t *K, const uint16_t *V,
                                     const uint16_t *Q_win, const float *U_k, const float *U_v,
                                     uint16_t *K_tilde, uint16_t *V_tilde, float *err, void *ws,
                                     size_t ws_bytes, hipStream_t stream);

/* Oja basis update with pooling and QR ([OJA] how it works: the Oja rule;
 * method details: prefill update on AvgPool(X, pool) with the empirical
 * covariance, decode update on the buffered tokens, re-orthonormalisation by
 * QR; appendix A.1).  For each (layer, kv head):
 *   X_p = rows of AvgPool(X[l][b][h][0..N), pool) for b = 0..B-1 (windows
 *         [i*pool, min((i+1)*pool, N)), a short tail averaged over its rows),
 *   n   = B * ceil(N/pool),  C = X_p^T X_p / n,
 *   U  <- Q factor of  U + eta (C U - U U^T C U)  (positive diagonal of R).
 *   U: fp32 [L][H_kv][D][R], IN/OUT (updated in place)
 *   X: bf16 [L][B][H_kv][S_stride][D], the first N = d->S tokens are used
 * pool >= 1 (1 = no pooling); eta finite.  The update is computed in fp64
 * after an fp32 accumulation of C. */
kvc_status kvc_oja_update(const kvc_dims *d, float *U, const uint16_t *X, int32_t pool, float eta,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/* Reconstruction before attention ([OJA] background: K^ = K~ U_k^T) with the
 * hybrid cache's full-rank anchors put back ([OJA] method details):
 *   X_hat[g][t][:] = X_tilde[g][t][:] U^T              for non-anchor t,
 *   X_hat[g][idx[g][i]][:] = anchor_rows[g][i][:] (bf16 widened exactly).
 *   X_tilde: fp32 [L][B][H_kv][S_stride][R];  U: fp32 [L][H_kv][D][R]
 *   anchor_idx: int32 [L*B*H_kv][k] (indices < S, unique); anchor_rows: bf16
 *   [L*B*H_kv][k][D]; both NULL iff k == 0
 *   X_hat: fp32 [L][B][H_kv][S_stride][D] (rows t >= S not written) */
kvc_status kvc_reconstruct(const kvc_dims *d, const float *X_tilde, const float *U,
                           const int32_t *anchor_idx, const uint16_t *anchor_rows, int64_t k,
                           float *X_hat, void *ws, size_t ws_bytes, hipStream_t stream);

/* Decode-step append ([OJA] method details, appendix A.1: each decoded token
 * joins the cache and the update buffer, its queries the scoring window):
 *   K[g][pos][:] = k_new[g][:],  V[g][pos][:] = v_new[g][:]      (g < L*B*H_kv),
 *   K_buf[g][slot][:] = k_new[g][:], V_buf[g][slot][:] = v_new[g][:]   (if given),
 *   Q_buf[h][slot][:] = q_new[h][:]  for the L*B*H_q query heads h   (if q_new given).
 * K, V: bf16 [L*B*H_kv][S_stride][D]; k_new, v_new: bf16 [L*B*H_kv][D];
 * K_buf, V_buf: bf16 [L*B*H_kv][T][D] (both or neither); q_new: bf16
 * [L*B*H_q][D]; Q_buf: bf16 [L*B*H_q][T][D].  0 <= pos < S_stride (d->S_stride,
 * or d->S when 0), 0 <= slot < T.  One launch; no workspace. */
kvc_status kvc_decode_append(const kvc_dims *d, int64_t pos, int64_t T, int64_t slot,
                             const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q_new,
                             uint16_t *K, uint16_t *V, uint16_t *K_buf, uint16_t *V_buf,
                             uint16_t *Q_buf, hipStream_t stream);

/* Reconstruction from bf16 storage: as kvc_reconstruct, with X_tilde and X_hat
 * bf16.  X_hat = bf16(X_tilde U^T), an fp32 accumulation of the exact bf16
 * X_tilde against U split as hi + lo, rounded to nearest even; anchor rows are
 * copied bit for bit.
 *   X_tilde: bf16 [L][B][H_kv][S_stride][R];  X_hat: bf16 [L][B][H_kv][S_stride][D] */
kvc_status kvc_reconstruct_bf16(const kvc_dims *d, const uint16_t *X_tilde, const float *U,
                                const int32_t *anchor_idx, const uint16_t *anchor_rows, int64_t k,
                                uint16_t *X_hat, void *ws, size_t ws_bytes, hipStream_t stream);

/* Compression with the reconstruction fused in ([OJA] background: K~ = K U_k
 * and K^ = K~ U_k^T; the OjaKV pass that re-projects the cache and rebuilds
 * K^, V^ for attention): everything kvc_lowrank_compress computes, plus
 *   K_hat[g][t][:] = K_tilde[g][t][:] U_k^T,  V_hat[g][t][:] = V_tilde[g][t][:] U_v^T
 * for EVERY token t < S, anchors not placed (select them from err with
 * kvc_topk_compact, then write their rows with kvc_place_anchors).  X~ is
 * taken from the projection's registers instead of being read back (4R fewer
 * bytes per head-token and tensor in fp32, 2R in bf16).  The
 * outputs equal those of kvc_lowrank_compress followed by kvc_reconstruct with
 * k = 0, bit for bit.
 *   K_hat: fp32 [L][B][H_kv][S_stride][D] (not NULL); V_hat: same, NULL iff V is NULL.
 * Other arguments, workspace (KVC_OP_LOWRANK_COMPRESS) and errors as
 * kvc_lowrank_compress. */
kvc_status kvc_lowrank_compress_reconstruct(const kvc_dims *d, const uint16_t *K, const uint16_t *V,
                                            const uint16_t *Q_win, const float *U_k, const float *U_v,
                                            float *K_tilde, float *V_tilde, float *err, float *K_hat,
                                            float *V_hat, void *ws, size_t ws_bytes, hipStream_t stream);

/* bf16 storage: as kvc_lowrank_compress_reconstruct with K~, V~, K^, V^ bf16;
 * equals kvc_lowrank_compress_bf16 followed by kvc_reconstruct_bf16 with k = 0,
 * bit for bit. */
kvc_status kvc_lowrank_compress_reconstruct_bf16(const kvc_dims *d, const uint16_t *K,
                                                 const uint16_t *V, const uint16_t *Q_win,
                                                 const float *U_k, const float *U_v, uint16_t *K_tilde,
                                                 uint16_t *V_tilde, float *err, uint16_t *K_hat,
                                                 uint16_t *V_hat, void *ws, size_t ws_bytes,
                                                 hipStream_t stream);

/* The hybrid cache's full-rank anchors put into a reconstruction ([OJA] method
 * details: anchor tokens keep their exact rows):
 *   X_hat[g][idx[g][i]][:] = anchor_rows[g][i][:]   (bf16 widened exactly), i < k.
 * Uses d->L, B, H_kv, S, S_stride, D only.  anchor_idx: int32 [L*B*H_kv][k]
 * (indices < S; an index outside [0, S) is skipped); anchor_rows: bf16
 * [L*B*H_kv][k][D]; X_hat: fp32 [L][B][H_kv][S_stride][D].  k = 0 does nothing. */
kvc_status kvc_place_anchors(const kvc_dims *d, const int32_t *anchor_idx, const uint16_t *anchor_rows,
                             int64_t k, float *X_hat, hipStream_t stream);

/* As kvc_place_anchors into a bf16 X_hat (rows copied bit for bit). */
kvc_status kvc_place_anchors_bf16(const kvc_dims *d, const int32_t *anchor_idx,
                                  const uint16_t *anchor_rows, int64_t k, uint16_t *X_hat,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
