/*
 * kvc_oracle.c -- plain, single-threaded CPU oracle for KV-cache token scoring,
 * eviction/compaction and hybrid low-rank compression.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library) shares no source, header, table or helper with this file.
 *
 * Conventions
 *   - Every floating-point quantity is carried in double precision.  bf16
 *     inputs are widened exactly (a bf16 value is the top half of an IEEE
 *     binary32), fp32 inputs are widened exactly.  Nothing is rounded inside;
 *     the caller decides whether and where to round to fp32.
 *   - Tensors are dense row-major.  A "slice" is one (layer, batch, kv head);
 *     per-token tensors of a slice are [S][D] with a slice stride of
 *     `s_stride` tokens (s_stride >= S).
 *   - Return value: 0 on success, a negative number on invalid arguments or a
 *     non-finite input (the pages define nothing for NaN or Inf).
 *
 * Sources (pages the method is described on):
 *   [MKV]  "ManifoldKV: Training-Free KV Cache Compression via Euclidean
 *          Outlier Detection" (ICML 2026 poster page), abstract and lay summary.
 *   [RKV]  "RippleKV: Cross-Layer KV Cache Allocation via Perturbation
 *          Propagation" (explainer page), "Sensitivity-Guided Budget
 *          Allocation": normalised sensitivities, exponential multipliers,
 *          clipping, rescaling to the global budget.
 *   [RFK]  "RefineKV" (project page): "Summarize" (contiguous clusters with
 *          mean keys, mean values and metadata), "Select" and the Figure 2
 *          risk-score formula.
 *   [OJA]  "OjaKV: Context-Aware Online Low-Rank KV Cache Compression"
 *          (papercache deep-notes page): the "how it works" display equations
 *          for e_t and the Oja rule, "background / low-rank attention",
 *          "method details", and appendix A.1 (Algorithm 1), A.4, A.9.
 *
 * Parity status: every function here is pinned by CPU tests against closed
 * forms, invariants, exact-rational brute force or a library routine.  The
 * decode-time re-projection reading used by the full-loop driver lives in the
 * Python wrapper and is marked "parity unpinned" there.  ora_refine_risk takes
 * readings of the attention-mass and logit-deviation terms, which the page names
 * without formulas; they are pinned by what the page says the scores are, the
 * cluster-wise terms of an upper bound on the attention-output error: the sum of
 * the clusters' RC bounds the error of attending with every cluster replaced by
 * its size-weighted representative (random and adversarial instances; a reading
 * that makes RC too small fails).  RC is not a bound of a single cluster's
 * replacement error, which the page only correlates with it.  Its arithmetic is
 * pinned by closed forms and a worked example of the printed Figure 2 formula
 * evaluated in 60-digit decimals.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_OK 0
#define ORA_EINVAL (-1)
#define ORA_ENONFINITE (-2)
#define ORA_ENOMEM (-3)

/* ---------------------------------------------------------------- codecs */

/* bf16 is the upper 16 bits of an IEEE-754 binary32; widening is exact. */
static double bf16_to_double(uint16_t h) {
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

double ora_bf16_to_f64(uint16_t h) { return bf16_to_double(h); }

/* ------------------------------------------------------- ManifoldKV score */

/* Mean of keys t in [t0, t1) of one slice, per channel ([MKV] "the key
 * centroid").  Plain summation in double, then one division. */
static void centroid_range(const uint16_t *Kslice, int64_t D, int64_t t0, int64_t t1,
                           double *mu) {
    for (int64_t c = 0; c < D; ++c) mu[c] = 0.0;
    for (int64_t t = t0; t < t1; ++t)
        for (int64_t c = 0; c < D; ++c) mu[c] += bf16_to_double(Kslice[t * D + c]);
    double n = (double)(t1 - t0);
    for (int64_t c = 0; c < D; ++c) mu[c] /= n;
}

/* Euclidean distance of key t to a centroid ([MKV] "Euclidean distance to the
 * key centroid", capturing angular and radial deviation). */
static double l2_distance(const uint16_t *krow, const double *mu, int64_t D) {
    double acc = 0.0;
    for (int64_t c = 0; c < D; ++c) {
        double diff = bf16_to_double(krow[c]) - mu[c];
        acc += diff * diff;
    }
    return sqrt(acc);
}

static int all_finite_bf16(const uint16_t *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if ((x[i] & 0x7f80u) == 0x7f80u) return 0;
    return 1;
}

/* WindowedManifoldKV ([MKV] abstract): each key is scored against the centroid
 * of its own contiguous window [jW, min((j+1)W, S)).  The last window may be
 * short; its mean is over the keys it actually holds.  W >= S is the global
 * scorer.  scores: [G][S]; centroids (nullable): [G][ceil(S/W)][D]. */
int ora_score_l2_windowed(const uint16_t *K, int64_t G, int64_t S, int64_t D, int64_t W,
                          double *scores, double *centroids) {
    if (G < 0 || S < 0 || D <= 0 || W <= 0 || (S > 0 && G > 0 && (!K || !scores)))
        return ORA_EINVAL;
    if (!all_finite_bf16(K, G * S * D)) return ORA_ENONFINITE;
    int64_t nwin = (S + W - 1) / W;
    double *mu = (double *)malloc(sizeof(double) * (size_t)D);
    if (!mu) return ORA_ENOMEM;
    for (int64_t g = 0; g < G; ++g) {
        const uint16_t *Kg = K + g * S * D;
        for (int64_t j = 0; j < nwin; ++j) {
            int64_t t0 = j * W;
            int64_t t1 = t0 + W < S ? t0 + W : S;
            centroid_range(Kg, D, t0, t1, mu);
            if (centroids) memcpy(centroids + (g * nwin + j) * D, mu, sizeof(double) * (size_t)D);
            for (int64_t t = t0; t < t1; ++t) scores[g * S + t] = l2_distance(Kg + t * D, mu, D);
        }
    }
    free(mu);
    return ORA_OK;
}

/* Global ManifoldKV score: one centroid over all S keys of the slice. */
int ora_score_l2(const uint16_t *K, int64_t G, int64_t S, int64_t D, double *scores,
                 double *centroid) {
    if (G < 0 || S < 0 || D <= 0 || (S > 0 && G > 0 && (!K || !scores))) return ORA_EINVAL;
    if (!all_finite_bf16(K, G * S * D)) return ORA_ENONFINITE;
    double *mu = (double *)malloc(sizeof(double) * (size_t)D);
    if (!mu) return ORA_ENOMEM;
    for (int64_t g = 0; g < G; ++g) {
        const uint16_t *Kg = K + g * S * D;
        if (S > 0) {
            centroid_range(Kg, D, 0, S, mu);
        } else {
            for (int64_t c = 0; c < D; ++c) mu[c] = 0.0; /* no keys: no centroid */
        }
        if (centroid) memcpy(centroid + g * D, mu, sizeof(double) * (size_t)D);
        for (int64_t t = 0; t < S; ++t) scores[g * S + t] = l2_distance(Kg + t * D, mu, D);
    }
    free(mu);
    return ORA_OK;
}

/* Cosine dissimilarity of key t to a centroid: 1 - cos(k_t, mu), the score of
 * the geometry-based baseline the ManifoldKV abstract contrasts with its L2
 * score (keys scored by cosine similarity to a global centroid; the most
 * dissimilar kept).  Where k_t or mu is the zero vector the cosine is taken as
 * 0 (score 1). */
static double cosine_dissimilarity(const uint16_t *krow, const double *mu, int64_t D) {
    double dot = 0.0, kk = 0.0, mm = 0.0;
    for (int64_t c = 0; c < D; ++c) {
        double x = bf16_to_double(krow[c]);
        dot += x * mu[c];
        kk += x * x;
        mm += mu[c] * mu[c];
    }
    if (kk == 0.0 || mm == 0.0) return 1.0;
    /* ||k|| ||mu|| as one square root of the product: for k = mu it is exactly
     * ||k||^2, so a key equal to its centroid scores exactly 0 */
    return 1.0 - dot / sqrt(kk * mm);
}

/* The cosine score against the centroid of each contiguous window of W keys
 * (W >= S: one global centroid), windows as in ora_score_l2_windowed. */
int ora_score_cosine_windowed(const uint16_t *K, int64_t G, int64_t S, int64_t D, int64_t W,
                              double *scores, double *centroids) {
    if (G < 0 || S < 0 || D <= 0 || W <= 0 || (S > 0 && G > 0 && (!K || !scores)))
        return ORA_EINVAL;
    if (!all_finite_bf16(K, G * S * D)) return ORA_ENONFINITE;
    int64_t nwin = (S + W - 1) / W;
    double *mu = (double *)malloc(sizeof(double) * (size_t)D);
    if (!mu) return ORA_ENOMEM;
    for (int64_t g = 0; g < G; ++g) {
        const uint16_t *Kg = K + g * S * D;
        for (int64_t j = 0; j < nwin; ++j) {
            int64_t t0 = j * W;
            int64_t t1 = t0 + W < S ? t0 + W : S;
            centroid_range(Kg, D, t0, t1, mu);
            if (centroids) memcpy(centroids + (g * nwin + j) * D, mu, sizeof(double) * (size_t)D);
            for (int64_t t = t0; t < t1; ++t) scores[g * S + t] = cosine_dissimilarity(Kg + t * D, mu, D);
        }
    }
    free(mu);
    return ORA_OK;
}

/* --------------------------------------------------------------- top-k */

typedef struct {
    float value;
    int32_t index;
} scored_t;

/* Order for retention: larger score first; equal scores -> lower index first.
 * +0.0 and -0.0 compare equal, as they do in IEEE arithmetic. */
static int cmp_retain(const void *a, const void *b) {
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->value > y->value) return -1;
    if (x->value < y->value) return 1;
    return (x->index > y->index) - (x->index < y->index);
}

static int cmp_int32(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Keep the k largest scores of each slice ([MKV]: keys far from the centroid
 * are the ones retained; [OJA] method details: the top-k error scores become
 * full-rank anchors).  Output: [G][k] indices in ascending (temporal) order.
 * The decision is taken on the fp32 scores given. */
int ora_topk(const float *scores, int64_t G, int64_t S, int64_t s_stride, int64_t k,
             int32_t *idx) {
    if (G < 0 || S < 0 || k < 0 || k > S || s_stride < S || S > INT32_MAX) return ORA_EINVAL;
    if (G == 0 || k == 0) return ORA_OK;
    scored_t *buf = (scored_t *)malloc(sizeof(scored_t) * (size_t)S);
    if (!buf) return ORA_ENOMEM;
    for (int64_t g = 0; g < G; ++g) {
        for (int64_t t = 0; t < S; ++t) {
            float v = scores[g * s_stride + t];
            if (!isfinite(v)) {
                free(buf);
                return ORA_ENONFINITE;
            }
            buf[t].value = v;
            buf[t].index = (int32_t)t;
        }
        qsort(buf, (size_t)S, sizeof(scored_t), cmp_retain);
        int32_t *out = idx + g * k;
        for (int64_t i = 0; i < k; ++i) out[i] = buf[i].index;
        qsort(out, (size_t)k, sizeof(int32_t), cmp_int32);
    }
    free(buf);
    return ORA_OK;
}

/* Compaction: out[g][i][:] = X[g][idx[g][i]][:] (bytes copied as they are). */
int ora_gather(const uint16_t *X, int64_t G, int64_t S, int64_t s_stride, int64_t D,
               const int32_t *idx, int64_t k, uint16_t *out) {
    if (G < 0 || S < 0 || D <= 0 || k < 0 || k > S || s_stride < S) return ORA_EINVAL;
    for (int64_t g = 0; g < G; ++g)
        for (int64_t i = 0; i < k; ++i) {
            int32_t t = idx[g * k + i];
            if (t < 0 || t >= S) return ORA_EINVAL;
            memcpy(out + (g * k + i) * D, X + (g * s_stride + (int64_t)t) * D,
                   sizeof(uint16_t) * (size_t)D);
        }
    return ORA_OK;
}

/* ------------------------------------------------------- OjaKV low rank */

/* Low-rank projection, residual and query-weighted error score for every
 * token of every slice ([OJA] background: K~ = K U_k, V~ = V U_v; method
 * details: r_t = k_t - U_k U_k^T k_t and
 *   e_t = 1/|W_t| * sum_{h, q in W_t} | q_{h,q}^T r_t / sqrt(d_h) | ).
 * The query window of kv head h is the H_q/H_kv query heads of its group
 * (heads h*g .. h*g+g-1), each with its W_q most recent queries, so that
 * |W_t| = g * W_q.
 *   K, V     : [L][B][H_kv][s_stride][D] bf16   (V nullable)
 *   Q        : [L][B][H_q][W_q][D] bf16          (nullable: no error score)
 *   Uk, Uv   : [L][H_kv][D][R] fp32, one basis per (layer, kv head)
 *   Kt, Vt   : [L][B][H_kv][s_stride][R]         (Vt nullable iff V is)
 *   err      : [L][B][H_kv][s_stride]            (nullable iff Q is)
 */
int ora_lowrank_compress(int64_t L, int64_t B, int64_t Hkv, int64_t Hq, int64_t S,
                         int64_t s_stride, int64_t D, int64_t R, int64_t Wq,
                         const uint16_t *K, const uint16_t *V, const uint16_t *Q,
                         const float *Uk, const float *Uv, double *Kt, double *Vt,
                         double *err) {
    if (L < 0 || B < 0 || Hkv <= 0 || D <= 0 || R <= 0 || R > D || S < 0 || s_stride < S)
        return ORA_EINVAL;
    if (!K || !Uk || !Kt) return ORA_EINVAL;
    if ((V == NULL) != (Vt == NULL) || (V && !Uv)) return ORA_EINVAL;
    if ((Q == NULL) != (err == NULL)) return ORA_EINVAL;
    if (Q && (Hq <= 0 || Hq % Hkv != 0 || Wq <= 0)) return ORA_EINVAL;
    int64_t grp = Q ? Hq / Hkv : 0;
    double *k = (double *)malloc(sizeof(double) * (size_t)(3 * D + R));
    if (!k) return ORA_ENOMEM;
    double *khat = k + D, *r = khat + D, *kt = r + D;
    double inv_sqrt_d = 1.0 / sqrt((double)D);

    for (int64_t l = 0; l < L; ++l)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < Hkv; ++h) {
                int64_t slice = (l * B + b) * Hkv + h;
                const float *U = Uk + (l * Hkv + h) * D * R;
                for (int64_t t = 0; t < S; ++t) {
                    const uint16_t *krow = K + (slice * s_stride + t) * D;
                    if (!all_finite_bf16(krow, D)) {
                        free(k);
                        return ORA_ENONFINITE;
                    }
                    for (int64_t c = 0; c < D; ++c) k[c] = bf16_to_double(krow[c]);
                    /* projection onto the basis: k~_j = sum_c k_c U[c][j] */
                    for (int64_t j = 0; j < R; ++j) {
                        double acc = 0.0;
                        for (int64_t c = 0; c < D; ++c) acc += k[c] * (double)U[c * R + j];
                        kt[j] = acc;
                        Kt[(slice * s_stride + t) * R + j] = acc;
                    }
                    if (!Q) continue;
                    /* reconstruction inside the residual, from the unrounded k~ */
                    for (int64_t c = 0; c < D; ++c) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < R; ++j) acc += kt[j] * (double)U[c * R + j];
                        khat[c] = acc;
                        r[c] = k[c] - khat[c];
                    }
                    /* query-weighted error over the group's recent-query window */
                    double e = 0.0;
                    for (int64_t hq = h * grp; hq < (h + 1) * grp; ++hq)
                        for (int64_t q = 0; q < Wq; ++q) {
                            const uint16_t *qrow = Q + (((l * B + b) * Hq + hq) * Wq + q) * D;
                            double dot = 0.0;
                            for (int64_t c = 0; c < D; ++c) dot += bf16_to_double(qrow[c]) * r[c];
                            e += fabs(dot * inv_sqrt_d);
                        }
                    err[slice * s_stride + t] = e / (double)(grp * Wq);
                }
                if (V) {
                    const float *Uvh = Uv + (l * Hkv + h) * D * R;
                    for (int64_t t = 0; t < S; ++t) {
                        const uint16_t *vrow = V + (slice * s_stride + t) * D;
                        if (!all_finite_bf16(vrow, D)) {
                            free(k);
                            return ORA_ENONFINITE;
                        }
                        for (int64_t j = 0; j < R; ++j) {
                            double acc = 0.0;
                            for (int64_t c = 0; c < D; ++c)
                                acc += bf16_to_double(vrow[c]) * (double)Uvh[c * R + j];
                            Vt[(slice * s_stride + t) * R + j] = acc;
                        }
                    }
                }
            }
    free(k);
    return ORA_OK;
}

/* Reconstruction before attention ([OJA] background: K^ = K~ U_k^T), with the
 * hybrid cache's full-rank anchors put back as they were stored ([OJA] method
 * details: top-k tokens kept at full rank).
 *   Xt   : [L][B][H_kv][s_stride][R] (double: the caller widens fp32 exactly)
 *   U    : [L][H_kv][D][R] fp32
 *   idx  : [L][B][H_kv][k] anchor token indices; rows: [..][k][D] bf16
 *   Xhat : [L][B][H_kv][s_stride][D]                                        */
int ora_reconstruct(int64_t L, int64_t B, int64_t Hkv, int64_t S, int64_t s_stride, int64_t D,
                    int64_t R, const double *Xt, const float *U, const int32_t *idx,
                    const uint16_t *rows, int64_t k, double *Xhat) {
    if (L < 0 || B < 0 || Hkv <= 0 || D <= 0 || R <= 0 || R > D || S < 0 || s_stride < S ||
        k < 0 || k > S)
        return ORA_EINVAL;
    if (!Xt || !U || !Xhat || (k > 0 && (!idx || !rows))) return ORA_EINVAL;
    for (int64_t l = 0; l < L; ++l)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < Hkv; ++h) {
                int64_t slice = (l * B + b) * Hkv + h;
                const float *Uh = U + (l * Hkv + h) * D * R;
                for (int64_t t = 0; t < S; ++t)
                    for (int64_t c = 0; c < D; ++c) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < R; ++j)
                            acc += Xt[(slice * s_stride + t) * R + j] * (double)Uh[c * R + j];
                        Xhat[(slice * s_stride + t) * D + c] = acc;
                    }
                for (int64_t i = 0; i < k; ++i) {
                    int32_t t = idx[slice * k + i];
                    if (t < 0 || t >= S) return ORA_EINVAL;
                    for (int64_t c = 0; c < D; ++c)
                        Xhat[(slice * s_stride + t) * D + c] =
                            bf16_to_double(rows[(slice * k + i) * D + c]);
                }
            }
    return ORA_OK;
}

/* --------------------------------------------------------- Oja + QR */

/* Local average pooling along tokens ([OJA] method details:
 * X_pooled = AvgPool(X, b); Algorithm 1 prefill step 1).  Windows are
 * [i*p, min((i+1)p, N)) with kernel = stride = p; a short tail window is
 * averaged over the tokens it holds.  X: [N][D] bf16 (one slice),
 * out: [ceil(N/p)][D]. */
int ora_avgpool(const uint16_t *X, int64_t N, int64_t D, int64_t p, double *out) {
    if (N < 0 || D <= 0 || p <= 0) return ORA_EINVAL;
    int64_t np = (N + p - 1) / p;
    for (int64_t i = 0; i < np; ++i) {
        int64_t t0 = i * p, t1 = t0 + p < N ? t0 + p : N;
        for (int64_t c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int64_t t = t0; t < t1; ++t) acc += bf16_to_double(X[t * D + c]);
            out[i * D + c] = acc / (double)(t1 - t0);
        }
    }
    return ORA_OK;
}

/* One Oja step on a batch ([OJA] how-it-works display equation and method
 * details):  C = (1/n) X^T X  (the empirical, uncentred second moment of the
 * n feature rows), U' = U + eta (C U - U U^T C U).  No re-orthonormalisation
 * here.  X: [n][D] (rows are tokens), U, Unew: [D][R]. */
int ora_oja_step(const double *X, int64_t n, int64_t D, int64_t R, const double *U, double eta,
                 double *Unew) {
    if (n <= 0 || D <= 0 || R <= 0 || R > D) return ORA_EINVAL;
    double *C = (double *)malloc(sizeof(double) * (size_t)(D * D + D * R + R * R));
    if (!C) return ORA_ENOMEM;
    double *CU = C + D * D, *UtCU = CU + D * R;
    for (int64_t a = 0; a < D; ++a)
        for (int64_t c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int64_t i = 0; i < n; ++i) acc += X[i * D + a] * X[i * D + c];
            C[a * D + c] = acc / (double)n;
        }
    for (int64_t a = 0; a < D; ++a)
        for (int64_t j = 0; j < R; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < D; ++c) acc += C[a * D + c] * U[c * R + j];
            CU[a * R + j] = acc;
        }
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < R; ++j) {
            double acc = 0.0;
            for (int64_t a = 0; a < D; ++a) acc += U[a * R + i] * CU[a * R + j];
            UtCU[i * R + j] = acc;
        }
    for (int64_t a = 0; a < D; ++a)
        for (int64_t j = 0; j < R; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < R; ++i) acc += U[a * R + i] * UtCU[i * R + j];
            Unew[a * R + j] = U[a * R + j] + eta * (CU[a * R + j] - acc);
        }
    free(C);
    return ORA_OK;
}

/* Thin QR by Gram-Schmidt, each column orthogonalised twice against the
 * columns before it ([OJA] method details: re-orthonormalise by QR after
 * every update).  Q: [D][R] with orthonormal columns spanning those of A,
 * taken with a positive diagonal of R, which makes Q unique. */
int ora_qr(const double *A, int64_t D, int64_t R, double *Q) {
    if (D <= 0 || R <= 0 || R > D) return ORA_EINVAL;
    double *v = (double *)malloc(sizeof(double) * (size_t)D);
    if (!v) return ORA_ENOMEM;
    for (int64_t j = 0; j < R; ++j) {
        for (int64_t a = 0; a < D; ++a) v[a] = A[a * R + j];
        for (int pass = 0; pass < 2; ++pass)
            for (int64_t i = 0; i < j; ++i) {
                double dot = 0.0;
                for (int64_t a = 0; a < D; ++a) dot += Q[a * R + i] * v[a];
                for (int64_t a = 0; a < D; ++a) v[a] -= dot * Q[a * R + i];
            }
        double nrm = 0.0;
        for (int64_t a = 0; a < D; ++a) nrm += v[a] * v[a];
        nrm = sqrt(nrm);
        if (!(nrm > 0.0)) {
            free(v);
            return ORA_EINVAL; /* rank deficient */
        }
        for (int64_t a = 0; a < D; ++a) Q[a * R + j] = v[a] / nrm;
    }
    free(v);
    return ORA_OK;
}

/* Basis update for every (layer, kv head) ([OJA] method details, two-phase
 * online update; Algorithm 1): pool each batch row's N tokens with window p,
 * stack the pooled rows of all B sequences (n = B * ceil(N/p) rows), take one
 * Oja step with the empirical second moment, then re-orthonormalise by QR.
 *   U_in : [L][H_kv][D][R] fp32,  U_out : [L][H_kv][D][R] double
 *   X    : [L][B][H_kv][n_stride][D] bf16, first N tokens of each slice used */
int ora_oja_update(int64_t L, int64_t B, int64_t Hkv, int64_t N, int64_t n_stride, int64_t D,
                   int64_t R, const float *U_in, const uint16_t *X, int64_t p, double eta,
                   double *U_out) {
    if (L < 0 || B <= 0 || Hkv <= 0 || N <= 0 || n_stride < N || D <= 0 || R <= 0 || R > D ||
        p <= 0)
        return ORA_EINVAL;
    if (!isfinite(eta)) return ORA_EINVAL;
    int64_t np = (N + p - 1) / p;
    double *Xp = (double *)malloc(sizeof(double) * (size_t)(B * np * D + 2 * D * R));
    if (!Xp) return ORA_ENOMEM;
    double *U = Xp + B * np * D, *Un = U + D * R;
    int rc = ORA_OK;
    for (int64_t l = 0; l < L && rc == ORA_OK; ++l)
        for (int64_t h = 0; h < Hkv && rc == ORA_OK; ++h) {
            for (int64_t b = 0; b < B; ++b) {
                const uint16_t *Xs = X + ((l * B + b) * Hkv + h) * n_stride * D;
                if (!all_finite_bf16(Xs, N * D)) {
                    rc = ORA_ENONFINITE;
                    break;
                }
                ora_avgpool(Xs, N, D, p, Xp + b * np * D);
            }
            if (rc != ORA_OK) break;
            const float *Uh = U_in + (l * Hkv + h) * D * R;
            for (int64_t i = 0; i < D * R; ++i) U[i] = (double)Uh[i];
            rc = ora_oja_step(Xp, B * np, D, R, U, eta, Un);
            if (rc == ORA_OK) rc = ora_qr(Un, D, R, U_out + (l * Hkv + h) * D * R);
        }
    free(Xp);
    return rc;
}

/* ------------------------------------------------------ RippleKV budgets */

/* Per-layer token budgets from per-layer sensitivities ([RKV] sensitivity-
 * guided budget allocation):
 *   s^_l = (s_l - min s) / (max s - min s)   (all 0 when the scores are equal)
 *   w_l  = r^{s^_l}, clipped to [1/gamma, gamma]
 *   b_l  = B * w_l / sum_m w_m               (real budgets summing to B)
 * Readings where the page is silent: a budget above S (a layer cannot keep more
 * tokens than it has) is set to S and the remaining budget is spread again over
 * the other layers in proportion to w, until none exceeds S; integer budgets
 * are the floors plus one for the layers with the largest fractional parts
 * (ties: the lower layer index) until they sum to B.
 * Requires r > 0, gamma >= 1, 0 <= B <= L * S. */
int ora_layer_budgets(const double *s, int64_t L, double r, double gamma, int64_t B, int64_t S,
                      int64_t *k) {
    if (L <= 0 || !s || !k || !(r > 0.0) || !(gamma >= 1.0) || S < 0 || B < 0 || B > L * S)
        return ORA_EINVAL;
    for (int64_t l = 0; l < L; ++l)
        if (!isfinite(s[l])) return ORA_ENONFINITE;
    double *w = (double *)malloc(sizeof(double) * (size_t)L * 2);
    int *capped = (int *)calloc((size_t)L, sizeof(int));
    if (!w || !capped) {
        free(w);
        free(capped);
        return ORA_ENOMEM;
    }
    double *b = w + L;
    double lo = s[0], hi = s[0];
    for (int64_t l = 1; l < L; ++l) {
        if (s[l] < lo) lo = s[l];
        if (s[l] > hi) hi = s[l];
    }
    for (int64_t l = 0; l < L; ++l) {
        double sn = hi > lo ? (s[l] - lo) / (hi - lo) : 0.0;
        double m = pow(r, sn);
        if (m < 1.0 / gamma) m = 1.0 / gamma;
        if (m > gamma) m = gamma;
        w[l] = m;
    }
    /* spread the budget; layers whose share exceeds S are capped and the rest re-spread */
    double left = (double)B;
    for (;;) {
        double wsum = 0.0;
        for (int64_t l = 0; l < L; ++l)
            if (!capped[l]) wsum += w[l];
        int changed = 0;
        for (int64_t l = 0; l < L; ++l) {
            if (capped[l]) continue;
            b[l] = wsum > 0.0 ? left * w[l] / wsum : 0.0;
            if (b[l] > (double)S) {
                capped[l] = 1;
                changed = 1;
            }
        }
        if (!changed) break;
        left = (double)B;
        for (int64_t l = 0; l < L; ++l)
            if (capped[l]) {
                b[l] = (double)S;
                left -= (double)S;
            }
    }
    /* integers: floors, then +1 by largest fractional part (ties: lower layer) */
    int64_t assigned = 0;
    for (int64_t l = 0; l < L; ++l) {
        k[l] = (int64_t)floor(b[l]);
        if (k[l] > S) k[l] = S;
        assigned += k[l];
    }
    while (assigned < B) {
        int64_t best = -1;
        double best_frac = -1.0;
        for (int64_t l = 0; l < L; ++l) {
            if (k[l] >= S) continue;
            double frac = b[l] - (double)k[l];
            if (frac > best_frac) {
                best_frac = frac;
                best = l;
            }
        }
        if (best < 0) break; /* cannot happen when B <= L * S */
        k[best] += 1;
        assigned += 1;
    }
    free(w);
    free(capped);
    return ORA_OK;
}

/* --------------------------------------------------- RefineKV summaries */

/* Cluster summaries ([RFK] "Summarize": the cache is cut into contiguous
 * clusters whose mean keys, mean values and metadata are cached).  For slice g
 * and cluster j = tokens [jc, min((j+1)c, S)):
 *   mu_k[g][j] = mean of its keys, mu_v[g][j] = mean of its values,
 *   radius[g][j] = max_t ||k_t - mu_k[g][j]||_2   (metadata for the logit bound),
 *   vnorm[g][j]  = max_t ||v_t||_2                (metadata for the value bound).
 * Shapes: K, V [G][S][D] bf16; mu_k, mu_v [G][nC][D]; radius, vnorm [G][nC],
 * nC = ceil(S/c). */
int ora_cluster_summaries(const uint16_t *K, const uint16_t *V, int64_t G, int64_t S, int64_t D,
                          int64_t c, double *mu_k, double *mu_v, double *radius, double *vnorm) {
    if (G < 0 || S <= 0 || D <= 0 || c <= 0 || !K || !V || !mu_k || !mu_v || !radius || !vnorm)
        return ORA_EINVAL;
    if (!all_finite_bf16(K, G * S * D) || !all_finite_bf16(V, G * S * D)) return ORA_ENONFINITE;
    int64_t nC = (S + c - 1) / c;
    for (int64_t g = 0; g < G; ++g) {
        const uint16_t *Kg = K + g * S * D, *Vg = V + g * S * D;
        for (int64_t j = 0; j < nC; ++j) {
            int64_t t0 = j * c, t1 = t0 + c < S ? t0 + c : S;
            double *mk = mu_k + (g * nC + j) * D, *mv = mu_v + (g * nC + j) * D;
            centroid_range(Kg, D, t0, t1, mk);
            centroid_range(Vg, D, t0, t1, mv);
            double rmax = 0.0, vmax = 0.0;
            for (int64_t t = t0; t < t1; ++t) {
                double dk = l2_distance(Kg + t * D, mk, D);
                double nv = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    double x = bf16_to_double(Vg[t * D + d]);
                    nv += x * x;
                }
                nv = sqrt(nv);
                if (dk > rmax) rmax = dk;
                if (nv > vmax) vmax = nv;
            }
            radius[g * nC + j] = rmax;
            vnorm[g * nC + j] = vmax;
        }
    }
    return ORA_OK;
}

/* Risk score of every cluster for one query ([RFK] "Select": importance x
 * distortion, and the Figure 2 formula
 *   RC = 2 p_C Vmax [ (cosh d_C - 1) / Dn + tanh(d_C / 2) ],  Dn = sum_C' p_C' cosh d_C').
 * Readings where the page only names the quantities:
 *   p_C  = n_C exp(z_C) / sum_C' n_C' exp(z_C'),  z_C = q . mu_C / sqrt(D)
 *          (the share of attention mass if every key of C had the mean's logit),
 *   d_C  = ||q|| radius_C / sqrt(D)
 *          (|q.k - q.mu_C| / sqrt(D) <= ||q|| ||k - mu_C|| / sqrt(D), Cauchy-Schwarz),
 *   Vmax = max_C vnorm_C (one value bound for the slice, as in Figure 2).
 * mu_k [G][nC][D], radius, vnorm [G][nC]; Q [G][nq][D] bf16 (the queries served
 * by each slice); RC [G][nq][nC]. */
int ora_refine_risk(const double *mu_k, const double *radius, const double *vnorm, int64_t G,
                    int64_t S, int64_t c, int64_t D, const uint16_t *Q, int64_t nq, double *RC) {
    if (G < 0 || S <= 0 || D <= 0 || c <= 0 || nq < 0 || !mu_k || !radius || !vnorm || (nq > 0 && (!Q || !RC)))
        return ORA_EINVAL;
    if (!all_finite_bf16(Q, G * nq * D)) return ORA_ENONFINITE;
    int64_t nC = (S + c - 1) / c;
    double *z = (double *)malloc(sizeof(double) * (size_t)nC);
    if (!z) return ORA_ENOMEM;
    double rs = 1.0 / sqrt((double)D);
    for (int64_t g = 0; g < G; ++g) {
        double vmax = 0.0;
        for (int64_t j = 0; j < nC; ++j)
            if (vnorm[g * nC + j] > vmax) vmax = vnorm[g * nC + j];
        for (int64_t i = 0; i < nq; ++i) {
            const uint16_t *q = Q + (g * nq + i) * D;
            double qn = 0.0, zmax = -INFINITY;
            for (int64_t d = 0; d < D; ++d) qn += bf16_to_double(q[d]) * bf16_to_double(q[d]);
            qn = sqrt(qn);
            for (int64_t j = 0; j < nC; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(q[d]) * mu_k[(g * nC + j) * D + d];
                z[j] = dot * rs;
                if (z[j] > zmax) zmax = z[j];
            }
            double psum = 0.0;
            for (int64_t j = 0; j < nC; ++j) {
                double n = (double)((j + 1) * c < S ? c : S - j * c);
                z[j] = n * exp(z[j] - zmax); /* unnormalised mass */
                psum += z[j];
            }
            double Dn = 0.0;
            for (int64_t j = 0; j < nC; ++j) Dn += (z[j] / psum) * cosh(qn * radius[g * nC + j] * rs);
            double *out = RC + (g * nq + i) * nC;
            for (int64_t j = 0; j < nC; ++j) {
                double p = z[j] / psum, dl = qn * radius[g * nC + j] * rs;
                out[j] = 2.0 * p * vmax * ((cosh(dl) - 1.0) / Dn + tanh(dl / 2.0));
            }
        }
    }
    free(z);
    return ORA_OK;
}

