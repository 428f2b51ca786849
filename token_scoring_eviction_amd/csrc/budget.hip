// RippleKV per-layer token budgets ("RippleKV: Cross-Layer KV Cache Allocation
// via Perturbation Propagation", sensitivity-guided budget allocation): the
// layer sensitivities are normalised to [0, 1], mapped to multipliers r^s,
// clipped to [1/gamma, gamma], and the global budget B is shared in proportion
// to them.  Host code (a handful of layers); the budgets then drive the per-slice
// select of kvc_topk_compact_ragged.
#include <algorithm>
#include <cmath>
#include <vector>

#include "kvc_internal.h"

extern "C" kvc_status kvc_layer_budgets(const double *sensitivity, int64_t L, double r, double gamma,
                                        int64_t B, int64_t S, int64_t *k_out) {
    if (!sensitivity || !k_out || L <= 0 || S < 0 || B < 0) return KVC_ERR_INVALID_ARGUMENT;
    if (!(r > 0.0) || !(gamma >= 1.0) || !std::isfinite(r) || !std::isfinite(gamma))
        return KVC_ERR_INVALID_ARGUMENT;
    if (S > 0 && L > INT64_MAX / S) return KVC_ERR_UNSUPPORTED;
    if (B > L * S) return KVC_ERR_INVALID_ARGUMENT;
    for (int64_t l = 0; l < L; ++l)
        if (!std::isfinite(sensitivity[l])) return KVC_ERR_INVALID_ARGUMENT;

    const auto mm = std::minmax_element(sensitivity, sensitivity + L);
    const double lo = *mm.first, hi = *mm.second;
    std::vector<double> mult(L), share(L, 0.0);
    std::vector<char> full(L, 0);
    for (int64_t l = 0; l < L; ++l) {
        const double norm = hi > lo ? (sensitivity[l] - lo) / (hi - lo) : 0.0;
        mult[l] = std::min(std::max(std::pow(r, norm), 1.0 / gamma), gamma);
    }
    // Shares in proportion to the multipliers.  A layer cannot keep more than its
    // S tokens: such a layer is pinned at S and the rest of the budget is shared
    // again by the others (each round pins at least one more layer).
    int64_t pinned = 0;
    for (;;) {
        const double budget = static_cast<double>(B) - static_cast<double>(S) * static_cast<double>(pinned);
        double wsum = 0.0;
        for (int64_t l = 0; l < L; ++l)
            if (!full[l]) wsum += mult[l];
        bool pinned_more = false;
        for (int64_t l = 0; l < L; ++l) {
            if (full[l]) continue;
            share[l] = wsum > 0.0 ? budget * mult[l] / wsum : 0.0;
            if (share[l] > static_cast<double>(S)) {
                full[l] = 1;
                pinned_more = true;
            }
        }
        if (!pinned_more) break;
        pinned = 0;
        for (int64_t l = 0; l < L; ++l)
            if (full[l]) {
                share[l] = static_cast<double>(S);
                ++pinned;
            }
    }
    // Whole tokens: floors, then one more for the largest fractional parts
    // (equal parts: the lower layer first) until the budgets add up to B.
    int64_t given = 0;
    for (int64_t l = 0; l < L; ++l) {
        k_out[l] = std::min<int64_t>(static_cast<int64_t>(std::floor(share[l])), S);
        given += k_out[l];
    }
    while (given < B) {
        int64_t pick = -1;
        double best = -1.0;
        for (int64_t l = 0; l < L; ++l) {
            if (k_out[l] >= S) continue;
            const double part = share[l] - static_cast<double>(k_out[l]);
            if (part > best) {
                best = part;
                pick = l;
            }
        }
        if (pick < 0) return KVC_ERR_INVALID_ARGUMENT;  // unreachable when B <= L * S
        ++k_out[pick];
        ++given;
    }
    return KVC_OK;
}
