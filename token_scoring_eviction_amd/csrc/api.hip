// Library-level entry points of libkvc: version, status text, workspace sizing.
#include "kvc_internal.h"

namespace kvc {
size_t score_workspace_bytes(int64_t G, int64_t S, int64_t W);
size_t topk_workspace_bytes(int64_t G, int64_t S, int64_t k);
size_t topk_ragged_workspace_bytes(int64_t G);
size_t compress_workspace_bytes(const kvc_dims *d);
size_t oja_workspace_bytes(const kvc_dims *d, int64_t pool);
size_t reconstruct_workspace_bytes(const kvc_dims *d);
size_t risk_bytes(int64_t G, int64_t S, int64_t c);
}  // namespace kvc

namespace kvc {
Options &options() {
    static Options opts;
    return opts;
}
}  // namespace kvc

extern "C" int kvc_abi_version(void) { return KVC_ABI_VERSION; }

extern "C" kvc_status kvc_set_option(kvc_option opt, int64_t value) {
    kvc::Options &o = kvc::options();
    switch (opt) {
        case KVC_OPTION_SCORE_PATH:
            if (value < 0 || value > 2) return KVC_ERR_INVALID_ARGUMENT;
            o.score_path.store(value, std::memory_order_relaxed);
            return KVC_OK;
        case KVC_OPTION_SCORE_SPIN_LIMIT:
            if (value < -1 || value > static_cast<int64_t>(UINT32_MAX)) return KVC_ERR_INVALID_ARGUMENT;
            o.spin_limit.store(value, std::memory_order_relaxed);
            return KVC_OK;
        case KVC_OPTION_GATHER_PATH:
            if (value < 0 || value > 1) return KVC_ERR_INVALID_ARGUMENT;
            o.gather_path.store(value, std::memory_order_relaxed);
            return KVC_OK;
        default:
            break;
    }
    return KVC_ERR_INVALID_ARGUMENT;
}

extern "C" kvc_status kvc_workspace_status(const void *ws, hipStream_t stream) {
    if (!ws || !kvc::aligned(ws, kvc::kWsAlign)) return KVC_ERR_INVALID_ARGUMENT;
    if (hipStreamSynchronize(stream) != hipSuccess) return KVC_ERR_HIP;
    uint32_t word = 0;
    if (hipMemcpy(&word, ws, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return KVC_ERR_HIP;
    if (word & kvc::kStatusBadBudget) return KVC_ERR_INVALID_ARGUMENT;
    return KVC_OK;
}

extern "C" const char *kvc_status_str(kvc_status s) {
    switch (s) {
        case KVC_OK: return "ok";
        case KVC_ERR_INVALID_ARGUMENT: return "invalid argument";
        case KVC_ERR_UNSUPPORTED: return "unsupported shape or parameter";
        case KVC_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case KVC_ERR_HIP: return "HIP runtime error";
        case KVC_ERR_WAIT_EXPIRED: return "an in-kernel wait expired (no longer reported)";
        default:
            break;
    }
    return "unknown status";
}

extern "C" size_t kvc_workspace_bytes(kvc_op op, const kvc_dims *d, int64_t k, int64_t W) {
    if (!d) return 0;
    const int64_t G = d->L * d->B * d->H_kv;
    switch (op) {
        case KVC_OP_SCORE_L2: return kvc::score_workspace_bytes(G, d->S, d->S);
        case KVC_OP_SCORE_L2_WINDOWED:
        case KVC_OP_SCORE_CENTROID: return kvc::score_workspace_bytes(G, d->S, W);
        case KVC_OP_TOPK_COMPACT: return kvc::topk_workspace_bytes(G, d->S, k);
        case KVC_OP_LOWRANK_COMPRESS: return kvc::compress_workspace_bytes(d);
        case KVC_OP_OJA_UPDATE: return kvc::oja_workspace_bytes(d, W);
        case KVC_OP_RECONSTRUCT: return kvc::reconstruct_workspace_bytes(d);
        case KVC_OP_TOPK_RAGGED: return kvc::topk_ragged_workspace_bytes(G);
        case KVC_OP_REFINE_RISK: return kvc::risk_bytes(G, d->S, k);
        default:
            break;
    }
    return 0;
}
