// Decode-step append of the OjaKV loop ("OjaKV: Context-Aware Online Low-Rank KV
// Cache Compression", method details and appendix A.1: each decoded token's key
// and value join the cache and the update buffer; the step's queries join the
// window that scores the next update).  One launch copies every new row to its
// places: 16 lanes per 256-byte row, 16-byte loads and stores.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kRowsPerBlock = kAppendThreads / 16;

__global__ __launch_bounds__(kAppendThreads) void decode_append_kernel(
    int64_t G, int64_t nq_rows, int64_t S_stride, int64_t pos, int64_t T, int64_t slot,
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new, const uint16_t *__restrict__ q_new,
    uint16_t *__restrict__ K, uint16_t *__restrict__ V, uint16_t *__restrict__ K_buf,
    uint16_t *__restrict__ V_buf, uint16_t *__restrict__ Q_buf) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 4);
    const int lane16 = threadIdx.x & 15;
    constexpr int64_t kRow = kHeadDim / 8;  // 16-byte pieces per row
    if (row < G) {  // key and value of slice `row`
        const uint4 kv = reinterpret_cast<const uint4 *>(k_new)[row * kRow + lane16];
        const uint4 vv = reinterpret_cast<const uint4 *>(v_new)[row * kRow + lane16];
        reinterpret_cast<uint4 *>(K)[(row * S_stride + pos) * kRow + lane16] = kv;
        reinterpret_cast<uint4 *>(V)[(row * S_stride + pos) * kRow + lane16] = vv;
        if (K_buf) reinterpret_cast<uint4 *>(K_buf)[(row * T + slot) * kRow + lane16] = kv;
        if (V_buf) reinterpret_cast<uint4 *>(V_buf)[(row * T + slot) * kRow + lane16] = vv;
    } else if (row < G + nq_rows && q_new) {  // query head row - G, into its window slot
        const int64_t h = row - G;
        reinterpret_cast<uint4 *>(Q_buf)[(h * T + slot) * kRow + lane16] =
            reinterpret_cast<const uint4 *>(q_new)[h * kRow + lane16];
    }
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_decode_append(const kvc_dims *d, int64_t pos, int64_t T, int64_t slot,
                                        const uint16_t *k_new, const uint16_t *v_new,
                                        const uint16_t *q_new, uint16_t *K, uint16_t *V,
                                        uint16_t *K_buf, uint16_t *V_buf, uint16_t *Q_buf,
                                        hipStream_t stream) {
    using namespace kvc;
    if (!d || d->L < 0 || d->B < 0 || d->H_kv < 0 || d->H_q < 0 || d->D <= 0) return KVC_ERR_INVALID_ARGUMENT;
    if (d->D != kHeadDim) return KVC_ERR_UNSUPPORTED;
    const int64_t stride = d->S_stride ? d->S_stride : d->S;
    if (pos < 0 || pos >= stride || T < 1 || slot < 0 || slot >= T) return KVC_ERR_INVALID_ARGUMENT;
    const int64_t G = d->L * d->B * d->H_kv;
    const int64_t nq = q_new ? d->L * d->B * d->H_q : 0;
    if (G == 0 && nq == 0) return KVC_OK;
    if (G > 0 && (!k_new || !v_new || !K || !V)) return KVC_ERR_INVALID_ARGUMENT;
    if ((K_buf == nullptr) != (V_buf == nullptr) || (q_new && !Q_buf)) return KVC_ERR_INVALID_ARGUMENT;
    const void *ptrs[] = {k_new, v_new, q_new, K, V, K_buf, V_buf, Q_buf};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return KVC_ERR_INVALID_ARGUMENT;
    const int64_t blocks = (G + nq + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks > INT32_MAX) return KVC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(decode_append_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kAppendThreads), 0, stream,
                       G, nq, stride, pos, T, slot, k_new, v_new, q_new, K, V, K_buf, V_buf, Q_buf);
    return launch_status();
}
