// Host runtime behind include/hata.h: argument validation, workspace plan,
// kernel launch sequencing.  Everything is enqueued on the caller's stream;
// nothing here allocates, synchronises or reads device memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hata.h"
#include "hata_internal.h"
#include "recall_plan.h"
#include "bits_plan.h"

using namespace hata;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_bits(int n_bits) {
    return n_bits == 32 || n_bits == 64 || n_bits == 128 || n_bits == 256;
}

hata_status check_cache(const hata_cache *c) {
    if (!c) return HATA_ERR_INVALID_ARG;
    if (c->head_dim != kHeadDim || !supported_bits(c->n_bits)) return HATA_ERR_UNSUPPORTED;
    if (c->batch <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0) return HATA_ERR_INVALID_ARG;
    if (c->n_q_heads % c->n_kv_heads) return HATA_ERR_UNSUPPORTED;
    const int G = c->n_q_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return HATA_ERR_UNSUPPORTED;
    if ((int64_t)c->batch * c->n_kv_heads > 65535) return HATA_ERR_UNSUPPORTED;
    if (c->max_ctx < 0 || c->max_ctx > (int64_t)INT32_MAX - 1) return HATA_ERR_INVALID_ARG;
    if (!c->k || !c->v || !c->codes || !c->seq_len || !c->ctrl) return HATA_ERR_INVALID_ARG;
    if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(c->codes)) return HATA_ERR_INVALID_ARG;
    return HATA_OK;
}

}  // namespace

extern "C" {

const char *hata_status_string(hata_status s) {
    switch (s) {
        case HATA_OK: return "ok";
        case HATA_ERR_INVALID_ARG: return "invalid argument";
        case HATA_ERR_UNSUPPORTED:
            return "unsupported shape (head_dim 128, n_bits in {32, 64, 128, 256}, G in {1, 2, 4, 8})";
        case HATA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case HATA_ERR_HIP: return "HIP launch failed";
        case HATA_ERR_SCRATCH_LIMIT:
            return "the cache needs more decode scratch than the allocation-free entry point holds";
    }
    return "unknown status";
}

hata_status hata_encode_keys(const uint16_t *keys, int64_t n_rows, int32_t n_heads,
                             int64_t row_stride, int64_t head_stride, const float *w_h,
                             uint32_t *codes_out, void *stream) {
    if (n_rows < 0 || n_heads <= 0 || n_heads > 65535) return HATA_ERR_INVALID_ARG;
    if (n_rows == 0) return HATA_OK;
    if (!keys || !w_h || !codes_out) return HATA_ERR_INVALID_ARG;
    if (row_stride < 0 || head_stride < 0) return HATA_ERR_INVALID_ARG;
    if (n_heads > 1 && head_stride < kHeadDim && row_stride < kHeadDim) return HATA_ERR_INVALID_ARG;
    // Bulk calls on the matrix cores (16-byte row pieces), small ones exact;
    // both give the same bits.
    const bool mfma = n_rows >= kMfmaMinRows && aligned16(keys) && row_stride % 8 == 0 &&
                      head_stride % 8 == 0 && aligned16(codes_out) &&
                      rows_shape_fits(n_rows, 1, row_stride);
    hipError_t e = mfma ? launch_encode_rows(keys, n_rows, n_heads, row_stride, head_stride, w_h,
                                             kBits, codes_out, static_cast<hipStream_t>(stream))
                        : launch_encode_exact(keys, n_rows, n_heads, row_stride, head_stride, w_h,
                                              codes_out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HATA_OK : HATA_ERR_HIP;
}

hata_status hata_encode_keys_nbits(const uint16_t *keys, int64_t n_rows, int32_t n_heads,
                                   int64_t row_stride, int64_t head_stride, const float *w_h,
                                   int32_t n_bits, uint32_t *codes_out, void *stream) {
    if (!supported_bits(n_bits)) return HATA_ERR_UNSUPPORTED;
    if (n_bits == kBits)
        return hata_encode_keys(keys, n_rows, n_heads, row_stride, head_stride, w_h, codes_out,
                                stream);
    if (n_rows < 0 || n_heads <= 0 || n_heads > 65535) return HATA_ERR_INVALID_ARG;
    if (n_rows == 0) return HATA_OK;
    if (!keys || !w_h || !codes_out) return HATA_ERR_INVALID_ARG;
    if (row_stride < 0 || head_stride < 0) return HATA_ERR_INVALID_ARG;
    if (n_heads > 1 && head_stride < kHeadDim && row_stride < kHeadDim) return HATA_ERR_INVALID_ARG;
    if (!aligned16(keys) || row_stride % 8 || head_stride % 8) return HATA_ERR_INVALID_ARG;
    hipError_t e = n_rows >= kMfmaMinRows && aligned16(codes_out) &&
                           rows_shape_fits(n_rows, 1, row_stride)
                       ? launch_encode_rows(keys, n_rows, n_heads, row_stride, head_stride, w_h,
                                            n_bits, codes_out, static_cast<hipStream_t>(stream))
                       : launch_encode_bits(keys, n_rows, n_heads, row_stride, head_stride, w_h,
                                            n_bits, codes_out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HATA_OK : HATA_ERR_HIP;
}

hata_status hata_append(const hata_cache *c, const uint16_t *k_new, const uint16_t *v_new,
                        const int32_t *n_new, int32_t t_max, const float *w_h, void *stream) {
    hata_status st = check_cache(c);
    if (st != HATA_OK) return st;
    if (t_max < 0 || !n_new || !w_h) return HATA_ERR_INVALID_ARG;
    if ((k_new == nullptr) != (v_new == nullptr)) return HATA_ERR_INVALID_ARG;
    if (t_max == 0) return HATA_OK;
    if (c->n_bits != kBits) {
        if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return HATA_ERR_INVALID_ARG;
        hipError_t e = t_max >= kMfmaMinRows &&
                               rows_shape_fits(t_max, c->batch, k_new ? (int64_t)c->n_kv_heads * kHeadDim : kHeadDim)
                           ? launch_append_rows(c->k, c->v, c->codes, c->seq_len, c->ctrl, c->batch,
                                                c->n_kv_heads, c->max_ctx, k_new, v_new, n_new,
                                                t_max, w_h, c->n_bits, static_cast<hipStream_t>(stream))
                           : launch_append_bits(c->k, c->v, c->codes, c->seq_len, c->ctrl, c->batch,
                                                c->n_kv_heads, c->max_ctx, k_new, v_new, n_new,
                                                t_max, w_h, c->n_bits, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? HATA_OK : HATA_ERR_HIP;
    }
    const bool mfma = t_max >= kMfmaMinRows && (k_new == nullptr || (aligned16(k_new) && aligned16(v_new))) &&
                      rows_shape_fits(t_max, c->batch, k_new ? (int64_t)c->n_kv_heads * kHeadDim : kHeadDim);
    hipError_t e = mfma ? launch_append_rows(c->k, c->v, c->codes, c->seq_len, c->ctrl, c->batch,
                                             c->n_kv_heads, c->max_ctx, k_new, v_new, n_new, t_max,
                                             w_h, kBits, static_cast<hipStream_t>(stream))
                        : launch_append_exact(c->k, c->v, c->codes, c->seq_len, c->ctrl, c->batch,
                                              c->n_kv_heads, c->max_ctx, k_new, v_new, n_new, t_max,
                                              w_h, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HATA_OK : HATA_ERR_HIP;
}

size_t hata_decode_workspace_bytes(const hata_cache *c, int32_t k_max) {
    if (!c || k_max < 0) return 0;
    if (c->head_dim != kHeadDim || !supported_bits(c->n_bits)) return 0;
    DecodePlan p;
    if (!make_decode_plan(c->batch, c->n_q_heads, c->n_kv_heads, c->max_ctx, c->n_bits, &p)) return 0;
    return p.total;
}

static hata_status decode_common(const hata_cache *c, const uint16_t *k_new,
                                 const uint16_t *v_new, const uint16_t *q, const float *w_h,
                                 const int32_t *topk, int32_t k_max, uint16_t *out,
                                 void *workspace, size_t ws_bytes, int32_t *sel_idx_out,
                                 uint16_t *scores_out, void *stream) {
    hata_status st = check_cache(c);
    if (st != HATA_OK) return st;
    if (!q || !w_h || !topk || !out || k_max < 0) return HATA_ERR_INVALID_ARG;
    if (!aligned16(q)) return HATA_ERR_INVALID_ARG;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return HATA_ERR_INVALID_ARG;
    DecodePlan p;
    if (!make_decode_plan(c->batch, c->n_q_heads, c->n_kv_heads, c->max_ctx, c->n_bits, &p))
        return HATA_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return HATA_ERR_WORKSPACE;
    hipError_t e = launch_decode(p, c->k, c->v, c->codes, c->seq_len, c->ctrl, k_new, v_new, q,
                                 w_h, topk, k_max, out, workspace, sel_idx_out, scores_out,
                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HATA_OK : HATA_ERR_HIP;
}

hata_status hata_decode_attn(const hata_cache *c, const uint16_t *q, const float *w_h,
                             const int32_t *topk, int32_t k_max, uint16_t *out,
                             void *workspace, size_t ws_bytes, int32_t *sel_idx_out,
                             uint16_t *scores_out, void *stream) {
    return decode_common(c, nullptr, nullptr, q, w_h, topk, k_max, out, workspace, ws_bytes,
                         sel_idx_out, scores_out, stream);
}

hata_status hata_decode_step(const hata_cache *c, const uint16_t *k_new, const uint16_t *v_new,
                             const uint16_t *q, const float *w_h, const int32_t *topk,
                             int32_t k_max, uint16_t *out, void *workspace, size_t ws_bytes,
                             int32_t *sel_idx_out, uint16_t *scores_out, void *stream) {
    if (!k_new || !v_new) return HATA_ERR_INVALID_ARG;
    return decode_common(c, k_new, v_new, q, w_h, topk, k_max, out, workspace, ws_bytes,
                         sel_idx_out, scores_out, stream);
}

hata_status hata_decode_step_static(const hata_cache *c, const uint16_t *k_new,
                                    const uint16_t *v_new, const uint16_t *q, const float *w_h,
                                    const int32_t *topk, int32_t k_max, uint16_t *out,
                                    int32_t *sel_idx_out, uint16_t *scores_out, void *stream) {
    hata_status st = check_cache(c);
    if (st != HATA_OK) return st;
    if (!k_new || !v_new || !q || !w_h || !topk || !out || k_max < 0) return HATA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new)) return HATA_ERR_INVALID_ARG;
    DecodePlan p;
    if (!make_decode_plan(c->batch, c->n_q_heads, c->n_kv_heads, c->max_ctx, c->n_bits, &p))
        return HATA_ERR_UNSUPPORTED;
    if (p.used > kStaticScratchBytes) return HATA_ERR_SCRATCH_LIMIT;
    hipError_t e = launch_decode_static(p, c->k, c->v, c->codes, c->seq_len, c->ctrl, k_new, v_new,
                                        q, w_h, topk, k_max, out, sel_idx_out, scores_out,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HATA_OK : HATA_ERR_HIP;
}

size_t hata_hash_train_workspace_bytes(int32_t n_q, int32_t n_k, int32_t n_bits) {
    TrainPlan p;
    return make_train_plan(n_q, n_k, n_bits, &p) ? p.total : 0;
}

hata_status hata_hash_labels(const uint16_t *q, int32_t n_q, const uint16_t *k, int32_t n_k,
                             float *labels, void *stream) {
    if (n_q < 0 || n_k < 0 || n_k > kMaxLabelKeys) return HATA_ERR_INVALID_ARG;
    if (n_q == 0 || n_k == 0) return HATA_OK;
    if (!q || !k || !labels) return HATA_ERR_INVALID_ARG;
    hipError_t e = launch_hash_labels(q, n_q, k, n_k, labels, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HATA_OK : HATA_ERR_HIP;
}

hata_status hata_hash_train_step(const uint16_t *q, int32_t n_q, const uint16_t *k, int32_t n_k,
                                 const float *labels, int32_t n_bits, float *w_h, float *adam_m,
                                 float *adam_v, int32_t step, const hata_train_params *params,
                                 float *loss_out, float *grad_out, void *workspace,
                                 size_t ws_bytes, void *stream) {
    if (n_bits != 32 && n_bits != 64 && n_bits != 128 && n_bits != 256) return HATA_ERR_UNSUPPORTED;
    if (!q || !k || !labels || !w_h || !params || !loss_out || step < 0) return HATA_ERR_INVALID_ARG;
    if (step > 0 && (!adam_m || !adam_v)) return HATA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k)) return HATA_ERR_INVALID_ARG;
    TrainPlan p;
    if (!make_train_plan(n_q, n_k, n_bits, &p)) return HATA_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return HATA_ERR_WORKSPACE;
    const TrainHyper hp{params->sigma, params->epsilon, params->eta, params->lambda,
                        params->lr, params->beta1, params->beta2, params->adam_eps};
    hipError_t e = launch_hash_train_step(p, q, k, labels, w_h, adam_m, adam_v, step, hp, loss_out,
                                          grad_out, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HATA_OK : HATA_ERR_HIP;
}

size_t hata_recall_workspace_bytes(const hata_cache *c) {
    if (!c) return 0;
    if (c->head_dim != kHeadDim || !supported_bits(c->n_bits)) return 0;
    RecallPlan p;
    if (!make_recall_plan(c->batch, c->n_q_heads, c->n_kv_heads, c->max_ctx, &p)) return 0;
    return p.total;
}

hata_status hata_exact_topk_recall(const hata_cache *c, const uint16_t *q, const int32_t *topk,
                                   int32_t k_max, const int32_t *sel_idx,
                                   const uint16_t *scores, int32_t *overlap_out,
                                   int32_t *tie_out, int32_t *exact_idx_out, void *workspace,
                                   size_t ws_bytes, void *stream) {
    hata_status st = check_cache(c);
    if (st != HATA_OK) return st;
    if (!q || !topk || !sel_idx || !scores || !overlap_out || !tie_out || k_max < 0)
        return HATA_ERR_INVALID_ARG;
    if (!aligned16(q)) return HATA_ERR_INVALID_ARG;
    RecallPlan p;
    if (!make_recall_plan(c->batch, c->n_q_heads, c->n_kv_heads, c->max_ctx, &p))
        return HATA_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return HATA_ERR_WORKSPACE;
    hipError_t e = launch_recall(p, c->n_bits, c->k, c->seq_len, q, topk, k_max, sel_idx, scores,
                                 overlap_out, tie_out, exact_idx_out, workspace,
                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HATA_OK : HATA_ERR_HIP;
}

}  // extern "C"
