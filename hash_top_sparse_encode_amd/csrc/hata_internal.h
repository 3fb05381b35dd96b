// Internal declarations shared by the host runtime (api.cpp) and the HIP
// kernel sources.  Not part of the public ABI (that is include/hata.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hata {

constexpr int kHeadDim = 128;
constexpr int kBits = 128;
constexpr int kWords = 4;

// ctrl[] word assignment (see hata_cache.ctrl in include/hata.h): global
// words first, then one 64-word (256-byte) line per (batch, KV head) unit
// and one per batch entry for the decode kernel.
constexpr int kCtrlStatus = 0;
constexpr int kCtrlAppendDone = 1;
constexpr int kCtrlUnitBase = 16;

// Decode-step plan: how the context is cut into scan chunks and attention
// splits, and where each buffer sits in the workspace.  A pure function of
// (batch, heads, max_ctx, code length) so hata_decode_workspace_bytes and
// hata_decode_attn agree.
struct DecodePlan {
    int B = 0, Hq = 0, Hkv = 0, G = 0, R = 0, NB = 0;
    int64_t max_ctx = 0;
    int64_t span = 0;    // keys per work item (scan and selection of one span)
    int n_chunks = 0;    // work items per unit: ceil(max_ctx / span)
    int n_items = 0;     // workgroups of the launch
    int64_t sstride = 0; // score row stride (elements) in the workspace
    size_t off_gen = 0, off_qtag = 0, off_unit_hist = 0, off_chunk_hist = 0, off_part_ml = 0,
           off_part_o = 0, off_scores = 0, total = 0;
    // Bytes actually touched: the score rows are used only when a span is
    // longer than the 8192 keys an item keeps in LDS.
    size_t used = 0;
};

bool make_decode_plan(int B, int Hq, int Hkv, int64_t max_ctx, int n_bits, DecodePlan *p);

// ---- launchers (return hipSuccess or the launch error) ----

hipError_t launch_append_exact(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                               int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                               const uint16_t *k_new, const uint16_t *v_new,
                               const int32_t *n_new, int t_max, const float *w,
                               hipStream_t s);

// The matrix-core bulk encoder is used from kMfmaMinRows rows on (rows read
// as 16-byte pieces, so keys / k_new / v_new 16-byte aligned and strides
// multiples of 8 elements).
constexpr int kMfmaMinRows = 64;

// Shapes the bulk encoder indexes in 32 bits: fewer than 2^32 groups of 64
// rows over all batch entries, and 63 row steps (elements) below 2^31.
inline bool rows_shape_fits(int64_t rows_per_entry, int64_t n_entries, int64_t row_step) {
    if (rows_per_entry < 0 || n_entries <= 0 || row_step < 0) return false;
    const int64_t groups = (rows_per_entry + 63) / 64;
    return groups <= (int64_t)0xFFFFFFFF / n_entries && row_step < ((int64_t)1 << 31) / 63;
}

// Bulk encoder on the matrix cores for every code length (encode_rows.hip):
// flat rows, and cache appends (K / V rows copied when k_new is given, the
// last workgroup publishes the lengths).  Same bits as the exact kernels.
hipError_t launch_encode_rows(const uint16_t *keys, int64_t n_rows, int n_heads, int64_t row_stride,
                              int64_t head_stride, const float *w, int n_bits, uint32_t *codes,
                              hipStream_t s);
hipError_t launch_append_rows(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                              int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                              const uint16_t *k_new, const uint16_t *v_new, const int32_t *n_new,
                              int t_max, const float *w, int n_bits, hipStream_t s);

hipError_t launch_encode_exact(const uint16_t *keys, int64_t n_rows, int n_heads,
                               int64_t row_stride, int64_t head_stride, const float *w,
                               uint32_t *codes, hipStream_t s);

// One decode step as a single persistent kernel.  k_new / v_new (bf16
// [B][Hkv][128]) append one token per sequence first; both null: no append.
hipError_t launch_decode(const DecodePlan &p, uint16_t *k_cache, uint16_t *v_cache,
                         uint32_t *codes, int32_t *seq_len, int32_t *ctrl,
                         const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                         const float *w, const int32_t *topk, int k_max, uint16_t *out, void *ws,
                         int32_t *sel_idx_out, uint16_t *scores_out, hipStream_t s);

// ---- training of W_H (train.hip) ----

constexpr int kMaxLabelKeys = 4096;  // keys per label batch (sorted in LDS)

struct TrainPlan {
    int n_q = 0, n_k = 0, n = 0, r = 0, n_parts = 0;
    size_t off_x = 0, off_h = 0, off_slope = 0, off_sb = 0, off_sa = 0, off_rs = 0, off_cs = 0,
           off_e = 0, off_mu = 0, off_gy = 0, off_grad = 0, off_colpart = 0, off_losspart = 0,
           total = 0;
};

struct TrainHyper {
    float sigma, epsilon, eta, lambda, lr, beta1, beta2, adam_eps;
};

bool make_train_plan(int n_q, int n_k, int n_bits, TrainPlan *p);

hipError_t launch_hash_labels(const uint16_t *q, int n_q, const uint16_t *k, int n_k, float *labels,
                              hipStream_t s);

hipError_t launch_hash_train_step(const TrainPlan &p, const uint16_t *q, const uint16_t *k,
                                  const float *labels, float *w, float *adam_m, float *adam_v,
                                  int step, const TrainHyper &hp, float *loss_out, float *grad_out,
                                  void *ws, hipStream_t s);

// The allocation-free decode step's scratch: a static device array of
// kStaticScratchBytes per GPU inside the library.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;

// hata_decode_step on that scratch: looks its address up once per device,
// clears the sections that must start at zero, then launches as
// launch_decode.  hipErrorInvalidValue if the plan needs more than the
// scratch holds.
hipError_t launch_decode_static(const DecodePlan &p, uint16_t *k_cache, uint16_t *v_cache,
                                uint32_t *codes, int32_t *seq_len, int32_t *ctrl,
                                const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                                const float *w, const int32_t *topk, int k_max, uint16_t *out,
                                int32_t *sel_idx_out, uint16_t *scores_out, hipStream_t s);

}  // namespace hata
