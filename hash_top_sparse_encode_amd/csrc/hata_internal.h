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
// (batch, heads, max_ctx) so hata_decode_workspace_bytes and
// hata_decode_attn agree.
struct DecodePlan {
    int B = 0, Hq = 0, Hkv = 0, G = 0, NB = 0;
    int64_t max_ctx = 0;
    int64_t span = 0;    // keys per work item (scan and selection of one span)
    int n_chunks = 0;    // work items per unit: ceil(max_ctx / span)
    int n_items = 0;     // workgroups of the launch
    int64_t sstride = 0; // score row stride (elements) in the workspace
    size_t off_gen = 0, off_qtag = 0, off_unit_hist = 0, off_chunk_hist = 0, off_part_ml = 0,
           off_part_o = 0, off_scores = 0, total = 0;
};

bool make_decode_plan(int B, int Hq, int Hkv, int64_t max_ctx, DecodePlan *p);

// ---- launchers (return hipSuccess or the launch error) ----

hipError_t launch_append_exact(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                               int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                               const uint16_t *k_new, const uint16_t *v_new,
                               const int32_t *n_new, int t_max, const float *w,
                               hipStream_t s);

// Bulk encoder on the matrix cores (identical bits; rows read as 16-byte
// pieces, so keys / k_new / v_new 16-byte aligned and strides multiples of
// 8 elements).  Used from kMfmaMinRows rows on.
constexpr int kMfmaMinRows = 64;

hipError_t launch_append_mfma(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                              int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                              const uint16_t *k_new, const uint16_t *v_new,
                              const int32_t *n_new, int t_max, const float *w, hipStream_t s);

hipError_t launch_encode_mfma(const uint16_t *keys, int64_t n_rows, int n_heads, int64_t row_stride,
                              int64_t head_stride, const float *w, uint32_t *codes, hipStream_t s);

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

}  // namespace hata
