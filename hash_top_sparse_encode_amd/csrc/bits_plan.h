// Internal declarations of the decode path for code lengths other than 128
// bits (32, 64 or 256), shared by the host runtime (api.cpp) and bits.hip.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hata {

constexpr int kBSpan = 8192;   // keys per scan / compaction workgroup
constexpr int kBChunk = 256;   // selected keys per attention workgroup

// Workspace layout of the multi-launch decode for r in {32, 64, 256}: a pure
// function of (batch, heads, max_ctx, r, k_max).
struct BitsPlan {
    int B = 0, Hq = 0, Hkv = 0, G = 0, R = 0, NB = 0, NBpad = 0, n_span = 0, n_chunk = 0;
    int k_max = 0;
    int64_t max_ctx = 0;
    size_t off_qcodes = 0, off_scores = 0, off_span_hist = 0, off_info = 0,
           off_sel = 0, off_part = 0, total = 0;
};

bool make_bits_plan(int B, int Hq, int Hkv, int64_t max_ctx, int n_bits, int k_max,
                    BitsPlan *p);

hipError_t launch_encode_bits(const uint16_t *keys, int64_t n_rows, int n_heads,
                              int64_t row_stride, int64_t head_stride, const float *w,
                              int n_bits, uint32_t *codes, hipStream_t s);

hipError_t launch_append_bits(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                              int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                              const uint16_t *k_new, const uint16_t *v_new, const int32_t *n_new,
                              int t_max, const float *w, int n_bits, hipStream_t s);

// k_new / v_new (bf16 [B][Hkv][128]) append one token per sequence first;
// both null: no append.
hipError_t launch_decode_bits(const BitsPlan &p, uint16_t *k_cache, uint16_t *v_cache,
                              uint32_t *codes, int32_t *seq_len, int32_t *ctrl,
                              const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                              const float *w, const int32_t *topk, uint16_t *out, void *ws,
                              int32_t *sel_idx_out, uint16_t *scores_out, hipStream_t s);

}  // namespace hata
