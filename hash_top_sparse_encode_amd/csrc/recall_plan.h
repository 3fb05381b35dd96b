// Internal declarations of the recall analysis, shared by the host runtime
// (api.cpp) and recall.hip.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hata {

// Recall analysis (exact top-k against the Hamming selection): workspace
// layout, a pure function of (batch, heads, max_ctx).
struct RecallPlan {
    int B = 0, Hq = 0, Hkv = 0, G = 0, n_kblk = 0;
    int64_t max_ctx = 0, zstride = 0;
    size_t off_zq = 0, off_norm2 = 0, off_band_idx = 0, off_band_z = 0, off_member = 0,
           total = 0;
};

bool make_recall_plan(int B, int Hq, int Hkv, int64_t max_ctx, RecallPlan *p);

hipError_t launch_recall(const RecallPlan &p, int n_bits, const uint16_t *k_cache, const int32_t *seq_len,
                         const uint16_t *q, const int32_t *topk, int k_max,
                         const int32_t *sel_idx, const uint16_t *scores, int32_t *overlap,
                         int32_t *tie, int32_t *exact_idx, void *ws, hipStream_t s);

}  // namespace hata
