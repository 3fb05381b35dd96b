// Internal declarations of the encoders for code lengths other than 128 bits
// (32, 64 or 256), shared by the host runtime (api.cpp) and bits.hip.  Not
// part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hata {

hipError_t launch_encode_bits(const uint16_t *keys, int64_t n_rows, int n_heads,
                              int64_t row_stride, int64_t head_stride, const float *w,
                              int n_bits, uint32_t *codes, hipStream_t s);

hipError_t launch_append_bits(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                              int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                              const uint16_t *k_new, const uint16_t *v_new, const int32_t *n_new,
                              int t_max, const float *w, int n_bits, hipStream_t s);

}  // namespace hata
