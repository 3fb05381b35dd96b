// Exact sign-code encoder kernels (HATA review: h(x) = sign(x W_H), r = 128,
// "Free parameters"; the key-code cache of Algorithm 1, Figure 2 caption).
//
// One workgroup of 128 threads per (row, head): the row is staged in LDS,
// thread j evaluates bit j as a sequential double sum (exact_sign), and
// each 64-lane wave packs its 64 bits with a ballot into two code words.
// Used for small appends (the decode step's one token per sequence), where
// a dense MFMA tile would be mostly empty.
#include "device_util.h"
#include "hata_internal.h"
#include "../../include/hata.h"

namespace hata {

// Pack the wave's 64 sign bits (bit j = lane + 64 * wave) into code words.
__device__ __forceinline__ void store_wave_bits(bool bit, uint32_t *code_row) {
    const uint64_t m = __ballot(bit);
    if ((threadIdx.x & 63) == 0) {
        const int w0 = (threadIdx.x >> 6) * 2;
        code_row[w0] = (uint32_t)m;
        code_row[w0 + 1] = (uint32_t)(m >> 32);
    }
}

__device__ __forceinline__ bool append_entry_valid(int64_t len, int n, int t_max,
                                                   int64_t max_ctx) {
    return n >= 0 && n <= t_max && len >= 0 && len + n <= max_ctx;
}

// grid: x = token t in [0, t_max), y = b * Hkv + kv.  block: 128.
__global__ __launch_bounds__(128) void k_append_exact(
    uint16_t *__restrict__ k_cache, uint16_t *__restrict__ v_cache, uint32_t *__restrict__ codes,
    int32_t *__restrict__ seq_len, int32_t *__restrict__ ctrl, int B, int Hkv, int64_t max_ctx,
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    const int32_t *__restrict__ n_new, int t_max, const float *__restrict__ w) {
    __shared__ float x[kHeadDim];
    __shared__ int s_last;
    const int t = blockIdx.x, unit = blockIdx.y, b = unit / Hkv, kv = unit % Hkv;
    const int j = threadIdx.x;
    const int64_t len = seq_len[b];
    const int n = n_new[b];
    const bool ok = append_entry_valid(len, n, t_max, max_ctx);
    if (ok && t < n) {
        const int64_t pos = len + t;
        const int64_t crow = ((int64_t)unit * max_ctx + pos) * kHeadDim;
        uint16_t kb;
        if (k_new) {
            const int64_t nrow = (((int64_t)b * t_max + t) * Hkv + kv) * kHeadDim;
            kb = k_new[nrow + j];
            k_cache[crow + j] = kb;
            v_cache[crow + j] = v_new[nrow + j];
        } else {
            kb = k_cache[crow + j];
        }
        float wv[kHeadDim];
        load_wcol(w + (int64_t)kv * kHeadDim * kBits + j, wv);
        x[j] = bf16_to_f32(kb);
        __syncthreads();
        const bool bit = exact_sign(x, wv);
        store_wave_bits(bit, codes + ((int64_t)unit * max_ctx + pos) * kWords);
    }
    // The last workgroup to finish publishes the new lengths: every
    // workgroup has read seq_len[] by then.
    __syncthreads();
    if (j == 0) {
        __threadfence();
        const unsigned total = gridDim.x * gridDim.y;
        const unsigned prev = atomicAdd((unsigned *)&ctrl[kCtrlAppendDone], 1u);
        s_last = (prev == total - 1);
    }
    __syncthreads();
    if (s_last) {
        __threadfence();
        for (int bb = j; bb < B; bb += blockDim.x) {
            const int64_t l = seq_len[bb];
            const int nn = n_new[bb];
            if (append_entry_valid(l, nn, t_max, max_ctx)) {
                seq_len[bb] = (int32_t)(l + nn);
            } else {
                const int flag = (nn < 0 || nn > t_max) ? HATA_DEV_BAD_NEW : HATA_DEV_APPEND_OVERFLOW;
                atomicOr(&ctrl[kCtrlStatus], flag);
            }
        }
        if (j == 0) ctrl[kCtrlAppendDone] = 0;
    }
}

// grid: x = row, y = head.  block: 128.  codes [n_rows][n_heads][4].
__global__ __launch_bounds__(128) void k_encode_exact(const uint16_t *__restrict__ keys,
                                                      int64_t row_stride, int64_t head_stride,
                                                      const float *__restrict__ w,
                                                      uint32_t *__restrict__ codes,
                                                      int n_heads, int64_t row0) {
    __shared__ float x[kHeadDim];
    const int64_t row = row0 + blockIdx.x;
    const int h = blockIdx.y, j = threadIdx.x;
    float wv[kHeadDim];
    load_wcol(w + (int64_t)h * kHeadDim * kBits + j, wv);
    x[j] = bf16_to_f32(keys[row * row_stride + (int64_t)h * head_stride + j]);
    __syncthreads();
    const bool bit = exact_sign(x, wv);
    store_wave_bits(bit, codes + (row * n_heads + h) * kWords);
}

hipError_t launch_append_exact(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                               int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                               const uint16_t *k_new, const uint16_t *v_new,
                               const int32_t *n_new, int t_max, const float *w,
                               hipStream_t s) {
    dim3 grid((unsigned)t_max, (unsigned)(B * Hkv));
    hipLaunchKernelGGL(k_append_exact, grid, dim3(128), 0, s, k_cache, v_cache, codes, seq_len,
                       ctrl, B, Hkv, max_ctx, k_new, v_new, n_new, t_max, w);
    return hipGetLastError();
}

hipError_t launch_encode_exact(const uint16_t *keys, int64_t n_rows, int n_heads,
                               int64_t row_stride, int64_t head_stride, const float *w,
                               uint32_t *codes, hipStream_t s) {
    const int64_t kMaxX = 1 << 30;
    for (int64_t r0 = 0; r0 < n_rows; r0 += kMaxX) {
        const int64_t n = n_rows - r0 < kMaxX ? n_rows - r0 : kMaxX;
        hipLaunchKernelGGL(k_encode_exact, dim3((unsigned)n, (unsigned)n_heads), dim3(128), 0, s,
                           keys, row_stride, head_stride, w, codes, n_heads, r0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace hata
