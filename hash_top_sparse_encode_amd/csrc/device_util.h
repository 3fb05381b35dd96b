// Device helpers for the gfx950 kernels: bf16 conversion, 64-lane wave and
// 256-thread block scans, exact sign bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hata {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// float -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Exclusive prefix sum over the 256 threads of a workgroup (4 waves of 64).
// Every thread must call it; `tmp` is 4 ints of LDS.  *total gets the sum.
__device__ __forceinline__ int block_excl_scan_256(int v, int *tmp, int *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) tmp[w] = x;
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int t = tmp[i];
        pre += (i < w) ? t : 0;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return pre + x - v;
}

// Exclusive prefix sum over the 256 threads of a workgroup for small values
// (0 <= v < 16): per wave, bit-plane ballots counted below each lane
// (mbcnt); across the 4 waves, one LDS exchange.  `tmp` is 8 ints of LDS
// used as two alternating halves (`phase` 0/1), so consecutive calls with
// alternating phases need only one barrier each.  Every thread must call it.
__device__ __forceinline__ int block_excl_scan_small(int v, int *tmp, int phase, int *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int pre = 0, wtot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint64_t m = __ballot((v >> b) & 1);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        pre += below << b;
        wtot += __popcll(m) << b;
    }
    int *slot = tmp + 4 * phase;
    if (lane == 0) slot[w] = wtot;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int x = slot[i];
        base += (i < w) ? x : 0;
        tot += x;
    }
    *total = tot;
    return base + pre;
}

// Sum over the 256 threads of a workgroup (64-bit).
__device__ __forceinline__ long long block_sum_256(long long v, long long *tmp) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if (lane == 0) tmp[w] = v;
    __syncthreads();
    long long t = tmp[0] + tmp[1] + tmp[2] + tmp[3];
    __syncthreads();
    return t;
}

// Column j of W (W[t][j], t = 0..127, column stride 128) into registers, all
// loads issued together so the exact dot product waits for one latency.
__device__ __forceinline__ void load_wcol(const float *__restrict__ wcol, float (&wv)[128]) {
#pragma unroll
    for (int t = 0; t < 128; ++t) wv[t] = wcol[t * 128];
}

// h(x)_j = [sum_{t=0..127} x_t * W[t][j] > 0] as a sequential double sum in
// ascending t.  Every product bf16 x fp32 is exact in double, so the fused
// multiply-add rounds exactly like add-after-multiply, and the result is the
// same as the plain double loop.  x: 128 floats (bf16 values), typically LDS.
__device__ __forceinline__ bool exact_sign(const float *x, const float (&wv)[128]) {
    double y = 0.0;
#pragma unroll
    for (int t = 0; t < 128; ++t) y = fma((double)x[t], (double)wv[t], y);
    return y > 0.0;
}

}  // namespace hata
