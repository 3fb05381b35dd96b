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

// DPP controls (GFX9 encoding): row_shr:n is kDppRowShr + n; row_bcast:15 and
// row_bcast:31 pass lane 15 (31) of a group of rows on to the following rows.
constexpr int kDppRowShr = 0x110, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes of a wave: a shift-and-add scan
// within each row of 16 lanes, then each row adds the totals of the rows
// before it (row_bcast:15 for rows 1 and 3, row_bcast:31 for rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 1, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 2, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 4, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 8, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xC, 0xF, false);
    return x;
}

// Sum over the lanes of a wave, in a scalar register.
__device__ __forceinline__ int wave_sum(int x) {
    return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

// Exclusive prefix sum over the 256 threads of a workgroup (4 waves of 64).
// Every thread must call it; `tmp` is 4 ints of LDS.  *total gets the sum.
__device__ __forceinline__ int block_excl_scan_256(int v, int *tmp, int *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
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

// Sums over the 256 threads of a workgroup of two values at once (each sum
// must fit in an int); `tmp` is 8 ints of LDS, written here and read after
// one barrier.  Every thread must call it.
__device__ __forceinline__ void block_sum2_256(int a, int b, int *tmp, int *sa, int *sb) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wa = wave_sum(a), wb = wave_sum(b);
    if (lane == 0) {
        tmp[w] = wa;
        tmp[4 + w] = wb;
    }
    __syncthreads();
    *sa = tmp[0] + tmp[1] + tmp[2] + tmp[3];
    *sb = tmp[4] + tmp[5] + tmp[6] + tmp[7];
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
