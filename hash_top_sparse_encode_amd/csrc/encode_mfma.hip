// Bulk sign-code encoder on the matrix cores (HATA review: h(x) = sign(x W_H)
// with r = 128 bits per head, "Free parameters"; the key-code cache of
// Algorithm 1 in the Figure 2 caption).  Used for prefill appends and
// hata_encode_keys; the decode step's single token per sequence uses the
// exact kernels.
//
// x W_H is a dense contraction: rows of x (bf16) against the 128 x 128 fp32
// W_H of their head.  W_H is split into two bf16 terms, W = W_hi + W_lo + r
// with |r| <= 2^-16 |W|, and y' = x W_hi + x W_lo is accumulated in fp32 by
// v_mfma_f32_16x16x32_bf16 (bf16 x bf16 products are exact in fp32).  Then
// |y' - x W| <= (2^-16 + gamma_256 (1 + 2^-7)) sum_t |x_t| |W_tj|
//            <= 3.1e-5 ||x||_2 ||W_:j||_2,
// and the sequential double sum that defines a bit is within 1.5e-14 of the
// same quantity (Higham, Accuracy and Stability of Numerical Algorithms,
// ch. 3-4).  A bit with |y'| > 2^-14 ||x|| ||W_:j|| + 2^-100 is therefore the
// sign of y'.  Every other bit is recomputed by the wave: a double-precision
// dot product over 64 lanes (two exact products per lane, then a lane sum
// with eight rounding levels, so within gamma_8 sum |p| of the exact sum)
// decides it when |s| > 2^-44 sum |p|; otherwise lane 0 runs the sequential
// double loop itself.
//
// Work split: grid.y = head; each workgroup keeps its head's W operands in
// registers (wave w: columns 32 w .. 32 w + 31, i.e. code word w) and W_H
// transposed in LDS for the recomputations, and walks 64-row tiles.  Lane
// (g, c) of a wave loads, for MFMA j, dims 32 j + 8 g .. + 8 of row c of each
// 16-row M tile (the A operand), so each load instruction reads whole
// 64-byte pieces of 16 rows; the B operand uses the same map of dims.
#include "device_util.h"
#include "hata_internal.h"
#include "../../include/hata.h"

namespace hata {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t uvec4 __attribute__((ext_vector_type(4)));

constexpr int kERows = 64;  // rows per tile
constexpr int kEThreads = 256;

struct EncArgs {
    int mode;  // 0: flat rows (hata_encode_keys), 1: cache append
    // mode 0
    const uint16_t *keys;
    int64_t row_stride, head_stride, n_rows;
    uint32_t *codes_out;
    // mode 1
    uint16_t *k_cache, *v_cache;
    uint32_t *codes;
    int32_t *seq_len, *ctrl;
    const int32_t *n_new;
    const uint16_t *k_new, *v_new;
    int B, Hkv, t_max;
    int64_t max_ctx;
    // both
    const float *w;
    int n_heads;
    int64_t tiles_per_seg;
    int n_seg;
};

struct ESmem {
    float wt[kBits][kHeadDim];     // W_H transposed: wt[j][t] = W[t][j]
    uint16_t xs[kERows][kHeadDim];  // the tile's rows (bf16)
};

__device__ __forceinline__ bool append_ok(int64_t len, int n, int t_max, int64_t max_ctx) {
    return n >= 0 && n <= t_max && len >= 0 && len + n <= max_ctx;
}

// Sum over the 64 lanes of a wave, in every lane: within each row of 16
// lanes by DPP (xor 1, xor 2, half-row mirror, row mirror: four additions),
// then the four row sums, read from lanes 0, 16, 32, 48, added in order
// (three more): eight rounding levels with the caller's pair sum.
__device__ __forceinline__ double dpp_f64(double v, int ctrl_id) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
    switch (ctrl_id) {
        case 0: lo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false); break;
        case 1: lo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false); break;
        case 2: lo = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xF, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xF, 0xF, false); break;
        default: lo = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xF, 0xF, false);
                 hi = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xF, 0xF, false); break;
    }
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double lane_f64(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double dsum64(double v) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v += dpp_f64(v, k);
    return ((lane_f64(v, 0) + lane_f64(v, 16)) + lane_f64(v, 32)) + lane_f64(v, 48);
}

// The exact bit (row R of the tile, column col): see the header comment.
__device__ __forceinline__ bool exact_bit(const ESmem &sm, int R, int col) {
    const int lane = threadIdx.x & 63;
    const double x0 = (double)bf16_to_f32(sm.xs[R][2 * lane]);
    const double x1 = (double)bf16_to_f32(sm.xs[R][2 * lane + 1]);
    const double p0 = x0 * (double)sm.wt[col][2 * lane], p1 = x1 * (double)sm.wt[col][2 * lane + 1];
    const double s = dsum64(p0 + p1);
    const double A = dsum64(fabs(p0) + fabs(p1));
    bool bit = s > 0.0;
    if (!(fabs(s) > 0x1p-44 * A)) {
        int b = 0;
        if (lane == 0) {
            double y = 0.0;  // the defining sequential sum
            for (int t = 0; t < kHeadDim; ++t)
                y = fma((double)bf16_to_f32(sm.xs[R][t]), (double)sm.wt[col][t], y);
            b = y > 0.0;
        }
        bit = __builtin_amdgcn_readfirstlane(b) != 0;
    }
    return bit;
}

// 2^-14 ||x|| ||W_:j|| + 2^-100: the band inside which y' does not decide.
__device__ __forceinline__ float band(float xnorm, float wnorm) {
    return 0x1p-14f * xnorm * wnorm + 0x1p-100f;
}

__global__ __launch_bounds__(kEThreads, 2) void k_encode_mfma(EncArgs a) {
    __shared__ ESmem sm;
    const int h = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, g = lane >> 4, c = lane & 15;
    const float *W = a.w + (int64_t)h * kHeadDim * kBits;

    // ---- W_H transposed into LDS, and this wave's B operands (columns
    // 32 wv + 16 nt + c, rows 32 j + 8 g + e) split into bf16 hi / lo terms
    for (int i = t; i < kHeadDim * kBits / 4; i += kEThreads) {
        // consecutive threads take consecutive rows: the LDS writes hit
        // consecutive banks
        const int row = i % kHeadDim, c4 = (i / kHeadDim) * 4;
        const float4 v = *reinterpret_cast<const float4 *>(W + row * kBits + c4);
        sm.wt[c4][row] = v.x;
        sm.wt[c4 + 1][row] = v.y;
        sm.wt[c4 + 2][row] = v.z;
        sm.wt[c4 + 3][row] = v.w;
    }
    bf16x8 bhi[2][4], blo[2][4];
    float wnorm[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int col = 32 * wv + 16 * nt + c;
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float wf = W[(32 * j + 8 * g + e) * kBits + col];
                const uint16_t hb = f32_to_bf16(wf);  // nearest even; NaN stays NaN
                const float hf = __uint_as_float((uint32_t)hb << 16);
                const uint16_t lb = f32_to_bf16(wf - hf);
                bhi[nt][j][e] = __builtin_bit_cast(__bf16, hb);
                blo[nt][j][e] = __builtin_bit_cast(__bf16, lb);
                ss = fmaf(wf, wf, ss);
            }
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        wnorm[nt] = sqrtf(ss) * (1.f + 0x1p-10f);
    }
    __syncthreads();

    const int64_t n_tiles = a.tiles_per_seg * a.n_seg;
    // the batch entry's length and row count, read again only when a tile
    // belongs to another entry (consecutive tiles mostly share one)
    int s_cur = -1;
    int64_t l0_cur = 0, rows_cur = 0;
    for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        const int s = (int)(tile / a.tiles_per_seg);
        const int64_t r0 = (tile % a.tiles_per_seg) * kERows;
        int64_t rows, l0 = 0;
        if (a.mode == 0) {
            rows = a.n_rows;
        } else {
            if (s != s_cur) {
                s_cur = s;
                l0_cur = a.seq_len[s];
                const int n = a.n_new[s];
                rows_cur = append_ok(l0_cur, n, a.t_max, a.max_ctx) ? n : 0;
            }
            l0 = l0_cur;
            rows = rows_cur;
        }
        if (r0 >= rows) continue;
        const int nr = rows - r0 < kERows ? (int)(rows - r0) : kERows;

        // ---- A operands (and the tile in LDS; the K/V rows to the cache)
        uvec4 xa[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int R = 16 * mt + c;
            const int64_t r = r0 + R;
            const uint16_t *src = nullptr;
            if (R < nr) {
                if (a.mode == 0) src = a.keys + r * a.row_stride + (int64_t)h * a.head_stride;
                else if (a.k_new) src = a.k_new + (((int64_t)s * a.t_max + r) * a.Hkv + h) * kHeadDim;
                else src = a.k_cache + (((int64_t)s * a.Hkv + h) * a.max_ctx + l0 + r) * kHeadDim;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xa[mt][j] = uvec4{0u, 0u, 0u, 0u};
                if (src) xa[mt][j] = *reinterpret_cast<const uvec4 *>(src + 32 * j + 8 * g);
            }
        }
        if (a.mode == 1 && a.k_new) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int R = 16 * mt + c;
                if (R < nr) {
                    const int64_t r = r0 + R;
                    const int64_t crow = (((int64_t)s * a.Hkv + h) * a.max_ctx + l0 + r) * kHeadDim;
                    const int64_t nrow = (((int64_t)s * a.t_max + r) * a.Hkv + h) * kHeadDim;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        *reinterpret_cast<uvec4 *>(a.k_cache + crow + 32 * j + 8 * g) = xa[mt][j];
                        *reinterpret_cast<uvec4 *>(a.v_cache + crow + 32 * j + 8 * g) =
                            *reinterpret_cast<const uvec4 *>(a.v_new + nrow + 32 * j + 8 * g);
                    }
                }
            }
        }
        __syncthreads();  // the previous tile's recomputations are done with xs
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uvec4 *>(&sm.xs[16 * mt + c][32 * j + 8 * g]) = xa[mt][j];

        // ---- row norms: row c of M tile mt, over the four lane groups
        float xnorm[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bf16x2 p = __builtin_bit_cast(bf16x2, xa[mt][j][q]);
                    ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
                }
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            xnorm[mt] = sqrtf(ss) * (1.f + 0x1p-10f);
        }

        // ---- y' on the matrix cores: acc[mt][nt] holds rows 16 mt + 4 g + i,
        // column 32 wv + 16 nt + c
        f32x4 acc[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 xb = __builtin_bit_cast(bf16x8, xa[mt][j]);
                    v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, bhi[nt][j], v, 0, 0, 0);
                    v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, blo[nt][j], v, 0, 0, 0);
                }
                acc[mt][nt] = v;
            }
        __syncthreads();  // xs complete for the recomputations

        // ---- bits: the decided ones by ballot in one straight pass (lane L
        // assembles the word of row L), then, only if some bit lies inside
        // the band, a second pass recomputes those exactly.
        float xnr[4][4];  // the norm of row 16 mt + 4 g + i
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) xnr[mt][i] = __shfl(xnorm[mt], 4 * g + i, 64);
        uint32_t wordv = 0;
        bool unsure = false;
        const int gg = (lane >> 2) & 3;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = 16 * mt + 4 * g + i < nr;
                uint64_t bits[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const float y = acc[mt][nt][i];
                    const bool sure = fabsf(y) > band(xnr[mt][i], wnorm[nt]);
                    unsure |= valid && !sure;
                    bits[nt] = __ballot(valid && sure && y > 0.f);
                }
                // lane L holds the word of row L: L = 16 mt + 4 gg + i
                const uint32_t wd = (uint32_t)((bits[0] >> (16 * gg)) & 0xFFFFu) |
                                    ((uint32_t)((bits[1] >> (16 * gg)) & 0xFFFFu) << 16);
                if ((lane >> 4) == mt && (lane & 3) == i) wordv = wd;
            }
        if (__ballot(unsure) != 0) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool valid = 16 * mt + 4 * g + i < nr;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const float y = acc[mt][nt][i];
                        uint64_t um = __ballot(valid && !(fabsf(y) > band(xnr[mt][i], wnorm[nt])));
                        while (um) {
                            const int lb = __builtin_ctzll(um);
                            um &= um - 1;
                            const int Rf = 16 * mt + 4 * (lb >> 4) + i;
                            const int cb = 16 * nt + (lb & 15);  // bit of the word
                            if (exact_bit(sm, Rf, 32 * wv + cb) && lane == Rf) wordv |= 1u << cb;
                        }
                    }
                }
        }
        if (lane < nr) {
            const int64_t r = r0 + lane;
            uint32_t *dst = a.mode == 0 ? a.codes_out + (r * a.n_heads + h) * kWords
                                        : a.codes + (((int64_t)s * a.Hkv + h) * a.max_ctx + l0 + r) * kWords;
            dst[wv] = wordv;
        }
    }

    if (a.mode == 1) {
        // The last workgroup to finish publishes the new lengths (every
        // workgroup has read seq_len[] by then).
        __syncthreads();
        int *last = reinterpret_cast<int *>(&sm.xs[0][0]);
        if (t == 0) {
            __threadfence();
            const unsigned total = gridDim.x * gridDim.y;
            const unsigned prev = atomicAdd((unsigned *)&a.ctrl[kCtrlAppendDone], 1u);
            *last = (prev == total - 1);
        }
        __syncthreads();
        if (*last) {
            __threadfence();
            for (int bb = t; bb < a.B; bb += kEThreads) {
                const int64_t l = a.seq_len[bb];
                const int nn = a.n_new[bb];
                if (append_ok(l, nn, a.t_max, a.max_ctx)) {
                    a.seq_len[bb] = (int32_t)(l + nn);
                } else {
                    const int flag = (nn < 0 || nn > a.t_max) ? HATA_DEV_BAD_NEW : HATA_DEV_APPEND_OVERFLOW;
                    atomicOr(&a.ctrl[kCtrlStatus], flag);
                }
            }
            if (t == 0) a.ctrl[kCtrlAppendDone] = 0;
        }
    }
}

static hipError_t launch_enc(EncArgs &a, int heads, int64_t tiles_per_head, hipStream_t s) {
    static_assert(sizeof(ESmem) <= 81920, "two workgroups per CU");  // of 160 KB
    // about two workgroups per CU in total, at most one per tile
    int64_t per_head = (512 + heads - 1) / heads;
    if (per_head > tiles_per_head) per_head = tiles_per_head;
    if (per_head < 1) per_head = 1;
    hipLaunchKernelGGL(k_encode_mfma, dim3((unsigned)per_head, (unsigned)heads), dim3(kEThreads), 0,
                       s, a);
    return hipGetLastError();
}

hipError_t launch_encode_mfma(const uint16_t *keys, int64_t n_rows, int n_heads, int64_t row_stride,
                              int64_t head_stride, const float *w, uint32_t *codes, hipStream_t s) {
    EncArgs a = {};
    a.mode = 0;
    a.keys = keys;
    a.row_stride = row_stride;
    a.head_stride = head_stride;
    a.n_rows = n_rows;
    a.codes_out = codes;
    a.w = w;
    a.n_heads = n_heads;
    a.n_seg = 1;
    a.tiles_per_seg = (n_rows + kERows - 1) / kERows;
    return launch_enc(a, n_heads, a.tiles_per_seg, s);
}

hipError_t launch_append_mfma(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                              int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                              const uint16_t *k_new, const uint16_t *v_new,
                              const int32_t *n_new, int t_max, const float *w, hipStream_t s) {
    EncArgs a = {};
    a.mode = 1;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.codes = codes;
    a.seq_len = seq_len;
    a.ctrl = ctrl;
    a.n_new = n_new;
    a.k_new = k_new;
    a.v_new = v_new;
    a.B = B;
    a.Hkv = Hkv;
    a.t_max = t_max;
    a.max_ctx = max_ctx;
    a.w = w;
    a.n_heads = Hkv;
    a.n_seg = B;
    a.tiles_per_seg = ((int64_t)t_max + kERows - 1) / kERows;
    return launch_enc(a, Hkv, a.tiles_per_seg * B, s);
}

}  // namespace hata
