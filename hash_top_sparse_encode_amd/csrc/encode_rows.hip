// Bulk sign-code encoder on the matrix cores for every code length
// r in {32, 64, 128, 256} (HATA review: h(x) = sign(x W_H), "Free
// parameters" and its hash-length ablation; the key-code cache of
// Algorithm 1 in the Figure 2 caption).  Used for hata_encode_keys,
// hata_encode_keys_nbits and prefill appends from 64 rows on.
//
// Exactness.  W_H is split into two bf16 terms, W = W_hi + W_lo + res with
// |res| <= 2^-16 |W|, and y' = x W_hi + x W_lo is accumulated in fp32 by
// v_mfma_f32_16x16x32_bf16 (bf16 x bf16 products are exact in fp32), so
// |y' - x W| <= (2^-16 + gamma_256 (1 + 2^-7)) sum_t |x_t||W_tj|
//            <= 3.1e-5 ||x||_2 ||W_:j||_2,
// and the sequential double sum that defines a bit is within 1.5e-14 of the
// same quantity (Higham, Accuracy and Stability of Numerical Algorithms,
// ch. 3-4).  A bit with |y'| > 2^-14 ||x|| ||W_:j|| + 2^-100 has the sign of
// y'.  Every other bit is recomputed: the defining sequential double sum
// itself, one lane per bit.  Rows or columns of zeros give exactly 0 (bit 0)
// and skip the band test.
//
// Work split.  One 768-thread workgroup per CU for one head (grid.y); its
// twelve waves work independently, with no barrier after the set-up: wave w
// takes 32-row groups w, w + 12 P, ... of the head (P workgroups per head),
// and while it computes one group the next group's rows are already loading
// into a second set of registers.  For a group, lane (g, c) of M tile m holds
// row 16 m + c, dims 32 j + 8 g .. + 8 for k step j (eight 16-byte loads,
// each instruction reading 64 contiguous bytes of 16 rows); the row norms
// follow, then r / 16 column tiles: the B operands of a tile (bf16 high and
// low parts of W_H, laid out per lane in LDS at the set-up) are read from
// LDS, 2 M tiles x 4 k steps x 2 parts of MFMA give y' for 32 rows x 16
// bits, the band test decides the bits by ballot, and lane L collects the
// bits of row L, then stores row L's r / 32 code words.  In-band bits are
// stored as 0 and listed in LDS (group, row, column); between groups, once
// the list is half full, and at the end, the wave resolves them (one lane per
// bit runs the defining sequential double sum, with W_H's column from LDS
// for r <= 128 or from memory for r = 256) and sets the bits that are 1.
#include "device_util.h"
#include "hata_internal.h"
#include "../../include/hata.h"

namespace hata {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t uvec4 __attribute__((ext_vector_type(4)));

constexpr int kRThreads = 768;
constexpr int kRWaves = kRThreads / 64;
constexpr int kRGroup = 32;      // rows per wave group (two M tiles)
constexpr int kRSegLds = 1024;   // batch entries whose lengths are kept in LDS
constexpr int kRList = 128;      // in-band bits a wave lists before resolving them

struct RowsArgs {
    int mode;  // 0: flat rows, 1: cache append
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
    const float *w;  // [heads][128][R]
    int n_heads;
    int64_t groups_per_seg;
    int n_seg;
};

template <int R>
struct RowsSmem {
    uvec4 bop[R / 16][4][2][64];   // B operands: column tile, k step, high / low part, lane
    float wt[R <= 128 ? R : 1][kHeadDim];  // W_H transposed (exact path, r <= 128)
    float wnorm[R];                // column norms ||W_:j|| (1 + 2^-10); -inf: a zero column
    uint32_t lgrp[kRWaves][kRList];  // listed in-band bits: the group ...
    uint16_t lrc[kRWaves][kRList];   // ... and row << 8 | column
    uint32_t xrow[kRWaves][64];    // a row staged for the exact path (bf16 pairs)
    int64_t seg_l0[kRSegLds];      // mode 1: each entry's length ...
    int32_t seg_rows[kRSegLds];    // ... and the rows it appends
    int last;
};

__device__ __forceinline__ bool rows_append_ok(int64_t len, int n, int t_max, int64_t max_ctx) {
    return n >= 0 && n <= t_max && len >= 0 && len + n <= max_ctx;
}

// A group: its batch entry s, first row r0, the entry's length l0 and the rows
// nr of the group (0 when past the work or the entry is skipped).
struct RGroup {
    int s;
    int64_t r0, l0;
    int nr;
};

template <int R>
__device__ __forceinline__ RGroup group_of(const RowsArgs &a, const RowsSmem<R> &sm, int64_t gi) {
    RGroup e{0, 0, 0, 0};
    e.s = (int)(gi / a.groups_per_seg);
    e.r0 = (gi - (int64_t)e.s * a.groups_per_seg) * kRGroup;
    int64_t rows;
    if (a.mode == 0) {
        rows = a.n_rows;
    } else if (e.s < kRSegLds) {
        e.l0 = sm.seg_l0[e.s];
        rows = sm.seg_rows[e.s];
    } else {
        e.l0 = a.seq_len[e.s];
        const int n = a.n_new[e.s];
        rows = rows_append_ok(e.l0, n, a.t_max, a.max_ctx) ? n : 0;
    }
    e.nr = e.r0 < rows ? (int)(rows - e.r0 < kRGroup ? rows - e.r0 : kRGroup) : 0;
    return e;
}

// Source of row r (0 .. 63) of a group of head h; rows past the group's
// count read its first row.
__device__ __forceinline__ const uint16_t *src_row(const RowsArgs &a, int h, const RGroup &e, int r) {
    const int64_t rr = e.r0 + (r < e.nr ? r : 0);
    if (a.mode == 0) return a.keys + rr * a.row_stride + (int64_t)h * a.head_stride;
    if (a.k_new) return a.k_new + (((int64_t)e.s * a.t_max + rr) * a.Hkv + h) * kHeadDim;
    return a.k_cache + (((int64_t)e.s * a.Hkv + h) * a.max_ctx + e.l0 + rr) * kHeadDim;
}

// Cache row (mode 1) of row r of a group.
__device__ __forceinline__ int64_t cache_row(const RowsArgs &a, int h, const RGroup &e, int r) {
    return ((int64_t)e.s * a.Hkv + h) * a.max_ctx + e.l0 + e.r0 + r;
}

// Sum over the 64 lanes, in every lane: DPP within rows of 16 (xor 1, xor 2,
// half-row and row mirrors), then the four row sums in order.
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

// Lane L keeps the code words of row L; set bit `col` of them to `bit` (col
// and bit uniform).
template <int R>
__device__ __forceinline__ void put_bit(uint32_t (&wd)[R / 32], int col, bool bit, bool mine) {
#pragma unroll
    for (int k = 0; k < R / 32; ++k)
        if (mine && k == (col >> 5)) wd[k] = bit ? (wd[k] | (1u << (col & 31))) : (wd[k] & ~(1u << (col & 31)));
}

// The eight 16-byte A-operand loads of a group (lane (g, c): rows c and
// 16 + c, dims 32 j + 8 g .. + 8).
__device__ __forceinline__ void load_group(const RowsArgs &a, int h, const RGroup &e, int g, int c,
                                           uvec4 (&xa)[2][4]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const uint16_t *src = src_row(a, h, e, 16 * m + c) + 8 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[m][j] = *reinterpret_cast<const uvec4 *>(src + 32 * j);
    }
}

// Codes of one group whose rows are in xa (see the header comment).
template <int R>
__device__ __forceinline__ void encode_group(const RowsArgs &a, RowsSmem<R> &sm, const float *W, int h,
                                             int64_t gi, const RGroup &e, const uvec4 (&xa)[2][4],
                                             int &n_list) {
    constexpr int NT = R / 16;   // column tiles
    constexpr int NW = R / 32;   // code words per row
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    // ---- row norms: lane (g, c) sums its 32 dims of row 16 m + c, the four
    // lanes of a row add theirs; lane L then takes 2^-14 ||x|| of rows
    // 16 m + 4 g + i (negative for a row of zeros, whose sums are exactly 0)
    float tx[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        float ss = 0.f;
        uint32_t nz = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bf16x2 p = __builtin_bit_cast(bf16x2, xa[m][j][q]);
                ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
                nz |= xa[m][j][q] & 0x7FFF7FFFu;
            }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        nz |= (uint32_t)__shfl_xor((int)nz, 16, 64);
        nz |= (uint32_t)__shfl_xor((int)nz, 32, 64);
        const float xn = nz ? sqrtf(ss) * (1.f + 0x1p-10f) * 0x1p-14f : -1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) tx[m][i] = __shfl(xn, 4 * g + i, 64);
    }
    // lane L (< 32) keeps row L = 16 mL + 4 gL + iL
    const int mL = (lane >> 4) & 1, gL = (lane >> 2) & 3, iL = lane & 3;
    uint32_t wd[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) wd[k] = 0u;
    const int list0 = n_list;  // this group's entries start here (uniform)
    bool overflow = false;
#pragma unroll 1
    for (int n = 0; n < NT; ++n) {
        bf16x8 bh[4], bl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bh[j] = __builtin_bit_cast(bf16x8, sm.bop[n][j][0][lane]);
            bl[j] = __builtin_bit_cast(bf16x8, sm.bop[n][j][1][lane]);
        }
        const float wn = sm.wnorm[16 * n + c];
        // four independent accumulator chains: the high and the low parts of
        // each M tile (their sum is one more rounding within the same bound)
        f32x4 ah[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        f32x4 al[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                ah[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[m][j]), bh[j],
                                                                ah[m], 0, 0, 0);
                al[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[m][j]), bl[j],
                                                                al[m], 0, 0, 0);
            }
        }
        // y' = ah + al: row 16 m + 4 g + i, column 16 n + c.  The band: a
        // zero row (tx < 0) or column (wn = -inf) gives a negative threshold,
        // so its exact 0 counts as decided; both zero gives +inf and the exact
        // path (which finds 0).  A bit is 1 where y' > max(threshold, 0), and
        // unsure where |y'| does not exceed the threshold.  Rows past the
        // group's count repeat row 0.
        uint32_t piece = 0u;
        bool unsure = false;
        float yv[2][4], th[2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                yv[m][i] = ah[m][i] + al[m][i];
                th[m][i] = fmaf(tx[m][i], wn, 0x1p-100f);
            }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint64_t pos = __builtin_amdgcn_ballot_w64(yv[m][i] > fmaxf(th[m][i], 0.f));
                unsure |= !(fabsf(yv[m][i]) > th[m][i]);
                if (mL == m && iL == i) piece = (uint32_t)(pos >> (16 * gL)) & 0xFFFFu;
            }
#pragma unroll
        for (int k = 0; k < NW; ++k)
            if (k == (n >> 1)) wd[k] |= piece << (16 * (n & 1));
        if (__builtin_amdgcn_ballot_w64(unsure) != 0) {
            // list the in-band bits (about 0.05 % of bits; their provisional
            // bit is 0), to be resolved later by flush_list
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint64_t uns = __builtin_amdgcn_ballot_w64(!(fabsf(yv[m][i]) > th[m][i]));
                    while (uns) {
                        const int lb = __builtin_ctzll(uns);
                        uns &= uns - 1;
                        const int row = 16 * m + 4 * (lb >> 4) + i;
                        if (row >= e.nr) continue;  // a repeat of row 0 past the group's count
                        if (n_list < kRList) {
                            if (lane == 0) {
                                sm.lgrp[wv][n_list] = (uint32_t)gi;
                                sm.lrc[wv][n_list] = (uint16_t)((row << 8) | (16 * n + (lb & 15)));
                            }
                            ++n_list;
                        } else {
                            overflow = true;
                        }
                    }
                }
        }
    }
    // ---- a group with more in-band bits than the list holds (degenerate
    // rows): its listed entries are dropped and every bit of it is decided
    // here, exactly, by the wave (the row through the wave's LDS row buffer,
    // lane l holding dims 2 l and 2 l + 1; W_H's column from LDS for
    // r <= 128, else from memory)
    if (overflow) {
        n_list = list0;
        const int total = e.nr * R;
        for (int b = 0; b < total; ++b) {
            const int row = b / R, col = b % R;
            if (c == (row & 15)) {
                const int m = row >> 4;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<uvec4 *>(&sm.xrow[wv][16 * j + 4 * g]) = m ? xa[1][j] : xa[0][j];
            }
            __builtin_amdgcn_wave_barrier();
            const uint32_t xp = sm.xrow[wv][lane];
            float w0, w1;
            if constexpr (R <= 128) {
                const float2 wp = *reinterpret_cast<const float2 *>(&sm.wt[col][2 * lane]);
                w0 = wp.x;
                w1 = wp.y;
            } else {
                w0 = W[(int64_t)(2 * lane) * R + col];
                w1 = W[(int64_t)(2 * lane + 1) * R + col];
            }
            __builtin_amdgcn_wave_barrier();
            const double p0 = (double)__uint_as_float(xp << 16) * (double)w0;
            const double p1 = (double)__uint_as_float(xp & 0xFFFF0000u) * (double)w1;
            const double sum = dsum64(p0 + p1);
            const double A = dsum64(fabs(p0) + fabs(p1));
            bool bit = sum > 0.0;
            if (!(fabs(sum) > 0x1p-44 * A)) {
                // the defining sequential sum, d = 0 .. 127 in order
                double ysq = 0.0;
                for (int l = 0; l < 64; ++l) {
                    const uint32_t xl = (uint32_t)__builtin_amdgcn_readlane((int)xp, l);
                    const float wa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w0), l));
                    const float wb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w1), l));
                    ysq = fma((double)__uint_as_float(xl << 16), (double)wa, ysq);
                    ysq = fma((double)__uint_as_float(xl & 0xFFFF0000u), (double)wb, ysq);
                }
                bit = ysq > 0.0;
            }
            put_bit<R>(wd, col, bit, lane == row);
        }
    }
    // ---- row L's code words
    if (lane < e.nr) {
        uint32_t *dst = a.mode == 0 ? a.codes_out + ((e.r0 + lane) * a.n_heads + h) * NW
                                    : a.codes + cache_row(a, h, e, lane) * NW;
        if constexpr (NW == 1) {
            dst[0] = wd[0];
        } else if constexpr (NW == 2) {
            *reinterpret_cast<uint2 *>(dst) = make_uint2(wd[0], wd[1]);
        } else {
#pragma unroll
            for (int k = 0; k < NW; k += 4)
                *reinterpret_cast<uvec4 *>(dst + k) = uvec4{wd[k], wd[k + 1], wd[k + 2], wd[k + 3]};
        }
    }
    // ---- appended rows into the cache: K from the registers, V copied
    if (a.mode == 1 && a.k_new) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int r = 16 * m + c;
            if (r < e.nr) {
                uint16_t *kd = a.k_cache + cache_row(a, h, e, r) * kHeadDim + 8 * g;
                uint16_t *vd = a.v_cache + cache_row(a, h, e, r) * kHeadDim + 8 * g;
                const uint16_t *vs = a.v_new + (((int64_t)e.s * a.t_max + e.r0 + r) * a.Hkv + h) * kHeadDim + 8 * g;
                uvec4 vv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) vv[j] = *reinterpret_cast<const uvec4 *>(vs + 32 * j);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    *reinterpret_cast<uvec4 *>(kd + 32 * j) = xa[m][j];
                    *reinterpret_cast<uvec4 *>(vd + 32 * j) = vv[j];
                }
            }
        }
    }
}

// Resolve a wave's listed in-band bits: one lane per bit runs the defining
// sequential double sum (d = 0 .. 127 in order; every product of a bf16 and
// an fp32 value is exact in double) and, where it is positive, sets the bit
// in the code word the wave has already stored (provisional bit 0).  The
// wave first waits for its own stores, so the word is in memory.
template <int R>
__device__ __forceinline__ void flush_list(const RowsArgs &a, RowsSmem<R> &sm, const float *W, int h, int count) {
    constexpr int NW = R / 32;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __builtin_amdgcn_s_waitcnt(0);
    for (int b = lane; b < count; b += 64) {
        const int64_t gi = sm.lgrp[wv][b];
        const int rc = sm.lrc[wv][b], row = rc >> 8, col = rc & 255;
        const RGroup e = group_of<R>(a, sm, gi);
        const uint16_t *xr = src_row(a, h, e, row);
        double y = 0.0;
        for (int d0 = 0; d0 < kHeadDim; d0 += 8) {
            const uvec4 xv = *reinterpret_cast<const uvec4 *>(xr + d0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = d0 + 2 * q;
                float w0, w1;
                if constexpr (R <= 128) {
                    w0 = sm.wt[col][d];
                    w1 = sm.wt[col][d + 1];
                } else {
                    w0 = W[(int64_t)d * R + col];
                    w1 = W[(int64_t)(d + 1) * R + col];
                }
                y = fma((double)__uint_as_float(xv[q] << 16), (double)w0, y);
                y = fma((double)__uint_as_float(xv[q] & 0xFFFF0000u), (double)w1, y);
            }
        }
        if (row < e.nr && y > 0.0) {
            uint32_t *word = (a.mode == 0 ? a.codes_out + ((e.r0 + row) * a.n_heads + h) * NW
                                          : a.codes + cache_row(a, h, e, row) * NW) + (col >> 5);
            atomicOr(word, 1u << (col & 31));
        }
    }
}

template <int R>
__global__ __launch_bounds__(kRThreads, 1) void k_encode_rows(RowsArgs a) {
    constexpr int NT = R / 16;   // column tiles
    __shared__ RowsSmem<R> sm;
    const int h = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, g = lane >> 4, c = lane & 15;
    const float *W = a.w + (int64_t)h * kHeadDim * R;

    // ---- set-up: B operands (lane (g, c) of column tile n, k step j holds
    // W[32 j + 8 g + e][16 n + c], e < 8, as bf16 high and low parts), W_H
    // transposed, the column norms, the entries' lengths
    for (int i = t; i < NT * 4 * 64; i += kRThreads) {
        const int l = i & 63, j = (i >> 6) & 3, n = i >> 8;
        const int col = 16 * n + (l & 15), d0 = 32 * j + 8 * (l >> 4);
        float wf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) wf[e] = W[(int64_t)(d0 + e) * R + col];
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const uint16_t h0 = f32_to_bf16(wf[e]), h1 = f32_to_bf16(wf[e + 1]);
            const uint16_t l0 = f32_to_bf16(wf[e] - __uint_as_float((uint32_t)h0 << 16));
            const uint16_t l1 = f32_to_bf16(wf[e + 1] - __uint_as_float((uint32_t)h1 << 16));
            hw[e / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lw[e / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        sm.bop[n][j][0][l] = uvec4{hw[0], hw[1], hw[2], hw[3]};
        sm.bop[n][j][1][l] = uvec4{lw[0], lw[1], lw[2], lw[3]};
        if constexpr (R <= 128) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.wt[col][d0 + e] = wf[e];
        }
    }
    for (int col = t; col < R; col += kRThreads) {
        float ss = 0.f;
        uint32_t nz = 0u;
        for (int d = 0; d < kHeadDim; ++d) {
            const float wf = W[(int64_t)d * R + col];
            ss = fmaf(wf, wf, ss);
            nz |= __float_as_uint(wf) & 0x7FFFFFFFu;
        }
        sm.wnorm[col] = nz ? sqrtf(ss) * (1.f + 0x1p-10f) : -INFINITY;
    }
    if (a.mode == 1) {
        for (int s = t; s < a.n_seg && s < kRSegLds; s += kRThreads) {
            const int64_t l0 = a.seq_len[s];
            const int n = a.n_new[s];
            sm.seg_l0[s] = l0;
            sm.seg_rows[s] = rows_append_ok(l0, n, a.t_max, a.max_ctx) ? n : 0;
        }
    }
    __syncthreads();

    // ---- the wave's groups, two register buffers: the next group loads
    // while this one is computed
    const int64_t n_groups = a.groups_per_seg * a.n_seg;
    const int64_t stride = (int64_t)gridDim.x * kRWaves;
    const RGroup none{0, 0, 0, 0};
    int64_t gi = (int64_t)blockIdx.x * kRWaves + wv;
    uvec4 xa0[2][4], xa1[2][4];
    int n_list = 0;  // in-band bits listed by this wave, not yet resolved (uniform)
    RGroup e0 = gi < n_groups ? group_of<R>(a, sm, gi) : none;
    if (e0.nr > 0) load_group(a, h, e0, g, c, xa0);
    while (gi < n_groups) {
        const int64_t gi1 = gi + stride;
        const RGroup e1 = gi1 < n_groups ? group_of<R>(a, sm, gi1) : none;
        if (e1.nr > 0) load_group(a, h, e1, g, c, xa1);
        if (e0.nr > 0) encode_group<R>(a, sm, W, h, gi, e0, xa0, n_list);
        if (n_list > kRList / 2) {
            flush_list<R>(a, sm, W, h, n_list);
            n_list = 0;
        }
        const int64_t gi2 = gi1 + stride;
        e0 = gi2 < n_groups ? group_of<R>(a, sm, gi2) : none;
        if (e0.nr > 0) load_group(a, h, e0, g, c, xa0);
        if (e1.nr > 0) encode_group<R>(a, sm, W, h, gi1, e1, xa1, n_list);
        if (n_list > kRList / 2) {
            flush_list<R>(a, sm, W, h, n_list);
            n_list = 0;
        }
        gi = gi2;
    }
    if (n_list > 0) flush_list<R>(a, sm, W, h, n_list);

    if (a.mode == 1) {
        // The last workgroup to finish publishes the new lengths (every
        // workgroup has read seq_len[] by then).
        __syncthreads();
        if (t == 0) {
            __threadfence();
            const unsigned total = gridDim.x * gridDim.y;
            const unsigned prev = atomicAdd((unsigned *)&a.ctrl[kCtrlAppendDone], 1u);
            sm.last = (prev == total - 1);
        }
        __syncthreads();
        if (sm.last) {
            __threadfence();
            for (int bb = t; bb < a.B; bb += kRThreads) {
                const int64_t l = a.seq_len[bb];
                const int nn = a.n_new[bb];
                if (rows_append_ok(l, nn, a.t_max, a.max_ctx)) {
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

template <int R>
hipError_t launch_rows(RowsArgs &a, int heads, int64_t groups_per_head, hipStream_t s) {
    static_assert(sizeof(RowsSmem<R>) <= 160 * 1024, "one workgroup per CU");
    // one workgroup per CU in total, at most one per eight groups
    int dev = 0, n_cu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
        n_cu = 256;
    int64_t per_head = (n_cu + heads - 1) / heads;
    const int64_t need = (groups_per_head + kRWaves - 1) / kRWaves;
    if (per_head > need) per_head = need;
    if (per_head < 1) per_head = 1;
    hipLaunchKernelGGL(k_encode_rows<R>, dim3((unsigned)per_head, (unsigned)heads), dim3(kRThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t dispatch_rows(RowsArgs &a, int n_bits, int heads, int64_t groups_per_head, hipStream_t s) {
    switch (n_bits) {
        case 32: return launch_rows<32>(a, heads, groups_per_head, s);
        case 64: return launch_rows<64>(a, heads, groups_per_head, s);
        case 128: return launch_rows<128>(a, heads, groups_per_head, s);
        case 256: return launch_rows<256>(a, heads, groups_per_head, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode_rows(const uint16_t *keys, int64_t n_rows, int n_heads, int64_t row_stride,
                              int64_t head_stride, const float *w, int n_bits, uint32_t *codes,
                              hipStream_t s) {
    RowsArgs a = {};
    a.mode = 0;
    a.keys = keys;
    a.row_stride = row_stride;
    a.head_stride = head_stride;
    a.n_rows = n_rows;
    a.codes_out = codes;
    a.w = w;
    a.n_heads = n_heads;
    a.n_seg = 1;
    a.groups_per_seg = (n_rows + kRGroup - 1) / kRGroup;
    return dispatch_rows(a, n_bits, n_heads, a.groups_per_seg, s);
}

hipError_t launch_append_rows(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                              int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                              const uint16_t *k_new, const uint16_t *v_new, const int32_t *n_new,
                              int t_max, const float *w, int n_bits, hipStream_t s) {
    RowsArgs a = {};
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
    a.groups_per_seg = ((int64_t)t_max + kRGroup - 1) / kRGroup;
    return dispatch_rows(a, n_bits, Hkv, a.groups_per_seg * B, s);
}

}  // namespace hata
