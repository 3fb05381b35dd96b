// Bulk sign-code encoder on the matrix cores for every code length
// r in {32, 64, 128, 256} (HATA review: h(x) = sign(x W_H), "Free
// parameters" and its hash-length ablation; the key-code cache of
// Algorithm 1 in the Figure 2 caption).  Used for hata_encode_keys,
// hata_encode_keys_nbits and prefill appends from 64 rows on.
//
// Exactness.  Column j of W_H is scaled to unit norm, W'_j = fl(W_j 2^e_j m_j)
// (a power of two, exact unless an element drops below the normal range, then
// a factor m_j in [1, 2), one rounding of 2^-24 per element), so that
// ||W'_j||_2 <= 1 + 2^-16; a sign is unchanged by a positive scale.  W' is
// split into two bf16 terms, W' = W'_hi + W'_lo + res with
// |res| <= 2^-16 |W'|, and y' = x W'_hi + x W'_lo is accumulated in fp32 by
// v_mfma_f32_16x16x32_bf16 (bf16 x bf16 products are exact in fp32), so
//   |y' - 2^e_j m_j x W_j| <= (2^-16 + 2^-24 + gamma_256 (1 + 2^-7))
//                             sum_t |x_t||W'_tj| <= 3.2e-5 ||x||_2
// (Cauchy-Schwarz; Higham, Accuracy and Stability of Numerical Algorithms,
// ch. 3-4), and the sequential double sum that defines a bit is within
// 1.5e-14 of x W.  So a
// bit with |y'| > th(x) = 2^-14 (1 + 2^-10) sqrt(ss) + 2^-72, ss the fp32 sum
// of squares of the row, has the sign of y'.  (The 2^-72 covers squares and
// products below the normal range, flushed or not.)  Every other bit is
// recomputed: the defining sequential double sum itself, one lane per bit.
// Rows of zeros give 0 (every bit 0), columns of zeros give 0, and a row with
// a non-finite value (threshold +inf) or a column with one (its W' taken as
// 0) sends its bits to the exact sum.
//
// Work split.  One 512-thread workgroup per CU for one head (grid.y); its
// eight waves work independently, with no barrier after the set-up: wave w
// takes 64-row groups w, w + 8 P, ... of the head (P workgroups per head),
// and while it computes one group the next group's rows are already loading
// into a second set of registers.  A group's offsets are scalar, its loads
// and stores a scalar base and a 32-bit lane offset.  The product is taken
// transposed, y'^T = W'^T x^T: the A operand is a 16-column tile of W'^T
// (its bf16 high and low parts, laid out per lane in LDS at the set-up and
// read once per tile for all 64 rows), the B operand the rows: lane (g, c)
// of row tile t holds row 16 t + c, dims 32 j + 8 g .. + 8 for k step j.
// The result then gives lane (g, c) the values of row 16 t + c at columns
// 16 n + 4 g + i, i < 4, so the threshold is one per lane and row tile.  Per
// column tile and element, the sign bit and the band flag (the sign of
// th - |y'|) are shifted into per-lane words (v_alignbit), while the next
// tile's products issue; after the tiles of a pass (128 columns, or r),
// lane swaps across the four lanes of a row (v_permlane32_swap,
// v_permlane16_swap) OR the sign pieces so that lane (g, c) holds code word
// 4 p + q(g) of its row, q(g) = {0, 2, 1, 3}[g], which it stores.  In-band
// bits get the provisional sign of y' and are listed in LDS (group, row,
// column) at each lane's place in one prefix sum over the wave; once the
// list holds 64, and at the end, the wave resolves them in whole rounds of
// 64 (one lane per bit runs the defining sequential double sum, with W_H's
// column from LDS for r <= 128 or from memory for r = 256) and sets or
// clears the bit.  A group with more in-band bits than the list holds is
// computed entirely by the exact sums.
#include "device_util.h"
#include "hata_internal.h"
#include "../../include/hata.h"

#include <climits>

namespace hata {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t uvec4 __attribute__((ext_vector_type(4)));

constexpr int kRThreads = 512;
constexpr int kRWaves = kRThreads / 64;
constexpr int kRTiles = 4;                 // row tiles of 16 per group
constexpr int kRGroup = 16 * kRTiles;      // rows per wave group
constexpr int kRSegLds = 1024;   // batch entries whose lengths are kept in LDS
constexpr int kRList = 128;      // in-band bits a wave lists before resolving them
// s_waitcnt vmcnt(16) (vmcnt low bits 3:0, high bits 15:14), expcnt and
// lgkmcnt left at their maxima
constexpr int kWaitAllButPrefetch = (1 << 14) | (0x7 << 4) | (0xF << 8);

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
    // both, chosen on the host (a choice between two pointer fields of the
    // argument block would be made through a private copy of it: a scratch
    // load before each use)
    const uint16_t *src_base;  // keys (mode 0), k_new or k_cache (mode 1)
    uint32_t *codes_base;      // codes_out (mode 0) or codes (mode 1)
    int src_step;              // elements from one row of a group to the next
    int code_step;             // code words from one row of a group to the next
    const float *w;  // [heads][128][R]
    int n_heads;
    int64_t groups_per_seg;
    int n_seg;
};

// Columns of W_H that are all zero, as the lanes of group g = lane / 16 need
// them: the bits of the code word(s) such a lane stores (word 4 p + q(g) of
// pass p), and its columns 16 (p PT + k) + 4 g + i of pass p at bit
// 4 (PT - 1 - k) + i (the layout of the band flags).
template <int R>
struct ZeroCols {
    uint32_t word[R == 256 ? 2 : 1];
    uint32_t flags[R == 256 ? 2 : 1];
};

template <int R>
struct RowsSmem {
    uvec4 aop[R / 16][4][2][64];   // A operands: column tile, k step, high / low part, lane
    // W_H transposed (exact path, r <= 128); rows padded so that lanes on
    // different columns read different banks
    float wt[R <= 128 ? R : 1][kHeadDim + 1];
    int col_exp[R];                // column scale: a power of two 2^e_j (INT_MIN: W' taken as 0) ...
    float col_mul[R];              // ... then a factor m_j in [1, 2)
    uint32_t zcol[R / 32];         // columns of W_H that are all zero, a bit per column
    ZeroCols<R> zlane[4];          // ... and as lane group g needs them
    uint32_t lgrp[kRWaves][kRList];  // listed in-band bits: the group ...
    uint16_t lrc[kRWaves][kRList];   // ... and row << 8 | column
    int64_t seg_l0[kRSegLds];      // mode 1: each entry's length ...
    int32_t seg_rows[kRSegLds];    // ... and the rows it appends
    int32_t seg_pre[kRSegLds + 1]; // ... and its first group among the head's non-empty ones
    int32_t wsum[kRWaves];
    int last;
};

__device__ __forceinline__ bool rows_append_ok(int64_t len, int n, int t_max, int64_t max_ctx) {
    return n >= 0 && n <= t_max && len >= 0 && len + n <= max_ctx;
}

// A group: its rows nr (0 when past the work or the entry is skipped) and
// where its first row is: src elements from src_base, code words from
// codes_base (row r of the group is r src_step and r code_step further; in
// mode 1 the first row's cache row is code / (R / 32)).
struct RGroup {
    int nr;
    int64_t src, code;
};

// A value the whole wave reads at one address, through the scalar cache (a
// vector load here would put an unknown number of loads in flight on some
// paths, and the compiler would then wait for every load before the next use
// of a prefetched group).  The lengths are not written while they are read.
__device__ __forceinline__ int32_t uniform_load(const int32_t *p) {
    return *(const __attribute__((address_space(4))) int32_t *)p;
}

// Group gs (rows 64 gs ..) of batch entry s (mode 0: s = 0), head h.  With
// Uniform (the same group in every lane), the lengths read from LDS are
// moved to scalar registers, so that the offsets are scalar arithmetic and
// the loads take a scalar base.
template <int R, bool Uniform>
__device__ __forceinline__ RGroup group_at(const RowsArgs &a, const RowsSmem<R> &sm, int h, int s,
                                           int64_t gs) {
    RGroup e{0, 0, 0};
    const int64_t r0 = gs * kRGroup;
    int64_t rows;
    if (a.mode == 0) {
        rows = a.n_rows;
        e.src = r0 * a.row_stride + (int64_t)h * a.head_stride;
        e.code = r0 * a.code_step + (int64_t)h * (R / 32);
    } else {
        int64_t l0;
        if (s < kRSegLds) {
            l0 = sm.seg_l0[s];
            rows = sm.seg_rows[s];
            if (Uniform) {
                const uint64_t l = (uint64_t)l0;
                l0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(l >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)l));
                rows = __builtin_amdgcn_readfirstlane((int)rows);
            }
        } else {
            l0 = uniform_load(a.seq_len + s);
            const int n = uniform_load(a.n_new + s);
            rows = rows_append_ok(l0, n, a.t_max, a.max_ctx) ? n : 0;
        }
        const int64_t row0 = ((int64_t)s * a.Hkv + h) * a.max_ctx + l0 + r0;  // cache row
        e.src = a.k_new ? (((int64_t)s * a.t_max + r0) * a.Hkv + h) * kHeadDim : row0 * kHeadDim;
        e.code = row0 * (R / 32);
    }
    e.nr = r0 < rows ? (int)(rows - r0 < kRGroup ? rows - r0 : kRGroup) : 0;
    return e;
}

// A group without rows, whose loads read row 0 of the head (entry 0's row 0
// in mode 1: a valid address whatever the entry's length).
__device__ __forceinline__ RGroup no_group(const RowsArgs &a, int h) {
    RGroup e{0, 0, 0};
    e.src = a.mode == 0 ? (int64_t)h * a.head_stride
                        : (a.k_new ? (int64_t)h * kHeadDim : (int64_t)h * a.max_ctx * kHeadDim);
    return e;
}

// Source of row r (0 .. 63) of a group; rows past the group's count read its
// first row.  The per-row part is 32-bit (the host keeps 63 src_step below
// 2^31), so the loads take a uniform base and a 32-bit lane offset.
__device__ __forceinline__ const uint16_t *src_row(const RowsArgs &a, const RGroup &e, int r) {
    const uint32_t rr = (uint32_t)(r < e.nr ? r : 0);
    return a.src_base + e.src + rr * (uint32_t)a.src_step;
}

// Code word k of row r of a group (a uniform base and a 32-bit byte
// offset: the store address form with the base in scalar registers).
template <int R>
__device__ __forceinline__ uint32_t *code_word(const RowsArgs &a, const RGroup &e, int r, int k) {
    char *base = reinterpret_cast<char *>(a.codes_base + e.code);
    return reinterpret_cast<uint32_t *>(
        base + (uint64_t)((uint32_t)r * (uint32_t)(4 * a.code_step) + 4u * (uint32_t)k));
}

// The lane number, as a value the compiler cannot move: what is formed from
// it stays where it is used instead of being hoisted out of the group loop
// and held in registers throughout.
__device__ __forceinline__ int lane_here() {
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    return ln;
}

// The sixteen 16-byte B-operand loads of a group (lane (g, c): rows 16 t + c,
// dims 32 j + 8 g .. + 8; each instruction reads 64 contiguous bytes of 16
// rows).  A group without rows comes as no_group: a valid address.
__device__ __forceinline__ void load_group(const RowsArgs &a, const RGroup &e, int g, int c,
                                           uvec4 (&xa)[kRTiles][4]) {
    // a uniform base and one 32-bit element offset per load: the address
    // form with the base in scalar registers
    // (in bytes: an element offset doubled could pass 2^32 as far as the
    // compiler knows)
    const char *base = reinterpret_cast<const char *>(a.src_base + e.src);
#pragma unroll
    for (int t = 0; t < kRTiles; ++t) {
        const int r = 16 * t + c;
        const uint32_t off = (uint32_t)(r < e.nr ? r : 0) * (uint32_t)(2 * a.src_step) + 16u * (uint32_t)g;
        // (the 64 j bytes added after the extension go into the
        // instructions' immediate offsets)
        const uvec4 *src = reinterpret_cast<const uvec4 *>(base + (uint64_t)off);
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[t][j] = src[4 * j];
    }
}

// Sum over the four lanes (g, c), g = 0 .. 3, of a column c, in every one of
// them (the same association in each).
__device__ __forceinline__ float sum_over_g(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const uint32_t su = __float_as_uint(s);
    const auto q = __builtin_amdgcn_permlane16_swap(su, su, false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ uint32_t or_over_g(uint32_t v) {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    const uint32_t s = p[0] | p[1];
    const auto q = __builtin_amdgcn_permlane16_swap(s, s, false, false);
    return q[0] | q[1];
}

// Four words u0..u3 in each lane (g, c) -> the OR over g of u_g, in lane
// (g, c): rows 0-1 and 2-3 of the wave trade halves, then rows 0/1 and 2/3.
__device__ __forceinline__ uint32_t or_transpose4(uint32_t u0, uint32_t u1, uint32_t u2, uint32_t u3) {
    const auto p = __builtin_amdgcn_permlane32_swap(u0, u2, false, false);
    const uint32_t a = p[0] | p[1];   // rows 0, 1: u0 over g and g ^ 2; rows 2, 3: u2
    const auto q = __builtin_amdgcn_permlane32_swap(u1, u3, false, false);
    const uint32_t b = q[0] | q[1];   // rows 0, 1: u1; rows 2, 3: u3
    const auto s = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return s[0] | s[1];               // row g: u_g over all g
}

// The defining sum of bit `col` of a row (sequential, d = 0 .. 127; every
// product of a bf16 and an fp32 value is exact in double).  The row is read
// in quarters of four 16-byte loads issued together.
// The defining sum of one bit: y = sum over d of x_d W_dj, sequentially in
// double (each product of a bf16 and an fp32 is exact in double).  W comes
// from the transposed copy in LDS (r <= 128) or from memory (r = 256).
// Wide (the flush at r = 256, where W comes from memory and the group just
// encoded has freed its registers): the row (16 pieces of 16 bytes) is
// loaded at once, so that its latency is paid once, then W a quarter at a
// time; otherwise a quarter of the row and of W at a time (at r <= 128 the
// wide form measured slower).
template <int R, bool Wide>
__device__ __forceinline__ double exact_sum(const RowsSmem<R> &sm, const float *W, const uint16_t *xr,
                                            int col) {
    if constexpr (!Wide) {
        double y = 0.0;
#pragma unroll 1
        for (int d0 = 0; d0 < kHeadDim; d0 += 32) {
            uvec4 xq[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) xq[k] = *reinterpret_cast<const uvec4 *>(xr + d0 + 8 * k);
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int d = d0 + 8 * k + 2 * q;
                    const float w0 = R <= 128 ? sm.wt[R <= 128 ? col : 0][d] : W[(int64_t)d * R + col];
                    const float w1 = R <= 128 ? sm.wt[R <= 128 ? col : 0][d + 1] : W[(int64_t)(d + 1) * R + col];
                    const uint32_t u = xq[k][q];
                    y = fma((double)__uint_as_float(u << 16), (double)w0, y);
                    y = fma((double)__uint_as_float(u & 0xFFFF0000u), (double)w1, y);
                }
        }
        return y;
    } else {
        static_assert(R > 128, "the wide form is for W read from memory");
        uvec4 xv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) xv[k] = *reinterpret_cast<const uvec4 *>(xr + 8 * k);
        double y = 0.0;
        // (a quarter of W at a time: with two in flight the flush would
        // not fit beside the prefetched group's registers)
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
            float wq[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) wq[i] = W[(int64_t)(32 * qt + i) * R + col];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = 8 * k + 2 * q;
                    const uint32_t u = xv[4 * qt + k][q];
                    y = fma((double)__uint_as_float(u << 16), (double)wq[i], y);
                    y = fma((double)__uint_as_float(u & 0xFFFF0000u), (double)wq[i + 1], y);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        return y;
    }
}

// Resolve a wave's listed in-band bits: one lane per bit runs the defining
// sum and sets or clears the bit in the code word the wave has already stored
// (with the provisional sign of y').  The wave first waits for its own
// stores, so the word is in memory.
template <int R>
__device__ __forceinline__ void flush_list(const RowsArgs &a, RowsSmem<R> &sm, const float *W, int h, int count) {
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll 1
    for (int b = lane; b < count; b += 64) {
        // (a 32-bit division: the host keeps the group count below 2^32)
        const uint32_t gi = sm.lgrp[wv][b], gps = (uint32_t)a.groups_per_seg;
        const uint32_t es = gi / gps;
        const int rc = sm.lrc[wv][b], row = rc >> 8, col = rc & 255;
        const RGroup e = group_at<R, false>(a, sm, h, (int)es, gi - es * gps);
        const double y = exact_sum<R, (R > 128)>(sm, W, src_row(a, e, row), col);
        uint32_t *word = code_word<R>(a, e, row, col >> 5);
        const uint32_t bit = 1u << (col & 31);
        if (y > 0.0)
            atomicOr(word, bit);
        else
            atomicAnd(word, ~bit);
    }
}

// Resolve the listed bits in whole rounds of 64, one per lane (a round
// costs the latency of its loads however few lanes it has), or all of them
// when `all`; the entries left over move to the front of the wave's list.
// Returns how many are left.
template <int R>
__device__ __forceinline__ int flush_rounds(const RowsArgs &a, RowsSmem<R> &sm, const float *W, int h,
                                            int count, bool all) {
    const int done = all ? count : (count & ~63);
    if (done > 0) flush_list<R>(a, sm, W, h, done);
    const int rest = count - done;   // below 64
    if (rest > 0) {
        const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        uint32_t gq = 0u;
        uint16_t rc = 0;
        if (lane < rest) {
            gq = sm.lgrp[wv][done + lane];
            rc = sm.lrc[wv][done + lane];
        }
        if (lane < rest) {
            sm.lgrp[wv][lane] = gq;
            sm.lrc[wv][lane] = rc;
        }
    }
    return rest;
}

// Every code word of a group by the defining sums (a group with more in-band
// bits than the list holds: rows with a non-finite value, degenerate rows):
// one lane per word.
template <int R>
__device__ __forceinline__ void exact_group(const RowsArgs &a, const RowsSmem<R> &sm, const float *W, int h,
                                            const RGroup &e) {
    constexpr int NW = R / 32;
    const int lane = threadIdx.x & 63;
#pragma unroll 1
    for (int w = lane; w < e.nr * NW; w += 64) {
        const int row = w / NW, k = w % NW;
        const uint16_t *xr = src_row(a, e, row);
        uint32_t word = 0u;
#pragma unroll 1
        for (int b = 0; b < 32; ++b)
            if (exact_sum<R, false>(sm, W, xr, 32 * k + b) > 0.0) word |= 1u << b;
        *code_word<R>(a, e, row, k) = word;
    }
}

// Column tiles per pass: a pass yields four code words (two for r = 64, one
// for r = 32) per row; r = 256 takes two passes over the group's registers.
template <int R>
constexpr int pass_tiles() { return R >= 128 ? 8 : R / 16; }

// The A operands of column tile n, k steps j0 and j0 + 1, into ah / al.
template <int R>
__device__ __forceinline__ void load_aop(const RowsSmem<R> &sm, int n, int j0, int lane, bf16x8 (&ah)[4],
                                         bf16x8 (&al)[4]) {
#pragma unroll
    for (int j = j0; j < j0 + 2; ++j) {
        ah[j] = __builtin_bit_cast(bf16x8, sm.aop[n][j][0][lane]);
        al[j] = __builtin_bit_cast(bf16x8, sm.aop[n][j][1][lane]);
    }
}

// y'^T of column tile n for the 64 rows: four independent accumulator chains
// (row tiles), the high and the low part of W' into the same one; k steps
// j0, j0 + 1.
__device__ __forceinline__ void tile_mfma(const bf16x8 (&ah)[4], const bf16x8 (&al)[4],
                                          const uvec4 (&xa)[kRTiles][4], int j0, f32x4 (&acc)[kRTiles]) {
#pragma unroll
    for (int j = j0; j < j0 + 2; ++j) {
#pragma unroll
        for (int t = 0; t < kRTiles; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[j], __builtin_bit_cast(bf16x8, xa[t][j]), acc[t],
                                                             0, 0, 0);
#pragma unroll
        for (int t = 0; t < kRTiles; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[j], __builtin_bit_cast(bf16x8, xa[t][j]), acc[t],
                                                             0, 0, 0);
    }
}

// Codes of one group whose rows are in xa (see the header comment).
template <int R>
__device__ __forceinline__ void encode_group(const RowsArgs &a, RowsSmem<R> &sm, const float *W, int h,
                                             int64_t gi, const RGroup &e, uvec4 (&xa)[kRTiles][4],
                                             int wv, int &n_list) {
    constexpr int NT = R / 16;          // column tiles
    constexpr int NW = R / 32;          // code words per row
    constexpr int PT = pass_tiles<R>();
    constexpr int NPASS = NT / PT;
    constexpr int PW = PT / 2;          // code words per pass (1, 2 or 4)
    constexpr int NPAIR = PW >= 2 ? PW / 2 : 1;
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    // The next group's sixteen loads were the last memory operations issued:
    // wait for everything before them (this group's rows, the previous
    // group's stores).  With no store left in flight the compiler's own waits
    // on this group's registers need not assume out-of-order completion
    // (which would make them wait for the prefetch too).
    __builtin_amdgcn_s_waitcnt(kWaitAllButPrefetch);
    // (an instruction between this wait and the first use below, so that the
    // compiler applies the wait before working out the use's own)
    asm volatile("s_nop 0");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kRTiles; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(xa[t][j]));   // uses stay after the wait
    // ---- tile 0's products, interleaved with the row norms below (the two
    // are independent; the norms' branch for rows of zeros comes after)
    bf16x8 ah[4], al[4];
    f32x4 acc[kRTiles], nxt[kRTiles];
    load_aop<R>(sm, 0, 0, lane, ah, al);
    load_aop<R>(sm, 0, 2, lane, ah, al);
#pragma unroll
    for (int t = 0; t < kRTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    tile_mfma(ah, al, xa, 0, acc);
    tile_mfma(ah, al, xa, 2, acc);
    // ---- thresholds: lane (g, c) sums the squares of its 32 dims of row
    // 16 t + c, the four lanes of the row add theirs.  A sum of 0 is a row of
    // zeros (threshold -1: every bit 0, decided) or of values too small to
    // square (threshold 2^-72); a non-finite sum gives +inf (the group goes
    // to the exact sums).
    float th[kRTiles];
    bool small = false, nonfinite = false;
#pragma unroll
    for (int t = 0; t < kRTiles; ++t) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // the element goes through a scalar: a bit cast of the vector
                // element expression itself reads element 0 with this compiler
                const uint32_t u = xa[t][j][q];
                const bf16x2 p = __builtin_bit_cast(bf16x2, u);
                ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
            }
        ss = sum_over_g(ss);
        // v_sqrt_f32 (1 ulp; the 2^-10 margin covers it)
        th[t] = ss < INFINITY ? fmaf(__builtin_amdgcn_sqrtf(ss), (1.f + 0x1p-10f) * 0x1p-14f, 0x1p-72f) : INFINITY;
        small |= ss == 0.f;
        nonfinite |= !(ss < INFINITY);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // tile 0's operands
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
#pragma unroll
    for (int m = 0; m < 8 * kRTiles; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    if (__builtin_amdgcn_ballot_w64(small) != 0) {
#pragma unroll
        for (int t = 0; t < kRTiles; ++t) {
            uint32_t nz = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) nz |= xa[t][j][q];
            if (or_over_g(nz & 0x7FFF7FFFu) == 0u) th[t] = -1.f;
        }
    }
    bool overflow = __builtin_amdgcn_ballot_w64(nonfinite) != 0;

    // ---- column tiles, in passes of PT.  Per tile: sign bits (1 for a
    // negative y') go in at bit 0 of the word being built: after the even
    // tile of a code word the lane holds its four bits at i, shifted up by
    // 12; after the odd one, at 16 + i and i, and rotating right by 16 - 4 g
    // puts them at 4 g + i and 16 + 4 g + i, their places in the word.
    // Completed words are paired across the two halves of the wave at once.
    // The band flags (sign of th - |y'|: 1 where the bit is decided) go into
    // dec[t], four bits per tile.  Tile n's band test and sign bits run while
    // tile n + 1's matrix products issue (the two are interleaved in the
    // schedule), and tile n + 2's A operands load behind them.
    const uint32_t rot = 16 - 4 * g;
    const int q = ((g & 1) << 1) | (g >> 1);
    uint32_t word[kRTiles][NPASS];   // lane (g, c): word q(g) of the pass, row 16 t + c
    uint32_t dec[kRTiles][NPASS];
    if (NT > 1) {
        load_aop<R>(sm, NT > 1 ? 1 : 0, 0, lane, ah, al);
        load_aop<R>(sm, NT > 1 ? 1 : 0, 2, lane, ah, al);
    }
#pragma unroll
    for (int t = 0; t < kRTiles; ++t) asm volatile("" : "+v"(acc[t]));
    __builtin_amdgcn_sched_barrier(0);
    // The tiles at a raised wave priority: of the two waves of a SIMD, the
    // one feeding the matrix core issues first, and the other's vector work
    // (listing, stores, norms) fills the gaps (measured 1 % faster at 128
    // bits, 2-4 % at 256).
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        uint32_t cur[kRTiles], held[kRTiles], pair[kRTiles][NPAIR];
#pragma unroll
        for (int t = 0; t < kRTiles; ++t) dec[t][p] = 0u;
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const int n = p * PT + k;
            // tile n + 1's products, then tile n + 2's operands
            if (n + 1 < NT) {
#pragma unroll
                for (int t = 0; t < kRTiles; ++t) nxt[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                tile_mfma(ah, al, xa, 0, nxt);
                if (n + 2 < NT) load_aop<R>(sm, n + 2 < NT ? n + 2 : 0, 0, lane, ah, al);
                tile_mfma(ah, al, xa, 2, nxt);
                if (n + 2 < NT) load_aop<R>(sm, n + 2 < NT ? n + 2 : 0, 2, lane, ah, al);
            }
            // tile n: band flags and sign bits
#pragma unroll
            for (int t = 0; t < kRTiles; ++t) {
                uint32_t d = dec[t][p], s = (k & 1) ? cur[t] : 0u;
#pragma unroll
                for (int i = 3; i >= 0; --i) {
                    d = __builtin_amdgcn_alignbit(d, __float_as_uint(th[t] - fabsf(acc[t][i])), 31);
                    s = __builtin_amdgcn_alignbit(s, __float_as_uint(acc[t][i]), 31);
                }
                dec[t][p] = d;
                if ((k & 1) == 0) {
                    cur[t] = s << 12;
                } else {
                    s = __builtin_amdgcn_alignbit(s, s, rot);
                    const int w = k >> 1;
                    if (PW == 1 || (w & 1)) {
                        const auto sw = __builtin_amdgcn_permlane32_swap(PW == 1 ? s : held[t], PW == 1 ? 0u : s,
                                                                         false, false);
                        pair[t][w >> 1] = sw[0] | sw[1];
                    } else {
                        held[t] = s;
                    }
                }
            }
            // keep each tile's work in its own stretch of the schedule, the
            // products and band test interleaved, the operand loads after the
            // products that read the registers they replace
            if (n + 1 < NT) {
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one product
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // two vector ALU
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);       // operand loads
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            }
#pragma unroll
            for (int t = 0; t < kRTiles; ++t) {
                asm volatile("" ::"v"(dec[t][p]));
                if (k & 1) {
                    if (PW == 1 || ((k >> 1) & 1)) asm volatile("" ::"v"(pair[t][k >> 2]));
                    else asm volatile("" ::"v"(held[t]));
                } else {
                    asm volatile("" ::"v"(cur[t]));
                }
                if (n + 1 < NT) asm volatile("" : "+v"(nxt[t]));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < kRTiles; ++t) acc[t] = nxt[t];
        }
        // ---- the second lane swap: lane (g, c) of row tile t ends with word
        // q(g) = {0, 2, 1, 3}[g] of the pass's four words of row 16 t + c
#pragma unroll
        for (int t = 0; t < kRTiles; ++t) {
            const auto sw = __builtin_amdgcn_permlane16_swap(pair[t][0], NPAIR > 1 ? pair[t][NPAIR > 1 ? 1 : 0] : 0u,
                                                             false, false);
            word[t][p] = sw[0] | sw[1];
        }
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- list the in-band bits: band flag 0, columns of zeros excepted
    // (their bit is 0), rows past the group's count skipped.  Flag bit
    // 4 (PT - 1 - k) + i of pass p is column 16 (p PT + k) + 4 g + i.  Each
    // lane writes its own entries, at its place in one prefix sum over the
    // wave of the lanes' counts.
    const int list0 = n_list;  // this group's entries start here (uniform)
    constexpr uint32_t kFlagMask = PT == 8 ? 0xFFFFFFFFu : (1u << (4 * PT)) - 1u;
    // (the zero-column masks are read from LDS here and before the stores,
    // at an index the compiler takes as new per group: kept in registers
    // across the loop they cost up to four more)
    int gz = g;
    asm volatile("" : "+v"(gz));
    const ZeroCols<R> &zc = sm.zlane[gz];
    uint32_t inb[NPASS][kRTiles];
    int cnt = 0;
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
#pragma unroll
        for (int t = 0; t < kRTiles; ++t) {
            inb[p][t] = 16 * t + c < e.nr ? ~dec[t][p] & kFlagMask & ~zc.flags[p] : 0u;
            cnt += __builtin_popcount(inb[p][t]);
        }
    if (__builtin_amdgcn_ballot_w64(cnt != 0) != 0) {
        const int incl = wave_incl_scan(cnt);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (n_list + total > kRList) {
            overflow = true;
        } else {
            int pos = n_list + incl - cnt;
#pragma unroll
            for (int p = 0; p < NPASS; ++p)
#pragma unroll
                for (int t = 0; t < kRTiles; ++t) {
                    uint32_t m = inb[p][t];
                    while (m) {
                        const int b = __builtin_ctz(m);
                        m &= m - 1;
                        const int col = 16 * (p * PT + PT - 1 - (b >> 2)) + 4 * g + (b & 3);
                        sm.lgrp[wv][pos] = (uint32_t)gi;
                        sm.lrc[wv][pos] = (uint16_t)(((16 * t + c) << 8) | col);
                        ++pos;
                    }
                }
            n_list += total;
        }
    }

    if (overflow) {
        // too many in-band bits, or a non-finite row: every word of the group
        // by the exact sums
        n_list = list0;
        exact_group<R>(a, sm, W, h, e);
    } else {
        // ---- store: lane (g, c) of row tile t writes word 4 p + q(g) of row
        // 16 t + c.  Codes are 1 for y' > 0: the complement of the sign bits,
        // with columns of zeros and rows of zeros at 0.
        // (the addresses are formed here from lane_here(), per group)
        const int ln = lane_here(), gg = (ln >> 4) & 3, cc = ln & 15;
        const int qq = ((gg & 1) << 1) | (gg >> 1);
        // (the masks read once, ahead of the selects below: read inside them
        // they would take one LDS round trip per row tile)
        uint32_t zw[NPASS];
#pragma unroll
        for (int p = 0; p < NPASS; ++p) zw[p] = sm.zlane[gg].word[p];
#pragma unroll
        for (int t = 0; t < kRTiles; ++t) {
            const int row = 16 * t + cc;
            const bool live = row < e.nr;
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const uint32_t o = th[t] < 0.f ? 0u : ~(word[t][p] | zw[p]);
                if (live && 4 * p + qq < NW) {
                    // streaming stores (the kernel touches a stored word
                    // again only for an in-band bit, by an atomic after its
                    // stores have completed); measured faster at r <= 128,
                    // not at 256
                    if constexpr (R <= 128)
                        __builtin_nontemporal_store(o, code_word<R>(a, e, row, 4 * p + qq));
                    else
                        *code_word<R>(a, e, row, 4 * p + qq) = o;
                }
            }
        }
    }
    // ---- appended rows into the cache: K from the registers, V copied
    if (a.mode == 1 && a.k_new) {
        const int ln = lane_here(), gk = (ln >> 4) & 3, ck = ln & 15;
#pragma unroll
        for (int t = 0; t < kRTiles; ++t) {
            const int r = 16 * t + ck;
            if (r < e.nr) {
                const int64_t crow = e.code / (R / 32) + r;   // cache row
                uint16_t *kd = a.k_cache + crow * kHeadDim + 8 * gk;
                uint16_t *vd = a.v_cache + crow * kHeadDim + 8 * gk;
                const uint16_t *vs = a.v_new + e.src + (int64_t)r * a.src_step + 8 * gk;
                uvec4 vv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) vv[j] = *reinterpret_cast<const uvec4 *>(vs + 32 * j);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    *reinterpret_cast<uvec4 *>(kd + 32 * j) = xa[t][j];
                    *reinterpret_cast<uvec4 *>(vd + 32 * j) = vv[j];
                }
            }
        }
    }
}

// The entry and group of non-empty group gq of a head (prefix sums in
// seg_pre; entries from s_from on): n_seg past the last one.
template <int R>
__device__ __forceinline__ int2 dense_at(const RowsSmem<R> &sm, int n_seg, int s_from, int64_t gq,
                                         int64_t n_dense) {
    if (gq >= n_dense) return int2{n_seg, 0};
    const int q = (int)gq;
    int s0 = s_from;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (q >= sm.seg_pre[s0 + 1]) ++s0;
    if (q >= sm.seg_pre[s0 + 1]) {  // binary search over (s0, n_seg)
        int lo = s0 + 1, hi = n_seg - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sm.seg_pre[mid] <= q) lo = mid;
            else hi = mid - 1;
        }
        s0 = lo;
    }
    s0 = __builtin_amdgcn_readfirstlane(s0);
    return int2{s0, q - sm.seg_pre[s0]};
}

// ---- the wave's groups, two register buffers: the next group loads
// while this one is computed.  Group gi of the head is group gi mod G of
// batch entry gi / G (G groups per entry); the wave takes every stride-th,
// from blockIdx.x * waves + wave, and steps the (entry, group) pair by
// (stride / G, stride mod G) with a carry (no division per step).  With the
// prefix sums (dense), group gi of the head is the non-empty group
// gi - seg_pre[s] of the entry s with seg_pre[s] <= gi < seg_pre[s + 1],
// found by stepping s forward (a binary search when the stride spans more
// than a few entries).  Returns the wave's in-band bits not yet resolved.
template <int R>
__device__ __forceinline__ int wave_groups(const RowsArgs &a, RowsSmem<R> &sm, const float *W, int h,
                                           int wv, int g, int c, bool dense) {
    const int64_t gps = a.groups_per_seg;
    const int64_t stride = (int64_t)gridDim.x * kRWaves;
    const int64_t step_s = stride / gps, step_g = stride - step_s * gps;
    const RGroup none = no_group(a, h);
    int64_t gi = (int64_t)blockIdx.x * kRWaves + wv;
    int64_t cs = gi / gps, cg = gi - cs * gps;   // entry and group of gi
    const int64_t n_dense = dense ? (int64_t)sm.seg_pre[a.n_seg] : 0;
    if (dense) {
        const int2 l = dense_at<R>(sm, a.n_seg, 0, gi, n_dense);
        cs = l.x;
        cg = l.y;
    }
    uvec4 xa0[kRTiles][4], xa1[kRTiles][4];
    int n_list = 0;  // in-band bits listed by this wave, not yet resolved (uniform)
    // The loads are issued whether or not the group has rows (one past the
    // work, or skipped, reads row 0 of the head: a valid address), so that
    // the count of loads in flight is the same on every path and a group's
    // use waits only for its own loads.  A group is listed for the exact
    // sums under its index among all of the head's group slots, entry *
    // groups_per_seg + group, which flush_list decodes.
    RGroup e0 = cs < a.n_seg ? group_at<R, true>(a, sm, h, (int)cs, cg) : none;
    int64_t sp0 = cs * gps + cg;
    load_group(a, e0.nr > 0 ? e0 : none, g, c, xa0);
    while (cs < a.n_seg) {
        const int64_t gi1 = gi + stride;
        if (dense) {
            const int2 l = dense_at<R>(sm, a.n_seg, (int)cs, gi1, n_dense);
            cs = l.x;
            cg = l.y;
        } else {
            cg += step_g;
            cs += step_s;
            if (cg >= gps) {
                cg -= gps;
                ++cs;
            }
        }
        const RGroup e1 = cs < a.n_seg ? group_at<R, true>(a, sm, h, (int)cs, cg) : none;
        const int64_t sp1 = cs * gps + cg;
        load_group(a, e1.nr > 0 ? e1 : none, g, c, xa1);
        if (e0.nr > 0) encode_group<R>(a, sm, W, h, sp0, e0, xa0, wv, n_list);
        if (n_list >= 64) n_list = flush_rounds<R>(a, sm, W, h, n_list, false);
        const int64_t gi2 = gi1 + stride;
        if (dense) {
            const int2 l = dense_at<R>(sm, a.n_seg, (int)cs, gi2, n_dense);
            cs = l.x;
            cg = l.y;
        } else {
            cg += step_g;
            cs += step_s;
            if (cg >= gps) {
                cg -= gps;
                ++cs;
            }
        }
        e0 = cs < a.n_seg ? group_at<R, true>(a, sm, h, (int)cs, cg) : none;
        sp0 = cs * gps + cg;
        load_group(a, e0.nr > 0 ? e0 : none, g, c, xa0);
        if (e1.nr > 0) encode_group<R>(a, sm, W, h, sp1, e1, xa1, wv, n_list);
        if (n_list >= 64) n_list = flush_rounds<R>(a, sm, W, h, n_list, false);
        gi = gi2;
    }
    return n_list;
}

template <int R>
__global__ __launch_bounds__(kRThreads, 1) void k_encode_rows(RowsArgs a) {
    constexpr int NT = R / 16;   // column tiles
    __shared__ RowsSmem<R> sm;
    const int h = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6), g = lane >> 4, c = lane & 15;
    const float *W = a.w + (int64_t)h * kHeadDim * R;

    // ---- set-up 1: per column, the scale that brings ||W_:j|| to 1: first a
    // power of two (from the largest element, exponent e: W 2^-e has elements
    // below 1 and a sum of squares that fp32 holds), then a factor in [1, 2);
    // and the zero columns
    if (t < R / 32) sm.zcol[t] = 0u;
    __syncthreads();
    for (int col = t; col < R; col += kRThreads) {
        float mx = 0.f;
        bool finite = true;
        for (int d = 0; d < kHeadDim; ++d) {
            const float v = fabsf(W[(int64_t)d * R + col]);
            finite = finite && v < INFINITY;
            mx = fmaxf(mx, v);
        }
        int s = INT_MIN;
        float m = 1.f;
        if (!finite) {
            // W' taken as 0: every bit of the column goes to the exact sum
        } else if (mx == 0.f) {
            atomicOr(&sm.zcol[col >> 5], 1u << (col & 31));
        } else {
            int e;
            frexpf(mx, &e);
            float ss = 0.f;
            for (int d = 0; d < kHeadDim; ++d) {
                const float v = ldexpf(W[(int64_t)d * R + col], -e);
                ss = fmaf(v, v, ss);
            }
            int f;
            frexpf(sqrtf(ss) * (1.f + 0x1p-10f), &f);
            s = -e - f;
            // W 2^s has a norm in (1/2, 1]; m = 1 / that norm brings it to 1
            float ss2 = 0.f;
            for (int d = 0; d < kHeadDim; ++d) {
                const float v = ldexpf(W[(int64_t)d * R + col], s);
                ss2 = fmaf(v, v, ss2);
            }
            m = 1.f / sqrtf(ss2);
        }
        sm.col_exp[col] = s;
        sm.col_mul[col] = m;
    }
    __syncthreads();
    // ---- set-up 2: A operands (lane (g, c) of column tile n, k step j holds
    // W'[32 j + 8 g + e][16 n + c], e < 8, as bf16 high and low parts), W_H
    // transposed, the entries' lengths
    for (int i = t; i < NT * 4 * 64; i += kRThreads) {
        const int l = i & 63, j = (i >> 6) & 3, n = i >> 8;
        const int col = 16 * n + (l & 15), d0 = 32 * j + 8 * (l >> 4);
        const int s = sm.col_exp[col];
        const float m = sm.col_mul[col];
        float wf[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) wf[q] = W[(int64_t)(d0 + q) * R + col];
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int q = 0; q < 8; q += 2) {
            const float v0 = s == INT_MIN ? 0.f : ldexpf(wf[q], s) * m;
            const float v1 = s == INT_MIN ? 0.f : ldexpf(wf[q + 1], s) * m;
            const uint16_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
            const uint16_t l0 = f32_to_bf16(v0 - __uint_as_float((uint32_t)h0 << 16));
            const uint16_t l1 = f32_to_bf16(v1 - __uint_as_float((uint32_t)h1 << 16));
            hw[q / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lw[q / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        sm.aop[n][j][0][l] = uvec4{hw[0], hw[1], hw[2], hw[3]};
        sm.aop[n][j][1][l] = uvec4{lw[0], lw[1], lw[2], lw[3]};
        if constexpr (R <= 128) {
#pragma unroll
            for (int q = 0; q < 8; ++q) sm.wt[col][d0 + q] = wf[q];
        }
    }
    // Batches of 16 to kRSegLds entries (lengths in LDS) also get the prefix
    // sum of their group counts, and when a quarter or more of
    // the head's group slots are empty (a ragged batch sets the group count
    // of every entry by its longest append) the waves step over the
    // non-empty groups only (64 ragged sequences of up to 64K keys: 1.41 ->
    // 1.32 ms; with few empty slots the search costs more than it saves).
    const bool scan_groups = a.mode == 1 && a.n_seg >= 16 && a.n_seg <= kRSegLds;
    int groups0 = 0, groups1 = 0;  // group counts of this thread's entries t and t + 512
    if (a.mode == 1) {
        for (int s = t; s < a.n_seg && s < kRSegLds; s += kRThreads) {
            const int64_t l0 = a.seq_len[s];
            const int n = a.n_new[s];
            const int rows = rows_append_ok(l0, n, a.t_max, a.max_ctx) ? n : 0;
            sm.seg_l0[s] = l0;
            sm.seg_rows[s] = rows;
            if (s < kRThreads) groups0 = (rows + kRGroup - 1) / kRGroup;
            else groups1 = (rows + kRGroup - 1) / kRGroup;
        }
    }
    if (scan_groups) {
        // exclusive prefix sum over entries 0 .. n_seg - 1: entry s is
        // thread s % 512's, pass s / 512
        int base = 0;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int v = pass == 0 ? groups0 : groups1;
            int incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int u = __shfl_up(incl, o, 64);
                if (lane >= o) incl += u;
            }
            if (lane == 63) sm.wsum[wv] = incl;
            __syncthreads();
            int before = base, total = base;
#pragma unroll
            for (int w2 = 0; w2 < kRWaves; ++w2) {
                const int ws = sm.wsum[w2];
                before += w2 < wv ? ws : 0;
                total += ws;
            }
            const int s = pass * kRThreads + t;
            if (s < a.n_seg) sm.seg_pre[s] = before + incl - v;
            if (s == a.n_seg - 1) sm.seg_pre[a.n_seg] = before + incl;
            if (t == 0 && a.n_seg == 0) sm.seg_pre[0] = 0;
            base = total;
            __syncthreads();
        }
    }
    __syncthreads();
    if (t < 4) {
        constexpr int PT = pass_tiles<R>();
        const int gz = t, q = ((gz & 1) << 1) | (gz >> 1);
#pragma unroll
        for (int p = 0; p < NT / PT; ++p) {
            sm.zlane[gz].word[p] = sm.zcol[4 * p + q < R / 32 ? 4 * p + q : 0];
            uint32_t f = 0u;
#pragma unroll
            for (int k = 0; k < PT; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = 16 * (p * PT + k) + 4 * gz + i;
                    f |= ((sm.zcol[col >> 5] >> (col & 31)) & 1u) << (4 * (PT - 1 - k) + i);
                }
            sm.zlane[gz].flags[p] = f;
        }
    }
    __syncthreads();

    const bool dense = scan_groups && 4 * (int64_t)sm.seg_pre[a.n_seg] <= 3 * a.n_seg * a.groups_per_seg;
    const int n_list = wave_groups<R>(a, sm, W, h, wv, g, c, dense);
    if (n_list > 0) flush_rounds<R>(a, sm, W, h, n_list, true);

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
    if (!rows_shape_fits(n_rows, 1, row_stride)) return hipErrorInvalidValue;
    RowsArgs a = {};
    a.mode = 0;
    a.keys = keys;
    a.row_stride = row_stride;
    a.head_stride = head_stride;
    a.n_rows = n_rows;
    a.codes_out = codes;
    a.src_base = keys;
    a.codes_base = codes;
    a.src_step = (int)row_stride;
    a.code_step = n_heads * (n_bits / 32);
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
    if (!rows_shape_fits(t_max, B, k_new ? (int64_t)Hkv * kHeadDim : kHeadDim)) return hipErrorInvalidValue;
    RowsArgs a = {};
    a.mode = 1;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.codes = codes;
    a.src_base = k_new ? k_new : k_cache;
    a.codes_base = codes;
    a.src_step = k_new ? Hkv * kHeadDim : kHeadDim;
    a.code_step = n_bits / 32;
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
