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
// Work split: grid.y = head; one 512-thread workgroup per CU walks 64-row
// tiles of its head.  Wave w (of 8) owns code bits 16 w .. 16 w + 15 and keeps
// their W operands in registers (for MFMA j, lane (g, c) holds dims
// 32 j + 8 g .. + 8 of column 16 w + c).  Tiles stream through kEBuf LDS
// buffers with global_load_lds (no registers; the next tiles are on their
// way while one is computed): waves 0-3 issue every tile's loads, always the
// same count, so their waits on the memory counter are exact; the tile rows
// are stored with their 16-byte chunks XOR-swizzled by row so that the A
// operand reads (16 rows, one chunk each) hit distinct banks.  W_H
// transposed stays in LDS for the recomputations.  Each wave's 16-bit halves
// of the code words go through LDS, and wave 4 stores whole words.
#include "device_util.h"
#include "hata_internal.h"
#include "../../include/hata.h"

namespace hata {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t uvec4 __attribute__((ext_vector_type(4)));

constexpr int kERows = 64;     // rows per tile
constexpr int kEThreads = 512;
constexpr int kEBuf = 4;       // tiles in LDS: one computed, three on their way
constexpr int kESegLds = 1024; // batch entries whose lengths are kept in LDS

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
    float wt[kBits][kHeadDim];             // W_H transposed: wt[j][t] = W[t][j]
    uint16_t xs[kEBuf][kERows][kHeadDim];  // tile rows (bf16), 16-byte chunks swizzled
    uint16_t half[kERows][2 * kWords];     // each wave's 16 code bits per row
    int64_t seg_l0[kESegLds];              // mode 1: each entry's length ...
    int32_t seg_rows[kESegLds];            // ... and rows to encode
    int last;
};

__device__ __forceinline__ bool append_ok(int64_t len, int n, int t_max, int64_t max_ctx) {
    return n >= 0 && n <= t_max && len >= 0 && len + n <= max_ctx;
}

// Chunk k (dims 8 k .. 8 k + 7) of tile row R sits at chunk k ^ (R & 15).
__device__ __forceinline__ int swz(int R, int k) { return k ^ (R & 15); }

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

// The exact bit (row R of the tile in xs, column col): see the header comment.
__device__ __forceinline__ bool exact_bit(const ESmem &sm, const uint16_t (*xs)[kHeadDim], int R, int col) {
    const int lane = threadIdx.x & 63;
    const int k = swz(R, lane >> 2), e = (2 * lane) & 7;  // dims 2 lane, 2 lane + 1
    const double x0 = (double)bf16_to_f32(xs[R][8 * k + e]);
    const double x1 = (double)bf16_to_f32(xs[R][8 * k + e + 1]);
    const double p0 = x0 * (double)sm.wt[col][2 * lane], p1 = x1 * (double)sm.wt[col][2 * lane + 1];
    const double s = dsum64(p0 + p1);
    const double A = dsum64(fabs(p0) + fabs(p1));
    bool bit = s > 0.0;
    if (!(fabs(s) > 0x1p-44 * A)) {
        int b = 0;
        if (lane == 0) {
            double y = 0.0;  // the defining sequential sum
            for (int t = 0; t < kHeadDim; ++t)
                y = fma((double)bf16_to_f32(xs[R][8 * swz(R, t >> 3) + (t & 7)]), (double)sm.wt[col][t], y);
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

// A tile: its batch entry s, first row r0, the entry's length l0 and rows nr
// in this tile (0 when the tile is past the work or the entry is skipped).
struct ETile {
    int s;
    int64_t r0, l0;
    int nr;
};

__device__ __forceinline__ ETile tile_of(const EncArgs &a, const ESmem &sm, int64_t tile, int64_t n_tiles) {
    ETile e{0, 0, 0, 0};
    if (tile >= n_tiles) return e;
    if (n_tiles <= 0x7FFFFFFF) {  // 32-bit division (the 64-bit one is a long routine)
        const uint32_t t32 = (uint32_t)tile, tps = (uint32_t)a.tiles_per_seg;
        e.s = (int)(t32 / tps);
        e.r0 = (int64_t)(t32 - (uint32_t)e.s * tps) * kERows;
    } else {
        e.s = (int)(tile / a.tiles_per_seg);
        e.r0 = (tile % a.tiles_per_seg) * kERows;
    }
    int64_t rows;
    if (a.mode == 0) {
        rows = a.n_rows;
    } else if (e.s < kESegLds) {
        e.l0 = sm.seg_l0[e.s];
        rows = sm.seg_rows[e.s];
    } else {
        e.l0 = a.seq_len[e.s];
        const int n = a.n_new[e.s];
        rows = append_ok(e.l0, n, a.t_max, a.max_ctx) ? n : 0;
    }
    e.nr = e.r0 < rows ? (int)(rows - e.r0 < kERows ? rows - e.r0 : kERows) : 0;
    return e;
}

// Source of key row r (0 .. 63) of a tile of head h; rows past the tile's
// count read its first row (or, for an empty tile, row 0 of the head).
__device__ __forceinline__ const uint16_t *tile_row(const EncArgs &a, int h, const ETile &e, int r) {
    const int64_t rr = e.nr > 0 ? e.r0 + (r < e.nr ? r : 0) : 0;
    if (a.mode == 0) return a.keys + rr * a.row_stride + (int64_t)h * a.head_stride;
    const int s = e.nr > 0 ? e.s : 0;
    const int64_t l0 = e.nr > 0 ? e.l0 : 0;
    if (a.k_new) return a.k_new + (((int64_t)s * a.t_max + rr) * a.Hkv + h) * kHeadDim;
    return a.k_cache + (((int64_t)s * a.Hkv + h) * a.max_ctx + l0 + rr) * kHeadDim;
}

// Waves 0-3: the tile's 64 rows into LDS buffer xb, four instructions per
// wave (one instruction fills four 256-byte rows; lane l writes chunk l & 15
// of row 4 r + (l >> 4), i.e. global chunk swz(row, l & 15)).
__device__ __forceinline__ void tile_issue(const EncArgs &a, int h, const ETile &e, uint16_t (*xb)[kHeadDim]) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 4 * wv + q, row = 4 * r + (lane >> 4);
        const uint16_t *src = tile_row(a, h, e, row) + 8 * swz(row, lane & 15);
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)&xb[4 * r][0], 16, 0, 0);
    }
}

// s_waitcnt with vmcnt(n) (n < 16), expcnt and lgkmcnt not waited for.
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F7C); break;  // 12
    }
}

__global__ __launch_bounds__(kEThreads, 1) void k_encode_mfma(EncArgs a) {
    __shared__ ESmem sm;
    const int h = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, g = lane >> 4, c = lane & 15;
    const float *W = a.w + (int64_t)h * kHeadDim * kBits;

    // ---- W_H transposed into LDS, the entries' lengths, and this wave's B
    // operands (column 16 wv + c, rows 32 j + 8 g + e) split into bf16 hi / lo
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
    if (a.mode == 1) {
        for (int s = t; s < a.n_seg && s < kESegLds; s += kEThreads) {
            const int64_t l0 = a.seq_len[s];
            const int n = a.n_new[s];
            sm.seg_l0[s] = l0;
            sm.seg_rows[s] = append_ok(l0, n, a.t_max, a.max_ctx) ? n : 0;
        }
    }
    bf16x8 bhi[4], blo[4];
    float wnorm;
    {
        const int col = 16 * wv + c;
        float wv32[4][8];  // all loads first, then the conversions
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) wv32[j][e] = W[(32 * j + 8 * g + e) * kBits + col];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float wf = wv32[j][e];
                const uint16_t hb = f32_to_bf16(wf);  // nearest even; NaN stays NaN
                const float hf = __uint_as_float((uint32_t)hb << 16);
                const uint16_t lb = f32_to_bf16(wf - hf);
                bhi[j][e] = __builtin_bit_cast(__bf16, hb);
                blo[j][e] = __builtin_bit_cast(__bf16, lb);
                ss = fmaf(wf, wf, ss);
            }
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        wnorm = sqrtf(ss) * (1.f + 0x1p-10f);
    }
    __syncthreads();  // W_H and the lengths in LDS

    const int64_t n_tiles = a.tiles_per_seg * a.n_seg;
    const int64_t ntk = blockIdx.x < n_tiles ? (n_tiles - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
    // the first kEBuf tiles on their way
    if (wv < 4) {
#pragma unroll
        for (int b = 0; b < kEBuf; ++b)
            tile_issue(a, h, tile_of(a, sm, blockIdx.x + (int64_t)b * gridDim.x, n_tiles), sm.xs[b]);
    }
    for (int64_t k = 0; k < ntk; ++k) {
        const int b = (int)(k % kEBuf);
        uint16_t (*xb)[kHeadDim] = sm.xs[b];
        const ETile e = tile_of(a, sm, blockIdx.x + k * gridDim.x, n_tiles);
        // waves 0-3 issued four loads per tile, the kEBuf - 1 later tiles'
        // after this one's: wait for this tile, then every wave may read it
        if (wv < 4) wait_vm(4 * (kEBuf - 1));
        __syncthreads();
        if (e.nr > 0) {
            // ---- A operands from LDS, row norms
            uvec4 xa[4][4];
            float xnorm[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int R = 16 * mt + c;
                float ss = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xa[mt][j] = *reinterpret_cast<const uvec4 *>(&xb[R][8 * swz(R, 4 * j + g)]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bf16x2 p = __builtin_bit_cast(bf16x2, xa[mt][j][q]);
                        ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
                    }
                }
                ss += __shfl_xor(ss, 16, 64);
                ss += __shfl_xor(ss, 32, 64);
                xnorm[mt] = sqrtf(ss) * (1.f + 0x1p-10f);
            }
            // ---- y' on the matrix cores: acc[mt] holds rows 16 mt + 4 g + i,
            // column 16 wv + c
            f32x4 acc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 xv = __builtin_bit_cast(bf16x8, xa[mt][j]);
                    v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, bhi[j], v, 0, 0, 0);
                    v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, blo[j], v, 0, 0, 0);
                }
                acc[mt] = v;
            }
            // ---- bits: the decided ones by ballot in one straight pass
            // (lane L assembles the 16 bits of row L), then, only if some bit
            // lies inside the band, a second pass recomputes those exactly
            float xnr[4][4];  // the norm of row 16 mt + 4 g + i
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) xnr[mt][i] = __shfl(xnorm[mt], 4 * g + i, 64);
            uint32_t hv = 0;
            bool unsure = false;
            const int gg = (lane >> 2) & 3;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool valid = 16 * mt + 4 * g + i < e.nr;
                    const float y = acc[mt][i];
                    const bool sure = fabsf(y) > band(xnr[mt][i], wnorm);
                    unsure |= valid && !sure;
                    const uint64_t bits = __ballot(valid && sure && y > 0.f);
                    // lane L holds the bits of row L: L = 16 mt + 4 gg + i
                    if ((lane >> 4) == mt && (lane & 3) == i) hv = (uint32_t)((bits >> (16 * gg)) & 0xFFFFu);
                }
            if (__ballot(unsure) != 0) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool valid = 16 * mt + 4 * g + i < e.nr;
                        uint64_t um = __ballot(valid && !(fabsf(acc[mt][i]) > band(xnr[mt][i], wnorm)));
                        while (um) {
                            const int lb = __builtin_ctzll(um);
                            um &= um - 1;
                            const int Rf = 16 * mt + 4 * (lb >> 4) + i;
                            const int cb = lb & 15;
                            if (exact_bit(sm, xb, Rf, 16 * wv + cb) && lane == Rf) hv |= 1u << cb;
                        }
                    }
            }
            sm.half[lane][wv] = (uint16_t)hv;
        }
        __syncthreads();  // every wave is done with xb and has its bits in LDS
        if (e.nr > 0 && wv == 4 && lane < e.nr) {
            // wave 4: whole code words of row lane (and, for appends of new
            // rows, the K / V rows into the cache)
            const int64_t r = e.r0 + lane;
            const uvec4 wd = *reinterpret_cast<const uvec4 *>(&sm.half[lane][0]);
            uvec4 *dst = reinterpret_cast<uvec4 *>(
                a.mode == 0 ? a.codes_out + (r * a.n_heads + h) * kWords
                            : a.codes + (((int64_t)e.s * a.Hkv + h) * a.max_ctx + e.l0 + r) * kWords);
            *dst = wd;
        }
        if (e.nr > 0 && a.mode == 1 && a.k_new && wv >= 4) {
            // rows of this tile into the cache: thread (wv - 4, lane) copies
            // 16-byte pieces; K from the sources (still cached), V from v_new
            for (int i = (wv - 4) * 64 + lane; i < e.nr * 16; i += 256) {
                const int rr = i >> 4, p = i & 15;
                const int64_t r = e.r0 + rr;
                const int64_t crow = (((int64_t)e.s * a.Hkv + h) * a.max_ctx + e.l0 + r) * kHeadDim;
                const int64_t nrow = (((int64_t)e.s * a.t_max + r) * a.Hkv + h) * kHeadDim;
                *reinterpret_cast<uvec4 *>(a.k_cache + crow + 8 * p) =
                    *reinterpret_cast<const uvec4 *>(a.k_new + nrow + 8 * p);
                *reinterpret_cast<uvec4 *>(a.v_cache + crow + 8 * p) =
                    *reinterpret_cast<const uvec4 *>(a.v_new + nrow + 8 * p);
            }
        }
        // the next tile of this buffer on its way (buffer b is free: the barrier above)
        if (wv < 4) tile_issue(a, h, tile_of(a, sm, blockIdx.x + (k + kEBuf) * gridDim.x, n_tiles), xb);
    }
    if (wv < 4) wait_vm(0);  // no load of ours lands after the kernel

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
    static_assert(sizeof(ESmem) <= 160 * 1024, "one workgroup per CU");
    // one workgroup per CU in total, at most one per tile
    int dev = 0, n_cu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
        n_cu = 256;
    int64_t per_head = (n_cu + heads - 1) / heads;
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
