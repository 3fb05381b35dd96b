// Encoders for code lengths other than 128 bits (r = 32, 64 or 256): the
// hash-length ablation of the HATA review ("Free parameters": rbit = 128 was
// chosen by ablation, accuracy rising from 32 to 128 bits and then flat).
// The method is the same at every r (h(x) = sign(x W_H) with W_H of 128 x r,
// rbit/32 words per cached key); the decode step is the same kernel at
// every length (decode_fused.h).  Here, for appends and flat rows too few
// for the matrix-core encoder:
//   k_encode_bits<R>   codes of flat rows or of appended cache rows.  Thread
//                      (row slot s, bit j) keeps column j of W_H in
//                      registers; rows are staged 64 at a time in LDS.  An
//                      fp32 fused multiply-add chain over d gives y' with
//                      |y' - y| <= gamma_128 sum_d |x_d w_dj| + 2^-119
//                      against the sequential double sum y, so the sign of
//                      y' is taken when |y'| > 2^-16 ||x|| ||w_j|| + 2^-100
//                      (and ||x|| ||w_j|| < 2^120, so no partial sum
//                      overflows); every other bit is the sequential double
//                      sum itself.  Bits are packed with wave ballots.
#include "device_util.h"
#include "hata_internal.h"
#include "bits_plan.h"
#include "../../include/hata.h"

namespace hata {

typedef uint32_t uvec4 __attribute__((ext_vector_type(4)));
typedef uint32_t uvec2 __attribute__((ext_vector_type(2)));

constexpr int kBThreads = 256;
constexpr int kBTile = 64;  // rows per encoder tile

__device__ __forceinline__ void unpack8b(const uvec4 &r, float (&f)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(r[j] << 16);
        f[2 * j + 1] = __uint_as_float(r[j] & 0xFFFF0000u);
    }
}

// ---------------------------------------------------------------- encoder

// A double sum over the 64 lanes of a wave, in every lane: within each row of
// 16 lanes by DPP (xor 1, xor 2, half-row mirror, row mirror), then the four
// row sums added in order: with the caller's pair sum, eight rounding levels.
template <int CTRL>
__device__ __forceinline__ double bdpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double blane_f64(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double bsum64(double v) {
    v += bdpp_f64<0xB1>(v);
    v += bdpp_f64<0x4E>(v);
    v += bdpp_f64<0x141>(v);
    v += bdpp_f64<0x140>(v);
    return ((blane_f64(v, 0) + blane_f64(v, 16)) + blane_f64(v, 32)) + blane_f64(v, 48);
}

// The exact bit of one (row, column), by the whole wave: lane l forms the
// exact double products of dims 2 l and 2 l + 1; their sum s is within
// gamma_8 sum|p| of the real sum, the sequential double sum that defines the
// bit within gamma_127 sum|p|, so the sign of s is the bit when
// |s| > 2^-44 sum|p|; otherwise lane 0 runs the sequential loop itself.
__device__ __attribute__((noinline)) bool wave_exact_bit(const float *xrow, const float *wcol, int R) {
    const int lane = threadIdx.x & 63;
    const double p0 = (double)xrow[2 * lane] * (double)wcol[(int64_t)(2 * lane) * R];
    const double p1 = (double)xrow[2 * lane + 1] * (double)wcol[(int64_t)(2 * lane + 1) * R];
    const double sv = bsum64(p0 + p1);
    const double A = bsum64(fabs(p0) + fabs(p1));
    bool bit = sv > 0.0;
    if (!(fabs(sv) > 0x1p-44 * A)) {
        int b = 0;
        if (lane == 0) {
            double y = 0.0;
            for (int d = 0; d < kHeadDim; ++d) y = fma((double)xrow[d], (double)wcol[(int64_t)d * R], y);
            b = y > 0.0;
        }
        bit = __builtin_amdgcn_readfirstlane(b) != 0;
    }
    return bit;
}

struct BitsEncArgs {
    int mode;  // 0: flat rows, 1: cache append
    const uint16_t *x;
    int64_t row_stride, head_stride, n_rows;
    uint32_t *codes;
    int n_heads;
    const float *w;
    uint16_t *k_cache, *v_cache;
    int32_t *seq_len, *ctrl;
    const int32_t *n_new;
    const uint16_t *k_new, *v_new;
    int B, Hkv, t_max;
    int64_t max_ctx;
};

__device__ __forceinline__ bool bits_append_ok(int64_t len, int n, int t_max, int64_t max_ctx) {
    return n >= 0 && n <= t_max && len >= 0 && len + n <= max_ctx;
}

template <int R>
__global__ void __launch_bounds__(kBThreads) k_encode_bits(BitsEncArgs a) {
    constexpr int W = R / 32;
    constexpr int P = kBThreads / R;  // rows computed at once
    __shared__ float xs[kBTile][kHeadDim];
    __shared__ double xn[kBTile];
    __shared__ int s_last;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int j = t % R, slot = t / R;
    const int role = a.mode;
    const int hy = (int)blockIdx.y;
    uint32_t *const codes_out = a.codes;

    // The rows this workgroup's grid column encodes, and their head.
    int head;
    int64_t n_rows;
    int64_t len = 0;
    int n_app = 0;
    bool entry_ok = true;
    int b_entry = 0;
    if (role == 0) {
        head = hy;
        n_rows = a.n_rows;
    } else {
        b_entry = hy / a.Hkv;
        head = hy - b_entry * a.Hkv;
        len = a.seq_len[b_entry];
        n_app = a.n_new[b_entry];
        entry_ok = bits_append_ok(len, n_app, a.t_max, a.max_ctx);
        n_rows = entry_ok ? n_app : 0;
    }

    // Column j of W_H (fp32) and its norm.
    float wv_[kHeadDim];
    const float *wc = a.w + (int64_t)head * kHeadDim * R + j;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) wv_[d] = wc[(int64_t)d * R];
    double nw2 = 0.0;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) nw2 = fma((double)wv_[d], (double)wv_[d], nw2);
    const double nw = sqrt(nw2);

    for (int64_t r0 = (int64_t)blockIdx.x * kBTile; r0 < n_rows;
         r0 += (int64_t)gridDim.x * kBTile) {
        __syncthreads();  // the previous tile's rows are no longer read
        // Stage 64 rows: 16-byte pieces, 4 per thread.
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int piece = t + k * kBThreads, rr = piece >> 4, c = piece & 15;
            const int64_t row = r0 + rr;
            uvec4 raw = {0u, 0u, 0u, 0u};
            if (row < n_rows) {
                const uint16_t *src;
                if (role == 0) {
                    src = a.x + row * a.row_stride + (int64_t)head * a.head_stride;
                } else {
                    const int64_t crow =
                        ((int64_t)hy * a.max_ctx + len + row) * kHeadDim;
                    if (a.k_new) {
                        const int64_t nrow = (((int64_t)b_entry * a.t_max + row) * a.Hkv + head) *
                                             kHeadDim;
                        src = a.k_new + nrow;
                        const uvec4 kv_k = *reinterpret_cast<const uvec4 *>(a.k_new + nrow + 8 * c);
                        const uvec4 kv_v = *reinterpret_cast<const uvec4 *>(a.v_new + nrow + 8 * c);
                        *reinterpret_cast<uvec4 *>(a.k_cache + crow + 8 * c) = kv_k;
                        *reinterpret_cast<uvec4 *>(a.v_cache + crow + 8 * c) = kv_v;
                    } else {
                        src = a.k_cache + crow;
                    }
                }
                raw = *reinterpret_cast<const uvec4 *>(src + 8 * c);
            }
            float f[8];
            unpack8b(raw, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[rr][8 * c + e] = f[e];
        }
        __syncthreads();
        // Row norms in double: four threads per row, 32 dims each.
        {
            const int rr = t >> 2, q4 = t & 3;
            double s = 0.0;
            for (int d = 0; d < 32; ++d) {
                const double v = xs[rr][32 * q4 + d];
                s = fma(v, v, s);
            }
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            if (q4 == 0) xn[rr] = sqrt(s);
        }
        __syncthreads();
        const int rows_here = (int)(n_rows - r0 < kBTile ? n_rows - r0 : kBTile);
        // Four rows per thread at a time (rows rb, rb + P, rb + 2P, rb + 3P):
        // four independent FMA chains share the W_H registers, so the
        // chains' latency overlaps.
        for (int rb = slot; rb < kBTile; rb += 4 * P) {
            float y4[4] = {0.f, 0.f, 0.f, 0.f};
            if (rb < rows_here) {
#pragma unroll
                for (int d = 0; d < kHeadDim; ++d) {
                    const float wd = wv_[d];
#pragma unroll
                    for (int q = 0; q < 4; ++q) y4[q] = fmaf(xs[rb + q * P][d], wd, y4[q]);
                }
            }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rr = rb + q * P;
            const int64_t row = r0 + rr;
            bool bit = false, unsure = false;
            if (rr < rows_here) {
            const float y = y4[q];
            const double nn = xn[rr] * nw;
            if (nn < 0x1p120 && fabs((double)y) > 0x1p-16 * nn + 0x1p-100) {
                bit = y > 0.f;
            } else {
                unsure = true;
            }
            }
            // the rare bits inside the band, one at a time by the whole wave
            uint64_t um = __ballot(unsure);
            while (um) {
                const int lb = __builtin_ctzll(um);
                um &= um - 1;
                const int rr_l = __builtin_amdgcn_readlane(rr, lb);
                const int j_l = __builtin_amdgcn_readlane(j, lb);
                const bool eb = wave_exact_bit(&xs[rr_l][0],
                                               a.w + (int64_t)head * kHeadDim * R + j_l, R);
                if (lane == lb) bit = eb;
            }
            const uint64_t m = __ballot(bit);
            if (row < n_rows) {
                uint32_t *out;
                if (role == 0) out = codes_out + (row * a.n_heads + head) * W;
                else out = codes_out + ((int64_t)hy * a.max_ctx + len + row) * W;
                if (R >= 64) {
                    // wave = 64 consecutive bits of one row
                    if (lane == 0) {
                        const int w0 = 2 * ((t % R) >> 6);
                        out[w0] = (uint32_t)m;
                        out[w0 + 1] = (uint32_t)(m >> 32);
                    }
                } else {
                    // R = 32: lanes 0-31 and 32-63 hold two rows
                    if (lane == 0 || lane == 32) out[0] = (uint32_t)(m >> lane);
                }
            }
        }
        }
    }
    (void)wv;
    if (a.mode != 1) return;
    // The last workgroup publishes the new lengths (every workgroup has read
    // seq_len by then).
    __syncthreads();
    if (t == 0) {
        __threadfence();
        const unsigned total = gridDim.x * gridDim.y;
        const unsigned prev = atomicAdd((unsigned *)&a.ctrl[kCtrlAppendDone], 1u);
        s_last = (prev == total - 1);
    }
    __syncthreads();
    if (s_last) {
        __threadfence();
        for (int bb = t; bb < a.B; bb += kBThreads) {
            const int64_t l = a.seq_len[bb];
            const int nn = a.n_new[bb];
            const bool ok = bits_append_ok(l, nn, a.t_max, a.max_ctx);
            if (ok) {
                a.seq_len[bb] = (int32_t)(l + nn);
            } else {
                const int flag = (nn < 0 || nn > a.t_max) ? HATA_DEV_BAD_NEW : HATA_DEV_APPEND_OVERFLOW;
                atomicOr(&a.ctrl[kCtrlStatus], flag);
            }
        }
        if (t == 0) a.ctrl[kCtrlAppendDone] = 0;
    }
}

template <int R>
static hipError_t launch_enc_bits(const BitsEncArgs &a, dim3 grid, hipStream_t s) {
    k_encode_bits<R><<<grid, kBThreads, 0, s>>>(a);
    return hipGetLastError();
}

static hipError_t dispatch_enc_bits(const BitsEncArgs &a, int n_bits, dim3 grid, hipStream_t s) {
    switch (n_bits) {
        case 32: return launch_enc_bits<32>(a, grid, s);
        case 64: return launch_enc_bits<64>(a, grid, s);
        case 128: return launch_enc_bits<128>(a, grid, s);
        case 256: return launch_enc_bits<256>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

static unsigned enc_grid_x(int64_t n_rows, int n_units) {
    int64_t tiles = (n_rows + kBTile - 1) / kBTile;
    // enough workgroups to fill the chip a few times over; each walks tiles
    const int64_t cap = (4096 + n_units - 1) / n_units;
    if (tiles > cap) tiles = cap;
    return (unsigned)(tiles < 1 ? 1 : tiles);
}

hipError_t launch_encode_bits(const uint16_t *keys, int64_t n_rows, int n_heads,
                              int64_t row_stride, int64_t head_stride, const float *w,
                              int n_bits, uint32_t *codes, hipStream_t s) {
    BitsEncArgs a = {};
    a.mode = 0;
    a.x = keys;
    a.row_stride = row_stride;
    a.head_stride = head_stride;
    a.n_rows = n_rows;
    a.codes = codes;
    a.n_heads = n_heads;
    a.w = w;
    return dispatch_enc_bits(a, n_bits, dim3(enc_grid_x(n_rows, n_heads), n_heads), s);
}

hipError_t launch_append_bits(uint16_t *k_cache, uint16_t *v_cache, uint32_t *codes,
                              int32_t *seq_len, int32_t *ctrl, int B, int Hkv, int64_t max_ctx,
                              const uint16_t *k_new, const uint16_t *v_new, const int32_t *n_new,
                              int t_max, const float *w, int n_bits, hipStream_t s) {
    BitsEncArgs a = {};
    a.mode = 1;
    a.codes = codes;
    a.w = w;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.seq_len = seq_len;
    a.ctrl = ctrl;
    a.n_new = n_new;
    a.k_new = k_new;
    a.v_new = v_new;
    a.B = B;
    a.Hkv = Hkv;
    a.t_max = t_max;
    a.max_ctx = max_ctx;
    return dispatch_enc_bits(a, n_bits, dim3(enc_grid_x(t_max, B * Hkv), B * Hkv), s);
}

}  // namespace hata
