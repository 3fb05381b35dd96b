// Code lengths other than 128 bits (r = 32, 64 or 256): the hash-length
// ablation of the HATA review ("Free parameters": rbit = 128 was chosen by
// ablation, accuracy rising from 32 to 128 bits and then flat).  The
// method is the same at every r (h(x) = sign(x W_H) with W_H of 128 x r,
// rbit/32 words per cached key, summed Hamming scores 0 .. G r, top-k,
// exact attention over the selected rows); the fused 128-bit decode kernel
// is specialised to four-word codes, so these lengths take a multi-launch
// path:
//   k_encode_bits<R>   codes of flat rows, of appended cache rows, or of the
//                      query heads.  Thread (row slot s, bit j) keeps column
//                      j of W_H in registers; rows are staged 64 at a time in
//                      LDS.  An fp32 fused multiply-add chain over d gives y'
//                      with |y' - y| <= gamma_128 sum_d |x_d w_dj| + 2^-119
//                      against the sequential double sum y, so the sign of
//                      y' is taken when |y'| > 2^-16 ||x|| ||w_j|| + 2^-100
//                      (and ||x|| ||w_j|| < 2^120, so no partial sum
//                      overflows); every other bit is the sequential double
//                      sum itself.  Bits are packed with wave ballots.
//   k_scan_bits<R>     per (unit, span of 8192 keys): summed Hamming scores
//                      (u16) and the span's score histogram.
//   k_compact_bits     per (unit, span): the cut T (first score whose
//                      cumulative count over the unit reaches k_eff, found
//                      from the spans' cumulative histograms), this span's
//                      offset in the selection and how many of its score-T
//                      keys it takes (ties go to the lowest indices, i.e. to
//                      the earlier spans first), then its selected indices in
//                      index order.
//   k_attend_bits      per (unit, chunk of 256 selected keys): softmax state
//                      (m, l, o) of each query head of the group.
//   k_merge_bits       per unit: the chunks merged in order, bf16 output.
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
    int mode;  // 0: flat rows, 1: cache append, 2: query heads, 3: 1 and 2 in one launch
    const uint16_t *x;
    int64_t row_stride, head_stride, n_rows;
    uint32_t *codes;
    uint32_t *qcodes;  // mode 3: where the query codes go
    int n_heads;
    const float *w;
    uint16_t *k_cache, *v_cache;
    int32_t *seq_len, *ctrl;
    const int32_t *n_new;  // null: one token for every entry (decode step)
    const uint16_t *k_new, *v_new;
    int B, Hkv, G, t_max;
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
    // mode 3: grid rows [0, B Hkv) append, the next Hkv rows encode the queries
    const int role = a.mode != 3 ? a.mode : ((int)blockIdx.y < a.B * a.Hkv ? 1 : 2);
    const int hy = (a.mode == 3 && role == 2) ? (int)blockIdx.y - a.B * a.Hkv : (int)blockIdx.y;
    uint32_t *const codes_out = (a.mode == 3 && role == 2) ? a.qcodes : a.codes;

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
    } else if (role == 1) {
        b_entry = hy / a.Hkv;
        head = hy - b_entry * a.Hkv;
        len = a.seq_len[b_entry];
        n_app = a.n_new ? a.n_new[b_entry] : 1;
        entry_ok = a.n_new ? bits_append_ok(len, n_app, a.t_max, a.max_ctx)
                           : (len >= 0 && len + 1 <= a.max_ctx);
        n_rows = entry_ok ? n_app : 0;
    } else {
        head = hy;
        n_rows = (int64_t)a.B * a.G;
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
                } else if (role == 1) {
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
                } else {
                    const int bb = (int)(row / a.G), g = (int)(row - (int64_t)bb * a.G);
                    src = a.x + ((int64_t)bb * a.Hkv * a.G + (int64_t)head * a.G + g) * kHeadDim;
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
                if (role == 0) {
                    out = codes_out + (row * a.n_heads + head) * W;
                } else if (role == 1) {
                    out = codes_out + ((int64_t)hy * a.max_ctx + len + row) * W;
                } else {
                    const int bb = (int)(row / a.G), g = (int)(row - (int64_t)bb * a.G);
                    out = codes_out + ((int64_t)bb * a.Hkv * a.G + (int64_t)head * a.G + g) * W;
                }
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
    if (a.mode != 1 && a.mode != 3) return;
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
            const int nn = a.n_new ? a.n_new[bb] : 1;
            const bool ok = a.n_new ? bits_append_ok(l, nn, a.t_max, a.max_ctx)
                                    : (l >= 0 && l + 1 <= a.max_ctx);
            if (ok) {
                a.seq_len[bb] = (int32_t)(l + nn);
            } else {
                const int flag = (a.n_new && (nn < 0 || nn > a.t_max)) ? HATA_DEV_BAD_NEW
                                                                        : HATA_DEV_APPEND_OVERFLOW;
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

// ---------------------------------------------------------------- decode

struct BitsDecArgs {
    const uint32_t *codes;
    const uint16_t *k, *v;
    const int32_t *seq_len;
    int32_t *ctrl;
    const uint16_t *q;
    const int32_t *topk;
    uint16_t *out;
    const uint32_t *qcodes;
    uint16_t *scores;   // [unit][max_ctx]
    int32_t *span_hist; // [unit][n_span][NBpad]
    int32_t *info;      // [unit][4]: T, k_eff
    int32_t *sel;       // [unit][k_max]
    float *part;        // [unit][n_chunk][G][2 + 128]
    int B, Hq, Hkv, G, NB, NBpad, n_span, n_chunk, k_max;
    int64_t max_ctx;
};

__device__ __forceinline__ int64_t bits_len(const BitsDecArgs &a, int b) {
    int64_t len = a.seq_len[b];
    return len < 0 ? 0 : (len > a.max_ctx ? a.max_ctx : len);
}

__device__ __forceinline__ int bits_keff(const BitsDecArgs &a, int b, int64_t len) {
    int64_t k = a.topk[b];
    k = k < 0 ? 0 : (k > a.k_max ? a.k_max : k);
    return (int)(k < len ? k : len);
}

template <int R>
__global__ void __launch_bounds__(kBThreads) k_scan_bits(BitsDecArgs a) {
    constexpr int W = R / 32;
    __shared__ uint32_t qs[8 * W];
    __shared__ int hist[8 * 256 + 1];
    const int span = blockIdx.x, unit = blockIdx.y, b = unit / a.Hkv, kv = unit - b * a.Hkv;
    const int t = threadIdx.x;
    const int64_t len = bits_len(a, b);
    if (t < a.G * W) qs[t] = a.qcodes[((int64_t)b * a.Hq + (int64_t)kv * a.G) * W + t];
    for (int i = t; i < a.NB; i += kBThreads) hist[i] = 0;
    __syncthreads();
    const int64_t i0 = (int64_t)span * kBSpan;
    const uint32_t *cb = a.codes + (int64_t)unit * a.max_ctx * W;
    uint16_t *sb = a.scores + (int64_t)unit * a.max_ctx;
    for (int k = 0; k < kBSpan / kBThreads; k += 4) {
        uint32_t kw[4][W];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + (int64_t)(k + u) * kBThreads + t;
            if (i < len) {
#pragma unroll
                for (int w = 0; w < W; ++w) kw[u][w] = cb[i * W + w];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + (int64_t)(k + u) * kBThreads + t;
            if (i < len) {
                int s = 0;
                for (int h = 0; h < a.G; ++h) {
#pragma unroll
                    for (int w = 0; w < W; ++w) s += __popc(qs[h * W + w] ^ kw[u][w]);
                }
                sb[i] = (uint16_t)s;
                atomicAdd(&hist[s], 1);
            }
        }
    }
    __syncthreads();
    // The span's cumulative histogram (keys scoring <= bin): each thread
    // sums a run of consecutive bins, one block scan places the runs.
    __shared__ int tmp[4];
    const int per = (a.NB + kBThreads - 1) / kBThreads;
    const int lo = t * per, hi = lo + per < a.NB ? lo + per : a.NB;
    int c = 0;
    for (int bin = lo; bin < hi; ++bin) c += hist[bin];
    int tot;
    int cum = block_excl_scan_256(c, tmp, &tot);
    int32_t *hrow = a.span_hist + ((int64_t)unit * a.n_span + span) * a.NBpad;
    for (int bin = lo; bin < hi; ++bin) {
        cum += hist[bin];
        hrow[bin] = cum;
    }
}

__global__ void __launch_bounds__(kBThreads) k_compact_bits(BitsDecArgs a) {
    __shared__ int tmp[8];
    __shared__ int c1[2 * kBThreads + 8];  // cumulative count at the end of each group of 8 bins
    __shared__ int c2[8];
    __shared__ int s_g, s_T, s_below, s_off, s_take;
    const int span = blockIdx.x, unit = blockIdx.y, b = unit / a.Hkv;
    const int t = threadIdx.x;
    const int64_t len = bits_len(a, b);
    const int ke = bits_keff(a, b, len);
    const int64_t i0 = (int64_t)span * kBSpan;
    int32_t *sel = a.sel + (int64_t)unit * a.k_max;
    if (span == 0) {
        if (t == 0) {
            const int64_t raw = a.seq_len[b];
            if (raw < 0 || raw > a.max_ctx) atomicOr(&a.ctrl[kCtrlStatus], HATA_DEV_BAD_LENGTH);
            if (a.topk[b] > a.k_max) atomicOr(&a.ctrl[kCtrlStatus], HATA_DEV_TOPK_CLAMPED);
            a.info[unit * 4 + 1] = ke;
        }
        for (int i = ke + t; i < a.k_max; i += kBThreads) sel[i] = -1;
    }
    if (ke == 0 || i0 >= len) return;
    // The cut T: the first bin where the unit's cumulative count (the sum of
    // its spans' cumulative histograms) reaches k_eff -- first among the ends
    // of groups of 8 bins, then within the group found.
    const int n_used = (int)((len + kBSpan - 1) / kBSpan);
    const int32_t *hb = a.span_hist + (int64_t)unit * a.n_span * a.NBpad;
    const int ngr = (a.NB + 7) / 8;
    for (int gi = t; gi < ngr; gi += kBThreads) {
        const int bin = 8 * gi + 7 < a.NB ? 8 * gi + 7 : a.NB - 1;
        int sum = 0;
#pragma unroll 8
        for (int sp = 0; sp < n_used; ++sp) sum += hb[(int64_t)sp * a.NBpad + bin];
        c1[gi] = sum;
    }
    __syncthreads();
    for (int gi = t; gi < ngr; gi += kBThreads)
        if (c1[gi] >= ke && (gi == 0 || c1[gi - 1] < ke)) s_g = gi;
    __syncthreads();
    const int g = s_g;
    if (t < 8) {
        const int bin = 8 * g + t;
        int sum = (int)len;  // bins past the last: the total
        if (bin < a.NB) {
            sum = 0;
#pragma unroll 8
            for (int sp = 0; sp < n_used; ++sp) sum += hb[(int64_t)sp * a.NBpad + bin];
        }
        c2[t] = sum;
    }
    __syncthreads();
    if (t < 8) {
        const int bin = 8 * g + t;
        const int prev = t == 0 ? (g == 0 ? 0 : c1[g - 1]) : c2[t - 1];
        if (bin < a.NB && c2[t] >= ke && prev < ke) {
            s_T = bin;
            s_below = prev;
        }
    }
    __syncthreads();
    const int T = s_T, need = ke - s_below;
    // This span's offset in the selection and its share of the score-T keys
    // (the earlier spans first).
    int carry_ties = 0, carry_off = 0;
    for (int s0 = 0; s0 <= span; s0 += kBThreads) {
        const int sp = s0 + t;
        int below = 0, ties = 0;
        if (sp <= span) {
            const int32_t *hr = hb + (int64_t)sp * a.NBpad;
            below = T > 0 ? hr[T - 1] : 0;
            ties = hr[T] - below;
        }
        int tt;
        const int ties_before = carry_ties + block_excl_scan_256(ties, tmp, &tt);
        int take_sp = need - ties_before;
        take_sp = take_sp < 0 ? 0 : (take_sp > ties ? ties : take_sp);
        int to;
        const int off_sp = carry_off + block_excl_scan_256(below + take_sp, tmp, &to);
        if (sp == span) {
            s_off = off_sp;
            s_take = take_sp;
        }
        carry_ties += tt;
        carry_off += to;
    }
    __syncthreads();
    const int off = s_off, take = s_take;
    if (span == 0 && t == 0) a.info[unit * 4 + 0] = T;
    const uint16_t *sb = a.scores + (int64_t)unit * a.max_ctx;
    int ties_seen = 0, written = 0;
    for (int c0 = 0; c0 < kBSpan; c0 += 8 * kBThreads) {
        int below_f = 0, tie_f = 0, nt = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t i = i0 + c0 + 8 * t + e;
            if (i < len) {
                const int s = sb[i];
                below_f |= (s < T) << e;
                tie_f |= (s == T) << e;
                nt += (s == T);
            }
        }
        int tt;
        int rank = ties_seen + block_excl_scan_256(nt, tmp, &tt);
        int sel_f = below_f, ns = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((tie_f >> e) & 1) {
                if (rank < take) sel_f |= 1 << e;
                ++rank;
            }
        }
        ns = __popc(sel_f);
        int ts;
        int pos = off + written + block_excl_scan_256(ns, tmp, &ts);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((sel_f >> e) & 1) {
                if (pos < ke) sel[pos] = (int32_t)(i0 + c0 + 8 * t + e);
                ++pos;
            }
        }
        ties_seen += tt;
        written += ts;
    }
}

// Sums over the 16 lanes of a row; every lane ends with the same bits.
__device__ __forceinline__ float bsum16(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// One chunk of up to 256 selected keys: wave w takes keys 64 w .. 64 w + 63,
// four at a time (a row of 16 lanes per key, 8 dims per lane), with an
// online softmax (base 2) per row and head; rows, then waves, are combined.
template <int G>
__global__ void __launch_bounds__(kBThreads) k_attend_bits(BitsDecArgs a) {
    __shared__ float wm[4][G], wl[4][G];
    __shared__ float wo[4][G][kHeadDim];
    const int chunk = blockIdx.x, unit = blockIdx.y, b = unit / a.Hkv, kv = unit - b * a.Hkv;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, sub = lane & 15, kk = lane >> 4;
    const int ke = a.info[unit * 4 + 1];
    const int c0 = chunk * kBChunk;
    if (c0 >= ke) return;
    const int64_t len = bits_len(a, b);
    const float qscale = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
    float qf[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const uvec4 r = *reinterpret_cast<const uvec4 *>(
            a.q + ((int64_t)b * a.Hq + (int64_t)kv * G + h) * kHeadDim + 8 * sub);
        unpack8b(r, qf[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[h][e] *= qscale;
    }
    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }
    const int32_t *sel = a.sel + (int64_t)unit * a.k_max;
    const uint16_t *kb = a.k + (int64_t)unit * a.max_ctx * kHeadDim + 8 * sub;
    const uint16_t *vb = a.v + (int64_t)unit * a.max_ctx * kHeadDim + 8 * sub;
    // This lane's 16 keys first (one round trip), then the K/V pieces four
    // iterations ahead of their use.
    int64_t keyv[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int p = c0 + wv * 64 + it * 4 + kk;
        const int64_t key = p < ke ? sel[p] : -1;
        keyv[it] = (key >= 0 && key < len) ? key : -1;  // uniform within the row
    }
    uvec4 kq[4], vq[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        kq[it] = vq[it] = uvec4{0u, 0u, 0u, 0u};
        if (keyv[it] >= 0) {
            kq[it] = *reinterpret_cast<const uvec4 *>(kb + keyv[it] * kHeadDim);
            vq[it] = *reinterpret_cast<const uvec4 *>(vb + keyv[it] * kHeadDim);
        }
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int sl = it & 3;
        const bool valid = keyv[it] >= 0;
        const uvec4 kr = kq[sl], vr = vq[sl];
        if (it + 4 < 16) {
            kq[sl] = vq[sl] = uvec4{0u, 0u, 0u, 0u};
            if (keyv[it + 4] >= 0) {
                kq[sl] = *reinterpret_cast<const uvec4 *>(kb + keyv[it + 4] * kHeadDim);
                vq[sl] = *reinterpret_cast<const uvec4 *>(vb + keyv[it + 4] * kHeadDim);
            }
        }
        float kf[8], vf[8];
        unpack8b(kr, kf);
        unpack8b(vr, vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float z = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) z = fmaf(qf[h][e], kf[e], z);
            z = bsum16(z);
            if (valid) {
                const float mn = fmaxf(m[h], z);
                const float sc = exp2f(m[h] - mn);  // 0 while m is -inf
                const float pz = exp2f(z - mn);
                l[h] = l[h] * sc + pz;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[h][e] = fmaf(pz, vf[e], o[h][e] * sc);
                m[h] = mn;
            }
        }
    }
    // Combine the four rows of the wave.
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float M = fmaxf(m[h], __shfl_xor(m[h], 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        const float sc = (m[h] == -INFINITY) ? 0.f : exp2f(m[h] - M);
        float lv = l[h] * sc;
        lv += __shfl_xor(lv, 16);
        lv += __shfl_xor(lv, 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float ov = o[h][e] * sc;
            ov += __shfl_xor(ov, 16);
            ov += __shfl_xor(ov, 32);
            o[h][e] = ov;
        }
        if (lane == 0) {
            wm[wv][h] = M;
            wl[wv][h] = lv;
        }
        if (lane < 16) {
#pragma unroll
            for (int e = 0; e < 8; ++e) wo[wv][h][8 * sub + e] = o[h][e];
        }
    }
    __syncthreads();
    // Combine the four waves: thread (h, d) pairs.
    float *pb = a.part + ((int64_t)unit * a.n_chunk + chunk) * G * (2 + kHeadDim);
    for (int idx = t; idx < G * kHeadDim; idx += kBThreads) {
        const int h = idx / kHeadDim, d = idx - h * kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][h]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float sc = (wm[w][h] == -INFINITY) ? 0.f : exp2f(wm[w][h] - M);
            L = fmaf(wl[w][h], sc, L);
            O = fmaf(wo[w][h][d], sc, O);
        }
        float *ph = pb + h * (2 + kHeadDim);
        if (d == 0) {
            ph[0] = M;
            ph[1] = L;
        }
        ph[2 + d] = O;
    }
}

__global__ void __launch_bounds__(kBThreads) k_merge_bits(BitsDecArgs a) {
    const int unit = blockIdx.x, b = unit / a.Hkv, kv = unit - b * a.Hkv;
    const int t = threadIdx.x;
    const int ke = a.info[unit * 4 + 1];
    const int nc = (ke + kBChunk - 1) / kBChunk;
    for (int idx = t; idx < a.G * kHeadDim; idx += kBThreads) {
        const int h = idx / kHeadDim, d = idx - h * kHeadDim;
        float r = 0.f;
        if (nc > 0) {
            float M = -INFINITY;
#pragma unroll 8
            for (int c = 0; c < nc; ++c) {
                const float *ph = a.part + (((int64_t)unit * a.n_chunk + c) * a.G + h) * (2 + kHeadDim);
                M = fmaxf(M, ph[0]);
            }
            float L = 0.f, O = 0.f;
#pragma unroll 8
            for (int c = 0; c < nc; ++c) {
                const float *ph = a.part + (((int64_t)unit * a.n_chunk + c) * a.G + h) * (2 + kHeadDim);
                const float sc = exp2f(ph[0] - M);
                L = fmaf(ph[1], sc, L);
                O = fmaf(ph[2 + d], sc, O);
            }
            r = O / L;
        }
        a.out[((int64_t)b * a.Hq + (int64_t)kv * a.G + h) * kHeadDim + d] = f32_to_bf16(r);
    }
}

bool make_bits_plan(int B, int Hq, int Hkv, int64_t max_ctx, int n_bits, int k_max,
                    BitsPlan *p) {
    if (B <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || max_ctx < 0 || k_max < 0) return false;
    if (n_bits != 32 && n_bits != 64 && n_bits != 128 && n_bits != 256) return false;
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return false;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    p->B = B;
    p->Hq = Hq;
    p->Hkv = Hkv;
    p->G = G;
    p->R = n_bits;
    p->NB = G * n_bits + 1;
    p->NBpad = (p->NB + 63) & ~63;
    p->max_ctx = max_ctx;
    p->k_max = k_max;
    p->n_span = (int)((max_ctx + kBSpan - 1) / kBSpan);
    if (p->n_span < 1) p->n_span = 1;
    p->n_chunk = (k_max + kBChunk - 1) / kBChunk;
    if (p->n_chunk < 1) p->n_chunk = 1;
    const size_t units = (size_t)B * Hkv;
    size_t off = 0;
    p->off_qcodes = off;
    off = up(off + (size_t)B * Hq * (n_bits / 32) * 4);
    p->off_scores = off;
    off = up(off + units * (size_t)max_ctx * 2);
    p->off_span_hist = off;
    off = up(off + units * p->n_span * (size_t)p->NBpad * 4);
    p->off_info = off;
    off = up(off + units * 4 * 4);
    p->off_sel = off;
    off = up(off + units * (size_t)k_max * 4);
    p->off_part = off;
    off = up(off + units * p->n_chunk * (size_t)G * (2 + kHeadDim) * 4);
    p->total = off;
    return true;
}

template <int R>
static hipError_t launch_scan_r(const BitsDecArgs &a, dim3 grid, hipStream_t s) {
    k_scan_bits<R><<<grid, kBThreads, 0, s>>>(a);
    return hipGetLastError();
}

template <int G>
static hipError_t launch_attend_g(const BitsDecArgs &a, dim3 grid, hipStream_t s) {
    k_attend_bits<G><<<grid, kBThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode_bits(const BitsPlan &p, uint16_t *k_cache, uint16_t *v_cache,
                              uint32_t *codes, int32_t *seq_len, int32_t *ctrl,
                              const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                              const float *w, const int32_t *topk, uint16_t *out, void *ws,
                              int32_t *sel_idx_out, uint16_t *scores_out, hipStream_t s) {
    char *wsb = static_cast<char *>(ws);
    hipError_t e;
    const int units = p.B * p.Hkv;
    uint32_t *qcodes = reinterpret_cast<uint32_t *>(wsb + p.off_qcodes);
    {
        // the step's append (one row per sequence) and the query codes
        BitsEncArgs ea = {};
        ea.mode = k_new ? 3 : 2;
        ea.x = q;
        ea.codes = k_new ? codes : qcodes;
        ea.qcodes = qcodes;
        ea.w = w;
        ea.k_cache = k_cache;
        ea.v_cache = v_cache;
        ea.seq_len = seq_len;
        ea.ctrl = ctrl;
        ea.n_new = nullptr;
        ea.k_new = k_new;
        ea.v_new = v_new;
        ea.B = p.B;
        ea.Hkv = p.Hkv;
        ea.G = p.G;
        ea.t_max = 1;
        ea.max_ctx = p.max_ctx;
        const int rows_y = k_new ? p.B * p.Hkv + p.Hkv : p.Hkv;
        e = dispatch_enc_bits(ea, p.R, dim3(enc_grid_x((int64_t)p.B * p.G, rows_y), rows_y), s);
        if (e != hipSuccess) return e;
    }
    BitsDecArgs a;
    a.codes = codes;
    a.k = k_cache;
    a.v = v_cache;
    a.seq_len = seq_len;
    a.ctrl = ctrl;
    a.q = q;
    a.topk = topk;
    a.out = out;
    a.qcodes = qcodes;
    a.scores = scores_out ? scores_out : reinterpret_cast<uint16_t *>(wsb + p.off_scores);
    a.span_hist = reinterpret_cast<int32_t *>(wsb + p.off_span_hist);
    a.info = reinterpret_cast<int32_t *>(wsb + p.off_info);
    a.sel = sel_idx_out ? sel_idx_out : reinterpret_cast<int32_t *>(wsb + p.off_sel);
    a.part = reinterpret_cast<float *>(wsb + p.off_part);
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.G = p.G;
    a.NB = p.NB;
    a.NBpad = p.NBpad;
    a.n_span = p.n_span;
    a.n_chunk = p.n_chunk;
    a.k_max = p.k_max;
    a.max_ctx = p.max_ctx;
    const dim3 sg(p.n_span, units);
    switch (p.R) {
        case 32: e = launch_scan_r<32>(a, sg, s); break;
        case 64: e = launch_scan_r<64>(a, sg, s); break;
        case 128: e = launch_scan_r<128>(a, sg, s); break;
        default: e = launch_scan_r<256>(a, sg, s); break;
    }
    if (e != hipSuccess) return e;
    k_compact_bits<<<sg, kBThreads, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 ag(p.n_chunk, units);
    switch (p.G) {
        case 1: e = launch_attend_g<1>(a, ag, s); break;
        case 2: e = launch_attend_g<2>(a, ag, s); break;
        case 4: e = launch_attend_g<4>(a, ag, s); break;
        default: e = launch_attend_g<8>(a, ag, s); break;
    }
    if (e != hipSuccess) return e;
    k_merge_bits<<<units, kBThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hata
