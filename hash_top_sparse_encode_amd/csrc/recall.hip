// Recall analysis of the Hamming selection: how much of the exact top-k it
// finds, and how large the tied bucket at its cut is.  This is the test the
// referee report of the HATA review asks for ("What would settle it": rank
// the keys by exact q.k and compare that top-k set with the Hamming-selected
// one; major comment 1: exact top-k agreement and the tie distribution).
//
// The exact logit of query head h and key i is z_i = sum_d q_d k_{i,d} as a
// sequential double sum over d = 0..127 (every bf16 x bf16 product is exact
// in double); the exact top-k keeps the k_eff largest z_i, the lower index
// first among equal values.
//
// k_logit_estimates streams every cached key once per (sequence, KV head)
// and forms fp32 estimates z'_i for the G query heads of the group (lane
// (g, c) of a row of 16 lanes multiplies dims 8c .. 8c + 7 in a chain of
// fused multiply-adds, then the row sums; the products are exact in fp32),
// plus the largest ||k_i||^2 of its keys in double.  Along every path there
// are at most 7 + 4 roundings, so with IEEE denormals and finite inputs
//   |z'_i - z_i| <= (gamma_11(fp32) + gamma_127(fp64)) sum_d |q_d k_{i,d}|
//                   + 2^-119
//                <= 2^-18 ||q|| max_j ||k_j|| + 2^-100 =: E
// (Cauchy-Schwarz; 2^-18 leaves a factor 5 over gamma_11).
//
// k_recall_select, one workgroup per (sequence, query head): a three-pass
// radix select finds t, the k_eff-th largest estimate.  Fewer than k_eff
// estimates exceed t, so a key with z' > t + 2E has at most k_eff - 2
// exact logits above its own: it is in.  At least k_eff estimates reach t,
// so a key with z' < t - 2E has k_eff exact logits above it: it is out.
// The keys in between (none to a few for Gaussian data) get z_i in the
// exact sequential order and are ranked by (z desc, index asc) for the
// places left.  Where ||q|| ||k|| could overflow fp32 every key is ranked
// exactly (correct, slow).  The workgroup then writes the exact set in
// ascending order (optional), counts how many of the Hamming selection's
// keys it holds, and for the first head of each group histograms the
// group's Hamming scores: the cut T (the k_eff-th smallest score), the keys
// below it and the keys tied at it.
#include "device_util.h"
#include "hata_internal.h"
#include "recall_plan.h"
#include "../../include/hata.h"

namespace hata {

typedef uint32_t uvec4 __attribute__((ext_vector_type(4)));

constexpr int kRecKeysPerBlock = 1024;  // keys per estimate workgroup (256 threads)
constexpr int kRecThreads = 1024;       // threads of a selection workgroup

struct RecallArgs {
    const uint16_t *k;
    const uint16_t *q;
    const int32_t *seq_len;
    const int32_t *topk;
    const int32_t *sel_idx;
    const uint16_t *scores;
    int32_t *overlap, *tie, *exact_idx;
    float *zq;         // [B][Hq][zstride] estimates
    double *norm2;     // [B * Hkv][n_kblk] largest ||k||^2 per estimate workgroup
    int32_t *band_idx; // [B][Hq][max_ctx] keys ranked exactly
    double *band_z;    // [B][Hq][max_ctx] their exact logits
    uint8_t *member;   // [B][Hq][max_ctx] exact top-k flag of those keys
    int B, Hq, Hkv, G, k_max, n_kblk, nbits;
    int64_t max_ctx, zstride;
};

__device__ __forceinline__ int64_t rec_len(const RecallArgs &a, int b) {
    int64_t len = a.seq_len[b];
    return len < 0 ? 0 : (len > a.max_ctx ? a.max_ctx : len);
}

__device__ __forceinline__ void unpack8(const uvec4 &r, float (&f)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(r[j] << 16);
        f[2 * j + 1] = __uint_as_float(r[j] & 0xFFFF0000u);
    }
}

// Sums over the 16 lanes of a row (xor-1 and xor-2 quad permutes, then the
// half-row and row mirrors).  Each step adds two values in either order, so
// every lane of the row ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const int64_t u = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(u & 0xFFFFFFFF), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ float rsum16(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return v;
}
__device__ __forceinline__ double rsum16_d(double v) {
    v += dpp_d<0xB1>(v);
    v += dpp_d<0x4E>(v);
    v += dpp_d<0x141>(v);
    v += dpp_d<0x140>(v);
    return v;
}

template <int G>
__global__ void __launch_bounds__(256) k_logit_estimates(RecallArgs a) {
    const int unit = blockIdx.y;
    const int b = unit / a.Hkv, kv = unit - b * a.Hkv;
    const int64_t len = rec_len(a, b);
    const int64_t blk0 = (int64_t)blockIdx.x * kRecKeysPerBlock;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, sub = lane & 15, kk = lane >> 4;
    __shared__ double wmax[4];
    double nmax = 0.0;
    if (blk0 < len) {
        float qf[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uvec4 r = *reinterpret_cast<const uvec4 *>(
                a.q + ((int64_t)b * a.Hq + kv * G + h) * kHeadDim + 8 * sub);
            unpack8(r, qf[h]);
        }
        const uint16_t *kb = a.k + (int64_t)unit * a.max_ctx * kHeadDim + 8 * sub;
        float *zb = a.zq + ((int64_t)b * a.Hq + kv * G) * a.zstride;
        for (int it = 0; it < kRecKeysPerBlock / 64; ++it) {
            const int64_t i0 = blk0 + it * 64 + wv * 16;  // this wave's 16 keys
            if (i0 >= len) break;
            uvec4 raw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t key = i0 + 4 * r + kk;
                raw[r] = key < len ? *reinterpret_cast<const uvec4 *>(kb + key * kHeadDim)
                                   : uvec4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float kf[8];
                unpack8(raw[r], kf);
                float acc[G];
                double n2 = 0.0;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    acc[h] = 0.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[h] = fmaf(qf[h][j], kf[j], acc[h]);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) n2 = fma((double)kf[j], (double)kf[j], n2);
#pragma unroll
                for (int h = 0; h < G; ++h) acc[h] = rsum16(acc[h]);
                n2 = rsum16_d(n2);
                const int64_t key = i0 + 4 * r + kk;
                if (key < len) {
                    nmax = fmax(nmax, n2);
                    if (sub < G) {
                        float v = acc[0];
#pragma unroll
                        for (int h = 1; h < G; ++h) v = (sub == h) ? acc[h] : v;
                        zb[sub * a.zstride + key] = v;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) nmax = fmax(nmax, __shfl_xor(nmax, off));
    if (lane == 0) wmax[wv] = nmax;
    __syncthreads();
    if (t == 0)
        a.norm2[(int64_t)unit * a.n_kblk + blockIdx.x] =
            fmax(fmax(wmax[0], wmax[1]), fmax(wmax[2], wmax[3]));
}

// ---- 1024-thread block primitives (16 waves) ----

// Inclusive prefix sum; `wt` is 16 ints of LDS.  *total gets the block sum.
__device__ __forceinline__ int scan_incl_1024(int v, int *wt, int *total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) wt[wv] = x;
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int s = wt[i];
        pre += (i < wv) ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return pre + x;
}

__device__ __forceinline__ double max_1024(double v, double *wd) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
    if (lane == 0) wd[wv] = v;
    __syncthreads();
    double m = wd[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmax(m, wd[i]);
    __syncthreads();
    return m;
}

// Order-preserving map of a float onto u32: larger float, larger key.
__device__ __forceinline__ uint32_t okey(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_okey(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct RecSmem {
    uint32_t hist[4096];  // radix passes use 2048 bins, the score histogram up to 8 * 256 + 1
    float qs[kHeadDim];
    int wt[16];
    double wd[16];
    int digit, need, nband;
};

// The cut of the group's Hamming selection: T = the k_eff-th smallest
// score, keys below T, keys at T.
__device__ void tie_bucket(const RecallArgs &a, RecSmem &sm, int unit, int64_t len, int ke) {
    const int t = threadIdx.x;
    const int nbins = a.nbits * a.G + 1;
    for (int j = t; j < 4096; j += kRecThreads) sm.hist[j] = 0;
    __syncthreads();
    const uint16_t *sc = a.scores + (int64_t)unit * a.max_ctx;
    // four independent loads in flight per thread
    for (int64_t i0 = t; i0 < len; i0 += 4 * kRecThreads) {
        int v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i = i0 + (int64_t)e * kRecThreads;
            v4[e] = i < len ? (int)sc[i] : -1;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (v4[e] >= 0) atomicAdd(&sm.hist[v4[e] < nbins ? v4[e] : nbins - 1], 1u);
    }
    __syncthreads();
    const int c = (int)(sm.hist[4 * t] + sm.hist[4 * t + 1] + sm.hist[4 * t + 2] +
                        sm.hist[4 * t + 3]);
    int tot;
    const int incl = scan_incl_1024(c, sm.wt, &tot);
    const int excl = incl - c;
    int32_t *out = a.tie + (int64_t)unit * 4;
    if (ke == 0) {
        if (t == 0) {
            out[0] = -1;
            out[1] = out[2] = out[3] = 0;
        }
    } else if (excl < ke && ke <= incl) {
        int cum = excl;
        for (int j = 0; j < 4; ++j) {
            const int bin = 4 * t + j, hv = (int)sm.hist[bin];
            if (cum + hv >= ke) {
                out[0] = bin;
                out[1] = cum;
                out[2] = hv;
                out[3] = ke;
                break;
            }
            cum += hv;
        }
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kRecThreads) k_recall_select(RecallArgs a) {
    __shared__ RecSmem sm;
    const int bh = blockIdx.x, b = bh / a.Hq, h = bh - b * a.Hq, kv = h / a.G;
    const int unit = b * a.Hkv + kv;
    const int t = threadIdx.x;
    const int64_t len = rec_len(a, b);
    int64_t kk = a.topk[b];
    kk = kk < 0 ? 0 : (kk > a.k_max ? a.k_max : kk);
    const int ke = (int)(kk < len ? kk : len);
    int32_t *ex = a.exact_idx ? a.exact_idx + (int64_t)bh * a.k_max : nullptr;

    if (h % a.G == 0) tie_bucket(a, sm, unit, len, ke);
    if (ke == 0) {
        if (ex)
            for (int j = t; j < a.k_max; j += kRecThreads) ex[j] = -1;
        if (t == 0) a.overlap[bh] = 0;
        return;
    }

    // The bound E from |q| and the largest key norm of the unit.
    if (t < kHeadDim) sm.qs[t] = bf16_to_f32(a.q[((int64_t)b * a.Hq + h) * kHeadDim + t]);
    const int nblk = (int)((len + kRecKeysPerBlock - 1) / kRecKeysPerBlock);
    double m = 0.0;
    for (int j = t; j < nblk; j += kRecThreads) m = fmax(m, a.norm2[(int64_t)unit * a.n_kblk + j]);
    const double kn2 = max_1024(m, sm.wd);  // (its barriers also publish qs)
    double qn2 = 0.0;
    for (int d = 0; d < kHeadDim; ++d) qn2 = fma((double)sm.qs[d], (double)sm.qs[d], qn2);
    const double prod = qn2 * kn2;
    const bool all_exact = !(prod < 0x1p240);  // ||q|| ||k|| >= 2^120: fp32 may overflow
    const double E = all_exact ? 0.0 : ldexp(sqrt(prod), -18) + 0x1p-100;

    const float *zrow = a.zq + (int64_t)bh * a.zstride;
    const int64_t bbase = (int64_t)bh * a.max_ctx;

    // Radix select of the ke-th largest estimate: 11 + 11 + 10 bits.
    float tval = 0.f;
    if (!all_exact) {
        uint32_t prefix = 0, pmask = 0;
        int need = ke;
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int nb = pass == 2 ? 1024 : 2048;
            for (int j = t; j < 2048; j += kRecThreads) sm.hist[j] = 0;
            __syncthreads();
            // four estimates per load (rows are padded to 64 entries; the
            // entries past len are not counted)
            for (int64_t i4 = 4 * (int64_t)t; i4 < len; i4 += 4 * kRecThreads) {
                const float4 v = *reinterpret_cast<const float4 *>(zrow + i4);
                const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t key = okey(e4[e]);
                    if (i4 + e < len && (key & pmask) == prefix)
                        atomicAdd(&sm.hist[(key >> shift) & (nb - 1)], 1u);
                }
            }
            __syncthreads();
            const int per = nb / kRecThreads;  // bins per thread, from the top
            int c = 0;
            for (int j = 0; j < per; ++j) c += (int)sm.hist[nb - 1 - (t * per + j)];
            int tot;
            const int incl = scan_incl_1024(c, sm.wt, &tot);
            const int excl = incl - c;
            if (excl < need && need <= incl) {
                int cum = excl;
                for (int j = 0; j < per; ++j) {
                    const int bin = nb - 1 - (t * per + j), hv = (int)sm.hist[bin];
                    if (cum + hv >= need) {
                        sm.digit = bin;
                        sm.need = need - cum;
                        break;
                    }
                    cum += hv;
                }
            }
            __syncthreads();
            prefix |= (uint32_t)sm.digit << shift;
            pmask |= (uint32_t)(nb - 1) << shift;
            need = sm.need;
            __syncthreads();
        }
        tval = from_okey(prefix);
    }
    const double hi = all_exact ? (double)INFINITY : (double)tval + 2.0 * E;
    const double lo = all_exact ? -(double)INFINITY : (double)tval - 2.0 * E;

    // Certainly in (above hi), certainly out (below lo), or ranked exactly.
    if (t == 0) sm.nband = 0;
    __syncthreads();
    int u = 0;
    for (int64_t i4 = 4 * (int64_t)t; i4 < len; i4 += 4 * kRecThreads) {
        const float4 v = *reinterpret_cast<const float4 *>(zrow + i4);
        const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i = i4 + e;
            const double z = e4[e];
            if (i >= len) {
            } else if (!all_exact && z > hi) {
                ++u;
            } else if (all_exact || z >= lo) {
                const int p = atomicAdd(&sm.nband, 1);
                a.band_idx[bbase + p] = (int)i;
            }
        }
    }
    int n_in;
    scan_incl_1024(u, sm.wt, &n_in);
    const int nband = sm.nband;
    __threadfence_block();
    __syncthreads();
    for (int p = t; p < nband; p += kRecThreads) {
        const int64_t i = a.band_idx[bbase + p];
        const uvec4 *kr = reinterpret_cast<const uvec4 *>(
            a.k + ((int64_t)unit * a.max_ctx + i) * kHeadDim);
        double z = 0.0;
#pragma unroll 2
        for (int c = 0; c < kHeadDim / 8; ++c) {
            float kf[8];
            unpack8(kr[c], kf);
#pragma unroll
            for (int j = 0; j < 8; ++j) z = fma((double)sm.qs[8 * c + j], (double)kf[j], z);
        }
        a.band_z[bbase + p] = z;
    }
    __threadfence_block();
    __syncthreads();
    const int places = ke - n_in;
    for (int p = t; p < nband; p += kRecThreads) {
        const double zp = a.band_z[bbase + p];
        const int ip = a.band_idx[bbase + p];
        int r = 0;
        for (int l = 0; l < nband; ++l) {
            const double zl = a.band_z[bbase + l];
            const int il = a.band_idx[bbase + l];
            r += (zl > zp) || (zl == zp && il < ip);
        }
        a.member[bbase + ip] = r < places ? 1 : 0;
    }
    __threadfence_block();
    __syncthreads();

    auto member = [&](int64_t i) -> int {
        if (all_exact) return a.member[bbase + i];
        const double z = zrow[i];
        if (z > hi) return 1;
        if (z >= lo) return a.member[bbase + i];
        return 0;
    };

    if (ex) {
        int base = 0;
        for (int64_t c0 = 0; c0 < len; c0 += 8 * kRecThreads) {
            int flags = 0, cnt = 0;
            for (int j = 0; j < 8; ++j) {
                const int64_t i = c0 + 8 * t + j;
                const int f = (i < len) ? member(i) : 0;
                flags |= f << j;
                cnt += f;
            }
            int tot;
            int pos = base + scan_incl_1024(cnt, sm.wt, &tot) - cnt;
            for (int j = 0; j < 8; ++j) {
                if ((flags >> j) & 1) {
                    if (pos < ke) ex[pos] = (int)(c0 + 8 * t + j);
                    ++pos;
                }
            }
            base += tot;
        }
        for (int j = ke + t; j < a.k_max; j += kRecThreads) ex[j] = -1;
    }

    const int32_t *sel = a.sel_idx + (int64_t)unit * a.k_max;
    int ov = 0;
    for (int j = t; j < ke; j += kRecThreads) {
        const int s = sel[j];
        if (s >= 0 && s < len) ov += member(s);
    }
    int ov_tot;
    scan_incl_1024(ov, sm.wt, &ov_tot);
    if (t == 0) a.overlap[bh] = ov_tot;
}

bool make_recall_plan(int B, int Hq, int Hkv, int64_t max_ctx, RecallPlan *p) {
    if (B <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || max_ctx < 0) return false;
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return false;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    p->B = B;
    p->Hq = Hq;
    p->Hkv = Hkv;
    p->G = G;
    p->max_ctx = max_ctx;
    p->zstride = (max_ctx + 63) & ~(int64_t)63;
    p->n_kblk = (int)((max_ctx + kRecKeysPerBlock - 1) / kRecKeysPerBlock);
    const size_t heads = (size_t)B * Hq, ctx = (size_t)max_ctx;
    size_t off = 0;
    p->off_zq = off;
    off = up(off + heads * (size_t)p->zstride * sizeof(float));
    p->off_norm2 = off;
    off = up(off + (size_t)B * Hkv * (size_t)(p->n_kblk > 0 ? p->n_kblk : 1) * sizeof(double));
    p->off_band_idx = off;
    off = up(off + heads * ctx * sizeof(int32_t));
    p->off_band_z = off;
    off = up(off + heads * ctx * sizeof(double));
    p->off_member = off;
    off = up(off + heads * ctx);
    p->total = off;
    return true;
}

hipError_t launch_recall(const RecallPlan &p, int n_bits, const uint16_t *k_cache, const int32_t *seq_len,
                         const uint16_t *q, const int32_t *topk, int k_max,
                         const int32_t *sel_idx, const uint16_t *scores, int32_t *overlap,
                         int32_t *tie, int32_t *exact_idx, void *ws, hipStream_t s) {
    RecallArgs a;
    char *w = static_cast<char *>(ws);
    a.k = k_cache;
    a.q = q;
    a.seq_len = seq_len;
    a.topk = topk;
    a.sel_idx = sel_idx;
    a.scores = scores;
    a.overlap = overlap;
    a.tie = tie;
    a.exact_idx = exact_idx;
    a.zq = reinterpret_cast<float *>(w + p.off_zq);
    a.norm2 = reinterpret_cast<double *>(w + p.off_norm2);
    a.band_idx = reinterpret_cast<int32_t *>(w + p.off_band_idx);
    a.band_z = reinterpret_cast<double *>(w + p.off_band_z);
    a.member = reinterpret_cast<uint8_t *>(w + p.off_member);
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.G = p.G;
    a.k_max = k_max;
    a.nbits = n_bits;
    a.n_kblk = p.n_kblk;
    a.max_ctx = p.max_ctx;
    a.zstride = p.zstride;
    if (p.n_kblk > 0) {
        const dim3 grid(p.n_kblk, p.B * p.Hkv);
        switch (p.G) {
            case 1: k_logit_estimates<1><<<grid, 256, 0, s>>>(a); break;
            case 2: k_logit_estimates<2><<<grid, 256, 0, s>>>(a); break;
            case 4: k_logit_estimates<4><<<grid, 256, 0, s>>>(a); break;
            default: k_logit_estimates<8><<<grid, 256, 0, s>>>(a); break;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    k_recall_select<<<p.B * p.Hq, kRecThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hata
