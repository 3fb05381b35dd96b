// Decode step of hash-aware top-k attention on gfx950 (HATA review,
// "What carries the argument": query code XOR every cached key code,
// popcount into a Hamming score, top-k, attention over the selected K/V;
// TopK by Hamming distance per Algorithm 3 as discussed in the referee
// report, major comment 1).
//
// Three kernels, all on the caller's stream:
//   k_qenc          one workgroup per (batch, KV head): exact sign codes of
//                   the group's G query heads; clears the unit's histogram
//                   and merge counter for this call.
//   k_scan          one workgroup per (scan chunk, unit): 16-byte code loads,
//                   G x (XOR + popcount) against the query codes held in
//                   scalar registers, u16 score store, LDS histogram of the
//                   0..128G score range; writes the chunk's cumulative
//                   histogram and adds its counts into the unit histogram.
//   k_select_attend one workgroup per (attention split, unit): finds the cut
//                   score T and the tie quota from the unit histogram, the
//                   ties already taken by earlier chunks from their
//                   cumulative histograms, re-reads its u16 scores, compacts
//                   the selected indices in index order into LDS, gathers
//                   their bf16 K/V rows (16 lanes per row, 16 bytes per
//                   lane) with an online softmax per 16-lane group, and
//                   writes one (m, l, o) partial per query head.  The last
//                   split of a unit to finish merges the partials in split
//                   order and stores the bf16 output.
#include "device_util.h"
#include "hata_internal.h"
#include "../../include/hata.h"

namespace hata {

constexpr int kListCap = 4096;  // selected indices buffered in LDS
constexpr int kSelBlock = 2048; // keys examined per selection round (256 x 8)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int64_t clamp_len(int64_t v, int64_t hi) {
    return v < 0 ? 0 : (v > hi ? hi : v);
}

// ------------------------------------------------------------------ qenc
// grid: B * Hkv; block: 128 (thread j = code bit j for every head of the group)
template <int G>
__global__ __launch_bounds__(128) void k_qenc(const uint16_t *__restrict__ q,
                                              const float *__restrict__ w, int Hkv, int NB,
                                              uint32_t *__restrict__ qcodes,
                                              uint32_t *__restrict__ unit_hist,
                                              uint32_t *__restrict__ done) {
    __shared__ float xq[G][kHeadDim];
    const int unit = blockIdx.x, b = unit / Hkv, kv = unit % Hkv, Hq = Hkv * G;
    const int j = threadIdx.x;
    float wv[kHeadDim];
    load_wcol(w + (int64_t)kv * kHeadDim * kBits + j, wv);
#pragma unroll
    for (int h = 0; h < G; ++h)
        xq[h][j] = bf16_to_f32(q[((int64_t)b * Hq + kv * G + h) * kHeadDim + j]);
    for (int i = j; i < NB; i += 128) unit_hist[(int64_t)unit * NB + i] = 0u;
    if (j == 0) done[unit] = 0u;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const bool bit = exact_sign(xq[h], wv);
        const uint64_t m = __ballot(bit);
        if ((j & 63) == 0) {
            uint32_t *dst = qcodes + ((int64_t)b * Hq + kv * G + h) * kWords + (j >> 6) * 2;
            dst[0] = (uint32_t)m;
            dst[1] = (uint32_t)(m >> 32);
        }
    }
}

// ------------------------------------------------------------------ scan
template <int G>
__device__ __forceinline__ int group_hamming(const uint4 &k, const uint32_t (&qc)[G][4]) {
    int s = 0;
#pragma unroll
    for (int h = 0; h < G; ++h)
        s += __popc(k.x ^ qc[h][0]) + __popc(k.y ^ qc[h][1]) + __popc(k.z ^ qc[h][2]) +
             __popc(k.w ^ qc[h][3]);
    return s;
}

// grid: (n_chunks, units); block 256
template <int G>
__global__ __launch_bounds__(256) void k_scan(const uint32_t *__restrict__ codes,
                                              const int32_t *__restrict__ seq_len,
                                              const uint32_t *__restrict__ qcodes,
                                              int64_t max_ctx, int Hkv, int chunk, int n_chunks,
                                              uint16_t *__restrict__ scores, int64_t sstride,
                                              uint16_t *__restrict__ chunk_hist,
                                              uint32_t *__restrict__ unit_hist) {
    constexpr int NB = G * kBits + 1;
    constexpr int PER = (NB + 255) / 256;
    __shared__ uint32_t hist[NB];
    __shared__ int scan_tmp[4];
    const int c = blockIdx.x, unit = blockIdx.y, b = unit / Hkv, kv = unit % Hkv;
    const int64_t len = clamp_len(seq_len[b], max_ctx);
    const int64_t c0 = (int64_t)c * chunk;
    if (c0 >= len) return;
    const int64_t c1 = c0 + chunk < len ? c0 + chunk : len;
    for (int i = threadIdx.x; i < NB; i += 256) hist[i] = 0u;
    uint32_t qc[G][4];
    const uint32_t *qsrc = qcodes + ((int64_t)b * Hkv * G + kv * G) * kWords;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) qc[h][t] = qsrc[h * 4 + t];
    __syncthreads();
    const uint4 *kc = reinterpret_cast<const uint4 *>(codes) + (int64_t)unit * max_ctx;
    uint16_t *sc = scores + (int64_t)unit * sstride;
    for (int64_t i = c0 + threadIdx.x; i < c1; i += 256) {
        const int s = group_hamming<G>(kc[i], qc);
        sc[i] = (uint16_t)s;
        atomicAdd(&hist[s], 1u);
    }
    __syncthreads();
    // cumulative histogram of the chunk, and its counts into the unit's
    uint32_t loc[PER];
    int tsum = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int bin = threadIdx.x * PER + e;
        loc[e] = bin < NB ? hist[bin] : 0u;
        tsum += (int)loc[e];
    }
    int tot;
    int run = block_excl_scan_256(tsum, scan_tmp, &tot);
    uint16_t *ch = chunk_hist + ((int64_t)unit * n_chunks + c) * NB;
    uint32_t *uh = unit_hist + (int64_t)unit * NB;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int bin = threadIdx.x * PER + e;
        if (bin < NB) {
            run += (int)loc[e];
            ch[bin] = (uint16_t)run;
            if (loc[e]) atomicAdd(&uh[bin], loc[e]);
        }
    }
}

// ------------------------------------------------------------------ select + attend

struct SoftmaxState {
    float m, l;
};

// Merge (m2, l2, o2) into (m, l, o): the log-sum-exp combination of two
// partial softmax sums in base 2.
__device__ __forceinline__ void lse_weights(float m1, float m2, float *M, float *a1, float *a2) {
    const float mm = fmaxf(m1, m2);
    *M = mm;
    *a1 = (m1 == -INFINITY) ? 0.f : exp2f(m1 - mm);
    *a2 = (m2 == -INFINITY) ? 0.f : exp2f(m2 - mm);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 &r, float (&f)[8]) {
    f[0] = __uint_as_float(r.x << 16);
    f[1] = __uint_as_float(r.x & 0xFFFF0000u);
    f[2] = __uint_as_float(r.y << 16);
    f[3] = __uint_as_float(r.y & 0xFFFF0000u);
    f[4] = __uint_as_float(r.z << 16);
    f[5] = __uint_as_float(r.z & 0xFFFF0000u);
    f[6] = __uint_as_float(r.w << 16);
    f[7] = __uint_as_float(r.w & 0xFFFF0000u);
}

template <int G>
__device__ __forceinline__ void attend_one(const uint4 &kr, const uint4 &vr,
                                           const float (&qs)[G][8], float (&m)[G], float (&l)[G],
                                           float (&o)[G][8]) {
    float kf[8], vf[8];
    unpack_bf16x8(kr, kf);
    unpack_bf16x8(vr, vf);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qs[h][e], kf[e], d);
        d += __shfl_xor(d, 1, 16);
        d += __shfl_xor(d, 2, 16);
        d += __shfl_xor(d, 4, 16);
        d += __shfl_xor(d, 8, 16);
        const float mn = fmaxf(m[h], d);
        const float a = exp2f(m[h] - mn);
        const float p = exp2f(d - mn);
        l[h] = fmaf(l[h], a, p);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = fmaf(o[h][e], a, p * vf[e]);
        m[h] = mn;
    }
}

// Attend over list[0..n): 16 groups of 16 lanes, group g takes entries
// g, g + 16, ...; lane l16 holds dims [8 l16, 8 l16 + 8).
template <int G>
__device__ __forceinline__ void attend_list(const uint16_t *__restrict__ Ku,
                                            const uint16_t *__restrict__ Vu, const int *list,
                                            int n, int grp, int l16, const float (&qs)[G][8],
                                            float (&m)[G], float (&l)[G], float (&o)[G][8]) {
    int j = grp;
    for (; j + 48 < n; j += 64) {
        const int i0 = list[j], i1 = list[j + 16], i2 = list[j + 32], i3 = list[j + 48];
        const uint4 k0 = *reinterpret_cast<const uint4 *>(Ku + (int64_t)i0 * kHeadDim + l16 * 8);
        const uint4 k1 = *reinterpret_cast<const uint4 *>(Ku + (int64_t)i1 * kHeadDim + l16 * 8);
        const uint4 k2 = *reinterpret_cast<const uint4 *>(Ku + (int64_t)i2 * kHeadDim + l16 * 8);
        const uint4 k3 = *reinterpret_cast<const uint4 *>(Ku + (int64_t)i3 * kHeadDim + l16 * 8);
        const uint4 v0 = *reinterpret_cast<const uint4 *>(Vu + (int64_t)i0 * kHeadDim + l16 * 8);
        const uint4 v1 = *reinterpret_cast<const uint4 *>(Vu + (int64_t)i1 * kHeadDim + l16 * 8);
        const uint4 v2 = *reinterpret_cast<const uint4 *>(Vu + (int64_t)i2 * kHeadDim + l16 * 8);
        const uint4 v3 = *reinterpret_cast<const uint4 *>(Vu + (int64_t)i3 * kHeadDim + l16 * 8);
        attend_one<G>(k0, v0, qs, m, l, o);
        attend_one<G>(k1, v1, qs, m, l, o);
        attend_one<G>(k2, v2, qs, m, l, o);
        attend_one<G>(k3, v3, qs, m, l, o);
    }
    for (; j < n; j += 16) {
        const int i0 = list[j];
        const uint4 k0 = *reinterpret_cast<const uint4 *>(Ku + (int64_t)i0 * kHeadDim + l16 * 8);
        const uint4 v0 = *reinterpret_cast<const uint4 *>(Vu + (int64_t)i0 * kHeadDim + l16 * 8);
        attend_one<G>(k0, v0, qs, m, l, o);
    }
}

// grid: (n_splits, units); block 256
template <int G>
__global__ __launch_bounds__(256) void k_select_attend(
    const uint16_t *__restrict__ k_cache, const uint16_t *__restrict__ v_cache,
    const int32_t *__restrict__ seq_len, const int32_t *__restrict__ topk, int k_max,
    const uint16_t *__restrict__ q, int64_t max_ctx, int Hkv, int chunk, int n_chunks, int cps,
    int n_splits, const uint16_t *__restrict__ scores, int64_t sstride,
    const uint16_t *__restrict__ chunk_hist, const uint32_t *__restrict__ unit_hist,
    float *__restrict__ partials, uint32_t *__restrict__ done, uint16_t *__restrict__ out,
    int32_t *__restrict__ sel_out, int32_t *__restrict__ ctrl) {
    constexpr int NB = G * kBits + 1;
    constexpr int PER = (NB + 255) / 256;
    __shared__ int s_list[kListCap];
    __shared__ int s_scan[4];
    __shared__ long long s_red[4];
    __shared__ int s_T;
    __shared__ int s_below;
    __shared__ int s_last;
    __shared__ float s_m[4][G], s_l[4][G];
    __shared__ float s_o[4][G][kHeadDim];

    const int split = blockIdx.x, unit = blockIdx.y, b = unit / Hkv, kv = unit % Hkv;
    const int Hq = Hkv * G;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l16 = tid & 15, grp = tid >> 4;

    const int64_t len_raw = seq_len[b];
    const int64_t len = clamp_len(len_raw, max_ctx);
    int64_t kreq = topk[b];
    if (kreq < 0) kreq = 0;
    if (split == 0 && kv == 0 && tid == 0) {
        int flags = 0;
        if (len != len_raw) flags |= HATA_DEV_BAD_LENGTH;
        if (kreq > k_max) flags |= HATA_DEV_TOPK_CLAMPED;
        if (flags) atomicOr(&ctrl[kCtrlStatus], flags);
    }
    if (kreq > k_max) kreq = k_max;
    const int64_t k_eff = kreq < len ? kreq : len;
    const int64_t s0 = (int64_t)split * cps * chunk;
    const int64_t s1 = s0 + (int64_t)cps * chunk < len ? s0 + (int64_t)cps * chunk : len;

    int32_t *sel_u = sel_out ? sel_out + (int64_t)unit * k_max : nullptr;
    if (sel_u && split == 0)
        for (int64_t p = k_eff + tid; p < k_max; p += 256) sel_u[p] = -1;

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    if (k_eff > 0 && s0 < s1) {
        // ---- cut score T: first bin whose cumulative count reaches k_eff
        const uint32_t *uh = unit_hist + (int64_t)unit * NB;
        uint32_t loc[PER];
        int tsum = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int bin = tid * PER + e;
            loc[e] = bin < NB ? uh[bin] : 0u;
            tsum += (int)loc[e];
        }
        if (tid == 0) {  // defaults keep every index in range even for an inconsistent histogram
            s_T = NB - 1;
            s_below = 0;
        }
        int tot;
        int run = block_excl_scan_256(tsum, s_scan, &tot);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int nxt = run + (int)loc[e];
            if ((int64_t)run < k_eff && (int64_t)nxt >= k_eff) {
                s_T = tid * PER + e;
                s_below = run;
            }
            run = nxt;
        }
        __syncthreads();
        const int T = s_T;
        const int64_t quota = k_eff - s_below;  // keys of score T to take, lowest index first

        // ---- what chunks before this split already took
        const int cf = split * cps;
        long long ties_b = 0, below_b = 0;
        for (int cc = tid; cc < cf; cc += 256) {
            const uint16_t *ch = chunk_hist + ((int64_t)unit * n_chunks + cc) * NB;
            const int hi = ch[T];
            const int lo = T > 0 ? ch[T - 1] : 0;
            ties_b += hi - lo;
            below_b += lo;
        }
        ties_b = block_sum_256(ties_b, s_red);
        below_b = block_sum_256(below_b, s_red);
        const int64_t rem_quota = quota - ties_b > 0 ? quota - ties_b : 0;
        int64_t out_pos = below_b + (ties_b < quota ? ties_b : quota);

        // ---- query slices, pre-scaled so exp2 gives exp((q.k)/sqrt(d))
        float qs[G][8];
        const float qscale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint4 r = *reinterpret_cast<const uint4 *>(
                q + ((int64_t)b * Hq + kv * G + h) * kHeadDim + l16 * 8);
            float f[8];
            unpack_bf16x8(r, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) qs[h][e] = f[e] * qscale;
        }

        const uint16_t *su = scores + (int64_t)unit * sstride;
        const uint16_t *Ku = k_cache + (int64_t)unit * max_ctx * kHeadDim;
        const uint16_t *Vu = v_cache + (int64_t)unit * max_ctx * kHeadDim;
        int64_t ties_acc = 0;
        int list_n = 0;
        for (int64_t base = s0; base < s1; base += kSelBlock) {
            const int64_t i0 = base + (int64_t)tid * 8;
            int sc[8];
            int n_eq = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sc[e] = (i0 + e < s1) ? (int)su[i0 + e] : 0x7FFFFFFF;
                n_eq += sc[e] == T;
            }
            int tie_tot;
            const int tie_pre = block_excl_scan_256(n_eq, s_scan, &tie_tot);
            int64_t tr = ties_acc + tie_pre;
            unsigned selmask = 0;
            int n_sel = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bool sel = sc[e] < T;
                if (sc[e] == T) {
                    sel = tr < rem_quota;
                    ++tr;
                }
                if (sel) {
                    selmask |= 1u << e;
                    ++n_sel;
                }
            }
            int sel_tot;
            const int sel_pre = block_excl_scan_256(n_sel, s_scan, &sel_tot);
            int p = list_n + sel_pre;
            int64_t gp = out_pos + sel_pre;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (selmask & (1u << e)) {
                    s_list[p++] = (int)(i0 + e);
                    if (sel_u && gp < k_max) sel_u[gp] = (int32_t)(i0 + e);
                    ++gp;
                }
            }
            __syncthreads();
            list_n += sel_tot;
            out_pos += sel_tot;
            ties_acc += tie_tot;
            if (list_n > kListCap - kSelBlock || base + kSelBlock >= s1) {
                attend_list<G>(Ku, Vu, s_list, list_n, grp, l16, qs, m, l, o);
                __syncthreads();
                list_n = 0;
            }
        }
    }

    // ---- combine the 4 groups of each wave (lanes l16, +16, +32, +48)
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float m2 = __shfl_xor(m[h], off, 64);
            const float l2 = __shfl_xor(l[h], off, 64);
            float M, a1, a2;
            lse_weights(m[h], m2, &M, &a1, &a2);
            l[h] = l[h] * a1 + l2 * a2;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float o2 = __shfl_xor(o[h][e], off, 64);
                o[h][e] = o[h][e] * a1 + o2 * a2;
            }
            m[h] = M;
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (lane == 0) {
                s_m[wv][h] = m[h];
                s_l[wv][h] = l[h];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) s_o[wv][h][lane * 8 + e] = o[h][e];
        }
    }
    __syncthreads();
    // ---- combine the 4 waves and write this split's partial
    float *pu = partials + ((int64_t)unit * n_splits + split) * G * kPartialStride;
    for (int pr = tid; pr < G * kHeadDim; pr += 256) {
        const int h = pr / kHeadDim, e = pr % kHeadDim;
        float M = s_m[0][h], L = s_l[0][h], O = s_o[0][h][e];
#pragma unroll
        for (int w2 = 1; w2 < 4; ++w2) {
            float Mn, a1, a2;
            lse_weights(M, s_m[w2][h], &Mn, &a1, &a2);
            L = L * a1 + s_l[w2][h] * a2;
            O = O * a1 + s_o[w2][h][e] * a2;
            M = Mn;
        }
        float *ph = pu + h * kPartialStride;
        ph[4 + e] = O;
        if (e == 0) {
            ph[0] = M;
            ph[1] = L;
        }
    }
    // ---- the last split of the unit merges all partials in split order
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const unsigned prev = atomicAdd(&done[unit], 1u);
        s_last = (prev == (unsigned)n_splits - 1);
    }
    __syncthreads();
    if (s_last) {
        __threadfence();
        const float *pb = partials + (int64_t)unit * n_splits * G * kPartialStride;
        for (int pr = tid; pr < G * kHeadDim; pr += 256) {
            const int h = pr / kHeadDim, e = pr % kHeadDim;
            float M = -INFINITY;
            for (int s = 0; s < n_splits; ++s) M = fmaxf(M, pb[(s * G + h) * kPartialStride]);
            float L = 0.f, O = 0.f;
            if (M != -INFINITY) {
                for (int s = 0; s < n_splits; ++s) {
                    const float *ph = pb + (s * G + h) * kPartialStride;
                    const float ms = ph[0];
                    const float a = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
                    L = fmaf(ph[1], a, L);
                    O = fmaf(ph[4 + e], a, O);
                }
            }
            out[((int64_t)b * Hq + kv * G + h) * kHeadDim + e] =
                L > 0.f ? f32_to_bf16(O / L) : (uint16_t)0;
        }
        if (tid == 0) done[unit] = 0u;
    }
}

// ------------------------------------------------------------------ plan + launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool make_decode_plan(int B, int Hq, int Hkv, int64_t max_ctx, DecodePlan *p) {
    if (B <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || max_ctx < 0) return false;
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return false;
    const int64_t units = (int64_t)B * Hkv;
    if (units > 65535) return false;
    DecodePlan d;
    d.B = B;
    d.Hq = Hq;
    d.Hkv = Hkv;
    d.G = G;
    d.NB = G * kBits + 1;
    d.max_ctx = max_ctx;
    int chunk = 4096;
    while (chunk > 1024 && units * ((max_ctx + chunk - 1) / chunk) < 1024) chunk >>= 1;
    d.chunk = chunk;
    d.n_chunks = (int)((max_ctx + chunk - 1) / chunk);
    if (d.n_chunks < 1) d.n_chunks = 1;
    const int target = (int)((512 + units - 1) / units);
    int cps = d.n_chunks / (target > 0 ? target : 1);
    if (cps < 1) cps = 1;
    if ((d.n_chunks + cps - 1) / cps > 64) cps = (d.n_chunks + 63) / 64;
    d.cps = cps;
    d.n_splits = (d.n_chunks + cps - 1) / cps;
    d.sstride = ((max_ctx + 63) / 64) * 64;
    size_t off = 0;
    d.off_qcodes = off;
    off = align256(off + (size_t)B * Hq * kWords * 4);
    d.off_unit_hist = off;
    off = align256(off + (size_t)units * d.NB * 4);
    d.off_done = off;
    off = align256(off + (size_t)units * 4);
    d.off_chunk_hist = off;
    off = align256(off + (size_t)units * d.n_chunks * d.NB * 2);
    d.off_partials = off;
    off = align256(off + (size_t)units * d.n_splits * G * kPartialStride * 4);
    d.off_scores = off;
    off = align256(off + (size_t)units * d.sstride * 2);
    d.total = off;
    *p = d;
    return true;
}

template <int G>
static hipError_t launch_decode_g(const DecodePlan &p, const uint16_t *k_cache,
                                  const uint16_t *v_cache, const uint32_t *codes,
                                  const int32_t *seq_len, int32_t *ctrl, const uint16_t *q,
                                  const float *w, const int32_t *topk, int k_max, uint16_t *out,
                                  void *ws, int32_t *sel_idx_out, uint16_t *scores_out,
                                  hipStream_t s) {
    char *base = static_cast<char *>(ws);
    uint32_t *qcodes = reinterpret_cast<uint32_t *>(base + p.off_qcodes);
    uint32_t *unit_hist = reinterpret_cast<uint32_t *>(base + p.off_unit_hist);
    uint32_t *done = reinterpret_cast<uint32_t *>(base + p.off_done);
    uint16_t *chunk_hist = reinterpret_cast<uint16_t *>(base + p.off_chunk_hist);
    float *partials = reinterpret_cast<float *>(base + p.off_partials);
    uint16_t *scores = scores_out ? scores_out : reinterpret_cast<uint16_t *>(base + p.off_scores);
    const int64_t sstride = scores_out ? p.max_ctx : p.sstride;
    const int units = p.B * p.Hkv;

    hipLaunchKernelGGL(k_qenc<G>, dim3(units), dim3(128), 0, s, q, w, p.Hkv, p.NB, qcodes,
                       unit_hist, done);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_scan<G>, dim3(p.n_chunks, units), dim3(256), 0, s, codes, seq_len,
                       qcodes, p.max_ctx, p.Hkv, p.chunk, p.n_chunks, scores, sstride,
                       chunk_hist, unit_hist);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_select_attend<G>, dim3(p.n_splits, units), dim3(256), 0, s, k_cache,
                       v_cache, seq_len, topk, k_max, q, p.max_ctx, p.Hkv, p.chunk, p.n_chunks,
                       p.cps, p.n_splits, scores, sstride, chunk_hist, unit_hist, partials, done,
                       out, sel_idx_out, ctrl);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodePlan &p, const uint16_t *k_cache, const uint16_t *v_cache,
                         const uint32_t *codes, const int32_t *seq_len, int32_t *ctrl,
                         const uint16_t *q, const float *w, const int32_t *topk, int k_max,
                         uint16_t *out, void *ws, int32_t *sel_idx_out, uint16_t *scores_out,
                         hipStream_t s) {
    switch (p.G) {
        case 1:
            return launch_decode_g<1>(p, k_cache, v_cache, codes, seq_len, ctrl, q, w, topk,
                                      k_max, out, ws, sel_idx_out, scores_out, s);
        case 2:
            return launch_decode_g<2>(p, k_cache, v_cache, codes, seq_len, ctrl, q, w, topk,
                                      k_max, out, ws, sel_idx_out, scores_out, s);
        case 4:
            return launch_decode_g<4>(p, k_cache, v_cache, codes, seq_len, ctrl, q, w, topk,
                                      k_max, out, ws, sel_idx_out, scores_out, s);
        case 8:
            return launch_decode_g<8>(p, k_cache, v_cache, codes, seq_len, ctrl, q, w, topk,
                                      k_max, out, ws, sel_idx_out, scores_out, s);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace hata
