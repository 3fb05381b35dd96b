// Training of the hash projection W_H on gfx950 (HATA review on pith.science,
// "What carries the argument" and "Assumptions & free parameters"; the label
// rule as the review's circularity check restates Section 3.1.2).
//
// One training step on a batch of n_q queries and n_k keys (bf16 rows of 128):
//   labels   per query, the top ceil(n_k / 10) keys by exact q.k (lower index
//            first among equal scores) get 20 - 19 t / (m - 1) by rank t, every
//            other key -1 (k_hash_labels: double-precision dot products in the
//            defining order, then a bitonic sort of (score, index) in LDS);
//   codes    H = 2 Sigmoid(sigma X W) - 1 and its slope, X = [queries; keys];
//   loss     L = epsilon L_sim + eta L_bal + lambda L_unc with
//              L_sim = (1 / n_q) sum_j sum_i s_ji |a_j - b_i|^2 / 4,
//              L_bal = sum_c mean_c(H)^2,
//              L_unc = |H^T H / n - I|^2;
//   gradient dL/dW = X^T (dL/dH o slope), with
//              dL_sim/da_j = (rowsum_j(S) a_j - (S B)_j) / (2 n_q),
//              dL_sim/db_i = (colsum_i(S) b_i - (S^T A)_i) / (2 n_q),
//              dL_bal/dh_v = 2 mean / n,  dL_unc/dH = (4 / n) H (H^T H / n - I);
//   update   Adam on W_H.
// Every contraction (X W, S B, S^T A, H^T H, H E, X^T G) runs on the matrix
// cores in fp32 (v_mfma_f32_16x16x4f32) through one tiled kernel with fused
// epilogues; sums over rows are reduced in double in a fixed order, so a step
// is deterministic.
#include <math.h>

#include "device_util.h"
#include "hata_internal.h"
#include "../../include/hata.h"

namespace hata {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 32;       // output tile of one workgroup (kTile x kTile)
constexpr int kTileK = 16;      // contraction depth staged through LDS per round
constexpr int kRowsPerPart = 256;

// ---------------------------------------------------------------- labels

// One workgroup per query.  z_i in double with the products (exact for bf16
// operands) accumulated in ascending d, as the definition; keys past n_k are
// sentinels (-inf, index past every key) that sort last.
__global__ __launch_bounds__(kThreads) void k_hash_labels(const uint16_t *__restrict__ q,
                                                          const uint16_t *__restrict__ k, int n_k,
                                                          int n_pad, float *__restrict__ labels) {
    __shared__ double z[kMaxLabelKeys];
    __shared__ int idx[kMaxLabelKeys];
    __shared__ double qd[kHeadDim];
    const int j = blockIdx.x, t = threadIdx.x;
    if (t < kHeadDim) qd[t] = (double)bf16_to_f32(q[(int64_t)j * kHeadDim + t]);
    __syncthreads();
    for (int i = t; i < n_pad; i += kThreads) {
        double s = -INFINITY;
        if (i < n_k) {
            const uint16_t *kr = k + (int64_t)i * kHeadDim;
            s = 0.0;
            for (int d = 0; d < kHeadDim; ++d) s = fma(qd[d], (double)bf16_to_f32(kr[d]), s);
        }
        z[i] = s;
        idx[i] = i;
    }
    // Bitonic sort: "before" = larger z, or equal z and smaller index.
    for (int size = 2; size <= n_pad; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            __syncthreads();
            for (int p = t; p < n_pad / 2; p += kThreads) {
                const int a = (p / stride) * 2 * stride + (p % stride), b = a + stride;
                const double za = z[a], zb = z[b];
                const int ia = idx[a], ib = idx[b];
                const bool b_first = zb > za || (zb == za && ib < ia);
                const bool a_first = za > zb || (za == zb && ia < ib);
                const bool swap = ((a & size) == 0) ? b_first : a_first;
                if (swap) {
                    z[a] = zb;
                    z[b] = za;
                    idx[a] = ib;
                    idx[b] = ia;
                }
            }
        }
    }
    __syncthreads();
    // the row of labels in LDS (over the scores, no longer needed), then out
    float *lab = reinterpret_cast<float *>(z);
    for (int i = t; i < n_k; i += kThreads) lab[i] = -1.0f;
    __syncthreads();
    const int m = (n_k + 9) / 10;
    for (int r = t; r < m; r += kThreads)
        lab[idx[r]] = (float)(m == 1 ? 20.0 : 20.0 - 19.0 * (double)r / (double)(m - 1));
    __syncthreads();
    for (int i = t; i < n_k; i += kThreads) labels[(int64_t)j * n_k + i] = lab[i];
}

// ---------------------------------------------------------------- GEMM

enum Epilogue { kEpiStore = 0, kEpiCodes = 1, kEpiCorr = 2, kEpiGrad = 3 };

struct GemmArgs {
    int M, N, K;
    const void *A;       // element (m, k) at A[m * a_m + k * a_k] (bf16 or fp32)
    int64_t a_m, a_k;
    const float *B;      // element (k, n) at B[k * b_k + n * b_n]
    int64_t b_k, b_n;
    float *C;            // C[m * c_m + n]
    int64_t c_m;
    float alpha;
    // kEpiCodes: C = 2 sigmoid(sigma acc) - 1, slope -> aux (same layout)
    float *aux;
    float sigma;
    // kEpiGrad: C = slope o (eps g_sim + eta 2 mu / n + lam (4 / n) acc)
    const float *H, *slope, *SB, *SA, *rs, *cs, *mu;
    int n_q, n;
    float eps, eta, lam;
};

template <typename TA>
__device__ __forceinline__ float load_a(const TA *p, int64_t i);
template <>
__device__ __forceinline__ float load_a<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_a<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
}

// Workgroup (bx, by) computes C[32 bx .. +32][32 by .. +32]; wave w the 16 x 16
// block (w / 2, w % 2).  Operand rounds of 16 along the contraction go
// through LDS; each feeds four v_mfma_f32_16x16x4f32 per wave (A: lane l holds
// A[l % 16][l / 16]; B: B[l / 16][l % 16]; the result: lane l holds rows
// 4 (l / 16) + i, column l % 16).  M, N multiples of 32, K of 16.
template <typename TA, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmArgs g) {
    __shared__ float As[kTileK][kTile + 1];
    __shared__ float Bs[kTileK][kTile + 1];
    const TA *A = static_cast<const TA *>(g.A);
    const int bm = blockIdx.x * kTile, bn = blockIdx.y * kTile;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wm = (w >> 1) * 16, wn = (w & 1) * 16;
    const bool a_krow = g.a_k == 1;  // k contiguous: 16 threads read 16 k of a row
    const bool b_nrow = g.b_n == 1;  // n contiguous: 32 threads read 32 n of a row
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < g.K; k0 += kTileK) {
#pragma unroll
        for (int e = t; e < kTile * kTileK; e += kThreads) {
            const int mm = a_krow ? e / kTileK : e % kTile, kk = a_krow ? e % kTileK : e / kTile;
            As[kk][mm] = load_a<TA>(A, (int64_t)(bm + mm) * g.a_m + (int64_t)(k0 + kk) * g.a_k);
            const int nn = b_nrow ? e % kTile : e / kTileK, kb = b_nrow ? e / kTile : e % kTileK;
            Bs[kb][nn] = g.B[(int64_t)(k0 + kb) * g.b_k + (int64_t)(bn + nn) * g.b_n];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kTileK; kk += 4) {
            const float a = As[kk + (lane >> 4)][wm + (lane & 15)];
            const float b = Bs[kk + (lane >> 4)][wn + (lane & 15)];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    const int col = bn + wn + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = bm + wm + 4 * (lane >> 4) + i;
        const int64_t o = (int64_t)row * g.c_m + col;
        const float v = acc[i];
        if (EPI == kEpiStore) {
            g.C[o] = g.alpha * v;
        } else if (EPI == kEpiCorr) {
            g.C[o] = g.alpha * v - (row == col ? 1.0f : 0.0f);
        } else if (EPI == kEpiCodes) {
            const float sg = 1.0f / (1.0f + expf(-g.sigma * v));
            g.C[o] = 2.0f * sg - 1.0f;
            g.aux[o] = 2.0f * g.sigma * sg * (1.0f - sg);
        } else {  // kEpiGrad: row is a query (row < n_q) or key row - n_q
            const float h = g.H[o];
            const float sim = row < g.n_q
                                  ? (g.rs[row] * h - g.SB[(int64_t)row * g.c_m + col])
                                  : (g.cs[row - g.n_q] * h - g.SA[(int64_t)(row - g.n_q) * g.c_m + col]);
            const float gh = g.eps * sim / (2.0f * (float)g.n_q) + g.eta * 2.0f * g.mu[col] / (float)g.n +
                             g.lam * 4.0f * v / (float)g.n;
            g.C[o] = gh * g.slope[o];
        }
    }
}

template <typename TA, int EPI>
hipError_t gemm(const GemmArgs &g, hipStream_t s) {
    hipLaunchKernelGGL((k_gemm<TA, EPI>), dim3(g.M / kTile, g.N / kTile), dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

// ---------------------------------------------------------------- small kernels

// X = [queries; keys], bf16 [n][128] (16-byte pieces).
__global__ __launch_bounds__(kThreads) void k_concat(const uint4 *__restrict__ q, int n_q,
                                                     const uint4 *__restrict__ k, int n_k,
                                                     uint4 *__restrict__ x) {
    const int64_t per_row = kHeadDim / 8, total = (int64_t)(n_q + n_k) * per_row;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads)
        x[i] = i < (int64_t)n_q * per_row ? q[i] : k[i - (int64_t)n_q * per_row];
}

// Block sum of a double over 256 threads; every thread gets the total.
__device__ __forceinline__ double block_sum_double(double v, double *tmp) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) tmp[w] = v;
    __syncthreads();
    return (tmp[0] + tmp[1]) + (tmp[2] + tmp[3]);
}

// Row sums of the labels (workgroups 0 .. n_q - 1) and column sums (the
// remaining workgroups, 256 keys each), in double, stored as float.
__global__ __launch_bounds__(kThreads) void k_label_sums(const float *__restrict__ S, int n_q, int n_k,
                                                         float *__restrict__ rs, float *__restrict__ cs) {
    __shared__ double tmp[4];
    const int t = threadIdx.x;
    if ((int)blockIdx.x < n_q) {
        const float *row = S + (int64_t)blockIdx.x * n_k;
        double s = 0.0;
        for (int i = t; i < n_k; i += kThreads) s += (double)row[i];
        s = block_sum_double(s, tmp);
        if (t == 0) rs[blockIdx.x] = (float)s;
    } else {
        const int i = ((int)blockIdx.x - n_q) * kThreads + t;
        if (i < n_k) {
            double s = 0.0;
            for (int j = 0; j < n_q; ++j) s += (double)S[(int64_t)j * n_k + i];
            cs[i] = (float)s;
        }
    }
}

// Partial column sums of H over parts of kRowsPerPart rows: part p, column c
// (threads stride the columns).
__global__ __launch_bounds__(kThreads) void k_col_parts(const float *__restrict__ H, int n, int r,
                                                        double *__restrict__ part) {
    const int p = blockIdx.x;
    const int v0 = p * kRowsPerPart, v1 = v0 + kRowsPerPart < n ? v0 + kRowsPerPart : n;
    for (int c = threadIdx.x; c < r; c += kThreads) {
        double s = 0.0;
        for (int v = v0; v < v1; ++v) s += (double)H[(int64_t)v * r + c];
        part[(int64_t)p * r + c] = s;
    }
}

// The loss terms, per part of kRowsPerPart rows (similarity and the rows'
// share of nothing else) and one more part for the r x r deviation E:
//   sim part: sum over its rows of rowsum |a|^2 - 2 a . SB (queries) or
//             colsum |b|^2 (keys);
//   last:     sum of E^2.
__global__ __launch_bounds__(kThreads) void k_loss_parts(const float *__restrict__ H, const float *__restrict__ SB,
                                                         const float *__restrict__ rs, const float *__restrict__ cs,
                                                         const float *__restrict__ E, int n_q, int n, int r,
                                                         double *__restrict__ part) {
    __shared__ double tmp[4];
    const int p = blockIdx.x, t = threadIdx.x;
    const int n_parts = (n + kRowsPerPart - 1) / kRowsPerPart;
    double s = 0.0;
    if (p < n_parts) {
        const int v = p * kRowsPerPart + t;
        if (v < n) {
            const float *hv = H + (int64_t)v * r;
            double sq = 0.0, dot = 0.0;
            for (int c = 0; c < r; ++c) {
                sq += (double)hv[c] * (double)hv[c];
                if (v < n_q) dot += (double)hv[c] * (double)SB[(int64_t)v * r + c];
            }
            s = v < n_q ? (double)rs[v] * sq - 2.0 * dot : (double)cs[v - n_q] * sq;
        }
    } else {
        for (int i = t; i < r * r; i += kThreads) s += (double)E[i] * (double)E[i];
    }
    s = block_sum_double(s, tmp);
    if (t == 0) part[p] = s;
}

// Column means (from the parts, in part order), then the loss: one workgroup.
__global__ __launch_bounds__(kThreads) void k_loss_final(const double *__restrict__ colpart, int n_parts,
                                                         const double *__restrict__ losspart, int n, int n_q,
                                                         int r, float eps, float eta, float lam,
                                                         float *__restrict__ mu, float *__restrict__ loss) {
    __shared__ double tmp[4];
    double bal = 0.0;
    for (int c = threadIdx.x; c < r; c += kThreads) {
        double s = 0.0;
        for (int p = 0; p < n_parts; ++p) s += colpart[(int64_t)p * r + c];
        const double m = s / (double)n;
        mu[c] = (float)m;
        bal += m * m;
    }
    bal = block_sum_double(bal, tmp);
    if (threadIdx.x == 0) {
        double sim = 0.0;
        for (int p = 0; p < n_parts; ++p) sim += losspart[p];
        sim = sim / (4.0 * (double)n_q);
        const double unc = losspart[n_parts];
        loss[0] = (float)((double)eps * sim + (double)eta * bal + (double)lam * unc);
        loss[1] = (float)sim;
        loss[2] = (float)bal;
        loss[3] = (float)unc;
    }
}

// Adam on W (c1 = 1 / (1 - b1^t), c2 = 1 / (1 - b2^t) from the host); the
// gradient is copied out when asked for.
__global__ __launch_bounds__(kThreads) void k_adam(float *__restrict__ w, float *__restrict__ m,
                                                   float *__restrict__ v, const float *__restrict__ g,
                                                   int64_t n, float lr, float b1, float b2, float e,
                                                   float c1, float c2, int update, float *__restrict__ g_out) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
        const float gi = g[i];
        if (g_out) g_out[i] = gi;
        if (update) {
            const float mi = b1 * m[i] + (1.0f - b1) * gi;
            const float vi = b2 * v[i] + (1.0f - b2) * gi * gi;
            m[i] = mi;
            v[i] = vi;
            w[i] = w[i] - lr * (mi * c1) / (sqrtf(vi * c2) + e);
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool make_train_plan(int n_q, int n_k, int n_bits, TrainPlan *p) {
    if (n_q <= 0 || n_k <= 0 || n_q % kTile || n_k % kTile) return false;
    if (n_bits != 32 && n_bits != 64 && n_bits != 128 && n_bits != 256) return false;
    if ((int64_t)n_q + n_k > (1 << 24)) return false;
    TrainPlan d;
    d.n_q = n_q;
    d.n_k = n_k;
    d.n = n_q + n_k;
    d.r = n_bits;
    d.n_parts = (d.n + kRowsPerPart - 1) / kRowsPerPart;
    const size_t n = (size_t)d.n, r = (size_t)n_bits;
    size_t off = 0;
    d.off_x = off;     off = align256(off + n * kHeadDim * 2);
    d.off_h = off;     off = align256(off + n * r * 4);
    d.off_slope = off; off = align256(off + n * r * 4);
    d.off_sb = off;    off = align256(off + (size_t)n_q * r * 4);
    d.off_sa = off;    off = align256(off + (size_t)n_k * r * 4);
    d.off_rs = off;    off = align256(off + (size_t)n_q * 4);
    d.off_cs = off;    off = align256(off + (size_t)n_k * 4);
    d.off_e = off;     off = align256(off + r * r * 4);
    d.off_mu = off;    off = align256(off + r * 4);
    d.off_gy = off;    off = align256(off + n * r * 4);
    d.off_grad = off;  off = align256(off + (size_t)kHeadDim * r * 4);
    d.off_colpart = off; off = align256(off + (size_t)d.n_parts * r * 8);
    d.off_losspart = off; off = align256(off + (size_t)(d.n_parts + 1) * 8);
    d.total = off;
    *p = d;
    return true;
}

hipError_t launch_hash_labels(const uint16_t *q, int n_q, const uint16_t *k, int n_k, float *labels,
                              hipStream_t s) {
    int n_pad = 1;
    while (n_pad < n_k) n_pad <<= 1;
    if (n_pad < 2) n_pad = 2;
    hipLaunchKernelGGL(k_hash_labels, dim3(n_q), dim3(kThreads), 0, s, q, k, n_k, n_pad, labels);
    return hipGetLastError();
}

hipError_t launch_hash_train_step(const TrainPlan &p, const uint16_t *q, const uint16_t *k,
                                  const float *labels, float *w, float *adam_m, float *adam_v,
                                  int step, const TrainHyper &hp, float *loss_out, float *grad_out,
                                  void *ws, hipStream_t s) {
    char *base = static_cast<char *>(ws);
    uint16_t *X = reinterpret_cast<uint16_t *>(base + p.off_x);
    float *H = reinterpret_cast<float *>(base + p.off_h);
    float *slope = reinterpret_cast<float *>(base + p.off_slope);
    float *SB = reinterpret_cast<float *>(base + p.off_sb);
    float *SA = reinterpret_cast<float *>(base + p.off_sa);
    float *rs = reinterpret_cast<float *>(base + p.off_rs);
    float *cs = reinterpret_cast<float *>(base + p.off_cs);
    float *E = reinterpret_cast<float *>(base + p.off_e);
    float *mu = reinterpret_cast<float *>(base + p.off_mu);
    float *gY = reinterpret_cast<float *>(base + p.off_gy);
    float *grad = reinterpret_cast<float *>(base + p.off_grad);
    double *colpart = reinterpret_cast<double *>(base + p.off_colpart);
    double *losspart = reinterpret_cast<double *>(base + p.off_losspart);
    const int n = p.n, r = p.r, nq = p.n_q, nk = p.n_k;
    hipError_t e;

    hipLaunchKernelGGL(k_concat, dim3(256), dim3(kThreads), 0, s, reinterpret_cast<const uint4 *>(q), nq,
                       reinterpret_cast<const uint4 *>(k), nk, reinterpret_cast<uint4 *>(X));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_label_sums, dim3(nq + (nk + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                       labels, nq, nk, rs, cs);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    GemmArgs g{};
    // codes and slopes: H = 2 sigmoid(sigma X W) - 1
    g = GemmArgs{};
    g.M = n; g.N = r; g.K = kHeadDim;
    g.A = X; g.a_m = kHeadDim; g.a_k = 1;
    g.B = w; g.b_k = r; g.b_n = 1;
    g.C = H; g.c_m = r; g.aux = slope; g.sigma = hp.sigma;
    if ((e = gemm<uint16_t, kEpiCodes>(g, s)) != hipSuccess) return e;
    // S B (queries' similarity pull) and S^T A (keys')
    g = GemmArgs{};
    g.M = nq; g.N = r; g.K = nk;
    g.A = labels; g.a_m = nk; g.a_k = 1;
    g.B = H + (int64_t)nq * r; g.b_k = r; g.b_n = 1;
    g.C = SB; g.c_m = r; g.alpha = 1.0f;
    if ((e = gemm<float, kEpiStore>(g, s)) != hipSuccess) return e;
    g = GemmArgs{};
    g.M = nk; g.N = r; g.K = nq;
    g.A = labels; g.a_m = 1; g.a_k = nk;
    g.B = H; g.b_k = r; g.b_n = 1;
    g.C = SA; g.c_m = r; g.alpha = 1.0f;
    if ((e = gemm<float, kEpiStore>(g, s)) != hipSuccess) return e;
    // E = H^T H / n - I
    g = GemmArgs{};
    g.M = r; g.N = r; g.K = n;
    g.A = H; g.a_m = 1; g.a_k = r;
    g.B = H; g.b_k = r; g.b_n = 1;
    g.C = E; g.c_m = r; g.alpha = 1.0f / (float)n;
    if ((e = gemm<float, kEpiCorr>(g, s)) != hipSuccess) return e;
    // column means and the loss
    hipLaunchKernelGGL(k_col_parts, dim3(p.n_parts), dim3(kThreads), 0, s, H, n, r, colpart);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_loss_parts, dim3(p.n_parts + 1), dim3(kThreads), 0, s, H, SB, rs, cs, E, nq, n, r,
                       losspart);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(kThreads), 0, s, colpart, p.n_parts, losspart, n, nq, r,
                       hp.epsilon, hp.eta, hp.lambda, mu, loss_out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dL/dY = slope o (eps dL_sim/dH + eta dL_bal/dH + lam (4 / n) H E)
    g = GemmArgs{};
    g.M = n; g.N = r; g.K = r;
    g.A = H; g.a_m = r; g.a_k = 1;
    g.B = E; g.b_k = r; g.b_n = 1;
    g.C = gY; g.c_m = r;
    g.H = H; g.slope = slope; g.SB = SB; g.SA = SA; g.rs = rs; g.cs = cs; g.mu = mu;
    g.n_q = nq; g.n = n; g.eps = hp.epsilon; g.eta = hp.eta; g.lam = hp.lambda;
    if ((e = gemm<float, kEpiGrad>(g, s)) != hipSuccess) return e;
    // dL/dW = X^T dL/dY
    g = GemmArgs{};
    g.M = kHeadDim; g.N = r; g.K = n;
    g.A = X; g.a_m = 1; g.a_k = kHeadDim;
    g.B = gY; g.b_k = r; g.b_n = 1;
    g.C = grad; g.c_m = r; g.alpha = 1.0f;
    if ((e = gemm<uint16_t, kEpiStore>(g, s)) != hipSuccess) return e;
    // Adam (step >= 1), or the gradient alone (step 0)
    const double c1 = step > 0 ? 1.0 / (1.0 - pow((double)hp.beta1, (double)step)) : 1.0;
    const double c2 = step > 0 ? 1.0 / (1.0 - pow((double)hp.beta2, (double)step)) : 1.0;
    const int64_t nw = (int64_t)kHeadDim * r;
    hipLaunchKernelGGL(k_adam, dim3((unsigned)((nw + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, w,
                       adam_m, adam_v, grad, nw, hp.lr, hp.beta1, hp.beta2, hp.adam_eps, (float)c1,
                       (float)c2, step > 0 ? 1 : 0, grad_out);
    return hipGetLastError();
}

}  // namespace hata
