/*
 * CPU oracle of the learning-to-hash objective that trains W_H (HATA).
 *
 * TEST INFRASTRUCTURE ONLY, like hata_oracle.c: only the tests, the smoke
 * check and the bench's CPU-baseline leg may load it; it shares nothing with
 * the GPU path.  Plain double-precision loops in the order the method states
 * its pieces, so that each can be checked by eye.
 *
 * What it follows (HATA review on pith.science, arXiv 2506.02572, "What
 * carries the argument" and "Assumptions & free parameters"; the labels as
 * the review's circularity check restates Section 3.1.2):
 *   - the relaxed hash h(x) = 2 Sigmoid(sigma x W_H) - 1, sigma = 0.1;
 *   - labels from qk scores: the top 10 % of a query's keys are positives
 *     with labels decaying linearly over [1, 20], every other key -1;
 *   - the objective: a similarity-weighted Hamming distance between query
 *     and key codes (weight epsilon = 0.01), a bit-balance penalty
 *     (eta = 2.0) and an uncorrelation penalty (lambda = 1.0).
 * The equations themselves (Eq. 7-9) are not printed on the pages; the
 * readings taken (each also listed in the design notes):
 *   - z_ji = q_j . k_i as a sequential double sum over d (bf16 products are
 *     exact in double); the keys of query j ranked by z descending, the lower
 *     index first among equal z; m = ceil(n_k / 10) positives; the key of rank
 *     t < m gets 20 - 19 t / (m - 1) (20 when m = 1), the rest -1;
 *   - D(a, b) = |a - b|^2 / 4, the relaxed Hamming distance (equal to the
 *     Hamming distance when a and b are +-1 codes);
 *   - L_sim = (1 / n_q) sum_j sum_i s_ji D(a_j, b_i) with a = h(q), b = h(k);
 *   - L_bal = sum_c mu_c^2, mu_c the mean of bit c over the n = n_q + n_k
 *     codes of the batch;
 *   - L_unc = |C - I|_F^2 with C = H^T H / n, H the n x r relaxed codes;
 *   - L = epsilon L_sim + eta L_bal + lambda L_unc;
 *   - the update: Adam (beta1 0.9, beta2 0.999, 1e-8), not named on the pages.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    double z;
    int32_t index;
} ranked_key;

static int by_z_desc_then_index(const void *a, const void *b) {
    const ranked_key *x = (const ranked_key *)a, *y = (const ranked_key *)b;
    if (x->z != y->z) return x->z > y->z ? -1 : 1;
    return x->index < y->index ? -1 : (x->index > y->index ? 1 : 0);
}

/*
 * Training labels.  q: bf16 [n_q][d]; k: bf16 [n_k][d].  labels: [n_q][n_k],
 * fully overwritten, each the float nearest to its double value.  Returns
 * 0, or -1 if memory runs out.
 */
int oracle_hash_labels(const uint16_t *q, int n_q, const uint16_t *k, int n_k, int d,
                       float *labels) {
    if (n_k <= 0) return 0;
    ranked_key *keys = (ranked_key *)malloc((size_t)n_k * sizeof *keys);
    if (!keys) return -1;
    const int m = (n_k + 9) / 10;
    for (int j = 0; j < n_q; ++j) {
        for (int i = 0; i < n_k; ++i) {
            double z = 0.0;
            for (int t = 0; t < d; ++t)
                z = z + bf16_to_double(q[(int64_t)j * d + t]) * bf16_to_double(k[(int64_t)i * d + t]);
            keys[i].z = z;
            keys[i].index = i;
        }
        qsort(keys, (size_t)n_k, sizeof *keys, by_z_desc_then_index);
        float *row = labels + (int64_t)j * n_k;
        for (int i = 0; i < n_k; ++i) row[i] = -1.0f;
        for (int t = 0; t < m; ++t) {
            double s = m == 1 ? 20.0 : 20.0 - 19.0 * (double)t / (double)(m - 1);
            row[keys[t].index] = (float)s;
        }
    }
    free(keys);
    return 0;
}

/*
 * Loss and gradient of the objective at W.  q: bf16 [n_q][d]; k: bf16
 * [n_k][d]; w: fp32 [d][r]; labels: fp32 [n_q][n_k].
 * loss_out[4] = (L, L_sim, L_bal, L_unc); grad: double [d][r], dL/dW.
 * Returns 0, or -1 if memory runs out.
 */
int oracle_hash_loss_grad(const uint16_t *q, int n_q, const uint16_t *k, int n_k, int d,
                          const float *w, int r, const float *labels, double sigma,
                          double epsilon, double eta, double lambda, double *loss_out,
                          double *grad) {
    const int n = n_q + n_k;
    double *x = (double *)malloc((size_t)n * d * sizeof(double));   /* [n][d]: queries, then keys */
    double *h = (double *)malloc((size_t)n * r * sizeof(double));   /* relaxed codes */
    double *dh = (double *)malloc((size_t)n * r * sizeof(double));  /* dh/dy */
    double *gh = (double *)calloc((size_t)n * r, sizeof(double));   /* dL/dh */
    double *mu = (double *)calloc((size_t)r, sizeof(double));
    double *cmat = (double *)calloc((size_t)r * r, sizeof(double));
    if (!x || !h || !dh || !gh || !mu || !cmat) {
        free(x); free(h); free(dh); free(gh); free(mu); free(cmat);
        return -1;
    }
    for (int v = 0; v < n; ++v)
        for (int t = 0; t < d; ++t)
            x[(int64_t)v * d + t] = v < n_q ? bf16_to_double(q[(int64_t)v * d + t])
                                            : bf16_to_double(k[(int64_t)(v - n_q) * d + t]);
    /* relaxed codes h = 2 sigmoid(sigma y) - 1 and their slope */
    for (int v = 0; v < n; ++v) {
        for (int c = 0; c < r; ++c) {
            double y = 0.0;
            for (int t = 0; t < d; ++t) y = y + x[(int64_t)v * d + t] * (double)w[(int64_t)t * r + c];
            double sg = 1.0 / (1.0 + exp(-sigma * y));
            h[(int64_t)v * r + c] = 2.0 * sg - 1.0;
            dh[(int64_t)v * r + c] = 2.0 * sigma * sg * (1.0 - sg);
        }
    }
    /* similarity term: every (query, key) pair */
    double l_sim = 0.0;
    for (int j = 0; j < n_q; ++j) {
        const double *a = h + (int64_t)j * r;
        for (int i = 0; i < n_k; ++i) {
            const double *b = h + (int64_t)(n_q + i) * r;
            const double s = (double)labels[(int64_t)j * n_k + i];
            double dist = 0.0;
            for (int c = 0; c < r; ++c) dist = dist + (a[c] - b[c]) * (a[c] - b[c]);
            l_sim = l_sim + s * dist / 4.0;
            /* d/da of s |a - b|^2 / 4 is s (a - b) / 2, and the opposite for b */
            for (int c = 0; c < r; ++c) {
                const double gc = epsilon * s * (a[c] - b[c]) / 2.0 / (double)n_q;
                gh[(int64_t)j * r + c] += gc;
                gh[(int64_t)(n_q + i) * r + c] -= gc;
            }
        }
    }
    l_sim = l_sim / (double)n_q;
    /* bit balance: the mean of each bit over the batch's codes */
    double l_bal = 0.0;
    for (int c = 0; c < r; ++c) {
        double s = 0.0;
        for (int v = 0; v < n; ++v) s = s + h[(int64_t)v * r + c];
        mu[c] = s / (double)n;
        l_bal = l_bal + mu[c] * mu[c];
    }
    for (int v = 0; v < n; ++v)
        for (int c = 0; c < r; ++c) gh[(int64_t)v * r + c] += eta * 2.0 * mu[c] / (double)n;
    /* uncorrelation: C = H^T H / n against the identity */
    double l_unc = 0.0;
    for (int c = 0; c < r; ++c) {
        for (int e = 0; e < r; ++e) {
            double s = 0.0;
            for (int v = 0; v < n; ++v) s = s + h[(int64_t)v * r + c] * h[(int64_t)v * r + e];
            const double dev = s / (double)n - (c == e ? 1.0 : 0.0);
            cmat[(int64_t)c * r + e] = dev;
            l_unc = l_unc + dev * dev;
        }
    }
    /* d/dH of |C - I|^2 is (4 / n) H (C - I) (C - I is symmetric) */
    for (int v = 0; v < n; ++v) {
        for (int c = 0; c < r; ++c) {
            double s = 0.0;
            for (int e = 0; e < r; ++e) s = s + h[(int64_t)v * r + e] * cmat[(int64_t)e * r + c];
            gh[(int64_t)v * r + c] += lambda * 4.0 * s / (double)n;
        }
    }
    /* through the sigmoid, then dL/dW = X^T dL/dY */
    for (int t = 0; t < d; ++t) {
        for (int c = 0; c < r; ++c) {
            double s = 0.0;
            for (int v = 0; v < n; ++v)
                s = s + x[(int64_t)v * d + t] * gh[(int64_t)v * r + c] * dh[(int64_t)v * r + c];
            grad[(int64_t)t * r + c] = s;
        }
    }
    loss_out[0] = epsilon * l_sim + eta * l_bal + lambda * l_unc;
    loss_out[1] = l_sim;
    loss_out[2] = l_bal;
    loss_out[3] = l_unc;
    free(x); free(h); free(dh); free(gh); free(mu); free(cmat);
    return 0;
}

/*
 * One Adam step on n parameters, in double: m = b1 m + (1 - b1) g,
 * v = b2 v + (1 - b2) g^2, w -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + e),
 * with t = step >= 1 the number of this update.
 */
void oracle_adam(double *w, double *m, double *v, const double *g, int64_t n, int step, double lr,
                 double b1, double b2, double e) {
    const double c1 = 1.0 - pow(b1, (double)step), c2 = 1.0 - pow(b2, (double)step);
    for (int64_t i = 0; i < n; ++i) {
        m[i] = b1 * m[i] + (1.0 - b1) * g[i];
        v[i] = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
        w[i] = w[i] - lr * (m[i] / c1) / (sqrt(v[i] / c2) + e);
    }
}
