/*
 * CPU oracle for the hash-aware top-k decode step (HATA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU path, and the GPU path never calls
 * it.  Plain, slow and direct on purpose: every step is written out in
 * double precision so that it can be checked against the method by eye.
 *
 * What it follows (HATA: Trainable and Hardware-Efficient Hash-Aware Top-k
 * Attention, arXiv 2506.02572, as reviewed on pith.science):
 *   - the hash h(x) = sign(x W_H) with r = 128 bits per head ("Free
 *     parameters": hash weight matrices W_H, hash length rbit = 128);
 *   - the key-code cache of rbit/32 32-bit words per key (Algorithm 1 in
 *     the caption of Figure 2);
 *   - the decode workflow: query code XOR every cached key code, popcount
 *     as the Hamming score, top-k lowest scores, exact attention over the
 *     selected K/V rows ("What carries the argument"; Referee report,
 *     major comment 1 on the TopK of Algorithm 3).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - sign(0) maps to bit 0: bit_j = [y_j > 0];
 *   - y_j is evaluated in double, summing over d in ascending order; each
 *     product bf16 x fp32 is exact in double;
 *   - bit j of a code lives in word j / 32 at position j % 32;
 *   - under grouped-query attention the G query heads of a KV head share
 *     its W_H and their Hamming distances are summed into one score per
 *     key; one selection serves the whole group;
 *   - ties at the cut are broken by the lowest key index; the selection
 *     is reported in ascending index order; k_eff = min(k, n);
 *   - attention logits are (q . k) / sqrt(d); softmax is exact in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Sign codes of n vectors.  x: bf16 bits, row i at x + i * x_stride,
 * d entries.  w: fp32 [d][r] (entry (t, j) at w[t * r + j]).  codes:
 * u32 [n][r / 32], fully overwritten.  Bit j of row i is 1 iff
 * sum_{t = 0..d-1} x[i][t] * w[t][j] > 0, the sum taken in double in
 * ascending t.
 */
void oracle_encode(const uint16_t *x, int64_t n, int64_t x_stride, int d,
                   const float *w, int r, uint32_t *codes) {
    int words = r / 32;
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t *row = x + i * x_stride;
        uint32_t *out = codes + i * words;
        for (int k = 0; k < words; ++k) out[k] = 0;
        for (int j = 0; j < r; ++j) {
            double y = 0.0;
            for (int t = 0; t < d; ++t)
                y = y + bf16_value(row[t]) * (double)w[(int64_t)t * r + j];
            if (y > 0.0) out[j / 32] |= (uint32_t)1 << (j % 32);
        }
    }
}

/*
 * Summed Hamming scores.  qcodes: u32 [G][r / 32] (the G query heads of
 * one group); kcodes: u32 [n][r / 32].  score[i] = sum over heads h and
 * bits j of [bit j of query h != bit j of key i], counted bit by bit.
 */
void oracle_hamming(const uint32_t *qcodes, int G, const uint32_t *kcodes, int64_t n, int r,
                    int32_t *score) {
    int words = r / 32;
    for (int64_t i = 0; i < n; ++i) {
        int32_t s = 0;
        for (int h = 0; h < G; ++h) {
            for (int j = 0; j < r; ++j) {
                uint32_t qb = (qcodes[h * words + j / 32] >> (j % 32)) & 1u;
                uint32_t kb = (kcodes[i * words + j / 32] >> (j % 32)) & 1u;
                if (qb != kb) s = s + 1;
            }
        }
        score[i] = s;
    }
}

typedef struct {
    int32_t score;
    int64_t index;
} scored_key;

static int by_score_then_index(const void *a, const void *b) {
    const scored_key *x = (const scored_key *)a, *y = (const scored_key *)b;
    if (x->score != y->score) return x->score < y->score ? -1 : 1;
    if (x->index != y->index) return x->index < y->index ? -1 : 1;
    return 0;
}

static int by_index(const void *a, const void *b) {
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

/*
 * Top-k lowest scores.  Sorts (score, index) ascending, keeps the first
 * k_eff = min(k, n) (k < 0 counts as 0), writes their indices in ascending
 * index order to idx[0..k_eff) and returns k_eff.  Returns -1 if memory
 * runs out.
 */
int64_t oracle_select(const int32_t *score, int64_t n, int64_t k, int64_t *idx) {
    int64_t k_eff = k < n ? k : n;
    if (k_eff <= 0) return 0;
    scored_key *all = (scored_key *)malloc((size_t)n * sizeof *all);
    if (!all) return -1;
    for (int64_t i = 0; i < n; ++i) {
        all[i].score = score[i];
        all[i].index = i;
    }
    qsort(all, (size_t)n, sizeof *all, by_score_then_index);
    for (int64_t i = 0; i < k_eff; ++i) idx[i] = all[i].index;
    free(all);
    qsort(idx, (size_t)k_eff, sizeof *idx, by_index);
    return k_eff;
}

/*
 * Exact softmax attention of G query vectors over the selected rows.
 * q: bf16 [G][d]; K, V: bf16 rows, row i at K + i * kv_stride; idx: m row
 * indices.  out: double [G][d].  For each head h:
 *   z_i = (sum_t q[h][t] * K[idx_i][t]) / sqrt(d),
 *   p_i = exp(z_i - max z) / sum_l exp(z_l - max z),
 *   out[h][t] = sum_i p_i * V[idx_i][t].
 * With m == 0 the output is zero.  Returns 0, or -1 if memory runs out.
 */
int oracle_attend(const uint16_t *q, int G, const uint16_t *K, const uint16_t *V,
                  int64_t kv_stride, int d, const int64_t *idx, int64_t m, double *out) {
    for (int64_t t = 0; t < (int64_t)G * d; ++t) out[t] = 0.0;
    if (m <= 0) return 0;
    double *z = (double *)malloc((size_t)m * sizeof *z);
    if (!z) return -1;
    double root_d = sqrt((double)d);
    for (int h = 0; h < G; ++h) {
        const uint16_t *qh = q + (int64_t)h * d;
        double zmax = -INFINITY;
        for (int64_t i = 0; i < m; ++i) {
            const uint16_t *krow = K + idx[i] * kv_stride;
            double dot = 0.0;
            for (int t = 0; t < d; ++t) dot = dot + bf16_value(qh[t]) * bf16_value(krow[t]);
            z[i] = dot / root_d;
            if (z[i] > zmax) zmax = z[i];
        }
        double denom = 0.0;
        for (int64_t i = 0; i < m; ++i) {
            z[i] = exp(z[i] - zmax);
            denom = denom + z[i];
        }
        double *oh = out + (int64_t)h * d;
        for (int64_t i = 0; i < m; ++i) {
            const uint16_t *vrow = V + idx[i] * kv_stride;
            double p = z[i] / denom;
            for (int t = 0; t < d; ++t) oh[t] = oh[t] + p * bf16_value(vrow[t]);
        }
    }
    free(z);
    return 0;
}

/*
 * The exact top-k of one query head, the comparison set that the referee
 * report of the HATA review asks for ("What would settle it": rank the keys
 * by their exact q.k scores and compare that top-k set with the Hamming
 * selection; major comment 1: exact top-k agreement).
 * q: bf16 [d]; K: bf16 rows, row i at K + i * kv_stride, n rows.
 *   z_i = sum_{t = 0..d-1} q[t] * K[i][t], a sequential double sum in
 *         ascending t (every product of two bf16 values is exact in double);
 *   the k_eff = min(k, n) keys of largest z_i are kept (k < 0 counts as 0),
 *   equal z_i going to the lower index; their indices are written to
 *   idx[0..k_eff) in ascending order.
 * Returns k_eff, or -1 if memory runs out.  The scale 1/sqrt(d) of the
 * logits does not change the order and is left out.
 */
typedef struct {
    double z;
    int64_t index;
} logit_key;

static int by_logit_desc_then_index(const void *a, const void *b) {
    const logit_key *x = (const logit_key *)a, *y = (const logit_key *)b;
    if (x->z != y->z) return x->z > y->z ? -1 : 1;
    if (x->index != y->index) return x->index < y->index ? -1 : 1;
    return 0;
}

int64_t oracle_exact_topk(const uint16_t *q, const uint16_t *K, int64_t kv_stride, int d,
                          int64_t n, int64_t k, int64_t *idx) {
    int64_t k_eff = k < n ? k : n;
    if (k_eff <= 0) return 0;
    logit_key *all = (logit_key *)malloc((size_t)n * sizeof *all);
    if (!all) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t *krow = K + i * kv_stride;
        double z = 0.0;
        for (int t = 0; t < d; ++t) z = z + bf16_value(q[t]) * bf16_value(krow[t]);
        all[i].z = z;
        all[i].index = i;
    }
    qsort(all, (size_t)n, sizeof *all, by_logit_desc_then_index);
    for (int64_t i = 0; i < k_eff; ++i) idx[i] = all[i].index;
    free(all);
    qsort(idx, (size_t)k_eff, sizeof *idx, by_index);
    return k_eff;
}
