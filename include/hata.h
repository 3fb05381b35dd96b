/*
 * hata.h -- C ABI of the MI355X (gfx950) hash-aware top-k decode-attention
 * library (libhata.so).
 *
 * The method (HATA: Trainable and Hardware-Efficient Hash-Aware Top-k
 * Attention, arXiv 2506.02572; review on pith.science, "What carries the
 * argument" and the Figure 2 caption with Algorithm 1): every cached key
 * and every query head is encoded to an r = 128-bit sign code
 * h(x) = sign(x W_H); the key codes are cached beside the KV cache
 * (rbit/32 = 4 words per key); at decode the query code is XORed against
 * every cached key code and popcounted into a Hamming score, the k keys of
 * lowest score are selected, and exact softmax attention runs over only
 * their K/V rows.
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must point to device memory that the
 *     caller owns and keeps alive until the stream has finished the call.
 *     The library never frees or retains them.
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL
 *     is the default stream).  No call allocates memory, synchronises the
 *     stream or reads device memory on the host, so the calls can be
 *     captured into a HIP graph.
 *   - Host-side argument checks return a status code; nothing aborts.  A
 *     non-OK status means nothing was enqueued.  Conditions only the device
 *     can see (a cache overflow, an out-of-range length) set bits in the
 *     cache's status word (HATA_DEV_*) and the affected batch entry is left
 *     unchanged or clamped as documented below.
 *   - Supported shapes: head_dim = 128, n_bits in {32, 64, 128, 256}, query
 *     heads a multiple G of KV heads with G in {1, 2, 4, 8}.  Other shapes
 *     return HATA_ERR_UNSUPPORTED.  Every code length (128 is the pages'
 *     choice; the others are their hash-length ablation, "Free
 *     parameters") runs the same single-launch decode.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Reentrant: the library keeps no mutable global state.  Calls that use
 *     the same cache or workspace must be ordered by the caller (same
 *     stream, or events).
 *
 * Code convention (a reading the pages leave open): bit j of a code is
 * [sum_d x_d * W_H[d][j] > 0] with the sum evaluated as a sequential
 * double-precision sum over d = 0..127 (each product is exact in double),
 * so a zero sum gives bit 0; bit j is stored in 32-bit word j / 32 at bit
 * position j % 32.  The GPU result is bit-identical to that definition:
 * fast products decide every bit whose margin is provably larger than
 * their error bound, and every other bit is recomputed in that exact order.
 */
#ifndef HATA_H
#define HATA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HATA_HEAD_DIM 128
#define HATA_N_BITS 128
#define HATA_CODE_WORDS 4

/* int32 words of the per-cache control block (see hata_cache.ctrl). */
#define HATA_CTRL_WORDS(batch, n_kv_heads) \
    (16 + 64 * ((int64_t)(batch) * (int64_t)(n_kv_heads) + (int64_t)(batch)))

typedef enum {
    HATA_OK = 0,
    HATA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad stride ... */
    HATA_ERR_UNSUPPORTED = 2, /* head_dim != 128, n_bits not in {32,64,128,256}, G not in {1,2,4,8} */
    HATA_ERR_WORKSPACE = 3,   /* workspace null or smaller than required */
    HATA_ERR_HIP = 4,         /* a HIP launch failed */
    HATA_ERR_SCRATCH_LIMIT = 5 /* hata_decode_step_static: the cache needs more than its scratch */
} hata_status;

/* Device status bits, OR-ed into ctrl[0] by kernels (sticky until the
 * caller clears them). */
#define HATA_DEV_APPEND_OVERFLOW 0x1 /* seq_len[b] + n_new[b] > max_ctx: entry b not appended */
#define HATA_DEV_BAD_LENGTH 0x2      /* seq_len[b] outside [0, max_ctx] at decode: clamped */
#define HATA_DEV_TOPK_CLAMPED 0x4    /* topk[b] > k_max at decode: clamped to k_max */
#define HATA_DEV_BAD_NEW 0x8         /* n_new[b] < 0 or > t_max at append: entry b skipped */
#define HATA_DEV_STALL 0x10          /* a decode wait timed out: outputs of that call invalid */

/*
 * Scheduling assumption of the decode (hata_decode_attn and
 * hata_decode_step, every code length).  The step is one kernel launch whose
 * workgroups hand results to each other: a work item waits for the query
 * codes of its (sequence, KV head) unit and, before it selects, for the
 * histogram counts of every other work item of that unit.  This needs those
 * other items to be running: workgroups start in block order and a unit's
 * items (at most 68: up to 4 query-code parts and 64 spans) fit on the GPU
 * together.  When the whole launch fits on
 * the GPU with 64 workgroup slots to spare, the items are also reordered for
 * balance, which needs every workgroup of the launch resident at once.  Both
 * hold on a GPU that no other kernel occupies while the step runs; kernels
 * running concurrently (other streams, other processes) that hold many CUs
 * can break them.  Every wait is bounded, so the launch always ends; if a
 * wait gave up, HATA_DEV_STALL is set in ctrl[0] and that call's outputs
 * (out, sel_idx_out, scores_out) are invalid.  The cache itself stays valid
 * (an appended row, its code and the new length are written as usual).
 * Recovery: zero-fill the workspace again, clear the status bit, and call
 * hata_decode_attn (no append) for the outputs.
 * Test control: the environment variable HATA_DECODE_WAIT_LIMIT, when set
 * to a number n below the built-in bounds, makes every such wait give up
 * after n re-reads, so that this path can be exercised.
 */

/*
 * A key/value cache with its key-code cache, all device memory owned by the
 * caller.  Sequence b, KV head g, position p:
 *   k, v  : bf16  [batch][n_kv_heads][max_ctx][128], row (b, g, p) at
 *           ((b * n_kv_heads + g) * max_ctx + p) * 128.  Device memory, or
 *           pinned host memory mapped into the device's address space
 *           (hipHostMalloc; pass its device address from
 *           hipHostGetDevicePointer): the offloaded layout of the HATA
 *           review ("offloaded" speed-ups in "Core claim"), where the codes,
 *           the scan and the selection stay in device memory and only the
 *           selected rows (and the appended ones) cross the host link.
 *   codes : u32   [batch][n_kv_heads][max_ctx][n_bits / 32]
 *   seq_len: int32 [batch], the number of valid positions of each sequence;
 *           positions [0, seq_len[b]) hold keys, values and codes.
 *   ctrl  : int32 [HATA_CTRL_WORDS(batch, n_kv_heads)], zero-filled by the
 *           caller once before first use; word 0 is the sticky device status
 *           (HATA_DEV_*); the other words are library counters that every
 *           call leaves at zero again.
 * This is the cache of Algorithm 1 in the Figure 2 caption of the review
 * (K_cache, V_cache, and the code cache of rbit/32 words per key).
 */
typedef struct {
    uint16_t *k;
    uint16_t *v;
    uint32_t *codes;
    int32_t *seq_len;
    int32_t *ctrl;
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim; /* must be 128 */
    int32_t n_bits;   /* 32, 64, 128 or 256 */
    int64_t max_ctx;
} hata_cache;

/*
 * Sign codes of a batch of key (or query) vectors: HashEncode(K) of
 * Algorithm 1 (Figure 2 caption of the review), h(x) = sign(x W_H).
 *   keys      device bf16; element (row n, head h, dim d) at
 *             keys[n * row_stride + h * head_stride + d] (strides in
 *             elements, d contiguous).
 *   n_rows    >= 0 rows; n_heads >= 1 heads, each with its own W_H.
 *   w_h       device fp32 [n_heads][128 (d)][128 (bit)].
 *   codes_out device u32 [n_rows][n_heads][4], fully overwritten.
 * Every bit is the exact sign of the code convention above.  From 64 rows
 * on (with keys 16-byte aligned and strides multiples of 8 elements) the
 * products run on the matrix cores, and every bit inside their error band is
 * recomputed; smaller or unaligned calls take the exact kernel.  The bits are
 * the same either way.
 * Errors: HATA_ERR_INVALID_ARG for null pointers (with n_rows > 0),
 * negative sizes or strides smaller than a row; HATA_ERR_HIP on launch
 * failure.
 */
hata_status hata_encode_keys(const uint16_t *keys, int64_t n_rows, int32_t n_heads,
                             int64_t row_stride, int64_t head_stride, const float *w_h,
                             uint32_t *codes_out, void *stream);

/*
 * hata_encode_keys for any supported code length r = n_bits (32, 64, 128 or
 * 256; the hash-length ablation of the review's "Free parameters"):
 *   w_h       device fp32 [n_heads][128 (d)][r (bit)].
 *   codes_out device u32 [n_rows][n_heads][r / 32].
 * Same bit convention and exactness.  For r != 128, keys must be 16-byte
 * aligned and both strides multiples of 8 elements (else
 * HATA_ERR_INVALID_ARG); r = 128 is hata_encode_keys itself.
 * Errors as hata_encode_keys, plus HATA_ERR_UNSUPPORTED for other n_bits.
 */
hata_status hata_encode_keys_nbits(const uint16_t *keys, int64_t n_rows, int32_t n_heads,
                                   int64_t row_stride, int64_t head_stride, const float *w_h,
                                   int32_t n_bits, uint32_t *codes_out, void *stream);

/*
 * Append new tokens to the cache (Algorithm 1's cache fill at prefill; one
 * token per sequence at decode): for each sequence b and t < n_new[b], key
 * row t of b goes to position seq_len[b] + t, its code is computed with the
 * KV head's W_H, and finally seq_len[b] += n_new[b].
 *   k_new, v_new device bf16 [batch][t_max][n_kv_heads][128] (token-major),
 *             or both NULL: the rows are already in the cache at
 *             [seq_len[b], seq_len[b] + n_new[b]) and only their codes are
 *             computed (encode in place).
 *   n_new     device int32 [batch], each in [0, t_max].
 *   t_max     host bound on n_new (sizes the launch); t_max = 0 is a no-op.
 *   w_h       device fp32 [n_kv_heads][128][n_bits].
 * Device-detected errors: an entry with seq_len[b] + n_new[b] > max_ctx is
 * not appended and sets HATA_DEV_APPEND_OVERFLOW; n_new[b] outside
 * [0, t_max] sets HATA_DEV_BAD_NEW and the entry is skipped.
 * Host errors: HATA_ERR_INVALID_ARG (null cache fields, exactly one of
 * k_new / v_new null, t_max < 0), HATA_ERR_UNSUPPORTED (shape).
 * From t_max >= 64 the codes are computed on the matrix cores (as in
 * hata_encode_keys; same bits).
 */
hata_status hata_append(const hata_cache *c, const uint16_t *k_new, const uint16_t *v_new,
                        const int32_t *n_new, int32_t t_max, const float *w_h, void *stream);

/* Bytes of device workspace hata_decode_attn / hata_decode_step need for
 * this cache: a function of batch, heads, max_ctx and n_bits (k_max only
 * has to be valid).  Returns 0 for an unsupported or invalid cache. */
size_t hata_decode_workspace_bytes(const hata_cache *c, int32_t k_max);

/*
 * One decode step of hash-aware top-k attention (the decode workflow of
 * Figure 2 in the review; TopK by Hamming distance as in its Algorithm 3,
 * referenced in the referee report):
 *   1. encode each query head with the W_H of its KV head
 *      (KV head of query head h = h / G);
 *   2. score every cached key i < seq_len[b] of KV head g by the sum over
 *      the group's G query heads of popcount(q_code XOR k_code[i])
 *      (range 0 .. n_bits G);
 *   3. select S = the k_eff = min(topk[b], k_max, seq_len[b]) keys of lowest
 *      (score, index) -- ties at the cut go to the lowest indices;
 *   4. for each query head: softmax over i in S of (q . k_i) / sqrt(128),
 *      output sum_i p_i v_i (fp32 accumulation), stored as bf16.
 *   q          device bf16 [batch][n_q_heads][128].
 *   w_h        device fp32 [n_kv_heads][128][n_bits].
 *   topk       device int32 [batch]; values < 0 count as 0, values above
 *              k_max are clamped (HATA_DEV_TOPK_CLAMPED).
 *   k_max      host upper bound of the budget, >= 0.
 *   out        device bf16 [batch][n_q_heads][128]; zero where k_eff = 0.
 *   workspace  device, >= hata_decode_workspace_bytes(c, k_max) bytes,
 *              256-byte aligned, zero-filled by the caller before its first
 *              use (and again after a call that set HATA_DEV_STALL).  It
 *              holds per-(sequence, KV head) launch counters that tag each
 *              call's intermediate results, so one workspace may serve
 *              several caches (layers) whose calls are ordered; the caller
 *              does not write it after the zero fill.
 *   sel_idx_out optional device int32 [batch][n_kv_heads][k_max]: the
 *              selected indices in ascending order, -1 after k_eff.
 *   scores_out optional device u16 [batch][n_kv_heads][max_ctx]: the
 *              summed Hamming scores of positions < seq_len[b].
 * Errors: HATA_ERR_INVALID_ARG, HATA_ERR_UNSUPPORTED, HATA_ERR_WORKSPACE,
 * HATA_ERR_HIP.
 */
hata_status hata_decode_attn(const hata_cache *c, const uint16_t *q, const float *w_h,
                             const int32_t *topk, int32_t k_max, uint16_t *out,
                             void *workspace, size_t ws_bytes, int32_t *sel_idx_out,
                             uint16_t *scores_out, void *stream);

/*
 * One whole decode step: append one token per sequence (as hata_append with
 * n_new[b] = 1 for every b), then hata_decode_attn over the grown context --
 * in a single kernel launch.
 *   k_new, v_new device bf16 [batch][n_kv_heads][128], the step's new key
 *                and value of every sequence.
 * A sequence whose cache is full (seq_len[b] == max_ctx) is not appended
 * (HATA_DEV_APPEND_OVERFLOW) and decodes over its existing context.  All
 * other arguments and errors as hata_decode_attn.
 */
hata_status hata_decode_step(const hata_cache *c, const uint16_t *k_new, const uint16_t *v_new,
                             const uint16_t *q, const float *w_h, const int32_t *topk,
                             int32_t k_max, uint16_t *out, void *workspace, size_t ws_bytes,
                             int32_t *sel_idx_out, uint16_t *scores_out, void *stream);

/*
 * hata_decode_step without a workspace argument, for callers that cannot
 * allocate device memory or hand one in: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The call allocates
 * nothing; the decode's scratch is a static device array of
 * HATA_STATIC_SCRATCH_BYTES inside the library (one per GPU, held until the
 * process ends; its address is looked up once per device on the first call
 * there).  Each call first clears the parts of that array that must start at
 * zero (a small fill kernel on `stream`), so calls may alternate between
 * caches of any shape; calls that overlap in time on one GPU (other streams,
 * other threads) share the array and race -- order them.
 * The array holds the decode workspace minus the score
 * rows of items longer than 8192 keys; caches whose layout needs more (for
 * example 64 sequences x 8 KV heads beyond 64K context) return
 * HATA_ERR_SCRATCH_LIMIT before anything is enqueued.  Arguments, results
 * and the other errors as hata_decode_step; the stall recovery (see the
 * scheduling note above) needs no workspace fill: the next call clears it.
 */
#define HATA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
hata_status hata_decode_step_static(const hata_cache *c, const uint16_t *k_new,
                                    const uint16_t *v_new, const uint16_t *q, const float *w_h,
                                    const int32_t *topk, int32_t k_max, uint16_t *out,
                                    int32_t *sel_idx_out, uint16_t *scores_out, void *stream);

/* Bytes of device workspace hata_exact_topk_recall needs for this cache
 * (depends on batch, heads and max_ctx only; about 17 bytes per position and
 * query head).  Returns 0 for an unsupported or invalid cache. */
size_t hata_recall_workspace_bytes(const hata_cache *c);

/*
 * Recall analysis of a Hamming selection -- the test the referee report of
 * the HATA review proposes ("What would settle it": compare the exact top-k
 * key set by q.k with the Hamming-selected one) and the tie analysis of its
 * major comment 1 (how many keys share the score at the cut).  Not part of
 * the decode step; call it after hata_decode_attn or hata_decode_step with
 * their debug outputs, on the same cache state and query.
 *   q          device bf16 [batch][n_q_heads][128], the step's query.
 *   topk, k_max as given to the decode call (k_eff = min(topk[b], k_max,
 *              seq_len[b]), topk < 0 counting as 0).
 *   sel_idx    device int32 [batch][n_kv_heads][k_max], the decode call's
 *              sel_idx_out.
 *   scores     device u16 [batch][n_kv_heads][max_ctx], its scores_out.
 *   overlap_out device int32 [batch][n_q_heads]: for query head h, the
 *              number of selected keys of its group that are in the exact
 *              top-k_eff of h.  The exact top-k ranks the keys i < seq_len[b]
 *              by z_i = sum_d q_d k_{i,d}, a sequential double sum over
 *              d = 0..127 (bf16 products are exact in double), largest
 *              first, the lower index first among equal z_i.
 *   tie_out    device int32 [batch][n_kv_heads][4]: (T, below, at, k_eff)
 *              with T the k_eff-th smallest Hamming score of the group,
 *              `below` the keys scoring under T and `at` the keys scoring T;
 *              (-1, 0, 0, 0) when k_eff = 0.
 *   exact_idx_out optional device int32 [batch][n_q_heads][k_max]: each
 *              query head's exact top-k indices in ascending order, -1 after
 *              k_eff.
 *   workspace  device, >= hata_recall_workspace_bytes(c) bytes, 256-byte
 *              aligned; no initial contents needed (scratch of this call).
 * The sets are identical to the definition above for finite inputs: fp32
 * estimates decide every key whose margin to the cut exceeds their proven
 * error bound, and the others are ranked on the exact double sums.
 * Errors: HATA_ERR_INVALID_ARG (null pointers, unaligned q, k_max < 0),
 * HATA_ERR_UNSUPPORTED, HATA_ERR_WORKSPACE, HATA_ERR_HIP.
 */
hata_status hata_exact_topk_recall(const hata_cache *c, const uint16_t *q, const int32_t *topk,
                                   int32_t k_max, const int32_t *sel_idx,
                                   const uint16_t *scores, int32_t *overlap_out,
                                   int32_t *tie_out, int32_t *exact_idx_out, void *workspace,
                                   size_t ws_bytes, void *stream);

/*
 * Training of the hash projection W_H: the learning-to-hash objective of the
 * HATA review ("What carries the argument": the relaxed code
 * h(x) = 2 Sigmoid(sigma x W_H) - 1 trained to minimise a similarity-weighted
 * Hamming distance between query and key codes plus bit-balance and
 * uncorrelation penalties; "Assumptions & free parameters": sigma = 0.1 and
 * the weights epsilon = 0.01, eta = 2.0, lambda = 1.0; the labels as its
 * circularity check restates them: the top 10 % of a query's keys by qk
 * score positive with labels decaying linearly over [1, 20], the rest -1).
 * The pages do not print the equations; the forms used (also in the oracle):
 *   L_sim = (1 / n_q) sum_j sum_i s_ji |h(q_j) - h(k_i)|^2 / 4,
 *   L_bal = sum_c (mean over the batch's n = n_q + n_k codes of bit c)^2,
 *   L_unc = |H^T H / n - I|_F^2 (H the n x r relaxed codes),
 *   L = epsilon L_sim + eta L_bal + lambda L_unc, and Adam updates.
 */
typedef struct {
    float sigma;    /* sigmoid scale of the relaxed code, 0.1 */
    float epsilon;  /* weight of L_sim, 0.01 */
    float eta;      /* weight of L_bal, 2.0 */
    float lambda;   /* weight of L_unc, 1.0 */
    float lr;       /* Adam step size */
    float beta1, beta2, adam_eps; /* Adam constants, e.g. 0.9, 0.999, 1e-8 */
} hata_train_params;

#define HATA_MAX_LABEL_KEYS 4096

/* Bytes of device workspace hata_hash_train_step needs (0 for unsupported
 * sizes: n_q and n_k must be positive multiples of 32, n_bits in
 * {32, 64, 128, 256}). */
size_t hata_hash_train_workspace_bytes(int32_t n_q, int32_t n_k, int32_t n_bits);

/*
 * Training labels of a batch.  q: device bf16 [n_q][128]; k: device bf16
 * [n_k][128] with n_k <= HATA_MAX_LABEL_KEYS; labels: device fp32
 * [n_q][n_k], fully overwritten.  For query j the keys are ranked by
 * z = q_j . k_i, a sequential double sum over d = 0..127 (bf16 products are
 * exact in double), larger z first and the lower index first among equal z;
 * with m = ceil(n_k / 10) the key of rank t < m gets 20 - 19 t / (m - 1)
 * (20 if m = 1), computed in double and rounded to float; every other key -1.
 * Inputs must be finite.  Errors: HATA_ERR_INVALID_ARG, HATA_ERR_HIP.
 */
hata_status hata_hash_labels(const uint16_t *q, int32_t n_q, const uint16_t *k, int32_t n_k,
                             float *labels, void *stream);

/*
 * One training step of W_H on a batch (all device pointers, 16-byte
 * aligned q and k):
 *   q, k      bf16 [n_q][128], [n_k][128]; n_q, n_k positive multiples of 32;
 *   labels    fp32 [n_q][n_k] (hata_hash_labels, or any labels);
 *   w_h       fp32 [128][n_bits], the weights; updated in place when step >= 1;
 *   adam_m, adam_v fp32 [128][n_bits], Adam's moments, zero before step 1
 *             (may be NULL when step = 0);
 *   step      0: loss and gradient only; t >= 1: then the t-th Adam update
 *             (bias corrections 1 - beta^t);
 *   params    host pointer to the hyperparameters;
 *   loss_out  fp32 [4]: (L, L_sim, L_bal, L_unc) at the weights before the
 *             update;
 *   grad_out  optional fp32 [128][n_bits]: dL/dW_H at those weights;
 *   workspace >= hata_hash_train_workspace_bytes(n_q, n_k, n_bits) bytes,
 *             256-byte aligned, no initial contents needed.
 * Every contraction runs on the matrix cores in fp32; sums over rows are
 * reduced in double in a fixed order (deterministic).
 * Errors: HATA_ERR_INVALID_ARG, HATA_ERR_UNSUPPORTED (n_bits),
 * HATA_ERR_WORKSPACE, HATA_ERR_HIP.
 */
hata_status hata_hash_train_step(const uint16_t *q, int32_t n_q, const uint16_t *k, int32_t n_k,
                                 const float *labels, int32_t n_bits, float *w_h, float *adam_m,
                                 float *adam_v, int32_t step, const hata_train_params *params,
                                 float *loss_out, float *grad_out, void *workspace,
                                 size_t ws_bytes, void *stream);

/* Static description of a status code (never NULL). */
const char *hata_status_string(hata_status s);

#ifdef __cplusplus
}
#endif

#endif /* HATA_H */
