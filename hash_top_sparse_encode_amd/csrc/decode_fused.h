// Decode step of hash-aware top-k attention on gfx950, as one kernel launch
// (HATA review, "What carries the argument": query code XOR every cached key
// code, popcount into a Hamming score, top-k, attention over the selected
// K/V; TopK by Hamming distance per the Algorithm 3 discussed in the referee
// report, major comment 1).
//
// Work items, one per workgroup, in block-index order:
//   PRO(u,p)   per unit u = (batch b, KV head g), four parts of 32 code
//              bits each: exact codes of the G query heads and of the step's
//              appended token, published as words tagged with the launch's
//              tag; part 0 also appends the K/V row.
//   WORK(u,c)  span c of the unit's keys (8192 keys, or a multiple of 8192
//              when a unit would need more than 64 items), in two phases:
//     scan     wave 0 polls the unit's tagged code words while waves 1-3
//              start the span's code stream (16-byte loads in 16 KB
//              sub-batches, four in flight); the group score of each key
//              from bit planes of the summed query codes (held in scalar
//              registers); scores kept in LDS (or the workspace for longer
//              spans) and counted into LDS sub-histograms of the 0..128G
//              range; the span's cumulative histogram published (tagged)
//              and its counts added into the unit histogram.
//     select   the span's candidates (scores up to a cut read off its own
//              histogram) are listed while the unit's other items finish;
//              once the unit histogram is complete (its counts sum to the
//              context length), the cut score T (first bin whose cumulative
//              count reaches k_eff) and, from the earlier spans' cumulative
//              histograms, the below-T and score-T keys before this span
//              (which fixes how many score-T keys it keeps: the lowest
//              indices win); the selection is then taken from the
//              candidates (or, if T lies above their cut, from all scores);
//     attend   gather of the selected bf16 K/V rows (V straight into LDS),
//              logits of 16-key tiles on the matrix cores, an online softmax
//              in base 2, P.V on the matrix cores as well; one (m, l, o)
//              partial per query head.  The last item of a unit to finish
//              merges the partials in item order into the bf16 output and
//              resets the unit's state.
//
// Ordering: a PRO part waits for nothing; a WORK item's scan waits for the
// PRO parts of its unit (smaller block indices), and its selection for the
// scans of every WORK item of its unit.  Workgroups of a grid are dealt to
// the eight XCDs in turn (block b to XCD b mod 8) and started in block order
// within each XCD, and a finished workgroup frees its slot.  Take the
// smallest unfinished block X: if X is WORK(u, c), the PRO parts of unit u
// (earlier blocks) are done, every workgroup that started after the
// finished ones holds an item of unit u or a later one, and the unit's
// unstarted items (at most 63) are the next in line on their XCDs; an XCD
// holds at least 64 of these workgroups at once (32 CUs x 2 or 3), so they
// all start, all scan, and unit u completes.  (When every unit's last item is moved to the end of the
// grid, see item_of, the host has checked that every workgroup of the launch
// is resident at once, so no wait depends on a workgroup yet to start.)
// Every wait also gives up after a bound (HATA_DEV_STALL), so the kernel
// always terminates, and no result depends on where a workgroup runs.  A
// unit's consecutive items land on different XCDs, which spreads each
// unit's traffic over all of them (keeping each unit on one XCD was
// measured slower: every XCD's share of the memory bandwidth is capped).
//
// Coherence across the eight XCDs without cache flushes: every value one
// workgroup produces for another is written with a device-scope relaxed
// atomic store (write-through, "sc1") or atomic add and read with
// device-scope atomic loads ("sc1"), which are served by the
// device-coherent level.  Readers need no separate "ready" counter: the
// PRO code words and the per-span cumulative histograms carry a tag (the
// unit's launch count on this workspace, plus one), so a reader re-reads
// until every word it uses carries this launch's tag, and the unit
// histogram is complete exactly when its counts sum to the context length.
// Only the split partials are published behind a counter (stores drained,
// then one atomic add), for the merge.  An agent-scope fence would write
// back / invalidate whole L2s instead, which costs more than the step.
#pragma once

#include "device_util.h"
#include "hata_internal.h"
#include "../../include/hata.h"

namespace hata {

constexpr int kThreads = 256;
constexpr int kSpanUnit = 8192;    // a work item's span of keys is a multiple of this
constexpr int kSub = 4;            // keys per thread in one sub-batch of code loads (1024 per workgroup)
constexpr int kMaxSplits = 64;     // work items per unit, at most (the merge width)
constexpr int kSelRound = 2048;    // 8 scores per thread per selection round
constexpr int kSelRounds = 4;      // selection rounds per batch (scores prefetched together)
constexpr int kListCap = kSelRounds * kSelRound;  // selected indices buffered in LDS
constexpr int kSpinLimit = 1 << 22;
constexpr int kPollLimit = 1 << 18;  // block-wide polls (each a full re-read)
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint16_t kNoScore = 0xFFFF;

typedef float fvec4 __attribute__((ext_vector_type(4)));
typedef uint32_t uvec4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


// per-unit counter words
constexpr int kAttn = 0, kNumCtr = 1;
// Bins of every earlier item's cumulative histogram read, ending at the
// candidate cut, along with the unit histogram.
constexpr int kWin = 8;
constexpr int kUnitWords = 64;  // one 256-byte line per unit (and per batch entry)

struct FusedArgs {
    uint16_t *k_cache;
    uint16_t *v_cache;
    uint32_t *codes;
    int32_t *seq_len;
    int32_t *ctrl;
    const uint16_t *k_new;  // [B][Hkv][128] or null (no append)
    const uint16_t *v_new;
    const uint16_t *q;
    const float *w;
    const int32_t *topk;
    uint16_t *out;
    int32_t *sel_out;        // optional debug output
    uint16_t *scores_dbg;    // optional debug output, row stride max_ctx
    uint16_t *scores;        // workspace, row stride sstride
    uint32_t *gen;           // per unit: launches completed on this workspace (tags are gen + 1)
    uint64_t *qtag;          // per unit: (G + 1) x 4 tagged code words (query heads, appended key)
    uint32_t *unit_hist;     // per unit: 128 G + 2 words (bins in pairs)
    uint64_t *chunk_hist;    // per unit and work item: tagged cumulative counts, 128 G + 1 bins
    float *part_ml;
    float *part_o;
    int64_t max_ctx;
    int64_t sstride;
    int B, Hkv, k_max;
    int64_t span;            // keys per work item
    int n_chunks;            // work items per unit
    int tails_last;          // every unit's last work item after all the others (see item_of)
    int resident;            // the whole grid fits on the chip at once (see item_of)
    int n_items;
    int spin_limit;          // bound of the query-code wait (re-reads by one wave)
    int poll_limit;          // bound of the histogram waits (block-wide re-reads)
    uint64_t *trace;         // phase timestamps (HATA_PHASE_TRACE builds), null: none
    int trace_items;         // workgroups the trace buffer has rows for
};

// Phase timestamps: in builds with HATA_PHASE_TRACE (libhata_trace.so),
// thread 0 of each workgroup writes the 100 MHz real-time clock at each of
// these points into trace[block][phase] (16 words per block), and the item
// it runs into word 15 (kind << 31 | unit << 8 | part or span).  Other
// builds compile the markers to nothing.
enum Phase {
    kPhStart = 0,      // first instruction
    kPhCodes = 1,      // PRO: code words published; WORK: query codes in LDS
    kPhScanned = 2,    // WORK: the span's scores counted
    kPhPublished = 3,  // WORK: histograms published
    kPhListed = 4,     // WORK: candidates listed
    kPhCut = 5,        // WORK: the unit's cut T known
    kPhTies = 6,       // WORK: the earlier items' below-T and score-T counts known
    kPhSelected = 7,   // WORK: the span's selection made (attention starts)
    kPhAttended = 8,   // WORK: attention done
    kPhPartial = 9,    // WORK: partial stored and counted
    kPhMerged = 10,    // the unit's last item: every partial read
    kPhEnd = 11,       // the workgroup's item done
    kPhItem = 15,
};
#ifdef HATA_PHASE_TRACE
#define HATA_PHASE(a, k)                                                                        \
    do {                                                                                        \
        if ((a).trace && threadIdx.x == 0 && (int)blockIdx.x < (a).trace_items)                 \
            (a).trace[(int64_t)blockIdx.x * 16 + (k)] = __builtin_amdgcn_s_memrealtime();        \
    } while (0)
// A diagnostic word of the workgroup's item in a trace slot of its own: 12
// the earlier spans' counts (bit 0 window hit, bit 1 read again, T from bit
// 8, tc from bit 20, the candidate count from bit 32), 13 the selected count
// (bit 30: taken from all scores), 14 the polls until the unit histogram was
// complete.
#define HATA_TRACE_WORD(a, k, v)                                                                \
    do {                                                                                        \
        if ((a).trace && threadIdx.x == 0 && (int)blockIdx.x < (a).trace_items)                 \
            (a).trace[(int64_t)blockIdx.x * 16 + (k)] = (uint64_t)(v);                          \
    } while (0)
#else
#define HATA_PHASE(a, k) \
    do {                 \
    } while (0)
#define HATA_TRACE_WORD(a, k, v) \
    do {                         \
    } while (0)
#endif

// ---------------------------------------------------------------- coherent access

__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float *p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t *>(p),
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ int add_dev(int32_t *p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this thread's memory operations have completed.
__device__ __forceinline__ void drain_memory() { __builtin_amdgcn_s_waitcnt(0); }

// A value known to be the same in every lane, moved to a scalar register
// (values read from LDS or reduced across the block are otherwise kept per
// lane).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- small helpers

__device__ __forceinline__ int64_t clamp_len(int64_t v, int64_t hi) {
    return v < 0 ? 0 : (v > hi ? hi : v);
}

// Context of batch entry b for this step.  seq_len is only rewritten once
// every item of the entry has finished, so all items see the same l0.
struct StepLen {
    int64_t l0;   // length before the append
    int64_t len;  // length this step attends over
    bool app;     // the step's token is appended at l0
};

__device__ __forceinline__ StepLen step_len(const FusedArgs &a, int b) {
    StepLen s;
    s.l0 = clamp_len(a.seq_len[b], a.max_ctx);
    s.app = a.k_new != nullptr && s.l0 + 1 <= a.max_ctx;
    s.len = s.l0 + (s.app ? 1 : 0);
    return s;
}

__device__ __forceinline__ int64_t step_keff_of(const FusedArgs &a, int64_t k, int64_t len) {
    if (k < 0) k = 0;
    if (k > a.k_max) k = a.k_max;
    return k < len ? k : len;
}

__device__ __forceinline__ int32_t *unit_ctr(const FusedArgs &a, int u, int which) {
    return a.ctrl + kCtrlUnitBase + kUnitWords * u + which;
}
__device__ __forceinline__ int32_t *batch_ctr(const FusedArgs &a, int b) {
    return a.ctrl + kCtrlUnitBase + kUnitWords * (a.B * a.Hkv + b);
}

// Every thread's device-scope stores complete, then thread 0 counts.
// Returns the counter's previous value (in thread 0).
__device__ __forceinline__ int wg_signal(int32_t *p) {
    drain_memory();
    __syncthreads();
    int prev = 0;
    if (threadIdx.x == 0) prev = add_dev(p, 1);
    return prev;
}

__device__ __forceinline__ void unpack_bf16x4(uint64_t r, float (&f)[4]) {
    const uint32_t lo = (uint32_t)r, hi = (uint32_t)(r >> 32);
    f[0] = __uint_as_float(lo << 16);
    f[1] = __uint_as_float(lo & 0xFFFF0000u);
    f[2] = __uint_as_float(hi << 16);
    f[3] = __uint_as_float(hi & 0xFFFF0000u);
}

// ---------------------------------------------------------------- shared memory

// A work item's two phases share memory.  Both begin with the span's scores
// (kept in LDS between the phases when the span is kSpanUnit keys).
template <int G, int R>
struct SmemScan {
    static constexpr int NB = G * R + 1;
    // sub-histograms: each wave counts into NH / 4 of them by lane, which
    // keeps equal scores of one instruction apart (LDS atomics on one address
    // serialise); at most 32 KB of them
    static constexpr int NH = NB <= 513 ? 16 : NB <= 1025 ? 8 : 4;
    uint16_t scores[kSpanUnit];
    uint32_t hist[NH][NB];
    int scan[4];
    uint32_t qc[G * (R / 32)];  // the unit's query codes, fetched by wave 0
    uint32_t app[R / 32];       // the appended key's code (when in this span)
    int tc;                   // candidate cut of the span (see slot_publish)
    uint32_t gen;             // the unit's launch generation
};

template <int G>
struct SmemSel {
    union {
        uint16_t scores[kSpanUnit];    // the span's scores, until the selection is made
        uint16_t vst[4][32][kHeadDim]; // attention: each wave's V rows of a round
        struct {
            float wm[4][G];
            float wl[4][G];
            float wo[4][G][kHeadDim];
        } cb;                          // after the attention: each wave's (m, l, o)
    };
    uint16_t list[kListCap];  // selected keys of a batch, as offsets from its first key
    uint16_t pb[4][2][G][32]; // per wave: softmax numerators as bf16 high and low parts
    int scan[8];
    int weq[4], wlt[4];  // per-wave counts of score-T and below-T keys in a batch
    int red[8];
    int T, below, cntT, last;
};

// Whether an item's own summed and cumulative histograms (scan.hist[0] and
// [1]) are still intact when its earlier spans' counts are needed: the
// selection phase writes its list (and the attention its staging rows) over
// the rest of the scan state first.
template <int G, int R>
constexpr bool own_hist_kept() {
    using Scan = SmemScan<G, R>;
    using Sel = SmemSel<G>;
    return __builtin_offsetof(Scan, hist) + 2 * sizeof(uint32_t) * (G * R + 1) <= __builtin_offsetof(Sel, list);
}

// PRO parts per unit: one per 32 code bits up to 128 bits; at 256 bits four
// parts of 64 bits each, so that the step's grid (with 17 spans a unit at
// 128K context) still fits on the chip at once.
__host__ __device__ constexpr int pro_parts(int r) { return r >= 256 ? 4 : r / 32; }
template <int R>
constexpr int pro_groups() { return R / 32 / pro_parts(R); }  // 32-column groups per part

template <int G, int R>
struct SmemPro {
    float x[G + 1][kHeadDim];                   // query heads, then the appended key or zeros
    float w[pro_groups<R>()][kHeadDim][32];     // this part's columns of W_H, 32 per group
    float py[4][G + 1][32];                     // per-wave partial sums
    float pa[4][G + 1][32];                     // per-wave partial sums of |products|
};

template <int G, int R>
union Smem {
    SmemScan<G, R> scan;
    SmemSel<G> sel;
    SmemPro<G, R> pro;
};

// ---------------------------------------------------------------- PRO(u)

// Part p of unit u computes code bits [32 NG p, 32 NG (p + 1)) of the G
// query heads and of the appended key (NG = pro_groups: one group of 32, two
// at 256 bits, one after the other); part 0 also copies the appended K/V
// rows and writes the outputs of an empty selection.
//
// Each bit is sign(y) with y = sum_t x[t] W[t][j] evaluated as a sequential
// double sum in ascending t (bf16 x fp32 products are exact in double).
// Fast path in fp32: sixteen-row segments summed by fused multiply-adds
// (the product is exact inside each), then combined in a fixed tree -- at
// most 18 roundings deep -- alongside A = sum |x[t] W[t][j]| formed the same
// way.  The fp32 result lies within gamma_18 A (u = 2^-24; about 2^-19.7 A)
// of the exact sum, and the sequential double sum within gamma_127 A
// (u = 2^-53) of it (Higham, Accuracy and Stability of Numerical Algorithms,
// ch. 4); products or sums that underflow add at most 2^-119 in all.  So
// when |y_f32| > 2^-16 A_f32 + 2^-100 the exact sum and the double sum both
// have its sign.  Any other bit (including non-finite inputs, which fail
// the test) is recomputed by the sequential double sum.
template <int G, int R>
__device__ __forceinline__ void item_pro(const FusedArgs &a, int u, int part, Smem<G, R> &sm) {
    constexpr int COLS = 32;
    constexpr int NG = pro_groups<R>();
    constexpr int W = R / 32;
    constexpr int NV = G + 1;                // query heads + appended key
    const int b = u / a.Hkv, kv = u % a.Hkv, Hq = a.Hkv * G;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    // Every load the part needs is issued before any is used, so they share
    // one round trip: its 128 x 32 NG slice of W_H (16 bytes per load), the x
    // rows (query heads, then the token's key: one 16-byte load per thread,
    // 16 threads per row), the unit's generation and the entry's length, and
    // for part 0 the top-k and the token's K/V words to append.
    constexpr int WQ = kHeadDim * COLS / 4 / kThreads;  // 4 per group
    fvec4 wq[NG][WQ];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const float *wk = a.w + (int64_t)kv * kHeadDim * R + (part * NG + g) * COLS;
#pragma unroll
        for (int r = 0; r < WQ; ++r) {
            const int f = r * kThreads + t;  // row f / 8, four columns at 4 (f % 8)
            wq[g][r] = *reinterpret_cast<const fvec4 *>(wk + (f >> 3) * R + 4 * (f & 7));
        }
    }
    // (Loads are issued by every lane, those with nothing to load reading the
    // unit's first query row, so that no branch separates them.)
    const int xv = t >> 4, d0 = (t & 15) * 8;
    const int64_t src = ((int64_t)b * a.Hkv + kv) * kHeadDim;
    const uint16_t *qrow = a.q + ((int64_t)b * Hq + kv * G) * kHeadDim;
    const uint16_t *xp = xv < G ? qrow + xv * kHeadDim + d0
                                : (xv == G && a.k_new ? a.k_new + src + d0 : qrow);
    const uint4 xr = *reinterpret_cast<const uint4 *>(xp);
    // the new K and V rows: 32 + 32 eight-byte words (threads 0-63)
    const uint16_t *kvp = t < 64 && a.k_new ? (t < 32 ? a.k_new + src + 4 * t : a.v_new + src + 4 * (t - 32)) : qrow;
    const uint64_t kvw = *reinterpret_cast<const uint64_t *>(kvp);
    const int32_t topk_b = a.topk[b];
    const uint32_t tag = ld_dev(a.gen + u) + 1u;
    const int64_t raw = a.seq_len[b];
    StepLen sl;
    sl.l0 = clamp_len(raw, a.max_ctx);
    sl.app = a.k_new != nullptr && sl.l0 + 1 <= a.max_ctx;
    sl.len = sl.l0 + (sl.app ? 1 : 0);
    const int nvec = G + (sl.app ? 1 : 0);
    if (t < NV * 16) {
        const uint32_t wds[4] = {xr.x, xr.y, xr.z, xr.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sm.pro.x[xv][d0 + 2 * e] = __uint_as_float(wds[e] << 16);
            sm.pro.x[xv][d0 + 2 * e + 1] = __uint_as_float(wds[e] & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        fvec4 *wl = reinterpret_cast<fvec4 *>(&sm.pro.w[g][0][0]);
#pragma unroll
        for (int r = 0; r < WQ; ++r) wl[r * kThreads + t] = wq[g][r];
    }
    // Part 0's stores: nothing in this launch waits for them (the unit's
    // attention reads the token's K/V from k_new / v_new, and its code word
    // from the published words), so they are issued and left in flight.
    if (part == 0) {
        const int64_t k_eff = step_keff_of(a, topk_b, sl.len);
        if (kv == 0 && t == 0) {
            int flags = 0;
            if (raw < 0 || raw > a.max_ctx) flags |= HATA_DEV_BAD_LENGTH;
            if (a.k_new != nullptr && !sl.app) flags |= HATA_DEV_APPEND_OVERFLOW;
            if (topk_b > a.k_max) flags |= HATA_DEV_TOPK_CLAMPED;
            if (flags) atomicOr(&a.ctrl[kCtrlStatus], flags);
        }
        if (sl.app && t < 64) {
            const int64_t row = (int64_t)u * a.max_ctx + sl.l0;
            if (t < 32) st_dev(reinterpret_cast<uint64_t *>(a.k_cache + row * kHeadDim) + t, kvw);
            else st_dev(reinterpret_cast<uint64_t *>(a.v_cache + row * kHeadDim) + (t - 32), kvw);
        }
        if (a.sel_out) {
            int32_t *su = a.sel_out + (int64_t)u * a.k_max;
            for (int64_t p = k_eff + t; p < a.k_max; p += kThreads) su[p] = -1;
        }
        if (k_eff == 0) {
            for (int i = t; i < G * kHeadDim; i += kThreads)
                a.out[((int64_t)b * Hq + kv * G) * kHeadDim + i] = 0;
        }
    }
#pragma unroll 1
    for (int g = 0; g < NG; ++g) {
        // the staged rows (and, after the first group, every read of the
        // previous group's partials)
        __syncthreads();
        // Segment sums: lane col = lane & 31 of wave w covers rows
        // [16 seg, 16 seg + 16) with seg = 2 w + (lane >> 5).
        {
            const int col = lane & 31, seg = 2 * wv + (lane >> 5);
            float ys[NV], as[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                ys[v] = 0.f;
                as[v] = 0.f;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 16 * seg + r;
                const float wf = sm.pro.w[g][row][col];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const float xf = sm.pro.x[v][row];
                    ys[v] = fmaf(xf, wf, ys[v]);
                    as[v] = fmaf(fabsf(xf), fabsf(wf), as[v]);
                }
            }
            // pair the wave's two segments, then park the wave's partials
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const float yo = __shfl_xor(ys[v], 32, 64), ao = __shfl_xor(as[v], 32, 64);
                if (lane < 32) {
                    sm.pro.py[wv][v][col] = ys[v] + yo;  // lower segment first
                    sm.pro.pa[wv][v][col] = as[v] + ao;
                }
            }
        }
        __syncthreads();
        // Decide bit (v, col) for v = t >> 5 (and v = 8 + (t >> 5) on a second
        // pass for G = 8): tree over the four waves, then the sign test.
#pragma unroll
        for (int pass = 0; pass < (NV + 7) / 8; ++pass) {
            const int v = pass * 8 + (t >> 5), col = t & 31;
            bool bit = false;
            if (v < NV) {
                const float y = (sm.pro.py[0][v][col] + sm.pro.py[1][v][col]) +
                                (sm.pro.py[2][v][col] + sm.pro.py[3][v][col]);
                const float A = (sm.pro.pa[0][v][col] + sm.pro.pa[1][v][col]) +
                                (sm.pro.pa[2][v][col] + sm.pro.pa[3][v][col]);
                if (fabsf(y) > fmaf(0x1p-16f, A, 0x1p-100f)) {
                    bit = y > 0.f;
                } else {
                    double ysq = 0.0;  // the defining sequential sum
                    for (int row = 0; row < kHeadDim; ++row)
                        ysq = fma((double)sm.pro.x[v][row], (double)sm.pro.w[g][row][col], ysq);
                    bit = ysq > 0.0;
                }
            }
            const uint64_t mb = __ballot(bit);
            if ((t & 31) == 0 && v < NV && sl.len > 0) {
                const uint32_t word = v < nvec ? (uint32_t)(((t >> 5) & 1) ? (mb >> 32) : mb) : 0u;
                st_dev(a.qtag + ((int64_t)u * NV + v) * W + part * NG + g, ((uint64_t)tag << 32) | word);
                if (v == G && sl.app) st_dev(a.codes + ((int64_t)u * a.max_ctx + sl.l0) * W + part * NG + g, word);
            }
        }
    }
    HATA_PHASE(a, kPhCodes);
}

// ---------------------------------------------------------------- scanners

// The group score of a key, sum over the G query heads of
// popcount(qcode_h XOR kcode), from the query codes summed bit by bit.  For
// code bit j let c_j (0..G) count the heads with bit j set: the key adds
// k_j ? G - c_j : c_j.  With G = 2^m, that per-bit value d_j has the bit
// planes
//   d_0 = c_0                                  (G - c and c share parity),
//   d_i = c_i ^ (k & (c_0 | .. | c_{i-1}))    for 0 < i < m (negation flips
//                                              the bits above the lowest set one),
//   d_m = k ? [c_j == 0] : c_m,
// so the score is popcount(c_0) + sum_i 2^i popcount(d_i).  For G = 4 that
// is five lane operations per code word instead of eight.
template <int G, int W>
struct QPlanes {
    static constexpr int M = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;  // G = 2^M
    static constexpr int NP = G == 1 ? 1 : G == 2 ? 2 : G == 4 ? 4 : 6;
    uint32_t p[NP][W];  // per code word; see query_planes
    int c0sum;          // popcount of the c_0 plane over the code
};

// A key's code: W 32-bit words (bit j in word j / 32).
template <int W>
struct KeyCode {
    uint32_t w[W];
};

// Planes of the query codes (uniform values, kept in scalar registers):
//   G = 1: {q}              G = 2: {c_1, z}
//   G = 4: {c_0, c_1, c_2, z}     G = 8: {c_0, c_1, c_0 | c_1, c_2, c_3, z}
// with z the bits where no head is set.
template <int G, int W>
__device__ __forceinline__ void query_planes(const uint32_t (&qc)[G][W], QPlanes<G, W> &qp) {
    constexpr int M = QPlanes<G, W>::M;
    qp.c0sum = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        uint32_t c[M + 1];
#pragma unroll
        for (int i = 0; i <= M; ++i) c[i] = 0u;
#pragma unroll
        for (int h = 0; h < G; ++h) {  // ripple-carry add of head h's bits
            uint32_t carry = qc[h][w];
#pragma unroll
            for (int i = 0; i <= M; ++i) {
                const uint32_t nc = c[i] ^ carry;
                carry &= c[i];
                c[i] = nc;
            }
        }
        uint32_t any = 0u;
#pragma unroll
        for (int i = 0; i <= M; ++i) any |= c[i];
        const uint32_t z = ~any;
        if constexpr (G == 1) {
            qp.p[0][w] = c[0];
        } else {
            qp.c0sum += __popc(c[0]);
            if constexpr (G == 2) {
                qp.p[0][w] = c[1];
                qp.p[1][w] = z;
            } else if constexpr (G == 4) {
                qp.p[0][w] = c[0];
                qp.p[1][w] = c[1];
                qp.p[2][w] = c[2];
                qp.p[3][w] = z;
            } else {
                qp.p[0][w] = c[0];
                qp.p[1][w] = c[1];
                qp.p[2][w] = c[0] | c[1];
                qp.p[3][w] = c[2];
                qp.p[4][w] = c[3];
                qp.p[5][w] = z;
            }
        }
    }
}

template <int G, int W>
__device__ __forceinline__ int group_hamming(const KeyCode<W> &k, const QPlanes<G, W> &qp) {
    if constexpr (G == 1) {
        int s = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) s += __popc(k.w[w] ^ qp.p[0][w]);
        return s;
    } else {
        int p1 = 0, p2 = 0, p3 = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const uint32_t x = k.w[w];
            if constexpr (G == 2) {
                p1 += __popc((x & qp.p[1][w]) | (~x & qp.p[0][w]));
            } else if constexpr (G == 4) {
                p1 += __popc(qp.p[1][w] ^ (x & qp.p[0][w]));
                p2 += __popc((x & qp.p[3][w]) | (~x & qp.p[2][w]));
            } else {
                p1 += __popc(qp.p[1][w] ^ (x & qp.p[0][w]));
                p2 += __popc(qp.p[3][w] ^ (x & qp.p[2][w]));
                p3 += __popc((x & qp.p[5][w]) | (~x & qp.p[4][w]));
            }
        }
        return qp.c0sum + 2 * p1 + 4 * p2 + 8 * p3;
    }
}

// Sub-batches of code loads in flight per workgroup: about 64 KB, and no
// more than the eight sub-batches of a span of kSpanUnit keys.
template <int R>
constexpr int scan_depth() { return R >= 64 ? 512 / R : 8; }

// Work item c of unit u: keys [c span, min((c + 1) span, len)).
struct Slot {
    int u, c;
    int64_t p0, p1;  // key range, empty if p0 >= p1
    StepLen sl;
    int64_t k_eff;   // the entry's top-k, clamped to [0, min(k_max, len)]
};

// The item's span within its cache row, before the entry's length is known
// (so its first code loads can be issued at once).
__device__ __forceinline__ Slot slot_row(const FusedArgs &a, int u, int c) {
    Slot s;
    s.u = u;
    s.c = c;
    s.p0 = (int64_t)c * a.span;
    s.p1 = s.p0 + a.span < a.max_ctx ? s.p0 + a.span : a.max_ctx;
    s.k_eff = 0;
    return s;
}

// The entry's length and top-k: the span cut to the length, k_eff.
__device__ __forceinline__ void slot_len(const FusedArgs &a, Slot &s) {
    const int b = s.u / a.Hkv;
    const int32_t topk_b = a.topk[b];
    s.sl = step_len(a, b);
    s.p1 = s.p0 + a.span < s.sl.len ? s.p0 + a.span : s.sl.len;
    s.k_eff = step_keff_of(a, topk_b, s.sl.len);
}

// One key's code: 4, 8, 16 or 32 bytes (two 16-byte loads).
template <int W>
__device__ __forceinline__ void load_code(const uint32_t *p, KeyCode<W> &k) {
    if constexpr (W == 1) {
        k.w[0] = *p;
    } else if constexpr (W == 2) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        k.w[0] = v.x;
        k.w[1] = v.y;
    } else {
#pragma unroll
        for (int h = 0; h < W / 4; ++h) {
            const uvec4 v = *reinterpret_cast<const uvec4 *>(p + 4 * h);
            k.w[4 * h] = v.x;
            k.w[4 * h + 1] = v.y;
            k.w[4 * h + 2] = v.z;
            k.w[4 * h + 3] = v.w;
        }
    }
}

// Issue the code loads of sub-batch sb of a chunk (thread t: keys
// p0 + 256 (kSub sb + r) + t, r < kSub: each instruction reads one
// contiguous run of 64 codes per wave).  A lane past the span re-reads the
// span's last key: every load is issued on every path, so the compiler's
// wait before a sub-batch is used counts exactly the loads issued after it
// (a load that some path skips would make it wait for every load in flight).
template <int W>
__device__ __forceinline__ void slot_issue(const FusedArgs &a, const Slot &s, int sb,
                                           KeyCode<W> (&buf)[kSub]) {
    const int t = threadIdx.x;
    const uint32_t *kc = a.codes + (int64_t)s.u * a.max_ctx * W;
#pragma unroll
    for (int r = 0; r < kSub; ++r) {
        const int64_t i = s.p0 + (int64_t)(kSub * sb + r) * kThreads + t;
        load_code<W>(kc + (i < s.p1 ? i : s.p1 - 1) * W, buf[r]);
    }
}

// Wave 0 only: the unit's generation and its PRO parts' tagged code words
// (query heads, then the appended key), re-read until every word carries
// this launch's tag (generation + 1), into LDS.  It runs after the wave has
// issued its first code loads: a workgroup's loads leave the CU in order,
// so the first read returns no later than those would anyway.
template <int G, int R>
__device__ __forceinline__ void slot_fetch_qcodes(const FusedArgs &a, const Slot &s, Smem<G, R> &sm) {
    constexpr int W = R / 32;
    constexpr int NW = (G + 1) * W;     // up to 72 words
    constexpr int NL = (NW + 63) / 64;  // words per lane
    const int lane = threadIdx.x & 63;
    const uint64_t *src = a.qtag + (int64_t)s.u * NW;
    const uint32_t tag = ld_dev(a.gen + s.u) + 1u;
    uint64_t v[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) v[j] = lane + 64 * j < NW ? ld_dev(src + lane + 64 * j) : (uint64_t)tag << 32;
    auto stale = [&]() {
        bool st = false;
#pragma unroll
        for (int j = 0; j < NL; ++j) st |= (uint32_t)(v[j] >> 32) != tag;
        return st;
    };
    for (int spins = 0; __ballot(stale()) != 0; ++spins) {
        if (spins > a.spin_limit) {
            if (lane == 0) atomicOr(&a.ctrl[kCtrlStatus], HATA_DEV_STALL);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < NL; ++j)
            if ((uint32_t)(v[j] >> 32) != tag) v[j] = ld_dev(src + lane + 64 * j);
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int i = lane + 64 * j;
        if (i < G * W) sm.scan.qc[i] = (uint32_t)v[j];
        else if (i < NW) sm.scan.app[i - G * W] = (uint32_t)v[j];
    }
    if (lane == 0) sm.scan.gen = tag;
}

// Query codes from LDS into scalar registers.
template <int G, int R>
__device__ __forceinline__ void qcodes_sgpr(const Smem<G, R> &sm, uint32_t (&qc)[G][R / 32]) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int w = 0; w < R / 32; ++w) qc[h][w] = __builtin_amdgcn_readfirstlane(sm.scan.qc[h * (R / 32) + w]);
}

// Scores of sub-batch sb, counted into the LDS sub-histograms and kept in
// LDS (spans of kSpanUnit keys) or stored to the workspace two to a 32-bit
// word.
template <int G, int R, bool LDS>
__device__ __forceinline__ void slot_score(const FusedArgs &a, const Slot &s, int sb,
                                           const KeyCode<R / 32> (&buf)[kSub],
                                           const QPlanes<G, R / 32> &qp, Smem<G, R> &sm) {
    constexpr int W = R / 32;
    const int t = threadIdx.x, wv = t >> 6;
    constexpr int HPW = SmemScan<G, R>::NH / 4;  // sub-histograms per wave
    uint32_t *wh = sm.scan.hist[wv * HPW + (t & (HPW - 1))];
    constexpr bool in_lds = LDS;
    const int n_span = (int)(s.p1 - s.p0);
    const int sub_lo = kSub * sb * kThreads;
    const int app_ii = s.sl.app ? (int)(s.sl.l0 - s.p0) : -1;
    if (in_lds && !a.scores_dbg && sub_lo + kSub * kThreads <= n_span &&
        (app_ii < sub_lo || app_ii >= sub_lo + kSub * kThreads)) {
        // a whole sub-batch of ordinary keys
#pragma unroll
        for (int r = 0; r < kSub; ++r) {
            const int ii = sub_lo + r * kThreads + t;
            const int sv = group_hamming<G, W>(buf[r], qp);
            atomicAdd(&wh[sv], 1u);
            sm.scan.scores[ii] = (uint16_t)sv;
        }
        return;
    }
    KeyCode<W> appv;
#pragma unroll
    for (int w = 0; w < W; ++w) appv.w[w] = sm.scan.app[w];
    uint16_t *sc = a.scores + (int64_t)s.u * a.sstride + s.p0;
    uint16_t *sd = a.scores_dbg ? a.scores_dbg + (int64_t)s.u * a.max_ctx + s.p0 : nullptr;
#pragma unroll
    for (int r = 0; r < kSub; ++r) {
        const int ii = sub_lo + r * kThreads + t;
        uint32_t sv = kNoScore;
        if (ii < n_span) {
            KeyCode<W> k;
#pragma unroll
            for (int w = 0; w < W; ++w) k.w[w] = (ii == app_ii) ? appv.w[w] : buf[r].w[w];
            sv = (uint32_t)group_hamming<G, W>(k, qp);
            atomicAdd(&wh[sv], 1u);
            if (sd) sd[ii] = (uint16_t)sv;
            if (in_lds) sm.scan.scores[ii] = (uint16_t)sv;
        }
        if (!in_lds) {
            const uint32_t nb = (uint32_t)__shfl_xor((int)sv, 1, 64);
            if (!(t & 1) && ii < n_span) st_dev(reinterpret_cast<uint32_t *>(sc + ii), sv | (nb << 16));
        }
    }
}

// The item's histogram: its cumulative counts (bin by bin, tagged with the
// unit's launch generation in the upper 32 bits) go to the item's row of
// chunk_hist, and its counts are added into the unit histogram two bins per
// 64-bit atomic.  Nothing waits for these writes: a reader knows the unit
// histogram is complete when its counts sum to the context length, and a
// row's entries are this launch's when they carry its tag.  Returns the
// span's candidate cut.
template <int G, int R>
__device__ __forceinline__ int slot_publish(const FusedArgs &a, const Slot &s, uint32_t gen, Smem<G, R> &sm) {
    constexpr int NB = G * R + 1;
    constexpr int NP = (NB + 1) / 2;
    constexpr int PER = (NB + kThreads - 1) / kThreads;
    const int t = threadIdx.x;
    __syncthreads();
    uint32_t loc[PER];
    int tsum = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int bin = t * PER + e;
        uint32_t v = 0;
        if (bin < NB) {
#pragma unroll
            for (int h = 0; h < SmemScan<G, R>::NH; ++h) v += sm.scan.hist[h][bin];
            sm.scan.hist[0][bin] = v;
        }
        loc[e] = v;
        tsum += (int)v;
    }
    if (t == 0) sm.scan.tc = NB - 1;
    int tot;
    int run = block_excl_scan_256(tsum, sm.scan.scan, &tot);  // its barriers publish hist[0]
    // The candidate cut: the first bin at which the span's cumulative count
    // reaches 1.5 times its proportional share of k_eff, plus 32.
    const int n_span = (int)(s.p1 - s.p0);
    const int64_t k_eff = s.k_eff;
    const int64_t share = (k_eff * n_span + s.sl.len - 1) / s.sl.len;
    const int64_t target = share + share / 2 + 32 < n_span ? share + share / 2 + 32 : n_span;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int bin = t * PER + e;
        if (bin < NB) {
            const int before = run;
            run += (int)loc[e];
            sm.scan.hist[1][bin] = (uint32_t)run;  // the cumulative row, published below
            if (before < target && run >= target) sm.scan.tc = bin;
        }
    }
    __syncthreads();
    // Wave 3 alone publishes, with every store a whole 512-byte line run: on
    // this architecture stores count against the issuing wave's memory
    // counter, and waves 0-2 poll next (a poll's wait would include them).
    // Its values come out of LDS before the barrier that frees the memory.
    constexpr int CW = (NB + 63) / 64, PW = (NP + 63) / 64;
    uint32_t cum[CW], cnt[PW][2];
    const int l = t & 63;
    if (t >= 3 * 64) {
#pragma unroll
        for (int k = 0; k < CW; ++k) cum[k] = l + 64 * k < NB ? sm.scan.hist[1][l + 64 * k] : 0u;
#pragma unroll
        for (int k = 0; k < PW; ++k) {
            const int pr = l + 64 * k;
            cnt[k][0] = pr < NP ? sm.scan.hist[0][2 * pr] : 0u;
            cnt[k][1] = 2 * pr + 1 < NB ? sm.scan.hist[0][2 * pr + 1] : 0u;
        }
    }
    const int tc = sm.scan.tc;
    __syncthreads();
    // a unit of one span: its histogram is the unit's, read from LDS by the
    // selection (nothing to publish)
    const bool single = s.sl.len <= a.span;
    if (t >= 3 * 64 && !single) {
        uint64_t *ch = a.chunk_hist + ((int64_t)s.u * a.n_chunks + s.c) * NB;
        const uint64_t tag = (uint64_t)gen << 32;
#pragma unroll
        for (int k = 0; k < CW; ++k)
            if (l + 64 * k < NB) st_dev(ch + l + 64 * k, tag | cum[k]);
        uint64_t *uh = reinterpret_cast<uint64_t *>(a.unit_hist) + (int64_t)s.u * NP;
#pragma unroll
        for (int k = 0; k < PW; ++k)
            if (cnt[k][0] | cnt[k][1])
                __hip_atomic_fetch_add(uh + l + 64 * k, (uint64_t)cnt[k][0] | ((uint64_t)cnt[k][1] << 32),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return tc;
}

// The unit's last WORK item, once every item of the unit has signalled (no
// item reads the unit histogram again in this launch, and every item's
// counts were added before its signal): the histogram is cleared for the
// unit's next launch.  The workspace's zero fill clears it before the first.
template <int G, int R>
__device__ __forceinline__ void unit_hist_clear(const FusedArgs &a, int u) {
    constexpr int NB = G * R + 1;
    for (int i = threadIdx.x; i < NB + 1; i += kThreads) st_dev(a.unit_hist + (int64_t)u * (NB + 1) + i, 0u);
}

// Thread 0 of the unit's last WORK item, once it knows it is the last: every
// item of the unit is past its waits and past reading the length, so the
// unit's counters are reset for the next launch, its generation advances,
// and the unit is counted as finished in its batch entry.  Returns the
// entry's count before this unit, for entry_done (its round trip can overlap
// other work first).  Nothing here needs to complete before the kernel ends.
__device__ __forceinline__ int unit_done(const FusedArgs &a, int u) {
    for (int w = 0; w < kNumCtr; ++w) st_dev(unit_ctr(a, u, w), 0);
    __hip_atomic_fetch_add(a.gen + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return add_dev(batch_ctr(a, u / a.Hkv), 1);
}

// After unit_done: the last unit of batch entry b to finish publishes the
// entry's new length (no item of the entry reads it any more) and clears the
// entry's count.  sl is the entry's length state of this launch.
__device__ __forceinline__ void entry_done(const FusedArgs &a, int b, const StepLen &sl, int prev) {
    if (prev != a.Hkv - 1) return;
    if (sl.app) st_dev(a.seq_len + b, (int32_t)(sl.l0 + 1));
    st_dev(batch_ctr(a, b), 0);
}

// Scan phase of work item (u, c), which also sets up its slot (cur): the
// span's codes in sub-batches of 1024 keys (4 to 32 KB), D of them in flight
// (up to 64 KB), issued in groups of D: every group but the last issues the
// next group's sub-batch in the slot it has just scored (sub-batches past
// the span re-read its last key and are not scored), so each sub-batch's
// wait leaves the later ones in flight.  Wave 0 then fetches the unit's code words (see
// slot_fetch_qcodes).  Scores go to LDS (or the workspace), the histograms
// are published.  Returns the span's candidate cut (-1 for an empty span);
// *gen gets the launch's tag.
template <int G, int R, bool LDS>
__device__ __forceinline__ int scan_phase(const FusedArgs &a, int u, int c, Slot &cur, uint32_t &gen,
                                          Smem<G, R> &sm) {
    constexpr int NB = G * R + 1;
    constexpr int W = R / 32;
    constexpr int D = scan_depth<R>();
    const int wv = threadIdx.x >> 6;
    // The first group's loads leave before the entry's length is read (they
    // stay inside the span's cache row; keys past the length are never
    // scored), the length and the top-k with them.
    cur = slot_row(a, u, c);
    KeyCode<W> buf[D][kSub];
#pragma unroll
    for (int d = 0; d < D; ++d) slot_issue<W>(a, cur, d, buf[d]);
    slot_len(a, cur);
    if (cur.p0 >= cur.p1) return -1;
    const int n_sub = (int)((cur.p1 - cur.p0 + kSub * kThreads - 1) / (kSub * kThreads));
    const int n_grp = (n_sub + D - 1) / D;
    for (int i = threadIdx.x; i < SmemScan<G, R>::NH * NB; i += kThreads) (&sm.scan.hist[0][0])[i] = 0u;
    if (wv == 0) slot_fetch_qcodes<G, R>(a, cur, sm);
    __syncthreads();
    gen = sm.scan.gen;
    HATA_PHASE(a, kPhCodes);
    uint32_t qc[G][W];
    qcodes_sgpr<G, R>(sm, qc);
    QPlanes<G, W> qp;
    query_planes<G, W>(qc, qp);
    for (int g = 0; g + 1 < n_grp; ++g) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            slot_score<G, R, LDS>(a, cur, g * D + d, buf[d], qp, sm);
            slot_issue<W>(a, cur, (g + 1) * D + d, buf[d]);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        if ((n_grp - 1) * D + d < n_sub) slot_score<G, R, LDS>(a, cur, (n_grp - 1) * D + d, buf[d], qp, sm);
    HATA_PHASE(a, kPhScanned);
    return slot_publish<G, R>(a, cur, gen, sm);
}

// ---------------------------------------------------------------- selection phase

// All-reduce over the 16 lanes of a row (lanes 16 g .. 16 g + 15): xor-1 and
// xor-2 quad permutes, then the half-row and row mirrors.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// The query heads as the A operand of v_mfma_f32_16x16x32_bf16: lane l holds
// row l % 16 (head; a copy of head G - 1 for rows >= G) and, for MFMA j, dims
// 32 j + 8 (l / 16) .. + 8 (the same dims its B operand brings for a key).
template <int G>
__device__ __forceinline__ void load_q_operand(const uint16_t *qg, bf16x8 (&qa)[4]) {
    // Rows h >= G repeat head G - 1 (their logits are never used), so every
    // lane loads and nothing waits for these loads before their first use.
    const int lane = threadIdx.x & 63, h = (lane & 15) < G ? (lane & 15) : G - 1, grp = lane >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        qa[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uvec4 *>(qg + h * kHeadDim + 32 * j + 8 * grp));
}

// s_waitcnt immediates (gfx9 encoding): wait for LDS operations only, or
// for vector memory loads only.
constexpr int kWaitLgkm0 = 0xC07F;  // vmcnt(63) expcnt(7) lgkmcnt(0)
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0) expcnt(7) lgkmcnt(15)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Four 16-bit values of four consecutive rows of a staged V tile, transposed
// by the LDS (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i % 4 of the 64-bit pieces addressed by lanes i / 4,
// i / 4 + 4, i / 4 + 8 and i / 4 + 12.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
}

// Attention over the rows Kb / Vb + list[0..n) (offsets from a batch's first
// key; the row at offset app_off is this step's appended key, read from
// kapp / vapp).  Each wave takes 32 keys of every 128: logits of two 16-key
// tiles by MFMA (for MFMA j, lane (g, c) brings dims 32 j + 8 g .. + 8 of key
// c of a tile, so each load instruction reads whole 64-byte pieces of 16
// rows; its accumulator holds heads 4 g .. 4 g + 3 of key c), an online
// softmax in base 2 per head (running m, l per lane for its four heads), and
// P.V by MFMA as well: P (heads x 32 keys) in bf16 high and low parts
// through LDS as the A operand, the V rows loaded straight into LDS
// (global_load_lds) and read back transposed as the B operand (lane (g, n)
// gets keys 8 g .. 8 g + 7 of dim n of a 16-dim block).  oacc[blk] holds O[4 g + i][16 blk + n] in
// lane (g, n).  Loads of a round are all issued before any is used.
template <int G>
__device__ __forceinline__ void attend_mfma(const uint16_t *__restrict__ Kb,
                                            const uint16_t *__restrict__ Vb,
                                            const uint16_t *__restrict__ kapp,
                                            const uint16_t *__restrict__ vapp, int app_off,
                                            const uint16_t *list, int n, const bf16x8 (&qa)[4],
                                            uint16_t (*vst)[kHeadDim], uint16_t (*pb)[G][32],
                                            float (&m)[4], float (&lsum)[4], f32x4 (&oacc)[8]) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, grp = lane >> 4, c = lane & 15;
    constexpr float kScale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
    for (int base = 32 * wv; base < n; base += 128) {
        const int kc = n - base < 32 ? n - base : 32;
        // K rows: key 16 tau + c, dims 32 j + 8 grp .. + 8 for MFMA j
        // (keys past kc read the round's first key: every lane loads, so no
        // branch separates these loads from the V loads below, and their
        // logits are masked)
        uvec4 kr[2][4];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const int kk = 16 * tau + c;
            const int off = (int)list[base + (kk < kc ? kk : 0)];
            const uint16_t *row = off == app_off ? kapp : Kb + off * kHeadDim;
#pragma unroll
            for (int j = 0; j < 4; ++j) kr[tau][j] = *reinterpret_cast<const uvec4 *>(row + 32 * j + 8 * grp);
        }
        // V rows straight into LDS: 16 bytes per lane, and one instruction
        // fills four consecutive 256-byte rows (lane l writes piece l), so
        // piece l of instruction r is key (l >> 4) + 4 r, dims 8 (l & 15) .. + 8.
        // Keys past kc repeat the round's first key (their P is zero).  The
        // previous round's reads of the staging rows have completed first.
        // (The row offsets are all read from the list first: an LDS read after
        // one of these loads would have to wait for it.)
        const uint16_t *vrow[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int key = (lane >> 4) + 4 * r;
            const int off = (int)list[base + (key < kc ? key : 0)];
            vrow[r] = (off == app_off ? vapp : Vb + off * kHeadDim) + 8 * (lane & 15);
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
        for (int r = 0; r < 8; ++r)
            __builtin_amdgcn_global_load_lds(vrow[r], (__attribute__((address_space(3))) void *)&vst[4 * r][0],
                                             16, 0, 0);
        // nothing that waits for the K rows is moved above the V loads
        __builtin_amdgcn_sched_barrier(0);
        // logits
        f32x4 acc[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            acc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], __builtin_bit_cast(bf16x8, kr[tau][j]),
                                                                   acc[tau], 0, 0, 0);
        }
        // online softmax for this lane's heads 4 grp + i; P to LDS as bf16
        // high and low parts ([head][key])
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool hv = 4 * grp + i < G;
            const float z0 = (hv && c < kc) ? acc[0][i] * kScale : -INFINITY;
            const float z1 = (hv && 16 + c < kc) ? acc[1][i] * kScale : -INFINITY;
            const float M = fmaxf(m[i], row16_max(fmaxf(z0, z1)));
            const float al = (M == -INFINITY) ? 1.f : exp2f(m[i] - M);
            const float p0 = (z0 == -INFINITY) ? 0.f : exp2f(z0 - M);
            const float p1 = (z1 == -INFINITY) ? 0.f : exp2f(z1 - M);
            lsum[i] = lsum[i] * al + row16_sum(p0 + p1);
            // the accumulators are zero until the wave has seen a key
            if (__ballot(m[i] != -INFINITY) != 0) {
#pragma unroll
                for (int blk = 0; blk < 8; ++blk) oacc[blk][i] *= al;
            }
            m[i] = M;
            if (hv) {
                const int h = (4 * grp + i) % G;
                const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;  // round to nearest even
                pb[0][h][c] = __builtin_bit_cast(uint16_t, h0);
                pb[0][h][16 + c] = __builtin_bit_cast(uint16_t, h1);
                pb[1][h][c] = __builtin_bit_cast(uint16_t, (__bf16)(p0 - (float)h0));
                pb[1][h][16 + c] = __builtin_bit_cast(uint16_t, (__bf16)(p1 - (float)h1));
            }
        }
        // P as the A operand: lane l holds head l % 16, keys 8 (l >> 4) .. + 8
        uvec4 pa[2] = {uvec4{0u, 0u, 0u, 0u}, uvec4{0u, 0u, 0u, 0u}};
        if (c < G) {
            pa[0] = *reinterpret_cast<const uvec4 *>(&pb[0][c][8 * grp]);
            pa[1] = *reinterpret_cast<const uvec4 *>(&pb[1][c][8 * grp]);
        }
        const bf16x8 ph = __builtin_bit_cast(bf16x8, pa[0]), pl = __builtin_bit_cast(bf16x8, pa[1]);
        // P.V: the B operand of 16-dim block blk, transposed from the staged
        // rows once their loads have landed
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
            const uint16_t *src = &vst[8 * grp + (c >> 2)][16 * blk + 4 * (c & 3)];
            const s16x4 b0 = lds_read_tr16(src), b1 = lds_read_tr16(src + 4 * kHeadDim);
            const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, oacc[blk], 0, 0, 0);
            oacc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, oacc[blk], 0, 0, 0);
        }
    }
}

// Exclusive prefix sum over the lanes of a wave for 0 <= v < 16 (bit-plane
// ballots counted below each lane); *total gets the wave's sum.
__device__ __forceinline__ int wave_excl_scan16(int v, int *total) {
    int pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint64_t m = __ballot((v >> b) & 1);
        pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0)) << b;
        tot += __popcll(m) << b;
    }
    *total = tot;
    return pre;
}

// Sum over the lanes of a wave for 0 <= v < 64.
__device__ __forceinline__ int wave_sum64(int v) {
    int tot = 0;
#pragma unroll
    for (int b = 0; b < 6; ++b) tot += __popcll(__ballot((v >> b) & 1)) << b;
    return tot;
}

// Bit masks over eight packed u16 scores (bit e: score e): le8 of the scores
// <= T, lt8 of the scores < T.  Per 16-bit half, with x <= 0x7FFF:
// (0x8000 + T) - x has bit 15 set iff x <= T, and no borrow crosses halves.
// kNoScore (0xFFFF) is first folded to 0x7FFF, still above every T.
__device__ __forceinline__ void cut_masks(const uint4 &v, int T, uint32_t &le8, uint32_t &lt8) {
    const uint32_t hle = (uint32_t)(0x8000 + T) * 0x10001u;
    const uint32_t hlt = (uint32_t)(0x8000 + T - 1) * 0x10001u;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t le = 0, lt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t x = w[k] & 0x7FFF7FFFu;
        const uint32_t a = hle - x, b = hlt - x;
        le |= (((a >> 15) & 1u) << (2 * k)) | ((a >> 31) << (2 * k + 1));
        lt |= (((b >> 15) & 1u) << (2 * k)) | ((b >> 31) << (2 * k + 1));
    }
    le8 = le;
    lt8 = lt;
}

// Score e (0..7) of eight packed u16 scores.
__device__ __forceinline__ int score_at(const uint4 &v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? (int)(w >> 16) : (int)(w & 0xFFFF);
}

// 8 consecutive scores from LDS at offset o (aligned); offsets at or past n
// read as kNoScore.
__device__ __forceinline__ uint4 lds_scores8(const uint16_t *sc, int o, int64_t n) {
    if (o >= n) return make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
    const uint4 v = *reinterpret_cast<const uint4 *>(sc + o);
    uint64_t lo = (uint64_t)v.x | ((uint64_t)v.y << 32), hi = (uint64_t)v.z | ((uint64_t)v.w << 32);
    const int64_t nv = n - o;
    if (nv < 4) lo |= ~0ull << (16 * nv);
    if (nv < 8) hi |= nv <= 4 ? ~0ull : ~0ull << (16 * (nv - 4));
    return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
}

// 8 consecutive scores from the workspace (aligned); keys at or past s1
// read as kNoScore.
__device__ __forceinline__ uint4 load_scores8(const uint16_t *su, int64_t i0, int64_t s1) {
    if (i0 >= s1) return make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
    const uint64_t *p = reinterpret_cast<const uint64_t *>(su + i0);
    uint64_t lo = ld_dev(p);
    uint64_t hi = (i0 + 4 < s1) ? ld_dev(p + 1) : ~0ull;
    const int64_t nv = s1 - i0;  // valid keys among the eight
    if (nv < 4) lo |= ~0ull << (16 * nv);
    else if (nv < 8) hi |= ~0ull << (16 * (nv - 4));
    return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
}

// Bit mask over eight packed u16 scores of those <= T (bit e: score e),
// as in cut_masks.
__device__ __forceinline__ uint32_t le_mask8(const uint4 &v, int T) {
    const uint32_t hle = (uint32_t)(0x8000 + T) * 0x10001u;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t le = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t a = hle - (w[k] & 0x7FFF7FFFu);
        le |= (((a >> 15) & 1u) << (2 * k)) | ((a >> 31) << (2 * k + 1));
    }
    return le;
}

// The span's keys with score <= tc (keys woff + 512 d + e, scores in pf),
// as offsets in index order into sm.sel.list.  Returns their count; the
// list is complete after the caller's next barrier.
template <int G, int R>
__device__ __forceinline__ int list_candidates(const uint4 (&pf)[kSelRounds], int tc, int woff,
                                               Smem<G, R> &sm) {
    constexpr int D = kSelRounds;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint32_t le8[D];
    int n = 0;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        le8[d] = le_mask8(pf[d], tc);
        n += __popc(le8[d]);
    }
    const int wn = wave_sum64(n);
    if (lane == 0) sm.sel.wlt[wv] = wn;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
        const int c = sm.sel.wlt[w2];
        base += w2 < wv ? c : 0;
        total += c;
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        int tot;
        int p = base + wave_excl_scan16(__popc(le8[d]), &tot);
        const int o0 = woff + d * 512;
        for (uint32_t mm = le8[d]; mm; mm &= mm - 1u) sm.sel.list[p++] = (uint16_t)(o0 + __builtin_ctz(mm));
        base += tot;
    }
    return total;
}

// One selection batch (keys rb + woff + 512 d + e, scores in pf): the keys
// below Tsel, and the score-Tsel keys while the split's running tie count
// (ties_acc before the batch) is below rem_quota, written to sm.sel.list in
// index order.  Returns the batch's selected count; *n_eq gets its count of
// score-Tsel keys.  Ends with the list written by every thread but no
// barrier after it.
template <int G, int R>
__device__ __forceinline__ int select_batch(const uint4 (&pf)[kSelRounds], int Tsel, int64_t rem_quota,
                                            int64_t ties_acc, int woff, Smem<G, R> &sm, int *n_eq) {
    constexpr int D = kSelRounds;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    // pass 1: this lane's keys below Tsel and up to Tsel as bit masks (bit e
    // of slot d: key woff + 512 d + e; past the end the words read as
    // kNoScore, which is above every Tsel), and the wave's counts
    uint32_t lt8[D], le8[D];
    int n_e = 0, n_l = 0;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        cut_masks(pf[d], Tsel, le8[d], lt8[d]);
        n_e += __popc(le8[d] & ~lt8[d]);
        n_l += __popc(lt8[d]);
    }
    {
        const int weq = wave_sum64(n_e), wlt = wave_sum64(n_l);
        if (lane == 0) {
            sm.sel.weq[wv] = weq;
            sm.sel.wlt[wv] = wlt;
        }
    }
    __syncthreads();
    // this wave's place in the batch: ties and selections of the waves before it
    int64_t tie_base = ties_acc;
    int sel_base = 0, batch_sel = 0, batch_eq = 0;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
        const int e2 = sm.sel.weq[w2], l2 = sm.sel.wlt[w2];
        const int64_t tb = ties_acc + batch_eq;
        int64_t take = rem_quota - tb;
        take = take < 0 ? 0 : (take > e2 ? e2 : take);
        const int sw = l2 + (int)take;
        if (w2 < wv) {
            tie_base += e2;
            sel_base += sw;
        }
        batch_eq += e2;
        batch_sel += sw;
    }
    // pass 2: select in index order (d, lane, e) and write the list.  The
    // score-Tsel keys are taken in index order while the split's tie count
    // is below rem_quota: a lane takes all or none of its ties, except the
    // one lane where the quota runs out, which takes the lowest ones.
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const uint32_t eq8 = le8[d] & ~lt8[d];
        const int ne = __popc(eq8);
        int ne_tot;
        const int64_t tr = tie_base + wave_excl_scan16(ne, &ne_tot);
        uint32_t sel8;
        if (tr + ne <= rem_quota) {
            sel8 = le8[d];
        } else if (tr >= rem_quota) {
            sel8 = lt8[d];
        } else {
            uint32_t take = 0, rest = eq8;
            for (int q = (int)(rem_quota - tr); q > 0; --q) {
                take |= rest & (0u - rest);  // lowest remaining tie
                rest &= rest - 1u;
            }
            sel8 = lt8[d] | take;
        }
        int ns_tot;
        int p = sel_base + wave_excl_scan16(__popc(sel8), &ns_tot);
        const int o0 = woff + d * 512;
        for (uint32_t mm = sel8; mm; mm &= mm - 1u) sm.sel.list[p++] = (uint16_t)(o0 + __builtin_ctz(mm));
        tie_base += ne_tot;
        sel_base += ns_tot;
    }
    *n_eq = batch_eq;
    return batch_sel;
}

// Exclusive prefix count of a 0/1 flag over the 256 threads in thread
// order; *total gets the count.  Two barriers; tmp holds four ints.
__device__ __forceinline__ int block_excl_count(bool f, int *tmp, int *total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint64_t m = __ballot(f);
    const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (lane == 0) tmp[wv] = __popcll(m);
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
        const int c = tmp[w2];
        base += w2 < wv ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return base + pre;
}

// Selection phase of work item (u, c), once every item of the unit has
// scanned: the cut T from the unit histogram, the score-T and below-T keys
// of the items before it from their cumulative histograms, then the span's
// selected keys compacted in index order (in batches of kListCap keys),
// gathered and attended; the (m, l, o) partials of the items are merged in
// item order by the last one.
template <int G, int R, bool LDS>
__device__ __forceinline__ bool sel_phase(const FusedArgs &a, const Slot &cur, int tc, uint32_t gen,
                                          Smem<G, R> &sm) {
    constexpr int D = kSelRounds;  // selection rounds of scores in flight
    constexpr int NB = G * R + 1;
    // Waves 0-2 poll the unit's histograms (PER bins and WPT window entries
    // per thread); wave 3 published this item's histograms, and its stores
    // would hold up a poll's wait behind them.
    constexpr int kPoll = 3 * 64;
    constexpr int PER = (NB + kPoll - 1) / kPoll;
    constexpr int WPT = (kMaxSplits * kWin + kPoll - 1) / kPoll;
    const int u = cur.u, s = cur.c;
    const int b = u / a.Hkv, kv = u % a.Hkv, Hq = a.Hkv * G;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const StepLen sl = cur.sl;
    const int64_t len = sl.len;
    const int64_t k_eff = cur.k_eff;
    const int64_t s0 = cur.p0, s1 = cur.p1;
    const int n_splits_u = (int)((len + a.span - 1) / a.span);
    if (k_eff == 0) {  // the outputs are zero (written by PRO part 0)
        const int prev = wg_signal(unit_ctr(a, u, kAttn));
        if (t == 0) sm.sel.last = (prev == n_splits_u - 1);
        __syncthreads();
        if (sm.sel.last) {
            unit_hist_clear<G, R>(a, u);
            if (t == 0) entry_done(a, b, sl, unit_done(a, u));
        }
        return sm.sel.last;
    }

    const uint16_t *su = a.scores + (int64_t)u * a.sstride;
    // batch layout: wave w holds keys [rb + 2048 w, rb + 2048 (w + 1)), lane
    // `lane` of it keys rb + 2048 w + 512 d + 8 lane + e (d < D, e < 8)
    const int woff = wv * (kSelRounds * kSelRound / 4) + 8 * lane;
    constexpr bool in_lds = LDS;
    uint4 pf[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        pf[d] = in_lds ? lds_scores8(sm.sel.scores, woff + d * 512, s1 - s0)
                       : load_scores8(su, s0 + woff + (int64_t)d * 512, s1);
    // ---- the unit histogram and a window of the earlier items' cumulative
    // histograms (bins tc - kWin + 1 .. tc), requested before the candidate
    // pass and read again until complete
    const uint32_t *uhr = a.unit_hist + (int64_t)u * (NB + 1);
    const uint64_t *chu = a.chunk_hist + (int64_t)u * a.n_chunks * NB;
    const uint64_t tag = (uint64_t)gen << 32;
    const int wlo = tc - (kWin - 1);
    uint32_t loc[PER] = {};
    uint64_t win[WPT] = {};
    // Every lane of waves 0-2 issues every read (entries it does not own
    // re-read word 0 and are masked where used: loc_ok, win_ok), so the
    // reads are all in flight before the first is waited for.
    auto read_state = [&]() {
        if (uni(t) >= kPoll) return;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int bin = t * PER + e;
            loc[e] = ld_dev(uhr + (bin < NB ? bin : 0));
        }
#pragma unroll
        for (int k = 0; k < WPT; ++k) {
            const int i = t + k * kPoll, cc = i / kWin, bin = wlo + i % kWin;
            win[k] = ld_dev(chu + ((cc < s && bin >= 0) ? (int64_t)cc * NB + bin : 0));
        }
    };
    auto loc_ok = [&](int e) { return t < kPoll && t * PER + e < NB; };
    auto win_ok = [&](int k) {
        const int i = t + k * kPoll;
        return t < kPoll && i / kWin < s && wlo + i % kWin >= 0;
    };
    // A unit of one span takes its own counts (still in LDS) as the unit
    // histogram, so its first pass below finds them complete.
    const bool single = n_splits_u == 1;
    if (single) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int bin = t * PER + e;
            loc[e] = (t < kPoll && bin < NB) ? sm.scan.hist[0][bin] : 0u;
        }
    } else {
        read_state();
    }
    // ---- meanwhile the span's candidates: every key up to the candidate
    // cut tc, in index order (spans kept in LDS)
    const int n_cand = in_lds ? uni(list_candidates<G, R>(pf, tc, woff, sm)) : -1;
    HATA_PHASE(a, kPhListed);
    // ---- the cut T, once every item of the unit has added its counts
    // (they then sum to len)
    for (int spins = 0;; ++spins) {
        int tsum = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) tsum += loc_ok(e) ? (int)loc[e] : 0;
        if (t == 0) {
            sm.sel.T = NB - 1;
            sm.sel.below = 0;
        }
        int tot;
        int run = block_excl_scan_256(tsum, sm.sel.scan, &tot);
        if ((int64_t)tot >= len) {
            HATA_TRACE_WORD(a, 14, spins);
            // T: first bin whose cumulative count reaches k_eff; below: the
            // count under T
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int nxt = run + (loc_ok(e) ? (int)loc[e] : 0);
                if ((int64_t)run < k_eff && (int64_t)nxt >= k_eff) {
                    sm.sel.T = t * PER + e;
                    sm.sel.below = run;
                    sm.sel.cntT = (int)loc[e];
                }
                run = nxt;
            }
            break;
        }
        if (spins > a.poll_limit) {
            if (t == 0) atomicOr(&a.ctrl[kCtrlStatus], HATA_DEV_STALL);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        read_state();
    }
    __syncthreads();
    const int T = uni(sm.sel.T);
    HATA_PHASE(a, kPhCut);
    // the query heads as MFMA operands (they arrive during the selection; read
    // earlier, the candidate pass would wait for them)
    bf16x8 qa[4];
    load_q_operand<G>(a.q + ((int64_t)b * Hq + kv * G) * kHeadDim, qa);
    // ---- score-T and below-T keys in the items before this one: from the
    // window when it holds bins T - 1 and T, else read (again) until every
    // entry carries this launch's tag
    long long tie = 0, lo = 0;
    // The unit's last span: the items before it are all the others, so its
    // counts come from the unit histogram less its own (still in LDS where
    // own_hist_kept holds: every code length but 256 bits at G = 8).
    const bool last_span = own_hist_kept<G, R>() && s == n_splits_u - 1;
    const bool in_win = !last_span && T <= tc && (T == 0 ? wlo <= 0 : T - 1 >= wlo);
    int bad = 0;
    if (last_span && t == 0) {
        tie = (long long)sm.sel.cntT - (long long)sm.scan.hist[0][T];
        lo = (long long)sm.sel.below - (T > 0 ? (long long)sm.scan.hist[1][T - 1] : 0ll);
    }
    if (in_win) {
#pragma unroll
        for (int k = 0; k < WPT; ++k) {
            const int i = t + k * kPoll, bin = wlo + i % kWin;
            if (win_ok(k)) {
                bad |= (win[k] & ~0xFFFFFFFFull) != tag;
                const long long cum = (uint32_t)win[k];
                if (bin == T) tie += cum;
                if (bin == T - 1) {
                    tie -= cum;
                    lo += cum;
                }
            }
        }
    }
    const bool reread = !last_span && (!in_win || __syncthreads_or(bad));
    HATA_TRACE_WORD(a, 12, (uint64_t)in_win | ((uint64_t)reread << 1) | ((uint64_t)T << 8) |
                               ((uint64_t)tc << 20) | ((uint64_t)(n_cand < 0 ? 0xFFFF : n_cand) << 32));
    if (reread) {
        for (int spins = 0;; ++spins) {
            tie = lo = 0;
            bad = 0;
            for (int cc = t; cc < s; cc += kThreads) {
                const uint64_t *chc = chu + (int64_t)cc * NB;
                const uint64_t h = ld_dev(chc + T);
                const uint64_t l = T > 0 ? ld_dev(chc + T - 1) : tag;
                bad |= ((h & ~0xFFFFFFFFull) != tag) | ((l & ~0xFFFFFFFFull) != tag);
                tie += (long long)(uint32_t)h - (long long)(uint32_t)l;
                lo += (uint32_t)l;
            }
            if (!__syncthreads_or(bad)) break;
            if (spins > a.poll_limit) {
                if (t == 0) atomicOr(&a.ctrl[kCtrlStatus], HATA_DEV_STALL);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    int ties_s, below_s;  // both at most the context length
    block_sum2_256((int)tie, (int)lo, sm.sel.red, &ties_s, &below_s);
    const int64_t ties_b = uni(ties_s), below_b = uni(below_s);
    HATA_PHASE(a, kPhTies);
    const int64_t quota = k_eff - uni(sm.sel.below);  // keys of score T to take, lowest index first
    const int64_t rem_quota = quota - ties_b > 0 ? quota - ties_b : 0;
    int64_t out_pos = below_b + (ties_b < quota ? ties_b : quota);

    int32_t *sel_u = a.sel_out ? a.sel_out + (int64_t)u * a.k_max : nullptr;
    const uint16_t *Ku = a.k_cache + (int64_t)u * a.max_ctx * kHeadDim;
    const uint16_t *Vu = a.v_cache + (int64_t)u * a.max_ctx * kHeadDim;
    const int64_t app_row = sl.app ? sl.l0 : -1;
    const uint16_t *kapp = sl.app ? a.k_new + ((int64_t)b * a.Hkv + kv) * kHeadDim : nullptr;
    const uint16_t *vapp = sl.app ? a.v_new + ((int64_t)b * a.Hkv + kv) * kHeadDim : nullptr;
    float m[4], l[4];
    f32x4 o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.f;
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) o[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (n_cand >= 0 && T <= tc) {
        // ---- the selection is among the candidates: keep those below T and
        // the first rem_quota of score T (index order), compacting the list
        // in place (a kept entry moves to a position <= its own)
        int n_sel = 0;
        int64_t ties_acc = 0;
        for (int i0 = 0; i0 < n_cand; i0 += kThreads) {
            const int i = i0 + t;
            const int off = i < n_cand ? (int)sm.sel.list[i] : 0;
            const int sc = i < n_cand ? (int)sm.sel.scores[off] : 0x7FFF;
            const uint64_t mlt = __ballot(sc < T), meq = __ballot(sc == T);
            const int lt_pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(mlt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mlt, 0));
            const int eq_pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(meq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)meq, 0));
            if (lane == 0) {
                sm.sel.wlt[wv] = __popcll(mlt);
                sm.sel.weq[wv] = __popcll(meq);
            }
            __syncthreads();
            int lt_b = 0, eq_b = 0, lt_tot = 0, eq_tot = 0;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const int cl = sm.sel.wlt[w2], ce = sm.sel.weq[w2];
                lt_b += w2 < wv ? cl : 0;
                eq_b += w2 < wv ? ce : 0;
                lt_tot += cl;
                eq_tot += ce;
            }
            const int64_t room = rem_quota - ties_acc > 0 ? rem_quota - ties_acc : 0;  // score-T keys still to take
            const int eq_before = eq_b + eq_pre;
            const bool take = sc < T || (sc == T && eq_before < room);
            const int pos = n_sel + lt_b + lt_pre + (int)(eq_before < room ? eq_before : room);
            __syncthreads();  // every entry of this round read, the counts too
            if (take) sm.sel.list[pos] = (uint16_t)off;
            n_sel = uni(n_sel + lt_tot + (int)(eq_tot < room ? eq_tot : room));
            ties_acc = uni(ties_acc + eq_tot);
        }
        __syncthreads();
        if (sel_u) {
            for (int i = t; i < n_sel; i += kThreads) {
                const int64_t gp = out_pos + i;
                if (gp >= 0 && gp < a.k_max) sel_u[gp] = (int32_t)(s0 + sm.sel.list[i]);
            }
        }
        HATA_PHASE(a, kPhSelected);
        HATA_TRACE_WORD(a, 13, n_sel);
        const int app_off = (app_row >= s0 && app_row < s1) ? (int)(app_row - s0) : -1;
        attend_mfma<G>(Ku + s0 * kHeadDim, Vu + s0 * kHeadDim, kapp, vapp, app_off, sm.sel.list,
                       n_sel, qa, sm.sel.vst[wv], sm.sel.pb[wv], m, l, o);
        __syncthreads();
    } else {
        if (n_cand >= 0) __syncthreads();  // the candidate list is read no further
        int64_t ties_acc = 0;
        for (int64_t rb = s0; rb < s1; rb += kListCap) {
            int batch_eq;
            const int batch_sel = select_batch<G, R>(pf, T, rem_quota, ties_acc, woff, sm, &batch_eq);
            // the next batch's scores are on their way during this one's attention
            if (rb + kListCap < s1) {
#pragma unroll
                for (int d = 0; d < D; ++d) pf[d] = load_scores8(su, rb + kListCap + woff + (int64_t)d * 512, s1);
            }
            __syncthreads();
            if (sel_u) {
                for (int i = t; i < batch_sel; i += kThreads) {
                    const int64_t gp = out_pos + i;
                    if (gp >= 0 && gp < a.k_max) sel_u[gp] = (int32_t)(rb + sm.sel.list[i]);
                }
            }
            out_pos += batch_sel;
            ties_acc += batch_eq;
            // the batch's selections through the attention
            if (rb == s0) HATA_PHASE(a, kPhSelected);
            if (rb == s0) HATA_TRACE_WORD(a, 13, (1u << 30) | batch_sel);
            const int app_off = (app_row >= rb && app_row < rb + kListCap) ? (int)(app_row - rb) : -1;
            attend_mfma<G>(Ku + rb * kHeadDim, Vu + rb * kHeadDim, kapp, vapp, app_off, sm.sel.list,
                           batch_sel, qa, sm.sel.vst[wv], sm.sel.pb[wv], m, l, o);
            __syncthreads();
        }
    }

    HATA_PHASE(a, kPhAttended);
    // ---- the waves' states into LDS, then combined per output
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (lane == 16 * (h >> 2)) {
            sm.sel.cb.wm[wv][h] = m[h & 3];
            sm.sel.cb.wl[wv][h] = l[h & 3];
        }
    }
    // lane (g, n) holds O[4 g + i][16 blk + n]
    if ((lane >> 4) < (G + 3) / 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * (lane >> 4) + i;
            if (h < G) {
#pragma unroll
                for (int blk = 0; blk < 8; ++blk) sm.sel.cb.wo[wv][h][16 * blk + (lane & 15)] = o[blk][i];
            }
        }
    }
    __syncthreads();
    // Output pair pr (floats 2 pr, 2 pr + 1 of the G x 128 block) is thread
    // pr's: with M the maximum of the waves' m for its head, wave w's state
    // weighs a_w = exp2(m_w - M).
    float *pml = a.part_ml + ((int64_t)u * a.n_chunks + s) * G * 2;
    uint64_t *po = reinterpret_cast<uint64_t *>(a.part_o + ((int64_t)u * a.n_chunks + s) * G * kHeadDim);
    for (int pr = t; pr < G * kHeadDim / 2; pr += kThreads) {
        const int h = pr / (kHeadDim / 2), e = 2 * (pr % (kHeadDim / 2));
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            mw[w2] = sm.sel.cb.wm[w2][h];
            M = fmaxf(M, mw[w2]);
        }
        float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const float aw = (mw[w2] == -INFINITY) ? 0.f : exp2f(mw[w2] - M);
            const float2 ow = *reinterpret_cast<const float2 *>(&sm.sel.cb.wo[w2][h][e]);
            L = fmaf(sm.sel.cb.wl[w2][h], aw, L);
            O0 = fmaf(ow.x, aw, O0);
            O1 = fmaf(ow.y, aw, O1);
        }
        if (single) {
            // the unit's only split: its state is the output (as the merge
            // below would compute it, with weight exp2(0) = 1)
            uint16_t *op = a.out + ((int64_t)b * Hq + kv * G) * kHeadDim + 2 * pr;
            op[0] = L > 0.f ? f32_to_bf16(O0 / L) : (uint16_t)0;
            op[1] = L > 0.f ? f32_to_bf16(O1 / L) : (uint16_t)0;
            continue;
        }
        st_dev(po + pr, (uint64_t)__float_as_uint(O0) | ((uint64_t)__float_as_uint(O1) << 32));
        if (e == 0) {
            st_dev(pml + 2 * h, M);
            st_dev(pml + 2 * h + 1, L);
        }
    }
    if (single) {
        // no partial, no count; the unit histogram received nothing, so it
        // is still clear for the next launch
        HATA_PHASE(a, kPhPartial);
        if (t == 0) entry_done(a, b, sl, unit_done(a, u));
        return true;
    }

    // ---- the last split of the unit merges all partials in split order
    const int prev = wg_signal(unit_ctr(a, u, kAttn));
    HATA_PHASE(a, kPhPartial);
    if (t == 0) sm.sel.last = (prev == n_splits_u - 1);
    __syncthreads();
    if (!sm.sel.last) return false;
    unit_hist_clear<G, R>(a, u);
    // Per split x and head h: weight w = exp2(m_x - M) with M the maximum
    // over splits; out = sum_x w o_x / sum_x w l_x.  Thread 0 first does the
    // unit's bookkeeping (its count returns with the loads below and is used
    // at the end).  Output pair pr (floats 2 pr, 2 pr + 1 of the G x 128
    // block, head pr / 64) is thread pr's (and pr + 256's), so each wave
    // covers whole heads: it loads every split's (m, l) of its heads into its
    // lanes (split x in lane x), forms the weights and sums by lane
    // reductions and reads weight x back with a lane read, with no exchange
    // between waves.  Partials are loaded for up to XB splits at a time.
    int entry_prev = 0;
    if (t == 0) entry_prev = unit_done(a, u);
    constexpr int NPR = G * kHeadDim / 2;
    constexpr int PPT = (NPR + kThreads - 1) / kThreads;
    constexpr int XB = 24 / PPT;
    const float *mlb = a.part_ml + (int64_t)u * a.n_chunks * G * 2;
    const uint64_t *ob = reinterpret_cast<const uint64_t *>(a.part_o + (int64_t)u * a.n_chunks * G * kHeadDim);
    const int n = n_splits_u;
    uint64_t ov[PPT][XB];
#pragma unroll
    for (int k = 0; k < PPT; ++k)
#pragma unroll
        for (int x = 0; x < XB; ++x) {
            const int pr = t + k * kThreads;
            ov[k][x] = (pr < NPR && x < n) ? ld_dev(ob + (int64_t)x * NPR + pr) : 0ull;
        }
    float wk[PPT], Lk[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int h = wv + 4 * k;  // the head of this wave's pairs t + 256 k
        float mx = -INFINITY, lx = 0.f;
        if (h < G && lane < n) {
            mx = ld_dev(mlb + 2 * (lane * G + h));
            lx = ld_dev(mlb + 2 * (lane * G + h) + 1);
        }
        float M = row16_max(mx);
        M = fmaxf(M, __shfl_xor(M, 16, 64));
        M = fmaxf(M, __shfl_xor(M, 32, 64));
        wk[k] = (mx == -INFINITY) ? 0.f : exp2f(mx - M);
        float L = row16_sum(lx * wk[k]);
        L += __shfl_xor(L, 16, 64);
        Lk[k] = L + __shfl_xor(L, 32, 64);
    }
    HATA_PHASE(a, kPhMerged);
    float O[PPT][2];
#pragma unroll
    for (int k = 0; k < PPT; ++k) O[k][0] = O[k][1] = 0.f;
    for (int x0 = 0; x0 < n; x0 += XB) {
        if (x0 > 0) {
#pragma unroll
            for (int k = 0; k < PPT; ++k)
#pragma unroll
                for (int x = 0; x < XB; ++x) {
                    const int pr = t + k * kThreads;
                    ov[k][x] = (pr < NPR && x0 + x < n) ? ld_dev(ob + (int64_t)(x0 + x) * NPR + pr) : 0ull;
                }
        }
#pragma unroll
        for (int x = 0; x < XB; ++x) {
            if (x0 + x < n) {
#pragma unroll
                for (int k = 0; k < PPT; ++k) {
                    const float wx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk[k]), x0 + x));
                    O[k][0] = fmaf(__uint_as_float((uint32_t)ov[k][x]), wx, O[k][0]);
                    O[k][1] = fmaf(__uint_as_float((uint32_t)(ov[k][x] >> 32)), wx, O[k][1]);
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int pr = t + k * kThreads;
        if (pr < NPR) {
            const float L = Lk[k];
            uint16_t *o = a.out + ((int64_t)b * Hq + kv * G) * kHeadDim + 2 * pr;
            o[0] = L > 0.f ? f32_to_bf16(O[k][0] / L) : (uint16_t)0;
            o[1] = L > 0.f ? f32_to_bf16(O[k][1] / L) : (uint16_t)0;
        }
    }
    if (t == 0) entry_done(a, b, sl, entry_prev);
    return true;
}

// ---------------------------------------------------------------- item order

struct Item {
    int kind;  // 0 PRO, 1 WORK
    int u, i;
};

// The tk-th item of a list of U units.  When the whole grid is resident at
// once (resident, set by the host): PRO(u, p) for every unit and part, then
// WORK(u, c) unit by unit, and with tails_last (more than one item per
// unit) each unit's last item, which often holds just the few keys past a
// multiple of the span, after every other item: blocks are dealt to the
// XCDs in turn and to their CUs in order, so an XCD's last blocks are the
// ones that land as a third workgroup on a CU, and the light items are then
// the ones sharing a CU with two full ones.  Otherwise unit by unit,
// PRO(u, p) then WORK(u, c).
template <int R>
__device__ __forceinline__ Item item_in(const FusedArgs &a, int U, int tk) {
    constexpr int P = pro_parts(R);  // PRO parts per unit
    Item it;
    if (!a.resident) {
        // unit by unit, each unit's PRO parts just before its WORK items, so
        // that a grid larger than the chip streams codes from its first
        // workgroups on
        const int per = P + a.n_chunks, r = tk % per;
        it.u = tk / per;
        it.kind = r < P ? 0 : 1;
        it.i = r < P ? r : r - P;
        return it;
    }
    if (tk < P * U) {
        it.kind = 0; it.u = tk / P; it.i = tk % P;
        return it;
    }
    tk -= P * U;
    it.kind = 1;
    const int full = U * (a.n_chunks - 1);
    if (a.tails_last && tk >= full) {
        it.u = tk - full; it.i = a.n_chunks - 1;
    } else if (a.tails_last) {
        it.u = tk / (a.n_chunks - 1); it.i = tk % (a.n_chunks - 1);
    } else {
        it.u = tk / a.n_chunks; it.i = tk % a.n_chunks;
    }
    return it;
}

template <int R>
__device__ __forceinline__ Item item_of(const FusedArgs &a, int tk) {
    return item_in<R>(a, a.B * a.Hkv, tk);
}

// WORK(u, c): scan the span, wait for the unit, select, gather, attend.
template <int G, int R, bool LDS>
__device__ __forceinline__ void item_work(const FusedArgs &a, int u, int c, Smem<G, R> &sm) {
    Slot cur;
    uint32_t gen;
    const int tc = scan_phase<G, R, LDS>(a, u, c, cur, gen, sm);
    if (tc < 0) return;
    HATA_PHASE(a, kPhPublished);
    __syncthreads();  // the LDS histograms and the selection state share memory
    sel_phase<G, R, LDS>(a, cur, uni(tc), (uint32_t)uni((int)gen), sm);
}

// Three workgroups per CU (two for G = 8): the register budget the
// compiler must meet.
template <int G, int R, bool LDS>
__global__ __launch_bounds__(kThreads, G <= 4 ? 3 : 2) void k_decode_fused(FusedArgs a) {
    __shared__ Smem<G, R> sm;
    HATA_PHASE(a, kPhStart);
    const Item it = item_of<R>(a, blockIdx.x);
    if (it.kind == 0) item_pro<G, R>(a, it.u, it.i, sm);
    else item_work<G, R, LDS>(a, it.u, it.i, sm);
#ifdef HATA_PHASE_TRACE
    HATA_PHASE(a, kPhEnd);
    if (a.trace && threadIdx.x == 0 && (int)blockIdx.x < a.trace_items)
        a.trace[(int64_t)blockIdx.x * 16 + kPhItem] =
            ((uint64_t)it.kind << 31) | ((uint64_t)it.u << 8) | (uint64_t)it.i;
#endif
}

// ---------------------------------------------------------------- launch

// The last-items-last order gives up the unit-by-unit order that lets a grid
// larger than the chip make progress, so it is only used when every
// workgroup of the launch can be resident at once, with kTailHeadroom slots
// to spare for workgroups of other kernels that may still hold CUs.  A grid
// that is not resident at once puts each unit's PRO parts just before its
// WORK items (all PRO parts first would hold the chip for several rounds of
// workgroups that stream nothing: 159.5 -> 125.4 us per step for 64 ragged
// sequences of up to 64K keys).
constexpr int kTailHeadroom = 64;

template <int G, int R>
hipError_t launch_g(FusedArgs &a, hipStream_t s) {
    int dev = 0, n_cu = 0, per_cu = 0;
    a.tails_last = 0;
    a.resident = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_fused<G, R, true>, kThreads, 0) ==
            hipSuccess)
        a.resident = (int64_t)a.n_items + kTailHeadroom <= (int64_t)per_cu * n_cu;
    a.tails_last = a.resident && a.n_chunks > 1;
    // spans of kSpanUnit keys keep their scores in LDS between the phases
    if (a.span <= kSpanUnit)
        hipLaunchKernelGGL((k_decode_fused<G, R, true>), dim3(a.n_items), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_decode_fused<G, R, false>), dim3(a.n_items), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// The step's kernel for code length R and group size G (each code length is
// compiled in a source of its own, decode_r<R>.hip).
template <int R>
hipError_t launch_fused(int G, FusedArgs &a, hipStream_t s) {
    switch (G) {
        case 1: return launch_g<1, R>(a, s);
        case 2: return launch_g<2, R>(a, s);
        case 4: return launch_g<4, R>(a, s);
        case 8: return launch_g<8, R>(a, s);
        default: return hipErrorInvalidValue;
    }
}

extern template hipError_t launch_fused<32>(int, FusedArgs &, hipStream_t);
extern template hipError_t launch_fused<64>(int, FusedArgs &, hipStream_t);
extern template hipError_t launch_fused<128>(int, FusedArgs &, hipStream_t);
extern template hipError_t launch_fused<256>(int, FusedArgs &, hipStream_t);

}  // namespace hata
