// Host side of the decode step (hata_decode_attn / hata_decode_step): the
// workspace plan, the launch (one kernel, compiled per code length in
// decode_r<R>.hip from decode_fused.h, which describes the kernel), and the
// allocation-free form on a static device scratch.
#include <stdlib.h>

#include <mutex>

#include "decode_fused.h"

namespace hata {

#ifdef HATA_PHASE_TRACE
// The trace buffer of the next launches (hata_phase_trace); a diagnostic of
// the trace build only.
static uint64_t *g_trace = nullptr;
static int g_trace_items = 0;
#endif

// ---------------------------------------------------------------- plan + launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool make_decode_plan(int B, int Hq, int Hkv, int64_t max_ctx, int n_bits, DecodePlan *p) {
    if (B <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || max_ctx < 0) return false;
    if (n_bits != 32 && n_bits != 64 && n_bits != 128 && n_bits != 256) return false;
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return false;
    const int64_t units = (int64_t)B * Hkv;
    if (units > 65535) return false;
    DecodePlan d;
    d.B = B;
    d.Hq = Hq;
    d.Hkv = Hkv;
    d.G = G;
    d.R = n_bits;
    d.NB = G * n_bits + 1;
    d.max_ctx = max_ctx;
    // work items: spans of a multiple of kSpanUnit keys, at most kMaxSplits
    // per unit (all of a unit's items must fit on the chip together)
    const int64_t ctx = max_ctx > 0 ? max_ctx : 1;
    const int64_t per = (ctx + (int64_t)kMaxSplits * kSpanUnit - 1) / ((int64_t)kMaxSplits * kSpanUnit);
    d.span = per * kSpanUnit;
    const int64_t C = (ctx + d.span - 1) / d.span;
    const int64_t items = units * (pro_parts(n_bits) + C);
    if (items > INT32_MAX / 2) return false;
    d.n_chunks = (int)C;
    d.n_items = (int)items;
    d.sstride = ((max_ctx + 63) / 64) * 64;
    size_t off = 0;
    d.off_gen = off;
    off = align256(off + (size_t)units * 4);
    d.off_qtag = off;
    off = align256(off + (size_t)units * (G + 1) * (n_bits / 32) * 8);
    d.off_unit_hist = off;
    off = align256(off + (size_t)units * (d.NB + 1) * 4);
    d.off_chunk_hist = off;
    off = align256(off + (size_t)units * d.n_chunks * d.NB * 8);
    d.off_part_ml = off;
    off = align256(off + (size_t)units * d.n_chunks * G * 2 * 4);
    d.off_part_o = off;
    off = align256(off + (size_t)units * d.n_chunks * G * kHeadDim * 4);
    d.off_scores = off;
    d.used = d.span <= kSpanUnit ? off : align256(off + (size_t)units * d.sstride * 2);
    off = align256(off + (size_t)units * d.sstride * 2);
    d.total = off;
    *p = d;
    return true;
}

hipError_t launch_decode(const DecodePlan &p, uint16_t *k_cache, uint16_t *v_cache,
                         uint32_t *codes, int32_t *seq_len, int32_t *ctrl,
                         const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                         const float *w, const int32_t *topk, int k_max, uint16_t *out, void *ws,
                         int32_t *sel_idx_out, uint16_t *scores_out, hipStream_t s) {
    char *base = static_cast<char *>(ws);
    FusedArgs a{};
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.codes = codes;
    a.seq_len = seq_len;
    a.ctrl = ctrl;
    a.k_new = k_new;
    a.v_new = v_new;
    a.q = q;
    a.w = w;
    a.topk = topk;
    a.out = out;
    a.sel_out = sel_idx_out;
    a.scores_dbg = scores_out;
    a.scores = reinterpret_cast<uint16_t *>(base + p.off_scores);
    a.sstride = p.sstride;
    a.gen = reinterpret_cast<uint32_t *>(base + p.off_gen);
    a.qtag = reinterpret_cast<uint64_t *>(base + p.off_qtag);
    a.unit_hist = reinterpret_cast<uint32_t *>(base + p.off_unit_hist);
    a.chunk_hist = reinterpret_cast<uint64_t *>(base + p.off_chunk_hist);
    a.part_ml = reinterpret_cast<float *>(base + p.off_part_ml);
    a.part_o = reinterpret_cast<float *>(base + p.off_part_o);
    a.max_ctx = p.max_ctx;
    a.B = p.B;
    a.Hkv = p.Hkv;
    a.k_max = k_max;
    a.span = p.span;
    a.n_chunks = p.n_chunks;
    a.n_items = p.n_items;
    // Bounds of the waits; HATA_DECODE_WAIT_LIMIT (a test control) lowers
    // both so that the waits give up and the stall path can be exercised.
    a.spin_limit = kSpinLimit;
    a.poll_limit = kPollLimit;
#ifdef HATA_PHASE_TRACE
    a.trace = g_trace;
    a.trace_items = g_trace_items;
#endif
    if (const char *e = getenv("HATA_DECODE_WAIT_LIMIT")) {
        const long v = strtol(e, nullptr, 10);
        if (v >= 0 && v < a.poll_limit) a.spin_limit = a.poll_limit = (int)v;
    }
    switch (p.R) {
        case 32: return launch_fused<32>(p.G, a, s);
        case 64: return launch_fused<64>(p.G, a, s);
        case 128: return launch_fused<128>(p.G, a, s);
        case 256: return launch_fused<256>(p.G, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hata

// ---------------------------------------------------------------- allocation-free form

namespace hata {

// The scratch of hata_decode_step_static.  In host code `scratch` only names
// the symbol; its device address (one per GPU) comes from
// hipGetSymbolAddress and is the only form passed to kernels or copies.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_addr[kMaxDevices];  // set once per device, never changed

hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_addr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

// Zero n 16-byte words at p (a fill kernel rather than hipMemsetAsync, so a
// captured graph replays it correctly).
__global__ __launch_bounds__(256) void k_zero16(uint4 *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t launch_decode_static(const DecodePlan &p, uint16_t *k_cache, uint16_t *v_cache,
                                uint32_t *codes, int32_t *seq_len, int32_t *ctrl,
                                const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                                const float *w, const int32_t *topk, int k_max, uint16_t *out,
                                int32_t *sel_idx_out, uint16_t *scores_out, hipStream_t s) {
    if (p.used > kStaticScratchBytes) return hipErrorInvalidValue;
    void *ws = nullptr;
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    // The launch generations, tagged code words, unit histograms and
    // cumulative span histograms must start at zero (they lie in front of
    // the split partials); the array keeps whatever the previous call on this
    // GPU left, possibly under another cache's layout.
    const int64_t n16 = (int64_t)(p.off_part_ml / 16);
    const int64_t blocks = n16 / 256 + 1 < 1024 ? n16 / 256 + 1 : 1024;
    hipLaunchKernelGGL(k_zero16, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint4 *>(ws), n16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode(p, k_cache, v_cache, codes, seq_len, ctrl, k_new, v_new, q, w, topk, k_max,
                         out, ws, sel_idx_out, scores_out, s);
}

}  // namespace hata

#ifdef HATA_PHASE_TRACE
// Trace build only: the decode launches that follow write their phase
// timestamps (see Phase in decode_fused.h) into buf, a device array of
// n_items x 16 uint64 (rows of workgroups beyond n_items are not written);
// null stops tracing.  Returns the workgroups of a launch for this cache
// (0 if the cache is not supported), so a caller can size buf first.
extern "C" int64_t hata_phase_trace(const hata_cache *c, uint64_t *buf, int64_t n_items) {
    hata::g_trace = buf;
    hata::g_trace_items = buf ? (int)(n_items < INT32_MAX ? n_items : INT32_MAX) : 0;
    hata::DecodePlan p;
    if (!c || !hata::make_decode_plan(c->batch, c->n_q_heads, c->n_kv_heads, c->max_ctx, c->n_bits, &p))
        return 0;
    return p.n_items;
}
#endif
