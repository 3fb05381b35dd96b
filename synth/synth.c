/*
 * Seeded synthetic input generator shared by the GPU path's tests/bench and
 * by the CPU oracle.  It holds random numbers and rounding only; none of the
 * hashing, scoring, selection or attention arithmetic lives here.
 *
 * Definitions (all published, restated here):
 *   - SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): the state advances by the golden-ratio
 *     increment 0x9E3779B97F4A7C15 and each output is the state passed
 *     through the variant-13 finaliser (xor-shift 30, multiply
 *     0xBF58476D1CE4E5B9, xor-shift 27, multiply 0x94D049BB133111EB,
 *     xor-shift 31).  Because the state is linear in the output number, the
 *     c-th output of a stream is computable directly: a counter-based
 *     generator.
 *   - A stream is named by (seed, tensor id): its starting state is output
 *     number `tensor` of the stream whose state starts at `seed`.
 *   - Uniforms: u = ((x >> 11) + 1) * 2^-53 lies in (0, 1]; v = (x >> 11) *
 *     2^-53 lies in [0, 1).
 *   - Normals: Box-Muller (1958).  Element i uses the pair p = i >> 1:
 *     u from output 2p, v from output 2p + 1, radius sqrt(-2 ln u), angle
 *     2*pi*v; even i takes the cosine branch, odd i the sine branch.
 *   - Narrowing: double -> float (round to nearest even, C cast) -> bf16
 *     (round to nearest even on the upper 16 bits).
 *
 * Plain C, single-threaded; callers split index ranges across threads.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_finalise(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Output number c (0-based) of the SplitMix64 stream whose state starts at s. */
static inline uint64_t sm64_output(uint64_t s, uint64_t c) {
    return sm64_finalise(s + (c + 1) * SM64_GAMMA);
}

static inline uint64_t stream_state(uint64_t seed, uint64_t tensor) {
    return sm64_output(seed, tensor);
}

static void normal_pair(uint64_t state, uint64_t p, double *z0, double *z1) {
    const double two_pi = 6.283185307179586476925286766559;
    double u = (double)((sm64_output(state, 2 * p) >> 11) + 1) * 0x1p-53;
    double v = (double)(sm64_output(state, 2 * p + 1) >> 11) * 0x1p-53;
    double rad = sqrt(-2.0 * log(u));
    double ang = two_pi * v;
    *z0 = rad * cos(ang);
    *z1 = rad * sin(ang);
}

/* Normals [start, start + count) of stream `state`, times `scale`, into out[]. */
static void normal_range(uint64_t state, uint64_t start, int64_t count, double scale,
                         double *out) {
    int64_t i = 0;
    while (i < count) {
        uint64_t e = start + (uint64_t)i;
        double z0, z1;
        normal_pair(state, e >> 1, &z0, &z1);
        if ((e & 1) == 0) {
            out[i++] = scale * z0;
            if (i < count) out[i++] = scale * z1;
        } else {
            out[i++] = scale * z1;
        }
    }
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) /* NaN: keep quiet */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* Raw SplitMix64 outputs, numbers [start, start + count) of stream (seed, tensor). */
void synth_u64(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count, uint64_t *out) {
    uint64_t s = stream_state(seed, tensor);
    for (int64_t i = 0; i < count; ++i) out[i] = sm64_output(s, start + (uint64_t)i);
}

/* The plain SplitMix64 stream seeded with `seed` (for the published test vector). */
void synth_sm64_stream(uint64_t seed, int64_t count, uint64_t *out) {
    for (int64_t i = 0; i < count; ++i) out[i] = sm64_output(seed, (uint64_t)i);
}

void synth_normal_f64(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count,
                      double scale, double *out) {
    normal_range(stream_state(seed, tensor), start, count, scale, out);
}

void synth_normal_f32(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count,
                      double scale, float *out) {
    uint64_t st = stream_state(seed, tensor);
    double buf[512];
    for (int64_t i = 0; i < count; i += 512) {
        int64_t n = count - i < 512 ? count - i : 512;
        normal_range(st, start + (uint64_t)i, n, scale, buf);
        for (int64_t j = 0; j < n; ++j) out[i + j] = (float)buf[j];
    }
}

void synth_normal_bf16(uint64_t seed, uint64_t tensor, uint64_t start, int64_t count,
                       double scale, uint16_t *out) {
    uint64_t st = stream_state(seed, tensor);
    double buf[512];
    for (int64_t i = 0; i < count; i += 512) {
        int64_t n = count - i < 512 ? count - i : 512;
        normal_range(st, start + (uint64_t)i, n, scale, buf);
        for (int64_t j = 0; j < n; ++j) out[i + j] = f32_to_bf16_rne((float)buf[j]);
    }
}

void synth_f64_to_bf16(const double *x, int64_t count, uint16_t *out) {
    for (int64_t i = 0; i < count; ++i) out[i] = f32_to_bf16_rne((float)x[i]);
}
