/*
 * Seeded, counter-based synthetic input generator.
 *
 * This module is input infrastructure only: it turns (seed, tensor id, element
 * index) into bits with a published mixing function and maps those bits onto the
 * value distributions of the workloads. It contains none of the decode step's
 * arithmetic. Both the CPU oracle runner and the GPU harness draw every input from
 * here, so the two sides see identical bits.
 *
 * Bit source: the SplitMix64 output finaliser (Steele, Lea & Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), used counter-style:
 *     mix64(z)   = three xor-shift / multiply rounds (constants of SplitMix64)
 *     key(s, t)  = mix64(mix64(s + GAMMA) + t * GAMMA)
 *     h(key, i)  = mix64(key + (i + 1) * GAMMA)            (all mod 2^64)
 * where GAMMA = 0x9E3779B97F4A7C15 is SplitMix64's increment, s the seed and t a
 * 64-bit tensor id chosen by the caller.
 *
 * Distributions (element i of a tensor with key k):
 *   packed uint4 codes : word i = high 32 bits of h(k, i); its 8 nibbles are 8
 *                        independent U{0..15} codes.
 *   U(a, b) -> f16     : u = (h(k,i) >> 40) * 2^-24 (exact), v = a + (b - a) * u in
 *                        double, rounded once to nearest-even binary16.
 *   N(mu, sigma) -> f32: Irwin-Hall sum of twelve 16-bit fields taken from
 *                        h(k,3i), h(k,3i+1), h(k,3i+2) (four fields each, low to
 *                        high); z = (sum - 393210) / 65536 is exact in f32;
 *                        value = mu + sigma * z evaluated in f32 (no contraction).
 *   N(mu, sigma) -> bf16: the f32 value above rounded to nearest-even bfloat16.
 *   tokens U{0..V-1}   : ((h(k,i) >> 32) * V) >> 32.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC synth.c -o libsynth.so
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tensor_id) {
    return mix64(mix64(seed + GAMMA) + tensor_id * GAMMA);
}

uint64_t synth_hash(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static inline uint64_t H(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* Round a finite double to the nearest binary16 (ties to even). */
static uint16_t f64_to_f16_rne(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (!(a < 65520.0)) return (uint16_t)(sign | 0x7C00);
    int e;
    frexp(a, &e);              /* a = m * 2^e with m in [0.5, 1) */
    int u = e - 1;             /* unbiased exponent of a */
    if (u < -14) u = -14;      /* subnormal quantum is 2^-24 */
    double q = ldexp(1.0, u - 10);
    double r = nearbyint(a / q); /* a / q is exact; default mode rounds to even */
    uint32_t ri = (uint32_t)r;
    uint16_t out;
    if (u == -14 && ri < 1024) {
        out = (uint16_t)ri;
    } else {
        if (ri == 2048) { ri = 1024; u++; }
        out = (uint16_t)(((u + 15) << 10) | (ri - 1024));
    }
    return (uint16_t)(sign | out);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    uint32_t bias = 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)((b + bias) >> 16);
}

static inline float irwin_hall12(uint64_t key, uint64_t i) {
    uint64_t s = 0;
    for (int r = 0; r < 3; r++) {
        uint64_t h = H(key, 3 * i + r);
        s += (h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + (h >> 48);
    }
    return (float)((int64_t)s - 393210) / 65536.0f;
}

/* out[i] = 8 packed U{0..15} codes, i in [0, n). */
void synth_codes_u32(uint64_t key, int64_t n, uint32_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (uint32_t)(H(key, i) >> 32);
}

/* Packed uint4 zero points for an [N][G] grid stored as [N][ceil(G/8)] words.
 * Element (n, word w) is drawn from index n*ceil(G/8)+w; nibbles past G are 0. */
void synth_zeros_u32(uint64_t key, int64_t N, int64_t G, uint32_t* out) {
    int64_t GW = (G + 7) / 8;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t w = 0; w < GW; w++) {
            uint32_t v = (uint32_t)(H(key, n * GW + w) >> 32);
            int64_t valid = G - 8 * w;
            if (valid < 8) v &= (uint32_t)((1ull << (4 * valid)) - 1);
            out[n * GW + w] = v;
        }
    }
}

void synth_uniform_f16(uint64_t key, int64_t n, double a, double b, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double u = (double)(H(key, i) >> 40) * (1.0 / 16777216.0);
        out[i] = f64_to_f16_rne(a + (b - a) * u);
    }
}

/* Uniform U(a,b) rounded to bfloat16: the double value is rounded to f32 and the
 * f32 to bfloat16 (both nearest-even). Used for bfloat16 group scales. */
void synth_uniform_bf16(uint64_t key, int64_t n, double a, double b, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double u = (double)(H(key, i) >> 40) * (1.0 / 16777216.0);
        double v = a + (b - a) * u;
        out[i] = f32_to_bf16_rne((float)v);
    }
}

/* N(mu, sigma) in f32 into a strided 3-D destination:
 * element (a, b, c) has value index (a*B + b)*C + c and lands at
 * out[a*sa + b*sb + c]. A plain vector is A = B = 1. */
void synth_normal_f32_3d(uint64_t key, int64_t A, int64_t B, int64_t C, int64_t sa, int64_t sb,
                         float mu, float sigma, float* out) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t a = 0; a < A; a++) {
        for (int64_t b = 0; b < B; b++) {
            float* dst = out + a * sa + b * sb;
            uint64_t base = (uint64_t)((a * B + b) * C);
            for (int64_t c = 0; c < C; c++) {
                float z = irwin_hall12(key, base + (uint64_t)c);
                float t = sigma * z;
                dst[c] = mu + t;
            }
        }
    }
}

/* One layer's K or V cache in its storage layout. Element (a, j, c) of the N(mu, sigma)
 * stream has the value index of synth_normal_f32_3d with B positions, (a*B + j)*C + c,
 * so a position's values do not depend on the layout. Positions j in [j0, B) land in
 * slot j mod slots of head a, out[(a*slots + j mod slots)*C + c], as f32 (dtype 0) or
 * as bf16 bits rounded to nearest even (dtype 1). A flat cache is slots >= B, j0 = 0;
 * a ring of W slots holding the last W positions is slots = W, j0 = max(0, B - W). */
void synth_normal_kv(uint64_t key, int64_t A, int64_t B, int64_t C, int64_t j0, int64_t slots, int dtype,
                     float mu, float sigma, void* out) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t a = 0; a < A; a++) {
        for (int64_t j = j0; j < B; j++) {
            const int64_t o = (a * slots + j % slots) * C;
            const uint64_t base = (uint64_t)((a * B + j) * C);
            for (int64_t c = 0; c < C; c++) {
                float v = mu + sigma * irwin_hall12(key, base + (uint64_t)c);
                if (dtype == 1)
                    ((uint16_t*)out)[o + c] = f32_to_bf16_rne(v);
                else
                    ((float*)out)[o + c] = v;
            }
        }
    }
}

void synth_normal_f32(uint64_t key, int64_t n, float mu, float sigma, float* out) {
    synth_normal_f32_3d(key, 1, 1, n, 0, 0, mu, sigma, out);
}

/* Rows [r0, r0+nr) of an N(mu, sigma) bf16 matrix with C columns (value index
 * r*C + c), written densely to out[(r-r0)*C + c]. */
void synth_normal_bf16_rows(uint64_t key, int64_t r0, int64_t nr, int64_t C, float mu, float sigma,
                            uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nr; r++) {
        for (int64_t c = 0; c < C; c++) {
            float z = irwin_hall12(key, (uint64_t)((r0 + r) * C + c));
            float t = sigma * z;
            out[r * C + c] = f32_to_bf16_rne(mu + t);
        }
    }
}

void synth_tokens(uint64_t key, int64_t n, int64_t vocab, int32_t* out) {
    for (int64_t i = 0; i < n; i++)
        out[i] = (int32_t)(((H(key, i) >> 32) * (uint64_t)vocab) >> 32);
}

/* Raw hash words, for the generator's own tests. */
void synth_raw(uint64_t key, int64_t n, uint64_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = H(key, i);
}

/* f64 -> f16 conversion exported for the generator's own tests. */
uint16_t synth_f64_to_f16(double v) { return f64_to_f16_rne(v); }
