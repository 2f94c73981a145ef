/*
 * CPU oracle for the single-token decode step of an OLMo-3-32B-shaped decoder with
 * 4-bit group-quantised weights.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain definition that the HIP
 * path is checked against. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load it; the product path never does. It shares no
 * code with the HIP library.
 *
 * Precision policy: inputs and outputs of every operation are f32 (the pages run
 * f32 activations and an f32 KV cache); every sum, product chain, norm, angle and
 * softmax inside an operation is evaluated in double and rounded to f32 once.
 * The card's roadmap also plans a bf16 KV cache that keeps only the window on the
 * sliding-window layers ("Limitations & roadmap"); when that format is selected, a
 * key or value is rounded to bfloat16 when it is stored and read back exactly.
 *
 * Sources (titles of the pages):
 *  - "ATLAS-OLMo-3-32B-Think-v4" model card: "Quantization recipe" (packing of
 *    int4 codes: column j in word j/8, little-endian nibble; per-group scales;
 *    W4 x f32 activations; bf16 lm_head), "Architecture deep-dive" table (GQA
 *    40/8, head_dim 128, sliding window 4,096 in a [SWA,SWA,SWA,full] x16 layout,
 *    post-norm + full-projection QK RMSNorm, RoPE theta 500,000, YaRN x8 with
 *    attention_factor ~1.208), "Why the 3:1 SWA layout matters" (SWA layers never
 *    look back more than 4,096 tokens).
 *  - "Olmo 3 32B" (llm-architectures-explained): field table (post norms only,
 *    q_norm/k_norm, rotary on the full head, not parallel, untied embeddings).
 *  - "OLMo 3 32B" (LLM Architecture KB), Architecture: the post-norm sits inside
 *    each residual branch; the query and key projections are RMS-normalised
 *    before their scores are taken (the page fixes no order against the rotary
 *    step: norm first, then rotation, is the reading used here); YaRN applies to
 *    the global layers alone.
 *  - "Olmo-3-1125-32B" (archdb): RMSNorm eps 1e-6, no projection biases,
 *    SwiGLU, YaRN on full-attention layers only.
 * Readings where the pages are silent are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- number formats (IEEE 754 binary16 / bfloat16 decoding) ---------------- */

double orc_f16_to_f64(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                 /* subnormal */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1024.0 + m, e - 25);                     /* (1 + m/1024) 2^(e-15) */
    return s ? -v : v;
}

double orc_bf16_to_f64(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

/* ---- 4-bit codes ---------------------------------------------------------- */

/* Code of column j in a packed row: word j/8, nibble j%8 at bits 4(j%8)..+3, the
 * lowest nibble holding the lowest column (model card, Quantization recipe). */
static inline int nib(const uint32_t* row, int64_t j) {
    return (int)((row[j / 8] >> (4 * (j % 8))) & 15u);
}

void orc_unpack_codes(const uint32_t* qw, int64_t N, int64_t K, uint8_t* codes) {
    for (int64_t n = 0; n < N; n++)
        for (int64_t j = 0; j < K; j++) codes[n * K + j] = (uint8_t)nib(qw + n * (K / 8), j);
}

/* Scale of (row n, group g): scale_dtype 0 = binary16, 1 = bfloat16. */
static inline double scale_at(const uint16_t* sc, int64_t G, int64_t n, int64_t g, int scale_dtype) {
    uint16_t b = sc[n * G + g];
    return scale_dtype ? orc_bf16_to_f64(b) : orc_f16_to_f64(b);
}

/* Zero point of (row n, group g). Zeros are packed 8 per word along the group
 * axis with the same nibble order as the codes (our reading; the pages' format is
 * symmetric). A NULL table means the symmetric form of the model card, where the
 * stored nibble is the signed value plus 8, i.e. a zero point of 8 for every group. */
static inline int zero_at(const uint32_t* zw, int64_t G, int64_t n, int64_t g) {
    if (!zw) return 8;
    return nib(zw + n * ((G + 7) / 8), g);
}

/* Dequantised weight matrix W[n][k] = (code - zero) * scale, with the group of
 * column k being k / group and G = ceil(K / group) groups per row (a partial last
 * group covers the remaining columns). The product of an integer in [-15, 15] and
 * a 16-bit float is exact in f32. */
void orc_dequant(const uint32_t* qw, const uint16_t* sc, const uint32_t* zw, int64_t N, int64_t K,
                 int64_t group, int scale_dtype, float* W) {
    int64_t G = (K + group - 1) / group;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        const uint32_t* row = qw + n * (K / 8);
        for (int64_t k = 0; k < K; k++) {
            int64_t g = k / group;
            W[n * K + k] = (float)((double)(nib(row, k) - zero_at(zw, G, n, g)) *
                                   scale_at(sc, G, n, g, scale_dtype));
        }
    }
}

/* y = W x with W the dequantised matrix above; double accumulation per row. */
void orc_w4_gemv(const uint32_t* qw, const uint16_t* sc, const uint32_t* zw, int64_t N, int64_t K,
                 int64_t group, int scale_dtype, const float* x, float* y) {
    int64_t G = (K + group - 1) / group;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        const uint32_t* row = qw + n * (K / 8);
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++) {
            int64_t g = k / group;
            double w = (double)(nib(row, k) - zero_at(zw, G, n, g)) * scale_at(sc, G, n, g, scale_dtype);
            acc += w * (double)x[k];
        }
        y[n] = (float)acc;
    }
}

/* y = W x for a bfloat16 matrix W [N][K] (the untied lm_head); exact upcast. */
void orc_bf16_gemv(const uint16_t* W, int64_t N, int64_t K, const float* x, float* y) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++) acc += orc_bf16_to_f64(W[n * K + k]) * (double)x[k];
        y[n] = (float)acc;
    }
}

/* ---- RMSNorm -------------------------------------------------------------- */

/* y = g * x / sqrt(mean(x^2) + eps) (RMSNorm with eps 1e-6, archdb norm fields). */
void orc_rmsnorm(const float* x, const float* g, int64_t n, double eps, float* y) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; i++) ss += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; i++) y[i] = (float)((double)g[i] * ((double)x[i] * r));
}

/* out = resid + g * x / sqrt(mean(x^2) + eps): the post-norm residual update
 * h = x + RMSNorm(sublayer(x)) of the reordered post-norm block. One rounding. */
void orc_rmsnorm_residual(const float* x, const float* g, const float* resid, int64_t n, double eps,
                          float* out) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; i++) ss += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; i++)
        out[i] = (float)((double)resid[i] + (double)g[i] * ((double)x[i] * r));
}

/* ---- RoPE / YaRN ---------------------------------------------------------- */

/* Rotary inverse frequencies for a head of D dims (D/2 pairs):
 *   inv_i = theta^(-2i/D).
 * With yarn_factor s > 1 the YaRN "NTK-by-parts" interpolation is applied
 * (Peng et al. 2023): a pair that turns r_i = L * inv_i / (2 pi) times over the
 * native context L keeps its frequency when r_i is above beta_fast and is divided
 * by s when r_i is below beta_slow, with a linear ramp in between. The ramp runs
 * over pair indices between the correction-range bounds
 *   b(beta) = D * ln(L / (2 pi beta)) / (2 ln theta),
 * rounded outward (low = floor b(beta_fast), high = ceil b(beta_slow)) -- our
 * reading of the correction-range fix the model card lists for YaRN:
 *   ramp_i = clamp((i - low) / (high - low), 0, 1)
 *   inv'_i = inv_i * (1 - ramp_i) + (inv_i / s) * ramp_i.                        */
void orc_rope_inv_freq(int D, double theta, double yarn_factor, double orig_max, double beta_fast,
                       double beta_slow, double* inv) {
    int P = D / 2;
    for (int i = 0; i < P; i++) inv[i] = pow(theta, -(2.0 * i) / (double)D);
    if (!(yarn_factor > 1.0)) return;
    const double two_pi = 6.283185307179586476925286766559;
    double b_fast = (double)D * log(orig_max / (two_pi * beta_fast)) / (2.0 * log(theta));
    double b_slow = (double)D * log(orig_max / (two_pi * beta_slow)) / (2.0 * log(theta));
    double low = floor(b_fast), high = ceil(b_slow);
    if (low < 0) low = 0;
    if (high > D - 1) high = D - 1;
    for (int i = 0; i < P; i++) {
        double ramp;
        if (high > low) ramp = ((double)i - low) / (high - low);
        else ramp = (double)i > low ? 1.0 : 0.0; /* bounds coincide: a step */
        if (ramp < 0) ramp = 0;
        if (ramp > 1) ramp = 1;
        inv[i] = inv[i] * (1.0 - ramp) + (inv[i] / yarn_factor) * ramp;
    }
}

/* YaRN attention factor (the magnitude scale on the rotated q and k):
 * 0.1 ln s + 1 for s > 1, else 1. The model card prints ~1.208 for s = 8. */
double orc_yarn_attention_factor(double yarn_factor) {
    return yarn_factor > 1.0 ? 0.1 * log(yarn_factor) + 1.0 : 1.0;
}

/* Rotate H heads of D dims in place at position pos: pair (i, i + D/2) turns by
 * phi = pos * inv_i (angle and sine/cosine in double) and is scaled by mscale:
 *   x_i' = m (x_i cos phi - x_{i+D/2} sin phi),  x_{i+D/2}' = m (x_{i+D/2} cos phi + x_i sin phi).
 * Rotate-half pairing (i, i + D/2) is our reading of the field table's statement that
 * the rotation covers the whole head. */
void orc_rope(float* x, int H, int D, int64_t pos, const double* inv, double mscale) {
    int P = D / 2;
    for (int h = 0; h < H; h++) {
        float* v = x + (int64_t)h * D;
        for (int i = 0; i < P; i++) {
            double phi = (double)pos * inv[i];
            double c = cos(phi), s = sin(phi);
            double a = v[i], b = v[i + P];
            v[i] = (float)(mscale * (a * c - b * s));
            v[i + P] = (float)(mscale * (b * c + a * s));
        }
    }
}

/* ---- attention ------------------------------------------------------------ */

/* Value of element i of a cache stored as f32 (kv_dtype 0) or as bfloat16 bits
 * (kv_dtype 1: the upper half of a binary32 pattern, so the value is exact). */
static inline double kv_at(const void* base, int kv_dtype, int64_t i) {
    if (kv_dtype == 1) {
        uint32_t b = (uint32_t)((const uint16_t*)base)[i] << 16;
        float f;
        memcpy(&f, &b, 4);
        return (double)f;
    }
    return (double)((const float*)base)[i];
}

/* GQA decode attention for one new token at position pos, over a cache in its
 * storage layout: K, V are [Hkv][slots][D] of f32 or bfloat16 (kv_dtype), and key j
 * is stored in slot j mod slots when ring != 0 (a sliding-window layer that keeps only
 * its window) and in slot j otherwise. Slot of pos already holds the new key/value.
 * Query head h reads KV head h / (Hq / Hkv). The keys attended are j in [lo, pos]
 * with lo = max(0, pos - window + 1) when window > 0 (the window counts the current
 * token) and lo = 0 for full attention (window == 0).
 *   s_j = scale * q . k_j ;  p = softmax(s) (max-subtracted) ;  o = sum_j p_j v_j
 * out: [Hq][D]. Everything in double. */
void orc_attention_kv(const float* q, const void* K, const void* V, int kv_dtype, int64_t slots, int ring, int Hq,
                      int Hkv, int D, int64_t pos, int64_t window, double scale, float* out) {
    int64_t lo = window > 0 ? pos - window + 1 : 0;
    if (lo < 0) lo = 0;
    int64_t n = pos - lo + 1;
    int grp = Hq / Hkv;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < Hq; h++) {
        int kv = h / grp;
        const float* qh = q + (int64_t)h * D;
        double* s = (double*)malloc(sizeof(double) * (size_t)n);
        int64_t* row = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);   /* element offset of key lo + t */
        double mx = -INFINITY;
        for (int64_t t = 0; t < n; t++) {
            int64_t j = lo + t;
            int64_t slot = ring ? j % slots : j;
            row[t] = ((int64_t)kv * slots + slot) * D;
            double dot = 0.0;
            for (int d = 0; d < D; d++) dot += (double)qh[d] * kv_at(K, kv_dtype, row[t] + d);
            s[t] = dot * scale;
            if (s[t] > mx) mx = s[t];
        }
        double den = 0.0;
        for (int64_t t = 0; t < n; t++) {
            s[t] = exp(s[t] - mx);
            den += s[t];
        }
        for (int d = 0; d < D; d++) {
            double acc = 0.0;
            for (int64_t t = 0; t < n; t++) acc += s[t] * kv_at(V, kv_dtype, row[t] + d);
            out[(int64_t)h * D + d] = (float)(acc / den);
        }
        free(row);
        free(s);
    }
}

/* The same over an f32 cache [Hkv][T_max][D] with key j in slot j. */
void orc_attention(const float* q, const float* K, const float* V, int Hq, int Hkv, int D, int64_t T_max,
                   int64_t pos, int64_t window, double scale, float* out) {
    orc_attention_kv(q, K, V, 0, T_max, 0, Hq, Hkv, D, pos, window, scale, out);
}

/* Storing an f32 value in a bfloat16 cache: round to nearest, ties to even. The
 * upper 16 bits of the binary32 pattern are kept; one unit in their last place is
 * added when the dropped lower 16 bits exceed half a unit, or equal half a unit and
 * the kept pattern is odd. A carry out of the significand moves into the exponent,
 * so values beyond the largest bfloat16 become infinity. A NaN stays a (quiet) NaN
 * with its sign. */
void orc_round_bf16(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) {
        uint32_t b;
        memcpy(&b, &x[i], 4);
        if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) {
            out[i] = (uint16_t)((b >> 16) | 0x0040u);
            continue;
        }
        uint32_t keep = b >> 16, rest = b & 0xFFFFu;
        if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1;
        out[i] = (uint16_t)keep;
    }
}

/* ---- elementwise ---------------------------------------------------------- */

/* z = silu(u) * v with silu(t) = t / (1 + e^-t) (SwiGLU feed-forward). */
void orc_swiglu(const float* u, const float* v, int64_t n, float* z) {
    for (int64_t i = 0; i < n; i++) {
        double t = u[i];
        z[i] = (float)(t / (1.0 + exp(-t)) * (double)v[i]);
    }
}

/* Index of the largest value; the lowest index wins ties. */
int64_t orc_argmax(const float* x, int64_t n) {
    int64_t best = 0;
    for (int64_t i = 1; i < n; i++)
        if (x[i] > x[best]) best = i;
    return best;
}

/* bfloat16 row gather with exact upcast (token embedding lookup). */
void orc_embed(const uint16_t* row, int64_t d, float* x) {
    for (int64_t i = 0; i < d; i++) x[i] = (float)orc_bf16_to_f64(row[i]);
}
