// RMSNorm + residual, and the full-projection QK RMSNorm + rotary embedding.
//
// Sources: "OLMo 3 32B" (LLM Architecture KB) -- reordered post-norm: RMSNorm on the
// attention and feed-forward outputs inside the residual branch, and RMSNorm on Q and
// K before the dot product; "ATLAS-OLMo-3-32B-Think-v4", Architecture deep-dive --
// full-projection QK-norm, RoPE theta 500,000, YaRN x8 (8,192 -> 65,536) with
// attention_factor ~1.208; "Olmo-3-1125-32B" -- eps 1e-6, YaRN on full-attention
// layers only.
#include <cmath>

#include "norm_rope.h"

namespace atlas {

// ---- RMSNorm + residual -----------------------------------------------------------------
// One block of 1024 threads. x is the sum of S partial vectors (stride n).
// out = resid + g * x / sqrt(mean(x^2) + eps) (resid may be null). When xq.planes is
// non-null, out is also encoded for the next W4 GEMV.
__global__ __launch_bounds__(1024) void rmsnorm_residual_kernel(const float* __restrict__ xpart, int S,
                                                                const float* __restrict__ g,
                                                                const float* resid, float* out, int n,
                                                                float eps, XQ xq) {
    extern __shared__ float s_out[];   // n floats
    __shared__ float red[16];
    float ss = 0.f;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        float v = 0.f;
        for (int r = 0; r < S; r++) v += xpart[(size_t)r * n + i];
        s_out[i] = v;
        ss += v * v;
    }
    ss = block_sum(ss, red);
    const float rinv = 1.0f / sqrtf(ss / (float)n + eps);
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        float v = g[i] * (s_out[i] * rinv);
        if (resid) v += resid[i];
        s_out[i] = v;
        out[i] = v;
    }
    if (xq.planes) {
        __syncthreads();
        const int nwords = n / 8;
        for (int base = 0; base < nwords; base += blockDim.x) {
            const int t = base + threadIdx.x;
            if (t < nwords) {
                float x8[8];
#pragma unroll
                for (int i = 0; i < 8; i++) x8[i] = s_out[8 * t + i];
                xq_encode_word(x8, xq, t >> 2, t & 3);
            }
        }
    }
}

int launch_rmsnorm_residual(const float* xpart, int S, const float* g, const float* resid, float* out, int n,
                            float eps, XQ xq, hipStream_t st) {
    prof_mark("rmsnorm_residual", st);
    ATLAS_KLAUNCH(rmsnorm_residual_kernel, dim3(1), dim3(1024), (size_t)n * 4, st, xpart, S, g, resid,
                       out, n, eps, xq);
    ATLAS_LAUNCH_CHECK("rmsnorm_residual_kernel");
    return ATLAS_OK;
}

// ---- rotary tables ----------------------------------------------------------------------
// inv_i = theta^(-2i/D); YaRN by-parts (Peng et al. 2023): pairs below the
// correction range keep their frequency, pairs above it are divided by the factor,
// with a linear blend across [floor b(beta_fast), ceil b(beta_slow)],
// b(beta) = D ln(L / (2 pi beta)) / (2 ln theta). Magnitude factor 0.1 ln s + 1.
void rope_table(const atlas_rope* r, int D, RopeTable* t) {
    const int P = D / 2;
    for (int i = 0; i < P; i++) t->inv[i] = std::pow(r->theta, -(2.0 * i) / (double)D);
    t->mscale = 1.0;
    if (r->yarn_factor > 1.0) {
        const double L = r->orig_max_pos;
        const double tp = 6.283185307179586476925286766559;
        auto bound = [&](double beta) { return (double)D * std::log(L / (tp * beta)) / (2.0 * std::log(r->theta)); };
        double lo = std::floor(bound(r->beta_fast)), hi = std::ceil(bound(r->beta_slow));
        lo = std::max(lo, 0.0);
        hi = std::min(hi, (double)(D - 1));
        for (int i = 0; i < P; i++) {
            double w = hi > lo ? ((double)i - lo) / (hi - lo) : ((double)i > lo ? 1.0 : 0.0);
            w = std::min(1.0, std::max(0.0, w));
            t->inv[i] = t->inv[i] * (1.0 - w) + t->inv[i] / r->yarn_factor * w;
        }
        t->mscale = r->attention_factor > 0.0 ? r->attention_factor : 0.1 * std::log(r->yarn_factor) + 1.0;
    } else if (r->attention_factor > 0.0) {
        t->mscale = r->attention_factor;
    }
}

// ---- QK-norm + RoPE (+ KV append) ---------------------------------------------------------
// One block of 1024 threads. q (nq = Hq*D values) and k (nk = Hkv*D values) are each
// the sum of S partials with stride `pstride`. Both are RMS-normalised over the whole
// projection, multiplied by their gains, rotated pairwise (i, i + D/2) by pos*inv_i
// and scaled by m. Results go to q_out / k_out; when k_cache is non-null, the rotated
// k and the raw v go to slot pos of the caches ([Hkv][T_max][D]).
__global__ __launch_bounds__(1024) void qk_norm_rope_kernel(QkArgs a) {
    extern __shared__ float sh[];   // nq + nk floats
    __shared__ float red[16];
    __shared__ float s_cos[128], s_sin[128];
    __shared__ int s_ok;
    const int nq = a.Hq * a.D, nk = a.Hkv * a.D, P = a.D / 2;
    float* sq = sh;
    float* sk = sh + nq;
    if (threadIdx.x == 0) {
        const int pos = *a.d_pos;
        int ok = pos >= 0 && (!a.k_cache || pos < a.T_max);
        s_ok = ok;
        if (!ok && a.status) *a.status = ATLAS_ERR_INVALID_ARG;
    }
    float ssq = 0.f, ssk = 0.f;
    for (int i = threadIdx.x; i < nq + nk; i += blockDim.x) {
        const float* src = i < nq ? a.q + i : a.k + (i - nq);
        float v = 0.f;
        for (int r = 0; r < a.S; r++) v += src[(size_t)r * a.pstride];
        sh[i] = v;
        if (i < nq) ssq += v * v; else ssk += v * v;
    }
    ssq = block_sum(ssq, red);
    ssk = block_sum(ssk, red);
    const int pos = *a.d_pos;
    if (threadIdx.x < P) {
        double s, c;
        sincos((double)pos * a.rope.inv[threadIdx.x], &s, &c);
        s_cos[threadIdx.x] = (float)(c * a.rope.mscale);
        s_sin[threadIdx.x] = (float)(s * a.rope.mscale);
    }
    const float rq = 1.0f / sqrtf(ssq / (float)nq + a.eps);
    const float rk = 1.0f / sqrtf(ssk / (float)nk + a.eps);
    for (int i = threadIdx.x; i < nq; i += blockDim.x) sq[i] = a.gq[i] * (sq[i] * rq);
    for (int i = threadIdx.x; i < nk; i += blockDim.x) sk[i] = a.gk[i] * (sk[i] * rk);
    __syncthreads();
    // rotate: one thread per pair
    const int npairs = (a.Hq + a.Hkv) * P;
    for (int t = threadIdx.x; t < npairs; t += blockDim.x) {
        const int h = t / P, i = t % P;
        float* base = h < a.Hq ? sq + h * a.D : sk + (h - a.Hq) * a.D;
        const float x0 = base[i], x1 = base[i + P];
        const float c = s_cos[i], s = s_sin[i];
        const float y0 = x0 * c - x1 * s;
        const float y1 = x1 * c + x0 * s;
        if (h < a.Hq) {
            a.q_out[h * a.D + i] = y0;
            a.q_out[h * a.D + i + P] = y1;
        } else {
            const int hk = h - a.Hq;
            if (a.k_out) {
                a.k_out[hk * a.D + i] = y0;
                a.k_out[hk * a.D + i + P] = y1;
            }
            if (a.k_cache && s_ok) {
                float* dst = a.k_cache + ((size_t)hk * a.T_max + pos) * a.D;
                dst[i] = y0;
                dst[i + P] = y1;
            }
        }
    }
    if (a.v_cache && s_ok) {
        for (int i = threadIdx.x; i < nk; i += blockDim.x) {
            float v = 0.f;
            for (int r = 0; r < a.S; r++) v += a.v[(size_t)r * a.pstride + i];
            const int hk = i / a.D, dd = i % a.D;
            a.v_cache[((size_t)hk * a.T_max + pos) * a.D + dd] = v;
        }
    }
}

int launch_qk_norm_rope(const QkArgs& a, hipStream_t st) {
    const size_t sh = (size_t)(a.Hq + a.Hkv) * a.D * 4;
    prof_mark("qk_norm_rope", st);
    ATLAS_KLAUNCH(qk_norm_rope_kernel, dim3(1), dim3(1024), sh, st, a);
    ATLAS_LAUNCH_CHECK("qk_norm_rope_kernel");
    return ATLAS_OK;
}

}  // namespace atlas

using namespace atlas;

extern "C" int atlas_rmsnorm_residual(const float* x, const float* g, const float* resid, float* out, int32_t n,
                                      float eps, void* stream) {
    ATLAS_CHECK_ARG(x && g && out, "null pointer");
    ATLAS_CHECK_ARG(n >= 1 && n <= 16384, "n=%d out of range [1, 16384]", n);
    ATLAS_CHECK_ARG(eps >= 0.f, "eps must be >= 0");
    return launch_rmsnorm_residual(x, 1, g, resid, out, n, eps, XQ{}, (hipStream_t)stream);
}

extern "C" int atlas_qk_norm_rope(float* q, float* k, const float* gq, const float* gk, int32_t Hq, int32_t Hkv,
                                  int32_t D, const int32_t* d_pos, const atlas_rope* rope, float eps,
                                  void* stream) {
    ATLAS_CHECK_ARG(q && k && gq && gk && d_pos && rope, "null pointer");
    ATLAS_CHECK_ARG(Hq >= 1 && Hkv >= 1, "bad head counts");
    ATLAS_CHECK_SHAPE(D >= 2 && D % 2 == 0 && D <= 256, "D=%d must be even and <= 256", D);
    ATLAS_CHECK_SHAPE((size_t)(Hq + Hkv) * D * 4 <= 60 * 1024, "projection too large for one block");
    ATLAS_CHECK_ARG(rope->theta > 1.0, "theta must be > 1");
    QkArgs a{};
    a.q = q;
    a.k = k;
    a.v = nullptr;
    a.S = 1;
    a.pstride = 0;
    a.gq = gq;
    a.gk = gk;
    a.q_out = q;
    a.k_out = k;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.eps = eps;
    a.d_pos = d_pos;
    rope_table(rope, D, &a.rope);
    return launch_qk_norm_rope(a, (hipStream_t)stream);
}
