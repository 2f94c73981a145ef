// On-device token sampling: temperature and nucleus (top-p) filtering with an
// inverse-CDF draw, the uniform variate given in device memory.
//
// Source: "ATLAS-OLMo-3-32B-Think-v4", Benchmarks and Prompting guide (the model is
// served with temperature 0.6 and top-p 0.95). The pages fix the settings, not the
// mechanics; the definition followed here: p_i is proportional to
// e_i = exp((l_i - max l) / T); the nucleus is the fewest most-probable tokens whose
// mass reaches top_p, tokens tied with the last one included, i.e. {i : e_i >= tau};
// the token is the first nucleus member, in ascending index order, whose cumulative
// mass exceeds u times the nucleus mass. T = 0 is greedy (lowest index on ties).
//
// No sort. Masses are summed as 64-bit integers (e_i in units of 2^-32, truncated), so
// every sum is exact and independent of order: the result is deterministic and a
// replayed graph draws the same token. tau is found by a radix select over the bit
// pattern of e (positive floats order like their patterns), one byte per pass:
//   1. sample_max_kernel   (256 blocks): per-block max and its lowest index;
//   2. sample_exp_kernel   (256 blocks): e_i = exp((l_i - max) / T) to the workspace
//      and a per-block histogram of the top byte of e_i weighted by its mass;
//   3. sample_select_kernel (one block): the top byte from the histograms, the other
//      three bytes by passes over e restricted to the prefix chosen so far, then the
//      draw: per-thread chunk masses, a block scan, and one scan inside the chunk
//      that holds the target.
#include <cmath>

#include "common.h"

namespace atlas {

constexpr int SMP_BLOCKS = 256, SMP_THREADS = 256, SMP_SEL_THREADS = 1024;
constexpr double SMP_FIX = 4294967296.0;   // 2^32: mass units per unit of e (e <= 1)
static_assert(SMP_THREADS == SMP_BLOCKS, "sample_exp_kernel reduces one block maximum per thread");

__device__ __forceinline__ uint64_t smp_mass(float e) { return (uint64_t)((double)e * SMP_FIX); }

// ---- 1. block maxima ----------------------------------------------------------------------
__global__ __launch_bounds__(SMP_THREADS) void sample_max_kernel(const float* __restrict__ l, int V, float* bmax,
                                                                 int* bidx) {
    __shared__ float sv[SMP_THREADS];
    __shared__ int si[SMP_THREADS];
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int i = blockIdx.x * SMP_THREADS + threadIdx.x; i < V; i += SMP_BLOCKS * SMP_THREADS) {
        const float v = l[i];
        if (v > best) {   // i increases, so the first index of a maximum is kept
            best = v;
            bi = i;
        }
    }
    sv[threadIdx.x] = best;
    si[threadIdx.x] = bi;
    __syncthreads();
    for (int o = SMP_THREADS / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            const float a = sv[threadIdx.x], b = sv[threadIdx.x + o];
            const int ia = si[threadIdx.x], ib = si[threadIdx.x + o];
            if (b > a || (b == a && ib < ia)) {
                sv[threadIdx.x] = b;
                si[threadIdx.x] = ib;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        bmax[blockIdx.x] = sv[0];
        bidx[blockIdx.x] = si[0];
    }
}

// ---- 2. e and the top-byte histogram ------------------------------------------------------------
__global__ __launch_bounds__(SMP_THREADS) void sample_exp_kernel(const float* __restrict__ l, int V,
                                                                 const float* __restrict__ bmax, float invT,
                                                                 float* __restrict__ e, uint64_t* __restrict__ hist) {
    __shared__ float red[SMP_THREADS];
    __shared__ unsigned long long h[256];
    red[threadIdx.x] = bmax[threadIdx.x];   // SMP_THREADS == SMP_BLOCKS
    h[threadIdx.x] = 0;
    __syncthreads();
    for (int o = SMP_THREADS / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    const float M = red[0];
    for (int i = blockIdx.x * SMP_THREADS + threadIdx.x; i < V; i += SMP_BLOCKS * SMP_THREADS) {
        const float v = expf((l[i] - M) * invT);
        const float ev = fminf(v, 1.0f);   // the maximum gives exactly 1
        e[i] = ev;
        atomicAdd(&h[__float_as_uint(ev) >> 24], (unsigned long long)smp_mass(ev));
    }
    __syncthreads();
    hist[(size_t)blockIdx.x * 256 + threadIdx.x] = h[threadIdx.x];
}

// ---- 3. threshold and draw (one block) -----------------------------------------------------------

// Chooses the bin (0..255) where the mass counted from the top bin down first reaches
// *target, and lowers *target by the mass of the bins above it. h: LDS [256]; every
// thread of the block calls it.
__device__ void smp_pick(unsigned long long* h, unsigned long long* suf, uint64_t* target, int* bin) {
    const int t = threadIdx.x;
    if (t < 256) suf[t] = h[t];
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {   // suffix sums: suf[b] = sum of h[b..255]
        unsigned long long add = 0;
        if (t < 256 && t + o < 256) add = suf[t + o];
        __syncthreads();
        if (t < 256) suf[t] += add;
        __syncthreads();
    }
    const uint64_t tg = *target;   // read by every thread before the one below lowers it
    __syncthreads();
    if (t < 256) {   // suf is non-increasing and suf[0] >= tg >= 1: exactly one bin matches
        const uint64_t above = t < 255 ? suf[t + 1] : 0;
        if (suf[t] >= tg && above < tg) {
            *bin = t;
            *target = tg - above;
        }
    }
    __syncthreads();
}

struct SampleArgs {
    const float* e;
    int V;
    const uint64_t* hist;   // [SMP_BLOCKS][256]
    const float* bmax;
    const int* bidx;
    int greedy;
    double top_p;
    const float* d_u;
    int32_t* out;
};

__global__ __launch_bounds__(SMP_SEL_THREADS) void sample_select_kernel(SampleArgs a) {
    __shared__ unsigned long long h[256], suf[256];
    __shared__ unsigned long long chunk[SMP_SEL_THREADS];
    __shared__ uint64_t s_target;
    __shared__ int s_bin;
    const int t = threadIdx.x;
    if (a.greedy) {   // first index of the maximum over the block partials
        if (t == 0) {
            float best = a.bmax[0];
            int bi = a.bidx[0];
            for (int b = 1; b < SMP_BLOCKS; b++)
                if (a.bmax[b] > best || (a.bmax[b] == best && a.bidx[b] < bi)) {
                    best = a.bmax[b];
                    bi = a.bidx[b];
                }
            *a.out = bi;
        }
        return;
    }
    // top byte: sum the block histograms
    if (t < 256) {
        unsigned long long s = 0;
        for (int b = 0; b < SMP_BLOCKS; b++) s += a.hist[(size_t)b * 256 + t];
        h[t] = s;
    }
    __syncthreads();
    if (t == 0) {
        unsigned long long tot = 0;
        for (int b = 0; b < 256; b++) tot += h[b];
        // tot < 2^53 (V < 2^21 tokens of mass <= 2^32), so the product is exact enough
        uint64_t tg = (uint64_t)ceil(a.top_p * (double)tot);
        s_target = tg < 1 ? 1 : (tg > tot ? tot : tg);
    }
    __syncthreads();
    smp_pick(h, suf, &s_target, &s_bin);
    uint32_t prefix = (uint32_t)s_bin;   // bits selected so far
    // bytes 2..4 of the threshold pattern
    for (int shift = 16; shift >= 0; shift -= 8) {
        if (t < 256) h[t] = 0;
        __syncthreads();
        auto add = [&](float ev) {
            const uint32_t b = __float_as_uint(ev);
            if ((b >> (shift + 8)) == prefix) atomicAdd(&h[(b >> shift) & 255u], (unsigned long long)smp_mass(ev));
        };
        // 16-byte loads, several in flight per thread (e is 16-byte aligned)
        const float4* e4 = reinterpret_cast<const float4*>(a.e);
        const int V4 = a.V >> 2;
#pragma unroll 4
        for (int i = t; i < V4; i += SMP_SEL_THREADS) {
            const float4 v = e4[i];
            add(v.x);
            add(v.y);
            add(v.z);
            add(v.w);
        }
        for (int i = 4 * V4 + t; i < a.V; i += SMP_SEL_THREADS) add(a.e[i]);
        __syncthreads();
        smp_pick(h, suf, &s_target, &s_bin);
        prefix = (prefix << 8) | (uint32_t)s_bin;
    }
    const uint32_t tau = prefix;
    // draw: chunk masses of the nucleus in index order, block scan, then the chunk;
    // chunks are whole 16-byte groups
    const int C = 4 * ((a.V + 4 * SMP_SEL_THREADS - 1) / (4 * SMP_SEL_THREADS));
    const int i0 = min(a.V, t * C), i1 = min(a.V, i0 + C);
    unsigned long long m = 0;
    {
        auto nmass = [&](float ev) { return __float_as_uint(ev) >= tau ? smp_mass(ev) : 0ull; };
        int i = i0;
#pragma unroll 4
        for (; i + 4 <= i1; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(a.e + i);
            m += nmass(v.x) + nmass(v.y) + nmass(v.z) + nmass(v.w);
        }
        for (; i < i1; i++) m += nmass(a.e[i]);
    }
    chunk[t] = m;
    __syncthreads();
    for (int o = 1; o < SMP_SEL_THREADS; o <<= 1) {   // inclusive scan
        const unsigned long long add = t >= o ? chunk[t - o] : 0ull;
        __syncthreads();
        chunk[t] += add;
        __syncthreads();
    }
    const unsigned long long total = chunk[SMP_SEL_THREADS - 1];
    float u = *a.d_u;
    u = u > 0.f ? u : 0.f;                      // u outside [0, 1) is clamped into it
    u = u < 1.f ? u : 0.99999994f;
    const unsigned long long tgt = (unsigned long long)((double)u * (double)total);   // < total
    const unsigned long long lo = t > 0 ? chunk[t - 1] : 0ull;
    if (lo <= tgt && tgt < chunk[t]) {          // exactly one thread: the chunk holding the target
        unsigned long long c = lo;
        for (int i = i0; i < i1; i++) {
            const float ev = a.e[i];
            if (__float_as_uint(ev) >= tau) {
                c += smp_mass(ev);
                if (c > tgt) {
                    *a.out = i;
                    break;
                }
            }
        }
    }
}

size_t sample_ws_bytes(int V) {
    return align_up((size_t)SMP_BLOCKS * 4, 256) * 2 + align_up((size_t)V * 4, 256) +
           align_up((size_t)SMP_BLOCKS * 256 * 8, 256);
}

}  // namespace atlas

using namespace atlas;

extern "C" size_t atlas_sample_workspace_bytes(int32_t vocab) {
    if (vocab < 1 || vocab > (1 << 21)) return 0;
    return sample_ws_bytes(vocab);
}

extern "C" int atlas_sample(const float* d_logits, int32_t vocab, float temperature, float top_p, const float* d_u,
                            int32_t* d_token, void* ws, size_t ws_bytes, void* stream) {
    ATLAS_CHECK_ARG(d_logits && d_token && ws, "null pointer");
    ATLAS_CHECK_ARG(vocab >= 1 && vocab <= (1 << 21), "vocab=%d outside [1, 2^21]", vocab);
    ATLAS_CHECK_ARG(std::isfinite(temperature) && temperature >= 0.f, "temperature must be finite and >= 0");
    const bool greedy = temperature == 0.f;
    ATLAS_CHECK_ARG(greedy || (top_p > 0.f && top_p <= 1.f), "top_p must be in (0, 1]");
    ATLAS_CHECK_ARG(greedy || d_u, "sampling needs the uniform variate d_u");
    const size_t need = sample_ws_bytes(vocab);
    if (ws_bytes < need) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
    char* base = (char*)ws;
    float* bmax = (float*)base;
    int* bidx = (int*)(base + align_up((size_t)SMP_BLOCKS * 4, 256));
    float* e = (float*)(base + 2 * align_up((size_t)SMP_BLOCKS * 4, 256));
    uint64_t* hist = (uint64_t*)((char*)e + align_up((size_t)vocab * 4, 256));
    hipStream_t st = (hipStream_t)stream;
    prof_mark("sample_max", st);
    ATLAS_KLAUNCH(sample_max_kernel, dim3(SMP_BLOCKS), dim3(SMP_THREADS), 0, st, d_logits, vocab, bmax, bidx);
    ATLAS_LAUNCH_CHECK("sample_max_kernel");
    if (!greedy) {
        prof_mark("sample_exp", st);
        ATLAS_KLAUNCH(sample_exp_kernel, dim3(SMP_BLOCKS), dim3(SMP_THREADS), 0, st, d_logits, vocab, bmax,
                      1.0f / temperature, e, hist);
        ATLAS_LAUNCH_CHECK("sample_exp_kernel");
    }
    SampleArgs a{};
    a.e = e;
    a.V = vocab;
    a.hist = hist;
    a.bmax = bmax;
    a.bidx = bidx;
    a.greedy = greedy ? 1 : 0;
    a.top_p = top_p;
    a.d_u = d_u;
    a.out = d_token;
    prof_mark("sample_select", st);
    ATLAS_KLAUNCH(sample_select_kernel, dim3(1), dim3(SMP_SEL_THREADS), 0, st, a);
    ATLAS_LAUNCH_CHECK("sample_select_kernel");
    return ATLAS_OK;
}
