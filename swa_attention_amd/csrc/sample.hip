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
// No sort of the vocabulary. Masses are summed as 64-bit integers (e_i in units of
// 2^-32, truncated), so every sum is exact and independent of order: the result is
// deterministic and a replayed graph draws the same token. tau is the bit pattern of e
// (positive floats order like their patterns) where the mass counted from the top
// first reaches ceil(top_p * total). Each block of the first three kernels owns a
// contiguous slice of the vocabulary:
//   1. sample_max_kernel  (256 blocks): per-slice max and its lowest index; clears the
//      histogram;
//   2. sample_exp_kernel  (256 blocks): e_i to the workspace and its mass added to a
//      histogram over the top 12 bits of e's pattern (sign, exponent and 3 mantissa
//      bits): an LDS histogram per block, then one integer atomic per non-empty bin;
//   3. sample_bin_kernel  (256 blocks): every block finds the 12-bit bin that holds
//      tau, sums the mass of its slice above that bin (certainly in the nucleus) and
//      writes the (index, e) of its elements inside the bin, the candidates, to its own
//      region in index order;
//   4. sample_draw_kernel (one block): the low 20 bits of tau: bits [19:12] from a
//      histogram of the candidates that the bin kernel adds up, then the few candidates
//      with that prefix resolved by one wave (radix passes of 8 and 4 bits over the
//      candidates when there are many), one thread per slice holding the slice's first
//      candidates in registers; each slice's nucleus mass (its
//      certain mass plus its candidates at or above tau); the slice holding the target
//      u * mass from a scan of the 256 slice masses; the token from a scan inside it.
#include <cmath>

#include "common.h"

namespace atlas {

constexpr int SMP_BLOCKS = 256, SMP_THREADS = 256, SMP_DRAW_THREADS = 256;
// e <= 1, so the top 12 bits of its pattern are at most 0x3F8: 1,024 bins hold them.
constexpr int SMP_BINS = 1024, SMP_SHIFT = 20;
// The histogram is kept in one copy per XCD (block b adds to copy b mod 8, the XCD it
// runs on), so the atomics of different XCDs never contend for one address.
constexpr int SMP_COPIES = 8;
constexpr int SMP_PF = 2;                  // slice elements per thread loaded ahead (slices of up to 512 at once)
constexpr int SMP_CAND_PF = 16;            // candidates per slice the draw loads with the counts
constexpr int SMP_SEL_MAX = 64;            // candidates with tau's 20-bit prefix that one wave resolves
constexpr double SMP_FIX = 4294967296.0;   // 2^32: mass units per unit of e (e <= 1)
static_assert(SMP_THREADS == SMP_BLOCKS, "sample_exp_kernel reduces one block maximum per thread");

__device__ __forceinline__ uint64_t smp_mass(float e) { return (uint64_t)((double)e * SMP_FIX); }
__device__ __forceinline__ uint64_t smp_mass_bits(uint32_t b) { return smp_mass(__uint_as_float(b)); }

// Contiguous slice of block b: [b * sl, min(V, (b + 1) * sl)).
__host__ __device__ inline int smp_slice(int V) { return ((V + SMP_BLOCKS - 1) / SMP_BLOCKS + 3) & ~3; }

struct SampleWs {
    float* bmax;
    int* bidx;
    float* e;                  // [V]
    uint64_t* hist;            // [SMP_COPIES][SMP_BINS] masses by the top 12 bits of e's pattern
    uint64_t* hist2;           // [SMP_COPIES][256] masses of the candidates by bits [19:12]
    uint64_t* certain;         // [SMP_BLOCKS] nucleus mass above tau's bin, per slice
    uint32_t* ncand;           // [SMP_BLOCKS] candidates of each slice
    uint2* cand;               // [SMP_BLOCKS][slice] (index, bits of e) of each slice's elements
                               //   inside tau's bin, in index order
    uint64_t* sel;             // [4]: bin, remaining target, total mass
};

// Block-wide exclusive scan of one 64-bit value per thread (blockDim.x a multiple of 64,
// at most 1024), with the total: DPP scans inside each wave, then the wave totals
// through LDS. wsum: LDS [16]. Every thread of the block calls it.
// A DPP move of a 64-bit value (both halves); lanes without a source, and the rows
// outside ROWS, read 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xF, true);
    return ((uint64_t)hi << 32) | lo;
}
// Inclusive scan over the 64 lanes of a wave: shifts by 1, 2, 4 and 8 lanes inside each
// row of 16 (row_shr), then each row's last lane broadcast to the next row (row_bcast:15
// into rows 1 and 3) and lane 31 to the upper half (row_bcast:31 into rows 2 and 3).
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
    x += dpp_u64<0x111>(x);
    x += dpp_u64<0x112>(x);
    x += dpp_u64<0x114>(x);
    x += dpp_u64<0x118>(x);
    x += dpp_u64<0x142, 0xA>(x);
    x += dpp_u64<0x143, 0xC>(x);
    return x;
}

__device__ uint64_t block_excl_scan(uint64_t v, uint64_t* wsum, uint64_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint64_t x = wave_incl_scan_u64(v);
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    uint64_t off = 0, tot = 0;
    for (int i = 0; i < nw; i++) {
        const uint64_t sw = wsum[i];
        off += i < w ? sw : 0ull;
        tot += sw;
    }
    *total = tot;
    __syncthreads();   // wsum is free for the next call
    return off + x - v;
}

// ---- 1. slice maxima --------------------------------------------------------------------
__global__ __launch_bounds__(SMP_THREADS) void sample_max_kernel(const float* __restrict__ l, int V, SampleWs w,
                                                                 int clear) {
    __shared__ float sv[SMP_THREADS];
    __shared__ int si[SMP_THREADS];
    const int sl = smp_slice(V), i0 = blockIdx.x * sl, i1 = min(V, i0 + sl);
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int i = i0 + threadIdx.x; i < i1; i += SMP_THREADS) {
        const float v = l[i];
        if (v > best) {   // i increases, so the first index of a maximum is kept
            best = v;
            bi = i;
        }
    }
    sv[threadIdx.x] = best;
    si[threadIdx.x] = bi;
    if (clear) {   // the histogram starts at zero
        for (int b = blockIdx.x * SMP_THREADS + threadIdx.x; b < SMP_COPIES * SMP_BINS; b += SMP_BLOCKS * SMP_THREADS)
            w.hist[b] = 0;
        for (int b = blockIdx.x * SMP_THREADS + threadIdx.x; b < SMP_COPIES * 256; b += SMP_BLOCKS * SMP_THREADS)
            w.hist2[b] = 0;
    }
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
        w.bmax[blockIdx.x] = sv[0];
        w.bidx[blockIdx.x] = si[0];
    }
}

// ---- 2. e and the histogram ------------------------------------------------------------------
__global__ __launch_bounds__(SMP_THREADS) void sample_exp_kernel(const float* __restrict__ l, int V, float invT,
                                                                 SampleWs w) {
    __shared__ float red[SMP_THREADS];
    __shared__ unsigned long long hb[SMP_BINS];
    // the slice's first logits are loaded with the slice maxima (they do not depend on
    // the maximum), so both loads are in flight together
    const int sl = smp_slice(V), i0 = blockIdx.x * sl, i1 = min(V, i0 + sl);
    float pre[SMP_PF];
#pragma unroll
    for (int k = 0; k < SMP_PF; k++) {
        const int i = i0 + (int)threadIdx.x + k * SMP_THREADS;
        pre[k] = l[i < i1 ? i : V - 1];   // (a clamped, unused load past the slice)
    }
    red[threadIdx.x] = w.bmax[threadIdx.x];   // SMP_THREADS == SMP_BLOCKS
    for (int b = threadIdx.x; b < SMP_BINS; b += SMP_THREADS) hb[b] = 0;
    __syncthreads();
    for (int o = SMP_THREADS / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    const float M = red[0];
    auto put = [&](int i, float li) {
        const float v = expf((li - M) * invT);
        const float ev = fminf(v, 1.0f);   // the maximum gives exactly 1
        w.e[i] = ev;
        const uint64_t ms = smp_mass(ev);
        if (ms) atomicAdd(&hb[__float_as_uint(ev) >> SMP_SHIFT], (unsigned long long)ms);
    };
#pragma unroll
    for (int k = 0; k < SMP_PF; k++) {
        const int i = i0 + (int)threadIdx.x + k * SMP_THREADS;
        if (i < i1) put(i, pre[k]);
    }
    for (int i = i0 + threadIdx.x + SMP_PF * SMP_THREADS; i < i1; i += SMP_THREADS) put(i, l[i]);
    __syncthreads();
    uint64_t* dst = w.hist + (size_t)(blockIdx.x % SMP_COPIES) * SMP_BINS;
    for (int b = threadIdx.x; b < SMP_BINS; b += SMP_THREADS)
        if (hb[b]) atomicAdd((unsigned long long*)&dst[b], hb[b]);
}

// ---- 3. tau's bin, certain masses and the candidate list ---------------------------------------
__global__ __launch_bounds__(SMP_THREADS) void sample_bin_kernel(int V, double top_p, SampleWs w) {
    __shared__ uint64_t tmp[16];
    __shared__ int s_bin;
    __shared__ uint64_t s_rem;
    const int t = threadIdx.x;
    // thread t holds the 4 bins [4 (255 - t), 4 (255 - t) + 4): thread 0 the highest
    constexpr int BPT = SMP_BINS / SMP_THREADS;
    const int b0 = (SMP_THREADS - 1 - t) * BPT;
    // thread t's consecutive elements [j0, j1) of the slice (below), their first SMP_PF
    // patterns loaded with the histogram (they do not depend on the bin)
    const int sl = smp_slice(V), i0 = blockIdx.x * sl, i1 = min(V, i0 + sl);
    const int per = (sl + SMP_THREADS - 1) / SMP_THREADS;
    const int j0 = min(i1, i0 + t * per), j1 = min(i1, j0 + per);
    uint32_t pe[SMP_PF];
#pragma unroll
    for (int k = 0; k < SMP_PF; k++) pe[k] = __float_as_uint(w.e[j0 + k < j1 ? j0 + k : V - 1]);
    auto bits_at = [&](int i) {
        uint32_t b = 0u;
#pragma unroll
        for (int k = 0; k < SMP_PF; k++) b = i == j0 + k ? pe[k] : b;
        return i - j0 < SMP_PF ? b : __float_as_uint(w.e[i]);
    };
    uint64_t hv[BPT] = {};
#pragma unroll
    for (int c = 0; c < SMP_COPIES; c++)
#pragma unroll
        for (int k = 0; k < BPT; k++) hv[k] += w.hist[(size_t)c * SMP_BINS + b0 + k];
    uint64_t own = 0;
#pragma unroll
    for (int k = 0; k < BPT; k++) own += hv[k];
    uint64_t total;
    const uint64_t above = block_excl_scan(own, tmp, &total);
    uint64_t tg = (uint64_t)ceil(top_p * (double)total);   // total < 2^53: exact enough
    tg = tg < 1 ? 1 : (tg > total ? total : tg);
    if (above < tg && above + own >= tg) {   // exactly one thread (own > 0)
        uint64_t c = above;
        for (int k = BPT - 1; k >= 0; k--) {
            if (c + hv[k] >= tg) {
                s_bin = b0 + k;
                s_rem = tg - c;
                break;
            }
            c += hv[k];
        }
    }
    __syncthreads();
    const uint32_t bin = (uint32_t)s_bin;
    if (blockIdx.x == 0 && t == 0) {
        w.sel[0] = bin;
        w.sel[1] = s_rem;
        w.sel[2] = total;
    }
    // this slice: mass above the bin, and its candidates in index order (thread t takes
    // the consecutive elements [i0 + t * per, i0 + (t + 1) * per) of the slice)
    uint64_t cm = 0, nmine = 0;
    for (int i = j0; i < j1; i++) {
        const uint32_t bits = bits_at(i);
        const uint32_t hbin = bits >> SMP_SHIFT;
        if (hbin > bin) cm += smp_mass_bits(bits);
        nmine += hbin == bin;
    }
    uint64_t nblk, blk;
    uint32_t pos = (uint32_t)block_excl_scan(nmine, tmp, &nblk);
    uint2* dst = w.cand + (size_t)blockIdx.x * sl;
    unsigned long long* h2 = (unsigned long long*)w.hist2 + (size_t)(blockIdx.x % SMP_COPIES) * 256;
    for (int i = j0; i < j1 && nmine; i++) {
        const uint32_t bits = bits_at(i);
        if ((bits >> SMP_SHIFT) == bin) {
            dst[pos++] = make_uint2((uint32_t)i, bits);
            // the draw's first radix pass: candidate masses by bits [19:12]
            atomicAdd(&h2[(bits >> 12) & 0xFFu], (unsigned long long)smp_mass_bits(bits));
        }
    }
    block_excl_scan(cm, tmp, &blk);   // block sum
    if (t == 0) {
        w.certain[blockIdx.x] = blk;
        w.ncand[blockIdx.x] = (uint32_t)nblk;
    }
}

// ---- 4. tau and the draw (one block) --------------------------------------------------------------

struct DrawArgs {
    SampleWs w;
    int V;
    int greedy;
    const float* d_u;
    int32_t* out;
};

__global__ __launch_bounds__(SMP_DRAW_THREADS) void sample_draw_kernel(DrawArgs a) {
    __shared__ unsigned long long h[256];
    __shared__ uint64_t tmp[16];
    __shared__ uint64_t s_target, s_lo;
    __shared__ int s_bin, s_blk;
    __shared__ uint32_t s_k, s_tau, s_sel[SMP_SEL_MAX];
    const int t = threadIdx.x;
    const SampleWs& w = a.w;
    if (a.greedy) {   // first index of the maximum over the slice partials
        if (t == 0) {
            float best = w.bmax[0];
            int bi = w.bidx[0];
            for (int b = 1; b < SMP_BLOCKS; b++)
                if (w.bmax[b] > best || (w.bmax[b] == best && w.bidx[b] < bi)) {
                    best = w.bmax[b];
                    bi = w.bidx[b];
                }
            *a.out = bi;
        }
        return;
    }
    // Thread t owns slice t: its candidate count, certain mass and first SMP_CAND_PF
    // candidates (loaded before it is known which exist; slice regions start at multiples
    // of 4 entries, so they are 16-byte aligned), and bin 255 - t of the bin kernel's
    // histogram of the candidates by bits [19:12] (thread 0 the highest).
    static_assert(SMP_DRAW_THREADS == SMP_BLOCKS, "one thread per slice");
    const int sl = smp_slice(a.V);
    uint2 pre[SMP_CAND_PF];
    {
        const uint4* src = reinterpret_cast<const uint4*>(w.cand + (size_t)t * sl);
#pragma unroll
        for (int k = 0; k < SMP_CAND_PF / 2; k++) {
            const uint4 q = src[min(k, sl / 2 - 1)];
            pre[2 * k] = make_uint2(q.x, q.y);
            pre[2 * k + 1] = make_uint2(q.z, q.w);
        }
    }
    const uint32_t cb = w.ncand[t];
    const uint64_t cert = w.certain[t];
    uint64_t h2own = 0;
#pragma unroll
    for (int c = 0; c < SMP_COPIES; c++) h2own += w.hist2[(size_t)c * 256 + 255 - t];
    if (t == 0) {
        s_target = w.sel[1];
        s_k = 0u;
        s_tau = 0u;
    }
    float u = *a.d_u;
    // f(bits) over this slice's candidates: the prefetched ones, then any further ones
    auto each_cand = [&](auto f) {
#pragma unroll
        for (int k = 0; k < SMP_CAND_PF; k++)
            if ((uint32_t)k < cb) f(pre[k].y);
        for (uint32_t k = SMP_CAND_PF; k < cb; k++) f(w.cand[(size_t)t * sl + k].y);
    };
    // low 20 bits of tau. Bits [19:12]: the bin (highest first) where the candidates' mass
    // from the top reaches the remaining target.
    uint32_t prefix = (uint32_t)w.sel[0];
    {
        uint64_t tot;
        __syncthreads();   // s_target
        const uint64_t tg = s_target;
        const uint64_t above = block_excl_scan(h2own, tmp, &tot);
        if (above < tg && above + h2own >= tg) {   // exactly one thread (h2own > 0)
            s_bin = 255 - t;
            s_target = tg - above;
        }
        __syncthreads();
        prefix = (prefix << 8) | (uint32_t)s_bin;
    }
    // The candidates with this 20-bit prefix (a handful, typically): with at most
    // SMP_SEL_MAX of them, tau is the largest pattern b among them whose mass at or above
    // b, C(b), reaches the remaining target (C falls as b rises), one lane per candidate.
    each_cand([&](uint32_t b) {
        if ((b >> 12) == prefix) {
            const uint32_t k = atomicAdd(&s_k, 1u);
            if (k < (uint32_t)SMP_SEL_MAX) s_sel[k] = b;
        }
    });
    __syncthreads();
    const uint32_t nsel = s_k;
    uint32_t tau;
    if (nsel <= (uint32_t)SMP_SEL_MAX) {
        if (t < (int)nsel) {
            const uint32_t bj = s_sel[t];
            uint64_t cge = 0;
            for (uint32_t i = 0; i < nsel; i++) {
                const uint32_t bi = s_sel[i];
                cge += bi >= bj ? smp_mass_bits(bi) : 0ull;
            }
            if (cge >= s_target) atomicMax(&s_tau, bj);
        }
        __syncthreads();
        tau = s_tau;
    } else {   // many equal or close values: radix passes over bits [11:4] and [3:0]
        for (int pass = 1; pass < 3; pass++) {
            const int shift = pass == 1 ? 4 : 0, width = pass == 2 ? 4 : 8;
            h[t] = 0;
            __syncthreads();
            each_cand([&](uint32_t b) {
                if ((b >> (shift + width)) == prefix)
                    atomicAdd(&h[(b >> shift) & ((1u << width) - 1u)], (unsigned long long)smp_mass_bits(b));
            });
            __syncthreads();
            // thread t holds bin 255 - t (bins past 2^width are empty)
            const uint64_t own = h[255 - t];
            const uint64_t tg = s_target;
            uint64_t tot;
            const uint64_t above = block_excl_scan(own, tmp, &tot);
            if (above < tg && above + own >= tg) {   // exactly one thread (own > 0)
                s_bin = 255 - t;
                s_target = tg - above;
            }
            __syncthreads();
            prefix = (prefix << width) | (uint32_t)s_bin;
        }
        tau = prefix;
    }
    // nucleus mass of this slice: its certain mass plus its candidates at or above tau
    uint64_t nm = cert;
    each_cand([&](uint32_t b) { nm += b >= tau ? smp_mass_bits(b) : 0ull; });
    uint64_t total;
    const uint64_t lo_b = block_excl_scan(nm, tmp, &total);
    u = u > 0.f ? u : 0.f;                      // u outside [0, 1) is clamped into it
    u = u < 1.f ? u : 0.99999994f;
    const uint64_t tgt = (uint64_t)((double)u * (double)total);   // < total
    if (lo_b <= tgt && tgt < lo_b + nm) {   // exactly one slice
        s_blk = t;
        s_lo = lo_b;
    }
    __syncthreads();
    // inside that slice: consecutive elements per thread, index order
    const int i0 = s_blk * sl, i1 = min(a.V, i0 + sl);
    const int per = (sl + SMP_DRAW_THREADS - 1) / SMP_DRAW_THREADS;
    const int j0 = min(i1, i0 + t * per), j1 = min(i1, j0 + per);
    uint64_t m = 0;
    for (int i = j0; i < j1; i++) {
        const uint32_t b = __float_as_uint(w.e[i]);
        m += b >= tau ? smp_mass_bits(b) : 0ull;
    }
    const uint64_t lo_t = s_lo + block_excl_scan(m, tmp, &total);
    if (lo_t <= tgt && tgt < lo_t + m) {   // exactly one thread: the elements holding the target
        uint64_t c = lo_t;
        for (int i = j0; i < j1; i++) {
            const uint32_t b = __float_as_uint(w.e[i]);
            if (b >= tau) {
                c += smp_mass_bits(b);
                if (c > tgt) {
                    *a.out = i;
                    break;
                }
            }
        }
    }
}

static size_t carve_ws(void* base, int V, SampleWs* w) {
    size_t off = 0;
    auto take = [&](size_t n) {
        void* p = base ? (char*)base + off : nullptr;
        off += align_up(n, 256);
        return p;
    };
    SampleWs s{};
    s.bmax = (float*)take((size_t)SMP_BLOCKS * 4);
    s.bidx = (int*)take((size_t)SMP_BLOCKS * 4);
    s.e = (float*)take((size_t)V * 4);
    s.hist = (uint64_t*)take((size_t)SMP_COPIES * SMP_BINS * 8);
    s.hist2 = (uint64_t*)take((size_t)SMP_COPIES * 256 * 8);
    s.certain = (uint64_t*)take((size_t)SMP_BLOCKS * 8);
    s.ncand = (uint32_t*)take((size_t)SMP_BLOCKS * 4);
    s.cand = (uint2*)take((size_t)SMP_BLOCKS * smp_slice(V) * 8);
    s.sel = (uint64_t*)take(4 * 8);
    if (w) *w = s;
    return off;
}

}  // namespace atlas

using namespace atlas;

extern "C" size_t atlas_sample_workspace_bytes(int32_t vocab) {
    if (vocab < 1 || vocab > (1 << 21)) return 0;
    return carve_ws(nullptr, vocab, nullptr);
}

extern "C" int atlas_sample(const float* d_logits, int32_t vocab, float temperature, float top_p, const float* d_u,
                            int32_t* d_token, void* ws, size_t ws_bytes, void* stream) {
    ATLAS_CHECK_ARG(d_logits && d_token && ws, "null pointer");
    ATLAS_CHECK_ARG(vocab >= 1 && vocab <= (1 << 21), "vocab=%d outside [1, 2^21]", vocab);
    ATLAS_CHECK_ARG(std::isfinite(temperature) && temperature >= 0.f, "temperature must be finite and >= 0");
    const bool greedy = temperature == 0.f;
    ATLAS_CHECK_ARG(greedy || (top_p > 0.f && top_p <= 1.f), "top_p must be in (0, 1]");
    ATLAS_CHECK_ARG(greedy || d_u, "sampling needs the uniform variate d_u");
    const size_t need = carve_ws(nullptr, vocab, nullptr);
    if (ws_bytes < need) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
    SampleWs w{};
    carve_ws(ws, vocab, &w);
    hipStream_t st = (hipStream_t)stream;
    prof_mark("sample_max", st);
    ATLAS_KLAUNCH(sample_max_kernel, dim3(SMP_BLOCKS), dim3(SMP_THREADS), 0, st, d_logits, vocab, w, greedy ? 0 : 1);
    ATLAS_LAUNCH_CHECK("sample_max_kernel");
    if (!greedy) {
        prof_mark("sample_exp", st);
        ATLAS_KLAUNCH(sample_exp_kernel, dim3(SMP_BLOCKS), dim3(SMP_THREADS), 0, st, d_logits, vocab,
                      1.0f / temperature, w);
        ATLAS_LAUNCH_CHECK("sample_exp_kernel");
        prof_mark("sample_bin", st);
        ATLAS_KLAUNCH(sample_bin_kernel, dim3(SMP_BLOCKS), dim3(SMP_THREADS), 0, st, vocab, (double)top_p, w);
        ATLAS_LAUNCH_CHECK("sample_bin_kernel");
    }
    DrawArgs a{};
    a.w = w;
    a.V = vocab;
    a.greedy = greedy ? 1 : 0;
    a.d_u = d_u;
    a.out = d_token;
    prof_mark("sample_draw", st);
    ATLAS_KLAUNCH(sample_draw_kernel, dim3(1), dim3(SMP_DRAW_THREADS), 0, st, a);
    ATLAS_LAUNCH_CHECK("sample_draw_kernel");
    return ATLAS_OK;
}
