// Fused kernels of the decode step. One decoder layer is six launches:
//   qkv      W_qkv x, where x = h + RMSNorm_pf(m) of the previous layer is rebuilt
//            and encoded by every block in its prologue (m summed from the down
//            projection's split-K partials);
//   attn     per (KV head, key split): full-projection QK RMSNorm, RoPE (+YaRN
//            factor), new key/value written to slot pos, then an online-softmax pass
//            over the split's keys for the Hq/Hkv query heads sharing the KV head;
//   merge    rescales the split partials into o and encodes it;
//   o        W_o o;
//   gate/up  h = x + RMSNorm_pa(a) rebuilt per block, then both SwiGLU projections
//            of the same rows and z = silu(gate) * up;
//   down     split-K W_down z; every block encodes its own range of z.
// Sources: "ATLAS-OLMo-3-32B-Think-v4" (Architecture deep-dive; Quantization
// recipe), "OLMo 3 32B" knowledge-base page (reordered post-norm; QK RMSNorm before
// the dot product), "Olmo-3-1125-32B" (eps, SwiGLU, YaRN on full layers only).
// No kernel uses atomics or waits on another block: every dependency is a launch
// boundary, and normalisation statistics are recomputed where they are needed.
// Prologue loads are issued all at once (one memory latency, not one per element)
// and weight loads of the first tile are in flight while the prologue runs.
#include <algorithm>

#include "decode_kernels.h"

namespace atlas {

// ---- shared prologue --------------------------------------------------------------------

constexpr int MAX_DOWN_SPLITS = 4;

__device__ __forceinline__ float4 f4_zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// The layer input described by src, in two halves: x_issue() issues every load into
// registers, x_finish() combines them into s_x[0..d) (block-wide; ends with a
// barrier). Kernels call x_issue() before their first weight load: loads complete in
// issue order, so inputs loaded after the weight prefetch would wait for it.
// NV4 >= d / (4 * blockDim.x). Indices past d are clamped to 0 (loads stay
// unconditional, which keeps the compiler's wait counting exact).
template <int NV4>
struct XRegs {
    float4 h[NV4], g[NV4];                  // EMBED: raw bf16 pairs in h[].x, h[].y
    float4 p[MAX_DOWN_SPLITS][NV4];
};

template <int NV4, bool RESID_ONLY = false>
__device__ __forceinline__ void x_issue(const XSource& src, int d, XRegs<NV4>& R) {
    const int n4 = d >> 2, bd = blockDim.x;
    if (!RESID_ONLY && src.mode == X_FROM_EMBED) {
        int tok = *src.d_token;
        if (tok < 0 || tok >= src.vocab) tok = 0;
        const uint2* row = reinterpret_cast<const uint2*>(src.emb + (size_t)tok * d);
#pragma unroll
        for (int j = 0; j < NV4; j++) {
            const int i = threadIdx.x + j * bd;
            const uint2 v = row[i < n4 ? i : 0];
            R.h[j] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), 0.f, 0.f);
        }
    } else if (!RESID_ONLY && src.mode == X_FROM_HIDDEN) {
        const float4* h4 = reinterpret_cast<const float4*>(src.hidden);
#pragma unroll
        for (int j = 0; j < NV4; j++) {
            const int i = threadIdx.x + j * bd;
            R.h[j] = h4[i < n4 ? i : 0];
        }
    } else {
        const float4* p4 = reinterpret_cast<const float4*>(src.m_part);
        const float4* h4 = reinterpret_cast<const float4*>(src.h);
        const float4* g4 = reinterpret_cast<const float4*>(src.g);
#pragma unroll
        for (int j = 0; j < NV4; j++) {
            const int i = threadIdx.x + j * bd, ic = i < n4 ? i : 0;
            R.h[j] = h4[ic];
            R.g[j] = g4[ic];
#pragma unroll
            for (int s = 0; s < MAX_DOWN_SPLITS; s++) R.p[s][j] = p4[(size_t)min(s, src.S - 1) * n4 + ic];
        }
    }
}

template <int NV4, bool RESID_ONLY = false>
__device__ void x_finish(const XSource& src, int d, const XRegs<NV4>& R, float* s_x, float* red) {
    const int n4 = d >> 2, bd = blockDim.x;
    float4* sx4 = reinterpret_cast<float4*>(s_x);
    if (!RESID_ONLY && src.mode == X_FROM_EMBED) {
#pragma unroll
        for (int j = 0; j < NV4; j++) {
            const int i = threadIdx.x + j * bd;
            const uint32_t lo = __float_as_uint(R.h[j].x), hi = __float_as_uint(R.h[j].y);
            if (i < n4)
                sx4[i] = make_float4(bf16_bits_to_f32(lo & 0xFFFFu), bf16_bits_to_f32(lo >> 16),
                                     bf16_bits_to_f32(hi & 0xFFFFu), bf16_bits_to_f32(hi >> 16));
        }
    } else if (!RESID_ONLY && src.mode == X_FROM_HIDDEN) {
#pragma unroll
        for (int j = 0; j < NV4; j++) {
            const int i = threadIdx.x + j * bd;
            if (i < n4) sx4[i] = R.h[j];
        }
    } else {
        float4 m[NV4];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NV4; j++) {
            const int i = threadIdx.x + j * bd;
            float4 v = R.p[0][j];
#pragma unroll
            for (int s = 1; s < MAX_DOWN_SPLITS; s++) {
                if (s < src.S) {
                    v.x += R.p[s][j].x;
                    v.y += R.p[s][j].y;
                    v.z += R.p[s][j].z;
                    v.w += R.p[s][j].w;
                }
            }
            if (i >= n4) v = f4_zero();
            m[j] = v;
            ss = fmaf(v.x, v.x, ss);
            ss = fmaf(v.y, v.y, ss);
            ss = fmaf(v.z, v.z, ss);
            ss = fmaf(v.w, v.w, ss);
        }
        ss = block_sum(ss, red);
        const float r = 1.0f / sqrtf(ss / (float)d + src.eps);
#pragma unroll
        for (int j = 0; j < NV4; j++) {
            const int i = threadIdx.x + j * bd;
            if (i < n4)
                sx4[i] = make_float4(R.h[j].x + R.g[j].x * (m[j].x * r), R.h[j].y + R.g[j].y * (m[j].y * r),
                                     R.h[j].z + R.g[j].z * (m[j].z * r), R.h[j].w + R.g[j].w * (m[j].w * r));
        }
    }
    __syncthreads();
}

template <int NV4>
__device__ void build_x(const XSource& src, int d, float* s_x, float* red) {
    XRegs<NV4> R;
    x_issue<NV4>(src, d, R);
    x_finish<NV4>(src, d, R, s_x, red);
}

template <int RB>
__device__ __forceinline__ void write_rows(const float acc[RB], int row0, int N, float* out, int lane) {
#pragma unroll
    for (int r = 0; r < RB; r++) {
        const float s = wave_sum(acc[r]);
        if (lane == 0 && row0 + r < N) out[row0 + r] = s;
    }
}

// Streaming pipeline of NS register stages. A wave owns tiles t0, t0+NW, ... (nt of
// them). Before the prologue it loads its first NS-1 tiles into R[0..NS-2]; each
// step then issues the load of the tile NS-1 positions ahead (pinned by a
// scheduling barrier) and reduces the oldest one, so NS-1 tiles per wave are always
// in flight. The main loop runs whole groups of NS tiles with unconditional loads
// (indices clamped to the wave's last tile, so the compiler's wait counting stays
// exact); the remainder needs no further loads.
__device__ __forceinline__ int wave_tiles(int t0, int t_end, int NW) {
    return t0 < t_end ? (t_end - t0 + NW - 1) / NW : 0;
}

template <int CPL, int RB, int NS>
__device__ __forceinline__ void prefetch_tiles(TileRegs<CPL> (&R)[NS], const W4View& W, const LaneMap<CPL, RB>& m,
                                               int t0, int nt, int NW) {
    // unconditional (a wave without tiles loads row 0): a branch here would make the
    // compiler wait for these loads wherever it waits for anything issued before them
#pragma unroll
    for (int k = 0; k < NS - 1; k++) load_tile(R[k], W, m, max(0, (t0 + min(k, nt - 1) * NW) * RB));
}

template <int CPL, int RB, int NS, class Epi>
__device__ __forceinline__ void stream_rows_epi(const W4View& W, const LaneMap<CPL, RB>& m, const LanePlanes<CPL>& P,
                                                TileRegs<CPL> (&R)[NS], int t0, int nt, int NW, Epi epi) {
    int i = 0;
    for (; i + NS <= nt; i += NS) {
#pragma unroll
        for (int k = 0; k < NS; k++) {
            load_tile(R[(k + NS - 1) % NS], W, m, (t0 + min(i + k + NS - 1, nt - 1) * NW) * RB);
            __builtin_amdgcn_sched_barrier(0);
            float acc[RB];
            tile_dot(R[k], P, m, W, acc);
            epi(acc, (t0 + (i + k) * NW) * RB);
        }
    }
#pragma unroll
    for (int k = 0; k < NS - 1; k++) {   // nt - i < NS tiles left, already loaded in R[0..]
        if (i + k < nt) {
            float acc[RB];
            tile_dot(R[k], P, m, W, acc);
            epi(acc, (t0 + (i + k) * NW) * RB);
        }
    }
}

template <int CPL, int RB, int NS>
__device__ __forceinline__ void stream_rows(const W4View& W, const LaneMap<CPL, RB>& m, const LanePlanes<CPL>& P,
                                            TileRegs<CPL> (&R)[NS], int t0, int nt, int NW, float* out,
                                            int lane) {
    stream_rows_epi<CPL, RB, NS>(W, m, P, R, t0, nt, NW,
                                 [&](const float (&acc)[RB], int row0) { write_rows<RB>(acc, row0, W.N, out, lane); });
}

// LDS carve for the GEMV kernels: [s_x: dx floats][planes CW*24][qs CW][isum CW]
struct GemvLds {
    float* s_x;
    uint32_t* s_pl;
    float* s_qs;
    int* s_is;
    __device__ GemvLds(uint32_t* smem, int dx, int CW) {
        s_x = reinterpret_cast<float*>(smem);
        s_pl = smem + dx;
        s_qs = reinterpret_cast<float*>(s_pl + CW * XQ_WORDS_PER_CHUNK);
        s_is = reinterpret_cast<int*>(s_qs + CW);
    }
};

constexpr int GEMV_NV4 = 3;   // float4 per thread of an input vector: d <= 3 * 4 * GEMV_THREADS = 6144
// Register stages: two, i.e. one tile (gate/up: one tile pair) in flight per wave
// beyond the one being reduced. Deeper rings (2-3 tiles in flight) were slower: a wave
// spends longer issuing them before its prologue, and eight waves per CU already keep
// the memory system busy.
template <int CPL>
constexpr int gemv_stages() { return 2; }
constexpr int GU_STAGES = 2;

// ---- qkv projection ----------------------------------------------------------------------

template <int CPL, int RB, bool RESID>
__device__ __forceinline__ void qkv_body(const QkvArgs& a) {
    extern __shared__ uint32_t smem[];
    __shared__ float red[16];
    __shared__ float s_ss[2][GEMV_THREADS / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
    GemvLds L(smem, a.d, a.CW);
    LaneMap<CPL, RB> m;
    m.init(lane, 0, a.CW, a.group);
    const int T = (a.W.N + RB - 1) / RB;
    const int t_begin = blockIdx.x * a.tiles_per_block, t_end = min(T, t_begin + a.tiles_per_block);
    const int t = t_begin + wave, nt = wave_tiles(t, t_end, NW);
    XRegs<GEMV_NV4> XR;
    x_issue<GEMV_NV4, RESID>(a.src, a.d, XR);
    __builtin_amdgcn_sched_barrier(0);
    TileRegs<CPL> R[gemv_stages<CPL>()];
    prefetch_tiles<CPL, RB, gemv_stages<CPL>()>(R, a.W, m, t, nt, NW);   // in flight during the prologue

    if (a.status && blockIdx.x == 0 && threadIdx.x == 0) {
        int ok = 1;
        if (a.src.mode == X_FROM_EMBED) {
            const int tok = *a.src.d_token;
            ok = tok >= 0 && tok < a.src.vocab;
        }
        *a.status = ok ? ATLAS_OK : ATLAS_ERR_INVALID_ARG;
    }
    x_finish<GEMV_NV4, RESID>(a.src, a.d, XR, L.s_x, red);
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < a.d; i += blockDim.x) a.x_out[i] = L.s_x[i];
    encode_lds(L.s_x, a.d, L.s_pl, L.s_qs, L.s_is);
    __syncthreads();
    LanePlanes<CPL> P;
    P.load(m, L.s_pl, L.s_qs, L.s_is, 0);
    // rows are written as they finish; lane 0 also sums the squares of its q rows and
    // of its k rows (the statistics of the full-projection QK RMSNorm)
    float ssq = 0.f, ssk = 0.f;
    stream_rows_epi<CPL, RB, gemv_stages<CPL>()>(a.W, m, P, R, t, nt, NW, [&](const float (&acc)[RB], int row0) {
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const float v = wave_sum(acc[r]);
            const int row = row0 + r;
            if (lane == 0 && row < a.W.N) a.qkv[row] = v;
            const float sq = v * v;
            ssq += row < a.nq ? sq : 0.f;
            ssk += (row >= a.nq && row < a.nq + a.nk) ? sq : 0.f;
        }
    });
    if (a.ssq_part) {
        if (lane == 0) {
            s_ss[0][wave] = ssq;
            s_ss[1][wave] = ssk;
        }
        __syncthreads();
        if (threadIdx.x < 2) {
            float v = 0.f;
            for (int w = 0; w < NW; w++) v += s_ss[threadIdx.x][w];
            a.ssq_part[2 * blockIdx.x + threadIdx.x] = v;
        }
    }
}

// layer 0 (input from the embedding or a hidden vector) and every later layer
template <int CPL, int RB>
__global__ __launch_bounds__(GEMV_THREADS) void qkv_kernel(QkvArgs a) {
    qkv_body<CPL, RB, false>(a);
}
template <int CPL, int RB>
__global__ __launch_bounds__(GEMV_THREADS) void qkv_resid_kernel(QkvArgs a) {
    qkv_body<CPL, RB, true>(a);
}

// ---- generic GEMV over an input already encoded in global memory ----------------------------

template <int CPL, int RB>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_planes_kernel(GemvPlanesArgs a) {
    extern __shared__ uint32_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
    const int kr = blockIdx.y, C0 = kr * a.CW;
    GemvLds L(smem, 0, a.CW);
    LaneMap<CPL, RB> m;
    m.init(lane, C0, a.CW, a.group);
    const int T = (a.W.N + RB - 1) / RB;
    const int t_begin = blockIdx.x * a.tiles_per_block, t_end = min(T, t_begin + a.tiles_per_block);
    const int t = t_begin + wave, nt = wave_tiles(t, t_end, NW);
    PlaneStage PS;
    planes_issue<GEMV_THREADS>(a.xq, C0, a.CW, PS);
    __builtin_amdgcn_sched_barrier(0);
    TileRegs<CPL> R[gemv_stages<CPL>()];
    prefetch_tiles<CPL, RB, gemv_stages<CPL>()>(R, a.W, m, t, nt, NW);
    planes_commit<GEMV_THREADS>(PS, a.CW, L.s_pl, L.s_qs, L.s_is);
    __syncthreads();
    LanePlanes<CPL> P;
    P.load(m, L.s_pl, L.s_qs, L.s_is, C0);
    stream_rows<CPL, RB, gemv_stages<CPL>()>(a.W, m, P, R, t, nt, NW, a.y + (size_t)kr * a.W.N, lane);
}

// ---- older / younger wave split ----------------------------------------------------------
// Tiles of a block split between its older and younger waves. On each SIMD the wave
// dispatched first (waves 0 .. NW/2 - 1 of a 512-thread block) is served first by the
// memory system and streams faster while both run; with equal shares the younger waves
// finish several microseconds later, streaming alone at a fraction of the bandwidth.
// The older waves take the fraction `old_frac` of the block's tiles, strided over
// NW/2 waves, the younger ones the rest.
struct WaveRange {
    int t, nt, stride;
};
__device__ __forceinline__ WaveRange wave_range(int t_begin, int t_end, int wave, int NW, float old_frac) {
    WaveRange r;
    const int HW = NW / 2, nb = max(t_end - t_begin, 0);
    const int n_old = min(nb, (int)(nb * old_frac + 0.5f));
    r.stride = HW;
    r.t = wave < HW ? t_begin + wave : t_begin + n_old + (wave - HW);
    r.nt = wave_tiles(r.t, wave < HW ? t_begin + n_old : t_end, HW);
    return r;
}

// ---- gate/up projections + SwiGLU ---------------------------------------------------------

template <int CPL, int RB>
__device__ __forceinline__ void swiglu_rows(const float ag[RB], const float au[RB], int row0, int N, float* z,
                                            int lane) {
#pragma unroll
    for (int rr = 0; rr < RB; rr++) {
        const float sg = wave_sum(ag[rr]);
        const float su = wave_sum(au[rr]);
        if (lane == 0 && row0 + rr < N) z[row0 + rr] = sg / (1.0f + __expf(-sg)) * su;
    }
}

template <int CPL, int RB>
__global__ __launch_bounds__(GEMV_THREADS) void gate_up_kernel(GateUpArgs a) {
    extern __shared__ uint32_t smem[];
    __shared__ float red[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
    GemvLds L(smem, a.d, a.CW);
    LaneMap<CPL, RB> m;
    m.init(lane, 0, a.CW, a.group);
    const int T = (a.Wg.N + RB - 1) / RB;
    const int t_begin = blockIdx.x * a.tiles_per_block, t_end = min(T, t_begin + a.tiles_per_block);
    const WaveRange wr = wave_range(t_begin, t_end, wave, NW, a.old_frac);
    const int t = wr.t, nt = wr.nt, TS = wr.stride;
    // h = x + g * a / rms(a): inputs loaded first, then the weight prefetch
    const int n4 = a.d >> 2, bd = blockDim.x;
    float4 va[GEMV_NV4], vx[GEMV_NV4], vg[GEMV_NV4];
    {
        const float4* a4 = reinterpret_cast<const float4*>(a.a);
        const float4* x4 = reinterpret_cast<const float4*>(a.x);
        const float4* g4 = reinterpret_cast<const float4*>(a.g);
#pragma unroll
        for (int j = 0; j < GEMV_NV4; j++) {
            const int i = threadIdx.x + j * bd, ic = i < n4 ? i : 0;
            va[j] = a4[ic];
            vx[j] = x4[ic];
            vg[j] = g4[ic];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    TileRegs<CPL> RG[GU_STAGES], RU[GU_STAGES];
    prefetch_tiles<CPL, RB, GU_STAGES>(RG, a.Wg, m, t, nt, TS);
    prefetch_tiles<CPL, RB, GU_STAGES>(RU, a.Wu, m, t, nt, TS);
    {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < GEMV_NV4; j++) {
            if (threadIdx.x + j * bd < n4) {
                ss = fmaf(va[j].x, va[j].x, ss);
                ss = fmaf(va[j].y, va[j].y, ss);
                ss = fmaf(va[j].z, va[j].z, ss);
                ss = fmaf(va[j].w, va[j].w, ss);
            }
        }
        ss = block_sum(ss, red);
        const float r = 1.0f / sqrtf(ss / (float)a.d + a.eps);
        float4* sx4 = reinterpret_cast<float4*>(L.s_x);
        float4* h4 = reinterpret_cast<float4*>(a.h_out);
#pragma unroll
        for (int j = 0; j < GEMV_NV4; j++) {
            const int i = threadIdx.x + j * bd;
            if (i < n4) {
                const float4 h = make_float4(vx[j].x + vg[j].x * (va[j].x * r), vx[j].y + vg[j].y * (va[j].y * r),
                                             vx[j].z + vg[j].z * (va[j].z * r), vx[j].w + vg[j].w * (va[j].w * r));
                sx4[i] = h;
                if (blockIdx.x == 0) h4[i] = h;
            }
        }
        __syncthreads();
    }
    encode_lds(L.s_x, a.d, L.s_pl, L.s_qs, L.s_is);
    __syncthreads();
    LanePlanes<CPL> P;
    P.load(m, L.s_pl, L.s_qs, L.s_is, 0);
    // same pipeline as stream_rows, over both matrices
    int i = 0;
    for (; i + GU_STAGES <= nt; i += GU_STAGES) {
#pragma unroll
        for (int k = 0; k < GU_STAGES; k++) {
            const int rl = (t + min(i + k + GU_STAGES - 1, nt - 1) * TS) * RB;
            load_tile(RG[(k + GU_STAGES - 1) % GU_STAGES], a.Wg, m, rl);
            load_tile(RU[(k + GU_STAGES - 1) % GU_STAGES], a.Wu, m, rl);
            __builtin_amdgcn_sched_barrier(0);
            float ag[RB], au[RB];
            tile_dot(RG[k], P, m, a.Wg, ag);
            tile_dot(RU[k], P, m, a.Wu, au);
            swiglu_rows<CPL, RB>(ag, au, (t + (i + k) * TS) * RB, a.Wg.N, a.z, lane);
        }
    }
#pragma unroll
    for (int k = 0; k < GU_STAGES - 1; k++) {
        if (i + k < nt) {
            float ag[RB], au[RB];
            tile_dot(RG[k], P, m, a.Wg, ag);
            tile_dot(RU[k], P, m, a.Wu, au);
            swiglu_rows<CPL, RB>(ag, au, (t + (i + k) * TS) * RB, a.Wg.N, a.z, lane);
        }
    }
}

// ---- down projection (split-K) --------------------------------------------------------------

constexpr int DOWN_MAX_ROUNDS = 3;   // CW <= 3 * GEMV_THREADS / 4 chunks
static_assert(DOWN_MAX_ROUNDS * GEMV_THREADS / 4 * XQ_WORDS_PER_CHUNK <= PLANE_REGS * 4 * GEMV_THREADS,
              "an encoded range must fit the register staging of planes_issue");

template <int CPL, int RB>
__global__ __launch_bounds__(GEMV_THREADS) void down_kernel(DownArgs a) {
    extern __shared__ uint32_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = blockDim.x >> 6;
    const int kr = blockIdx.y, C0 = kr * a.CW;
    GemvLds L(smem, 0, a.CW);
    LaneMap<CPL, RB> m;
    m.init(lane, C0, a.CW, a.group);
    const int T = (a.W.N + RB - 1) / RB;
    const int t_begin = blockIdx.x * a.tiles_per_block, t_end = min(T, t_begin + a.tiles_per_block);
    const WaveRange wr = wave_range(t_begin, t_end, wave, NW, a.old_frac);
    const int t = wr.t, nt = wr.nt;
    // this block's range of z, loaded before the weight prefetch and encoded into LDS
    const int nwords = a.CW * 4;
    float4 u[DOWN_MAX_ROUNDS], v[DOWN_MAX_ROUNDS];
    {
        const float4* zb = reinterpret_cast<const float4*>(a.z + (size_t)C0 * XQ_CHUNK);
#pragma unroll
        for (int r = 0; r < DOWN_MAX_ROUNDS; r++) {
            const int w = threadIdx.x + r * blockDim.x, wc = w < nwords ? w : 0;
            u[r] = zb[2 * wc];
            v[r] = zb[2 * wc + 1];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    TileRegs<CPL> R[gemv_stages<CPL>()];
    prefetch_tiles<CPL, RB, gemv_stages<CPL>()>(R, a.W, m, t, nt, wr.stride);
    {
        XQ o;
        o.planes = L.s_pl;
        o.qs = L.s_qs;
        o.isum = L.s_is;
#pragma unroll
        for (int r = 0; r < DOWN_MAX_ROUNDS; r++) {
            const int w = threadIdx.x + r * blockDim.x;
            if (w < nwords) {   // whole quads in or out
                const float x8[8] = {u[r].x, u[r].y, u[r].z, u[r].w, v[r].x, v[r].y, v[r].z, v[r].w};
                xq_encode_word(x8, o, w >> 2, w & 3);
            }
        }
    }
    __syncthreads();
    LanePlanes<CPL> P;
    P.load(m, L.s_pl, L.s_qs, L.s_is, C0);
    stream_rows<CPL, RB, gemv_stages<CPL>()>(a.W, m, P, R, t, nt, wr.stride, a.m_part + (size_t)kr * a.W.N, lane);
}

// ---- attention ---------------------------------------------------------------------------------
//
// grid (S, Hkv), 256 threads. 16 lanes hold one key (8 dims each); the four 16-lane
// groups of each wave are independent key streams with their own online softmax,
// combined at the end. Queries stay in registers. The cache holds f32 or bf16
// elements (KVB), and key j sits in slot j, or in slot j mod slots on a
// sliding-window ring.

// One key and value of a 16-lane stream as loaded: 8 f32 of each (two 16-byte
// loads), or 8 bf16 of each (one 16-byte load), widened only when consumed so that
// the loads stay in flight.
template <bool KVB>
struct KvRegs {
    f32x4_t k0, k1, v0, v1;
    __device__ __forceinline__ void unpack(float (&kx)[8], float (&vx)[8]) const {
        kx[0] = k0.x; kx[1] = k0.y; kx[2] = k0.z; kx[3] = k0.w; kx[4] = k1.x; kx[5] = k1.y; kx[6] = k1.z; kx[7] = k1.w;
        vx[0] = v0.x; vx[1] = v0.y; vx[2] = v0.z; vx[3] = v0.w; vx[4] = v1.x; vx[5] = v1.y; vx[6] = v1.z; vx[7] = v1.w;
    }
};
template <>
struct KvRegs<true> {
    u32x4_t k, v;
    __device__ __forceinline__ void unpack(float (&kx)[8], float (&vx)[8]) const {
        const uint32_t kw[4] = {k.x, k.y, k.z, k.w}, vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {   // element 2i in the low half of word i
            kx[2 * i] = __uint_as_float(kw[i] << 16);
            kx[2 * i + 1] = __uint_as_float(kw[i] & 0xFFFF0000u);
            vx[2 * i] = __uint_as_float(vw[i] << 16);
            vx[2 * i + 1] = __uint_as_float(vw[i] & 0xFFFF0000u);
        }
    }
};

// 2^x on the hardware exponential (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Keys in flight per 16-lane stream: 1 (a ring of two). Deeper rings (2 and 4 keys) were
// slower on both layer types: their registers (256 with spills at 4 keys) cost more
// than the extra loads gain; 16 streams per block, two blocks per CU, already keep 32
// keys (32 KB) in flight per CU.
constexpr int ATTN_KV_STAGES = 2;
// A bf16 key and value take half the registers of f32 ones: the ring holds two pairs of
// keys, and each online-softmax update takes a pair (one rescale of the accumulators per
// two keys, which trims the VALU work per key where that work, not HBM, sets the pace).
constexpr int ATTN_KV_STAGES_BF16 = 2;
constexpr int ATTN_KEYS_PER_STEP_BF16 = 2;
constexpr int ATTN_WAVES = ATTN_THREADS / 64;
constexpr int ATTN_STREAMS = 4 * ATTN_WAVES;                        // 16-lane key streams per block
constexpr int ATTN_SSQ_REGS = ATTN_SSQ_MAX_BLOCKS / ATTN_THREADS;   // sums-of-squares partials per thread
constexpr int ATTN_QF_REGS = 8 * 128 / ATTN_THREADS;                 // query values per thread (G <= 8)

// FUSED: q/k/v come raw from the qkv projection (norm, rotary and KV append here);
// otherwise q is final and the cache already holds the new key.
template <int G, bool FUSED, bool KVB>
__global__ __launch_bounds__(ATTN_THREADS, ATTN_WAVES <= 4 && G <= 5 ? 2 : 1) void attn_kernel(AttnFusedArgs a) {
    constexpr int D = 128;
    __shared__ float s_q[G][D];
    __shared__ float s_kn[D], s_vn[D];
    __shared__ float s_cos[64], s_sin[64];
    __shared__ float red[16];
    __shared__ float s_wm[ATTN_WAVES][G], s_wl[ATTN_WAVES][G];
    __shared__ float s_wacc[ATTN_WAVES][G][D];
    const int s = blockIdx.x, kv = blockIdx.y, bz = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane & 15, grp = lane >> 4;
    const int nq = a.Hq * D, nk = a.Hkv * D;
    // the position through a vector load (a scalar load would be waited for together
    // with the kernel arguments, before anything else is issued)
    const int pos_v = a.d_pos[bz + (int)__builtin_amdgcn_mbcnt_lo(0u, 0u)];
    float* part0 = a.part + (size_t)bz * a.part_stride + (size_t)(kv * G) * a.S * ATTN_PART_F;
    // Prologue inputs first (loads complete in issue order): the qkv kernel's per-block
    // sums of squares, this block's q heads and k/v head, and their gains. None depends
    // on the position, whose load is still in flight.
    float ps_q[ATTN_SSQ_REGS], ps_k[ATTN_SSQ_REGS];
    float xq0[2], xq1[2], gq0[2], gq1[2], vnew = 0.f;
    float qf[ATTN_QF_REGS];
    const double inv_i = a.inv[threadIdx.x & 63];   // kernel-argument array: a memory load
    if (!FUSED) {
#pragma unroll
        for (int r = 0; r < ATTN_QF_REGS; r++)
            qf[r] = a.q_final[(size_t)bz * a.q_stride + (size_t)kv * G * D +
                              min((int)threadIdx.x + r * ATTN_THREADS, G * D - 1)];
    } else {
#pragma unroll
        for (int j = 0; j < ATTN_SSQ_REGS; j++) {
            const int b = threadIdx.x + j * ATTN_THREADS, bc = b < a.n_ssq ? b : 0;
            const float2 v = reinterpret_cast<const float2*>(a.ssq_part)[bc];
            ps_q[j] = v.x;
            ps_k[j] = v.y;
        }
#pragma unroll
        for (int r = 0; r < 2; r++) {
            const int t = threadIdx.x + r * ATTN_THREADS;
            const int tt = t < (G + 1) * 64 ? t : 0;
            const int hh = tt >> 6, i = tt & 63;
            const bool isk = hh == G;
            const int base = isk ? nq + kv * D : (kv * G + hh) * D;
            const float* g = isk ? a.g_k + kv * D : a.g_q + (kv * G + hh) * D;
            xq0[r] = a.qkv[base + i];
            xq1[r] = a.qkv[base + i + 64];
            gq0[r] = g[i];
            gq1[r] = g[i + 64];
        }
        vnew = a.qkv[nq + nk + kv * D + (threadIdx.x & (D - 1))];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int pos = __builtin_amdgcn_readfirstlane(pos_v);
    const bool pos_ok = pos >= 0 && pos < a.T_max && (a.ring || pos < a.slots);
    if (!pos_ok) {
        for (int t = threadIdx.x; t < G * (2 + D); t += blockDim.x) {
            const int h = t / (2 + D), e = t % (2 + D);
            part0[((size_t)h * a.S + s) * ATTN_PART_F + e] = e == 0 ? -INFINITY : 0.f;
        }
        if (a.status && s == 0 && kv == 0 && threadIdx.x == 0) *a.status = ATLAS_ERR_INVALID_ARG;
        return;
    }
    int lo = a.window > 0 ? pos - a.window + 1 : 0;
    if (lo < 0) lo = 0;
    const int nkeys = pos - lo + 1;
    const int Lk = (nkeys + a.S - 1) / a.S;
    const int k0 = lo + s * Lk;
    int cnt = min(Lk, lo + nkeys - k0);
    if (cnt < 0) cnt = 0;
    const int stream = wave * 4 + grp;
    // Slots: key jb + i (jb the split's first key) is in slot sb + i, wrapped once on a
    // ring. The keys of one call span at most `slots` positions (a ring holds the
    // whole window), and on a flat cache jb + i <= pos < slots never wraps.
    const int slots = (int)a.slots;
    const int jb = cnt > 0 ? k0 : lo;
    const int sb = a.ring ? jb % slots : jb;
    const size_t head0 = (size_t)bz * a.seq_stride + (size_t)kv * a.slots * D;
    // K/V of key i of this split (clamped into the split)
    auto load_kv = [&](int i, KvRegs<KVB>& r) {
        int sl = sb + (cnt > 0 ? min(i, cnt - 1) : 0);
        sl -= sl >= slots ? slots : 0;
        const size_t e = head0 + (size_t)sl * D + 8 * sub;
        if constexpr (KVB) {
            r.k = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>((const uint16_t*)a.k_cache + e));
            r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>((const uint16_t*)a.v_cache + e));
        } else {
            const f32x4_t* kp = reinterpret_cast<const f32x4_t*>((const float*)a.k_cache + e);
            const f32x4_t* vp = reinterpret_cast<const f32x4_t*>((const float*)a.v_cache + e);
            r.k0 = __builtin_nontemporal_load(kp);
            r.k1 = __builtin_nontemporal_load(kp + 1);
            r.v0 = __builtin_nontemporal_load(vp);
            r.v1 = __builtin_nontemporal_load(vp + 1);
        }
    };
    // ring of NS steps of KP keys per stream; the first NS-1 steps are in flight during
    // the prologue
    constexpr int NS = KVB ? ATTN_KV_STAGES_BF16 : ATTN_KV_STAGES;
    constexpr int KP = KVB ? ATTN_KEYS_PER_STEP_BF16 : 1;
    KvRegs<KVB> rkv[NS][KP];
#pragma unroll
    for (int k = 0; k < NS - 1; k++)
#pragma unroll
        for (int e = 0; e < KP; e++) load_kv(stream + ATTN_STREAMS * (k * KP + e), rkv[k][e]);
    // (keys past the stream's last one are clamped loads of valid rows, never consumed)

    if (FUSED) {
        // pin the partial sums here, after the key/value prefetch: otherwise the
        // compiler may add them up right after their loads and wait for them there
#pragma unroll
        for (int j = 0; j < ATTN_SSQ_REGS; j++) asm volatile("" : "+v"(ps_q[j]), "+v"(ps_k[j]));
        float ssq = 0.f, ssk = 0.f;
#pragma unroll
        for (int j = 0; j < ATTN_SSQ_REGS; j++) {
            if (threadIdx.x + j * ATTN_THREADS < a.n_ssq) {
                ssq += ps_q[j];
                ssk += ps_k[j];
            }
        }
        ssq = block_sum(ssq, red);
        ssk = block_sum(ssk, red);
        const float rq = 1.0f / sqrtf(ssq / (float)nq + a.eps);
        const float rk = 1.0f / sqrtf(ssk / (float)nk + a.eps);
        if (threadIdx.x < 64) {
            // angle pos * inv in f64, reduced to [-pi, pi] in f64, then sine/cosine in f32
            const double ang = (double)pos * inv_i;
            const double rr = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
            float sn, cs;
            sincosf((float)rr, &sn, &cs);
            s_cos[threadIdx.x] = cs * (float)a.mscale;
            s_sin[threadIdx.x] = sn * (float)a.mscale;
        }
        // a bf16 cache stores the rounded value, and the new token attends to what is stored
        if (threadIdx.x < D) s_vn[threadIdx.x] = KVB ? bf16_bits_to_f32(f32_to_bf16_rne(vnew)) : vnew;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 2; r++) {
            const int t = threadIdx.x + r * ATTN_THREADS;
            if (t < (G + 1) * 64) {
                const int hh = t >> 6, i = t & 63;
                const bool isk = hh == G;
                const float rr = isk ? rk : rq;
                const float x0 = gq0[r] * (xq0[r] * rr), x1 = gq1[r] * (xq1[r] * rr);
                const float c = s_cos[i], sn = s_sin[i];
                const float y0 = x0 * c - x1 * sn, y1 = x1 * c + x0 * sn;
                if (isk) {
                    s_kn[i] = KVB ? bf16_bits_to_f32(f32_to_bf16_rne(y0)) : y0;
                    s_kn[i + 64] = KVB ? bf16_bits_to_f32(f32_to_bf16_rne(y1)) : y1;
                } else {
                    s_q[hh][i] = y0;
                    s_q[hh][i + 64] = y1;
                }
            }
        }
        __syncthreads();
        if (pos >= k0 && pos < k0 + cnt && threadIdx.x < D) {   // the split that holds the new token
            const size_t off = head0 + (size_t)(a.ring ? pos % slots : pos) * D + threadIdx.x;
            if constexpr (KVB) {   // already rounded: the upper half is the value
                ((uint16_t*)a.k_cache)[off] = (uint16_t)(__float_as_uint(s_kn[threadIdx.x]) >> 16);
                ((uint16_t*)a.v_cache)[off] = (uint16_t)(__float_as_uint(s_vn[threadIdx.x]) >> 16);
            } else {
                ((float*)a.k_cache)[off] = s_kn[threadIdx.x];
                ((float*)a.v_cache)[off] = s_vn[threadIdx.x];
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < ATTN_QF_REGS; r++) {
            const int t = threadIdx.x + r * ATTN_THREADS;
            if (t < G * D) s_q[t / D][t % D] = qf[r];
        }
        __syncthreads();
    }

    // scores in base-2 units: q carries the softmax scale and log2(e), so each
    // exponential is one exp2; the partial's maximum goes back to natural units
    const float qs = a.scale * 1.4426950408889634f;
    float q[G][8];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) q[h][i] = s_q[h][8 * sub + i] * qs;
    float mh[G], lh[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; h++) {
        mh[h] = -INFINITY;
        lh[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) acc[h][i] = 0.f;
    }
    // This stream's keys are stream, stream + ATTN_STREAMS, ... (< cnt): nks of them, in
    // nst steps of KP keys. The ring holds NS steps; each step loads the step NS-1 ahead
    // and consumes the oldest. Whole groups of NS steps run with unconditional (clamped)
    // loads so that the compiler's wait counting stays exact; the remainder is already
    // loaded. The new token's key and value come from LDS (the cache write above may
    // still be in flight).
    const int nks = cnt > stream ? (cnt - stream + ATTN_STREAMS - 1) / ATTN_STREAMS : 0;
    const int nst = (nks + KP - 1) / KP;
    auto consume = [&](int slot, int st) {
        float kx[KP][8], vx[KP][8];
#pragma unroll
        for (int e = 0; e < KP; e++) {
            rkv[slot][e].unpack(kx[e], vx[e]);
            if (FUSED && k0 + stream + ATTN_STREAMS * (st * KP + e) == pos) {
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    kx[e][i] = s_kn[8 * sub + i];
                    vx[e][i] = s_vn[8 * sub + i];
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; h++) {
            float sc[KP], mn = mh[h];
#pragma unroll
            for (int e = 0; e < KP; e++) {
                float dsum = 0.f;
#pragma unroll
                for (int i = 0; i < 8; i++) dsum = fmaf(q[h][i], kx[e][i], dsum);
                sc[e] = row16_sum(dsum);
                if (KP > 1 && st * KP + e >= nks) sc[e] = -INFINITY;   // past the stream's last key
                mn = fmaxf(mn, sc[e]);
            }
            const float c = exp2_fast(mh[h] - mn);
            float p[KP], psum = 0.f;
#pragma unroll
            for (int e = 0; e < KP; e++) {
                p[e] = exp2_fast(sc[e] - mn);
                psum += p[e];
            }
            lh[h] = fmaf(lh[h], c, psum);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                float t = p[KP - 1] * vx[KP - 1][i];
#pragma unroll
                for (int e = KP - 2; e >= 0; e--) t = fmaf(p[e], vx[e][i], t);
                acc[h][i] = fmaf(acc[h][i], c, t);
            }
            mh[h] = mn;
        }
    };
    int it = 0;
    for (; it + NS <= nst; it += NS) {
#pragma unroll
        for (int k = 0; k < NS; k++) {
            const int slot = (k + NS - 1) % NS;
#pragma unroll
            for (int e = 0; e < KP; e++)
                load_kv(stream + ATTN_STREAMS * min((it + k + NS - 1) * KP + e, nks - 1), rkv[slot][e]);
            __builtin_amdgcn_sched_barrier(0);
            consume(k, it + k);
        }
    }
#pragma unroll
    for (int k = 0; k < NS - 1; k++)
        if (it + k < nst) consume(k, it + k);
    // combine the four streams of the wave (lanes l, l^16, l^32, l^48)
#pragma unroll
    for (int h = 0; h < G; h++) {
        // lane-swap butterflies (v_permlane16/32_swap): register moves, not LDS permutes
        const float M = xor32_max(xor16_max(mh[h]));
        const float w = (M == -INFINITY) ? 0.f : exp2_fast(mh[h] - M);
        const float l = xor32_sum(xor16_sum(lh[h] * w));
#pragma unroll
        for (int e = 0; e < 8; e++) acc[h][e] = xor32_sum(xor16_sum(acc[h][e] * w));
        if (lane == 0) {
            s_wm[wave][h] = M;
            s_wl[wave][h] = l;
        }
        if (grp == 0)
#pragma unroll
            for (int e = 0; e < 8; e++) s_wacc[wave][h][8 * sub + e] = acc[h][e];
    }
    __syncthreads();
    // combine the four waves and write the split partial
    for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
        const int h = t / D, dd = t % D;
        float M = s_wm[0][h];
#pragma unroll
        for (int w = 1; w < ATTN_WAVES; w++) M = fmaxf(M, s_wm[w][h]);
        float l = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < ATTN_WAVES; w++) {
            const float e = (s_wm[w][h] == -INFINITY) ? 0.f : exp2_fast(s_wm[w][h] - M);
            l = fmaf(s_wl[w][h], e, l);
            o = fmaf(s_wacc[w][h][dd], e, o);
        }
        float* dst = part0 + ((size_t)h * a.S + s) * ATTN_PART_F;
        dst[2 + dd] = o;
        if (dd == 0) {
            dst[0] = M * 0.6931471805599453f;
            dst[1] = l;
        }
    }
}

// ---- merge of the key splits -----------------------------------------------------------------
// grid Hq, 128 threads: o = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s.
constexpr int MERGE_MAX_S = 1024;
__global__ __launch_bounds__(128) void merge_kernel(MergeArgs a) {
    __shared__ float s_w[MERGE_MAX_S];
    __shared__ float s_wl[MERGE_MAX_S];
    __shared__ float s_o[128];
    __shared__ float s_M;
    const int h = blockIdx.x, d = threadIdx.x;
    const float* p = a.part + (size_t)blockIdx.y * a.part_stride + (size_t)h * a.S * ATTN_PART_F;
    // up to MERGE_REG_S split accumulators are loaded at once, in flight while the
    // maxima are reduced (32: the split count of 8 KV heads at one block per CU)
    constexpr int MERGE_REG_S = 32;
    const bool in_regs = a.S <= MERGE_REG_S;
    float accv[MERGE_REG_S];
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < MERGE_REG_S; j++) accv[j] = p[(size_t)min(j, a.S - 1) * ATTN_PART_F + 2 + d];
    }
    for (int s0 = 0; s0 < a.S; s0 += 8 * 128) {
        float mloc[8], lloc[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int s = s0 + d + j * 128, sc = s < a.S ? s : 0;
            mloc[j] = p[(size_t)sc * ATTN_PART_F];
            lloc[j] = p[(size_t)sc * ATTN_PART_F + 1];
        }
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int s = s0 + d + j * 128;
            if (s < a.S) {
                s_w[s] = mloc[j];
                s_wl[s] = lloc[j];
            }
        }
    }
    __syncthreads();
    if (d < 64) {
        float M = -INFINITY;
        for (int s = d; s < a.S; s += 64) M = fmaxf(M, s_w[s]);
        M = wave_max(M);
        if (d == 0) s_M = M;
    }
    __syncthreads();
    const float M = s_M;
    for (int s = d; s < a.S; s += 128) {
        const float m = s_w[s];
        const float w = (m == -INFINITY || M == -INFINITY) ? 0.f : __expf(m - M);
        s_w[s] = w;
        s_wl[s] = w * s_wl[s];
    }
    __syncthreads();
    float L = 0.f, o = 0.f;
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < MERGE_REG_S; j++) {
            if (j < a.S) {
                o = fmaf(s_w[j], accv[j], o);
                L += s_wl[j];
            }
        }
    }
    for (int s0 = 0; s0 < (in_regs ? 0 : a.S); s0 += 16) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const int s = min(s0 + j, a.S - 1);
            v[j] = p[(size_t)s * ATTN_PART_F + 2 + d];
        }
#pragma unroll
        for (int j = 0; j < 16; j++) {
            if (s0 + j < a.S) {
                o = fmaf(s_w[s0 + j], v[j], o);
                L += s_wl[s0 + j];
            }
        }
    }
    const float r = L > 0.f ? o / L : 0.f;
    if (a.o) a.o[(size_t)blockIdx.y * a.o_stride + (size_t)h * 128 + d] = r;
    if (a.xq.planes) {
        s_o[d] = r;
        __syncthreads();
        if (d < 16) {
            float x8[8];
#pragma unroll
            for (int i = 0; i < 8; i++) x8[i] = s_o[8 * d + i];
            xq_encode_word(x8, a.xq, h * 4 + (d >> 2), d & 3);
        }
    }
    if (a.bq.p) {
        s_o[d] = r;
        __syncthreads();
        if (d < 16) {   // one row of 16 lanes encodes the head's 128 values
            float x8[8];
#pragma unroll
            for (int i = 0; i < 8; i++) x8[i] = s_o[8 * d + i];
            bq_encode_row16(x8, a.bq, blockIdx.y, h * 128 + 8 * d, h);
        }
    }
}

// ---- final norm, bf16 lm_head and argmax partials ------------------------------------------------
//
// 512 threads; every block rebuilds the last layer's output and its final RMSNorm
// (d <= 8192), then each wave streams whole rows: lane l reads 16-byte words
// l, l+64, ... of the row (KW per lane); two rows are in flight per wave.

constexpr int HEAD_THREADS = 512;
template <int KW>
__global__ __launch_bounds__(HEAD_THREADS) void head_kernel(HeadArgs a) {
    __shared__ float s_x[8192];
    __shared__ float red[16];
    __shared__ float s_v[HEAD_THREADS / 64];
    __shared__ int s_i[HEAD_THREADS / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, NW = HEAD_THREADS / 64;
    const int nw = a.d / 8;
    const int r0 = blockIdx.x * a.rows_per_block, r1 = min(a.V, r0 + a.rows_per_block);
    auto load_row = [&](int row, uint4 (&w)[KW]) {
        const u32x4_t* W = reinterpret_cast<const u32x4_t*>(a.lm + (size_t)min(row, a.V - 1) * a.d);
#pragma unroll
        for (int j = 0; j < KW; j++) {
            const int wd = lane + 64 * j;
            const u32x4_t v = __builtin_nontemporal_load(W + (wd < nw ? wd : 0));
            w[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    XRegs<8192 / 4 / HEAD_THREADS> XR;
    x_issue<8192 / 4 / HEAD_THREADS, true>(a.src, a.d, XR);
    __builtin_amdgcn_sched_barrier(0);
    uint4 wa[KW], wb[KW];
    int row = r0 + wave;
    load_row(row, wa);   // unconditional (clamped), see prefetch_tiles
    x_finish<8192 / 4 / HEAD_THREADS, true>(a.src, a.d, XR, s_x, red);
    if (a.hidden_out && blockIdx.x == 0)
        for (int i = threadIdx.x; i < a.d; i += blockDim.x) a.hidden_out[i] = s_x[i];
    float ss = 0.f;
    for (int i = threadIdx.x; i < a.d; i += blockDim.x) ss = fmaf(s_x[i], s_x[i], ss);
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)a.d + a.eps);
    for (int i = threadIdx.x; i < a.d; i += blockDim.x) s_x[i] = a.g_final[i] * (s_x[i] * r);
    __syncthreads();
    float xr[KW][8];
#pragma unroll
    for (int j = 0; j < KW; j++) {
        const int wd = lane + 64 * j;
#pragma unroll
        for (int i = 0; i < 8; i++) xr[j][i] = wd < nw ? s_x[8 * wd + i] : 0.f;
    }
    float best = -INFINITY;
    int besti = 0x7FFFFFFF;
    auto dot_row = [&](const uint4 (&w)[KW]) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < KW; j++) {
            const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                acc = fmaf(__uint_as_float(ww[q] << 16), xr[j][2 * q], acc);
                acc = fmaf(__uint_as_float(ww[q] & 0xFFFF0000u), xr[j][2 * q + 1], acc);
            }
        }
        return wave_sum(acc);
    };
    for (; row < r1; row += 2 * NW) {
        const int row2 = row + NW;
        if (row2 < r1) load_row(row2, wb);
        __builtin_amdgcn_sched_barrier(0);
        float v = dot_row(wa);
        if (lane == 0) a.logits[row] = v;
        if (v > best) {   // rows increase within a wave: the first maximum stays
            best = v;
            besti = row;
        }
        if (row2 >= r1) break;
        if (row2 + NW < r1) load_row(row2 + NW, wa);
        __builtin_amdgcn_sched_barrier(0);
        v = dot_row(wb);
        if (lane == 0) a.logits[row2] = v;
        if (v > best) {
            best = v;
            besti = row2;
        }
    }
    if (lane == 0) {
        s_v[wave] = best;
        s_i[wave] = besti;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = s_v[0];
        int bi = s_i[0];
        for (int w = 1; w < NW; w++)
            if (s_v[w] > b || (s_v[w] == b && s_i[w] < bi)) {
                b = s_v[w];
                bi = s_i[w];
            }
        a.bmax[blockIdx.x] = b;
        a.bidx[blockIdx.x] = bi;
    }
}

__global__ __launch_bounds__(1024) void final_hidden_kernel(XSource src, int d, float* out) {
    __shared__ float s_x[8192];
    __shared__ float red[16];
    build_x<8192 / 4 / 1024>(src, d, s_x, red);
    for (int i = threadIdx.x; i < d; i += blockDim.x) out[i] = s_x[i];
}

__global__ __launch_bounds__(1024) void argmax_final2_kernel(const float* bmax, const int* bidx, int nb, int32_t* out) {
    __shared__ float s_v[1024];
    __shared__ int s_i[1024];
    float b = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int i = threadIdx.x; i < nb; i += blockDim.x)
        if (bmax[i] > b || (bmax[i] == b && bidx[i] < bi)) {
            b = bmax[i];
            bi = bidx[i];
        }
    s_v[threadIdx.x] = b;
    s_i[threadIdx.x] = bi;
    __syncthreads();
    for (int off = 512; off > 0; off >>= 1) {
        if (threadIdx.x < off) {
            const float v = s_v[threadIdx.x + off];
            const int vi = s_i[threadIdx.x + off];
            if (v > s_v[threadIdx.x] || (v == s_v[threadIdx.x] && vi < s_i[threadIdx.x])) {
                s_v[threadIdx.x] = v;
                s_i[threadIdx.x] = vi;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = s_i[0] == 0x7FFFFFFF ? 0 : s_i[0];
}

// ---- host-side planning and launch ---------------------------------------------------------------

GemvShape gemv_shape(int N, int K, bool split_k, int target_blocks, int max_cpl) {
    GemvShape g{};
    const int C = K / XQ_CHUNK;
    int best_s = -1, best_rb = 1, best_cpl = 0;
    double best_u = -1;
    for (int s = 1; s <= (split_k ? std::min(C, MAX_DOWN_SPLITS) : 1); s++) {
        if (C % s) continue;
        const int cw = C / s;
        if (cw * 4 > DOWN_MAX_ROUNDS * GEMV_THREADS) continue;
        for (int rb = 2; rb >= 1; rb--) {
            if (rb == 2 && (2 * cw) % 64) continue;
            const int cpl = (rb * cw + 63) / 64;
            if (cpl > max_cpl) continue;
            const double u = (double)(rb * cw) / (64.0 * cpl);
            if (u > best_u + 1e-9) {
                best_u = u;
                best_s = s;
                best_rb = rb;
                best_cpl = cpl;
            }
        }
        if (best_s > 0) break;   // fewest ranges first
    }
    if (best_s < 0) return g;   // CPL stays 0: unsupported
    g.S = best_s;
    g.CW = C / best_s;
    g.RB = best_rb;
    g.CPL = best_cpl;
    const int T = (N + g.RB - 1) / g.RB;
    int bx = std::max(1, target_blocks / g.S);
    bx = std::min(bx, T);
    g.tiles_per_block = (T + bx - 1) / bx;
    g.blocks = (T + g.tiles_per_block - 1) / g.tiles_per_block;
    return g;
}

#define GEMV_CASE(KERNEL, C_, R_, grid, lds, st, args)                                         \
    if (s.CPL == C_ && s.RB == R_) {                                                            \
        ATLAS_KLAUNCH((KERNEL<C_, R_>), grid, dim3(GEMV_THREADS), lds, st, args);          \
        ATLAS_LAUNCH_CHECK(#KERNEL);                                                            \
        return ATLAS_OK;                                                                        \
    }
#define GEMV_DISPATCH5(KERNEL, grid, lds, st, args)                                             \
    GEMV_CASE(KERNEL, 1, 1, grid, lds, st, args) GEMV_CASE(KERNEL, 2, 1, grid, lds, st, args)   \
    GEMV_CASE(KERNEL, 3, 1, grid, lds, st, args) GEMV_CASE(KERNEL, 4, 1, grid, lds, st, args)   \
    GEMV_CASE(KERNEL, 5, 1, grid, lds, st, args) GEMV_CASE(KERNEL, 1, 2, grid, lds, st, args)   \
    GEMV_CASE(KERNEL, 2, 2, grid, lds, st, args) GEMV_CASE(KERNEL, 3, 2, grid, lds, st, args)   \
    GEMV_CASE(KERNEL, 4, 2, grid, lds, st, args) GEMV_CASE(KERNEL, 5, 2, grid, lds, st, args)   \
    return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, #KERNEL ": no instance for CPL=%d RB=%d", s.CPL, s.RB);
#define GEMV_DISPATCH3(KERNEL, grid, lds, st, args)                                             \
    GEMV_CASE(KERNEL, 1, 1, grid, lds, st, args) GEMV_CASE(KERNEL, 2, 1, grid, lds, st, args)   \
    GEMV_CASE(KERNEL, 3, 1, grid, lds, st, args) GEMV_CASE(KERNEL, 1, 2, grid, lds, st, args)   \
    GEMV_CASE(KERNEL, 2, 2, grid, lds, st, args) GEMV_CASE(KERNEL, 3, 2, grid, lds, st, args)   \
    return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, #KERNEL ": no instance for CPL=%d RB=%d", s.CPL, s.RB);

int launch_qkv(const QkvArgs& a0, const GemvShape& s, hipStream_t st) {
    QkvArgs a = a0;
    a.CW = s.CW;
    a.tiles_per_block = s.tiles_per_block;
    const size_t lds = (size_t)a.d * 4 + planes_lds_bytes(s.CW);
    prof_mark("w4_gemv_qkv", st);
    if (a.src.mode == X_FROM_RESIDUAL) {
        GEMV_DISPATCH5(qkv_resid_kernel, dim3(s.blocks), lds, st, a);
    }
    GEMV_DISPATCH5(qkv_kernel, dim3(s.blocks), lds, st, a);
}

int launch_gemv_planes(const GemvPlanesArgs& a0, const GemvShape& s, hipStream_t st, const char* label) {
    GemvPlanesArgs a = a0;
    a.CW = s.CW;
    a.tiles_per_block = s.tiles_per_block;
    prof_mark(label, st);
    GEMV_DISPATCH5(gemv_planes_kernel, dim3(s.blocks, s.S), planes_lds_bytes(s.CW), st, a);
}

int launch_gate_up(const GateUpArgs& a0, const GemvShape& s, hipStream_t st) {
    GateUpArgs a = a0;
    a.CW = s.CW;
    a.tiles_per_block = s.tiles_per_block;
    const size_t lds = (size_t)a.d * 4 + planes_lds_bytes(s.CW);
    prof_mark("w4_gemv_gate_up", st);
    GEMV_DISPATCH3(gate_up_kernel, dim3(s.blocks), lds, st, a);
}

int launch_down(const DownArgs& a0, const GemvShape& s, hipStream_t st) {
    DownArgs a = a0;
    a.CW = s.CW;
    a.tiles_per_block = s.tiles_per_block;
    prof_mark("w4_gemv_down", st);
    GEMV_DISPATCH5(down_kernel, dim3(s.blocks, s.S), planes_lds_bytes(s.CW), st, a);
}

// Key splits per KV head: at least 64 keys each, and at most one block per CU over the
// KV heads (more, smaller blocks measured slower at 16K: 512 blocks of 4 waves lost to
// 256). Past 1,024 keys per split the key loop outweighs the per-block prologue and two
// blocks per CU pay off (65,536 keys, 8 KV heads: 64 us against 72 us).
constexpr int ATTN_GRID_BLOCKS = 256;
int attn_splits(int64_t maxkeys, int Hkv) {
    int64_t S = (maxkeys + 63) / 64;
    int64_t cap = std::max(1, (ATTN_GRID_BLOCKS + Hkv - 1) / Hkv);
    if (maxkeys > 1024 * cap) cap = std::max(1, (2 * ATTN_GRID_BLOCKS + Hkv - 1) / Hkv);
    if (S > cap) S = cap;
    if (S < 1) S = 1;
    return (int)S;
}

int launch_attn_fused(const AttnFusedArgs& a, int G, hipStream_t st) {
    dim3 grid(a.S, a.Hkv, std::max(1, a.batch));
    prof_mark(a.window > 0 ? "attn_window" : "attn_full", st);
    switch (G) {
#define C(G_)                                                                           \
    case G_:                                                                            \
        if (a.kv_bf16) {                                                                            \
            if (a.fused) ATLAS_KLAUNCH((attn_kernel<G_, true, true>), grid, dim3(ATTN_THREADS), 0, st, a); \
            else ATLAS_KLAUNCH((attn_kernel<G_, false, true>), grid, dim3(ATTN_THREADS), 0, st, a);        \
        } else {                                                                                    \
            if (a.fused) ATLAS_KLAUNCH((attn_kernel<G_, true, false>), grid, dim3(ATTN_THREADS), 0, st, a); \
            else ATLAS_KLAUNCH((attn_kernel<G_, false, false>), grid, dim3(ATTN_THREADS), 0, st, a);        \
        }                                                                                           \
        break;
        C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8)
#undef C
        default: return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, "Hq/Hkv=%d > 8", G);
    }
    ATLAS_LAUNCH_CHECK("attn_kernel");
    return ATLAS_OK;
}

int launch_merge(const MergeArgs& a, hipStream_t st) {
    if (a.S > MERGE_MAX_S) return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, "too many key splits (%d)", a.S);
    prof_mark("attn_merge", st);
    ATLAS_KLAUNCH(merge_kernel, dim3(a.Hq, std::max(1, a.batch)), dim3(128), 0, st, a);
    ATLAS_LAUNCH_CHECK("merge_kernel");
    return ATLAS_OK;
}

int launch_head(const HeadArgs& a, int blocks, hipStream_t st) {
    const int kw = (a.d / 8 + 63) / 64;
    prof_mark("lm_head_bf16", st);
    if (kw <= 2) ATLAS_KLAUNCH((head_kernel<2>), dim3(blocks), dim3(HEAD_THREADS), 0, st, a);
    else if (kw <= 4) ATLAS_KLAUNCH((head_kernel<4>), dim3(blocks), dim3(HEAD_THREADS), 0, st, a);
    else if (kw <= 10) ATLAS_KLAUNCH((head_kernel<10>), dim3(blocks), dim3(HEAD_THREADS), 0, st, a);
    else if (kw <= 16) ATLAS_KLAUNCH((head_kernel<16>), dim3(blocks), dim3(HEAD_THREADS), 0, st, a);
    else return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, "d=%d too large for the lm_head kernel", a.d);
    ATLAS_LAUNCH_CHECK("head_kernel");
    return ATLAS_OK;
}

int launch_final_hidden(const XSource& src, int d, float* out, hipStream_t st) {
    prof_mark("final_hidden", st);
    ATLAS_KLAUNCH(final_hidden_kernel, dim3(1), dim3(1024), 0, st, src, d, out);
    ATLAS_LAUNCH_CHECK("final_hidden_kernel");
    return ATLAS_OK;
}

int launch_argmax_final(const float* bmax, const int* bidx, int nb, int32_t* out, hipStream_t st) {
    prof_mark("argmax", st);
    ATLAS_KLAUNCH(argmax_final2_kernel, dim3(1), dim3(1024), 0, st, bmax, bidx, nb, out);
    ATLAS_LAUNCH_CHECK("argmax_final_kernel");
    return ATLAS_OK;
}

}  // namespace atlas
