// GQA decode attention over an f32 KV cache, split over the key range with an
// online-softmax merge.
//
// Sources: "ATLAS-OLMo-3-32B-Think-v4", Architecture deep-dive (GQA 40 query / 8 KV
// heads of 128; sliding window 4,096 on three of every four layers, full context on
// the fourth) and Why the 3:1 SWA layout matters (SWA layers never look back more
// than 4,096 tokens); f32 KV cache (VRAM breakdown).
//
// With only 8 KV heads a decode step cannot fill 256 compute units one head per
// workgroup, so each KV head's key range is cut into S splits. A workgroup reads its
// splits's keys and values once for all Hq/Hkv query heads that share them, and
// writes a partial (max m, sum l, unnormalised acc[D]) per query head; the merge
// rescales the partials by exp(m_s - max_s m_s).
#include "attention.h"

namespace atlas {

// keys [lo, hi] of the step; window > 0 counts the current token
__device__ __forceinline__ void key_range(int pos, int window, int* lo, int* n) {
    int l = window > 0 ? pos - window + 1 : 0;
    if (l < 0) l = 0;
    *lo = l;
    *n = pos - l + 1;
}

// grid (S, Hkv), 256 threads. 16 lanes cover one key (8 dims each), a wave 4 keys,
// the block 16 keys per step.
template <int G>
__global__ __launch_bounds__(256) void gqa_partial_kernel(AttnArgs a) {
    extern __shared__ float s_p[];          // [G][Lmax] scores, then probabilities
    __shared__ float s_red[4][G][128];
    __shared__ float s_stat[2][G];
    __shared__ float red[16];
    const int s = blockIdx.x, kv = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane & 15, grp = lane >> 4;
    const int pos = *a.d_pos;
    const bool pos_ok = pos >= 0 && pos < a.T_max;
    int lo, nkeys;
    key_range(pos_ok ? pos : 0, a.window, &lo, &nkeys);
    const int L = (nkeys + a.S - 1) / a.S;
    const int k0 = lo + s * L;
    int cnt = min(L, lo + nkeys - k0);
    if (cnt < 0 || !pos_ok) cnt = 0;

    // queries of this KV head's group, dims [8*sub, 8*sub+8)
    float q[G][8];
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float4* qp = reinterpret_cast<const float4*>(a.q + (size_t)(kv * G + h) * 128 + 8 * sub);
        float4 u = qp[0], v = qp[1];
        q[h][0] = u.x; q[h][1] = u.y; q[h][2] = u.z; q[h][3] = u.w;
        q[h][4] = v.x; q[h][5] = v.y; q[h][6] = v.z; q[h][7] = v.w;
    }
    const float* Kh = a.k_cache + (size_t)kv * a.T_max * 128;
    const float* Vh = a.v_cache + (size_t)kv * a.T_max * 128;

    // scores
    for (int kk = wave * 4 + grp; kk < ((cnt + 15) & ~15); kk += 16) {
        const bool ok = kk < cnt;
        const float4* kp = reinterpret_cast<const float4*>(Kh + (size_t)(k0 + (ok ? kk : 0)) * 128 + 8 * sub);
        float4 u = kp[0], v = kp[1];
        const float kx[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < G; h++) {
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) d = fmaf(q[h][i], kx[i], d);
            d = row16_sum(d);
            if (ok && sub == 0) s_p[h * a.Lmax + kk] = d * a.scale;
        }
    }
    __syncthreads();
    // per-head max and exp
#pragma unroll
    for (int h = 0; h < G; h++) {
        float m = -INFINITY;
        for (int i = threadIdx.x; i < cnt; i += 256) m = fmaxf(m, s_p[h * a.Lmax + i]);
        m = wave_max(m);
        if (lane == 0) s_red[0][h][wave] = m;
    }
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        s_stat[0][h] = fmaxf(fmaxf(s_red[0][h][0], s_red[0][h][1]), fmaxf(s_red[0][h][2], s_red[0][h][3]));
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float m = s_stat[0][h];
        float l = 0.f;
        for (int i = threadIdx.x; i < cnt; i += 256) {
            const float p = __expf(s_p[h * a.Lmax + i] - m);
            s_p[h * a.Lmax + i] = p;
            l += p;
        }
        l = block_sum(l, red);
        if (threadIdx.x == 0) s_stat[1][h] = l;
    }
    __syncthreads();
    // values
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) acc[h][i] = 0.f;
    for (int kk = wave * 4 + grp; kk < cnt; kk += 16) {
        const float4* vp = reinterpret_cast<const float4*>(Vh + (size_t)(k0 + kk) * 128 + 8 * sub);
        float4 u = vp[0], v = vp[1];
        const float vx[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float p = s_p[h * a.Lmax + kk];
#pragma unroll
            for (int i = 0; i < 8; i++) acc[h][i] = fmaf(p, vx[i], acc[h][i]);
        }
    }
    // reduce the 4 key groups of a wave, then the 4 waves
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float v = acc[h][i];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[h][i] = v;
        }
    __syncthreads();
    if (grp == 0) {
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int i = 0; i < 8; i++) s_red[wave][h][8 * sub + i] = acc[h][i];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < G * 128; t += 256) {
        const int h = t / 128, d = t % 128;
        const float v = s_red[0][h][d] + s_red[1][h][d] + s_red[2][h][d] + s_red[3][h][d];
        float* dst = a.part + ((size_t)(kv * G + h) * a.S + s) * ATTN_PART;
        dst[2 + d] = v;
        if (d == 0) {
            dst[0] = cnt > 0 ? s_stat[0][h] : -INFINITY;
            dst[1] = cnt > 0 ? s_stat[1][h] : 0.f;
        }
    }
}

// grid Hq, 128 threads: o[h][d] = sum_s e^{m_s - M} acc_s[d] / sum_s e^{m_s - M} l_s.
// Optionally encodes o for the next W4 GEMV (chunks of 32 dims).
__global__ __launch_bounds__(128) void gqa_merge_kernel(const float* __restrict__ part, int S, float* out, XQ xq) {
    __shared__ float s_o[128];
    const int h = blockIdx.x, d = threadIdx.x;
    const float* p = part + (size_t)h * S * ATTN_PART;
    float M = -INFINITY;
    for (int s = 0; s < S; s++) M = fmaxf(M, p[s * ATTN_PART]);
    float l = 0.f, o = 0.f;
    for (int s = 0; s < S; s++) {
        const float m = p[s * ATTN_PART];
        if (m == -INFINITY) continue;
        const float w = __expf(m - M);
        l = fmaf(w, p[s * ATTN_PART + 1], l);
        o = fmaf(w, p[s * ATTN_PART + 2 + d], o);
    }
    const float r = l > 0.f ? o / l : 0.f;
    out[(size_t)h * 128 + d] = r;
    if (xq.planes) {
        s_o[d] = r;
        __syncthreads();
        if (d < 16) {
            float x8[8];
#pragma unroll
            for (int i = 0; i < 8; i++) x8[i] = s_o[8 * d + i];
            xq_encode_word(x8, xq, h * 4 + (d >> 2), d & 3);
        }
    }
}

AttnPlan plan_attention(int Hq, int Hkv, int64_t T_max, int window) {
    AttnPlan p{};
    int64_t maxkeys = window > 0 ? std::min<int64_t>(window, T_max) : T_max;
    int S = (int)((maxkeys + 63) / 64);
    int cap = std::max(1, 1024 / Hkv);
    if (S > cap) S = cap;
    if (S < 1) S = 1;
    p.S = S;
    p.Lmax = (int)((maxkeys + S - 1) / S);
    p.part_bytes = (size_t)Hq * S * ATTN_PART * 4;
    return p;
}

int launch_attention(const AttnArgs& a0, const AttnPlan& p, int G, XQ xq, float* out, hipStream_t st) {
    AttnArgs a = a0;
    a.S = p.S;
    a.Lmax = p.Lmax;
    const size_t sh = (size_t)G * p.Lmax * 4;
    if (sh > 64 * 1024) return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, "attention split too long (%d keys)", p.Lmax);
    dim3 grid(p.S, a.Hkv);
    switch (G) {
#define C(G_)                                                                                \
    case G_:                                                                                 \
        hipLaunchKernelGGL((gqa_partial_kernel<G_>), grid, dim3(256), sh, st, a);            \
        break;
        C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8)
#undef C
        default: return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, "Hq/Hkv=%d > 8", G);
    }
    ATLAS_LAUNCH_CHECK("gqa_partial_kernel");
    hipLaunchKernelGGL(gqa_merge_kernel, dim3(a.Hkv * G), dim3(128), 0, st, a.part, p.S, out, xq);
    ATLAS_LAUNCH_CHECK("gqa_merge_kernel");
    return ATLAS_OK;
}

}  // namespace atlas

using namespace atlas;

extern "C" size_t atlas_gqa_decode_workspace_bytes(int32_t Hq, int32_t Hkv, int32_t D, int64_t T_max) {
    if (Hq < 1 || Hkv < 1 || D != 128 || T_max < 1) return 0;
    return plan_attention(Hq, Hkv, T_max, 0).part_bytes;
}

extern "C" int atlas_gqa_decode(const float* q, const float* k_cache, const float* v_cache, int32_t Hq,
                                int32_t Hkv, int32_t D, int64_t T_max, const int32_t* d_pos, int32_t window,
                                float softmax_scale, float* out, void* ws, size_t ws_bytes, void* stream) {
    ATLAS_CHECK_ARG(q && k_cache && v_cache && d_pos && out && ws, "null pointer");
    ATLAS_CHECK_ARG(Hq >= 1 && Hkv >= 1 && T_max >= 1, "bad sizes");
    ATLAS_CHECK_SHAPE(D == 128, "head_dim %d unsupported (128 only)", D);
    ATLAS_CHECK_SHAPE(Hq % Hkv == 0 && Hq / Hkv <= 8, "Hq/Hkv must be an integer <= 8");
    ATLAS_CHECK_ARG(window >= 0, "window must be >= 0");
    ATLAS_CHECK_ARG(T_max <= (int64_t)1 << 30, "T_max too large");
    AttnPlan p = plan_attention(Hq, Hkv, T_max, window);
    const size_t need = plan_attention(Hq, Hkv, T_max, 0).part_bytes;
    if (ws_bytes < need) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
    AttnArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.part = (float*)ws;
    a.Hkv = Hkv;
    a.T_max = T_max;
    a.d_pos = d_pos;
    a.window = window;
    a.scale = softmax_scale;
    return launch_attention(a, p, Hq / Hkv, XQ{}, out, (hipStream_t)stream);
}
