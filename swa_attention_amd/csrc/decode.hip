// The single-token decode step: embedding, the layer stack, final norm, bf16 lm_head
// and greedy argmax.
//
// Sources: "ATLAS-OLMo-3-32B-Think-v4" -- Architecture deep-dive (64 layers in a
// [SWA, SWA, SWA, full] x16 layout, GQA 40/8, post-norm + QK-norm, YaRN only where
// the layer is full) and VRAM breakdown (W4 weights, bf16 lm_head, f32 KV cache);
// "OLMo 3 32B" (LLM Architecture KB) -- reordered post-norm: h = x + N(attn(x)),
// y = h + N(mlp(h)); "Olmo 3 32B" field table -- untied embedding and head.
#include <cstring>
#include <vector>

#include "attention.h"
#include "decode.h"
#include "gemv.h"
#include "norm_rope.h"

namespace atlas {

// ---- small kernels ----------------------------------------------------------------------

// x = bf16 embedding row of *d_token (or a copy of hidden_in); encode x; reset status.
__global__ __launch_bounds__(1024) void input_kernel(const int32_t* d_token, const uint16_t* emb, int vocab,
                                                     const float* hidden_in, int d, float* x, XQ xq,
                                                     int* status) {
    extern __shared__ float s_x[];   // d floats
    __shared__ int s_tok;
    if (threadIdx.x == 0) {
        int tok = d_token ? *d_token : 0;
        if (d_token && (tok < 0 || tok >= vocab)) {
            *status = ATLAS_ERR_INVALID_ARG;
            tok = 0;
        } else {
            *status = ATLAS_OK;
        }
        s_tok = tok;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        float v = d_token ? bf16_bits_to_f32(emb[(size_t)s_tok * d + i]) : hidden_in[i];
        s_x[i] = v;
        x[i] = v;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < d / 8; t += blockDim.x) {
        float x8[8];
#pragma unroll
        for (int i = 0; i < 8; i++) x8[i] = s_x[8 * t + i];
        xq_encode_word(x8, xq, t >> 2, t & 3);
    }
}

// z = silu(u) * v with u, v the sums of S partial vectors; z is written and encoded.
// One thread per 8 elements (quads form 32-element chunks).
__global__ __launch_bounds__(256) void swiglu_encode_kernel(const float* __restrict__ up_g, const float* __restrict__ up_u,
                                                            int S, int n, float* z, XQ xq) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t < n / 8) {
        float x8[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int e = 8 * t + i;
            float g = 0.f, u = 0.f;
            for (int r = 0; r < S; r++) {
                g += up_g[(size_t)r * n + e];
                u += up_u[(size_t)r * n + e];
            }
            const float si = g / (1.0f + __expf(-g));
            x8[i] = si * u;
            z[e] = x8[i];
        }
        xq_encode_word(x8, xq, t >> 2, t & 3);
    }
}

// bf16 lm_head GEMV with a per-block (max, first index) reduction.
// Each wave streams whole rows: lane l reads 16-byte words l, l+64, ... of the row.
constexpr int LM_KMAX_WORDS = 16;   // d <= 64 * 16 * 8 = 8192
__global__ __launch_bounds__(256) void lm_head_kernel(const uint16_t* __restrict__ W, int V, int d,
                                                      const float* __restrict__ x, float* __restrict__ logits,
                                                      float* __restrict__ bmax, int* __restrict__ bidx,
                                                      int rows_per_block) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = d / 8;             // 16-byte words per row
    float xr[LM_KMAX_WORDS][8];
#pragma unroll
    for (int j = 0; j < LM_KMAX_WORDS; j++) {
        const int wd = lane + 64 * j;
        if (wd < nw) {
            const float4* p = reinterpret_cast<const float4*>(x) + 2 * wd;
            float4 a = p[0], b = p[1];
            xr[j][0] = a.x; xr[j][1] = a.y; xr[j][2] = a.z; xr[j][3] = a.w;
            xr[j][4] = b.x; xr[j][5] = b.y; xr[j][6] = b.z; xr[j][7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++) xr[j][i] = 0.f;
        }
    }
    const int r0 = blockIdx.x * rows_per_block;
    const int r1 = min(V, r0 + rows_per_block);
    float best = -INFINITY;
    int besti = 0x7FFFFFFF;
    for (int r = r0 + wave; r < r1; r += 4) {
        const uint4* row = reinterpret_cast<const uint4*>(W + (size_t)r * d);
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < LM_KMAX_WORDS; j++) {
            const int wd = lane + 64 * j;
            if (wd < nw) {
                const uint4 w = row[wd];
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    acc = fmaf(__uint_as_float(ww[q] << 16), xr[j][2 * q], acc);
                    acc = fmaf(__uint_as_float(ww[q] & 0xFFFF0000u), xr[j][2 * q + 1], acc);
                }
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) logits[r] = acc;
        if (acc > best) {   // rows increase within a wave: the first maximum is kept
            best = acc;
            besti = r;
        }
    }
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    if (lane == 0) {
        s_v[wave] = best;
        s_i[wave] = besti;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = s_v[0];
        int bi = s_i[0];
        for (int w = 1; w < 4; w++)
            if (s_v[w] > b || (s_v[w] == b && s_i[w] < bi)) {
                b = s_v[w];
                bi = s_i[w];
            }
        bmax[blockIdx.x] = b;
        bidx[blockIdx.x] = bi;
    }
}

__global__ __launch_bounds__(1024) void argmax_final_kernel(const float* bmax, const int* bidx, int nb, int32_t* out) {
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

// ---- workspace layout ---------------------------------------------------------------------

struct Carver {
    char* base;
    size_t off = 0;
    void* take(size_t n) {
        void* p = base ? base + off : nullptr;
        off += align_up(n, 256);
        return p;
    }
};

struct DecodeWs {
    int* status;
    float *x, *h, *q, *o, *yhat, *z, *logits, *bmax;
    int* bidx;
    XQ xq_x, xq_h, xq_o, xq_z;
    float *qkv_part, *a_part, *g_part, *u_part, *m_part, *attn_part;
    size_t bytes;
};

static DecodeWs carve(const atlas_model* m, void* base) {
    DecodeWs w{};
    Carver c{(char*)base};
    const int nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    GemvPlan pqkv = plan_gemv(nqkv, m->d), po = plan_gemv(m->d, nq), pg = plan_gemv(m->dff, m->d),
             pd = plan_gemv(m->d, m->dff);
    AttnPlan pa = plan_attention(m->hq, m->hkv, m->t_max, 0);
    w.status = (int*)c.take(256);
    w.x = (float*)c.take((size_t)m->d * 4);
    w.h = (float*)c.take((size_t)m->d * 4);
    w.q = (float*)c.take((size_t)nq * 4);
    w.o = (float*)c.take((size_t)nq * 4);
    w.yhat = (float*)c.take((size_t)m->d * 4);
    w.z = (float*)c.take((size_t)m->dff * 4);
    w.xq_x = xq_view(c.take(xq_bytes(m->d)), m->d);
    w.xq_h = xq_view(c.take(xq_bytes(m->d)), m->d);
    w.xq_o = xq_view(c.take(xq_bytes(nq)), nq);
    w.xq_z = xq_view(c.take(xq_bytes(m->dff)), m->dff);
    w.qkv_part = (float*)c.take((size_t)pqkv.S * nqkv * 4);
    w.a_part = (float*)c.take((size_t)po.S * m->d * 4);
    w.g_part = (float*)c.take((size_t)pg.S * m->dff * 4);
    w.u_part = (float*)c.take((size_t)pg.S * m->dff * 4);
    w.m_part = (float*)c.take((size_t)pd.S * m->d * 4);
    w.attn_part = (float*)c.take(pa.part_bytes);
    const int nb = LM_BLOCKS;
    w.logits = (float*)c.take((size_t)std::max(m->vocab, 1) * 4);
    w.bmax = (float*)c.take((size_t)nb * 4);
    w.bidx = (int*)c.take((size_t)nb * 4);
    w.bytes = c.off;
    return w;
}

int validate_model(const atlas_model* m) {
    ATLAS_CHECK_ARG(m != nullptr, "null model");
    ATLAS_CHECK_ARG(m->layers != nullptr && m->n_layers >= 1, "model has no layers");
    ATLAS_CHECK_SHAPE(m->hd == 128, "head_dim %d unsupported (128 only)", m->hd);
    ATLAS_CHECK_SHAPE(m->hq >= 1 && m->hkv >= 1 && m->hq % m->hkv == 0 && m->hq / m->hkv <= 8,
                      "head counts %d/%d unsupported", m->hq, m->hkv);
    ATLAS_CHECK_SHAPE(m->d % 32 == 0 && m->d <= 16384, "d=%d must be a multiple of 32 and <= 16384", m->d);
    ATLAS_CHECK_SHAPE(m->dff % 32 == 0, "dff=%d must be a multiple of 32", m->dff);
    ATLAS_CHECK_SHAPE((m->hq + m->hkv) * m->hd * 4 <= 60 * 1024, "q/k projection too large");
    ATLAS_CHECK_ARG(m->t_max >= 1 && m->t_max <= (int64_t)1 << 30, "bad t_max");
    ATLAS_CHECK_ARG(m->window >= 0, "bad window");
    ATLAS_CHECK_ARG(m->eps >= 0.f, "bad eps");
    const int nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    for (int l = 0; l < m->n_layers; l++) {
        const atlas_layer& L = m->layers[l];
        struct { const atlas_w4* w; int N, K; const char* name; } ws[5] = {
            {&L.qkv, nqkv, m->d, "qkv"}, {&L.o, m->d, nq, "o"}, {&L.gate, m->dff, m->d, "gate"},
            {&L.up, m->dff, m->d, "up"}, {&L.down, m->d, m->dff, "down"}};
        for (auto& e : ws) {
            int rc = validate_w4(e.w);
            if (rc) return fail(rc, "layer %d %s: %s", l, e.name, atlas_last_error());
            ATLAS_CHECK_SHAPE(e.w->N == e.N && e.w->K == e.K, "layer %d %s: shape %dx%d, expected %dx%d", l,
                              e.name, e.w->N, e.w->K, e.N, e.K);
            ATLAS_CHECK_SHAPE(plan_gemv(e.N, e.K).CW > 0, "layer %d %s: K=%d unsupported", l, e.name, e.K);
        }
        ATLAS_CHECK_ARG(L.g_q && L.g_k && L.g_pa && L.g_pf, "layer %d: null gain", l);
        ATLAS_CHECK_ARG(L.k_cache && L.v_cache, "layer %d: null KV cache", l);
        ATLAS_CHECK_ARG(L.type == 0 || L.type == 1, "layer %d: type must be 0 or 1", l);
    }
    return ATLAS_OK;
}

size_t decode_ws_bytes(const atlas_model* m) { return carve(m, nullptr).bytes; }

}  // namespace atlas

using namespace atlas;

extern "C" size_t atlas_decode_workspace_bytes(const atlas_model* m) {
    if (validate_model(m) != ATLAS_OK) return 0;
    return decode_ws_bytes(m);
}

extern "C" int atlas_decode_step(const atlas_model* m, const int32_t* d_token, const float* d_hidden_in,
                                 const int32_t* d_pos, float* d_hidden_out, float* d_logits, int32_t* d_argmax,
                                 void* ws, size_t ws_bytes, void* stream) {
    int rc = validate_model(m);
    if (rc) return rc;
    ATLAS_CHECK_ARG(d_pos != nullptr, "null d_pos");
    ATLAS_CHECK_ARG(d_token || d_hidden_in, "need d_token or d_hidden_in");
    ATLAS_CHECK_ARG(!d_token || m->embedding, "token input needs an embedding table");
    const bool head = d_logits || d_argmax;
    ATLAS_CHECK_ARG(!head || (m->lm_head && m->g_final && m->vocab >= 1), "lm_head/g_final/vocab missing");
    ATLAS_CHECK_ARG(ws != nullptr, "null workspace");
    const size_t need = decode_ws_bytes(m);
    if (ws_bytes < need) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
    hipStream_t st = (hipStream_t)stream;
    DecodeWs w = carve(m, ws);
    const int nq = m->hq * m->hd, nk = m->hkv * m->hd, nqkv = nq + 2 * nk;

    hipLaunchKernelGGL(input_kernel, dim3(1), dim3(1024), (size_t)m->d * 4, st, d_token, m->embedding, m->vocab,
                       d_hidden_in, m->d, w.x, w.xq_x, w.status);
    ATLAS_LAUNCH_CHECK("input_kernel");

    RopeTable rt_swa, rt_full;
    rope_table(&m->rope_swa, m->hd, &rt_swa);
    rope_table(&m->rope_full, m->hd, &rt_full);
    const GemvPlan pqkv = plan_gemv(nqkv, m->d), po = plan_gemv(m->d, nq), pg = plan_gemv(m->dff, m->d),
                   pd = plan_gemv(m->d, m->dff);

    for (int l = 0; l < m->n_layers; l++) {
        const atlas_layer& L = m->layers[l];
        // qkv projection
        rc = launch_gemv(gemv_args(&L.qkv, w.xq_x, w.qkv_part), pqkv, st);
        if (rc) return rc;
        // full-projection QK-norm, RoPE, KV append
        QkArgs qa{};
        qa.q = w.qkv_part;
        qa.k = w.qkv_part + nq;
        qa.v = w.qkv_part + nq + nk;
        qa.S = pqkv.S;
        qa.pstride = (size_t)nqkv;
        qa.gq = L.g_q;
        qa.gk = L.g_k;
        qa.q_out = w.q;
        qa.k_out = nullptr;
        qa.k_cache = L.k_cache;
        qa.v_cache = L.v_cache;
        qa.T_max = m->t_max;
        qa.Hq = m->hq;
        qa.Hkv = m->hkv;
        qa.D = m->hd;
        qa.eps = m->eps;
        qa.d_pos = d_pos;
        qa.status = w.status;
        qa.rope = L.type == 1 ? rt_full : rt_swa;
        rc = launch_qk_norm_rope(qa, st);
        if (rc) return rc;
        // attention
        AttnArgs aa{};
        aa.q = w.q;
        aa.k_cache = L.k_cache;
        aa.v_cache = L.v_cache;
        aa.part = w.attn_part;
        aa.Hkv = m->hkv;
        aa.T_max = m->t_max;
        aa.d_pos = d_pos;
        aa.window = L.type == 1 ? 0 : m->window;
        aa.scale = 1.0f / sqrtf((float)m->hd);
        rc = launch_attention(aa, plan_attention(m->hq, m->hkv, m->t_max, aa.window), m->hq / m->hkv, w.xq_o,
                              w.o, st);
        if (rc) return rc;
        // o projection, post-attention norm + residual
        rc = launch_gemv(gemv_args(&L.o, w.xq_o, w.a_part), po, st);
        if (rc) return rc;
        rc = launch_rmsnorm_residual(w.a_part, po.S, L.g_pa, w.x, w.h, m->d, m->eps, w.xq_h, st);
        if (rc) return rc;
        // SwiGLU feed-forward
        rc = launch_gemv(gemv_args(&L.gate, w.xq_h, w.g_part), pg, st);
        if (rc) return rc;
        rc = launch_gemv(gemv_args(&L.up, w.xq_h, w.u_part), pg, st);
        if (rc) return rc;
        hipLaunchKernelGGL(swiglu_encode_kernel, dim3((m->dff / 8 + 255) / 256), dim3(256), 0, st, w.g_part,
                           w.u_part, pg.S, m->dff, w.z, w.xq_z);
        ATLAS_LAUNCH_CHECK("swiglu_encode_kernel");
        rc = launch_gemv(gemv_args(&L.down, w.xq_z, w.m_part), pd, st);
        if (rc) return rc;
        // post-feed-forward norm + residual -> next layer's input
        rc = launch_rmsnorm_residual(w.m_part, pd.S, L.g_pf, w.h, w.x, m->d, m->eps, w.xq_x, st);
        if (rc) return rc;
    }
    if (d_hidden_out) {
        hipError_t e = hipMemcpyAsync(d_hidden_out, w.x, (size_t)m->d * 4, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return fail(ATLAS_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
    }
    if (head) {
        rc = launch_rmsnorm_residual(w.x, 1, m->g_final, nullptr, w.yhat, m->d, m->eps, XQ{}, st);
        if (rc) return rc;
        ATLAS_CHECK_SHAPE(m->d % 8 == 0 && m->d / 8 <= 64 * LM_KMAX_WORDS, "d=%d too large for lm_head", m->d);
        float* logits = d_logits ? d_logits : w.logits;
        const int rpb = (m->vocab + LM_BLOCKS - 1) / LM_BLOCKS;
        const int nb = (m->vocab + rpb - 1) / rpb;
        hipLaunchKernelGGL(lm_head_kernel, dim3(nb), dim3(256), 0, st, m->lm_head, m->vocab, m->d, w.yhat, logits,
                           w.bmax, w.bidx, rpb);
        ATLAS_LAUNCH_CHECK("lm_head_kernel");
        if (d_argmax) {
            hipLaunchKernelGGL(argmax_final_kernel, dim3(1), dim3(1024), 0, st, w.bmax, w.bidx, nb, d_argmax);
            ATLAS_LAUNCH_CHECK("argmax_final_kernel");
        }
    }
    return ATLAS_OK;
}

extern "C" int atlas_device_status(const void* ws, void* stream, int32_t* status_out) {
    ATLAS_CHECK_ARG(ws && status_out, "null pointer");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(status_out, ws, 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(ATLAS_ERR_HIP, "status read: %s", hipGetErrorString(e));
    return ATLAS_OK;
}
