// The single-token decode step: layer stack, final norm, bf16 lm_head and greedy
// argmax, as six fused launches per layer (decode_kernels.hip) plus two for the head.
//
// Sources: "ATLAS-OLMo-3-32B-Think-v4" -- Architecture deep-dive (64 layers in a
// [SWA, SWA, SWA, full] x16 layout, GQA 40/8, post-norm + QK-norm, YaRN only on the
// full layers) and VRAM breakdown (W4 weights, bf16 lm_head, f32 KV cache);
// "OLMo 3 32B" (LLM Architecture KB) -- reordered post-norm h = x + N(attn(x)),
// y = h + N(mlp(h)); "Olmo 3 32B" field table -- untied embedding and head.
#include <cmath>

#include "decode.h"
#include "decode_kernels.h"
#include "gemv.h"
#include "norm_rope.h"

namespace atlas {

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
    float *x, *h, *qkv, *ssq, *attn_part, *a, *z, *m_part, *logits, *bmax;
    int* bidx;
    XQ xq_o;
    size_t bytes;
};

struct DecodePlan {
    GemvShape qkv, o, gu, down;
    int S_swa, S_full, S_max;
    int head_blocks;
};

static DecodePlan make_plan(const atlas_model* m) {
    DecodePlan p{};
    const int nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    p.qkv = gemv_shape(nqkv, m->d, false, 256, 3);
    p.o = gemv_shape(m->d, nq, false, 256, 3);
    p.gu = gemv_shape(m->dff, m->d, false, 256, 3);
    p.down = gemv_shape(m->d, m->dff, true, 256, 4);
    const int64_t swa_keys = m->window > 0 ? std::min<int64_t>(m->window, m->t_max) : m->t_max;
    p.S_swa = attn_splits(swa_keys, m->hkv);
    p.S_full = attn_splits(m->t_max, m->hkv);
    p.S_max = std::max(p.S_swa, p.S_full);
    p.head_blocks = 256;
    return p;
}

static DecodeWs carve(const atlas_model* m, const DecodePlan& p, void* base) {
    DecodeWs w{};
    Carver c{(char*)base};
    const int nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    w.status = (int*)c.take(256);
    w.x = (float*)c.take((size_t)m->d * 4);
    w.h = (float*)c.take((size_t)m->d * 4);
    w.qkv = (float*)c.take((size_t)nqkv * 4);
    w.ssq = (float*)c.take((size_t)p.qkv.blocks * 2 * 4);
    w.attn_part = (float*)c.take((size_t)m->hq * p.S_max * ATTN_PART_F * 4);
    w.xq_o = xq_view(c.take(xq_bytes(nq)), nq);
    w.a = (float*)c.take((size_t)m->d * 4);
    w.z = (float*)c.take((size_t)m->dff * 4);
    w.m_part = (float*)c.take((size_t)std::max(p.down.S, 1) * m->d * 4);
    w.logits = (float*)c.take((size_t)std::max(m->vocab, 1) * 4);
    w.bmax = (float*)c.take((size_t)p.head_blocks * 4);
    w.bidx = (int*)c.take((size_t)p.head_blocks * 4);
    w.bytes = c.off;
    return w;
}

int validate_model(const atlas_model* m) {
    ATLAS_CHECK_ARG(m != nullptr, "null model");
    ATLAS_CHECK_ARG(m->layers != nullptr && m->n_layers >= 1, "model has no layers");
    ATLAS_CHECK_SHAPE(m->hd == 128, "head_dim %d unsupported (128 only)", m->hd);
    ATLAS_CHECK_SHAPE(m->hq >= 1 && m->hkv >= 1 && m->hq % m->hkv == 0 && m->hq / m->hkv <= 8,
                      "head counts %d/%d unsupported", m->hq, m->hkv);
    ATLAS_CHECK_SHAPE(m->d % 32 == 0 && m->d >= 32 && m->d <= 6144, "d=%d must be a multiple of 32 in [32, 6144]",
                      m->d);
    ATLAS_CHECK_SHAPE(m->dff % 32 == 0 && m->dff >= 32, "dff=%d must be a multiple of 32", m->dff);
    ATLAS_CHECK_ARG(m->t_max >= 1 && m->t_max <= (int64_t)1 << 30, "bad t_max");
    ATLAS_CHECK_ARG(m->window >= 0, "bad window");
    ATLAS_CHECK_ARG(m->eps >= 0.f, "bad eps");
    ATLAS_CHECK_ARG(m->kv_dtype == 0 || m->kv_dtype == 1, "kv_dtype must be 0 (f32) or 1 (bf16)");
    ATLAS_CHECK_ARG(!m->swa_ring || m->window > 0, "a sliding-window ring needs window > 0");
    const int nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    const DecodePlan p = make_plan(m);
    ATLAS_CHECK_SHAPE(p.qkv.CPL && p.o.CPL && p.gu.CPL && p.down.CPL, "projection shapes unsupported");
    ATLAS_CHECK_SHAPE(p.S_max <= 1024, "too many key splits");
    ATLAS_CHECK_SHAPE(p.qkv.blocks <= ATTN_SSQ_MAX_BLOCKS, "qkv projection needs too many blocks");
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
        }
        ATLAS_CHECK_SHAPE(L.gate.group == L.up.group, "layer %d: gate and up must share the group size", l);
        ATLAS_CHECK_ARG(L.g_q && L.g_k && L.g_pa && L.g_pf, "layer %d: null gain", l);
        ATLAS_CHECK_ARG(L.k_cache && L.v_cache, "layer %d: null KV cache", l);
        ATLAS_CHECK_ARG(L.type == 0 || L.type == 1, "layer %d: type must be 0 or 1", l);
    }
    return ATLAS_OK;
}

size_t decode_ws_bytes(const atlas_model* m) { return carve(m, make_plan(m), nullptr).bytes; }

static W4View view(const atlas_w4& w) {
    return w4_view(w.qweight, w.scales, w.zeros, w.N, w.K, w.group, w.scale_dtype);
}

// The layer stack for one token. Layer 0 reads its input from `first`; every later
// layer rebuilds it from the previous layer's down partials.
int run_decode_layers(const atlas_model* m, const XSource& first, const int32_t* d_pos, void* ws, hipStream_t st,
                      XSource* last_out) {
    const DecodePlan p = make_plan(m);
    DecodeWs w = carve(m, p, ws);
    RopeTable rt_swa, rt_full;
    rope_table(&m->rope_swa, m->hd, &rt_swa);
    rope_table(&m->rope_full, m->hd, &rt_full);
    int rc;
    for (int l = 0; l < m->n_layers; l++) {
        const atlas_layer& L = m->layers[l];
        // 1. qkv projection of x (x rebuilt from the previous layer's down partials)
        QkvArgs qa{};
        qa.W = view(L.qkv);
        if (l == 0) {
            qa.src = first;
        } else {
            qa.src.mode = X_FROM_RESIDUAL;
            qa.src.m_part = w.m_part;
            qa.src.S = p.down.S;
            qa.src.h = w.h;
            qa.src.g = m->layers[l - 1].g_pf;
            qa.src.eps = m->eps;
        }
        qa.d = m->d;
        qa.group = L.qkv.group;
        qa.qkv = w.qkv;
        qa.x_out = w.x;
        qa.status = l == 0 ? w.status : nullptr;
        qa.ssq_part = w.ssq;
        qa.nq = m->hq * m->hd;
        qa.nk = m->hkv * m->hd;
        if ((rc = launch_qkv(qa, p.qkv, st))) return rc;
        // 2. QK-norm, rotary, KV append and split attention
        AttnFusedArgs aa{};
        aa.qkv = w.qkv;
        aa.g_q = L.g_q;
        aa.g_k = L.g_k;
        aa.k_cache = L.k_cache;
        aa.v_cache = L.v_cache;
        aa.T_max = m->t_max;
        aa.ring = (m->swa_ring && L.type == 0) ? 1 : 0;
        aa.slots = aa.ring ? m->window : m->t_max;
        aa.kv_bf16 = m->kv_dtype;
        aa.d_pos = d_pos;
        aa.Hq = m->hq;
        aa.Hkv = m->hkv;
        aa.window = L.type == 1 ? 0 : m->window;
        aa.S = L.type == 1 ? p.S_full : p.S_swa;
        aa.scale = 1.0f / std::sqrt((float)m->hd);
        aa.eps = m->eps;
        const RopeTable& rt = L.type == 1 ? rt_full : rt_swa;
        for (int i = 0; i < 64; i++) aa.inv[i] = rt.inv[i];
        aa.mscale = rt.mscale;
        aa.part = w.attn_part;
        aa.status = w.status;
        aa.fused = 1;
        aa.ssq_part = w.ssq;
        aa.n_ssq = p.qkv.blocks;
        if ((rc = launch_attn_fused(aa, m->hq / m->hkv, st))) return rc;
        // 3. merge the key splits into o (encoded for the o projection)
        MergeArgs ma{};
        ma.part = w.attn_part;
        ma.S = aa.S;
        ma.Hq = m->hq;
        ma.o = nullptr;
        ma.xq = w.xq_o;
        if ((rc = launch_merge(ma, st))) return rc;
        // 4. o projection
        GemvPlanesArgs oa{};
        oa.W = view(L.o);
        oa.xq = w.xq_o;
        oa.group = L.o.group;
        oa.y = w.a;
        if ((rc = launch_gemv_planes(oa, p.o, st, "w4_gemv_o"))) return rc;
        // 5. h = x + RMSNorm_pa(a); gate/up projections + SwiGLU
        GateUpArgs ga{};
        ga.Wg = view(L.gate);
        ga.Wu = view(L.up);
        ga.a = w.a;
        ga.x = w.x;
        ga.g = L.g_pa;
        ga.eps = m->eps;
        ga.d = m->d;
        ga.group = L.gate.group;
        ga.h_out = w.h;
        ga.old_frac = GEMV_OLD_FRAC;
        ga.z = w.z;
        if ((rc = launch_gate_up(ga, p.gu, st))) return rc;
        // 6. down projection (split-K partials)
        DownArgs da{};
        da.W = view(L.down);
        da.z = w.z;
        da.group = L.down.group;
        da.m_part = w.m_part;
        da.old_frac = GEMV_OLD_FRAC;
        if ((rc = launch_down(da, p.down, st))) return rc;
    }
    XSource lo{};
    lo.mode = X_FROM_RESIDUAL;
    lo.m_part = w.m_part;
    lo.S = p.down.S;
    lo.h = w.h;
    lo.g = m->layers[m->n_layers - 1].g_pf;
    lo.eps = m->eps;
    *last_out = lo;
    return ATLAS_OK;
}

int run_head(const atlas_model* m, const XSource& last, void* ws, float* hidden_out, float* logits_out,
             int32_t* argmax_out, hipStream_t st) {
    const DecodePlan p = make_plan(m);
    DecodeWs w = carve(m, p, ws);
    int rc;
    if (logits_out || argmax_out) {
        HeadArgs ha{};
        ha.lm = m->lm_head;
        ha.V = m->vocab;
        ha.d = m->d;
        ha.rows_per_block = (m->vocab + p.head_blocks - 1) / p.head_blocks;
        ha.src = last;
        ha.g_final = m->g_final;
        ha.eps = m->eps;
        ha.hidden_out = hidden_out;
        ha.logits = logits_out ? logits_out : w.logits;
        ha.bmax = w.bmax;
        ha.bidx = w.bidx;
        const int nb = (m->vocab + ha.rows_per_block - 1) / ha.rows_per_block;
        if ((rc = launch_head(ha, nb, st))) return rc;
        if (argmax_out && (rc = launch_argmax_final(w.bmax, w.bidx, nb, argmax_out, st))) return rc;
    } else if (hidden_out) {
        if ((rc = launch_final_hidden(last, m->d, hidden_out, st))) return rc;
    }
    return ATLAS_OK;
}

}  // namespace atlas

using namespace atlas;

extern "C" size_t atlas_decode_workspace_bytes(const atlas_model* m) {
    if (validate_model(m) != ATLAS_OK) return 0;
    return decode_ws_bytes(m);
}

namespace atlas {

int check_decode_args(const atlas_model* m, const int32_t* d_token, const float* d_hidden_in, const int32_t* d_pos,
                      const float* d_logits, const int32_t* d_argmax) {
    int rc = validate_model(m);
    if (rc) return rc;
    ATLAS_CHECK_ARG(d_pos != nullptr, "null d_pos");
    ATLAS_CHECK_ARG(d_token || d_hidden_in, "need d_token or d_hidden_in");
    ATLAS_CHECK_ARG(!d_token || m->embedding, "token input needs an embedding table");
    const bool head = d_logits || d_argmax;
    ATLAS_CHECK_ARG(!head || (m->lm_head && m->g_final && m->vocab >= 1), "lm_head/g_final/vocab missing");
    return ATLAS_OK;
}

}  // namespace atlas

extern "C" int atlas_decode_step(const atlas_model* m, const int32_t* d_token, const float* d_hidden_in,
                                 const int32_t* d_pos, float* d_hidden_out, float* d_logits, int32_t* d_argmax,
                                 void* ws, size_t ws_bytes, void* stream) {
    int rc = check_decode_args(m, d_token, d_hidden_in, d_pos, d_logits, d_argmax);
    if (rc) return rc;
    ATLAS_CHECK_ARG(ws != nullptr, "null workspace");
    const size_t need = decode_ws_bytes(m);
    if (ws_bytes < need) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
    hipStream_t st = (hipStream_t)stream;
    XSource first{};
    if (d_token) {
        first.mode = X_FROM_EMBED;
        first.d_token = d_token;
        first.emb = m->embedding;
        first.vocab = m->vocab;
    } else {
        first.mode = X_FROM_HIDDEN;
        first.hidden = d_hidden_in;
    }
    XSource last{};
    if ((rc = run_decode_layers(m, first, d_pos, ws, st, &last))) return rc;
    return run_head(m, last, ws, d_hidden_out, d_logits, d_argmax, st);
}

extern "C" int atlas_device_status(const void* ws, void* stream, int32_t* status_out) {
    ATLAS_CHECK_ARG(ws && status_out, "null pointer");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(status_out, ws, 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(ATLAS_ERR_HIP, "status read: %s", hipGetErrorString(e));
    return ATLAS_OK;
}
