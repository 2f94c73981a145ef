// Prefill: process a prompt through every layer, writing its KV slots, and return the
// last token's logits and greedy argmax; plus the standalone W4 GEMM entry point.
//
// Source: "ATLAS-OLMo-3-32B-Think-v4", Limitations & roadmap -- prefill is defined as
// the prompt run token by token through the decode path (the parity definition here),
// and its planned replacement is a batched, tiled GEMM prefill, which this is: per
// layer one W4 GEMM each for qkv, o, gate+up (SwiGLU fused) and down over all n
// positions, with QK norm/rotary/KV write, causal attention and the residual norms
// as per-position kernels (prefill_kernels.hip).
#include <cmath>

#include "decode.h"
#include "gemv.h"
#include "norm_rope.h"
#include "prefill_kernels.h"

namespace atlas {

namespace {

struct PrefillWs {
    void* dec;       // decode workspace (status word, head partials)
    float *X, *QKV, *A;
    uint16_t *p1h, *p1l, *p2h, *p2l;
    int8_t *qh, *qm, *ql;  // int8 digit planes of the next GEMM's input [n][K]
    float *qs, *qsum;      // and its per-(row, group) scales and sums [n][K / group]
    void *k_new, *v_new;   // prompt keys / values [Hkv][n][hd] in the cache's element type
    int ld1;
    size_t bytes;
};

constexpr int PF_QKV_SPLIT_MAX = 2;   // K ranges of the qkv GEMM (see pf_ksplit)

PrefillWs carve_prefill(const atlas_model* m, int n, void* base) {
    PrefillWs w{};
    char* b = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        void* p = b ? b + off : nullptr;
        off += align_up(bytes, 256);
        return p;
    };
    const int nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    w.ld1 = std::max(m->d, nq);
    w.dec = take(decode_ws_bytes(m));
    w.X = (float*)take((size_t)n * m->d * 4);
    w.QKV = (float*)take((size_t)n * PF_QKV_SPLIT_MAX * nqkv * 4);   // K-split partials per row
    w.A = (float*)take((size_t)n * 2 * m->d * 4);   // o / down output: up to two K-split partials per row
    w.p1h = (uint16_t*)take((size_t)n * w.ld1 * 2);
    w.p1l = (uint16_t*)take((size_t)n * w.ld1 * 2);
    w.p2h = (uint16_t*)take((size_t)n * m->dff * 2);
    w.p2l = (uint16_t*)take((size_t)n * m->dff * 2);
    const int kmax = std::max(w.ld1, m->dff);
    w.qh = (int8_t*)take((size_t)n * kmax);
    w.qm = (int8_t*)take((size_t)n * kmax);
    w.ql = (int8_t*)take((size_t)n * kmax);
    w.qs = (float*)take((size_t)n * (kmax / 128 + 1) * 4);
    w.qsum = (float*)take((size_t)n * (kmax / 128 + 1) * 4);
    const size_t kv_bytes = (size_t)m->hkv * n * m->hd * (m->kv_dtype == 1 ? 2 : 4);
    w.k_new = take(kv_bytes);
    w.v_new = take(kv_bytes);
    w.bytes = off;
    return w;
}

W4View view(const atlas_w4& w) { return w4_view(w.qweight, w.scales, w.zeros, w.N, w.K, w.group, w.scale_dtype); }

int validate_prefill_model(const atlas_model* m) {
    for (int l = 0; l < m->n_layers; l++) {
        const atlas_layer& L = m->layers[l];
        const atlas_w4* ws[5] = {&L.qkv, &L.o, &L.gate, &L.up, &L.down};
        for (const atlas_w4* w : ws)
            ATLAS_CHECK_SHAPE(gemm_supported(w->group), "prefill needs group 32 or a multiple of 64 (layer %d: %d)", l,
                              w->group);
        ATLAS_CHECK_SHAPE(L.gate.group == L.up.group && L.gate.scale_dtype == L.up.scale_dtype,
                          "gate and up must share group and scale type");
    }
    return ATLAS_OK;
}

GemmArgs gemm(const uint16_t* hi, const uint16_t* lo, int lda, const atlas_w4& w, int M) {
    GemmArgs g{};
    g.a_hi = hi;
    g.a_lo = lo;
    g.lda = lda;
    g.W0 = view(w);
    g.W1 = g.W0;
    g.M = M;
    g.N = w.N;
    g.K = w.K;
    g.group = w.group;
    return g;
}

// K splits of the qkv, o and down GEMMs: the most ranges up to `most` (two here) with whole
// groups and 128-column tiles. At 1,200 positions the 64 x 128 tiles fill the
// two-blocks-per-CU grid (512 per round) poorly: o and down have 760 tiles (1.5 rounds;
// split in two, 2.97), qkv 1,064 (2.08 rounds; split in two, 4.16). The consumers add the
// partials: the residual kernel (o, down), the head (the last down), the rotary kernel (qkv).
// Four qkv ranges made the GEMM no faster than two and doubled the rotary kernel's reads.
int pf_ksplit(const atlas_w4& w, int most) {
    for (int s = most; s > 1; s--) {
        const int c = w.K / s;
        if (w.K % s == 0 && c % w.group == 0 && c % 128 == 0) return s;
    }
    return 1;
}

void set_split(GemmArgs& g, int S, int d) {
    g.ksplit = S;
    g.kchunk = S > 1 ? g.K / S : 0;
    g.c_split = S > 1 ? (size_t)d : 0;   // partial s of row t at C + t ldc + s d
}

// The workspace's int8 digit planes as the GEMM input (the int8 matrix-core kernel for
// groups of 128, 256 or 512); other groups keep the bf16 planes. attach_i8() makes the
// digits from the bf16 planes first; use_i8() takes digits a producing kernel wrote.
void use_i8(GemmArgs& g, const PrefillWs& w) {
    g.q_hi = w.qh;
    g.q_mid = w.qm;
    g.q_lo = w.ql;
    g.q_s = w.qs;
    g.q_sum = w.qsum;
    g.ldq = g.K;
    g.ldqs = g.K / g.group;
}

int attach_i8(GemmArgs& g, const PrefillWs& w, hipStream_t st) {
    if (!gemm_i8_supported(g.group, g.K)) return ATLAS_OK;
    const int rc = launch_pf_quant8(g.a_hi, g.a_lo, g.lda, g.M, g.K, g.group, w.qh, w.qm, w.ql, w.qs, w.qsum, st);
    if (rc) return rc;
    use_i8(g, w);
    return ATLAS_OK;
}

// Whether the residual kernel writes the int8 digits of the next GEMM's input (a W4
// matrix with K = d) in place of its bf16 planes; then no quantisation pass runs.
bool residual_digits(const atlas_w4& next, int d) {
    return gemm_i8_supported(next.group, d) && residual_digits_ok(next.group, d);
}

}  // namespace

}  // namespace atlas

using namespace atlas;

extern "C" size_t atlas_prefill_workspace_bytes(const atlas_model* m, int32_t n_tokens) {
    if (validate_model(m) != ATLAS_OK || n_tokens < 1) return 0;
    return carve_prefill(m, n_tokens, nullptr).bytes;
}

extern "C" int atlas_prefill(const atlas_model* m, const int32_t* d_tokens, int32_t n_tokens, int32_t start_pos,
                             float* d_last_logits, int32_t* d_argmax, void* ws, size_t ws_bytes, void* stream) {
    int rc = validate_model(m);
    if (rc) return rc;
    if ((rc = validate_prefill_model(m))) return rc;
    ATLAS_CHECK_ARG(d_tokens && ws, "null pointer");
    ATLAS_CHECK_ARG(n_tokens >= 1, "n_tokens must be >= 1");
    ATLAS_CHECK_ARG(start_pos >= 0 && (int64_t)start_pos + n_tokens <= m->t_max,
                    "positions %d..%d exceed T_max=%lld", start_pos, start_pos + n_tokens - 1,
                    (long long)m->t_max);
    ATLAS_CHECK_ARG(m->embedding, "prefill needs an embedding table");
    const bool head = d_last_logits || d_argmax;
    ATLAS_CHECK_ARG(!head || (m->lm_head && m->g_final && m->vocab >= 1), "lm_head/g_final/vocab missing");
    const PrefillWs w = carve_prefill(m, n_tokens, ws);
    if (ws_bytes < w.bytes) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, w.bytes);
    hipStream_t st = (hipStream_t)stream;
    const int n = n_tokens, d = m->d, nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    RopeTable rt_swa, rt_full;
    rope_table(&m->rope_swa, m->hd, &rt_swa);
    rope_table(&m->rope_full, m->hd, &rt_full);

    if ((rc = launch_pf_embed(d_tokens, n, m->embedding, m->vocab, d, w.X, w.p1h, w.p1l, w.ld1, (int*)w.dec, st)))
        return rc;
    bool qkv_digits = false;   // the previous layer's residual wrote the qkv input as int8 digits
    for (int l = 0; l < m->n_layers; l++) {
        const atlas_layer& L = m->layers[l];
        const bool last = l == m->n_layers - 1;
        // qkv projection of all positions
        GemmArgs qa = gemm(w.p1h, w.p1l, w.ld1, L.qkv, n);
        const int sq = pf_ksplit(L.qkv, PF_QKV_SPLIT_MAX);
        qa.C = w.QKV;
        qa.ldc = sq * nqkv;
        set_split(qa, sq, nqkv);
        if (qkv_digits) use_i8(qa, w);
        else if ((rc = attach_i8(qa, w, st))) return rc;
        if ((rc = launch_w4_gemm(qa, 0, st, "pf_gemm_qkv"))) return rc;
        // QK norm and rotary; the prompt keys/values into the prompt KV buffers
        PfRopeArgs ra{};
        ra.qkv = w.QKV;
        ra.ld = sq * nqkv;
        ra.S = sq;
        ra.pstride = nqkv;
        ra.n = n;
        ra.start_pos = start_pos;
        ra.Hq = m->hq;
        ra.Hkv = m->hkv;
        ra.g_q = L.g_q;
        ra.g_k = L.g_k;
        ra.eps = m->eps;
        const RopeTable& rt = L.type == 1 ? rt_full : rt_swa;
        for (int i = 0; i < 64; i++) ra.inv[i] = rt.inv[i];
        ra.mscale = rt.mscale;
        ra.k_new = w.k_new;
        ra.v_new = w.v_new;
        ra.kv_bf16 = m->kv_dtype;
        if ((rc = launch_pf_rope(ra, st))) return rc;
        const bool ring = m->swa_ring && L.type == 0;
        const int64_t slots = ring ? m->window : m->t_max;
        // causal attention; output planes for the o projection
        PfAttnArgs aa{};
        aa.qkv = w.QKV;
        aa.ld_qkv = sq * nqkv;   // q rotated in place in the first partial
        aa.k_cache = L.k_cache;
        aa.v_cache = L.v_cache;
        aa.slots = slots;
        aa.ring = ring ? 1 : 0;
        aa.kv_bf16 = m->kv_dtype;
        aa.k_new = w.k_new;
        aa.v_new = w.v_new;
        aa.n = n;
        aa.start_pos = start_pos;
        aa.Hq = m->hq;
        aa.Hkv = m->hkv;
        aa.window = L.type == 1 ? 0 : m->window;
        aa.scale = 1.0f / std::sqrt((float)m->hd);
        aa.o_hi = w.p1h;
        aa.o_lo = w.p1l;
        aa.ldo = w.ld1;
        if ((rc = launch_pf_attn(aa, st))) return rc;
        // the prompt's keys and values into the cache, after every query has read them
        PfCommitArgs ca{};
        ca.k_new = w.k_new;
        ca.v_new = w.v_new;
        ca.k_cache = L.k_cache;
        ca.v_cache = L.v_cache;
        ca.slots = slots;
        ca.ring = aa.ring;
        ca.kv_bf16 = m->kv_dtype;
        ca.n = n;
        ca.start_pos = start_pos;
        ca.Hkv = m->hkv;
        if ((rc = launch_pf_commit(ca, st))) return rc;
        // o projection, h = x + RMSNorm_pa(a)
        GemmArgs oa = gemm(w.p1h, w.p1l, w.ld1, L.o, n);
        oa.C = w.A;
        oa.ldc = 2 * d;
        const int so = pf_ksplit(L.o, 2);
        set_split(oa, so, d);
        if ((rc = attach_i8(oa, w, st))) return rc;
        if ((rc = launch_w4_gemm(oa, 0, st, "pf_gemm_o"))) return rc;
        const bool gu_digits = residual_digits(L.gate, d);
        const Q8Out q_gu{w.qh, w.qm, w.ql, w.qs, w.qsum, L.gate.group};
        if ((rc = launch_pf_residual(w.X, w.A, 2 * d, so, L.g_pa, n, d, m->eps, w.p1h, w.p1l, w.ld1, st,
                                     gu_digits ? &q_gu : nullptr)))
            return rc;
        // gate/up with SwiGLU, then down
        GemmArgs ga = gemm(w.p1h, w.p1l, w.ld1, L.gate, n);
        ga.W1 = view(L.up);
        ga.z_hi = w.p2h;
        ga.z_lo = w.p2l;
        ga.ldz = m->dff;
        if (gu_digits) use_i8(ga, w);
        else if ((rc = attach_i8(ga, w, st))) return rc;
        // With groups of 128 the gate/up kernel writes z as the down projection's int8
        // digits (in the z planes' place), so no quantisation pass runs between the two
        const bool z_digits = i8r_swiglu_digits_ok(ga, L.down.group) && gemm_i8_supported(L.down.group, m->dff);
        if (z_digits) {
            ga.zq_hi = reinterpret_cast<int8_t*>(w.p2h);   // [n][dff] each; p2h holds two planes
            ga.zq_mid = ga.zq_hi + (size_t)n * m->dff;
            ga.zq_lo = reinterpret_cast<int8_t*>(w.p2l);   // p2l the third and the per-group values
            ga.zq_s = reinterpret_cast<float*>(ga.zq_lo + (size_t)n * m->dff);
            ga.zq_sum = ga.zq_s + (size_t)n * (m->dff / 128);
            ga.zq_ld = m->dff;
            ga.zq_lds = m->dff / 128;
        }
        if ((rc = launch_w4_gemm(ga, 1, st, "pf_gemm_gate_up"))) return rc;
        GemmArgs da = gemm(w.p2h, w.p2l, m->dff, L.down, n);
        da.C = w.A;
        da.ldc = 2 * d;
        const int sd = pf_ksplit(L.down, 2);
        set_split(da, sd, d);
        if (z_digits) {
            da.q_hi = ga.zq_hi;
            da.q_mid = ga.zq_mid;
            da.q_lo = ga.zq_lo;
            da.q_s = ga.zq_s;
            da.q_sum = ga.zq_sum;
            da.ldq = ga.zq_ld;
            da.ldqs = ga.zq_lds;
        } else if ((rc = attach_i8(da, w, st))) {
            return rc;
        }
        if ((rc = launch_w4_gemm(da, 0, st, "pf_gemm_down"))) return rc;
        // y = h + RMSNorm_pf(m): the last layer leaves it to the head (last position only)
        qkv_digits = !last && residual_digits(m->layers[l + 1].qkv, d);
        const Q8Out q_qkv{w.qh, w.qm, w.ql, w.qs, w.qsum, last ? 128 : m->layers[l + 1].qkv.group};
        if (!last || !head)
            if ((rc = launch_pf_residual(w.X, w.A, 2 * d, sd, L.g_pf, n, d, m->eps, w.p1h, w.p1l, w.ld1, st,
                                         qkv_digits ? &q_qkv : nullptr)))
                return rc;
    }
    if (!head) return ATLAS_OK;
    XSource lastx{};
    lastx.mode = X_FROM_RESIDUAL;
    lastx.m_part = w.A + (size_t)(n - 1) * 2 * d;   // the down partials of the last row, d apart
    lastx.S = pf_ksplit(m->layers[m->n_layers - 1].down, 2);
    lastx.h = w.X + (size_t)(n - 1) * d;
    lastx.g = m->layers[m->n_layers - 1].g_pf;
    lastx.eps = m->eps;
    return run_head(m, lastx, w.dec, nullptr, d_last_logits, d_argmax, st);
}

// ---- standalone W4 GEMM ---------------------------------------------------------------------

namespace {
struct GemmWs {
    uint16_t *hi, *lo;   // bf16 planes [M][K]
    int8_t *qh, *qm, *ql;   // int8 digit planes [M][K]
    float *qs, *qsum;       // [M][K / 128 + 1]
    size_t bytes;
};
GemmWs carve_gemm(int M, int K, void* base) {
    GemmWs w{};
    char* b = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        void* p = b ? b + off : nullptr;
        off += align_up(bytes, 256);
        return p;
    };
    w.hi = (uint16_t*)take((size_t)M * K * 2);
    w.lo = (uint16_t*)take((size_t)M * K * 2);
    w.qh = (int8_t*)take((size_t)M * K);
    w.qm = (int8_t*)take((size_t)M * K);
    w.ql = (int8_t*)take((size_t)M * K);
    w.qs = (float*)take((size_t)M * (K / 128 + 1) * 4);
    w.qsum = (float*)take((size_t)M * (K / 128 + 1) * 4);
    w.bytes = off;
    return w;
}
}  // namespace

extern "C" size_t atlas_w4_gemm_workspace_bytes(const atlas_w4* W, int32_t M) {
    if (validate_w4(W) != ATLAS_OK || M < 1) return 0;
    return carve_gemm(M, W->K, nullptr).bytes;
}

extern "C" int atlas_w4_gemm(const atlas_w4* W, const float* A, int32_t M, float* C, void* ws, size_t ws_bytes,
                             void* stream) {
    int rc = validate_w4(W);
    if (rc) return rc;
    ATLAS_CHECK_ARG(A && C && ws, "null pointer");
    ATLAS_CHECK_ARG(M >= 1, "M must be >= 1");
    ATLAS_CHECK_SHAPE(gemm_supported(W->group), "W4 GEMM needs group 32 or a multiple of 64 (got %d)", W->group);
    const GemmWs w = carve_gemm(M, W->K, ws);
    if (ws_bytes < w.bytes) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, w.bytes);
    hipStream_t st = (hipStream_t)stream;
    if ((rc = launch_pf_split(A, M, W->K, W->K, w.hi, w.lo, W->K, st))) return rc;
    GemmArgs g = gemm(w.hi, w.lo, W->K, *W, M);
    g.C = C;
    g.ldc = W->N;
    // more than 16 rows with groups of 128-512: the int8 matrix-core kernel; otherwise the
    // bf16 kernels (a few rows take the small-row paths)
    if (M > 16 && gemm_i8_supported(W->group, W->K)) {
        if ((rc = launch_pf_quant8(w.hi, w.lo, W->K, M, W->K, W->group, w.qh, w.qm, w.ql, w.qs, w.qsum, st)))
            return rc;
        g.q_hi = w.qh;
        g.q_mid = w.qm;
        g.q_lo = w.ql;
        g.q_s = w.qs;
        g.q_sum = w.qsum;
        g.ldq = W->K;
        g.ldqs = W->K / W->group;
    }
    return launch_w4_gemm(g, 0, st, "w4_gemm");
}
