// GQA decode attention entry points, split over the key range with an online-softmax
// merge (kernels in decode_kernels.hip), over an f32 KV cache or over any of the
// cache formats the decode step supports (f32 or bf16 elements; key j in slot j, or
// in slot j mod slots of a sliding-window ring).
//
// Sources: "ATLAS-OLMo-3-32B-Think-v4", Architecture deep-dive (GQA 40 query / 8 KV
// heads of 128; sliding window 4,096 on three of every four layers, full context on
// the fourth) and Why the 3:1 SWA layout matters (sliding-window layers look back at
// most 4,096 tokens); f32 KV cache (VRAM breakdown); Limitations & roadmap (bf16 KV
// and a window-sized cache on the sliding-window layers, planned).
//
// With only 8 KV heads a decode step cannot fill 256 compute units one head per
// workgroup, so each KV head's key range is cut into S splits. A workgroup reads its
// split's keys and values once for all Hq/Hkv query heads sharing them and writes a
// partial (max m, sum l, unnormalised acc[D]) per query head; the merge rescales the
// partials by exp(m_s - max_s m_s).
#include "decode_kernels.h"

using namespace atlas;

extern "C" size_t atlas_gqa_decode_workspace_bytes(int32_t Hq, int32_t Hkv, int32_t D, int64_t T_max) {
    if (Hq < 1 || Hkv < 1 || D != 128 || T_max < 1) return 0;
    return (size_t)Hq * attn_splits(T_max, Hkv) * ATTN_PART_F * 4;
}

extern "C" int atlas_gqa_decode_kv(const float* q, const void* k_cache, const void* v_cache,
                                   const atlas_kv_layout* layout, int32_t Hq, int32_t Hkv, int32_t D,
                                   const int32_t* d_pos, int32_t window, float softmax_scale, float* out, void* ws,
                                   size_t ws_bytes, void* stream) {
    ATLAS_CHECK_ARG(q && k_cache && v_cache && layout && d_pos && out && ws, "null pointer");
    const int64_t slots = layout->slots;
    ATLAS_CHECK_ARG(Hq >= 1 && Hkv >= 1 && slots >= 1, "bad sizes");
    ATLAS_CHECK_SHAPE(D == 128, "head_dim %d unsupported (128 only)", D);
    ATLAS_CHECK_SHAPE(Hq % Hkv == 0 && Hq / Hkv <= 8, "Hq/Hkv must be an integer <= 8");
    ATLAS_CHECK_ARG(window >= 0, "window must be >= 0");
    ATLAS_CHECK_ARG(slots <= (int64_t)1 << 30, "slots too large");
    ATLAS_CHECK_ARG(layout->kv_dtype == 0 || layout->kv_dtype == 1, "kv_dtype must be 0 (f32) or 1 (bf16)");
    ATLAS_CHECK_ARG(!layout->ring || (window > 0 && window <= slots), "a ring needs 0 < window <= slots");
    const size_t need = atlas_gqa_decode_workspace_bytes(Hq, Hkv, D, slots);
    if (ws_bytes < need) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
    const int64_t maxkeys = window > 0 ? std::min<int64_t>(window, slots) : slots;
    AttnFusedArgs a{};
    a.k_cache = const_cast<void*>(k_cache);   // read only when fused == 0
    a.v_cache = const_cast<void*>(v_cache);
    a.T_max = layout->ring ? (int64_t)INT32_MAX : slots;
    a.slots = slots;
    a.ring = layout->ring ? 1 : 0;
    a.kv_bf16 = layout->kv_dtype;
    a.d_pos = d_pos;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.window = window;
    a.S = attn_splits(maxkeys, Hkv);
    a.scale = softmax_scale;
    a.part = (float*)ws;
    a.fused = 0;
    a.q_final = q;
    hipStream_t st = (hipStream_t)stream;
    int rc = launch_attn_fused(a, Hq / Hkv, st);
    if (rc) return rc;
    MergeArgs m{};
    m.part = (float*)ws;
    m.S = a.S;
    m.Hq = Hq;
    m.o = out;
    return launch_merge(m, st);
}

extern "C" int atlas_gqa_decode(const float* q, const float* k_cache, const float* v_cache, int32_t Hq,
                                int32_t Hkv, int32_t D, int64_t T_max, const int32_t* d_pos, int32_t window,
                                float softmax_scale, float* out, void* ws, size_t ws_bytes, void* stream) {
    const atlas_kv_layout flat{0, 0, T_max};
    return atlas_gqa_decode_kv(q, k_cache, v_cache, &flat, Hq, Hkv, D, d_pos, window, softmax_scale, out, ws,
                               ws_bytes, stream);
}
