// Prefill: process a prompt through every layer, writing its KV slots, and return the
// last token's logits and greedy argmax.
//
// Source: "ATLAS-OLMo-3-32B-Think-v4", Limitations & roadmap -- prefill defined as the
// prompt run token by token through the decode path (our parity definition).
// This entry point currently runs exactly that definition: one decode step per
// prompt token, positions start_pos + t read from device memory.
#include "decode.h"

namespace atlas {

__global__ void positions_kernel(int32_t* pos, int n, int start) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) pos[i] = start + i;
}

static size_t prefill_ws(const atlas_model* m, int n) {
    return decode_ws_bytes(m) + align_up((size_t)n * 4, 256);
}

}  // namespace atlas

using namespace atlas;

extern "C" size_t atlas_prefill_workspace_bytes(const atlas_model* m, int32_t n_tokens) {
    if (validate_model(m) != ATLAS_OK || n_tokens < 1) return 0;
    return prefill_ws(m, n_tokens);
}

extern "C" int atlas_prefill(const atlas_model* m, const int32_t* d_tokens, int32_t n_tokens, int32_t start_pos,
                             float* d_last_logits, int32_t* d_argmax, void* ws, size_t ws_bytes, void* stream) {
    int rc = validate_model(m);
    if (rc) return rc;
    ATLAS_CHECK_ARG(d_tokens && ws, "null pointer");
    ATLAS_CHECK_ARG(n_tokens >= 1, "n_tokens must be >= 1");
    ATLAS_CHECK_ARG(start_pos >= 0 && (int64_t)start_pos + n_tokens <= m->t_max,
                    "positions %d..%d exceed T_max=%lld", start_pos, start_pos + n_tokens - 1,
                    (long long)m->t_max);
    ATLAS_CHECK_ARG(m->embedding, "prefill needs an embedding table");
    const size_t need = prefill_ws(m, n_tokens);
    if (ws_bytes < need) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
    hipStream_t st = (hipStream_t)stream;
    const size_t dws = decode_ws_bytes(m);
    int32_t* pos = (int32_t*)((char*)ws + dws);
    prof_mark("positions", st);
    ATLAS_KLAUNCH(positions_kernel, dim3((n_tokens + 255) / 256), dim3(256), 0, st, pos, n_tokens, start_pos);
    ATLAS_LAUNCH_CHECK("positions_kernel");
    for (int t = 0; t < n_tokens; t++) {
        const bool last = t == n_tokens - 1;
        rc = atlas_decode_step(m, d_tokens + t, nullptr, pos + t, nullptr, last ? d_last_logits : nullptr,
                               last ? d_argmax : nullptr, ws, dws, stream);
        if (rc) return rc;
    }
    return ATLAS_OK;
}
