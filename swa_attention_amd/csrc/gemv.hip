// W4 (4-bit group-quantised) GEMV entry point, activation encoding and dequant.
//
// Source: "ATLAS-OLMo-3-32B-Think-v4" model card, Quantization recipe (packed int4
// weights with per-group scales multiplied against f32 activations, dequantised
// inline). The card's A100 kernel maps one warp to one output row; here the matrix
// is streamed with 16-byte loads where every lane owns fixed 32-column chunks of the
// reduction axis, and the dequantisation is folded into exact integer dot products
// (v_dot8_i32_i4) between the raw 4-bit codes and a 24-bit block-fixed-point
// encoding of x (see common.h). Per 32 weights a lane spends one xor per code word,
// six dot8 per word and a short per-chunk epilogue that applies the zero point and
// the group scale.
#include "decode_kernels.h"
#include "gemv.h"

namespace atlas {

// ---- activation encoding kernel -------------------------------------------------------
// One thread per 8-element word; quads of threads form a 32-element chunk.
__global__ __launch_bounds__(256) void xq_encode_kernel(const float* __restrict__ x, int K, XQ out) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int nwords = K / 8;
    if (t < nwords) {  // K % 32 == 0, so every quad is entirely inside or outside
        float x8[8];
        const float4* p = reinterpret_cast<const float4*>(x) + 2 * t;
        float4 a = p[0], b = p[1];
        x8[0] = a.x; x8[1] = a.y; x8[2] = a.z; x8[3] = a.w;
        x8[4] = b.x; x8[5] = b.y; x8[6] = b.z; x8[7] = b.w;
        xq_encode_word(x8, out, t >> 2, t & 3);
    }
}

// Sum of S partial vectors [S][N] -> y[N].
__global__ void sum_partials_kernel(const float* __restrict__ part, int S, int N, float* __restrict__ y) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < N) {
        float s = 0.f;
        for (int r = 0; r < S; r++) s += part[(size_t)r * N + i];
        y[i] = s;
    }
}

// Dequantise: out[n][k] = (code - zero) * scale, exact.
__global__ void w4_dequant_kernel(W4View a, int group, float* __restrict__ out) {
    const int KW = a.KW, G = a.G, GW = a.GW;
    const size_t total = (size_t)a.N * KW;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        const size_t n = i / KW;
        const int wi = (int)(i % KW);
        const uint32_t word = a.qweight[i];
        for (int e = 0; e < 8; e++) {
            const int k = wi * 8 + e;
            const int g = k / group;
            const int z = a.zsym ? 8 : (int)((a.zeros[n * GW + (g >> 3)] >> ((g & 7) * 4)) & 15u);
            const int c = (int)((word >> (4 * e)) & 15u);
            out[n * a.K + k] = (float)(c - z) * scale_to_f32(a.scales[n * G + g], a.scale_dtype);
        }
    }
}

// ---- host side --------------------------------------------------------------------------

int validate_w4(const atlas_w4* W) {
    ATLAS_CHECK_ARG(W != nullptr, "null atlas_w4");
    ATLAS_CHECK_ARG(W->qweight && W->scales, "null qweight/scales");
    ATLAS_CHECK_ARG(W->N >= 1 && W->K >= 1, "bad shape N=%d K=%d", W->N, W->K);
    ATLAS_CHECK_SHAPE(W->K % 32 == 0, "K=%d must be a multiple of 32", W->K);
    ATLAS_CHECK_SHAPE(W->group >= 32 && W->group % 32 == 0, "group=%d must be a positive multiple of 32",
                      W->group);
    ATLAS_CHECK_ARG(W->scale_dtype == 0 || W->scale_dtype == 1, "scale_dtype must be 0 or 1");
    ATLAS_CHECK_ARG(((uintptr_t)W->qweight & 15) == 0, "qweight must be 16-byte aligned");
    return ATLAS_OK;
}




int launch_xq_encode(const float* x, int K, XQ out, hipStream_t st) {
    const int nwords = K / 8;
    prof_mark("xq_encode", st);
    ATLAS_KLAUNCH(xq_encode_kernel, dim3((nwords + 255) / 256), dim3(256), 0, st, x, K, out);
    ATLAS_LAUNCH_CHECK("xq_encode_kernel");
    return ATLAS_OK;
}

int launch_sum_partials(const float* part, int S, int N, float* y, hipStream_t st) {
    prof_mark("sum_partials", st);
    ATLAS_KLAUNCH(sum_partials_kernel, dim3((N + 255) / 256), dim3(256), 0, st, part, S, N, y);
    ATLAS_LAUNCH_CHECK("sum_partials_kernel");
    return ATLAS_OK;
}


// at most 4 chunks per lane (the wider tiles hold fewer loads in flight); 5 only where
// no split of K fits 4
GemvShape standalone_shape(int N, int K) {
    GemvShape p = gemv_shape(N, K, true, 256, 4);
    return p.CPL ? p : gemv_shape(N, K, true, 256, 5);
}

size_t gemv_workspace_bytes(int N, int K) {
    GemvShape p = standalone_shape(N, K);
    size_t b = align_up(xq_bytes(K), 256);
    if (p.S > 1) b += align_up((size_t)p.S * N * 4, 256);
    return b;
}

}  // namespace atlas

using namespace atlas;

extern "C" size_t atlas_w4_gemv_workspace_bytes(const atlas_w4* W) {
    if (validate_w4(W) != ATLAS_OK) return 0;
    return gemv_workspace_bytes(W->N, W->K);
}

extern "C" int atlas_w4_gemv(const atlas_w4* W, const float* x, float* y, void* ws, size_t ws_bytes,
                             void* stream) {
    int rc = validate_w4(W);
    if (rc) return rc;
    ATLAS_CHECK_ARG(x && y, "null x or y");
    ATLAS_CHECK_ARG(ws != nullptr, "null workspace");
    const size_t need = gemv_workspace_bytes(W->N, W->K);
    if (ws_bytes < need) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
    GemvShape p = standalone_shape(W->N, W->K);
    ATLAS_CHECK_SHAPE(p.CPL > 0, "K=%d cannot be split into ranges the kernel supports", W->K);
    hipStream_t st = (hipStream_t)stream;
    XQ xq = xq_view(ws, W->K);
    if ((rc = launch_xq_encode(x, W->K, xq, st))) return rc;
    float* part = p.S > 1 ? (float*)((char*)ws + align_up(xq_bytes(W->K), 256)) : y;
    GemvPlanesArgs a{};
    a.W = w4_view(W->qweight, W->scales, W->zeros, W->N, W->K, W->group, W->scale_dtype);
    a.xq = xq;
    a.group = W->group;
    a.y = part;
    if ((rc = launch_gemv_planes(a, p, st, "w4_gemv"))) return rc;
    if (p.S > 1) return launch_sum_partials(part, p.S, W->N, y, st);
    return ATLAS_OK;
}

extern "C" int atlas_w4_dequant(const atlas_w4* W, float* out, void* stream) {
    int rc = validate_w4(W);
    if (rc) return rc;
    ATLAS_CHECK_ARG(out != nullptr, "null out");
    const W4View a = w4_view(W->qweight, W->scales, W->zeros, W->N, W->K, W->group, W->scale_dtype);
    prof_mark("w4_dequant", (hipStream_t)stream);
    ATLAS_KLAUNCH(w4_dequant_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream, a, W->group, out);
    ATLAS_LAUNCH_CHECK("w4_dequant_kernel");
    return ATLAS_OK;
}
