// W4 (4-bit group-quantised) GEMV for batch-1 decode on gfx950.
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

// ---- GEMV kernel ----------------------------------------------------------------------
//
// Work decomposition. The reduction axis is cut into S ranges of CW chunks
// (blockIdx.y selects the range; partial sums go to y_part[range][row]). Rows are
// processed in tiles of RB rows; inside a tile lane l owns the CPL "virtual chunks"
// vc = l + 64 j (j < CPL), i.e. row vc / CW of the tile and chunk vc % CW of the
// range, with RB * CW <= 64 * CPL. A lane's chunks are the same for every tile, so
// its slice of the encoded x stays in registers while the wave streams rows.
// The block stages the encoded x range in LDS once; waves take tiles w, w+4, ...
// of the block's contiguous tile range.

template <int CPL, int RB>
__global__ __launch_bounds__(256) void w4_gemv_kernel(GemvArgs a) {
    extern __shared__ uint32_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kr = blockIdx.y;
    const int CW = a.CW;
    const int C0 = kr * CW;                      // first chunk of this range
    const int KW = a.K / 8;                      // words per row
    const int G = (a.K + a.group - 1) / a.group;
    const int GW = (G + 7) / 8;

    // tiles of this block
    const int T = (a.N + RB - 1) / RB;
    const int t_begin = blockIdx.x * a.tiles_per_block;
    const int t_end = min(T, t_begin + a.tiles_per_block);

    // lane items
    int rt[CPL], ch[CPL], gi[CPL];
    bool valid[CPL];
#pragma unroll
    for (int j = 0; j < CPL; j++) {
        int vc = lane + 64 * j;
        valid[j] = vc < RB * CW;
        rt[j] = valid[j] ? vc / CW : 0;
        ch[j] = valid[j] ? C0 + vc % CW : C0;
        gi[j] = ch[j] * XQ_CHUNK / a.group;
    }

    // stage the encoded x range in LDS: CW chunks x 24 words, then qs, isum
    uint32_t* s_pl = smem;
    float* s_qs = reinterpret_cast<float*>(smem + CW * XQ_WORDS_PER_CHUNK);
    int* s_is = reinterpret_cast<int*>(s_qs + CW);
    {
        const uint4* src = reinterpret_cast<const uint4*>(a.xq.planes + (size_t)C0 * XQ_WORDS_PER_CHUNK);
        uint4* dst = reinterpret_cast<uint4*>(s_pl);
        for (int i = threadIdx.x; i < CW * XQ_WORDS_PER_CHUNK / 4; i += 256) dst[i] = src[i];
        for (int i = threadIdx.x; i < CW; i += 256) {
            s_qs[i] = a.xq.qs[C0 + i];
            s_is[i] = a.xq.isum[C0 + i];
        }
    }
    __syncthreads();
    uint32_t pl[CPL][XQ_WORDS_PER_CHUNK];
    float qs[CPL], icf[CPL];
#pragma unroll
    for (int j = 0; j < CPL; j++) {
        const uint4* s4 = reinterpret_cast<const uint4*>(s_pl + (ch[j] - C0) * XQ_WORDS_PER_CHUNK);
#pragma unroll
        for (int q = 0; q < XQ_WORDS_PER_CHUNK / 4; q++) {
            uint4 v = s4[q];
            pl[j][4 * q + 0] = v.x; pl[j][4 * q + 1] = v.y; pl[j][4 * q + 2] = v.z; pl[j][4 * q + 3] = v.w;
        }
        qs[j] = s_qs[ch[j] - C0];
        icf[j] = (float)s_is[ch[j] - C0];
    }

    for (int t = t_begin + wave; t < t_end; t += 4) {
        const int row0 = t * RB;
        uint4 w[CPL];
        uint32_t zw[CPL];
        uint16_t sb[CPL];
#pragma unroll
        for (int j = 0; j < CPL; j++) {
            const int row = row0 + rt[j];
            const bool ok = valid[j] && row < a.N;
            const int rr = ok ? row : 0;
            w[j] = reinterpret_cast<const uint4*>(a.qweight + (size_t)rr * KW)[ch[j]];
            sb[j] = ok ? a.scales[(size_t)rr * G + gi[j]] : (uint16_t)0;
            zw[j] = a.zeros ? a.zeros[(size_t)rr * GW + (gi[j] >> 3)] : 0x88888888u;
        }
        float acc[RB];
#pragma unroll
        for (int r = 0; r < RB; r++) acc[r] = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; j++) {
            int D[XQ_PLANES] = {0, 0, 0, 0, 0, 0};
            const uint32_t wq[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int u = (int)(wq[q] ^ 0x88888888u);
#pragma unroll
                for (int p = 0; p < XQ_PLANES; p++)
                    D[p] = __builtin_amdgcn_sdot8(u, (int)pl[j][q * XQ_PLANES + p], D[p], false);
            }
            const int E0 = D[0] + (D[1] << 4) + (D[2] << 8);
            const int E1 = D[3] + (D[4] << 4) + (D[5] << 8);
            const float f = fmaf(4096.f, (float)E1, (float)E0);
            const int z = (zw[j] >> ((gi[j] & 7) * 4)) & 15;
            const float tt = fmaf((float)(8 - z), icf[j], f);
            const float c = scale_to_f32(sb[j], a.scale_dtype) * qs[j] * tt;
            if (RB == 1) {
                acc[0] += c;
            } else {
#pragma unroll
                for (int r = 0; r < RB; r++) acc[r] += (rt[j] == r) ? c : 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const float s = wave_sum(acc[r]);
            const int row = row0 + r;
            if (lane == 0 && row < a.N) a.y[(size_t)kr * a.N + row] = s;
        }
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
__global__ void w4_dequant_kernel(GemvArgs a, float* __restrict__ out) {
    const int KW = a.K / 8;
    const int G = (a.K + a.group - 1) / a.group;
    const int GW = (G + 7) / 8;
    const size_t total = (size_t)a.N * KW;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        const size_t n = i / KW;
        const int wi = (int)(i % KW);
        const uint32_t word = a.qweight[i];
        for (int e = 0; e < 8; e++) {
            const int k = wi * 8 + e;
            const int g = k / a.group;
            const int z = a.zeros ? (int)((a.zeros[n * GW + (g >> 3)] >> ((g & 7) * 4)) & 15u) : 8;
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

GemvPlan plan_gemv(int N, int K) {
    GemvPlan p{};
    const int C = K / XQ_CHUNK;
    // candidate K-range widths: divisors of C no larger than 320 chunks
    int best_cw = -1, best_rb = 1, best_cpl = 5;
    double best_util = -1.0;
    int best_s = 1 << 30;
    for (int s = 1; s <= C; s++) {
        if (C % s) continue;
        const int cw = C / s;
        if (cw > 320) continue;
        for (int rb = 2; rb >= 1; rb--) {
            if (rb == 2 && (2 * cw) % 64 != 0) continue;
            const int cpl = (rb * cw + 63) / 64;
            if (cpl > 5) continue;
            const double util = (double)(rb * cw) / (64.0 * cpl);
            if (util > best_util + 1e-9 || (util > best_util - 1e-9 && s < best_s)) {
                best_util = util;
                best_cw = cw;
                best_rb = rb;
                best_cpl = cpl;
                best_s = s;
            }
        }
        if (best_util >= 0.999) break;
    }
    p.CW = best_cw;
    p.S = best_cw > 0 ? C / best_cw : 0;
    p.RB = best_rb;
    p.CPL = best_cpl;
    const int T = (N + p.RB - 1) / p.RB;
    // aim for ~1024 blocks over all ranges, at least 4 tiles per block
    int target_blocks = (p.S > 0) ? (1024 + p.S - 1) / p.S : 1;
    int tpb = (T + target_blocks - 1) / target_blocks;
    if (tpb < 4) tpb = 4;
    p.tiles_per_block = tpb;
    p.blocks_x = (T + tpb - 1) / tpb;
    p.lds_bytes = (size_t)p.CW * (XQ_WORDS_PER_CHUNK * 4 + 8);
    return p;
}

int launch_gemv(const GemvArgs& a0, const GemvPlan& p, hipStream_t st) {
    GemvArgs a = a0;
    a.CW = p.CW;
    a.tiles_per_block = p.tiles_per_block;
    dim3 grid(p.blocks_x, p.S), block(256);
#define L(CPL_, RB_)                                                                      \
    if (p.CPL == CPL_ && p.RB == RB_) {                                                   \
        hipLaunchKernelGGL((w4_gemv_kernel<CPL_, RB_>), grid, block, p.lds_bytes, st, a); \
        ATLAS_LAUNCH_CHECK("w4_gemv_kernel");                                             \
        return ATLAS_OK;                                                                  \
    }
    L(1, 1) L(2, 1) L(3, 1) L(4, 1) L(5, 1) L(1, 2) L(2, 2) L(3, 2) L(4, 2) L(5, 2)
#undef L
    return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, "no GEMV kernel for CPL=%d RB=%d", p.CPL, p.RB);
}

int launch_xq_encode(const float* x, int K, XQ out, hipStream_t st) {
    const int nwords = K / 8;
    hipLaunchKernelGGL(xq_encode_kernel, dim3((nwords + 255) / 256), dim3(256), 0, st, x, K, out);
    ATLAS_LAUNCH_CHECK("xq_encode_kernel");
    return ATLAS_OK;
}

int launch_sum_partials(const float* part, int S, int N, float* y, hipStream_t st) {
    hipLaunchKernelGGL(sum_partials_kernel, dim3((N + 255) / 256), dim3(256), 0, st, part, S, N, y);
    ATLAS_LAUNCH_CHECK("sum_partials_kernel");
    return ATLAS_OK;
}

GemvArgs gemv_args(const atlas_w4* W, XQ xq, float* y) {
    GemvArgs a{};
    a.qweight = W->qweight;
    a.scales = W->scales;
    a.zeros = W->zeros;
    a.N = W->N;
    a.K = W->K;
    a.group = W->group;
    a.scale_dtype = W->scale_dtype;
    a.xq = xq;
    a.y = y;
    return a;
}

size_t gemv_workspace_bytes(int N, int K) {
    GemvPlan p = plan_gemv(N, K);
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
    GemvPlan p = plan_gemv(W->N, W->K);
    ATLAS_CHECK_SHAPE(p.CW > 0, "K=%d cannot be split into ranges of <= 320 chunks", W->K);
    hipStream_t st = (hipStream_t)stream;
    XQ xq = xq_view(ws, W->K);
    rc = launch_xq_encode(x, W->K, xq, st);
    if (rc) return rc;
    float* part = p.S > 1 ? (float*)((char*)ws + align_up(xq_bytes(W->K), 256)) : y;
    rc = launch_gemv(gemv_args(W, xq, part), p, st);
    if (rc) return rc;
    if (p.S > 1) return launch_sum_partials(part, p.S, W->N, y, st);
    return ATLAS_OK;
}

extern "C" int atlas_w4_dequant(const atlas_w4* W, float* out, void* stream) {
    int rc = validate_w4(W);
    if (rc) return rc;
    ATLAS_CHECK_ARG(out != nullptr, "null out");
    GemvArgs a = gemv_args(W, XQ{}, nullptr);
    hipLaunchKernelGGL(w4_dequant_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream, a, out);
    ATLAS_LAUNCH_CHECK("w4_dequant_kernel");
    return ATLAS_OK;
}
