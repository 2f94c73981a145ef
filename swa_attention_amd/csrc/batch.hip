// Batched decode: one token for each of B sequences (own token, position and KV cache,
// shared weights), the weights read once per step for all of them.
//
// Source: "ATLAS-OLMo-3-32B-Think-v4", Limitations & roadmap (batch-1 serving today,
// batched decode planned). A batch is by definition B independent decode steps. With
// B tokens the projections are skinny matrix products, so they run on the prefill's
// matrix-core W4 GEMM over B rows (split over K for the narrow ones, so that the grid
// still covers the chip), and the lm_head, read once for all rows, on bf16 matrix cores.
// Per layer:
//   w4_gemm (qkv, split-K) -> bd_rope (sum of the splits, QK norm, rotary at each
//   row's position, k/v into that sequence's cache) -> attn_kernel over (splits, KV
//   heads, sequences) -> merge -> pf_split -> w4_gemm (o, split-K) -> bd_residual ->
//   w4_gemm (gate+up, SwiGLU) -> w4_gemm (down, split-K) -> bd_residual
// then bd_final_norm -> bd_head (logits [B][V]) -> bd_argmax_rows.
#include <cmath>

#include "bgemv.h"
#include "decode.h"
#include "gemv.h"
#include "norm_rope.h"
#include "prefill_kernels.h"

namespace atlas {

typedef __bf16 bd_bf16x8_t __attribute__((ext_vector_type(8)));

// Sum of `parts` partial values at stride `stride` (split-K results): eight independent
// accumulators, so that eight loads are in flight at once.
__device__ __forceinline__ float bd_sum_parts(const float* p, int parts, size_t stride) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int q = 0;
    for (; q + 8 <= parts; q += 8)
#pragma unroll
        for (int u = 0; u < 8; u++) s[u] += p[(size_t)(q + u) * stride];
    for (; q < parts; q++) s[0] += p[(size_t)q * stride];
    return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

__device__ __forceinline__ void bd_split(float x, uint32_t& hi, uint32_t& lo) {
    hi = f32_to_bf16_rne_finite(x);
    lo = f32_to_bf16_rne_finite(x - __uint_as_float(hi << 16));
}

// ---- QK norm, rotary and KV store per sequence -------------------------------------------------

struct BdRopeArgs {
    float* qkv;                // [B][ld]: the sum of the split partials; q rotated in place
    const float* part;         // [parts][B][ld] partial projections
    int parts;
    size_t part_stride;
    int ld, Hq, Hkv;
    const float *g_q, *g_k;
    float eps;
    double inv[64];
    double mscale;
    const int32_t* d_pos;      // [B]
    void* k_cache;             // [B][Hkv][slots][128], f32 or bf16
    void* v_cache;
    int64_t slots, seq_stride, T_max;
    int ring, kv_bf16;
    int* status;
};

// One block per sequence; the summed row stays in LDS (dynamic, ld floats) between the
// norms and the rotation, and every global load of the partials is issued before the
// first barrier.
// The sum of `parts` partial rows (N columns from p, N = 4 or 8), in partial order. With
// up to 8 partials the count is a template argument: every load is issued before the
// first add, so their latencies overlap; more partials are summed in a loop.
template <int P, int N>
__device__ __forceinline__ void bd_sum_fixed(const float* p, size_t stride, float (&out)[N]) {
    float4 a[P][N / 4];
#pragma unroll
    for (int q = 0; q < P; q++)
#pragma unroll
        for (int c = 0; c < N / 4; c++) a[q][c] = *reinterpret_cast<const float4*>(p + (size_t)q * stride + 4 * c);
#pragma unroll
    for (int c = 0; c < N / 4; c++) {
        float4 s = a[0][c];
#pragma unroll
        for (int q = 1; q < P; q++) {
            s.x += a[q][c].x; s.y += a[q][c].y; s.z += a[q][c].z; s.w += a[q][c].w;
        }
        out[4 * c] = s.x; out[4 * c + 1] = s.y; out[4 * c + 2] = s.z; out[4 * c + 3] = s.w;
    }
}
template <int N>
__device__ __forceinline__ void bd_sum(const float* p, int parts, size_t stride, float (&out)[N]) {
    switch (parts) {
        case 1: bd_sum_fixed<1, N>(p, stride, out); return;
        case 2: bd_sum_fixed<2, N>(p, stride, out); return;
        case 3: bd_sum_fixed<3, N>(p, stride, out); return;
        case 4: bd_sum_fixed<4, N>(p, stride, out); return;
        case 5: bd_sum_fixed<5, N>(p, stride, out); return;
        case 6: bd_sum_fixed<6, N>(p, stride, out); return;
        case 7: bd_sum_fixed<7, N>(p, stride, out); return;
        case 8: bd_sum_fixed<8, N>(p, stride, out); return;
        default: break;
    }
#pragma unroll
    for (int c = 0; c < N; c++) out[c] = p[c];
    for (int q = 1; q < parts; q++)
#pragma unroll
        for (int c = 0; c < N; c++) out[c] += p[(size_t)q * stride + c];
}

// One block of BD_ROPE_NT threads per sequence. Every load is issued before the first
// is used: the position, up to BD_ROPE_NV float4 of each of the first BD_ROPE_MAXP
// partial rows per thread, and the gains of the thread's first BD_ROPE_NR rotation pairs
// (rows, partials and pairs beyond these take the loops after them).
constexpr int BD_ROPE_NT = 1024, BD_ROPE_NV = 2, BD_ROPE_MAXP = 4, BD_ROPE_NR = 3;
__global__ __launch_bounds__(BD_ROPE_NT) void bd_rope_kernel(BdRopeArgs a) {
    constexpr int D = 128, NT = BD_ROPE_NT;
    extern __shared__ float s_row[];   // [ld]
    __shared__ float red[2][16];
    __shared__ float s_cos[64], s_sin[64];
    const int t = blockIdx.x, tid = threadIdx.x;
    const int pos = a.d_pos[t];
    const int nq = a.Hq * D, nk = a.Hkv * D;
    const int lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
    const int n4 = a.ld >> 2, npairs = (a.Hq + a.Hkv) * 64;   // ld, nq, nk multiples of 4
    const float* prow = a.part + (size_t)t * a.ld;
    float4 pv[BD_ROPE_NV][BD_ROPE_MAXP];
#pragma unroll
    for (int j = 0; j < BD_ROPE_NV; j++) {
        const int i4 = tid + NT * j, ic = i4 < n4 ? i4 : 0;
#pragma unroll
        for (int q = 0; q < BD_ROPE_MAXP; q++)
            pv[j][q] = *reinterpret_cast<const float4*>(prow + (size_t)min(q, a.parts - 1) * a.part_stride + 4 * ic);
    }
    float g0[BD_ROPE_NR], g1[BD_ROPE_NR];
#pragma unroll
    for (int r = 0; r < BD_ROPE_NR; r++) {
        const int u = tid + NT * r, uc = u < npairs ? u : 0;
        const int h = uc >> 6, i = uc & 63;
        const float* g = h >= a.Hq ? a.g_k + (h - a.Hq) * D : a.g_q + h * D;
        g0[r] = g[i];
        g1[r] = g[i + 64];
    }
    float sq = 0.f, sk = 0.f;
    auto add_row = [&](int i4, float4 v) {   // v: the sum of the partials of float4 i4
        const int i = 4 * i4;
        *reinterpret_cast<float4*>(&s_row[i]) = v;
        const float ss = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        sq += i < nq ? ss : 0.f;
        sk += (i >= nq && i < nq + nk) ? ss : 0.f;
    };
    auto more_parts = [&](int i4, float4& v) {
        for (int q = BD_ROPE_MAXP; q < a.parts; q++) {
            const float4 u = *reinterpret_cast<const float4*>(prow + (size_t)q * a.part_stride + 4 * i4);
            v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
        }
    };
#pragma unroll
    for (int j = 0; j < BD_ROPE_NV; j++) {
        const int i4 = tid + NT * j;
        if (i4 < n4) {
            float4 v = pv[j][0];
#pragma unroll
            for (int q = 1; q < BD_ROPE_MAXP; q++) {
                if (q < a.parts) {
                    v.x += pv[j][q].x; v.y += pv[j][q].y; v.z += pv[j][q].z; v.w += pv[j][q].w;
                }
            }
            more_parts(i4, v);
            add_row(i4, v);
        }
    }
    for (int i4 = tid + NT * BD_ROPE_NV; i4 < n4; i4 += NT) {
        float4 v = *reinterpret_cast<const float4*>(prow + 4 * i4);
        for (int q = 1; q < min(a.parts, BD_ROPE_MAXP); q++) {
            const float4 u = *reinterpret_cast<const float4*>(prow + (size_t)q * a.part_stride + 4 * i4);
            v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
        }
        more_parts(i4, v);
        add_row(i4, v);
    }
    const bool ok = pos >= 0 && pos < a.T_max;
    if (threadIdx.x < 64 && ok) {
        const double ang = (double)pos * a.inv[threadIdx.x];
        const double rr = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
        float sn, cs;
        sincosf((float)rr, &sn, &cs);
        s_cos[threadIdx.x] = cs * (float)a.mscale;
        s_sin[threadIdx.x] = sn * (float)a.mscale;
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    if (lane == 0) {
        red[0][w] = sq;
        red[1][w] = sk;
    }
    __syncthreads();
    float* row = a.qkv + (size_t)t * a.ld;
    if (!ok) {   // the attention of this row reports it too; nothing is stored in the cache
        for (int i = threadIdx.x; i < nq; i += blockDim.x) row[i] = s_row[i];
        if (threadIdx.x == 0) *a.status = ATLAS_ERR_INVALID_ARG;
        return;
    }
    sq = 0.f;
    sk = 0.f;
    for (int i = 0; i < nw; i++) {
        sq += red[0][i];
        sk += red[1][i];
    }
    const float rq = 1.0f / sqrtf(sq / (float)nq + a.eps);
    const float rk = 1.0f / sqrtf(sk / (float)nk + a.eps);
    const int slot = a.ring ? pos % (int)a.slots : pos;
    const size_t cache0 = (size_t)t * a.seq_stride + (size_t)slot * D;
    auto rotate = [&](int u, float ga, float gb) {   // pair u: dims i and i + 64 of head u / 64
        const int h = u >> 6, i = u & 63;
        const bool isk = h >= a.Hq;
        const float rr = isk ? rk : rq;
        const int base = h * D;
        const float x0 = ga * (s_row[base + i] * rr), x1 = gb * (s_row[base + i + 64] * rr);
        const float c = s_cos[i], sn = s_sin[i];
        const float y0 = x0 * c - x1 * sn, y1 = x1 * c + x0 * sn;
        if (isk) {
            const size_t e = cache0 + (size_t)(h - a.Hq) * a.slots * D + i;
            if (a.kv_bf16) {
                ((uint16_t*)a.k_cache)[e] = (uint16_t)f32_to_bf16_rne(y0);
                ((uint16_t*)a.k_cache)[e + 64] = (uint16_t)f32_to_bf16_rne(y1);
            } else {
                ((float*)a.k_cache)[e] = y0;
                ((float*)a.k_cache)[e + 64] = y1;
            }
        } else {
            row[base + i] = y0;
            row[base + i + 64] = y1;
        }
    };
    static_assert(BD_ROPE_NR == 3, "three preloaded pairs");
    if (tid < npairs) rotate(tid, g0[0], g1[0]);
    if (tid + NT < npairs) rotate(tid + NT, g0[1], g1[1]);
    if (tid + 2 * NT < npairs) rotate(tid + 2 * NT, g0[2], g1[2]);
    for (int u = tid + NT * BD_ROPE_NR; u < npairs; u += NT) {
        const int h = u >> 6, i = u & 63;
        const float* g = h >= a.Hq ? a.g_k + (h - a.Hq) * D : a.g_q + h * D;
        rotate(u, g[i], g[i + 64]);
    }
    for (int u = threadIdx.x; u < nk; u += blockDim.x) {
        const int h = u / D, i = u % D;
        const size_t e = cache0 + (size_t)h * a.slots * D + i;
        const float v = s_row[nq + nk + u];
        if (a.kv_bf16) ((uint16_t*)a.v_cache)[e] = (uint16_t)f32_to_bf16_rne(v);
        else ((float*)a.v_cache)[e] = v;
    }
}

// ---- residual with split partials, final norm --------------------------------------------------

// X[t] += g * A[t] / rms(A[t]) with A[t] the sum of `parts` partial rows; then the bf16
// planes of the new X[t] for the next projection.
__global__ __launch_bounds__(1024) void bd_residual_kernel(float* X, const float* part, int parts, size_t part_stride,
                                                         const float* g, int d, float eps, uint16_t* p_hi,
                                                         uint16_t* p_lo, int ldp) {
    extern __shared__ float s_a[];   // [d]
    __shared__ float red[16];
    const int t = blockIdx.x;
    float ss = 0.f;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        const float v = bd_sum_parts(part + (size_t)t * d + i, parts, part_stride);
        s_a[i] = v;
        ss = fmaf(v, v, ss);
    }
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    float* x = X + (size_t)t * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        const float h = x[i] + g[i] * (s_a[i] * r);
        x[i] = h;
        uint32_t hi, lo;
        bd_split(h, hi, lo);
        p_hi[(size_t)t * ldp + i] = (uint16_t)hi;
        p_lo[(size_t)t * ldp + i] = (uint16_t)lo;
    }
}

// y = g * X[t] / rms(X[t]) as bf16 planes (the final norm before the lm_head).
__global__ __launch_bounds__(1024) void bd_final_norm_kernel(const float* X, const float* g, int d, float eps,
                                                           uint16_t* y_hi, uint16_t* y_lo, int ldy) {
    __shared__ float red[16];
    const int t = blockIdx.x;
    const float* x = X + (size_t)t * d;
    float ss = 0.f;
    for (int i = threadIdx.x; i < d; i += blockDim.x) ss = fmaf(x[i], x[i], ss);
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        uint32_t hi, lo;
        bd_split(g[i] * (x[i] * r), hi, lo);
        y_hi[(size_t)t * ldy + i] = (uint16_t)hi;
        y_lo[(size_t)t * ldy + i] = (uint16_t)lo;
    }
}

// z = silu(g) * u with g, u the sums of `parts` partial rows [parts][B][n], as the bf16
// planes of the down projection's input. One thread per element.
__global__ __launch_bounds__(256) void bd_swiglu_kernel(const float* gp, const float* up, int parts, size_t part_stride,
                                                       int total, uint16_t* z_hi, uint16_t* z_lo) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const float g = bd_sum_parts(gp + i, parts, part_stride), u = bd_sum_parts(up + i, parts, part_stride);
    uint32_t hi, lo;
    bd_split(g / (1.0f + __expf(-g)) * u, hi, lo);
    z_hi[i] = (uint16_t)hi;
    z_lo[i] = (uint16_t)lo;
}

// ---- the same for the int8-plane projections (B <= 8, see bgemv.hip) -------------------------

// Sum of `parts` partial rows at 8 consecutive columns, in split order.
__device__ __forceinline__ void bd_sum8(const float* p, int parts, size_t stride, float out[8]) {
    float v[8];
    bd_sum(p, parts, stride, v);
#pragma unroll
    for (int c = 0; c < 8; c++) out[c] = v[c];
}

// X[t] += g * A[t] / rms(A[t]) (A[t] the sum of `parts` partial rows), then X[t] encoded
// for the next projection. One block of whole waves per row; thread i holds columns
// 8 i .. 8 i + 7, and the block covers the encoding's padded width (16 threads per 128
// columns).
__global__ __launch_bounds__(1024) void bd_residual_q_kernel(float* X, const float* part, int parts,
                                                           size_t part_stride, const float* g, int d, float eps,
                                                           BQ q) {
    __shared__ float red[16];
    const int t = blockIdx.x, col0 = 8 * threadIdx.x;
    const bool on = col0 < d;
    float a[8], x[8], gv[8];
    float ss = 0.f;
    float* xr = X + (size_t)t * d + col0;
    if (on) {   // the residual and the gain are loaded before the block sum, with the partials
        const float4 x0 = *reinterpret_cast<const float4*>(xr), x1 = *reinterpret_cast<const float4*>(xr + 4);
        x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w; x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
#pragma unroll
        for (int j = 0; j < 8; j++) gv[j] = g[col0 + j];   // the caller's gains: 4-byte aligned only
        bd_sum8(part + (size_t)t * d + col0, parts, part_stride, a);
#pragma unroll
        for (int j = 0; j < 8; j++) ss = fmaf(a[j], a[j], ss);
    }
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    if (on) {
#pragma unroll
        for (int j = 0; j < 8; j++) x[j] = x[j] + gv[j] * (a[j] * r);
        *reinterpret_cast<float4*>(xr) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(xr + 4) = make_float4(x[4], x[5], x[6], x[7]);
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) x[j] = 0.f;
    }
    if (col0 < q.ldq) bq_encode_row16(x, q, t, col0, threadIdx.x >> 4);   // whole rows of 16 lanes
}

// z = silu(g) * u (g, u the sums of `parts` partial rows [parts][B][n]), encoded for the
// down projection. Grid (blocks over 16 threads per 128 columns, B).
__global__ __launch_bounds__(256) void bd_swiglu_q_kernel(const float* gp, const float* up, int parts,
                                                         size_t part_stride, int n, BQ q) {
    const int t = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x, col0 = 8 * i;
    float z[8];
    if (col0 < n) {
        float gv[8], uv[8];
        bd_sum8(gp + (size_t)t * n + col0, parts, part_stride, gv);
        bd_sum8(up + (size_t)t * n + col0, parts, part_stride, uv);
#pragma unroll
        for (int j = 0; j < 8; j++) z[j] = gv[j] / (1.0f + __expf(-gv[j])) * uv[j];
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) z[j] = 0.f;
    }
    if (col0 < q.ldq) bq_encode_row16(z, q, t, col0, i >> 4);   // whole rows of 16 lanes
}

// ---- lm_head over the batch: bf16 matrix cores, weights streamed once --------------------------

// logits[m][n] = sum_k W[n][k] y[m][k] for m < B (<= 16), n < V (d % 64 == 0). One wave
// per BD_HEAD_TILES x 16 vocabulary rows, on v_mfma_f32_16x16x32_bf16 with y = hi + lo.
//
// Loads. A wave instruction that reads 16 rows x 64 bytes (the MFMA operand layout: lane
// l holds row l % 16, bytes 16 (l / 16)) streams this matrix at about 3.7 TB/s, one that
// reads 8 whole 128-byte lines at about 5.1 (5.4 nontemporal), measured with loads alone
// on this grid. So a step takes one 128-byte line (64 columns) of each of a tile's 16
// rows in two nontemporal loads: X, rows 0-7, and Y, rows 8-15, lane l reading row
// l % 8 (+8 for Y) at bytes 16 (l / 8) of the line. Rotating a 16-lane row by 8 lanes
// (DPP row_ror:8) swaps its halves, so
//   B0 = X with lanes 8-15 of each row taken from Y rotated: lane l holds row l % 16,
//        16-byte chunk 2 (l / 16) of the line;
//   B1 = Y with lanes 0-7 of each row taken from X rotated: row l % 16, chunk 2 (l / 16) + 1;
// two bank-masked DPP moves per dword, no LDS. The A operands follow the same order:
// y[l % 16][64 t + 16 (l / 16) ..+8] for B0, the next 8 columns for B1.
//
// Ring. The loads of the step BD_HEAD_AHEAD on are issued after each step's products;
// scheduling barriers keep the compiler from hoisting them above the products (the loads
// then reuse the slot's registers, so the loop needs no copies) or sinking them to their
// use (which would empty the ring): a step waits only for its own loads. EVEN: the steps
// are a multiple of BD_HEAD_AHEAD; otherwise the steps past the end multiply their
// (clamped, in-bounds) reloads by zero activations rather than branch round them.
constexpr int BD_HEAD_WAVES = 4, BD_HEAD_TILES = 4, BD_HEAD_AHEAD = 2;
constexpr int BD_DPP_ROW_ROR8 = 0x128;
__device__ __forceinline__ uint32_t bd_halves(uint32_t keep, uint32_t rot, int bank_mask_is_high) {
    return bank_mask_is_high ? (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)rot, BD_DPP_ROW_ROR8, 0xF, 0xC, false)
                             : (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)rot, BD_DPP_ROW_ROR8, 0xF, 0x3, false);
}
template <bool EVEN>
__global__ __launch_bounds__(64 * BD_HEAD_WAVES) void bd_head_kernel(const uint16_t* __restrict__ y_hi,
                                                                      const uint16_t* __restrict__ y_lo, int ldy,
                                                                      int B, const uint16_t* __restrict__ W, int V,
                                                                      int d, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = (blockIdx.x * BD_HEAD_WAVES + wave) * 16 * BD_HEAD_TILES;
    if (n0 >= V) return;
    const int l16 = lane & 15;
    const int m = min(l16, B - 1);
    const u32x4_t* wrow[BD_HEAD_TILES][2];
#pragma unroll
    for (int i = 0; i < BD_HEAD_TILES; i++)
#pragma unroll
        for (int h = 0; h < 2; h++)
            wrow[i][h] = reinterpret_cast<const u32x4_t*>(W + (size_t)min(n0 + 16 * i + 8 * h + (lane & 7), V - 1) * d +
                                                          8 * (lane >> 3));
    const uint4* yh = reinterpret_cast<const uint4*>(y_hi + (size_t)m * ldy + 16 * (lane >> 4));
    const uint4* yl = reinterpret_cast<const uint4*>(y_lo + (size_t)m * ldy + 16 * (lane >> 4));
    const int steps = d / 64;   // one 128-byte line of each row per step
    // d is a positive multiple of 64 (checked before launch): with no loop guard the
    // compiler keeps the ring's first loads in slot order rather than sinking them past it
    __builtin_assume(steps > 0);
    u32x4_t wv[BD_HEAD_AHEAD][BD_HEAD_TILES][2];
    uint4 yv[BD_HEAD_AHEAD][4];   // hi B0, hi B1, lo B0, lo B1
    auto load = [&](int s, int st) {
        yv[s][0] = yh[8 * st];
        yv[s][1] = yh[8 * st + 1];
        yv[s][2] = yl[8 * st];
        yv[s][3] = yl[8 * st + 1];
#pragma unroll
        for (int i = 0; i < BD_HEAD_TILES; i++)
#pragma unroll
            for (int h = 0; h < 2; h++) wv[s][i][h] = __builtin_nontemporal_load(wrow[i][h] + 8 * st);
    };
#pragma unroll
    for (int s = 0; s < BD_HEAD_AHEAD; s++) {
        load(s, min(s, steps - 1));
        __builtin_amdgcn_sched_barrier(0);   // slots issue in step order, as the loop refills them
    }
    f32x4_t acc[BD_HEAD_TILES];
#pragma unroll
    for (int i = 0; i < BD_HEAD_TILES; i++) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < steps; s0 += BD_HEAD_AHEAD) {
#pragma unroll
        for (int s = 0; s < BD_HEAD_AHEAD; s++) {
            const int st = s0 + s;
            const bool live = EVEN || st < steps;
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            const bd_bf16x8_t h0 = __builtin_bit_cast(bd_bf16x8_t, live ? yv[s][0] : z);
            const bd_bf16x8_t h1 = __builtin_bit_cast(bd_bf16x8_t, live ? yv[s][1] : z);
            const bd_bf16x8_t lo0 = __builtin_bit_cast(bd_bf16x8_t, live ? yv[s][2] : z);
            const bd_bf16x8_t lo1 = __builtin_bit_cast(bd_bf16x8_t, live ? yv[s][3] : z);
#pragma unroll
            for (int i = 0; i < BD_HEAD_TILES; i++) {
                const u32x4_t x = wv[s][i][0], y = wv[s][i][1];
                const uint4 b0 = make_uint4(bd_halves(x[0], y[0], 1), bd_halves(x[1], y[1], 1),
                                            bd_halves(x[2], y[2], 1), bd_halves(x[3], y[3], 1));
                const uint4 b1 = make_uint4(bd_halves(y[0], x[0], 0), bd_halves(y[1], x[1], 0),
                                            bd_halves(y[2], x[2], 0), bd_halves(y[3], x[3], 0));
                const bd_bf16x8_t w0 = __builtin_bit_cast(bd_bf16x8_t, b0), w1 = __builtin_bit_cast(bd_bf16x8_t, b1);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h0, w0, acc[i], 0, 0, 0);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo0, w0, acc[i], 0, 0, 0);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h1, w1, acc[i], 0, 0, 0);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo1, w1, acc[i], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            load(s, min(st + BD_HEAD_AHEAD, steps - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // acc[i][r] = logits[row 4 (l / 16) + r][column n0 + 16 i + l % 16]
#pragma unroll
    for (int i = 0; i < BD_HEAD_TILES; i++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int mm = 4 * (lane >> 4) + r, nn = n0 + 16 * i + l16;
            if (mm < B && nn < V) logits[(size_t)mm * V + nn] = acc[i][r];
        }
}

// First index of the maximum of each row of logits [B][V].
__global__ __launch_bounds__(1024) void bd_argmax_rows_kernel(const float* logits, int V, int32_t* out) {
    __shared__ float sv[1024];
    __shared__ int si[1024];
    const float* row = logits + (size_t)blockIdx.x * V;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    auto see = [&](float v, int i) {   // i increases per thread: the first maximum is kept
        if (v > best) {
            best = v;
            bi = i;
        }
    };
    // up to three leading elements, then 16-byte loads (each thread's indices increase)
    const int lead = min(V, (int)(((16 - ((uintptr_t)row & 15)) & 15) / 4));
    if ((int)threadIdx.x < lead) see(row[threadIdx.x], threadIdx.x);
    const float4* r4 = reinterpret_cast<const float4*>(row + lead);
    const int V4 = (V - lead) >> 2;
#pragma unroll 4
    for (int i = threadIdx.x; i < V4; i += 1024) {
        const float4 v = r4[i];
        const int j = lead + 4 * i;
        see(v.x, j);
        see(v.y, j + 1);
        see(v.z, j + 2);
        see(v.w, j + 3);
    }
    for (int i = lead + 4 * V4 + threadIdx.x; i < V; i += 1024) see(row[i], i);
    sv[threadIdx.x] = best;
    si[threadIdx.x] = bi;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) {
            const float x = sv[threadIdx.x + o];
            const int ix = si[threadIdx.x + o];
            if (x > sv[threadIdx.x] || (x == sv[threadIdx.x] && ix < si[threadIdx.x])) {
                sv[threadIdx.x] = x;
                si[threadIdx.x] = ix;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = si[0];
}

// ---- host ----------------------------------------------------------------------------------------

constexpr int BD_MAX_BATCH = 16;

// Splits of K for a GEMM of `tiles` 128-row output tiles over a few rows. With one tile
// row the blocks are few and each is bound by the latency of its K loop, so the K range
// is cut (at most 32 ranges, each a whole number of groups and 64-column tiles): the
// smallest count with tiles * s >= target, else the largest that fits.
int bd_ksplit(int tiles, int K, int group, int target) {
    int best = 1;
    for (int s = 2; s <= 32; s++) {
        if (K % s) continue;
        const int c = K / s;
        if (c % 64 || c % group) continue;
        best = s;
        if (tiles * s >= target) break;
    }
    return best;
}
// Split targets in 128-row tiles, measured at 8 sequences on the 32B shapes: the
// small-row kernel runs two 4-wave blocks per CU, so gate/up (4 splits, 432 blocks) and
// down (24 splits, 480 blocks) are best just under one 512-block round (5 and 27 splits
// spill into a second: 63 and 69 us against 53 and 54); qkv and o are best at 8 and 10
// splits (19 and 16 us against 25 and 18 at 20 and 40).
constexpr int BD_SPLIT_TARGET_ATTN_PROJ = 384, BD_SPLIT_TARGET_MLP = 768;

struct BatchPlan {
    int sq, so, sg, sd;   // K splits of the qkv, o, gate/up and down projections
    int S_swa, S_full, S_max;
    bool bq;              // projections on int8 planes (bgemv.hip); else the bf16-plane GEMM
};

// Whether every projection of every layer takes the int8-plane batched GEMV.
static bool batch_bq_ok(const atlas_model* m, int B) {
    if (B > BG_MAX_B || m->d % 64 || m->d > 8192) return false;
    for (int l = 0; l < m->n_layers; l++) {
        const atlas_layer& L = m->layers[l];
        const atlas_w4* ws[5] = {&L.qkv, &L.o, &L.gate, &L.up, &L.down};
        for (const atlas_w4* w : ws) {
            const W4View v = w4_view(w->qweight, w->scales, w->zeros, w->N, w->K, w->group, w->scale_dtype);
            if (!bgemv_supported(v, w->group)) return false;
        }
        if (L.gate.group != L.up.group) return false;
    }
    return true;
}

static BatchPlan batch_plan(const atlas_model* m, int B) {
    BatchPlan p{};
    const int nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    p.bq = batch_bq_ok(m, B);
    const int MT = (B + 63) / 64;
    p.sq = bd_ksplit(MT * ((nqkv + 127) / 128), m->d, m->layers[0].qkv.group, BD_SPLIT_TARGET_ATTN_PROJ);
    p.so = bd_ksplit(MT * ((m->d + 127) / 128), nq, m->layers[0].o.group, BD_SPLIT_TARGET_ATTN_PROJ);
    p.sg = bd_ksplit(MT * ((m->dff + 127) / 128), m->d, m->layers[0].gate.group, BD_SPLIT_TARGET_MLP);
    p.sd = bd_ksplit(MT * ((m->d + 127) / 128), m->dff, m->layers[0].down.group, BD_SPLIT_TARGET_MLP);
    for (int l = 1; l < m->n_layers; l++) {   // one plan for every layer: take splits all layers allow
        const atlas_layer& L = m->layers[l];
        if (m->d % (p.sq * L.qkv.group) || (m->d / p.sq) % 64) p.sq = 1;
        if (nq % (p.so * L.o.group) || (nq / p.so) % 64) p.so = 1;
        if (m->d % (p.sg * L.gate.group) || (m->d / p.sg) % 64) p.sg = 1;
        if (m->dff % (p.sd * L.down.group) || (m->dff / p.sd) % 64) p.sd = 1;
    }
    if (p.bq) {   // the int8-plane GEMV picks its own K split
        p.sq = bgemv_splits(m->d, nqkv);
        p.so = bgemv_splits(nq, m->d);
        p.sg = bgemv_splits(m->d, m->dff, m->dff);
        p.sd = bgemv_splits(m->dff, m->d);
    }
    const int64_t swa_keys = m->window > 0 ? std::min<int64_t>(m->window, m->t_max) : m->t_max;
    // key splits sized as for half the (KV head, sequence) blocks: at 8 sequences, 8 on the
    // window (32.0 us against 35.4 at 4) and 16 on full layers (no change); four times as
    // many made full layers slower (119 us)
    p.S_swa = attn_splits(swa_keys, std::max(1, m->hkv * B / 2));
    p.S_full = attn_splits(m->t_max, std::max(1, m->hkv * B / 2));
    p.S_max = std::max(p.S_swa, p.S_full);
    return p;
}

struct BatchWs {
    int* status;
    float *X, *qkv, *qkv_part, *o, *attn_part, *a_part, *g_part, *u_part, *logits;
    uint16_t *p1h, *p1l, *p2h, *p2l;
    int ld1;
    void* bq;             // int8 planes of the current projection input (plan.bq)
    size_t bytes;
};

static BatchWs carve_batch(const atlas_model* m, int B, const BatchPlan& p, void* base, bool need_logits) {
    BatchWs w{};
    char* b = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        void* q = b ? b + off : nullptr;
        off += align_up(bytes, 256);
        return q;
    };
    const int nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    w.ld1 = std::max(m->d, nq);
    w.status = (int*)take(256);
    w.X = (float*)take((size_t)B * m->d * 4);
    w.qkv = (float*)take((size_t)B * nqkv * 4);
    w.qkv_part = (float*)take((size_t)p.sq * B * nqkv * 4);
    w.o = (float*)take((size_t)B * nq * 4);
    w.attn_part = (float*)take((size_t)B * m->hq * p.S_max * ATTN_PART_F * 4);
    w.a_part = (float*)take((size_t)std::max(p.so, p.sd) * B * m->d * 4);
    w.g_part = (float*)take((size_t)p.sg * B * m->dff * 4);
    w.u_part = (float*)take((size_t)p.sg * B * m->dff * 4);
    w.p1h = (uint16_t*)take((size_t)B * w.ld1 * 2);
    w.p1l = (uint16_t*)take((size_t)B * w.ld1 * 2);
    w.p2h = (uint16_t*)take((size_t)B * m->dff * 2);
    w.p2l = (uint16_t*)take((size_t)B * m->dff * 2);
    w.logits = need_logits ? (float*)take((size_t)B * m->vocab * 4) : nullptr;
    w.bq = p.bq ? take(bq_bytes(B, std::max(std::max(m->d, nq), m->dff))) : nullptr;
    w.bytes = off;
    return w;
}

static W4View bview(const atlas_w4& w) { return w4_view(w.qweight, w.scales, w.zeros, w.N, w.K, w.group, w.scale_dtype); }

static GemmArgs bgemm(const uint16_t* hi, const uint16_t* lo, int lda, const atlas_w4& w, int M) {
    GemmArgs g{};
    g.a_hi = hi;
    g.a_lo = lo;
    g.lda = lda;
    g.W0 = bview(w);
    g.W1 = g.W0;
    g.M = M;
    g.N = w.N;
    g.K = w.K;
    g.group = w.group;
    return g;
}

static int validate_batch(const atlas_model* m, int B) {
    int rc = validate_model(m);
    if (rc) return rc;
    ATLAS_CHECK_ARG(B >= 1 && B <= BD_MAX_BATCH, "batch=%d outside [1, %d]", B, BD_MAX_BATCH);
    ATLAS_CHECK_ARG(m->embedding, "batched decode needs an embedding table");
    ATLAS_CHECK_SHAPE(m->d % 64 == 0, "batched decode needs d %% 64 == 0 (d=%d)", m->d);
    for (int l = 0; l < m->n_layers; l++) {
        const atlas_layer& L = m->layers[l];
        const atlas_w4* ws[5] = {&L.qkv, &L.o, &L.gate, &L.up, &L.down};
        for (const atlas_w4* w : ws)
            ATLAS_CHECK_SHAPE(gemm_supported(w->group), "batched decode needs group 32 or a multiple of 64 (layer %d)",
                              l);
    }
    return ATLAS_OK;
}

}  // namespace atlas

using namespace atlas;

extern "C" size_t atlas_decode_batch_workspace_bytes(const atlas_model* m, int32_t batch) {
    if (validate_batch(m, batch) != ATLAS_OK) return 0;
    return carve_batch(m, batch, batch_plan(m, batch), nullptr, true).bytes;
}

extern "C" int atlas_decode_batch(const atlas_model* m, const int32_t* d_tokens, const int32_t* d_pos, int32_t batch,
                                  float* d_hidden_out, float* d_logits, int32_t* d_argmax, void* ws, size_t ws_bytes,
                                  void* stream) {
    int rc = validate_batch(m, batch);
    if (rc) return rc;
    ATLAS_CHECK_ARG(d_tokens && d_pos && ws, "null pointer");
    const bool head = d_logits || d_argmax;
    ATLAS_CHECK_ARG(!head || (m->lm_head && m->g_final && m->vocab >= 1), "lm_head/g_final/vocab missing");
    const int B = batch;
    const BatchPlan p = batch_plan(m, B);
    const BatchWs w = carve_batch(m, B, p, ws, true);
    if (ws_bytes < w.bytes) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, w.bytes);
    hipStream_t st = (hipStream_t)stream;
    const int d = m->d, nq = m->hq * m->hd, nqkv = (m->hq + 2 * m->hkv) * m->hd;
    RopeTable rt_swa, rt_full;
    rope_table(&m->rope_swa, m->hd, &rt_swa);
    rope_table(&m->rope_full, m->hd, &rt_full);
    // the embedding kernel writes the status word first (ATLAS_OK, or a bad token id)
    if ((rc = launch_pf_embed(d_tokens, B, m->embedding, m->vocab, d, w.X, w.p1h, w.p1l, w.ld1, w.status, st)))
        return rc;
    const BQ q_d = p.bq ? bq_carve(w.bq, B, d) : BQ{};       // inputs of qkv and gate/up
    const BQ q_nq = p.bq ? bq_carve(w.bq, B, nq) : BQ{};     // input of o
    const BQ q_ff = p.bq ? bq_carve(w.bq, B, m->dff) : BQ{}; // input of down
    if (p.bq && (rc = launch_bq_encode(w.X, d, B, d, q_d, st))) return rc;
    // whole waves (the block sum reads every lane), covering the encoding's padded width
    const unsigned res_threads = (unsigned)align_up((size_t)16 * ((d + 127) / 128), 64);
    for (int l = 0; l < m->n_layers; l++) {
        const atlas_layer& L = m->layers[l];
        const bool ring = m->swa_ring && L.type == 0;
        const int64_t slots = ring ? m->window : m->t_max;
        const int64_t seq_stride = (int64_t)m->hkv * slots * m->hd;
        // qkv projection of the B rows, split over K
        if (p.bq) {
            const BgemvOut o{w.qkv_part, (size_t)B * nqkv, nqkv};
            if ((rc = launch_bgemv(bview(L.qkv), L.qkv.group, nullptr, q_d, B, o, nullptr, st, "bd_gemv_qkv")))
                return rc;
        } else {
            GemmArgs qa = bgemm(w.p1h, w.p1l, w.ld1, L.qkv, B);
            qa.C = w.qkv_part;
            qa.ldc = nqkv;
            qa.ksplit = p.sq;
            qa.kchunk = d / p.sq;
            qa.c_split = (size_t)B * nqkv;
            if ((rc = launch_w4_gemm(qa, 0, st, "bd_gemm_qkv"))) return rc;
        }
        // QK norm, rotary at each row's position, k/v into each sequence's cache
        BdRopeArgs ra{};
        ra.qkv = w.qkv;
        ra.part = w.qkv_part;
        ra.parts = p.sq;
        ra.part_stride = (size_t)B * nqkv;
        ra.ld = nqkv;
        ra.Hq = m->hq;
        ra.Hkv = m->hkv;
        ra.g_q = L.g_q;
        ra.g_k = L.g_k;
        ra.eps = m->eps;
        const RopeTable& rt = L.type == 1 ? rt_full : rt_swa;
        for (int i = 0; i < 64; i++) ra.inv[i] = rt.inv[i];
        ra.mscale = rt.mscale;
        ra.d_pos = d_pos;
        ra.k_cache = L.k_cache;
        ra.v_cache = L.v_cache;
        ra.slots = slots;
        ra.seq_stride = seq_stride;
        ra.T_max = m->t_max;
        ra.ring = ring ? 1 : 0;
        ra.kv_bf16 = m->kv_dtype;
        ra.status = w.status;
        prof_mark("bd_qk_norm_rope", st);
        ATLAS_KLAUNCH(bd_rope_kernel, dim3(B), dim3(1024), (size_t)nqkv * 4, st, ra);
        ATLAS_LAUNCH_CHECK("bd_rope_kernel");
        // attention per sequence, then the merge into o rows
        AttnFusedArgs aa{};
        aa.k_cache = L.k_cache;
        aa.v_cache = L.v_cache;
        aa.T_max = m->t_max;
        aa.slots = slots;
        aa.ring = ring ? 1 : 0;
        aa.kv_bf16 = m->kv_dtype;
        aa.d_pos = d_pos;
        aa.Hq = m->hq;
        aa.Hkv = m->hkv;
        aa.window = L.type == 1 ? 0 : m->window;
        aa.S = L.type == 1 ? p.S_full : p.S_swa;
        aa.scale = 1.0f / std::sqrt((float)m->hd);
        aa.part = w.attn_part;
        aa.status = w.status;
        aa.fused = 0;
        aa.q_final = w.qkv;
        aa.batch = B;
        aa.q_stride = nqkv;
        aa.seq_stride = seq_stride;
        aa.part_stride = (int64_t)m->hq * aa.S * ATTN_PART_F;
        if ((rc = launch_attn_fused(aa, m->hq / m->hkv, st))) return rc;
        MergeArgs ma{};
        ma.part = w.attn_part;
        ma.S = aa.S;
        ma.Hq = m->hq;
        ma.o = p.bq ? nullptr : w.o;
        if (p.bq) ma.bq = q_nq;   // the o projection's input, encoded by the merge
        ma.batch = B;
        ma.part_stride = aa.part_stride;
        ma.o_stride = nq;
        if ((rc = launch_merge(ma, st))) return rc;
        if (p.bq) {
            // o projection, h = x + RMSNorm_pa(a); gate/up, SwiGLU; down, y = h + RMSNorm_pf(m)
            const BgemvOut oo{w.a_part, (size_t)B * d, d};
            if ((rc = launch_bgemv(bview(L.o), L.o.group, nullptr, q_nq, B, oo, nullptr, st, "bd_gemv_o"))) return rc;
            prof_mark("bd_residual_norm", st);
            ATLAS_KLAUNCH(bd_residual_q_kernel, dim3(B), dim3(res_threads), 0, st, w.X, w.a_part, p.so, (size_t)B * d,
                          L.g_pa, d, m->eps, q_d);
            ATLAS_LAUNCH_CHECK("bd_residual_q_kernel");
            const size_t gstride = (size_t)B * m->dff;
            const BgemvOut og{w.g_part, gstride, m->dff}, ou{w.u_part, gstride, m->dff};
            const W4View wu = bview(L.up);
            if ((rc = launch_bgemv(bview(L.gate), L.gate.group, &wu, q_d, B, og, &ou, st, "bd_gemv_gate_up"))) return rc;
            prof_mark("bd_swiglu", st);
            ATLAS_KLAUNCH(bd_swiglu_q_kernel, dim3((unsigned)((q_ff.ldq / 8 + 255) / 256), B), dim3(256), 0, st,
                          w.g_part, w.u_part, p.sg, gstride, m->dff, q_ff);
            ATLAS_LAUNCH_CHECK("bd_swiglu_q_kernel");
            const BgemvOut od{w.a_part, (size_t)B * d, d};
            if ((rc = launch_bgemv(bview(L.down), L.down.group, nullptr, q_ff, B, od, nullptr, st, "bd_gemv_down")))
                return rc;
            prof_mark("bd_residual_norm", st);
            ATLAS_KLAUNCH(bd_residual_q_kernel, dim3(B), dim3(res_threads), 0, st, w.X, w.a_part, p.sd, (size_t)B * d,
                          L.g_pf, d, m->eps, q_d);
            ATLAS_LAUNCH_CHECK("bd_residual_q_kernel");
            continue;
        }
        if ((rc = launch_pf_split(w.o, B, nq, nq, w.p1h, w.p1l, w.ld1, st))) return rc;
        // o projection (split over K), h = x + RMSNorm_pa(a)
        GemmArgs oa = bgemm(w.p1h, w.p1l, w.ld1, L.o, B);
        oa.C = w.a_part;
        oa.ldc = d;
        oa.ksplit = p.so;
        oa.kchunk = nq / p.so;
        oa.c_split = (size_t)B * d;
        if ((rc = launch_w4_gemm(oa, 0, st, "bd_gemm_o"))) return rc;
        prof_mark("bd_residual_norm", st);
        ATLAS_KLAUNCH(bd_residual_kernel, dim3(B), dim3(1024), (size_t)d * 4, st, w.X, w.a_part, p.so, (size_t)B * d,
                      L.g_pa, d, m->eps, w.p1h, w.p1l, w.ld1);
        ATLAS_LAUNCH_CHECK("bd_residual_kernel");
        // gate/up with SwiGLU, then down (split over K), y = h + RMSNorm_pf(m)
        // gate and up as two split-K GEMMs into partials; SwiGLU sums them
        const size_t gstride = (size_t)B * m->dff;
        for (int which = 0; which < 2; which++) {
            GemmArgs ga = bgemm(w.p1h, w.p1l, w.ld1, which ? L.up : L.gate, B);
            ga.C = which ? w.u_part : w.g_part;
            ga.ldc = m->dff;
            ga.ksplit = p.sg;
            ga.kchunk = d / p.sg;
            ga.c_split = gstride;
            if ((rc = launch_w4_gemm(ga, 0, st, which ? "bd_gemm_up" : "bd_gemm_gate"))) return rc;
        }
        prof_mark("bd_swiglu", st);
        ATLAS_KLAUNCH(bd_swiglu_kernel, dim3((unsigned)((gstride + 255) / 256)), dim3(256), 0, st, w.g_part, w.u_part,
                      p.sg, gstride, (int)gstride, w.p2h, w.p2l);
        ATLAS_LAUNCH_CHECK("bd_swiglu_kernel");
        GemmArgs da = bgemm(w.p2h, w.p2l, m->dff, L.down, B);
        da.C = w.a_part;
        da.ldc = d;
        da.ksplit = p.sd;
        da.kchunk = m->dff / p.sd;
        da.c_split = (size_t)B * d;
        if ((rc = launch_w4_gemm(da, 0, st, "bd_gemm_down"))) return rc;
        prof_mark("bd_residual_norm", st);
        ATLAS_KLAUNCH(bd_residual_kernel, dim3(B), dim3(1024), (size_t)d * 4, st, w.X, w.a_part, p.sd, (size_t)B * d,
                      L.g_pf, d, m->eps, w.p1h, w.p1l, w.ld1);
        ATLAS_LAUNCH_CHECK("bd_residual_kernel");
    }
    if (d_hidden_out) {
        rc = hipMemcpyAsync(d_hidden_out, w.X, (size_t)B * d * 4, hipMemcpyDeviceToDevice, st) == hipSuccess
                 ? ATLAS_OK
                 : fail(ATLAS_ERR_HIP, "hidden copy failed");
        if (rc) return rc;
    }
    if (!head) return ATLAS_OK;
    prof_mark("bd_final_norm", st);
    ATLAS_KLAUNCH(bd_final_norm_kernel, dim3(B), dim3(1024), 0, st, w.X, m->g_final, d, m->eps, w.p1h, w.p1l, w.ld1);
    ATLAS_LAUNCH_CHECK("bd_final_norm_kernel");
    float* logits = d_logits ? d_logits : w.logits;
    const int head_blocks = (m->vocab + 16 * BD_HEAD_TILES * BD_HEAD_WAVES - 1) / (16 * BD_HEAD_TILES * BD_HEAD_WAVES);
    prof_mark("bd_lm_head", st);
    if ((d / 64) % BD_HEAD_AHEAD == 0)
        ATLAS_KLAUNCH(bd_head_kernel<true>, dim3(head_blocks), dim3(64 * BD_HEAD_WAVES), 0, st, w.p1h, w.p1l, w.ld1, B,
                      m->lm_head, m->vocab, d, logits);
    else
        ATLAS_KLAUNCH(bd_head_kernel<false>, dim3(head_blocks), dim3(64 * BD_HEAD_WAVES), 0, st, w.p1h, w.p1l, w.ld1, B,
                      m->lm_head, m->vocab, d, logits);
    ATLAS_LAUNCH_CHECK("bd_head_kernel");
    if (d_argmax) {
        prof_mark("bd_argmax", st);
        ATLAS_KLAUNCH(bd_argmax_rows_kernel, dim3(B), dim3(1024), 0, st, logits, m->vocab, d_argmax);
        ATLAS_LAUNCH_CHECK("bd_argmax_rows_kernel");
    }
    return ATLAS_OK;
}
