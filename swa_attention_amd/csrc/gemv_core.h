// Device-side streaming core of the integer-dot W4 GEMV (see common.h for the
// activation encoding). Shared by the standalone GEMV and the fused decode kernels.
//
// Decomposition. A block owns one reduction range of CW 32-column chunks (the
// encoded x of that range sits in LDS) and a contiguous range of row tiles. A tile
// is RB rows. Inside a tile, lane l owns the CPL "virtual chunks" vc = l + 64 j
// (j < CPL): row vc / CW of the tile and chunk vc % CW of the range
// (RB * CW <= 64 * CPL). A lane's chunks are the same for every tile, so its slice
// of the encoded x is loaded from LDS into registers once and the wave then only
// streams weights: one 16-byte load, one scale and one zero word per chunk and row.
// Waves take every NWAVE-th tile of the block; loads of the next tile are issued
// before the current one is reduced (two register stages).
#pragma once
#include "common.h"

namespace atlas {

struct W4View {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint32_t* zeros;   // never null: without a zero table it aliases qweight
    int zsym;                // 1: no zero table, zero point 8 for every group
    int zstride;             // words per row of the zero table (0 when aliased)
    int N, K, G, GW, KW, scale_dtype;
};

// Without a zero table the zero-word loads read word g/8 < K/8 of qweight's first
// row (always in bounds) and the result is replaced by the symmetric zero point, so
// tile loads carry no branch.
__host__ __device__ inline W4View w4_view(const uint32_t* q, const uint16_t* s, const uint32_t* z, int N, int K,
                                          int group, int sd) {
    W4View v;
    v.qweight = q;
    v.scales = s;
    v.zsym = z == nullptr;
    v.zeros = z ? z : q;
    v.N = N;
    v.K = K;
    v.G = (K + group - 1) / group;
    v.GW = (v.G + 7) / 8;
    v.zstride = z ? v.GW : 0;
    v.KW = K / 8;
    v.scale_dtype = sd;
    return v;
}

template <int CPL, int RB>
struct LaneMap {
    int rt[CPL];      // row within the tile
    int ch[CPL];      // global chunk index
    int gi[CPL];      // group index of the chunk
    bool valid[CPL];

    __device__ void init(int lane, int C0, int CW, int group) {
#pragma unroll
        for (int j = 0; j < CPL; j++) {
            const int vc = lane + 64 * j;
            valid[j] = vc < RB * CW;
            rt[j] = valid[j] ? vc / CW : 0;
            ch[j] = C0 + (valid[j] ? vc % CW : 0);
            gi[j] = ch[j] * XQ_CHUNK / group;
        }
    }
};

template <int CPL>
struct LanePlanes {
    uint32_t pl[CPL][XQ_WORDS_PER_CHUNK];
    float qs[CPL];
    float icf[CPL];

    // from an LDS copy of the range: planes [CW][24], qs [CW], isum [CW]
    template <int RB>
    __device__ void load(const LaneMap<CPL, RB>& m, const uint32_t* s_pl, const float* s_qs, const int* s_is,
                         int C0) {
#pragma unroll
        for (int j = 0; j < CPL; j++) {
            const int c = m.ch[j] - C0;
            const uint4* s4 = reinterpret_cast<const uint4*>(s_pl + c * XQ_WORDS_PER_CHUNK);
#pragma unroll
            for (int q = 0; q < XQ_WORDS_PER_CHUNK / 4; q++) {
                const uint4 v = s4[q];
                pl[j][4 * q + 0] = v.x;
                pl[j][4 * q + 1] = v.y;
                pl[j][4 * q + 2] = v.z;
                pl[j][4 * q + 3] = v.w;
            }
            qs[j] = m.valid[j] ? s_qs[c] : 0.f;
            icf[j] = (float)s_is[c];
        }
    }
};

template <int CPL>
struct TileRegs {
    uint4 w[CPL];
    uint32_t zw[CPL];
    uint16_t sb[CPL];
};

// Branch-free: rows past N are clamped (their sums are never stored) and invalid lane
// items read chunk C0 (their contribution is zeroed through qs = 0). Weights are read
// once per step, so they are loaded non-temporally (streaming cache policy) and do not
// push the activations and partial sums out of L2.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <int CPL, int RB>
__device__ __forceinline__ void load_tile(TileRegs<CPL>& T, const W4View& W, const LaneMap<CPL, RB>& m, int row0) {
#pragma unroll
    for (int j = 0; j < CPL; j++) {
        const size_t rr = (size_t)min(row0 + m.rt[j], W.N - 1);
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W.qweight + rr * W.KW) + m.ch[j]);
        T.w[j] = make_uint4(v.x, v.y, v.z, v.w);
        T.sb[j] = __builtin_nontemporal_load(W.scales + rr * W.G + m.gi[j]);
        T.zw[j] = __builtin_nontemporal_load(W.zeros + rr * W.zstride + (m.gi[j] >> 3));   // raw: used in tile_dot
    }
}

// Per-lane partial sums of the RB rows of a tile.
template <int CPL, int RB>
__device__ __forceinline__ void tile_dot(const TileRegs<CPL>& T, const LanePlanes<CPL>& P, const LaneMap<CPL, RB>& m,
                                         const W4View& W, float acc[RB]) {
#pragma unroll
    for (int r = 0; r < RB; r++) acc[r] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; j++) {
        int D[XQ_PLANES] = {0, 0, 0, 0, 0, 0};
        const uint32_t wq[4] = {T.w[j].x, T.w[j].y, T.w[j].z, T.w[j].w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int u = (int)(wq[q] ^ 0x88888888u);
#pragma unroll
            for (int p = 0; p < XQ_PLANES; p++)
                D[p] = __builtin_amdgcn_sdot8(u, (int)P.pl[j][q * XQ_PLANES + p], D[p], false);
        }
        const int E0 = D[0] + (D[1] << 4) + (D[2] << 8);
        const int E1 = D[3] + (D[4] << 4) + (D[5] << 8);
        const float f = fmaf(4096.f, (float)E1, (float)E0);
        const int z = W.zsym ? 8 : (int)((T.zw[j] >> ((m.gi[j] & 7) * 4)) & 15u);
        const float tt = fmaf((float)(8 - z), P.icf[j], f);
        const float c = scale_to_f32(T.sb[j], W.scale_dtype) * P.qs[j] * tt;
        if (RB == 1) {
            acc[0] += c;
        } else {
#pragma unroll
            for (int r = 0; r < RB; r++) acc[r] += (m.rt[j] == r) ? c : 0.f;
        }
    }
}

// Copy of an encoded range (chunks [C0, C0+CW)) from global memory into LDS, staged
// through registers: planes_issue() issues every load (callers do so before their
// weight prefetch, since loads complete in issue order), planes_commit() stores them.
// Needs blockDim.x == NT, CW * 6 <= PLANE_REGS * NT and CW <= NT.
constexpr int PLANE_REGS = 5;
struct PlaneStage {
    uint4 v[PLANE_REGS];
    float qs;
    int is;
};

template <int NT>
__device__ __forceinline__ void planes_issue(const XQ& xq, int C0, int CW, PlaneStage& S) {
    const uint4* src = reinterpret_cast<const uint4*>(xq.planes + (size_t)C0 * XQ_WORDS_PER_CHUNK);
    const int n = CW * XQ_WORDS_PER_CHUNK / 4;
#pragma unroll
    for (int j = 0; j < PLANE_REGS; j++) {
        const int i = (int)threadIdx.x + j * NT;
        S.v[j] = src[i < n ? i : 0];
    }
    const int c = (int)threadIdx.x < CW ? (int)threadIdx.x : 0;
    S.qs = xq.qs[C0 + c];
    S.is = xq.isum[C0 + c];
}

template <int NT>
__device__ __forceinline__ void planes_commit(const PlaneStage& S, int CW, uint32_t* s_pl, float* s_qs, int* s_is) {
    const int n = CW * XQ_WORDS_PER_CHUNK / 4;
    uint4* dst = reinterpret_cast<uint4*>(s_pl);
    const uint4 v0 = S.v[0], v1 = S.v[1], v2 = S.v[2], v3 = S.v[3], v4 = S.v[4];
    const int i = (int)threadIdx.x;
    if (i < n) dst[i] = v0;
    if (i + NT < n) dst[i + NT] = v1;
    if (i + 2 * NT < n) dst[i + 2 * NT] = v2;
    if (i + 3 * NT < n) dst[i + 3 * NT] = v3;
    if (i + 4 * NT < n) dst[i + 4 * NT] = v4;
    if (i < CW) {
        s_qs[i] = S.qs;
        s_is[i] = S.is;
    }
}
static_assert(PLANE_REGS == 5, "planes_commit stores five registers");

// Encode `n` floats held in LDS (n % 32 == 0) into LDS planes; all threads of the
// block call it (quads of lanes form a chunk).
__device__ __forceinline__ void encode_lds(const float* s_x, int n, uint32_t* s_pl, float* s_qs, int* s_is) {
    XQ o;
    o.planes = s_pl;
    o.qs = s_qs;
    o.isum = s_is;
    const int nwords = n / 8;
    for (int base = 0; base < nwords; base += blockDim.x) {
        const int t = base + threadIdx.x;
        if (t < nwords) {   // whole quads are inside or outside (nwords % 4 == 0, blockDim % 64 == 0)
            float x8[8];
            const float4* p = reinterpret_cast<const float4*>(s_x + 8 * t);
            const float4 a = p[0], b = p[1];
            x8[0] = a.x; x8[1] = a.y; x8[2] = a.z; x8[3] = a.w;
            x8[4] = b.x; x8[5] = b.y; x8[6] = b.z; x8[7] = b.w;
            xq_encode_word(x8, o, t >> 2, t & 3);
        }
    }
}

// LDS bytes of an encoded range of CW chunks.
__host__ __device__ inline size_t planes_lds_bytes(int CW) { return (size_t)CW * (XQ_WORDS_PER_CHUNK * 4 + 8); }

}  // namespace atlas
