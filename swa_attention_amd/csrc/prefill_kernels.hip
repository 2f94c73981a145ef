// Prefill of a whole prompt on the matrix cores.
//
// Source: "ATLAS-OLMo-3-32B-Think-v4" -- Limitations & roadmap (prefill defined as the
// prompt run through the decode path token by token; the planned fix is a batched,
// tiled GEMM prefill) and the layer definition of the decode path (Architecture
// deep-dive; Quantization recipe). Every position t of the prompt computes exactly
// what the decode step computes at pos = start_pos + t; here the n positions of a
// layer are processed together:
//   - the four W4 projections are GEMMs on MFMA (v_mfma_f32_16x16x32_bf16): each
//     block dequantises one quantisation group of a 128-row weight tile into LDS as
//     exact small integers (code - zero) in bf16, multiplies it with the activations
//     held as two bf16 planes (x = hi + lo carries 16 significant bits, so the
//     products match f32 inputs to about 2^-17), accumulates the group in f32 and
//     adds it to the output scaled by the group's scale;
//   - QK RMSNorm, rotary embedding and the KV write run one block per position;
//   - causal (windowed) GQA attention runs per (16 positions, KV head) with the
//     query heads of the group in separate waves, on bf16 MFMA with hi/lo operands
//     (hi*hi + hi*lo + lo*hi: about 2^-16 relative per product);
//   - the post-attention and post-MLP residual norms run one block per position.
#include "prefill_kernels.h"

namespace atlas {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short bf16x4_t __attribute__((ext_vector_type(4)));   // four bf16 (operand of the 16x16x16 MFMA)

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) (x - hi is exact in f32)
__device__ __forceinline__ void pf_split(float x, uint32_t& hi, uint32_t& lo) {
    hi = f32_to_bf16_rne_finite(x);
    lo = f32_to_bf16_rne_finite(x - __uint_as_float(hi << 16));
}

// Store 4 consecutive values of a row as bf16 planes.
__device__ __forceinline__ void store_split4(const float4 v, uint16_t* hi, uint16_t* lo) {
    uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
    pf_split(v.x, h0, l0);
    pf_split(v.y, h1, l1);
    pf_split(v.z, h2, l2);
    pf_split(v.w, h3, l3);
    *reinterpret_cast<uint2*>(hi) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
    *reinterpret_cast<uint2*>(lo) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
}

// ---- W4 GEMM ------------------------------------------------------------------------------
//
// Block tile 64 (rows of A) x 128 (rows of W; mode 1: 64 of W0 and the same 64 of W1),
// four waves of 32 x 64, k tiles of 64 through LDS. The products of one quantisation
// group are accumulated on their own and added to the output times the group's
// scale (per row of W) when the group ends; groups are multiples of 32 columns, so
// every MFMA k-step of 32 lies in one group. The next k tile's A planes and codes are
// loaded into registers while the current one is multiplied. Tiles are numbered so
// that consecutive tile numbers land on one XCD (blocks are dealt to the 8 XCDs
// round robin) with the row tiles of A fastest: the tiles sharing a weight tile run
// together on one XCD's L2.

constexpr int GM_BM = 64, GM_BN = 128, GM_BK = 64, GM_THREADS = 256;

template <int MODE>
__global__ __launch_bounds__(GM_THREADS) void w4_gemm_kernel(GemmArgs a) {
    constexpr int LDK = GM_BK + 8;                   // padded LDS row (bf16)
    constexpr int A_PER = GM_BM * GM_BK / 8 / GM_THREADS;   // uint4 per thread and plane: 2
    static_assert(GM_BN * GM_BK / 32 == GM_THREADS, "one uint4 of codes per thread");
    __shared__ __align__(16) uint16_t sAh[GM_BM * LDK];
    __shared__ __align__(16) uint16_t sAl[GM_BM * LDK];
    __shared__ __align__(16) uint16_t sB[GM_BN * LDK];
    __shared__ float sS[2][GM_BN];

    const int MT = (a.M + GM_BM - 1) / GM_BM;
    const int NW_ = MODE ? GM_BN / 2 : GM_BN;   // output columns per tile
    const int NT = (a.N + NW_ - 1) / NW_;
    const int T = MT * NT, Wk = T * a.ksplit, per = (Wk + 7) / 8;
    const int Lw = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (Lw >= Wk) return;
    const int L = Lw % T, split = Lw / T;
    const int k_lo = split * a.kchunk, k_hi = a.ksplit > 1 ? k_lo + a.kchunk : a.K;
    const int m0 = (L % MT) * GM_BM, n0 = (L / MT) * NW_;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int l16 = lane & 15, l4 = lane >> 4;
    const int KT = (k_hi - k_lo + GM_BK - 1) / GM_BK;

    // weight-tile row r -> matrix (second one for r >= 64 in mode 1) and row (clamped to N - 1)
    auto second = [&](int r) { return MODE && r >= GM_BN / 2; };
    auto wrow = [&](int r) { return min(n0 + (second(r) ? r - GM_BN / 2 : r), a.N - 1); };
    // tile-local W row of N fragment nf of this wave
    auto bcol = [&](int nf) { return MODE ? (nf < 2 ? wn * 32 + 16 * nf : 64 + wn * 32 + 16 * (nf - 2)) : wn * 64 + 16 * nf; };

    // this thread's uint4 of codes: W row br, 32 columns from bc
    const int br = tid / (GM_BK / 32), bc = 32 * (tid % (GM_BK / 32));
    const int brow = wrow(br);
    const uint32_t* b_q = second(br) ? a.W1.qweight : a.W0.qweight;   // both matrices share N, K, group
    const uint32_t* b_z = second(br) ? a.W1.zeros : a.W0.zeros;
    const int b_zstride = second(br) ? a.W1.zstride : a.W0.zstride;
    const int b_zsym = second(br) ? a.W1.zsym : a.W0.zsym;
    const int KW = a.W0.KW, GG = a.W0.G;
    // the two scale slots of a k tile (group 32: one per k-step; otherwise slot 0)
    const int srow = tid & (GM_BN - 1), sslot = tid / GM_BN;
    const uint16_t* s_p = (second(srow) ? a.W1.scales : a.W0.scales) + (size_t)wrow(srow) * GG;
    const int s_dtype = second(srow) ? a.W1.scale_dtype : a.W0.scale_dtype;

    uint4 rAh0, rAh1, rAl0, rAl1, rB;
    uint32_t rZ;
    uint16_t rS;
    static_assert(A_PER == 2, "two uint4 per thread and plane");
    // A row / column of this thread's two uint4 per plane
    const int ar0 = tid / (GM_BK / 8), ac0 = 8 * (tid % (GM_BK / 8));
    const int ar1 = (tid + GM_THREADS) / (GM_BK / 8), ac1 = 8 * ((tid + GM_THREADS) % (GM_BK / 8));
    const size_t arow0 = (size_t)min(m0 + ar0, a.M - 1) * a.lda, arow1 = (size_t)min(m0 + ar1, a.M - 1) * a.lda;
#define LOAD_TILE_K(kt_)                                                                                     \
    do {                                                                                                     \
        const int kb_ = k_lo + (kt_) * GM_BK;                                                                \
        const size_t o0_ = arow0 + min(kb_ + ac0, a.K - 8), o1_ = arow1 + min(kb_ + ac1, a.K - 8);           \
        rAh0 = *reinterpret_cast<const uint4*>(a.a_hi + o0_);                                                \
        rAl0 = *reinterpret_cast<const uint4*>(a.a_lo + o0_);                                                \
        rAh1 = *reinterpret_cast<const uint4*>(a.a_hi + o1_);                                                \
        rAl1 = *reinterpret_cast<const uint4*>(a.a_lo + o1_);                                                \
        const int kc_ = min(kb_ + bc, a.K - 32);                                                             \
        const u32x4_t v_ = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(b_q + (size_t)brow * KW + kc_ / 8)); \
        rB = make_uint4(v_.x, v_.y, v_.z, v_.w);                                                             \
        rZ = b_z[(size_t)brow * b_zstride + ((kc_ / a.group) >> 3)];                                         \
        rS = s_p[min((kb_ + 32 * sslot) / a.group, GG - 1)];                                                 \
    } while (0)

    f32x4_t acc[2][4], accg[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            accg[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

    LOAD_TILE_K(0);
    for (int kt = 0; kt < KT; kt++) {
        const int kb = k_lo + kt * GM_BK, kn = min(GM_BK, k_hi - kb);
        __syncthreads();   // the previous tile's fragments have been read
        *reinterpret_cast<uint4*>(&sAh[ar0 * LDK + ac0]) = rAh0;
        *reinterpret_cast<uint4*>(&sAl[ar0 * LDK + ac0]) = rAl0;
        *reinterpret_cast<uint4*>(&sAh[ar1 * LDK + ac1]) = rAh1;
        *reinterpret_cast<uint4*>(&sAl[ar1 * LDK + ac1]) = rAl1;
        {
            const int kc = min(kb + bc, a.K - 32);
            const int z = b_zsym ? 8 : (int)((rZ >> (((kc / a.group) & 7) * 4)) & 15u);
            const uint32_t w4[4] = {rB.x, rB.y, rB.z, rB.w};
            uint32_t o[16];
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    // (code - zero) is an integer in [-15, 15]: exact in bf16
                    const float v0 = (float)((int)((w4[q] >> (4 * e)) & 15u) - z);
                    const float v1 = (float)((int)((w4[q] >> (4 * e + 4)) & 15u) - z);
                    o[q * 4 + e / 2] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xFFFF0000u);
                }
            uint4* dst = reinterpret_cast<uint4*>(&sB[br * LDK + bc]);
#pragma unroll
            for (int q = 0; q < 4; q++) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        }
        sS[sslot][srow] = scale_to_f32(rS, s_dtype);
        __syncthreads();
        if (kt + 1 < KT) LOAD_TILE_K(kt + 1);   // in flight during the products below

        for (int ks = 0; ks < kn / 32; ks++) {
            const int k = ks * 32 + 8 * l4;
            bf16x8_t ah[2], al[2], b[4];
#pragma unroll
            for (int mf = 0; mf < 2; mf++) {
                const int row = wm * 32 + mf * 16 + l16;
                ah[mf] = *reinterpret_cast<const bf16x8_t*>(&sAh[row * LDK + k]);
                al[mf] = *reinterpret_cast<const bf16x8_t*>(&sAl[row * LDK + k]);
            }
#pragma unroll
            for (int nf = 0; nf < 4; nf++) b[nf] = *reinterpret_cast<const bf16x8_t*>(&sB[(bcol(nf) + l16) * LDK + k]);
#pragma unroll
            for (int mf = 0; mf < 2; mf++)
#pragma unroll
                for (int nf = 0; nf < 4; nf++) {
                    const f32x4_t c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[mf], b[nf], accg[mf][nf], 0, 0, 0);
                    accg[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[mf], b[nf], c, 0, 0, 0);
                }
            const int kabs = kb + 32 * ks + 32;
            if (kabs % a.group == 0 || kabs >= k_hi) {   // group ends: scale and add
                const int slot = a.group == 32 ? ks : 0;
#pragma unroll
                for (int nf = 0; nf < 4; nf++) {
                    const float s = sS[slot][bcol(nf) + l16];
#pragma unroll
                    for (int mf = 0; mf < 2; mf++) {
#pragma unroll
                        for (int r = 0; r < 4; r++) acc[mf][nf][r] = fmaf(s, accg[mf][nf][r], acc[mf][nf][r]);
                        accg[mf][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
        }
    }

    // epilogue: D[row 4*l4 + r][col l16] of each fragment
#pragma unroll
    for (int mf = 0; mf < 2; mf++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = m0 + wm * 32 + mf * 16 + 4 * l4 + r;
            if (row >= a.M) continue;
            if (MODE == 0) {
#pragma unroll
                for (int nf = 0; nf < 4; nf++) {
                    const int col = n0 + bcol(nf) + l16;
                    if (col < a.N) a.C[split * a.c_split + (size_t)row * a.ldc + col] = acc[mf][nf][r];
                }
            } else {
#pragma unroll
                for (int f = 0; f < 2; f++) {
                    const int col = n0 + wn * 32 + 16 * f + l16;
                    if (col < a.N) {
                        const float gt = acc[mf][f][r], up = acc[mf][f + 2][r];
                        uint32_t hi, lo;
                        pf_split(gt / (1.0f + __expf(-gt)) * up, hi, lo);
                        a.z_hi[(size_t)row * a.ldz + col] = (uint16_t)hi;
                        a.z_lo[(size_t)row * a.ldz + col] = (uint16_t)lo;
                    }
                }
            }
        }
#undef LOAD_TILE_K
}

// ---- W4 GEMM on the int8 matrix cores ---------------------------------------------------------
//
// The same product with v_mfma_i32_16x16x64_i8, which does twice the bf16 rate's work per
// instruction. A is a 24-bit fixed-point copy per row and quantisation group (A ~ s v,
// v = 65536 h + 256 m + l, the digits as three int8 planes, see pf_quant8_kernel); the
// weights enter as their raw 4-bit codes c in [0, 15] (a mask and a shift per word: the
// low nibbles of a word are its columns 0,2,4,6 and the high nibbles 1,3,5,7, the byte
// order of the A planes). Per group each digit plane's products are exact in int32;
//   I = 65536 sum(c h) + 256 sum(c m) + sum(c l) - z sum(v)
// is formed in f32 (about 2^-24 of its terms) and added to the output times s_w s_x. The tile is 64 rows of A x 128 rows of W
// (mode 1: 64 of W0 and the same 64 of W1), four waves of 32 x 64, k tiles of 128 through
// LDS (groups are multiples of 128), the next k tile in registers while the current one
// is multiplied, tiles numbered XCD by XCD as in w4_gemm_kernel.
constexpr int G8_BM = 64, G8_BN = 128, G8_BK = 128, G8_THREADS = 256;
static_assert(G8_BM == GM_BM && G8_BN == GM_BN, "the launcher counts tiles of both kernels alike");
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ __launch_bounds__(G8_THREADS) void w4_gemm_i8_kernel(GemmArgs a) {
    constexpr int LDB = G8_BK + 16;   // padded LDS row in bytes
    __shared__ __align__(16) int8_t sAh[G8_BM * LDB];
    __shared__ __align__(16) int8_t sAm[G8_BM * LDB];
    __shared__ __align__(16) int8_t sAl[G8_BM * LDB];
    __shared__ __align__(16) int8_t sB[G8_BN * LDB];
    __shared__ float sSw[G8_BN];
    __shared__ int sZ[G8_BN];
    __shared__ float sSx[G8_BM];
    __shared__ float sSX[G8_BM];

    const int MT = (a.M + G8_BM - 1) / G8_BM;
    const int NW_ = MODE ? G8_BN / 2 : G8_BN;   // output columns per tile
    const int NT = (a.N + NW_ - 1) / NW_;
    const int T = MT * NT, Wk = T * a.ksplit, per = (Wk + 7) / 8;
    const int Lw = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (Lw >= Wk) return;
    const int L = Lw % T, split = Lw / T;
    const int k_lo = split * a.kchunk, k_hi = a.ksplit > 1 ? k_lo + a.kchunk : a.K;
    const int m0 = (L % MT) * G8_BM, n0 = (L / MT) * NW_;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int l16 = lane & 15, l4 = lane >> 4;
    const int KT = (k_hi - k_lo) / G8_BK;

    auto second = [&](int r) { return MODE && r >= G8_BN / 2; };
    auto wrow = [&](int r) { return min(n0 + (second(r) ? r - G8_BN / 2 : r), a.N - 1); };
    auto bcol = [&](int nf) { return MODE ? (nf < 2 ? wn * 32 + 16 * nf : 64 + wn * 32 + 16 * (nf - 2)) : wn * 64 + 16 * nf; };

    // codes: thread t -> W row t/2, 64 columns from 64 (t % 2)
    const int br = tid >> 1, bc = 64 * (tid & 1);
    const uint32_t* b_q = (second(br) ? a.W1.qweight : a.W0.qweight) + (size_t)wrow(br) * a.W0.KW + bc / 8;
    // the group's scale (threads < 128, W row t) or zero (threads >= 128, W row t - 128)
    const int srow = tid & (G8_BN - 1);
    const bool zthread = tid >= G8_BN;
    const W4View& Ws = second(srow) ? a.W1 : a.W0;
    const uint16_t* s_p = Ws.scales + (size_t)wrow(srow) * Ws.G;
    const uint32_t* z_p = Ws.zeros + (size_t)wrow(srow) * Ws.zstride;
    const int s_dtype = Ws.scale_dtype, zsym = Ws.zsym;
    // A digits: thread t -> rows t/8 and t/8 + 32, 16 bytes from 16 (t % 8) of each plane
    const int ar = tid >> 3, ac = 16 * (tid & 7);
    const size_t ao0 = (size_t)min(m0 + ar, a.M - 1) * a.ldq + ac;
    const size_t ao1 = (size_t)min(m0 + ar + 32, a.M - 1) * a.ldq + ac;
    const size_t qo = (size_t)min(m0 + (tid & (G8_BM - 1)), a.M - 1) * a.ldqs;

    uint4 rAh0, rAh1, rAm0, rAm1, rAl0, rAl1, rB0, rB1;
    uint32_t rZ;
    uint16_t rS;
    float rSx, rSX;
    auto load_k = [&](int kt) {
        const int kb = k_lo + kt * G8_BK, g = kb / a.group;
        rAh0 = *reinterpret_cast<const uint4*>(a.q_hi + ao0 + kb);
        rAh1 = *reinterpret_cast<const uint4*>(a.q_hi + ao1 + kb);
        rAm0 = *reinterpret_cast<const uint4*>(a.q_mid + ao0 + kb);
        rAm1 = *reinterpret_cast<const uint4*>(a.q_mid + ao1 + kb);
        rAl0 = *reinterpret_cast<const uint4*>(a.q_lo + ao0 + kb);
        rAl1 = *reinterpret_cast<const uint4*>(a.q_lo + ao1 + kb);
        const u32x4_t* bp = reinterpret_cast<const u32x4_t*>(b_q + kb / 8);
        const u32x4_t v0 = __builtin_nontemporal_load(bp), v1 = __builtin_nontemporal_load(bp + 1);
        rB0 = make_uint4(v0.x, v0.y, v0.z, v0.w);
        rB1 = make_uint4(v1.x, v1.y, v1.z, v1.w);
        rS = s_p[g];
        rZ = z_p[g >> 3];
        rSx = a.q_s[qo + g];
        rSX = a.q_sum[qo + g];
    };

    f32x4_t acc[2][4];
    i32x4_t ah_acc[2][4], am_acc[2][4], al_acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            ah_acc[i][j] = i32x4_t{0, 0, 0, 0};
            am_acc[i][j] = i32x4_t{0, 0, 0, 0};
            al_acc[i][j] = i32x4_t{0, 0, 0, 0};
        }

    load_k(0);
    for (int kt = 0; kt < KT; kt++) {
        const int kb = k_lo + kt * G8_BK;
        __syncthreads();   // the previous tile's fragments have been read
        *reinterpret_cast<uint4*>(&sAh[ar * LDB + ac]) = rAh0;
        *reinterpret_cast<uint4*>(&sAh[(ar + 32) * LDB + ac]) = rAh1;
        *reinterpret_cast<uint4*>(&sAm[ar * LDB + ac]) = rAm0;
        *reinterpret_cast<uint4*>(&sAm[(ar + 32) * LDB + ac]) = rAm1;
        *reinterpret_cast<uint4*>(&sAl[ar * LDB + ac]) = rAl0;
        *reinterpret_cast<uint4*>(&sAl[(ar + 32) * LDB + ac]) = rAl1;
        {
            const uint32_t w[8] = {rB0.x, rB0.y, rB0.z, rB0.w, rB1.x, rB1.y, rB1.z, rB1.w};
            uint4* dst = reinterpret_cast<uint4*>(&sB[br * LDB + bc]);
#pragma unroll
            for (int q = 0; q < 4; q++)
                dst[q] = make_uint4(w[2 * q] & 0x0F0F0F0Fu, (w[2 * q] >> 4) & 0x0F0F0F0Fu, w[2 * q + 1] & 0x0F0F0F0Fu,
                                    (w[2 * q + 1] >> 4) & 0x0F0F0F0Fu);
        }
        if (zthread) sZ[srow] = zsym ? 8 : (int)((rZ >> (((kb / a.group) & 7) * 4)) & 15u);
        else sSw[srow] = scale_to_f32(rS, s_dtype);
        if (tid < G8_BM) {
            sSx[tid] = rSx;
            sSX[tid] = rSX;
        }
        __syncthreads();
        if (kt + 1 < KT) load_k(kt + 1);   // in flight during the products below

#pragma unroll
        for (int ks = 0; ks < G8_BK / 64; ks++) {
            const int k = ks * 64 + 16 * l4;
            i32x4_t ah[2], am[2], al[2], b[4];
#pragma unroll
            for (int mf = 0; mf < 2; mf++) {
                const int row = wm * 32 + mf * 16 + l16;
                ah[mf] = *reinterpret_cast<const i32x4_t*>(&sAh[row * LDB + k]);
                am[mf] = *reinterpret_cast<const i32x4_t*>(&sAm[row * LDB + k]);
                al[mf] = *reinterpret_cast<const i32x4_t*>(&sAl[row * LDB + k]);
            }
#pragma unroll
            for (int nf = 0; nf < 4; nf++) b[nf] = *reinterpret_cast<const i32x4_t*>(&sB[(bcol(nf) + l16) * LDB + k]);
#pragma unroll
            for (int mf = 0; mf < 2; mf++)
#pragma unroll
                for (int nf = 0; nf < 4; nf++) {
                    ah_acc[mf][nf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[mf], b[nf], ah_acc[mf][nf], 0, 0, 0);
                    am_acc[mf][nf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(am[mf], b[nf], am_acc[mf][nf], 0, 0, 0);
                    al_acc[mf][nf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al[mf], b[nf], al_acc[mf][nf], 0, 0, 0);
                }
        }
        if ((kb + G8_BK) % a.group == 0) {   // group ends: combine the digit sums, scale and add
#pragma unroll
            for (int nf = 0; nf < 4; nf++) {
                const int n = bcol(nf) + l16;
                const float sw = sSw[n];
                const int z = sZ[n];
#pragma unroll
                for (int mf = 0; mf < 2; mf++) {
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int m = wm * 32 + mf * 16 + 4 * l4 + r;
                        const float I = fmaf(65536.f, (float)ah_acc[mf][nf][r],
                                             fmaf(256.f, (float)am_acc[mf][nf][r], (float)al_acc[mf][nf][r])) -
                                        (float)z * sSX[m];
                        acc[mf][nf][r] = fmaf(I, sw * sSx[m], acc[mf][nf][r]);
                    }
                    ah_acc[mf][nf] = i32x4_t{0, 0, 0, 0};
                    am_acc[mf][nf] = i32x4_t{0, 0, 0, 0};
                    al_acc[mf][nf] = i32x4_t{0, 0, 0, 0};
                }
            }
        }
    }

    // epilogue: D[row 4*l4 + r][col l16] of each fragment
#pragma unroll
    for (int mf = 0; mf < 2; mf++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = m0 + wm * 32 + mf * 16 + 4 * l4 + r;
            if (row >= a.M) continue;
            if (MODE == 0) {
#pragma unroll
                for (int nf = 0; nf < 4; nf++) {
                    const int col = n0 + bcol(nf) + l16;
                    if (col < a.N) a.C[split * a.c_split + (size_t)row * a.ldc + col] = acc[mf][nf][r];
                }
            } else {
#pragma unroll
                for (int f = 0; f < 2; f++) {
                    const int col = n0 + wn * 32 + 16 * f + l16;
                    if (col < a.N) {
                        const float gt = acc[mf][f][r], up = acc[mf][f + 2][r];
                        uint32_t hi, lo;
                        pf_split(gt / (1.0f + __expf(-gt)) * up, hi, lo);
                        a.z_hi[(size_t)row * a.ldz + col] = (uint16_t)hi;
                        a.z_lo[(size_t)row * a.ldz + col] = (uint16_t)lo;
                    }
                }
            }
        }
}

// Largest 24-bit activation integer of the int8 path: 127 * 65536 (see pf_quant8_kernel).
constexpr float Q8_MAX = 8323072.f;

// ---- the int8 GEMM with a ring of LDS stages filled by direct-to-LDS loads ------------------
//
// The same product as w4_gemm_i8_kernel on a 64 x 256 tile (mode 1: 128 rows of W0 and the
// same 128 of W1) with eight waves of 32 x 64, k tiles of 128. Everything a k tile needs
// (the three A digit planes, the raw 4-bit codes, and per row the scale word, the zero
// word, q_s and q_sum of the tile's group) is copied from global memory straight into one
// of GR_STAGES LDS stages by global_load_lds (16 bytes per lane for the planes and codes, 4
// for the rest): the copies need no registers, so two k tiles stay in flight while a
// third is multiplied. Each wave waits (vmcnt) for its own copies of the tile about to be
// used and a block barrier publishes them. The copies are issued from inline assembly,
// which the compiler does not count; the loop issues no other vector-memory loads, so
// the waits written here are exact. The codes are unpacked per MFMA fragment (a mask and
// a shift per word) after their LDS read.
constexpr int GR_BM = 64, GR_BN = 256, GR_BK = 128, GR_THREADS = 512, GR_STAGES = 3;
constexpr int GR_A_PLANE = GR_BM * GR_BK;                  // bytes of one digit plane per stage
constexpr int GR_A_BYTES = 3 * GR_A_PLANE;                 // 24,576
constexpr int GR_B_BYTES = GR_BN * GR_BK / 2;              // 16,384: 4-bit codes
constexpr int GR_SMALL = 2 * 4 * GR_BN + 2 * 4 * GR_BM;   // scale and zero words per W row, q_s and q_sum per A row
constexpr int GR_STAGE = GR_A_BYTES + GR_B_BYTES + GR_SMALL;  // 43,520
constexpr size_t GR_LDS = (size_t)GR_STAGES * GR_STAGE;       // 130,560
// copies per stage and wave: A 24 and B 16 instructions of 1 KB over the 8 waves (3 and 2
// each); the 10 small ones of 256 B (4 scale, 4 zero, q_s, q_sum) by waves 0-4, 2 each
constexpr int GR_COPIES_BIG = 5, GR_COPIES_SMALL = 2;

// 16 bytes per lane from g into LDS at lds (wave-uniform byte address) + 16 * lane. The
// copies take their LDS address from m0, which each statement sets itself; m0 cannot be
// declared clobbered in inline assembly, so the kernel that uses these must not rely on m0
// anywhere else (w4_gemm_i8r_kernel does not: its code has no other m0 access). The
// compiler's own global_load_lds would be waited for with vmcnt(0) before every LDS read,
// which empties the ring; it is used for that reason only through these statements.
__device__ __forceinline__ void gr_copy16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}
// 4 bytes per lane from g into LDS at lds + 4 * lane
__device__ __forceinline__ void gr_copy4(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory");
}
// LDS byte offset of 16-byte chunk c of row r in a plane of 128-byte rows (XOR swizzle
// over the eight chunks of a row, so that the 16 rows of an MFMA fragment read spread
// over the banks)
__device__ __forceinline__ int gr_a_off(int r, int c) { return r * GR_BK + ((c ^ (r & 7)) << 4); }
// the same for the 64-byte code rows of B (four chunks)
__device__ __forceinline__ int gr_b_off(int r, int c) { return r * (GR_BK / 2) + ((c ^ ((r >> 1) & 3)) << 4); }

// G128: the group is one k tile (128 columns), so every tile starts and ends a group and the
// epilogue is straight-line code the compiler can interleave with the MFMAs.
// Mode-1 epilogue with groups of 128 (the tile's 128 z columns are one group of every row):
// z = silu(gate) * up, split into bf16 planes and summed back (z' = hi + lo, the value
// pf_quant8_kernel reads from the planes), then quantised to the down projection's int8
// digits exactly as pf_quant8_kernel does: the row's group maximum gives the power of two
// s, v = rint(z' / s) clamped to Q8_MAX, digits v = 65536 h + 256 m + l, and per row the
// group's s and its sum of v (an exact int32 for 128 columns). A row's 32 columns of a
// wave sit in one 16-lane row (two per lane): DPP row reductions, then the four column
// waves meet in LDS. The digits are staged in LDS in their stored order (bytes of every
// 8 columns as 0,2,4,6,1,3,5,7; rows padded to 144 bytes against bank conflicts) and
// leave as 16-byte stores. The staging uses the ring stage `free_stage`, which no wave
// reads any more, so the first barrier is the one that publishes the maxima. Every
// thread of the block runs it (rows past M are computed and not stored).
constexpr int GR_ZROW = 144;   // LDS bytes per staged digit row
__device__ __forceinline__ int dpp_row16_sum_i(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);    // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);    // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true);   // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, true);   // row_mirror
    return v;
}
__device__ __forceinline__ float dpp_row16_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return v;
}
__device__ __forceinline__ void gr_swiglu_digits(const GemmArgs& a, const f32x4_t (&acc)[2][4], int8_t* lds, int m0,
                                                 int n0, int wm, int wn, int l16, int l4, int tid) {
    float zx[2][2][4];
#pragma unroll
    for (int mf = 0; mf < 2; mf++)
#pragma unroll
        for (int f = 0; f < 2; f++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float gt = acc[mf][f][r], up = acc[mf][f + 2][r];
                uint32_t hi, lo;
                pf_split(gt / (1.0f + __expf(-gt)) * up, hi, lo);
                zx[mf][f][r] = bf16_bits_to_f32(hi) + bf16_bits_to_f32(lo);
            }
    float* s_max = reinterpret_cast<float*>(lds);       // [64 rows][4 column waves]
    int* s_sum = reinterpret_cast<int*>(lds + 1024);    // [64][4]
    int8_t* s_dig = lds + 2048;                          // [3 planes][64 rows][GR_ZROW]
    constexpr int PL = 64 * GR_ZROW;
#pragma unroll
    for (int mf = 0; mf < 2; mf++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float mx = dpp_row16_max(fmaxf(fabsf(zx[mf][0][r]), fabsf(zx[mf][1][r])));
            if (l16 == 0) s_max[(wm * 32 + mf * 16 + 4 * l4 + r) * 4 + wn] = mx;
        }
    __syncthreads();
#pragma unroll
    for (int mf = 0; mf < 2; mf++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int rl = wm * 32 + mf * 16 + 4 * l4 + r;
            const float mx = fmaxf(fmaxf(s_max[rl * 4], s_max[rl * 4 + 1]), fmaxf(s_max[rl * 4 + 2], s_max[rl * 4 + 3]));
            int e;
            (void)frexpf(mx / Q8_MAX, &e);   // s = 2^e >= max|z'| / Q8_MAX (s = 1 for a zero group)
            const float inv = ldexpf(1.f, -e);
            int sum = 0;
#pragma unroll
            for (int f = 0; f < 2; f++) {
                const int v = (int)fminf(fmaxf(rintf(zx[mf][f][r] * inv), -Q8_MAX), Q8_MAX);
                sum += v;
                const int ld = ((v + 128) & 255) - 128;
                const int v1 = (v - ld) >> 8;   // exact: v - ld is a multiple of 256
                const int md = ((v1 + 128) & 255) - 128;
                const int hd = (v1 - md) >> 8;
                const int c = wn * 32 + 16 * f + l16, i = c & 7;
                const int o = rl * GR_ZROW + (c & ~7) + ((i & 1) ? 4 + (i >> 1) : (i >> 1));
                s_dig[o] = (int8_t)hd;
                s_dig[PL + o] = (int8_t)md;
                s_dig[2 * PL + o] = (int8_t)ld;
            }
            sum = dpp_row16_sum_i(sum);
            if (l16 == 0) s_sum[rl * 4 + wn] = sum;
        }
    __syncthreads();
    int8_t* planes[3] = {a.zq_hi, a.zq_mid, a.zq_lo};
    for (int u = tid; u < 3 * 64 * 8; u += GR_THREADS) {
        const int p = u >> 9, rl = (u >> 3) & 63, ch = u & 7;
        const int row = m0 + rl;
        if (row < a.M)
            *reinterpret_cast<uint4*>(planes[p] + (size_t)row * a.zq_ld + n0 + 16 * ch) =
                *reinterpret_cast<const uint4*>(s_dig + p * PL + rl * GR_ZROW + 16 * ch);
    }
    if (tid < 64 && m0 + tid < a.M) {
        const float mx = fmaxf(fmaxf(s_max[tid * 4], s_max[tid * 4 + 1]), fmaxf(s_max[tid * 4 + 2], s_max[tid * 4 + 3]));
        int e;
        (void)frexpf(mx / Q8_MAX, &e);
        const int sum = s_sum[tid * 4] + s_sum[tid * 4 + 1] + s_sum[tid * 4 + 2] + s_sum[tid * 4 + 3];
        const size_t o = (size_t)(m0 + tid) * a.zq_lds + n0 / GR_BK;
        a.zq_s[o] = ldexpf(1.f, e);
        a.zq_sum[o] = (float)sum;
    }
}
static_assert(2048 + 3 * 64 * GR_ZROW <= GR_STAGE, "the z digits fit one ring stage");

template <int MODE, bool G128>
__global__ __launch_bounds__(GR_THREADS) void w4_gemm_i8r_kernel(GemmArgs a) {
    extern __shared__ __align__(16) int8_t gr_lds[];
    const int MT = (a.M + GR_BM - 1) / GR_BM;
    const int NW_ = MODE ? GR_BN / 2 : GR_BN;   // output columns per tile
    const int NT = (a.N + NW_ - 1) / NW_;
    const int T = MT * NT, Wk = T * a.ksplit, per = (Wk + 7) / 8;
    const int Lw = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (Lw >= Wk) return;
    const int L = Lw % T, split = Lw / T;
    const int k_lo = split * a.kchunk, k_hi = a.ksplit > 1 ? k_lo + a.kchunk : a.K;
    const int m0 = (L % MT) * GR_BM, n0 = (L / MT) * NW_;
    const int KT = (k_hi - k_lo) / GR_BK;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int l16 = lane & 15, l4 = lane >> 4;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int8_t*)gr_lds;

    // W row of tile row r (mode 1: rows >= 128 are W1's copy of rows r - 128), clamped
    auto second = [&](int r) { return MODE && r >= GR_BN / 2; };
    auto wrow = [&](int r) { return min(n0 + (second(r) ? r - GR_BN / 2 : r), a.N - 1); };
    auto bcol = [&](int nf) {
        return MODE ? (nf < 2 ? wn * 32 + 16 * nf : GR_BN / 2 + wn * 32 + 16 * (nf - 2)) : wn * 64 + 16 * nf;
    };

    // ---- copies of k tile kt into stage st -------------------------------------------------------
    // A: instruction i (24 per stage, wave w takes 3w..3w+2) covers plane i / 8, rows
    // 8 (i % 8) .. + 7: lane l -> row 8 (i % 8) + l / 8, LDS chunk l % 8, which holds global
    // chunk (l % 8) ^ (row & 7). B: instruction i (16, wave w takes 2w, 2w + 1) covers W rows
    // 16 i .. + 15: lane l -> row 16 i + l / 4, LDS chunk l % 4 holding global chunk
    // (l % 4) ^ ((row >> 1) & 3). Small: instruction j (waves 0-4, 2 each): j < 4 scale
    // words of W rows 64 j + lane, 4 <= j < 8 zero words of rows 64 (j - 4) + lane, j = 8
    // q_s and j = 9 q_sum of A row lane.
    // N * G is even (checked by the launcher), so the dword holding scale e (of N * G) starts
    // at e & ~1 and ends inside the table
    // the k-independent part of each plane and code copy's source (column k_lo)
    const int8_t* a_src[3];
    uint32_t a_dst[3];
#pragma unroll
    for (int q = 0; q < 3; q++) {
        const int i = 3 * wave + q, p = i >> 3, rb = 8 * (i & 7);
        const int r = rb + (lane >> 3), c = (lane & 7) ^ (r & 7);
        const int8_t* plane = p == 0 ? a.q_hi : (p == 1 ? a.q_mid : a.q_lo);
        a_src[q] = plane + (size_t)min(m0 + r, a.M - 1) * a.ldq + k_lo + 16 * c;
        a_dst[q] = (uint32_t)(p * GR_A_PLANE + rb * GR_BK);
    }
    const int8_t* b_src[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int i = 2 * wave + q, r = 16 * i + (lane >> 2), c = (lane & 3) ^ ((r >> 1) & 3);
        const uint32_t* qw = second(r) ? a.W1.qweight : a.W0.qweight;
        b_src[q] = reinterpret_cast<const int8_t*>(qw + (size_t)wrow(r) * a.W0.KW + k_lo / 8 + 4 * c);
    }
    auto issue = [&](int kt, int st) {
        const int kb = k_lo + kt * GR_BK, g = kb / a.group;
        const uint32_t sbase = lds0 + (uint32_t)(st * GR_STAGE);
#pragma unroll
        for (int q = 0; q < 3; q++)
            gr_copy16(a_src[q] + kt * GR_BK, __builtin_amdgcn_readfirstlane(sbase + a_dst[q]));
#pragma unroll
        for (int q = 0; q < 2; q++)
            gr_copy16(b_src[q] + kt * (GR_BK / 2),
                      __builtin_amdgcn_readfirstlane(sbase + GR_A_BYTES + 16 * (2 * wave + q) * (GR_BK / 2)));
        if (wave < 5) {
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const int j = 2 * wave + q;
                const uint32_t dst = sbase + GR_A_BYTES + GR_B_BYTES + 256 * j;
                const void* src;
                if (j < 4) {   // the dword holding the 16-bit scale of (row, g)
                    const int r = 64 * j + lane;
                    const int e = wrow(r) * a.W0.G + g;
                    src = (second(r) ? a.W1.scales : a.W0.scales) + (e & ~1);
                } else if (j < 8) {
                    const int r = 64 * (j - 4) + lane;
                    src = second(r) ? a.W1.zeros + (size_t)wrow(r) * a.W1.zstride + (g >> 3)
                                    : a.W0.zeros + (size_t)wrow(r) * a.W0.zstride + (g >> 3);
                } else {
                    const float* base = j == 8 ? a.q_s : a.q_sum;
                    src = base + (size_t)min(m0 + lane, a.M - 1) * a.ldqs + g;
                }
                gr_copy4(src, __builtin_amdgcn_readfirstlane(dst));
            }
        }
    };
    // wait until this wave's copies of the oldest stage in flight have landed, with
    // `newer` stages issued after it
    auto wait_copies = [&](int newer) {
        if (newer == 0) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        else if (wave < 5) __builtin_amdgcn_s_waitcnt(0x0F70 | (GR_COPIES_BIG + GR_COPIES_SMALL));
        else __builtin_amdgcn_s_waitcnt(0x0F70 | GR_COPIES_BIG);
    };
    static_assert(GR_STAGES == 3 && GR_COPIES_BIG + GR_COPIES_SMALL < 16, "one newer stage fits vmcnt's low bits");

    f32x4_t acc[2][4];
    i32x4_t ah_acc[2][4], am_acc[2][4], al_acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            ah_acc[i][j] = i32x4_t{0, 0, 0, 0};
            am_acc[i][j] = i32x4_t{0, 0, 0, 0};
            al_acc[i][j] = i32x4_t{0, 0, 0, 0};
        }

    issue(0, 0);
    if (KT > 1) issue(1, 1);
    for (int kt = 0; kt < KT; kt++) {
        const int st = kt % GR_STAGES, kb = k_lo + kt * GR_BK;
        wait_copies(kt + 1 < KT ? 1 : 0);
        __syncthreads();   // tile kt is in LDS, and every wave is done with tile kt - 1
        if (kt + 2 < KT) issue(kt + 2, (kt + 2) % GR_STAGES);   // into the stage of tile kt - 1
        const bool gstart = G128 || kb % a.group == 0;
        const int8_t* sA = gr_lds + st * GR_STAGE;
        const int8_t* sB = sA + GR_A_BYTES;
#pragma unroll
        for (int ks = 0; ks < GR_BK / 64; ks++) {
            i32x4_t ah[2], am[2], al[2], b[4];
#pragma unroll
            for (int mf = 0; mf < 2; mf++) {
                const int row = wm * 32 + mf * 16 + l16, o = gr_a_off(row, 4 * ks + l4);
                ah[mf] = *reinterpret_cast<const i32x4_t*>(sA + o);
                am[mf] = *reinterpret_cast<const i32x4_t*>(sA + GR_A_PLANE + o);
                al[mf] = *reinterpret_cast<const i32x4_t*>(sA + 2 * GR_A_PLANE + o);
            }
#pragma unroll
            for (int nf = 0; nf < 4; nf++) {
                // codes of columns 64 ks + 16 l4 .. + 15: 8 bytes at byte 32 ks + 8 l4 of the row
                const int row = bcol(nf) + l16;
                const uint2 w = *reinterpret_cast<const uint2*>(sB + gr_b_off(row, 2 * ks + (l4 >> 1)) + 8 * (l4 & 1));
                b[nf] = i32x4_t{(int)(w.x & 0x0F0F0F0Fu), (int)((w.x >> 4) & 0x0F0F0F0Fu), (int)(w.y & 0x0F0F0F0Fu),
                                (int)((w.y >> 4) & 0x0F0F0F0Fu)};
            }
#pragma unroll
            for (int mf = 0; mf < 2; mf++)
#pragma unroll
                for (int nf = 0; nf < 4; nf++) {
                    if (ks == 0 && gstart) {   // a group's first products start from zero
                        const i32x4_t z4 = {0, 0, 0, 0};
                        ah_acc[mf][nf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[mf], b[nf], z4, 0, 0, 0);
                        am_acc[mf][nf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(am[mf], b[nf], z4, 0, 0, 0);
                        al_acc[mf][nf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al[mf], b[nf], z4, 0, 0, 0);
                    } else {
                        ah_acc[mf][nf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[mf], b[nf], ah_acc[mf][nf], 0, 0, 0);
                        am_acc[mf][nf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(am[mf], b[nf], am_acc[mf][nf], 0, 0, 0);
                        al_acc[mf][nf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al[mf], b[nf], al_acc[mf][nf], 0, 0, 0);
                    }
                }
        }
        if (G128 || (kb + GR_BK) % a.group == 0) {   // group ends: combine the digit sums, scale and add
            // I = 65536 sum(c h) + 256 sum(c m) + sum(c l) - z sum(v), with the first two
            // sums joined in int32 before one conversion (|256 sum(c h) + sum(c m)| < 2^28
            // for groups of up to 512 columns: c <= 15, |h| <= 127, |m| <= 128)
            const int g = kb / a.group;
            const uint32_t* sSw = reinterpret_cast<const uint32_t*>(sB + GR_B_BYTES);
            const uint32_t* sZ = sSw + GR_BN;
            const float* sSx = reinterpret_cast<const float*>(sZ + GR_BN);
            const float* sSX = sSx + GR_BM;
            f32x4_t sx[2], sX[2];   // rows wm * 32 + mf * 16 + 4 l4 + r
#pragma unroll
            for (int mf = 0; mf < 2; mf++) {
                const int mb = wm * 32 + mf * 16 + 4 * l4;
                sx[mf] = *reinterpret_cast<const f32x4_t*>(sSx + mb);
                sX[mf] = *reinterpret_cast<const f32x4_t*>(sSX + mb);
            }
#pragma unroll
            for (int nf = 0; nf < 4; nf++) {
                const int n = bcol(nf) + l16;
                const int e = wrow(n) * a.W0.G + g;
                const uint32_t sw_word = sSw[n];
                const float sw = scale_to_f32((uint16_t)((e & 1) ? sw_word >> 16 : sw_word & 0xFFFFu), a.W0.scale_dtype);
                const float nz = -(float)(a.W0.zsym ? 8 : (int)((sZ[n] >> ((g & 7) * 4)) & 15u));
#pragma unroll
                for (int mf = 0; mf < 2; mf++) {
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int y = ah_acc[mf][nf][r] * 256 + am_acc[mf][nf][r];
                        float I = fmaf(256.f, (float)y, (float)al_acc[mf][nf][r]);
                        I = fmaf(nz, sX[mf][r], I);
                        acc[mf][nf][r] = fmaf(I * sw, sx[mf][r], acc[mf][nf][r]);
                    }
                }
            }
        }
    }

    if constexpr (MODE == 1 && G128) {
        if (a.zq_hi) {   // z quantised here for the down projection's int8 kernel
            // the stage of k tile KT - 2 (any stage but tile 0's when KT = 1): every wave has
            // passed the barrier of the last iteration, so none still reads it
            gr_swiglu_digits(a, acc, gr_lds + ((KT + 1) % GR_STAGES) * GR_STAGE, m0, n0, wm, wn, l16, l4, tid);
            return;
        }
    }
    // epilogue: D[row 4*l4 + r][col l16] of each fragment
#pragma unroll
    for (int mf = 0; mf < 2; mf++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = m0 + wm * 32 + mf * 16 + 4 * l4 + r;
            if (row >= a.M) continue;
            if (MODE == 0) {
#pragma unroll
                for (int nf = 0; nf < 4; nf++) {
                    const int col = n0 + bcol(nf) + l16;
                    if (col < a.N) a.C[split * a.c_split + (size_t)row * a.ldc + col] = acc[mf][nf][r];
                }
            } else {
#pragma unroll
                for (int f = 0; f < 2; f++) {
                    const int col = n0 + wn * 32 + 16 * f + l16;
                    if (col < a.N) {
                        const float gt = acc[mf][f][r], up = acc[mf][f + 2][r];
                        uint32_t hi, lo;
                        pf_split(gt / (1.0f + __expf(-gt)) * up, hi, lo);
                        a.z_hi[(size_t)row * a.ldz + col] = (uint16_t)hi;
                        a.z_lo[(size_t)row * a.ldz + col] = (uint16_t)lo;
                    }
                }
            }
        }
}

// Group-scaled 24-bit fixed point digits of A = hi + lo (bf16 planes) for
// w4_gemm_i8_kernel. Each lane takes 8 consecutive columns, group/8 lanes of one wave a
// group (group <= 512): s is the power of two with max|x| / Q8_MAX <= s (so x / s is
// exact and only its rounding to an integer errs, by at most s / 2 <= max|x| / Q8_MAX),
// v = rint(x / s) with |v| <= Q8_MAX = 127 * 65536, split into balanced digits
// v = 65536 h + 256 m + l with l, m in [-128, 127] and h in [-127, 127]; bytes stored in
// the order 0,2,4,6,1,3,5,7 of the 8 columns; q_sum = sum of v over the group (f32).
__global__ __launch_bounds__(256) void pf_quant8_kernel(const uint16_t* hi, const uint16_t* lo, int lda, int M, int K,
                                                        int group, int8_t* q_hi, int8_t* q_mid, int8_t* q_lo,
                                                        float* q_s, float* q_sum) {
    const int m = blockIdx.y;
    const int b8 = blockIdx.x * 256 + threadIdx.x, nb = K / 8, lanes = group / 8;
    const bool on = b8 < nb;   // whole groups are on or off (256 * 8 and K are multiples of group)
    float x[8];
    if (on) {
        const uint4 h = *reinterpret_cast<const uint4*>(hi + (size_t)m * lda + 8 * b8);
        const uint4 l = *reinterpret_cast<const uint4*>(lo + (size_t)m * lda + 8 * b8);
        const uint32_t hw[4] = {h.x, h.y, h.z, h.w}, lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            x[2 * i] = bf16_bits_to_f32(hw[i] & 0xFFFFu) + bf16_bits_to_f32(lw[i] & 0xFFFFu);
            x[2 * i + 1] = bf16_bits_to_f32(hw[i] >> 16) + bf16_bits_to_f32(lw[i] >> 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) x[i] = 0.f;
    }
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) mx = fmaxf(mx, fabsf(x[i]));
    for (int o = 1; o < lanes; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    int e;
    (void)frexpf(mx / Q8_MAX, &e);   // s = 2^e >= max|x| / Q8_MAX (s = 1 for a zero group)
    const float inv = ldexpf(1.f, -e);
    int v[8];
    double sum = 0.0;   // integers below 2^33: exact
#pragma unroll
    for (int i = 0; i < 8; i++) {
        v[i] = (int)fminf(fmaxf(rintf(x[i] * inv), -Q8_MAX), Q8_MAX);
        sum += (double)v[i];
    }
    for (int o = 1; o < lanes; o <<= 1) sum += __shfl_xor(sum, o);
    if (!on) return;
    uint32_t H[2] = {0u, 0u}, Mw[2] = {0u, 0u}, Lw[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int ld = ((v[i] + 128) & 255) - 128;
        const int v1 = (v[i] - ld) >> 8;   // exact: v - ld is a multiple of 256
        const int md = ((v1 + 128) & 255) - 128;
        const int hd = (v1 - md) >> 8;
        const int word = i & 1, byte = i >> 1;   // column i -> position (i even: i/2, odd: 4 + i/2)
        H[word] |= ((uint32_t)hd & 0xFFu) << (8 * byte);
        Mw[word] |= ((uint32_t)md & 0xFFu) << (8 * byte);
        Lw[word] |= ((uint32_t)ld & 0xFFu) << (8 * byte);
    }
    const size_t o8 = (size_t)m * K + 8 * b8;
    *reinterpret_cast<uint2*>(q_hi + o8) = make_uint2(H[0], H[1]);
    *reinterpret_cast<uint2*>(q_mid + o8) = make_uint2(Mw[0], Mw[1]);
    *reinterpret_cast<uint2*>(q_lo + o8) = make_uint2(Lw[0], Lw[1]);
    if (b8 % lanes == 0) {
        const int ng = K / group;
        q_s[(size_t)m * ng + b8 / lanes] = ldexpf(1.f, e);
        q_sum[(size_t)m * ng + b8 / lanes] = (float)sum;
    }
}

// ---- the same product for a few rows ---------------------------------------------------------
//
// For M <= 16 (a decode batch) one 16-row MFMA tile covers A: the 64-row tile above would
// spend 4x the matrix-core work on rows that do not exist. Mode 0 only, with split-K.
// Per block: 16 rows x 128 columns; wave w owns columns 32w..32w+31 (two 16x16
// fragments). Staging as above: codes dequantised to (c - z) in bf16 into LDS, A as bf16
// hi/lo planes, per-group f32 accumulation scaled at the group's end, the next k tile's
// loads in flight during the current one's products (deeper register rings were slower).
__global__ __launch_bounds__(GM_THREADS) void w4_gemm16_kernel(GemmArgs a) {
    constexpr int BM = 16, LDK = GM_BK + 8;
    __shared__ __align__(16) uint16_t sAh[BM * LDK];
    __shared__ __align__(16) uint16_t sAl[BM * LDK];
    __shared__ __align__(16) uint16_t sB[GM_BN * LDK];
    __shared__ float sS[2][GM_BN];
    const int NT = (a.N + GM_BN - 1) / GM_BN;
    const int Wk = NT * a.ksplit, per = (Wk + 7) / 8;
    const int Lw = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (Lw >= Wk) return;
    const int n0 = (Lw % NT) * GM_BN, split = Lw / NT;
    const int k_lo = split * a.kchunk, k_hi = a.ksplit > 1 ? k_lo + a.kchunk : a.K;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, l4 = lane >> 4;
    const int KT = (k_hi - k_lo + GM_BK - 1) / GM_BK;

    // codes: W row br of the tile, 32 columns from bc (one uint4 per thread)
    const int br = tid / (GM_BK / 32), bc = 32 * (tid % (GM_BK / 32));
    const int brow = min(n0 + br, a.N - 1);
    const int KW = a.W0.KW, GG = a.W0.G;
    const int srow = tid & (GM_BN - 1), sslot = tid / GM_BN;
    const uint16_t* s_p = a.W0.scales + (size_t)min(n0 + srow, a.N - 1) * GG;
    // A: threads 0..127 stage the hi plane, 128..255 the lo plane: row ar, 8 columns from ac
    const int pl = tid >> 7, ar = (tid & 127) / (GM_BK / 8), ac = 8 * (tid % (GM_BK / 8));
    const uint16_t* a_src = (pl ? a.a_lo : a.a_hi) + (size_t)min(ar, a.M - 1) * a.lda;
    uint16_t* a_dst = pl ? sAl : sAh;
    uint4 rA, rB;
    uint32_t rZ;
    uint16_t rS;
    auto load = [&](int kt) {
        const int kb = k_lo + kt * GM_BK;
        rA = *reinterpret_cast<const uint4*>(a_src + min(kb + ac, a.K - 8));
        const int kc = min(kb + bc, a.K - 32);
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.W0.qweight + (size_t)brow * KW + kc / 8));
        rB = make_uint4(v.x, v.y, v.z, v.w);
        rZ = a.W0.zeros[(size_t)brow * a.W0.zstride + ((kc / a.group) >> 3)];
        rS = s_p[min((kb + 32 * sslot) / a.group, GG - 1)];
    };
    f32x4_t acc[2], accg[2];
#pragma unroll
    for (int f = 0; f < 2; f++) {
        acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        accg[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    load(0);
    for (int kt = 0; kt < KT; kt++) {
        const int kb = k_lo + kt * GM_BK, kn = min(GM_BK, k_hi - kb);
        __syncthreads();   // the previous tile's fragments have been read
        *reinterpret_cast<uint4*>(&a_dst[ar * LDK + ac]) = rA;
        {
            const int kc = min(kb + bc, a.K - 32);
            const int z = a.W0.zsym ? 8 : (int)((rZ >> (((kc / a.group) & 7) * 4)) & 15u);
            const uint32_t w4[4] = {rB.x, rB.y, rB.z, rB.w};
            uint32_t o[16];
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float v0 = (float)((int)((w4[q] >> (4 * e)) & 15u) - z);
                    const float v1 = (float)((int)((w4[q] >> (4 * e + 4)) & 15u) - z);
                    o[q * 4 + e / 2] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xFFFF0000u);
                }
            uint4* dst = reinterpret_cast<uint4*>(&sB[br * LDK + bc]);
#pragma unroll
            for (int q = 0; q < 4; q++) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        }
        sS[sslot][srow] = scale_to_f32(rS, a.W0.scale_dtype);
        __syncthreads();
        if (kt + 1 < KT) load(kt + 1);   // in flight during the products below
        for (int ks = 0; ks < kn / 32; ks++) {
            const int k = ks * 32 + 8 * l4;
            const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&sAh[l16 * LDK + k]);
            const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&sAl[l16 * LDK + k]);
#pragma unroll
            for (int f = 0; f < 2; f++) {
                const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(&sB[(wave * 32 + 16 * f + l16) * LDK + k]);
                const f32x4_t c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, accg[f], 0, 0, 0);
                accg[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, c, 0, 0, 0);
            }
            const int kabs = kb + 32 * ks + 32;
            if (kabs % a.group == 0 || kabs >= k_hi) {   // group ends: scale and add
                const int slot = a.group == 32 ? ks : 0;
#pragma unroll
                for (int f = 0; f < 2; f++) {
                    const float sc = sS[slot][wave * 32 + 16 * f + l16];
#pragma unroll
                    for (int r = 0; r < 4; r++) acc[f][r] = fmaf(sc, accg[f][r], acc[f][r]);
                    accg[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    }
    // D[row 4 l4 + r][column l16] of each fragment
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int row = 4 * l4 + r;
        if (row >= a.M) continue;
#pragma unroll
        for (int f = 0; f < 2; f++) {
            const int col = n0 + wave * 32 + 16 * f + l16;
            if (col < a.N) a.C[split * a.c_split + (size_t)row * a.ldc + col] = acc[f][r];
        }
    }
}

// ---- a few rows, weights straight to the matrix cores --------------------------------------------
//
// The same product for M <= 16 without LDS staging or block barriers. The roles swap:
// the W4 rows are the MFMA A operand (16 weight rows per tile) and the M activation rows
// the B operand (16 columns), so each wave streams its own rows with no dependence on
// other waves. A wave owns SK_TILES tiles (64 weight rows) and walks its K range 128
// columns at a time:
//  - lane l loads 16 bytes of codes of row l % 16 (columns 32 (l / 16) .. +32) per tile;
//  - a per-wave 4 x 4 word transpose through LDS gives lane l, for k-step j, the 8 codes
//    of columns 32 j + 8 (l / 16) .. +8, i.e. every k-step of 32 is a contiguous,
//    group-aligned block of columns, so per-group scaling works as in the kernels above;
//  - codes become (c - z) in bf16 (exact), the activations come as bf16 hi/lo planes
//    (one 16-byte load per plane and k-step, shared by the wave's tiles);
//  - per group: f32 products accumulated, then scaled by each weight row's group scale.
// Needs the K range of every split to be a multiple of 128 (the dispatcher checks).
constexpr int SK_TILES = 4, SK_WAVES = 4;

// One 128-column step of a wave's tiles as loaded: codes (16 bytes per lane and tile),
// the zero word, the scale of the lane's own row and 32-column group, the activations.
struct SkStep {
    u32x4_t cw[SK_TILES];
    uint32_t zw[SK_TILES];
    uint16_t sw[SK_TILES];
    bf16x8_t bh[4], bl[4];
};

__global__ __launch_bounds__(64 * SK_WAVES) void w4_skinny_kernel(GemmArgs a) {
    __shared__ __align__(16) uint32_t s_tr[SK_WAVES][SK_TILES * 16 * 16];   // code transpose, 1 KB per tile
    __shared__ float s_sc[SK_WAVES][SK_TILES * 16 * 4];                     // scales [tile][row][k-step]
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int Nw = (a.N + 16 * SK_TILES - 1) / (16 * SK_TILES);   // wave tiles per split
    const int gw = blockIdx.x * SK_WAVES + w;
    if (gw >= Nw * a.ksplit) return;   // whole waves; no block barrier below
    const int wt = gw % Nw, split = gw / Nw;
    const int r_base = wt * 16 * SK_TILES;
    const int k_lo = split * a.kchunk, k_hi = a.ksplit > 1 ? k_lo + a.kchunk : a.K;
    const W4View& W = a.W0;
    const int KW = W.KW, G = W.G;
    uint32_t* tr = s_tr[w];
    float* sc = s_sc[w];
    const int m = min(row, a.M - 1);   // activation row of this lane's B operand
    const uint16_t* xh = a.a_hi + (size_t)m * a.lda + 8 * q;
    const uint16_t* xl = a.a_lo + (size_t)m * a.lda + 8 * q;
    int wrow[SK_TILES];
#pragma unroll
    for (int t = 0; t < SK_TILES; t++) wrow[t] = min(r_base + 16 * t + row, a.N - 1);
    auto load = [&](int k0, SkStep& S) {
        k0 = min(k0, k_hi - 128);   // past the end: a valid step, never used
#pragma unroll
        for (int t = 0; t < SK_TILES; t++) {
            S.cw[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W.qweight + (size_t)wrow[t] * KW + (k0 + 32 * q) / 8));
            S.zw[t] = W.zeros[(size_t)wrow[t] * W.zstride + ((k0 / a.group) >> 3)];
            S.sw[t] = W.scales[(size_t)wrow[t] * G + (k0 + 32 * q) / a.group];
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            S.bh[j] = *reinterpret_cast<const bf16x8_t*>(xh + k0 + 32 * j);
            S.bl[j] = *reinterpret_cast<const bf16x8_t*>(xl + k0 + 32 * j);
        }
    };
    f32x4_t acc[SK_TILES], accg[SK_TILES];
#pragma unroll
    for (int t = 0; t < SK_TILES; t++) {
        acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        accg[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    auto compute = [&](int k0, const SkStep& S) {
        // transpose: word j' of lane (row, q') to [t][row][j'][q']; lane (row, q) reads
        // [t][row][q][0..3] = the codes of columns 32 j + 8 q, j = 0..3. Scales: lane
        // (row, q) holds row's scale for k-step q; [t][row][q]
#pragma unroll
        for (int t = 0; t < SK_TILES; t++) {
            const uint32_t wv[4] = {S.cw[t].x, S.cw[t].y, S.cw[t].z, S.cw[t].w};
#pragma unroll
            for (int j = 0; j < 4; j++) tr[((t * 16 + row) * 4 + j) * 4 + q] = wv[j];
            sc[(t * 16 + row) * 4 + q] = scale_to_f32(S.sw[t], W.scale_dtype);
        }
        __builtin_amdgcn_wave_barrier();   // LDS accesses of one wave complete in order
#pragma unroll
        for (int t = 0; t < SK_TILES; t++) {
            const uint4 tv = *reinterpret_cast<const uint4*>(&tr[((t * 16 + row) * 4 + q) * 4]);
            const uint32_t tw[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int g = (k0 + 32 * j) / a.group;
                const int z = W.zsym ? 8 : (int)((S.zw[t] >> ((g & 7) * 4)) & 15u);
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float v0 = (float)((int)((tw[j] >> (4 * e)) & 15u) - z);
                    const float v1 = (float)((int)((tw[j] >> (4 * e + 4)) & 15u) - z);
                    o[e / 2] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xFFFF0000u);
                }
                const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
                accg[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, S.bh[j], accg[t], 0, 0, 0);
                accg[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, S.bl[j], accg[t], 0, 0, 0);
                const int kabs = k0 + 32 * j + 32;
                if (kabs % a.group == 0 || kabs >= k_hi) {   // group ends: scale each weight row
#pragma unroll
                    for (int r = 0; r < 4; r++) acc[t][r] = fmaf(sc[(t * 16 + 4 * q + r) * 4 + j], accg[t][r], acc[t][r]);
                    accg[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
        __builtin_amdgcn_wave_barrier();   // the reads finish before the next step's writes
    };
    // two steps in flight: the next step's loads are issued before this one is computed
    SkStep S0, S1;
    load(k_lo, S0);
    for (int k0 = k_lo; k0 < k_hi; k0 += 256) {
        load(k0 + 128, S1);
        compute(k0, S0);
        if (k0 + 128 < k_hi) {
            load(k0 + 256, S0);
            compute(k0 + 128, S1);
        }
    }
    // D[weight row 4 q + r][activation row l % 16] of each tile
    if (row < a.M) {
#pragma unroll
        for (int t = 0; t < SK_TILES; t++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int fr = r_base + 16 * t + 4 * q + r;
                if (fr < a.N) a.C[split * a.c_split + (size_t)row * a.ldc + fr] = acc[t][r];
            }
    }
}

// ---- per-position kernels ----------------------------------------------------------------

// X[t] = f32(embedding[tokens[t]]) and its bf16 planes. Block 0 also validates every
// token id (invalid ids read row 0 and set the status word).
__global__ __launch_bounds__(256) void pf_embed_kernel(const int32_t* tokens, int n, const uint16_t* emb, int vocab,
                                                      int d, float* X, uint16_t* p_hi, uint16_t* p_lo, int ldp,
                                                      int* status) {
    const int t = blockIdx.x;
    if (t == 0 && status) {
        __shared__ int s_bad;
        if (threadIdx.x == 0) s_bad = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += blockDim.x)
            if (tokens[i] < 0 || tokens[i] >= vocab) s_bad = 1;
        __syncthreads();
        if (threadIdx.x == 0) *status = s_bad ? ATLAS_ERR_INVALID_ARG : ATLAS_OK;
    }
    int tok = tokens[t];
    if (tok < 0 || tok >= vocab) tok = 0;
    const uint2* row = reinterpret_cast<const uint2*>(emb + (size_t)tok * d);
    for (int i = threadIdx.x; i < d / 4; i += blockDim.x) {
        const uint2 v = row[i];
        const float4 x = make_float4(bf16_bits_to_f32(v.x & 0xFFFFu), bf16_bits_to_f32(v.x >> 16),
                                     bf16_bits_to_f32(v.y & 0xFFFFu), bf16_bits_to_f32(v.y >> 16));
        reinterpret_cast<float4*>(X + (size_t)t * d)[i] = x;
        store_split4(x, p_hi + (size_t)t * ldp + 4 * i, p_lo + (size_t)t * ldp + 4 * i);
    }
}

// Full-projection QK RMSNorm, rotary embedding (x attention factor) at position
// start_pos + t, q written back in place, k and v written to row t of the prompt KV
// buffers (rounded to bf16 when the cache is bf16: what is stored is what attends).
// One block per position: the S partial projections are added into an LDS copy of the
// row (dynamic shared memory, (Hq + 2 Hkv) * 128 floats), which every later read uses.
// NE > 0 (S <= 2, (Hq + 2 Hkv) * 128 <= 256 NE, Hq * 128 a multiple of 256, at most 256 NR
// rotation pairs): every load of the block (the partial rows, the gains of the thread's
// rotation pairs) is issued before the first use, and the sums of squares come from the
// registers in the order of the LDS loop of NE = 0.
template <int NE, int NR>
__global__ __launch_bounds__(256) void pf_rope_kernel(PfRopeArgs a) {
    constexpr int D = 128;
    extern __shared__ float s_row[];
    __shared__ float red[16];
    __shared__ float s_cos[64], s_sin[64];
    const int t = blockIdx.x, pos = a.start_pos + t;
    const int nq = a.Hq * D, nk = a.Hkv * D, nqkv = nq + 2 * nk;
    float* row = a.qkv + (size_t)t * a.ld;
    float sq = 0.f, sk = 0.f;
    float g0[NR > 0 ? NR : 1], g1[NR > 0 ? NR : 1];
    if constexpr (NE > 0) {
        float v0[NE], v1[NE];
        const size_t p1 = a.S > 1 ? (size_t)a.pstride : 0;
#pragma unroll
        for (int k = 0; k < NE; k++) {
            const int i = threadIdx.x + 256 * k, ic = i < nqkv ? i : 0;
            v0[k] = row[ic];
            v1[k] = row[p1 + ic];
        }
#pragma unroll
        for (int r = 0; r < NR; r++) {
            const int u = threadIdx.x + 256 * r, uc = u < (a.Hq + a.Hkv) * 64 ? u : 0;
            const int h = uc >> 6, i = uc & 63;
            const float* g = h >= a.Hq ? a.g_k + (h - a.Hq) * D : a.g_q + h * D;
            g0[r] = g[i];
            g1[r] = g[i + 64];
        }
#pragma unroll
        for (int k = 0; k < NE; k++) {
            const int i = threadIdx.x + 256 * k;
            const float v = a.S > 1 ? v0[k] + v1[k] : v0[k];
            if (i < nqkv) s_row[i] = v;
            if (i < nq) sq = fmaf(v, v, sq);
        }
#pragma unroll
        for (int k = 0; k < NE; k++) {
            const int i = threadIdx.x + 256 * k;
            const float v = a.S > 1 ? v0[k] + v1[k] : v0[k];
            if (i >= nq && i < nq + nk) sk = fmaf(v, v, sk);
        }
        __syncthreads();
    } else {
        for (int i = threadIdx.x; i < nqkv; i += blockDim.x) {
            float v = row[i];
            for (int s = 1; s < a.S; s++) v += row[(size_t)s * a.pstride + i];
            s_row[i] = v;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nq; i += blockDim.x) sq = fmaf(s_row[i], s_row[i], sq);
        for (int i = threadIdx.x; i < nk; i += blockDim.x) sk = fmaf(s_row[nq + i], s_row[nq + i], sk);
    }
    sq = block_sum(sq, red);
    sk = block_sum(sk, red);
    const float rq = 1.0f / sqrtf(sq / (float)nq + a.eps);
    const float rk = 1.0f / sqrtf(sk / (float)nk + a.eps);
    if (threadIdx.x < 64) {
        const double ang = (double)pos * a.inv[threadIdx.x];
        const double rr = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
        float sn, cs;
        sincosf((float)rr, &sn, &cs);
        s_cos[threadIdx.x] = cs * (float)a.mscale;
        s_sin[threadIdx.x] = sn * (float)a.mscale;
    }
    __syncthreads();
    const int npairs = (a.Hq + a.Hkv) * 64;
    auto rotate = [&](int u, float ga, float gb) {
        const int h = u >> 6, i = u & 63;
        const bool isk = h >= a.Hq;
        const float rr = isk ? rk : rq;
        const int base = h * D;   // q heads, then k heads, in the projection row
        const float x0 = ga * (s_row[base + i] * rr), x1 = gb * (s_row[base + i + 64] * rr);
        const float c = s_cos[i], sn = s_sin[i];
        const float y0 = x0 * c - x1 * sn, y1 = x1 * c + x0 * sn;
        if (isk) {
            const size_t e = ((size_t)(h - a.Hq) * a.n + t) * D + i;
            if (a.kv_bf16) {
                ((uint16_t*)a.k_new)[e] = (uint16_t)f32_to_bf16_rne(y0);
                ((uint16_t*)a.k_new)[e + 64] = (uint16_t)f32_to_bf16_rne(y1);
            } else {
                ((float*)a.k_new)[e] = y0;
                ((float*)a.k_new)[e + 64] = y1;
            }
        } else {
            row[base + i] = y0;
            row[base + i + 64] = y1;
        }
    };
    if constexpr (NR > 0) {
#pragma unroll
        for (int r = 0; r < NR; r++)
            if (threadIdx.x + 256 * r < npairs) rotate(threadIdx.x + 256 * r, g0[r], g1[r]);
    } else {
        for (int u = threadIdx.x; u < npairs; u += blockDim.x) {
            const int h = u >> 6, i = u & 63;
            const float* g = h >= a.Hq ? a.g_k + (h - a.Hq) * D : a.g_q + h * D;
            rotate(u, g[i], g[i + 64]);
        }
    }
    for (int u = threadIdx.x; u < nk; u += blockDim.x) {
        const int h = u / D, i = u % D;
        const size_t e = ((size_t)h * a.n + t) * D + i;
        const float v = s_row[nq + nk + u];
        if (a.kv_bf16) ((uint16_t*)a.v_new)[e] = (uint16_t)f32_to_bf16_rne(v);
        else ((float*)a.v_new)[e] = v;
    }
}

// One block per committed position: copies its Hkv x 128 keys and values from the
// prompt buffers into the cache slot (j mod slots on a ring).
__global__ __launch_bounds__(256) void pf_commit_kernel(PfCommitArgs a) {
    constexpr int D = 128;
    const int end = a.start_pos + a.n;
    const int first = a.ring ? max(a.start_pos, end - (int)a.slots) : a.start_pos;
    const int j = first + blockIdx.x, t = j - a.start_pos;
    const int slot = a.ring ? j % (int)a.slots : j;
    const int esz = a.kv_bf16 ? 2 : 4;
    const int nv = a.Hkv * D * esz / 16;   // 16-byte vectors per position and tensor
    const int per_head = D * esz / 16;
    for (int u = threadIdx.x; u < 2 * nv; u += blockDim.x) {
        const int isv = u >= nv, w = isv ? u - nv : u, h = w / per_head, c = w % per_head;
        const uint4* src = reinterpret_cast<const uint4*>((const char*)(isv ? a.v_new : a.k_new) +
                                                          (((size_t)h * a.n + t) * D) * esz) + c;
        uint4* dst = reinterpret_cast<uint4*>((char*)(isv ? a.v_cache : a.k_cache) +
                                              (((size_t)h * a.slots + slot) * D) * esz) + c;
        *dst = *src;
    }
}

// Digits of the int8 path for 4 consecutive columns held by one lane, quantised as
// pf_quant8_kernel quantises its planes (x' = hi + lo, the row's group maximum, s = 2^e,
// v = rint(x' / s), balanced digits), for groups of 128 or 256 columns: the group's lanes
// are 32 or 64 consecutive lanes of a wave (LPG), so maxima and sums are DPP row
// reductions plus lane swaps. Column c of an 8-column block goes to byte (c & 1) * 4 +
// c / 2: the lane with the block's first 4 columns stores word 0 (columns 0, 2, 4, 6), its
// neighbour word 1, each from its own two bytes and the neighbour's.
template <int LPG>
__device__ __forceinline__ void q8_digits4(float4 x, int8_t* q_hi, int8_t* q_mid, int8_t* q_lo, float* q_s,
                                           float* q_sum, size_t row_q, size_t row_g, int col0, int group) {
    float xs[4] = {x.x, x.y, x.z, x.w};
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint32_t hi, lo;
        pf_split(xs[j], hi, lo);
        xs[j] = bf16_bits_to_f32(hi) + bf16_bits_to_f32(lo);
        mx = fmaxf(mx, fabsf(xs[j]));
    }
    mx = fmaxf(mx, dpp_f<0xB1>(mx));
    mx = fmaxf(mx, dpp_f<0x4E>(mx));
    mx = fmaxf(mx, dpp_f<0x141>(mx));
    mx = fmaxf(mx, dpp_f<0x140>(mx));
    mx = xor16_max(mx);
    if (LPG == 64) mx = xor32_max(mx);
    int e;
    (void)frexpf(mx / Q8_MAX, &e);   // s = 2^e >= max|x'| / Q8_MAX (s = 1 for a zero group)
    const float inv = ldexpf(1.f, -e);
    int sum = 0;
    uint32_t hw[2] = {0u, 0u}, mw[2] = {0u, 0u}, lw[2] = {0u, 0u};   // [even columns, odd columns]
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int v = (int)fminf(fmaxf(rintf(xs[j] * inv), -Q8_MAX), Q8_MAX);
        sum += v;
        const int ld = ((v + 128) & 255) - 128;
        const int v1 = (v - ld) >> 8;   // exact: v - ld is a multiple of 256
        const int md = ((v1 + 128) & 255) - 128;
        const int hd = (v1 - md) >> 8;
        const int sh = 8 * (j >> 1);
        hw[j & 1] |= ((uint32_t)hd & 0xFFu) << sh;
        mw[j & 1] |= ((uint32_t)md & 0xFFu) << sh;
        lw[j & 1] |= ((uint32_t)ld & 0xFFu) << sh;
    }
    const bool first = ((col0 >> 2) & 1) == 0;   // the block's columns 0-3 (else 4-7)
    auto word = [&](const uint32_t (&w)[2]) {     // this lane's word of the block
        const uint32_t give = first ? w[1] : w[0];   // what the neighbour needs
        const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0xB1, 0xF, 0xF, false);   // lane ^ 1
        return first ? (w[0] | (got << 16)) : (got | (w[1] << 16));
    };
    const uint32_t H = word(hw), Mm = word(mw), Lw = word(lw);
    const size_t o = row_q + (size_t)(col0 & ~7) + (first ? 0 : 4);
    *reinterpret_cast<uint32_t*>(q_hi + o) = H;
    *reinterpret_cast<uint32_t*>(q_mid + o) = Mm;
    *reinterpret_cast<uint32_t*>(q_lo + o) = Lw;
    // exact int32 sums: |v| <= Q8_MAX, at most 256 of them
    sum += __builtin_amdgcn_update_dpp(0, sum, 0xB1, 0xF, 0xF, true);
    sum += __builtin_amdgcn_update_dpp(0, sum, 0x4E, 0xF, 0xF, true);
    sum += __builtin_amdgcn_update_dpp(0, sum, 0x141, 0xF, 0xF, true);
    sum += __builtin_amdgcn_update_dpp(0, sum, 0x140, 0xF, 0xF, true);
    {
        const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)sum, (uint32_t)sum, false, false);
        sum = (int)r[0] + (int)r[1];
    }
    if (LPG == 64) {
        const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)sum, (uint32_t)sum, false, false);
        sum = (int)r[0] + (int)r[1];
    }
    if (col0 % group == 0) {
        q_s[row_g + col0 / group] = ldexpf(1.f, e);
        q_sum[row_g + col0 / group] = (float)sum;
    }
}

// X[t] += g * A[t] / rms(A[t]) with A[t] the sum of S (1 or 2) partial rows (row t's at
// A + t lda and A + t lda + d); then the next GEMM's input from the new X[t]: its bf16
// planes, or (q_hi set; groups of 128 or 256) its int8 digits, scales and group sums as
// pf_quant8_kernel would make them from those planes. One block of 256 threads per row;
// d % 4 == 0, and with digits d is a multiple of 1,024 so that every pass of the block
// covers whole groups. NV > 0: d <= 1,024 NV, and every input of the row (partials,
// residual, gains) is loaded into registers before the first use, one pass; NV = 0: two
// passes over the row.
template <int NV>
__global__ __launch_bounds__(256) void pf_residual_kernel(float* X, const float* A, int lda, int S, const float* g,
                                                         int d, float eps, uint16_t* p_hi, uint16_t* p_lo, int ldp,
                                                         int8_t* q_hi, int8_t* q_mid, int8_t* q_lo, float* q_s,
                                                         float* q_sum, int group) {
    __shared__ float red[16];
    const int t = blockIdx.x;
    const float4* a4 = reinterpret_cast<const float4*>(A + (size_t)t * lda);
    const float4* b4 = reinterpret_cast<const float4*>(A + (size_t)t * lda + (S > 1 ? d : 0));
    auto part = [&](int i) {
        float4 v = a4[i];
        if (S > 1) {
            const float4 w = b4[i];
            v = make_float4(v.x + w.x, v.y + w.y, v.z + w.z, v.w + w.w);
        }
        return v;
    };
    float4* x4 = reinterpret_cast<float4*>(X + (size_t)t * d);
    const float4* g4 = reinterpret_cast<const float4*>(g);
    auto emit = [&](int i, float4 v, float4 x, float4 gg, float r) {
        const float4 h = make_float4(x.x + gg.x * (v.x * r), x.y + gg.y * (v.y * r), x.z + gg.z * (v.z * r),
                                     x.w + gg.w * (v.w * r));
        x4[i] = h;
        if (q_hi) {
            const size_t rq = (size_t)t * d, rg = (size_t)t * (d / group);
            if (group == 128) q8_digits4<32>(h, q_hi, q_mid, q_lo, q_s, q_sum, rq, rg, 4 * i, group);
            else q8_digits4<64>(h, q_hi, q_mid, q_lo, q_s, q_sum, rq, rg, 4 * i, group);
        } else {
            store_split4(h, p_hi + (size_t)t * ldp + 4 * i, p_lo + (size_t)t * ldp + 4 * i);
        }
    };
    const int n4 = d / 4;
    if constexpr (NV > 0) {
        float4 pa[NV], pb[NV], xv[NV], gv[NV];
#pragma unroll
        for (int j = 0; j < NV; j++) {
            const int i = threadIdx.x + 256 * j, ic = i < n4 ? i : 0;
            pa[j] = a4[ic];
            pb[j] = b4[ic];   // the first partial again when S = 1 (not added)
            xv[j] = x4[ic];
            gv[j] = g4[ic];
        }
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NV; j++) {
            if (S > 1) pa[j] = make_float4(pa[j].x + pb[j].x, pa[j].y + pb[j].y, pa[j].z + pb[j].z, pa[j].w + pb[j].w);
            if (threadIdx.x + 256 * j < n4)
                ss = fmaf(pa[j].x, pa[j].x, fmaf(pa[j].y, pa[j].y, fmaf(pa[j].z, pa[j].z, fmaf(pa[j].w, pa[j].w, ss))));
        }
        ss = block_sum(ss, red);
        const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
        for (int j = 0; j < NV; j++) {
            const int i = threadIdx.x + 256 * j;
            if (i < n4) emit(i, pa[j], xv[j], gv[j], r);
        }
    } else {
        float ss = 0.f;
        for (int i = threadIdx.x; i < n4; i += blockDim.x) {
            const float4 v = part(i);
            ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
        }
        ss = block_sum(ss, red);
        const float r = 1.0f / sqrtf(ss / (float)d + eps);
        for (int i = threadIdx.x; i < n4; i += blockDim.x) emit(i, part(i), x4[i], g4[i], r);
    }
}

// bf16 planes of an f32 matrix [M][K] (row stride ldx) into [M][ldp]; K % 4 == 0.
__global__ __launch_bounds__(256) void pf_split_kernel(const float* X, int K, int ldx, uint16_t* p_hi, uint16_t* p_lo,
                                                      int ldp) {
    const int t = blockIdx.x;
    const float4* x4 = reinterpret_cast<const float4*>(X + (size_t)t * ldx);
    for (int i = threadIdx.x; i < K / 4; i += blockDim.x)
        store_split4(x4[i], p_hi + (size_t)t * ldp + 4 * i, p_lo + (size_t)t * ldp + 4 * i);
}

// ---- causal GQA attention over a block of 16 positions ------------------------------------
//
// grid (ceil(n / 16), Hkv), one wave per query head of the KV group. Keys come in
// tiles of 16 through LDS (shared by the group's heads): K as bf16 hi/lo planes, V the
// same but transposed ([dim][key]). Per wave: S (16 positions x 16 keys) = Q K^T over
// the 128 dimensions on 16x16x32 bf16 MFMAs, masked to each position's window, online
// softmax per position, O += P V on 16x16x16 bf16 MFMAs (P re-laid out through LDS);
// each product is hi*hi + hi*lo + lo*hi of the split operands (with a bf16 cache the
// keys and values are exact in bf16, their lo planes vanish, and hi*hi + lo*hi
// remain). The output is written
// as bf16 planes for the o projection.
constexpr int PF_QT = 16;

// 4 consecutive K or V values (dims 4c..4c+3) of key j of KV head kv (f32 caches):
// from the cache for j < start_pos (slot j, or j mod slots on a ring: start_pos - slots
// < j there), from the prompt buffer otherwise.
__device__ __forceinline__ float4 pf_kv4_f32(const void* cache, const void* fresh, const PfAttnArgs& a, int kv, int j,
                                             int c, int sp) {
    constexpr int D = 128;
    size_t e;
    const void* base;
    if (j >= a.start_pos) {
        base = fresh;
        e = ((size_t)kv * a.n + (j - a.start_pos)) * D + 4 * c;
    } else {
        int sl = j;
        if (a.ring) {   // sp = start_pos mod slots, 0 < start_pos - j < slots
            sl = sp - (a.start_pos - j);
            sl += sl < 0 ? (int)a.slots : 0;
        }
        base = cache;
        e = ((size_t)kv * a.slots + sl) * D + 4 * c;
    }
    return *reinterpret_cast<const float4*>((const float*)base + e);
}

// Raw bf16 bits of dims 8c..8c+7 of key j (bf16 caches), from the same places as pf_kv4_f32.
__device__ __forceinline__ uint4 pf_kv8_bf16(const void* cache, const void* fresh, const PfAttnArgs& a, int kv, int j,
                                             int c, int sp) {
    constexpr int D = 128;
    size_t e;
    const void* base;
    if (j >= a.start_pos) {
        base = fresh;
        e = ((size_t)kv * a.n + (j - a.start_pos)) * D + 8 * c;
    } else {
        int sl = j;
        if (a.ring) {
            sl = sp - (a.start_pos - j);
            sl += sl < 0 ? (int)a.slots : 0;
        }
        base = cache;
        e = ((size_t)kv * a.slots + sl) * D + 8 * c;
    }
    return *reinterpret_cast<const uint4*>((const uint16_t*)base + e);
}

template <int G, bool KVB>
__global__ __launch_bounds__(64 * G) void pf_attn_kernel(PfAttnArgs a) {
    constexpr int D = 128, KPB = D + 8, VTP = 16 + 4, PP = 20;
    constexpr int NT = 64 * G;
    constexpr int EPL = KVB ? 8 : 4;            // cache elements per 16-byte load
    constexpr int NLD = 16 * D / EPL;           // 16-byte loads per tile of K (and of V)
    constexpr int NPT = (NLD + NT - 1) / NT;    // per thread
    // two LDS stages: the tile being multiplied and the next one being stored
    __shared__ __align__(16) uint16_t sKh[2][16 * KPB];   // keys as bf16 planes: K = hi + lo
    __shared__ __align__(16) uint16_t sKl[2][16 * KPB];
    __shared__ __align__(16) uint16_t sVth[2][D * VTP];   // values transposed ([dim][key]) as bf16 planes
    __shared__ __align__(16) uint16_t sVtl[2][D * VTP];
    __shared__ __align__(16) float sP[G][16 * PP];
    // grid (Hkv, query tiles): the longest query tiles (most causal keys) of every KV head
    // are dispatched first, so that they start before the short ones
    const int t0 = (gridDim.y - 1 - blockIdx.y) * PF_QT, kv = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, l4 = lane >> 4;
    const int head = kv * G + wave;
    const int t_last = min(t0 + PF_QT, a.n) - 1;
    const int p_first = a.start_pos + t0, p_last = a.start_pos + t_last;
    const int klo = a.window > 0 ? max(0, p_first - a.window + 1) : 0;
    const int khi = p_last;

    // Q fragments as bf16 planes (Q = hi + lo): lane holds Q[position t0 + l16][32 ks + 8 l4 + i],
    // i < 8, for the k-step ks of 32 dims (A operand layout of the 16x16x32 bf16 MFMA)
    bf16x8_t qh[4], ql[4];
    {
        const float4* q = reinterpret_cast<const float4*>(a.qkv + (size_t)min(t0 + l16, a.n - 1) * a.ld_qkv + head * D);
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const float4 u = q[8 * ks + 2 * l4], v = q[8 * ks + 2 * l4 + 1];
            uint32_t h[8], lo[8];
            pf_split(u.x, h[0], lo[0]);
            pf_split(u.y, h[1], lo[1]);
            pf_split(u.z, h[2], lo[2]);
            pf_split(u.w, h[3], lo[3]);
            pf_split(v.x, h[4], lo[4]);
            pf_split(v.y, h[5], lo[5]);
            pf_split(v.z, h[6], lo[6]);
            pf_split(v.w, h[7], lo[7]);
            qh[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                                             h[6] | (h[7] << 16)));
            ql[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16),
                                                             lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)));
        }
    }
    float m[4], l[4];
    f32x4_t o[8];
#pragma unroll
    for (int r = 0; r < 4; r++) {
        m[r] = -INFINITY;
        l[r] = 0.f;
    }
#pragma unroll
    for (int gi = 0; gi < 8; gi++) o[gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int sp = a.ring ? a.start_pos % (int)a.slots : 0;
    // The raw K/V words of the next key tile are loaded into registers while the current
    // tile is multiplied; at the top of the next iteration they are split into planes and
    // stored into the free LDS stage. Load u (< NLD) of a tile is key u / (D / EPL),
    // 16-byte chunk u % (D / EPL); the loads are unconditional (u clamped to NLD - 1).
    uint4 rk[NPT], rv[NPT];
    auto issue = [&](int kb) {
        // A tile wholly inside the prompt (every tile when start_pos = 0) reads the prompt
        // buffer directly; only a tile that reaches below start_pos goes through the
        // per-key choice of buffer and the ring's slot map. kb is uniform: no divergence.
        const bool fresh_tile = kb >= a.start_pos;
        const size_t fresh0 = ((size_t)kv * a.n + (fresh_tile ? kb - a.start_pos : 0)) * D;
#pragma unroll
        for (int r = 0; r < NPT; r++) {
            const int u = min(tid + r * NT, NLD - 1);
            const int kr = u / (D / EPL), c = u % (D / EPL);
            const int j = min(kb + kr, khi);
            if constexpr (KVB) {
                if (fresh_tile) {
                    const size_t e = fresh0 + (size_t)(j - kb) * D + 8 * c;
                    rk[r] = *reinterpret_cast<const uint4*>((const uint16_t*)a.k_new + e);
                    rv[r] = *reinterpret_cast<const uint4*>((const uint16_t*)a.v_new + e);
                } else {
                    rk[r] = pf_kv8_bf16(a.k_cache, a.k_new, a, kv, j, c, sp);
                    rv[r] = pf_kv8_bf16(a.v_cache, a.v_new, a, kv, j, c, sp);
                }
            } else {
                float4 k4, v4;
                if (fresh_tile) {
                    const size_t e = fresh0 + (size_t)(j - kb) * D + 4 * c;
                    k4 = *reinterpret_cast<const float4*>((const float*)a.k_new + e);
                    v4 = *reinterpret_cast<const float4*>((const float*)a.v_new + e);
                } else {
                    k4 = pf_kv4_f32(a.k_cache, a.k_new, a, kv, j, c, sp);
                    v4 = pf_kv4_f32(a.v_cache, a.v_new, a, kv, j, c, sp);
                }
                rk[r] = __builtin_bit_cast(uint4, k4);
                rv[r] = __builtin_bit_cast(uint4, v4);
            }
        }
    };
    auto store = [&](int st) {
#pragma unroll
        for (int r = 0; r < NPT; r++) {
            const int u = tid + r * NT;
            if (u >= NLD) continue;
            const int kr = u / (D / EPL), c = u % (D / EPL);
            if constexpr (KVB) {   // a bf16 value is its own hi plane; its lo plane is zero and never staged
                *reinterpret_cast<uint4*>(&sKh[st][kr * KPB + 8 * c]) = rk[r];
                const uint32_t w[4] = {rv[r].x, rv[r].y, rv[r].z, rv[r].w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    sVth[st][(8 * c + 2 * e) * VTP + kr] = (uint16_t)(w[e] & 0xFFFFu);
                    sVth[st][(8 * c + 2 * e + 1) * VTP + kr] = (uint16_t)(w[e] >> 16);
                }
            } else {
                const float4 k4 = __builtin_bit_cast(float4, rk[r]);
                uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
                pf_split(k4.x, h0, l0);
                pf_split(k4.y, h1, l1);
                pf_split(k4.z, h2, l2);
                pf_split(k4.w, h3, l3);
                *reinterpret_cast<uint2*>(&sKh[st][kr * KPB + 4 * c]) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
                *reinterpret_cast<uint2*>(&sKl[st][kr * KPB + 4 * c]) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
                const float4 v4 = __builtin_bit_cast(float4, rv[r]);
                const float ve[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    uint32_t vh, vl;
                    pf_split(ve[e], vh, vl);
                    sVth[st][(4 * c + e) * VTP + kr] = (uint16_t)vh;
                    sVtl[st][(4 * c + e) * VTP + kr] = (uint16_t)vl;
                }
            }
        }
    };
    if (klo <= khi) issue(klo);
    int st = 0;
    for (int kb = klo; kb <= khi; kb += 16, st ^= 1) {
        // Stage st was last read two iterations ago; every wave has passed the barrier of
        // the previous iteration since, so none still reads it.
        store(st);
        __syncthreads();   // tile kb is in stage st
        if (kb + 16 <= khi) issue(kb + 16);
        // scores Q K^T: hi*hi + hi*lo + lo*hi (the lo*lo term is below 2^-16 of the product)
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const bf16x8_t kh = *reinterpret_cast<const bf16x8_t*>(&sKh[st][l16 * KPB + 32 * ks + 8 * l4]);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[ks], kh, sc, 0, 0, 0);
            if constexpr (!KVB) {
                const bf16x8_t kl = *reinterpret_cast<const bf16x8_t*>(&sKl[st][l16 * KPB + 32 * ks + 8 * l4]);
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[ks], kl, sc, 0, 0, 0);
            }
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[ks], kh, sc, 0, 0, 0);
        }
        // sc[r] = S[position 4 l4 + r][key kb + l16]
        const int j = kb + l16;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int ti = t0 + 4 * l4 + r, pi = a.start_pos + ti;
            const int lo_i = a.window > 0 ? max(0, pi - a.window + 1) : 0;
            const bool valid = ti < a.n && j <= pi && j >= lo_i;
            const float sv = valid ? sc[r] * a.scale : -INFINITY;
            float mt = sv;
            mt = fmaxf(mt, dpp_f<0xB1>(mt));
            mt = fmaxf(mt, dpp_f<0x4E>(mt));
            mt = fmaxf(mt, dpp_f<0x141>(mt));
            mt = fmaxf(mt, dpp_f<0x140>(mt));
            const float mn = fmaxf(m[r], mt);
            const float corr = (mn == -INFINITY) ? 1.f : __expf(m[r] - mn);
            const float p = valid ? __expf(sv - mn) : 0.f;
            l[r] = fmaf(l[r], corr, row16_sum(p));
            m[r] = mn;
#pragma unroll
            for (int gi = 0; gi < 8; gi++) o[gi][r] *= corr;
            sP[wave][(4 * l4 + r) * PP + l16] = p;
        }
        // O += P V on 16x16x16 bf16 MFMAs, hi*hi + hi*lo + lo*hi: A operand P[position l16][key
        // 4 l4 + i], B operand V[key 4 l4 + i][dim 16 gi + l16] (four keys of one dim: a row of V^T)
        {
            const float4 pv = *reinterpret_cast<const float4*>(&sP[wave][l16 * PP + 4 * l4]);
            uint32_t h0, q0, h1, q1, h2, q2, h3, q3;
            pf_split(pv.x, h0, q0);
            pf_split(pv.y, h1, q1);
            pf_split(pv.z, h2, q2);
            pf_split(pv.w, h3, q3);
            const bf16x4_t ph = __builtin_bit_cast(bf16x4_t, make_uint2(h0 | (h1 << 16), h2 | (h3 << 16)));
            const bf16x4_t pl = __builtin_bit_cast(bf16x4_t, make_uint2(q0 | (q1 << 16), q2 | (q3 << 16)));
#pragma unroll
            for (int gi = 0; gi < 8; gi++) {
                const bf16x4_t vh = *reinterpret_cast<const bf16x4_t*>(&sVth[st][(16 * gi + l16) * VTP + 4 * l4]);
                o[gi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vh, o[gi], 0, 0, 0);
                if constexpr (!KVB) {
                    const bf16x4_t vl = *reinterpret_cast<const bf16x4_t*>(&sVtl[st][(16 * gi + l16) * VTP + 4 * l4]);
                    o[gi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vl, o[gi], 0, 0, 0);
                }
                o[gi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vh, o[gi], 0, 0, 0);
            }
        }
    }
    // o[gi][r] = O[position 4 l4 + r][dim 16 gi + l16]
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int ti = t0 + 4 * l4 + r;
        if (ti >= a.n) continue;
        const float inv = 1.0f / l[r];
        uint16_t* hi = a.o_hi + (size_t)ti * a.ldo + head * D;
        uint16_t* lo = a.o_lo + (size_t)ti * a.ldo + head * D;
#pragma unroll
        for (int gi = 0; gi < 8; gi++) {
            uint32_t h, lw;
            pf_split(o[gi][r] * inv, h, lw);
            hi[16 * gi + l16] = (uint16_t)h;
            lo[16 * gi + l16] = (uint16_t)lw;
        }
    }
}

// ---- launchers ------------------------------------------------------------------------------

int gemm_supported(int group) { return group >= 32 && (group == 32 || group % GM_BK == 0); }
int gemm_i8_supported(int group, int K) { return group % G8_BK == 0 && group <= 512 && K % group == 0; }

int launch_pf_quant8(const uint16_t* hi, const uint16_t* lo, int lda, int M, int K, int group, int8_t* q_hi,
                     int8_t* q_mid, int8_t* q_lo, float* q_s, float* q_sum, hipStream_t st) {
    ATLAS_CHECK_SHAPE(gemm_i8_supported(group, K) && lda % 8 == 0 && lda >= K && M >= 1,
                      "int8 planes need a group of 128, 256 or 512 dividing K (group %d, K %d, lda %d)", group, K, lda);
    ATLAS_KLAUNCH(pf_quant8_kernel, dim3((K / 8 + 255) / 256, M), dim3(256), 0, st, hi, lo, lda, M, K, group, q_hi,
                  q_mid, q_lo, q_s, q_sum);
    ATLAS_LAUNCH_CHECK("pf_quant8_kernel");
    return ATLAS_OK;
}

static bool i8r_uses_ring(const GemmArgs& a, int mode) {
    const bool same_w = mode == 0 || (a.W1.G == a.W0.G && a.W1.KW == a.W0.KW && a.W1.zsym == a.W0.zsym &&
                                      a.W1.zstride == a.W0.zstride && a.W1.scale_dtype == a.W0.scale_dtype);
    return same_w && ((size_t)a.N * a.W0.G) % 2 == 0;
}

bool i8r_swiglu_digits_ok(const GemmArgs& a, int down_group) {
    return a.q_hi && a.group == GR_BK && down_group == GR_BK && a.N % GR_BK == 0 && a.ksplit == 1 &&
           i8r_uses_ring(a, 1);
}

int launch_w4_gemm(const GemmArgs& a, int mode, hipStream_t st, const char* label) {
    ATLAS_CHECK_SHAPE(gemm_supported(a.group), "prefill GEMM needs group 32 or a multiple of 64 (got %d)", a.group);
    ATLAS_CHECK_SHAPE(a.K % 32 == 0 && a.K >= 32 && a.lda % 8 == 0, "prefill GEMM shape K=%d lda=%d", a.K, a.lda);
    const int NW_ = mode ? GM_BN / 2 : GM_BN;
    const int MT = (a.M + GM_BM - 1) / GM_BM, NT = (a.N + NW_ - 1) / NW_;
    ATLAS_CHECK_SHAPE(a.ksplit == 1 || (mode == 0 && a.ksplit > 1 && a.kchunk * a.ksplit == a.K &&
                                        a.kchunk % GM_BK == 0 && a.kchunk % a.group == 0),
                      "bad K split (%d x %d of K=%d)", a.ksplit, a.kchunk, a.K);
    prof_mark(label, st);
    if (a.q_hi) {   // int8 digit planes: the int8 matrix-core kernel
        ATLAS_CHECK_SHAPE(gemm_i8_supported(a.group, a.K) && (a.ksplit == 1 || a.kchunk % G8_BK == 0) &&
                              a.ldq % 16 == 0 && a.ldq >= a.K &&
                              a.ldqs >= a.K / a.group && a.q_mid && a.q_lo && a.q_s && a.q_sum,
                          "int8 GEMM needs a group of 128, 256 or 512 dividing K, K ranges of whole 128-column "
                          "tiles, ldq %% 16 == 0");
        if (i8r_uses_ring(a, mode)) {   // the LDS-ring kernel
            static bool attr_set[4] = {false, false, false, false};
            const int g128 = a.group == GR_BK ? 1 : 0, v = 2 * mode + g128;
            ATLAS_CHECK_SHAPE(!a.zq_hi || (v == 3 && a.N % GR_BK == 0 && a.zq_ld % 16 == 0 && a.zq_mid && a.zq_lo &&
                                           a.zq_s && a.zq_sum),
                              "int8 digits of z need mode 1 with groups of 128 on the ring kernel");
            const void* fns[4] = {(const void*)w4_gemm_i8r_kernel<0, false>, (const void*)w4_gemm_i8r_kernel<0, true>,
                                  (const void*)w4_gemm_i8r_kernel<1, false>, (const void*)w4_gemm_i8r_kernel<1, true>};
            if (!attr_set[v]) {
                if (hipFuncSetAttribute(fns[v], hipFuncAttributeMaxDynamicSharedMemorySize, (int)GR_LDS) != hipSuccess)
                    return fail(ATLAS_ERR_HIP, "int8 GEMM: LDS attribute");
                attr_set[v] = true;
            }
            const int NWr = mode ? GR_BN / 2 : GR_BN;
            const int Tr = ((a.M + GR_BM - 1) / GR_BM) * ((a.N + NWr - 1) / NWr) * a.ksplit, br = 8 * ((Tr + 7) / 8);
            switch (v) {
                case 0: ATLAS_KLAUNCH((w4_gemm_i8r_kernel<0, false>), dim3(br), dim3(GR_THREADS), GR_LDS, st, a); break;
                case 1: ATLAS_KLAUNCH((w4_gemm_i8r_kernel<0, true>), dim3(br), dim3(GR_THREADS), GR_LDS, st, a); break;
                case 2: ATLAS_KLAUNCH((w4_gemm_i8r_kernel<1, false>), dim3(br), dim3(GR_THREADS), GR_LDS, st, a); break;
                default: ATLAS_KLAUNCH((w4_gemm_i8r_kernel<1, true>), dim3(br), dim3(GR_THREADS), GR_LDS, st, a); break;
            }
            ATLAS_LAUNCH_CHECK("w4_gemm_i8r_kernel");
            return ATLAS_OK;
        }
        ATLAS_CHECK_SHAPE(!a.zq_hi, "int8 digits of z need the ring kernel");
        const int T8 = MT * NT * a.ksplit, b8 = 8 * ((T8 + 7) / 8);
        if (mode == 0) ATLAS_KLAUNCH((w4_gemm_i8_kernel<0>), dim3(b8), dim3(G8_THREADS), 0, st, a);
        else ATLAS_KLAUNCH((w4_gemm_i8_kernel<1>), dim3(b8), dim3(G8_THREADS), 0, st, a);
        ATLAS_LAUNCH_CHECK("w4_gemm_i8_kernel");
        return ATLAS_OK;
    }
    const int krange = a.ksplit > 1 ? a.kchunk : a.K;
    if (mode == 0 && a.M <= 16 && krange % 128 == 0) {   // a few rows: weights straight to the matrix cores
        const int Nw = (a.N + 16 * SK_TILES - 1) / (16 * SK_TILES);
        const int bs = (Nw * a.ksplit + SK_WAVES - 1) / SK_WAVES;
        ATLAS_KLAUNCH(w4_skinny_kernel, dim3(bs), dim3(64 * SK_WAVES), 0, st, a);
        ATLAS_LAUNCH_CHECK("w4_skinny_kernel");
        return ATLAS_OK;
    }
    if (mode == 0 && a.M <= 16) {   // a few rows: one 16-row tile
        const int T16 = NT * a.ksplit, b16 = 8 * ((T16 + 7) / 8);
        ATLAS_KLAUNCH(w4_gemm16_kernel, dim3(b16), dim3(GM_THREADS), 0, st, a);
        ATLAS_LAUNCH_CHECK("w4_gemm16_kernel");
        return ATLAS_OK;
    }
    const int T = MT * NT * a.ksplit, blocks = 8 * ((T + 7) / 8);
    if (mode == 0) ATLAS_KLAUNCH((w4_gemm_kernel<0>), dim3(blocks), dim3(GM_THREADS), 0, st, a);
    else ATLAS_KLAUNCH((w4_gemm_kernel<1>), dim3(blocks), dim3(GM_THREADS), 0, st, a);
    ATLAS_LAUNCH_CHECK("w4_gemm_kernel");
    return ATLAS_OK;
}

int launch_pf_embed(const int32_t* tokens, int n, const uint16_t* emb, int vocab, int d, float* X, uint16_t* p_hi,
                    uint16_t* p_lo, int ldp, int* status, hipStream_t st) {
    prof_mark("pf_embed", st);
    ATLAS_KLAUNCH(pf_embed_kernel, dim3(n), dim3(256), 0, st, tokens, n, emb, vocab, d, X, p_hi, p_lo, ldp, status);
    ATLAS_LAUNCH_CHECK("pf_embed_kernel");
    return ATLAS_OK;
}

int launch_pf_rope(const PfRopeArgs& a, hipStream_t st) {
    const int nqkv = (a.Hq + 2 * a.Hkv) * 128;
    ATLAS_CHECK_SHAPE(a.S >= 1 && a.S <= 4 && (a.S == 1 || a.pstride >= nqkv) && a.ld >= (a.S - 1) * a.pstride + nqkv &&
                          nqkv * 4 <= 64 * 1024,
                      "qkv partials: S=%d pstride=%d ld=%d", a.S, a.pstride, a.ld);
    prof_mark("pf_qk_norm_rope", st);
    const int nq = a.Hq * 128, npairs = (a.Hq + a.Hkv) * 64;
    if (a.S <= 2 && nqkv <= 256 * 28 && nq % 256 == 0 && npairs <= 256 * 12)
        ATLAS_KLAUNCH((pf_rope_kernel<28, 12>), dim3(a.n), dim3(256), (size_t)nqkv * 4, st, a);
    else
        ATLAS_KLAUNCH((pf_rope_kernel<0, 0>), dim3(a.n), dim3(256), (size_t)nqkv * 4, st, a);
    ATLAS_LAUNCH_CHECK("pf_rope_kernel");
    return ATLAS_OK;
}

int launch_pf_commit(const PfCommitArgs& a, hipStream_t st) {
    const int npos = a.ring ? (int)std::min<int64_t>(a.n, a.slots) : a.n;
    prof_mark("pf_kv_commit", st);
    ATLAS_KLAUNCH(pf_commit_kernel, dim3(npos), dim3(256), 0, st, a);
    ATLAS_LAUNCH_CHECK("pf_commit_kernel");
    return ATLAS_OK;
}

int launch_pf_attn(const PfAttnArgs& a, hipStream_t st) {
    const int G = a.Hq / a.Hkv;
    dim3 grid(a.Hkv, (a.n + PF_QT - 1) / PF_QT);
    prof_mark(a.window > 0 ? "pf_attn_window" : "pf_attn_full", st);
    switch (G) {
#define C(G_)                                                                   \
    case G_:                                                                    \
        if (a.kv_bf16) ATLAS_KLAUNCH((pf_attn_kernel<G_, true>), grid, dim3(64 * G_), 0, st, a);    \
        else ATLAS_KLAUNCH((pf_attn_kernel<G_, false>), grid, dim3(64 * G_), 0, st, a);              \
        break;
        C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8)
#undef C
        default: return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, "Hq/Hkv=%d > 8", G);
    }
    ATLAS_LAUNCH_CHECK("pf_attn_kernel");
    return ATLAS_OK;
}

int launch_pf_split(const float* X, int M, int K, int ldx, uint16_t* p_hi, uint16_t* p_lo, int ldp, hipStream_t st) {
    prof_mark("pf_split", st);
    ATLAS_KLAUNCH(pf_split_kernel, dim3(M), dim3(256), 0, st, X, K, ldx, p_hi, p_lo, ldp);
    ATLAS_LAUNCH_CHECK("pf_split_kernel");
    return ATLAS_OK;
}

bool residual_digits_ok(int group, int d) { return (group == 128 || group == 256) && d % 1024 == 0; }

int launch_pf_residual(float* X, const float* A, int lda, int S, const float* g, int n, int d, float eps,
                       uint16_t* p_hi, uint16_t* p_lo, int ldp, hipStream_t st, const Q8Out* q) {
    ATLAS_CHECK_SHAPE((S == 1 || S == 2) && lda % 4 == 0 && lda >= S * d && d % 4 == 0, "residual partials");
    ATLAS_CHECK_SHAPE(!q || residual_digits_ok(q->group, d), "residual digits: group %d, d %d", q ? q->group : 0, d);
    prof_mark("pf_residual_norm", st);
    int8_t *qh = q ? q->hi : nullptr, *qm = q ? q->mid : nullptr, *ql = q ? q->lo : nullptr;
    float *qs = q ? q->s : nullptr, *qsum = q ? q->sum : nullptr;
    const int qg = q ? q->group : 128;
    if (d <= 4 * 256 * 5)
        ATLAS_KLAUNCH((pf_residual_kernel<5>), dim3(n), dim3(256), 0, st, X, A, lda, S, g, d, eps, p_hi, p_lo, ldp, qh,
                      qm, ql, qs, qsum, qg);
    else
        ATLAS_KLAUNCH((pf_residual_kernel<0>), dim3(n), dim3(256), 0, st, X, A, lda, S, g, d, eps, p_hi, p_lo, ldp, qh,
                      qm, ql, qs, qsum, qg);
    ATLAS_LAUNCH_CHECK("pf_residual_kernel");
    return ATLAS_OK;
}

}  // namespace atlas
