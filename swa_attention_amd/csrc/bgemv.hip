// Batched decode projections on the int8 matrix cores: y[v] = W x[v] for a few vectors
// (B <= 8) of one W4 matrix, or two sharing a launch, reading the weights once.
//
// Source: "ATLAS-OLMo-3-32B-Think-v4", Limitations & roadmap (batched decode after the
// batch-1 path); the product is the W4 projection of "What ATLAS implements for the W4
// path" for each vector of the batch.
//
// Operands. v_mfma_i32_16x16x64_i8 takes A = the raw 4-bit codes c of 16 weight rows
// (a mask and a shift per code word: low nibbles are a word's columns 0,2,4,6, high
// nibbles 1,3,5,7) and B = 16 columns of activation digits: columns 0-7 of the first
// MFMA are the h digits of vectors 0-7, columns 8-15 their m digits, columns 0-7 of the
// second the l digits (see BQ: the encoders store them fragment by fragment, so each
// B operand is one contiguous kilobyte). Per 128-column block and row the three digit sums are
// exact in int32; with Y = 256 sum(c h) + sum(c m) and L = sum(c l),
//   sum((c - z) n) = 256 (Y - z sy) + (L - z sl)
// is formed from two exact integers and one f32 fma, then scaled by s_w s_x into the
// row's f32 sum.
//
// Work. K is cut into chunks of 512 columns (4 blocks; the last chunk may be shorter,
// its last block 64 columns). A block has CB waves, one per chunk of its K range, and a
// run of 16-row tiles; each wave keeps its chunk's activation fragments in registers
// (8 k-steps x 2 MFMAs) and streams the tiles, one tile's loads in flight while the
// previous tile is multiplied. Each lane reads 16 bytes of one row per block, so one
// wave instruction reads 16 rows x 64 contiguous bytes (plain loads: measured within
// 5% of 512-byte row runs on this matrix shape, where nontemporal ones lost 17%). The
// chunk partials of each tile meet in LDS and are summed in chunk order, so results do
// not depend on timing. K ranges too long for one block (CB chunks) are split over
// blocks into partial sums.
#include "bgemv.h"
#include "gemv.h"

namespace atlas {

typedef int bg_i32x4 __attribute__((ext_vector_type(4)));

size_t bq_bytes(int rows, int K) {
    const int nb = (K + 127) / 128;
    return (size_t)nb * 4096 + 3 * align_up((size_t)rows * nb * 4, 256);
}

BQ bq_carve(void* base, int rows, int K) {
    BQ q{};
    q.nbs = (K + 127) / 128;
    q.ldq = q.nbs * 128;
    char* b = (char*)base;
    q.p = (int8_t*)b;
    const size_t off = (size_t)q.nbs * 4096;
    const size_t sb = align_up((size_t)rows * q.nbs * 4, 256);
    q.sy = (int*)(b + off);
    q.sl = (int*)(b + off + sb);
    q.sx = (float*)(b + off + 2 * sb);
    return q;
}

// ---- encoding ---------------------------------------------------------------------------------

// One thread per 8 columns: grid (blocks over 16 * nb threads, B).
__global__ __launch_bounds__(256) void bq_encode_kernel(const float* X, int ldx, int K, BQ q) {
    const int v = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;   // 8-column group
    const int col0 = 8 * i;
    float x[8];
    if (col0 < K) {
        const float4 a = *reinterpret_cast<const float4*>(X + (size_t)v * ldx + col0);
        const float4 b = *reinterpret_cast<const float4*>(X + (size_t)v * ldx + col0 + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) x[j] = 0.f;
    }
    if (col0 < q.ldq) bq_encode_row16(x, q, v, col0, i >> 4);   // whole rows of 16 lanes (ldq % 128 == 0)
}

int launch_bq_encode(const float* X, int ldx, int B, int K, const BQ& q, hipStream_t st) {
    ATLAS_CHECK_SHAPE(K % 8 == 0 && ldx % 4 == 0 && K <= q.ldq, "encode: K=%d ldx=%d", K, ldx);
    const int threads = q.ldq / 8;   // whole 16-lane rows: ldq is a multiple of 128
    prof_mark("bq_encode", st);
    ATLAS_KLAUNCH(bq_encode_kernel, dim3((threads + 255) / 256, B), dim3(256), 0, st, X, ldx, K, q);
    ATLAS_LAUNCH_CHECK("bq_encode_kernel");
    return ATLAS_OK;
}

// ---- the GEMV ----------------------------------------------------------------------------------

constexpr int BG_NBM = 6;   // blocks of 128 columns per wave chunk, at most (template NB)
// tiles in flight per wave (register stages): four, three for 6-block chunks (whose
// fourth stage would not fit in 256 registers); two for waves of at most BG_SHORT_TPB
// tiles, whose first loads are most of their work (a deeper ring only makes the
// launch's opening burst larger)
template <int NB>
constexpr int bg_stages() { return NB >= 6 ? 3 : 4; }
constexpr int BG_SHORT_TPB = 4;

struct BgemvArgs {
    W4View W0, W1;
    int T0, T1;             // 16-row tiles of W0, then of W1
    BQ x;
    int B, K, group;
    int NBT;                // blocks of 128 columns (the last may hold 64)
    int NB, CB, S, TPB;     // blocks per chunk, waves (chunks) per block, K splits, tiles per block
    int NBy;                // > 0: waves 4-7 take chunks of NBy blocks, waves 0-3 of NB (CB = 8)
    BgemvOut o0, o1;
};

template <int NB>
struct BgStage {
    uint32_t cw[NB][4];       // codes of block t: the lane's 16 bytes of its row
    uint32_t sr[NB > 4 ? 2 : 1];   // raw scale and zero word of (row 4q + c % 4, block c / 4
    uint32_t zr[NB > 4 ? 2 : 1];   //   and 4 + c / 4), converted only when multiplied
};

// One 32-bit value per (row, block): the group scale as f32 (whose low 13 bits are
// zero, since it comes from f16 or bf16) with the zero point in its low 4 bits.
__device__ __forceinline__ uint32_t bg_scale_zero(uint32_t sraw, uint32_t zw, int g, int sdt, int zsym) {
    const float s = scale_to_f32((uint16_t)sraw, sdt);
    const uint32_t z = zsym ? 8u : (zw >> (4 * (g & 7))) & 15u;
    return __float_as_uint(s) | z;
}

template <int SRC>
__device__ __forceinline__ uint32_t bg_bcast16(uint32_t v) {   // lane SRC of each row of 16
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x10 | (SRC << 5));
}

template <int NB, int NS>
__global__ __launch_bounds__(512) void bgemv_kernel(BgemvArgs a) {
    extern __shared__ float4 s_part[];   // [TPB][CB][64]
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, q = lane >> 4;
    const int split = (int)blockIdx.x % a.S, tb = (int)blockIdx.x / a.S;
    const int chunk = split * a.CB + w;
    // first block and length of this wave's chunk. With NBy > 0 the older wave of each
    // SIMD (waves 0-3, served first by the memory system) takes the longer chunk, so that
    // the two waves of a SIMD finish together
    const int w4 = w & 3;
    const int blk0 = a.NBy ? split * 4 * (NB + a.NBy) + (w < 4 ? w4 * NB : 4 * NB + w4 * a.NBy) : chunk * NB;
    const int nb = max(0, min(a.NBy && w >= 4 ? a.NBy : NB, a.NBT - blk0));   // blocks of this wave
    const int kc0 = blk0 * 128;
    const bool tail = (a.K & 127) != 0 && blk0 + nb == a.NBT;   // its last block holds 64 columns
    const int Ttot = a.T0 + a.T1;
    const int it0 = tb * a.TPB, nit = min(a.TPB, Ttot - it0);
    const int B = a.B;

    // activation fragments of this wave's chunk: k-step 2t + u, MFMA j; slot 16 j + c is
    // plane (16 j + c) / 8 of vector (16 j + c) % 8 (plane 3: zero)
    bg_i32x4 bf[2 * NB][2];
    int gsy[NB], gsl[NB];
    float gsx[NB];
    {
        const int vv = min(c & 7, B - 1);
#pragma unroll
        for (int t = 0; t < NB; t++) {
            const int tt = min(t, max(nb, 1) - 1);
#pragma unroll
            for (int u = 0; u < 2; u++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int idx = 16 * j + c, pl = idx >> 3, vec = idx & 7;
                    const int8_t* src = a.x.p + (size_t)((blk0 + tt) * 2 + u) * 2048 + j * 1024 + 16 * lane;
                    bf[2 * t + u][j] = bg_i32x4{0, 0, 0, 0};
                    if (pl < 3 && vec < B && t < nb) bf[2 * t + u][j] = *reinterpret_cast<const bg_i32x4*>(src);
                }
            const size_t o = (size_t)vv * a.x.nbs + min(blk0 + tt, a.x.nbs - 1);
            gsy[t] = a.x.sy[o];
            gsl[t] = a.x.sl[o];
            gsx[t] = a.x.sx[o];
        }
    }

    // loads only (no use of a loaded value here, so nothing waits for them): codes of
    // the chunk's blocks (clamped to the last block for the short last chunk), raw scale
    // and zero words
    const int nbl = max(nb, 1) - 1;
    auto load = [&](int it, BgStage<NB>& S) {
        const int T = it0 + min(it, nit - 1);
        const bool second = T >= a.T0;
        const W4View& W = second ? a.W1 : a.W0;
        const int tl = second ? T - a.T0 : T;
        const int row = min(16 * tl + c, W.N - 1);
        const uint32_t* rq = W.qweight + (size_t)row * W.KW + kc0 / 8;
#pragma unroll
        for (int t = 0; t < NB; t++) {
            const int tt = min(t, nbl);
            const int qq = (tail && tt == nbl) ? (q & 1) : q;   // no read past the row's end
            const uint4 v = *reinterpret_cast<const uint4*>(rq + 16 * tt + 4 * qq);
            S.cw[t][0] = v.x;
            S.cw[t][1] = v.y;
            S.cw[t][2] = v.z;
            S.cw[t][3] = v.w;
        }
        const int rs = min(16 * tl + 4 * q + (c & 3), W.N - 1);
#pragma unroll
        for (int h = 0; h < (NB > 4 ? 2 : 1); h++) {
            const int g = min((kc0 + 128 * min(4 * h + (c >> 2), nbl)) / a.group, W.G - 1);
            S.sr[h] = W.scales[(size_t)rs * W.G + g];
            S.zr[h] = W.zeros[(size_t)rs * W.zstride + (g >> 3)];
        }
    };

    const int sdt = a.W0.scale_dtype, zsym = a.W0.zsym;   // both matrices share the format
    auto compute = [&](int it, const BgStage<NB>& S) {
        uint32_t sz[NB > 4 ? 2 : 1];
#pragma unroll
        for (int h = 0; h < (NB > 4 ? 2 : 1); h++) {
            const int g = min((kc0 + 128 * min(4 * h + (c >> 2), nbl)) / a.group, a.W0.G - 1);
            sz[h] = bg_scale_zero(S.sr[h], S.zr[h], g, sdt, zsym);
        }
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NB; t++) {
            if (t < nb) {
                const uint32_t* wv = S.cw[t];
                const bg_i32x4 a0 = {(int)(wv[0] & 0x0F0F0F0Fu), (int)((wv[0] >> 4) & 0x0F0F0F0Fu),
                                     (int)(wv[1] & 0x0F0F0F0Fu), (int)((wv[1] >> 4) & 0x0F0F0F0Fu)};
                const bg_i32x4 a1 = {(int)(wv[2] & 0x0F0F0F0Fu), (int)((wv[2] >> 4) & 0x0F0F0F0Fu),
                                     (int)(wv[3] & 0x0F0F0F0Fu), (int)((wv[3] >> 4) & 0x0F0F0F0Fu)};
                bg_i32x4 d0 = {0, 0, 0, 0}, d1 = {0, 0, 0, 0};
                d0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bf[2 * t][0], d0, 0, 0, 0);
                d1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bf[2 * t][1], d1, 0, 0, 0);
                d0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bf[2 * t + 1][0], d0, 0, 0, 0);
                d1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bf[2 * t + 1][1], d1, 0, 0, 0);
                const uint32_t szt = sz[t >> 2];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    // D[row 4 q + r][column c]: the m sums of vector c sit in column c + 8
                    uint32_t v;
                    switch (4 * (t & 3) + r) {   // scale | zero of row 4 q + r, block t
#define BGC(k) case k: v = bg_bcast16<k>(szt); break;
                        BGC(0) BGC(1) BGC(2) BGC(3) BGC(4) BGC(5) BGC(6) BGC(7)
                        BGC(8) BGC(9) BGC(10) BGC(11) BGC(12) BGC(13) BGC(14) default: v = bg_bcast16<15>(szt);
#undef BGC
                    }
                    const int z = (int)(v & 15u);
                    const float sw = __uint_as_float(v & ~15u);
                    const int H = d0[r];
                    const int Mv = __builtin_amdgcn_update_dpp(0, d0[r], 0x128, 0xF, 0xF, false);   // row_ror:8
                    const int L = d1[r];
                    const int Y = H * 256 + Mv - z * gsy[t];
                    const int Lz = L - z * gsl[t];
                    const float f = fmaf(256.f, (float)Y, (float)Lz);
                    acc[r] = fmaf(f, sw * gsx[t], acc[r]);
                }
            }
        }
        s_part[(it * a.CB + w) * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    };

    // NS-stage register ring: the loads of tile it + NS - 1 are issued before tile it is
    // multiplied. Every load is issued (past the last tile they re-read its addresses,
    // from L2), so the compiler can count the loads in flight and waits only for the
    // oldest stage.
    BgStage<NB> S[NS];
#pragma unroll
    for (int k = 0; k < NS - 1; k++) load(k, S[k]);
    for (int it = 0; it < nit; it += NS) {
#pragma unroll
        for (int k = 0; k < NS; k++) {
            load(it + k + NS - 1, S[(k + NS - 1) % NS]);
            if (it + k < nit) compute(it + k, S[k]);
        }
    }
    __syncthreads();
    // y[split][v][row] = sum over the block's chunks, in chunk order
    const float* sp = reinterpret_cast<const float*>(s_part);
    const int per = B * 16;
    for (int o = threadIdx.x; o < nit * per; o += blockDim.x) {
        const int it = o / per, rem = o - it * per, v = rem >> 4, rr = rem & 15;
        const int ln = (rr >> 2) * 16 + v, r = rr & 3;
        float sum = 0.f;
        for (int ww = 0; ww < a.CB; ww++) sum += sp[((it * a.CB + ww) * 64 + ln) * 4 + r];
        const int T = it0 + it;
        const bool second = T >= a.T0;
        const int tl = second ? T - a.T0 : T;
        const int row = 16 * tl + rr;
        const int N = second ? a.W1.N : a.W0.N;
        if (row < N) {
            const BgemvOut& out = second ? a.o1 : a.o0;
            out.y[(size_t)split * out.ys + (size_t)v * out.ldy + row] = sum;
        }
    }
}

bool bgemv_supported(const W4View& W, int group) {
    return W.K % 64 == 0 && W.K >= 64 && group > 0 && group % 128 == 0;
}

struct BgShape {
    int NBT, NB, CB, S;
    int NBy = 0;   // > 0: chunks of NB blocks for waves 0-3 and NBy for waves 4-7 (CB = 8)
};

// Waves per SIMD that the registers of a chunk of NB blocks allow (at the stage counts
// of bg_stages).
static int bg_waves_per_simd(int NB) { return NB <= 1 ? 8 : NB == 2 ? 4 : NB == 3 ? 3 : 2; }

// Chunks of NB blocks, CB waves per block (at most 8), S blocks along K. Timed at 8
// vectors on the decode shapes (chunk lengths 1-6, each with its best split):
//   qkv 7,168 x 5,120:    13.4 us at 4 blocks (18.0 at 5, one split)
//   o 5,120 x 6,144:      14.7 us at 4 blocks (17.7 at 6)
//   gate+up 2 x 27,648 x 5,120: 38.9 us at 5 blocks, one split (43.4 at 4; 200+ at 1-2)
//   down 5,120 x 27,648:  27.9 us at 6 blocks (28.9 at 2, 31.1 at 4)
// and, at those chunk lengths, every divisor of the chunk count as the waves per block:
// the largest (up to 8) was fastest for all four (qkv 12.7 us at 5 against 13.4-14.4,
// o 12.3 at 6 against 12.8-15.5, gate+up 40.9 at 8 against 43-54, down 28.1 at 6
// against 29-33).
// Each wave loads its chunk's activation fragments (about 3 KB per block, from L2) once,
// so a chunk pays off over many tiles: with many row tiles (a wide matrix) the longest
// chunk that covers K in one block of waves; otherwise 4 blocks (6 for a long K),
// K split over blocks. The waves of a block: the largest divisor of the chunk count up
// to 8.
static BgShape bg_shape(int K, int tiles) {
    BgShape sh{(K + 127) / 128, 1, 1, (K + 127) / 128};
    static const int wide[6] = {6, 5, 4, 3, 2, 1}, narrow_short[6] = {4, 3, 2, 6, 5, 1},
                     narrow_long[6] = {6, 4, 3, 2, 5, 1};
    const bool is_wide = tiles >= 1024;
    if (is_wide && sh.NBT % 40 == 0 && sh.NBT / 40 <= 1) {   // 6 + 4 blocks per SIMD's wave pair
        sh.NB = 6;
        sh.NBy = 4;
        sh.CB = 8;
        sh.S = sh.NBT / 40;
        return sh;
    }
    if (!is_wide && K > 8192 && sh.NBT % 36 == 0) {   // 5 + 4 blocks per SIMD's wave pair, K split
        sh.NB = 5;
        sh.NBy = 4;
        sh.CB = 8;
        sh.S = sh.NBT / 36;
        return sh;
    }
    const int* order = is_wide ? wide : (K <= 8192 ? narrow_short : narrow_long);
    for (int i = 0; i < 6; i++) {
        const int nb = order[i];
        if (sh.NBT % nb) continue;
        const int nch = sh.NBT / nb;
        if (is_wide && nch > 8) continue;   // one split of K
        int cb = 1;
        for (int d = std::min(8, nch); d >= 1; d--)
            if (nch % d == 0) {
                cb = d;
                break;
            }
        sh.NB = nb;
        sh.CB = cb;
        sh.S = nch / cb;
        return sh;
    }
    // no chunk length divides the blocks evenly with one split: one block per chunk
    int cb = 1;
    for (int d = std::min(8, sh.NBT); d >= 1; d--)
        if (sh.NBT % d == 0) {
            cb = d;
            break;
        }
    sh.NB = 1;
    sh.CB = cb;
    sh.S = sh.NBT / cb;
    return sh;
}

int bgemv_splits(int K, int N0, int N1) { return bg_shape(K, (N0 + 15) / 16 + (N1 + 15) / 16).S; }

// Tiles per block: the fewest tiles per wave over all rounds of the grid (blocks per CU
// from the registers of the chunk), preferring a single round; at most 150 KB of LDS
// partials per CU.
static int bg_tiles_per_block(int Ttot, int S, int CB, int NB) {
    const int bpc = std::max(1, bg_waves_per_simd(NB) * 4 / CB), slots = 256 * bpc;
    int best = 1, best_cost = 1 << 30, best_rounds = 1 << 30;
    for (int tpb = 1; tpb * CB * bpc <= 150 && tpb <= Ttot; tpb++) {
        const int blocks = S * ((Ttot + tpb - 1) / tpb);
        const int rounds = (blocks + slots - 1) / slots;
        const int cost = rounds * tpb;
        if (cost < best_cost || (cost == best_cost && rounds < best_rounds)) {
            best = tpb;
            best_cost = cost;
            best_rounds = rounds;
        }
    }
    return best;
}

template <int NB, int NS>
static int bg_launch(const BgemvArgs& a, int blocks, size_t lds, hipStream_t st) {
    static bool attr_set = false;   // per instantiation: LDS partials above 64 KB
    if (!attr_set) {
        if (hipFuncSetAttribute((const void*)bgemv_kernel<NB, NS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024) != hipSuccess)
            return fail(ATLAS_ERR_HIP, "bgemv: LDS attribute");
        attr_set = true;
    }
    ATLAS_KLAUNCH((bgemv_kernel<NB, NS>), dim3(blocks), dim3(64 * a.CB), lds, st, a);
    return ATLAS_OK;
}

int launch_bgemv(const W4View& W0, int group, const W4View* W1, const BQ& x, int B, const BgemvOut& o0,
                 const BgemvOut* o1, hipStream_t st, const char* label) {
    ATLAS_CHECK_SHAPE(B >= 1 && B <= BG_MAX_B, "batched GEMV: B=%d", B);
    ATLAS_CHECK_SHAPE(bgemv_supported(W0, group), "batched GEMV: K=%d group=%d", W0.K, group);
    ATLAS_CHECK_SHAPE(W0.K <= x.ldq, "batched GEMV: K=%d > encoded %d", W0.K, x.ldq);
    if (W1)
        ATLAS_CHECK_SHAPE(W1->K == W0.K && W1->G == W0.G && W1->zsym == W0.zsym && W1->scale_dtype == W0.scale_dtype,
                          "batched GEMV: the two matrices differ in format");
    const int tiles = (W0.N + 15) / 16 + (W1 ? (W1->N + 15) / 16 : 0);
    const BgShape sh = bg_shape(W0.K, tiles);
    BgemvArgs a{};
    a.W0 = W0;
    a.W1 = W1 ? *W1 : W0;
    a.T0 = (W0.N + 15) / 16;
    a.T1 = W1 ? (W1->N + 15) / 16 : 0;
    a.x = x;
    a.B = B;
    a.K = W0.K;
    a.group = group;
    a.NBT = sh.NBT;
    a.NB = sh.NB;
    a.NBy = sh.NBy;
    a.CB = sh.CB;
    a.S = sh.S;
    a.TPB = bg_tiles_per_block(a.T0 + a.T1, a.S, a.CB, a.NB);
    a.o0 = o0;
    a.o1 = o1 ? *o1 : o0;
    const int blocks = a.S * ((a.T0 + a.T1 + a.TPB - 1) / a.TPB);
    const size_t lds = (size_t)a.TPB * a.CB * 64 * sizeof(float4);
    prof_mark(label, st);
    const bool short_run = a.TPB <= BG_SHORT_TPB;
    switch (a.NB) {
#define BGL(nb_)                                                                                           \
    case nb_: {                                                                                            \
        if (short_run) {                                                                                   \
            if (int rc_ = bg_launch<nb_, 2>(a, blocks, lds, st)) return rc_;                               \
        } else if (int rc_ = bg_launch<nb_, bg_stages<nb_>()>(a, blocks, lds, st)) {                       \
            return rc_;                                                                                    \
        }                                                                                                  \
        break;                                                                                             \
    }
        BGL(1) BGL(2) BGL(3) BGL(4) BGL(5) BGL(6)
#undef BGL
        default: return fail(ATLAS_ERR_UNSUPPORTED_SHAPE, "bgemv: chunk of %d blocks", a.NB);
    }
    ATLAS_LAUNCH_CHECK("bgemv_kernel");
    return ATLAS_OK;
}

}  // namespace atlas

using namespace atlas;

static size_t gemv_batch_ws(const atlas_w4* W, int B) {
    const int S = bgemv_splits(W->K, W->N, 0);
    size_t b = align_up(bq_bytes(B, W->K), 256);
    if (S > 1) b += align_up((size_t)S * B * W->N * 4, 256);
    return b;
}

static int validate_gemv_batch(const atlas_w4* W, int B) {
    int rc = validate_w4(W);
    if (rc) return rc;
    ATLAS_CHECK_ARG(B >= 1 && B <= BG_MAX_B, "B=%d outside [1, %d]", B, BG_MAX_B);
    const W4View v = w4_view(W->qweight, W->scales, W->zeros, W->N, W->K, W->group, W->scale_dtype);
    ATLAS_CHECK_SHAPE(bgemv_supported(v, W->group), "batched GEMV needs K %% 64 == 0 and a group that is a multiple "
                      "of 128 (K=%d group=%d)", W->K, W->group);
    return ATLAS_OK;
}

extern "C" size_t atlas_w4_gemv_batch_workspace_bytes(const atlas_w4* W, int32_t B) {
    if (validate_gemv_batch(W, B) != ATLAS_OK) return 0;
    return gemv_batch_ws(W, B);
}

extern "C" int atlas_w4_gemv_batch(const atlas_w4* W, const float* x, int32_t B, float* y, void* ws, size_t ws_bytes,
                                   void* stream) {
    int rc = validate_gemv_batch(W, B);
    if (rc) return rc;
    ATLAS_CHECK_ARG(x && y && ws, "null x, y or workspace");
    const size_t need = gemv_batch_ws(W, B);
    if (ws_bytes < need) return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
    hipStream_t st = (hipStream_t)stream;
    const BQ q = bq_carve(ws, B, W->K);
    if ((rc = launch_bq_encode(x, W->K, B, W->K, q, st))) return rc;
    const int S = bgemv_splits(W->K, W->N, 0);
    float* part = S > 1 ? (float*)((char*)ws + align_up(bq_bytes(B, W->K), 256)) : y;
    const W4View v = w4_view(W->qweight, W->scales, W->zeros, W->N, W->K, W->group, W->scale_dtype);
    const BgemvOut o{part, (size_t)B * W->N, W->N};
    if ((rc = launch_bgemv(v, W->group, nullptr, q, B, o, nullptr, st, "w4_gemv_batch"))) return rc;
    if (S > 1) return launch_sum_partials(part, S, B * W->N, y, st);
    return ATLAS_OK;
}
