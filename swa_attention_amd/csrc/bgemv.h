// Batched W4 GEMV on the int8 matrix cores (internal interface).
#pragma once
#include "gemv_core.h"

namespace atlas {

// A few activation vectors x[v] (v < 8) of K columns as 24-bit block fixed point: per
// block of 128 columns, s = 2^e and integers n = rint(x / s) with |n| <= 127 * 2^16,
// split into balanced digits n = 65536 h + 256 m + l (h, m, l int8). The digits are
// stored in the order the batched GEMV's MFMA B operand takes them, 4 KB per block:
// fragment (block b, k-step u of the block, MFMA j) is 64 lanes x 16 bytes at
// ((b * 2 + u) * 2 + j) * 1024, lane 16 q + c holding columns 32 q + 16 u .. + 15 of the
// block (the bytes of every 8 columns in the order 0,2,4,6,1,3,5,7) of plane
// (16 j + c) / 8 of vector (16 j + c) % 8; the slots of plane 3 and of absent vectors
// are never written (the GEMV does not load them). Per (vector, block): sy = sum of
// (256 h + m), sl = sum of l, sx = s.
struct BQ {
    int8_t* p;
    int ldq;          // K rounded up to a multiple of 128 (the encoded width)
    int* sy;
    int* sl;
    float* sx;
    int nbs;          // blocks per vector row of sy, sl, sx (ldq / 128)
};

constexpr int BG_MAX_B = 8;          // vectors per launch

size_t bq_bytes(int rows, int K);
BQ bq_carve(void* base, int rows, int K);

// Whether the batched GEMV takes W with groups of `group` columns (K % 64 == 0, group a
// multiple of 128).
bool bgemv_supported(const W4View& W, int group);
// Partial sums the batched GEMV writes for W0 [N0][K] (and W1 [N1][K] in the same
// launch): its split of K over blocks.
int bgemv_splits(int K, int N0, int N1 = 0);

// y[s][v][n] (s < bgemv_splits(K), split stride ys, vector stride ldy) partial products
// of W [N][K] with x[v], v < B. With W1 (same K and group), the launch also computes
// y1 = W1 x the same way.
struct BgemvOut {
    float* y;
    size_t ys;
    int ldy;
};
int launch_bgemv(const W4View& W0, int group, const W4View* W1, const BQ& x, int B, const BgemvOut& o0,
                 const BgemvOut* o1, hipStream_t st, const char* label);
// Encodes rows X [B][ldx] (K columns, K % 8 == 0) into q.
int launch_bq_encode(const float* X, int ldx, int B, int K, const BQ& q, hipStream_t st);

constexpr float BQ_MAX = 8323072.f;   // 127 * 65536

__device__ __forceinline__ int row16_sum_i(int v) {
    v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);   // row_half_mirror
    v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);   // row_mirror
    return v;
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return v;
}

// Encoding of the 128-column block `blk` of vector v held by one row of 16 lanes (lane
// j of the row: the 8 columns col0 = 128 blk + 8 j .. + 7, zero past the end). Every lane
// of the wave takes part (the block maximum and sums are row reductions); the row's
// first lane writes the block's scale and digit sums.
__device__ __forceinline__ void bq_encode_row16(const float x[8], const BQ& q, int v, int col0, int blk) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) mx = fmaxf(mx, fabsf(x[i]));
    mx = row16_max(mx);
    int e;
    (void)frexpf(mx / BQ_MAX, &e);   // s = 2^e >= max|x| / BQ_MAX (s = 1 for a zero block)
    const float inv = ldexpf(1.f, -e);
    uint32_t H[2] = {0u, 0u}, M[2] = {0u, 0u}, L[2] = {0u, 0u};
    int sy = 0, sl = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int n = (int)fminf(fmaxf(rintf(x[i] * inv), -BQ_MAX), BQ_MAX);   // x * inv is exact
        const int l = ((n + 128) & 255) - 128;
        const int n1 = (n - l) >> 8;   // exact: n - l is a multiple of 256
        const int m = ((n1 + 128) & 255) - 128;
        const int h = (n1 - m) >> 8;
        sy += n1;
        sl += l;
        const int word = i & 1, sh = 8 * (i >> 1);   // column i -> byte i/2 (even i) or 4 + i/2 (odd)
        H[word] |= ((uint32_t)h & 0xFFu) << sh;
        M[word] |= ((uint32_t)m & 0xFFu) << sh;
        L[word] |= ((uint32_t)l & 0xFFu) << sh;
    }
    sy = row16_sum_i(sy);
    sl = row16_sum_i(sl);
    // columns 8 j16 .. + 7 of the block (j16 = lane in the row): k-step u = (j16 / 2) % 2,
    // lane quarter q = j16 / 4, byte half j16 % 2 of the 16-byte fragment slot; plane P of
    // vector v sits in slot 8 P + v (MFMA (8 P + v) / 16, column (8 P + v) % 16)
    const int j16 = threadIdx.x & 15, u = (j16 >> 1) & 1, qq = j16 >> 2;
    int8_t* base = q.p + (size_t)blk * 4096 + u * 2048 + (size_t)qq * 256 + 8 * (j16 & 1);
    *reinterpret_cast<uint2*>(base + v * 16) = make_uint2(H[0], H[1]);             // slot v: MFMA 0
    *reinterpret_cast<uint2*>(base + (8 + v) * 16) = make_uint2(M[0], M[1]);       // slot 8 + v: MFMA 0
    *reinterpret_cast<uint2*>(base + 1024 + v * 16) = make_uint2(L[0], L[1]);      // slot 16 + v: MFMA 1
    if ((threadIdx.x & 15) == 0) {
        const size_t o = (size_t)v * q.nbs + blk;
        q.sy[o] = sy;
        q.sl[o] = sl;
        q.sx[o] = ldexpf(1.f, e);
    }
}

}  // namespace atlas
