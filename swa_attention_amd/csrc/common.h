// Shared device and host helpers of libatlas (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>

#include "../../include/atlas.h"

namespace atlas {

// ---- host-side error reporting ---------------------------------------------------

void set_error(const char* fmt, ...);
int fail(int status, const char* fmt, ...);
void prof_mark(const char* label, hipStream_t st);   // no-op unless profiling
// Start/stop events for the launch announced by the last prof_mark (null when not
// profiling). The dispatch itself stamps them, so they bracket the kernel's execution.
void prof_take(hipEvent_t* start, hipEvent_t* stop);
#define ATLAS_KLAUNCH(kern, grid, block, shmem, st, ...)                                   \
    do {                                                                                   \
        hipEvent_t e0_, e1_;                                                               \
        prof_take(&e0_, &e1_);                                                             \
        hipExtLaunchKernelGGL(kern, grid, block, shmem, st, e0_, e1_, 0u, __VA_ARGS__);    \
    } while (0)

#define ATLAS_CHECK_ARG(cond, ...)                                              \
    do {                                                                        \
        if (!(cond)) return ::atlas::fail(ATLAS_ERR_INVALID_ARG, __VA_ARGS__);  \
    } while (0)
#define ATLAS_CHECK_SHAPE(cond, ...)                                                 \
    do {                                                                             \
        if (!(cond)) return ::atlas::fail(ATLAS_ERR_UNSUPPORTED_SHAPE, __VA_ARGS__); \
    } while (0)
#define ATLAS_LAUNCH_CHECK(what)                                                            \
    do {                                                                                    \
        hipError_t e_ = hipGetLastError();                                                  \
        if (e_ != hipSuccess)                                                               \
            return ::atlas::fail(ATLAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e_));     \
    } while (0)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- wave-level reductions (64 lanes) ------------------------------------------------
// DPP steps inside each row of 16 lanes (quad xor 1, quad xor 2, half-row mirror,
// row mirror: every lane ends with its row's total), then two lane-xor exchanges
// across rows.

// Every control used here reads a valid lane for every lane; bound_ctrl with a zero old
// value lets the compiler fold the move into the consuming add or max (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    return v;
}

// Butterflies across rows with gfx950's lane-swap instructions. With both operands
// equal to v, v_permlane16_swap returns (v of the even row of the lane's row pair,
// v of the odd row) at the lane's position, and v_permlane32_swap the same for the
// two halves of the wave; combining the two results gives every lane the reduction
// over itself and lane ^ 16 (lane ^ 32), in the same order for both lanes.
__device__ __forceinline__ float xor16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum(float v) { return xor32_sum(xor16_sum(row16_sum(v))); }

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return xor32_max(xor16_max(v));
}

__device__ __forceinline__ float quad_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    return v;
}

__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    return v;
}

__device__ __forceinline__ int quad_sum_i(int v) {
    v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
    v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
    return v;
}

// Block-wide sum; every thread gets the result. `red` holds >= 16 floats of LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; i++) t += red[i];
    return t;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// bfloat16 bits of x, rounded to nearest with ties to even (a carry from the
// significand moves into the exponent, so overflow gives infinity); NaN stays a quiet
// NaN with its sign.
// Round to nearest even for finite x (the activation splits of the prefill).
__device__ __forceinline__ uint32_t f32_to_bf16_rne_finite(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The same for any x, branch-free (values stored in a bf16 KV cache).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet_nan = (u >> 16) | 0x40u;
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? quiet_nan : rounded;
}

__device__ __forceinline__ float scale_to_f32(uint16_t b, int scale_dtype) {
    return scale_dtype ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// ---- activation encoding for the integer-dot W4 GEMV ----------------------------------
//
// A GEMV input x[K] is encoded once per vector, per chunk of 32 consecutive elements
// (one 16-byte word quad of packed codes):
//   e_c = exponent with max|x| < 2^e_c over the chunk, q_c = 2^(e_c - 22),
//   i_k = rint(x_k / q_c), |i_k| <= 2^22 (a 24-bit block floating-point mantissa),
//   i_k = sum_{p<6} 16^p d_{k,p} with balanced digits d in [-8, 7],
//   plane word (c, w, p) = the eight digits d_{k,p} of k = 32c + 8w .. 32c + 8w + 7
//   packed as signed nibbles in the same order as the weight codes.
// With weight codes c_k (4-bit, in the packing order of the weights) and s = 8 the
// nibble bias removed by xor 0x88888888:
//   sum_k (c_k - z) x_k = q_c * ( sum_p 16^p dot8(c - 8, d_p) - (z - 8) * sum_k i_k )
// for a chunk inside one quantisation group. The digit dot products are exact in
// int32; the result differs from the f32 value of x only by the rounding of x to
// 2^-22 of its chunk maximum.

constexpr int XQ_PLANES = 6;
constexpr int XQ_CHUNK = 32;              // elements per chunk
constexpr int XQ_WORDS_PER_CHUNK = 24;    // 4 words x 6 planes

struct XQ {                 // views into an encoded vector
    uint32_t* planes;       // [C][4][6]
    float* qs;              // [C]
    int* isum;              // [C]
};

__host__ __device__ inline size_t xq_bytes(int K) {
    size_t C = (size_t)K / XQ_CHUNK;
    return C * (XQ_WORDS_PER_CHUNK * 4 + 8);
}
__host__ __device__ inline XQ xq_view(void* base, int K) {
    size_t C = (size_t)K / XQ_CHUNK;
    XQ v;
    v.planes = (uint32_t*)base;
    v.qs = (float*)((char*)base + C * XQ_WORDS_PER_CHUNK * 4);
    v.isum = (int*)((char*)base + C * (XQ_WORDS_PER_CHUNK * 4 + 4));
    return v;
}

// Byte k of the result r_k is byte k' of X[0..3] for k' = 0, 1, 2: r_k = [X0.k', X1.k',
// X2.k', X3.k'] (v_perm_b32 selects bytes of the 8-byte pair {hi, lo}).
__device__ __forceinline__ void xq_gather_bytes(const uint32_t (&X)[4], uint32_t& r0, uint32_t& r1, uint32_t& r2) {
    const uint32_t a = __builtin_amdgcn_perm(X[1], X[0], 0x05010400u);   // X0.0 X1.0 X0.1 X1.1
    const uint32_t b = __builtin_amdgcn_perm(X[3], X[2], 0x05010400u);   // X2.0 X3.0 X2.1 X3.1
    const uint32_t c = __builtin_amdgcn_perm(X[1], X[0], 0x07030602u);   // X0.2 X1.2 X0.3 X1.3
    const uint32_t d = __builtin_amdgcn_perm(X[3], X[2], 0x07030602u);   // X2.2 X3.2 X2.3 X3.3
    r0 = __builtin_amdgcn_perm(b, a, 0x05040100u);
    r1 = __builtin_amdgcn_perm(b, a, 0x07060302u);
    r2 = __builtin_amdgcn_perm(d, c, 0x05040100u);
}

// Encode word `w` (8 elements x8[0..7]) of chunk `c`; the 4 threads of a chunk must
// be lanes 4j..4j+3 of one wave (quad) and call this together.
__device__ __forceinline__ void xq_encode_word(const float x8[8], XQ out, int c, int w) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(x8[i]));
    m = quad_max(m);
    int e = (m > 0.f) ? __builtin_amdgcn_frexp_expf(m) : 0;   // m < 2^e
    // v = rint(x 2^(22-e)), |v| < 2^22: adding 1.5 * 2^23 rounds to the nearest even
    // integer and leaves 0x4B400000 + v in the bits. b = v + 0x888888 lies in [0, 16^6):
    // its nibbles n_p are the balanced digits of v plus 8 (v = sum_p (n_p - 8) 16^p), and
    // the 4-bit pattern of the digit n_p - 8 is n_p ^ 8 (applied to whole plane words).
    constexpr float ROUND = 12582912.0f;                      // 1.5 * 2^23
    constexpr uint32_t ROUND_BITS = 0x4B400000u;
    const int sh = 22 - e;
    uint32_t b[8], su = 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t u = __float_as_uint(__builtin_amdgcn_ldexpf(x8[i], sh) + ROUND);
        su += u;
        b[i] = u + (0x888888u - ROUND_BITS);
    }
    int s = quad_sum_i((int)(su - 8u * ROUND_BITS));
    // nibble transpose: plane p holds nibble p of the 8 values, value i in nibble i.
    // Pair the values (2k, 2k+1) into bytes (E: even nibbles, O: odd nibbles of b), then
    // gather byte k of the four pairs with byte permutes.
    uint32_t E[4], O[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        E[k] = (b[2 * k] & 0x0F0F0F0Fu) | ((b[2 * k + 1] << 4) & 0xF0F0F0F0u);
        O[k] = ((b[2 * k] >> 4) & 0x0F0F0F0Fu) | (b[2 * k + 1] & 0xF0F0F0F0u);
    }
    uint32_t pl[XQ_PLANES];
    xq_gather_bytes(E, pl[0], pl[2], pl[4]);
    xq_gather_bytes(O, pl[1], pl[3], pl[5]);
    uint32_t* dst = out.planes + (size_t)c * XQ_WORDS_PER_CHUNK + w * XQ_PLANES;
#pragma unroll
    for (int p = 0; p < XQ_PLANES; p++) dst[p] = pl[p] ^ 0x88888888u;
    if (w == 0) {
        out.qs[c] = __builtin_amdgcn_ldexpf(1.0f, e - 22);
        out.isum[c] = s;
    }
}

}  // namespace atlas
