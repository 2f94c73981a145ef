// Kernels of the matrix-core prefill (prefill_kernels.hip).
#pragma once
#include "decode_kernels.h"

namespace atlas {

// C = A W^T for a W4 matrix W [N][K] and activations A [M][K] given as two bf16 planes
// (A = hi + lo, see pf_split): mode 0 writes C f32 [M][ldc]; mode 1 takes a second
// matrix W1 of the same shape and writes z = silu(A W^T) * (A W1^T) as bf16 planes.
struct GemmArgs {
    const uint16_t* a_hi;
    const uint16_t* a_lo;
    int lda;
    W4View W0, W1;
    int M, N, K, group;
    float* C;
    int ldc;
    uint16_t* z_hi;
    uint16_t* z_lo;
    int ldz;
    // split-K (mode 0 only): ksplit ranges of kchunk columns (whole groups and k tiles);
    // split s writes its partial product to C + s * c_split. ksplit = 1: no split.
    int ksplit = 1, kchunk = 0;
    size_t c_split = 0;
    // Int8 digit planes of A for w4_gemm_i8_kernel (null: the bf16 planes are used):
    // A[m][k] ~ q_s[m][g] * (65536 q_hi + 256 q_mid + q_lo)[m][k] for group g of column
    // k, the bytes of every 8 columns stored in the order 0,2,4,6,1,3,5,7; q_sum[m][g]
    // is the sum of the group's 24-bit values. Row strides ldq (bytes), ldqs (groups).
    const int8_t* q_hi = nullptr;
    const int8_t* q_mid = nullptr;
    const int8_t* q_lo = nullptr;
    const float* q_s = nullptr;
    const float* q_sum = nullptr;
    int ldq = 0, ldqs = 0;
    // Mode 1 on the int8 ring kernel with groups of 128 (i8r_swiglu_digits_ok): when
    // zq_hi is set, z is written as the down projection's int8 digits in the layout above
    // (row strides zq_ld bytes and zq_lds groups of 128) instead of bf16 planes.
    int8_t* zq_hi = nullptr;
    int8_t* zq_mid = nullptr;
    int8_t* zq_lo = nullptr;
    float* zq_s = nullptr;
    float* zq_sum = nullptr;
    int zq_ld = 0, zq_lds = 0;
};

// KV of the prompt: keys j < start_pos come from the layer's cache ([Hkv][slots][128],
// key j in slot j or, on a ring, j mod slots), keys of the prompt from the prompt
// buffers ([Hkv][n][128]); both hold f32 or bf16 elements (kv_bf16).
struct PfAttnArgs {
    const float* qkv;          // [n][ld_qkv]: q rows already normalised and rotated
    int ld_qkv;
    const void* k_cache;
    const void* v_cache;
    int64_t slots;
    int ring, kv_bf16;
    const void* k_new;
    const void* v_new;
    int n, start_pos, Hq, Hkv, window;
    float scale;
    uint16_t* o_hi;            // [n][ldo] bf16 planes of the attention output (Hq*128 used)
    uint16_t* o_lo;
    int ldo;
};

struct PfRopeArgs {
    float* qkv;                // [n][ld]: S partial projections per row, pstride apart; q is
                               // written back normalised and rotated into the first
    int ld, n, start_pos, Hq, Hkv;
    const float *g_q, *g_k;
    float eps;
    double inv[64];
    double mscale;
    void* k_new;               // [Hkv][n][128] prompt keys / values, f32 or bf16 (kv_bf16)
    void* v_new;
    int kv_bf16;
    int S = 1, pstride = 0;    // K-split partials of the qkv GEMM (1..4)
};

// Prompt KV -> cache: positions j in [max(start_pos, start_pos + n - slots), start_pos + n)
// on a ring (earlier prompt positions would be overwritten by later ones), all of
// them otherwise.
struct PfCommitArgs {
    const void* k_new;
    const void* v_new;
    void* k_cache;
    void* v_cache;
    int64_t slots;
    int ring, kv_bf16, n, start_pos, Hkv;
};

int gemm_supported(int group);
int gemm_i8_supported(int group, int K);
int launch_pf_quant8(const uint16_t* hi, const uint16_t* lo, int lda, int M, int K, int group, int8_t* q_hi,
                     int8_t* q_mid, int8_t* q_lo, float* q_s, float* q_sum, hipStream_t st);
int launch_w4_gemm(const GemmArgs& a, int mode, hipStream_t st, const char* label);
// Whether a mode-1 launch of a (with its int8 digits attached) runs on the ring kernel with
// groups of 128 and can write z as int8 digits (zq_*) for a down projection with groups of 128.
bool i8r_swiglu_digits_ok(const GemmArgs& a, int down_group);
int launch_pf_embed(const int32_t* tokens, int n, const uint16_t* emb, int vocab, int d, float* X, uint16_t* p_hi,
                    uint16_t* p_lo, int ldp, int* status, hipStream_t st);
int launch_pf_rope(const PfRopeArgs& a, hipStream_t st);
int launch_pf_commit(const PfCommitArgs& a, hipStream_t st);
int launch_pf_attn(const PfAttnArgs& a, hipStream_t st);
int launch_pf_split(const float* X, int M, int K, int ldx, uint16_t* p_hi, uint16_t* p_lo, int ldp, hipStream_t st);
// Destination of int8 digits made in place of bf16 planes (layout as in GemmArgs, row
// strides K bytes and K / group groups).
struct Q8Out {
    int8_t *hi, *mid, *lo;
    float *s, *sum;
    int group;
};
// Whether the residual kernel can write the next GEMM's int8 digits for this group and d.
bool residual_digits_ok(int group, int d);
int launch_pf_residual(float* X, const float* A, int lda, int S, const float* g, int n, int d, float eps,
                       uint16_t* p_hi, uint16_t* p_lo, int ldp, hipStream_t st, const Q8Out* q = nullptr);

}  // namespace atlas
