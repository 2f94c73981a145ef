// Fused kernels of the decode step (internal interface).
#pragma once
#include "bgemv.h"
#include "gemv_core.h"

namespace atlas {

constexpr int GEMV_THREADS = 512;   // 8 waves per GEMV block
constexpr int ATTN_THREADS = 256;   // 4 waves = 16 key streams per attention block
constexpr int ATTN_PART_F = 130;    // m, l, acc[128] per (query head, split)
constexpr int ATTN_SSQ_MAX_BLOCKS = 512;   // qkv blocks whose sums of squares attention reads
// Share of a GEMV block's row tiles given to its older waves (the first of the two
// waves of each SIMD). Measured on the gate/up projection (2 x 27,648 x 5,120): an even
// split leaves the younger waves streaming alone for ~5.5 us at the end; 0.63 is the
// shortest.
constexpr float GEMV_OLD_FRAC = 0.63f;

// How a QKV block obtains the layer input x.
enum XMode { X_FROM_EMBED = 0, X_FROM_HIDDEN = 1, X_FROM_RESIDUAL = 2 };

struct XSource {
    int mode;
    const int32_t* d_token;     // X_FROM_EMBED
    const uint16_t* emb;        //   bf16 [vocab][d]
    int vocab;
    const float* hidden;        // X_FROM_HIDDEN: f32 [d]
    const float* m_part;        // X_FROM_RESIDUAL: x = h + g * m / rms(m), m = sum of S partials
    int S;
    const float* h;
    const float* g;
    float eps;
};

struct QkvArgs {
    W4View W;
    XSource src;
    int d, group, CW, tiles_per_block;
    float* qkv;          // [N] out
    float* x_out;        // [d] out (block 0): the layer input, kept for the residual
    int* status;         // reset to OK by block 0 (or set on a bad token id)
    float* ssq_part;     // [blocks][2] out (may be null): per-block sums of squares of the
    int nq, nk;          //   q rows [0, nq) and the k rows [nq, nq + nk)
};

struct AttnFusedArgs {
    const float* qkv;          // raw projection: q [Hq*D], k [Hkv*D], v [Hkv*D]
    const float *g_q, *g_k;
    void* k_cache;             // [Hkv][slots][D], f32 or bf16 (kv_bf16)
    void* v_cache;
    int64_t T_max;             // positions accepted: [0, T_max)
    int64_t slots;             // positions stored per KV head
    int ring;                  // 1: key j in slot j mod slots; 0: slot j
    int kv_bf16;               // 1: bf16 elements, rounded to nearest even when stored
    const int32_t* d_pos;
    int Hq, Hkv, window, S;
    float scale, eps;
    double inv[64];            // rotary inverse frequencies (D = 128)
    double mscale;
    float* part;               // [Hq][S][130]
    int* status;
    int fused;                 // 1: q/k/v from qkv with norm + rotary + KV append; 0: q final, cache ready
    const float* q_final;      // fused == 0
    const float* ssq_part;     // fused: [n_ssq][2] sums of squares of q and k (qkv kernel)
    int n_ssq;
    // batched decode (fused == 0): sequence z = blockIdx.z reads q_final + z * q_stride,
    // position d_pos[z], caches + z * seq_stride elements, and writes part + z * part_stride
    int batch;                 // 0 or 1: one sequence
    int64_t q_stride, seq_stride, part_stride;
};

struct MergeArgs {
    const float* part;
    int S, Hq;
    float* o;     // may be null
    XQ xq;        // planes may be null
    BQ bq;        // p may be null: o of sequence blockIdx.y as int8 planes (one head = one 128-column block)
    // batched: sequence y = blockIdx.y reads part + y * part_stride, writes o + y * o_stride
    int batch;    // 0 or 1: one sequence
    int64_t part_stride, o_stride;
};

struct GemvPlanesArgs {    // encoded input already in global memory
    W4View W;
    XQ xq;
    int group, CW, tiles_per_block;
    float* y;              // [S][N] (blockIdx.y = range)
};

struct GateUpArgs {
    W4View Wg, Wu;
    const float *a, *x, *g;     // h = x + g * a / rms(a)
    float eps;
    int d, group, CW, tiles_per_block;
    float old_frac;             // share of a block's tiles streamed by its older waves
    float* h_out;               // block 0
    float* z;                   // [dff]
};

struct DownArgs {
    W4View W;
    const float* z;             // f32 [K]
    int group, CW, tiles_per_block;
    float old_frac;             // share of a block's tiles streamed by its older waves
    float* m_part;              // [S][N]
};

struct HeadArgs {
    const uint16_t* lm;         // bf16 [V][d]
    int V, d, rows_per_block;
    XSource src;                // X_FROM_RESIDUAL: last layer's output
    const float* g_final;
    float eps;
    float* hidden_out;          // may be null (block 0)
    float* logits;
    float* bmax;
    int* bidx;
};

struct GemvShape {
    int CPL, RB, CW, S, tiles_per_block, blocks;
};
// Reduction ranges, tile shape and grid of a W4 GEMV. max_cpl bounds the register
// footprint (the gate/up kernel holds two matrices' tiles and uses 3).
GemvShape gemv_shape(int N, int K, bool split_k, int target_blocks, int max_cpl = 5);

int launch_qkv(const QkvArgs& a, const GemvShape& s, hipStream_t st);
int launch_attn_fused(const AttnFusedArgs& a, int G, hipStream_t st);
int launch_merge(const MergeArgs& a, hipStream_t st);
int launch_gemv_planes(const GemvPlanesArgs& a, const GemvShape& s, hipStream_t st, const char* label);
int launch_gate_up(const GateUpArgs& a, const GemvShape& s, hipStream_t st);
int launch_down(const DownArgs& a, const GemvShape& s, hipStream_t st);
int launch_head(const HeadArgs& a, int blocks, hipStream_t st);
int launch_final_hidden(const XSource& src, int d, float* out, hipStream_t st);
int launch_argmax_final(const float* bmax, const int* bidx, int nb, int32_t* out, hipStream_t st);

int attn_splits(int64_t maxkeys, int Hkv);

}  // namespace atlas
