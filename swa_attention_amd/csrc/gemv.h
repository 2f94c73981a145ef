// Internal interface of the W4 GEMV kernels.
#pragma once
#include "common.h"

namespace atlas {

struct GemvArgs {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint32_t* zeros;
    int N, K, group, scale_dtype;
    XQ xq;          // encoded input
    float* y;       // [S][N] partial sums (S = 1: the result)
    int CW;         // chunks per reduction range
    int tiles_per_block;
};

struct GemvPlan {
    int CW, S, RB, CPL;
    int tiles_per_block, blocks_x;
    size_t lds_bytes;
};

int validate_w4(const atlas_w4* W);
GemvPlan plan_gemv(int N, int K);
GemvArgs gemv_args(const atlas_w4* W, XQ xq, float* y);
int launch_gemv(const GemvArgs& a, const GemvPlan& p, hipStream_t st);
int launch_xq_encode(const float* x, int K, XQ out, hipStream_t st);
int launch_sum_partials(const float* part, int S, int N, float* y, hipStream_t st);
size_t gemv_workspace_bytes(int N, int K);

}  // namespace atlas
