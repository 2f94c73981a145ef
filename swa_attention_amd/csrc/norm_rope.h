// Internal interface of the norm / rotary kernels.
#pragma once
#include "common.h"

namespace atlas {

struct RopeTable {
    double inv[128];   // D/2 inverse frequencies (D <= 256)
    double mscale;     // magnitude factor applied to cos and sin
};

struct QkArgs {
    const float* q;     // [S] partials of q (stride pstride)
    const float* k;
    const float* v;     // may be null (no append)
    int S;
    size_t pstride;
    const float *gq, *gk;
    float* q_out;
    float* k_out;       // may be null
    float *k_cache, *v_cache;
    int64_t T_max;
    int Hq, Hkv, D;
    float eps;
    const int32_t* d_pos;
    int* status;        // device status word, may be null
    RopeTable rope;
};

void rope_table(const atlas_rope* r, int D, RopeTable* t);
int launch_rmsnorm_residual(const float* xpart, int S, const float* g, const float* resid, float* out, int n,
                            float eps, XQ xq, hipStream_t st);
int launch_qk_norm_rope(const QkArgs& a, hipStream_t st);

}  // namespace atlas
