// Internal interface of the decode attention kernels.
#pragma once
#include <algorithm>

#include "common.h"

namespace atlas {

constexpr int ATTN_PART = 130;   // m, l, acc[128] per (query head, split)

struct AttnArgs {
    const float* q;        // [Hq][128]
    const float* k_cache;  // [Hkv][T_max][128]
    const float* v_cache;
    float* part;           // [Hq][S][ATTN_PART]
    int Hkv;
    int64_t T_max;
    const int32_t* d_pos;
    int window;
    float scale;
    int S, Lmax;
};

struct AttnPlan {
    int S, Lmax;
    size_t part_bytes;
};

AttnPlan plan_attention(int Hq, int Hkv, int64_t T_max, int window);
int launch_attention(const AttnArgs& a, const AttnPlan& p, int G, XQ xq, float* out, hipStream_t st);

}  // namespace atlas
