// Internal interface of the GEMV entry point helpers.
#pragma once
#include "gemv_core.h"

namespace atlas {

int validate_w4(const atlas_w4* W);
int launch_xq_encode(const float* x, int K, XQ out, hipStream_t st);
int launch_sum_partials(const float* part, int S, int N, float* y, hipStream_t st);
size_t gemv_workspace_bytes(int N, int K);

}  // namespace atlas
