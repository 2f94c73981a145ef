// Internal interface of the decode step.
#pragma once
#include "decode_kernels.h"

namespace atlas {

int validate_model(const atlas_model* m);
size_t decode_ws_bytes(const atlas_model* m);
// Host-side checks of atlas_decode_step's arguments other than the workspace.
int check_decode_args(const atlas_model* m, const int32_t* d_token, const float* d_hidden_in, const int32_t* d_pos,
                      const float* d_logits, const int32_t* d_argmax);
int run_decode_layers(const atlas_model* m, const XSource& first, const int32_t* d_pos, void* ws, hipStream_t st,
                      XSource* last_out);
int run_head(const atlas_model* m, const XSource& last, void* ws, float* hidden_out, float* logits_out,
             int32_t* argmax_out, hipStream_t st);

}  // namespace atlas
