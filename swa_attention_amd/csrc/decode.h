// Internal interface of the decode step.
#pragma once
#include "common.h"

namespace atlas {

constexpr int LM_BLOCKS = 1024;   // lm_head workgroups (argmax partials)

int validate_model(const atlas_model* m);
size_t decode_ws_bytes(const atlas_model* m);

}  // namespace atlas
