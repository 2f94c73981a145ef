// Achievable read bandwidth: a plain streaming read of a device buffer. The decode
// kernels' rooflines are graded against the 8 TB/s peak; this gives the ceiling a
// kernel that does nothing but read reaches on the same device, for comparison.
#include "common.h"

namespace atlas {

constexpr int STREAM_THREADS = 256;
constexpr int STREAM_UNROLL = 4;
constexpr uint32_t STREAM_SENTINEL = 0x9E3779B9u;
typedef unsigned int stream_u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride read of n16 16-byte words, STREAM_UNROLL loads in flight per thread. The
// XOR of everything read is stored only if it equals a sentinel: the loads cannot be
// dropped, and (almost) nothing is written.
__global__ __launch_bounds__(STREAM_THREADS) void stream_read_kernel(const stream_u32x4* p, size_t n16,
                                                                    uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (STREAM_UNROLL - 1) * stride < n16; i += STREAM_UNROLL * stride) {
        stream_u32x4 v[STREAM_UNROLL];
#pragma unroll
        for (int u = 0; u < STREAM_UNROLL; u++) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < STREAM_UNROLL; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const stream_u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == STREAM_SENTINEL) sink[0] = acc;
}

}  // namespace atlas

using namespace atlas;

extern "C" int atlas_stream_read(const void* d_buf, size_t bytes, uint32_t* d_sink, int32_t blocks, void* stream) {
    ATLAS_CHECK_ARG(d_buf && d_sink, "null pointer");
    ATLAS_CHECK_ARG(bytes >= 16 && bytes % 16 == 0, "bytes=%zu must be a positive multiple of 16", bytes);
    ATLAS_CHECK_ARG(((uintptr_t)d_buf & 15) == 0, "buffer must be 16-byte aligned");
    ATLAS_CHECK_ARG(blocks >= 1 && blocks <= 65536, "blocks=%d outside [1, 65536]", blocks);
    hipStream_t st = (hipStream_t)stream;
    prof_mark("stream_read", st);
    ATLAS_KLAUNCH(stream_read_kernel, dim3(blocks), dim3(STREAM_THREADS), 0, st, (const stream_u32x4*)d_buf,
                  bytes / 16, d_sink);
    ATLAS_LAUNCH_CHECK("stream_read_kernel");
    return ATLAS_OK;
}
