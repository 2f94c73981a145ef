// The decode step for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation): the same
// launches as atlas_decode_step, with the workspace taken from a fixed scratch area
// that the library holds in device memory. The call allocates nothing.
//
// The scratch area is a file-scope device array, so every GPU the library runs on
// holds its own copy at its own address until the process ends. Host code never
// passes the array's name to a kernel (on the host that name is only a stand-in,
// not a device address); it passes the address hipGetSymbolAddress returned for the
// device, looked up once per device and kept.
#include <mutex>

#include "decode.h"

namespace atlas {

static __device__ __align__(256) unsigned char scratch[ATLAS_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES];
static std::mutex g_scratch_mu;

// Device address of this device's scratch area (looked up on the first call for the
// device, with that device current).
static int scratch_address(hipStream_t st, void** out) {
    int dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATLAS_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(ATLAS_ERR_HIP, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return fail(ATLAS_ERR_HIP, "current device: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(ATLAS_ERR_HIP, "select device %d: %s", dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t er = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess || p == nullptr)
            return fail(ATLAS_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
        if (er != hipSuccess) return fail(ATLAS_ERR_HIP, "restore device %d: %s", cur, hipGetErrorString(er));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ATLAS_OK;
}

__global__ void copy_status_kernel(const int* ws_status, int32_t* out) { *out = *ws_status; }

}  // namespace atlas

using namespace atlas;

extern "C" int atlas_decode_step_noalloc(const atlas_model* m, const int32_t* d_token, const float* d_hidden_in,
                                         const int32_t* d_pos, float* d_hidden_out, float* d_logits,
                                         int32_t* d_argmax, int32_t* d_status_out, void* stream) {
    int rc = check_decode_args(m, d_token, d_hidden_in, d_pos, d_logits, d_argmax);
    if (rc) return rc;
    const size_t need = decode_ws_bytes(m);
    if (need > (size_t)ATLAS_NOALLOC_SCRATCH_BYTES)
        return fail(ATLAS_ERR_WORKSPACE_TOO_SMALL,
                    "this model's decode step needs %zu bytes of workspace; the fixed scratch area holds %zu "
                    "(use atlas_decode_step with a workspace of atlas_decode_workspace_bytes())",
                    need, (size_t)ATLAS_NOALLOC_SCRATCH_BYTES);
    hipStream_t st = (hipStream_t)stream;
    void* ws = nullptr;
    if ((rc = scratch_address(st, &ws))) return rc;
    if ((rc = atlas_decode_step(m, d_token, d_hidden_in, d_pos, d_hidden_out, d_logits, d_argmax, ws,
                                (size_t)ATLAS_NOALLOC_SCRATCH_BYTES, stream)))
        return rc;
    if (d_status_out) {
        prof_mark("noalloc_status", st);
        ATLAS_KLAUNCH(copy_status_kernel, dim3(1), dim3(1), 0, st, (const int*)ws, d_status_out);
        ATLAS_LAUNCH_CHECK("copy_status_kernel");
    }
    return ATLAS_OK;
}
