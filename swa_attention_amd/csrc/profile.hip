// Optional per-launch timing: while enabled, every kernel launch of the library is
// preceded by a hipEvent recorded on the launch stream, labelled with the launch's
// role; atlas_profile_stop() records a closing event, synchronises and attributes
// the time between consecutive events to the earlier label.
#include <cstring>
#include <string>
#include <vector>

#include "common.h"

namespace atlas {

struct Profiler {
    bool on = false;
    std::vector<hipEvent_t> ev;
    std::vector<const char*> label;
    size_t used = 0;
    hipStream_t st = nullptr;
    bool overflow = false;
};
static Profiler g_prof;

void prof_mark(const char* label, hipStream_t st) {
    Profiler& p = g_prof;
    if (!p.on) return;
    if (p.used >= p.ev.size()) {
        p.overflow = true;
        return;
    }
    if (p.used == 0) p.st = st;
    (void)hipEventRecord(p.ev[p.used], st);
    p.label[p.used] = label;
    p.used++;
}

}  // namespace atlas

using namespace atlas;

extern "C" int atlas_profile_start(int32_t capacity) {
    Profiler& p = g_prof;
    ATLAS_CHECK_ARG(capacity >= 2 && capacity <= (1 << 20), "capacity out of range");
    for (auto e : p.ev) (void)hipEventDestroy(e);
    p.ev.assign((size_t)capacity, nullptr);
    p.label.assign((size_t)capacity, nullptr);
    for (auto& e : p.ev) {
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return fail(ATLAS_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    }
    p.used = 0;
    p.overflow = false;
    p.on = true;
    return ATLAS_OK;
}

extern "C" int atlas_profile_stop(atlas_profile_entry* out, int32_t max_entries, int32_t* n_entries) {
    Profiler& p = g_prof;
    ATLAS_CHECK_ARG(out && n_entries && max_entries >= 0, "null pointer");
    ATLAS_CHECK_ARG(p.on, "profiling not started");
    p.on = false;
    ATLAS_CHECK_ARG(!p.overflow && p.used < p.ev.size(), "profile capacity exceeded");
    *n_entries = 0;
    if (p.used == 0) return ATLAS_OK;
    (void)hipEventRecord(p.ev[p.used], p.st);
    hipError_t err = hipEventSynchronize(p.ev[p.used]);
    if (err != hipSuccess) return fail(ATLAS_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(err));
    int n = 0;
    for (size_t i = 0; i < p.used; i++) {
        float ms = 0.f;
        (void)hipEventElapsedTime(&ms, p.ev[i], p.ev[i + 1]);
        int k = 0;
        while (k < n && std::strncmp(out[k].name, p.label[i], sizeof(out[k].name) - 1) != 0) k++;
        if (k == n) {
            if (n >= max_entries) continue;
            std::memset(&out[n], 0, sizeof(out[n]));
            std::strncpy(out[n].name, p.label[i], sizeof(out[n].name) - 1);
            n++;
        }
        out[k].count += 1;
        out[k].total_ms += ms;
    }
    *n_entries = n;
    return ATLAS_OK;
}
