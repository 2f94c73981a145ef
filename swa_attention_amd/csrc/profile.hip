// Optional per-launch timing. While enabled, every kernel launch of the library gets
// a pair of hipEvents that the dispatch itself stamps (hipExtLaunchKernel start/stop
// events), labelled with the launch's role; atlas_profile_stop() synchronises and
// sums, per label, the time between each launch's start and stop stamps.
#include <cstring>
#include <string>
#include <vector>

#include "common.h"

namespace atlas {

struct Profiler {
    bool on = false;
    std::vector<hipEvent_t> ev0, ev1;
    std::vector<const char*> label;
    size_t used = 0;
    long pending = -1;
    hipStream_t st = nullptr;
    bool overflow = false;
};
static Profiler g_prof;

void prof_mark(const char* label, hipStream_t st) {
    Profiler& p = g_prof;
    p.pending = -1;
    if (!p.on) return;
    if (p.used >= p.ev0.size()) {
        p.overflow = true;
        return;
    }
    p.st = st;
    p.label[p.used] = label;
    p.pending = (long)p.used++;
}

void prof_take(hipEvent_t* start, hipEvent_t* stop) {
    Profiler& p = g_prof;
    *start = *stop = nullptr;
    if (p.on && p.pending >= 0) {
        *start = p.ev0[(size_t)p.pending];
        *stop = p.ev1[(size_t)p.pending];
    }
    p.pending = -1;
}

static void destroy_events(Profiler& p) {
    for (auto e : p.ev0) (void)hipEventDestroy(e);
    for (auto e : p.ev1) (void)hipEventDestroy(e);
    p.ev0.clear();
    p.ev1.clear();
}

}  // namespace atlas

using namespace atlas;

extern "C" int atlas_profile_start(int32_t capacity) {
    Profiler& p = g_prof;
    ATLAS_CHECK_ARG(capacity >= 1 && capacity <= (1 << 20), "capacity out of range");
    destroy_events(p);
    p.ev0.assign((size_t)capacity, nullptr);
    p.ev1.assign((size_t)capacity, nullptr);
    p.label.assign((size_t)capacity, nullptr);
    for (size_t i = 0; i < p.ev0.size(); i++) {
        hipError_t err = hipEventCreate(&p.ev0[i]);
        if (err == hipSuccess) err = hipEventCreate(&p.ev1[i]);
        if (err != hipSuccess) return fail(ATLAS_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    }
    p.used = 0;
    p.pending = -1;
    p.overflow = false;
    p.on = true;
    return ATLAS_OK;
}

extern "C" int atlas_profile_stop(atlas_profile_entry* out, int32_t max_entries, int32_t* n_entries) {
    Profiler& p = g_prof;
    ATLAS_CHECK_ARG(out && n_entries && max_entries >= 0, "null pointer");
    ATLAS_CHECK_ARG(p.on, "profiling not started");
    p.on = false;
    ATLAS_CHECK_ARG(!p.overflow, "profile capacity exceeded");
    *n_entries = 0;
    if (p.used == 0) return ATLAS_OK;
    hipError_t err = hipEventSynchronize(p.ev1[p.used - 1]);
    if (err == hipSuccess) err = hipStreamSynchronize(p.st);
    if (err != hipSuccess) return fail(ATLAS_ERR_HIP, "profile sync: %s", hipGetErrorString(err));
    int n = 0;
    for (size_t i = 0; i < p.used; i++) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, p.ev0[i], p.ev1[i]) != hipSuccess) continue;
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
