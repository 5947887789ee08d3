// Optional per-kernel GPU timing: when enabled, each launch is bracketed by two HIP events
// on its own stream, so the measured time is the kernel's time on that stream.
#include <hip/hip_runtime.h>

#include <cstring>
#include <string>
#include <vector>

#include "plan_impl.hpp"

namespace {

constexpr int kMaxRecords = 8192;

struct Record {
    const char* name;
    int slot;
};

bool g_on = false;
std::string g_only;                 // when non-empty, only this kernel is timed
std::vector<hipEvent_t> g_events;   // 2 per record slot, created on enable
std::vector<Record> g_records;
int g_open = -1;

}  // namespace

namespace medusa {

void prof_begin(const char* name, hipStream_t stream) {
    g_open = -1;
    if (!g_on) return;
    if (!g_only.empty() && g_only != name) return;
    const int slot = (int)g_records.size();
    if (slot >= kMaxRecords || 2 * slot + 1 >= (int)g_events.size()) {
        g_open = -1;
        return;
    }
    if (hipEventRecord(g_events[2 * slot], stream) != hipSuccess) {
        g_open = -1;
        return;
    }
    g_records.push_back({name, slot});
    g_open = slot;
}

void prof_end(hipStream_t stream) {
    if (!g_on || g_open < 0) return;
    hipEventRecord(g_events[2 * g_open + 1], stream);
    g_open = -1;
}

}  // namespace medusa

extern "C" {

medusa_status medusa_profile_enable(int on) {
    if (on) {
        medusa_status st = medusa_internal_device_check();
        if (st != MEDUSA_OK) return st;
        if (g_events.empty()) {
            const int n = 2 * 8192;
            g_events.resize(n);
            for (int i = 0; i < n; ++i) {
                hipError_t e = hipEventCreate(&g_events[i]);
                if (e != hipSuccess) {
                    g_events.resize(i);
                    return medusa_internal_hip_error(e);
                }
            }
        }
    }
    g_on = on != 0;
    return MEDUSA_OK;
}

medusa_status medusa_profile_only(const char* kernel) {
    g_only = kernel ? kernel : "";
    return MEDUSA_OK;
}

medusa_status medusa_profile_reset(void) {
    g_records.clear();
    g_open = -1;
    return MEDUSA_OK;
}

medusa_status medusa_profile_query(const char* kernel, double* total_ms, int* launches) {
    if (!kernel || !total_ms || !launches) return MEDUSA_ERR_NULL;
    double sum = 0.0;
    int n = 0;
    for (const Record& r : g_records) {
        if (std::strcmp(r.name, kernel) != 0) continue;
        hipError_t e = hipEventSynchronize(g_events[2 * r.slot + 1]);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_events[2 * r.slot], g_events[2 * r.slot + 1]);
        if (e != hipSuccess) return medusa_internal_hip_error(e);
        sum += ms;
        ++n;
    }
    *total_ms = sum;
    *launches = n;
    return MEDUSA_OK;
}

}  // extern "C"
