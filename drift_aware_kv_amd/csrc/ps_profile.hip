// ps_profile.hip -- opt-in per-kernel timing with HIP events.
//
// When enabled (ps_profile_begin), every kernel the library enqueues is
// bracketed by a pair of events recorded on the stream the kernel runs on, so
// the elapsed time of each pair is that launch's duration on that stream.
// Events are created once in ps_profile_begin (never inside the compute
// calls); launches beyond the requested capacity are counted but not timed.
// Kernels whose work depends on the data (a Lloyd pass skips the windows at
// a fixed point) also count the units of work they processed into a device
// counter per launch, so that a launch's duration can be set against the work
// it did.  Meant for single-threaded benchmarking; off by default.
#include "ps_common.h"
#include "ps_profile.h"

#include <stdio.h>
#include <string.h>

#include <map>
#include <string>
#include <vector>

namespace {

struct Rec {
    const char* name;
    hipEvent_t a, b;
    unsigned units;   // units of work of the launch, 0 if not counted
};

bool g_on = false;
std::vector<Rec> g_recs;
size_t g_used = 0, g_dropped = 0;
hipEvent_t g_pending_start = nullptr;
int* g_work = nullptr;          // device counters, one per record

}  // namespace

namespace ps_prof {

bool enabled() { return g_on; }

void before(const char* name, hipStream_t s, unsigned units)
{
    if (g_used >= g_recs.size()) {
        g_pending_start = nullptr;
        ++g_dropped;
        return;
    }
    Rec& r = g_recs[g_used];
    r.name = name;
    r.units = units;
    g_pending_start = r.a;
    (void)hipEventRecord(r.a, s);
}

int* work_slot()
{
    return (g_pending_start && g_work) ? g_work + g_used : nullptr;
}

void after(hipStream_t s)
{
    if (!g_pending_start) return;
    (void)hipEventRecord(g_recs[g_used].b, s);
    ++g_used;
    g_pending_start = nullptr;
}

}  // namespace ps_prof

extern "C" ps_status ps_profile_begin(int32_t max_launches)
{
    if (max_launches < 1) return PS_ERR_RANGE;
    for (Rec& r : g_recs) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    g_recs.clear();
    if (g_work) (void)hipFree(g_work);
    g_work = nullptr;
    g_used = g_dropped = 0;
    g_recs.resize((size_t)max_launches);
    for (Rec& r : g_recs) {
        r.name = nullptr;
        r.units = 0;
        if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) {
            g_recs.clear();
            return PS_ERR_DEVICE;
        }
    }
    if (hipMalloc((void**)&g_work, sizeof(int) * (size_t)max_launches) != hipSuccess ||
        hipMemset(g_work, 0, sizeof(int) * (size_t)max_launches) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        (void)hipGetLastError();
        g_recs.clear();
        return PS_ERR_DEVICE;
    }
    g_on = true;
    return PS_OK;
}

extern "C" ps_status ps_profile_end(void)
{
    g_on = false;
    return PS_OK;
}

extern "C" ps_status ps_profile_summary(char* buf, size_t len)
{
    if (!buf || len == 0) return PS_ERR_NULL;
    struct Agg {
        int n = 0;
        double tot = 0, mn = 1e30, mx = 0;
        unsigned long long done = 0, units = 0;
    };
    std::vector<int> work(g_used, 0);
    for (size_t i = 0; i < g_used; ++i)
        if (hipEventSynchronize(g_recs[i].b) != hipSuccess) return PS_ERR_DEVICE;
    if (g_used && g_work &&
        hipMemcpy(work.data(), g_work, sizeof(int) * g_used, hipMemcpyDeviceToHost) != hipSuccess)
        return PS_ERR_DEVICE;
    std::map<std::string, Agg> agg;
    for (size_t i = 0; i < g_used; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_recs[i].a, g_recs[i].b) != hipSuccess) return PS_ERR_DEVICE;
        Agg& a = agg[g_recs[i].name];
        a.n += 1;
        a.tot += ms;
        a.mn = ms < a.mn ? ms : a.mn;
        a.mx = ms > a.mx ? ms : a.mx;
        if (g_recs[i].units) {
            a.units += g_recs[i].units;
            a.done += (unsigned long long)work[i];
        }
    }
    std::string out;
    char line[512];
    for (auto& kv : agg) {
        snprintf(line, sizeof line, "%s\t%d\t%.6f\t%.6f\t%.6f\t%llu\t%llu\n", kv.first.c_str(), kv.second.n,
                 kv.second.tot, kv.second.mn, kv.second.mx, kv.second.done, kv.second.units);
        out += line;
    }
    snprintf(line, sizeof line, "#dropped\t%zu\n", g_dropped);
    out += line;
    if (out.size() + 1 > len) return PS_ERR_RANGE;
    memcpy(buf, out.c_str(), out.size() + 1);
    return PS_OK;
}
