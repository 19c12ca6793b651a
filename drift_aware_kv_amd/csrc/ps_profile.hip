// ps_profile.hip -- opt-in per-kernel timing with HIP events.
//
// When enabled (ps_profile_begin), every kernel the library enqueues is
// bracketed by a pair of events recorded on the stream the kernel runs on, so
// the elapsed time of each pair is that launch's duration on that stream.
// Events are created once in ps_profile_begin (never inside the compute
// calls); launches beyond the requested capacity are counted but not timed.
// Meant for single-threaded benchmarking; off by default.
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
};

bool g_on = false;
std::vector<Rec> g_recs;
size_t g_used = 0, g_dropped = 0;
hipEvent_t g_pending_start = nullptr;

}  // namespace

namespace ps_prof {

bool enabled() { return g_on; }

void before(const char* name, hipStream_t s)
{
    if (g_used >= g_recs.size()) {
        g_pending_start = nullptr;
        ++g_dropped;
        return;
    }
    Rec& r = g_recs[g_used];
    r.name = name;
    g_pending_start = r.a;
    (void)hipEventRecord(r.a, s);
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
    g_used = g_dropped = 0;
    g_recs.resize((size_t)max_launches);
    for (Rec& r : g_recs) {
        r.name = nullptr;
        if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) {
            g_recs.clear();
            return PS_ERR_DEVICE;
        }
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
    };
    std::map<std::string, Agg> agg;
    for (size_t i = 0; i < g_used; ++i) {
        if (hipEventSynchronize(g_recs[i].b) != hipSuccess) return PS_ERR_DEVICE;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_recs[i].a, g_recs[i].b) != hipSuccess) return PS_ERR_DEVICE;
        Agg& a = agg[g_recs[i].name];
        a.n += 1;
        a.tot += ms;
        a.mn = ms < a.mn ? ms : a.mn;
        a.mx = ms > a.mx ? ms : a.mx;
    }
    std::string out;
    char line[256];
    for (auto& kv : agg) {
        snprintf(line, sizeof line, "%s\t%d\t%.6f\t%.6f\t%.6f\n", kv.first.c_str(), kv.second.n,
                 kv.second.tot, kv.second.mn, kv.second.mx);
        out += line;
    }
    snprintf(line, sizeof line, "#dropped\t%zu\n", g_dropped);
    out += line;
    if (out.size() + 1 > len) return PS_ERR_RANGE;
    memcpy(buf, out.c_str(), out.size() + 1);
    return PS_OK;
}
