// ps_profile.h -- internal hooks of the opt-in kernel timer (see ps_profile.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace ps_prof {
bool enabled();
// `units` > 0: the launch is made of that many units of work (tiles, rows,
// clusters) and its kernel counts the units it actually processed into
// work_slot(); 0: every launch does its full work
void before(const char* name, hipStream_t s, unsigned units = 0);
void after(hipStream_t s);
int* work_slot();   // device counter of the launch being recorded, or nullptr
}  // namespace ps_prof

// Enqueue a kernel; when the timer is on, bracket it with events on `stream`.
#define PS_LAUNCH(name, kernel, grid, block, shm, stream, ...)                 \
    do {                                                                        \
        const bool ps_prof_on_ = ps_prof::enabled();                            \
        if (ps_prof_on_) ps_prof::before(name, stream);                         \
        hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__);      \
        if (ps_prof_on_) ps_prof::after(stream);                                \
    } while (0)

// The same for a kernel whose work depends on the data (it skips windows or
// clusters that cannot change): its last argument is an int* that it
// increments by the units it processed, NULL when the timer is off.
#define PS_LAUNCH_COUNTED(name, units, kernel, grid, block, shm, stream, ...)    \
    do {                                                                        \
        const bool ps_prof_on_ = ps_prof::enabled();                            \
        if (ps_prof_on_) ps_prof::before(name, stream, (unsigned)(units));      \
        int* ps_work_ = ps_prof_on_ ? ps_prof::work_slot() : nullptr;           \
        hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__, ps_work_); \
        if (ps_prof_on_) ps_prof::after(stream);                                \
    } while (0)
