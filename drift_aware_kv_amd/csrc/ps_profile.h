// ps_profile.h -- internal hooks of the opt-in kernel timer (see ps_profile.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace ps_prof {
bool enabled();
void before(const char* name, hipStream_t s);
void after(hipStream_t s);
}  // namespace ps_prof

// Enqueue a kernel; when the timer is on, bracket it with events on `stream`.
#define PS_LAUNCH(name, kernel, grid, block, shm, stream, ...)                 \
    do {                                                                        \
        const bool ps_prof_on_ = ps_prof::enabled();                            \
        if (ps_prof_on_) ps_prof::before(name, stream);                         \
        hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__);      \
        if (ps_prof_on_) ps_prof::after(stream);                                \
    } while (0)
