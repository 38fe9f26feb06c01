// Internal: optional per-kernel timing with HIP events attached to the
// dispatch itself (hipExtLaunchKernel start/stop events: the timestamps are
// taken when the kernel starts and ends, as a kernel trace does).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace coli {

// Take the next event pair for kernel `name`; false when profiling is off or
// the pool is used up.
bool prof_take(const char* name, hipEvent_t* start, hipEvent_t* stop);

// The next launch() on this thread is timed under `name`.
void prof_tag(const char* name);
const char* prof_pending();

struct ProfTag {
    explicit ProfTag(const char* name) { prof_tag(name); }
    ~ProfTag() { prof_tag(nullptr); }
};

// Every kernel of the library is launched through here.
template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream,
                   Args... args) {
    hipEvent_t a = nullptr, b = nullptr;
    const char* name = prof_pending();
    if (name && prof_take(name, &a, &b)) {
        prof_tag(nullptr);
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, a, b, 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
    }
}

}  // namespace coli
