// Internal: optional per-kernel event timing (see profile.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace coli {
int prof_start(hipStream_t stream);                          // -1 when profiling is off
void prof_stop(int slot, const char* name, hipStream_t stream);

struct ProfScope {
    int slot;
    const char* name;
    hipStream_t stream;
    ProfScope(const char* n, hipStream_t s) : slot(prof_start(s)), name(n), stream(s) {}
    ~ProfScope() { prof_stop(slot, name, stream); }
};
}  // namespace coli
