// Optional kernel timing: HIP events attached to the dispatch of tagged
// kernels (hipExtLaunchKernel start/stop events). Off unless
// coli_profile_enable() pre-allocates a pool; every timed launch takes the
// next (start, stop) pair.
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace coli {
namespace {

struct Record {
    const char* name;
    hipEvent_t start, stop;
};

struct ProfState {
    std::mutex mu;
    std::vector<hipEvent_t> pool;   // 2 per record
    std::vector<Record> recs;
    size_t capacity = 0;
};

ProfState& state() {
    static ProfState s;
    return s;
}

}  // namespace

static thread_local const char* t_pending = nullptr;

void prof_tag(const char* name) { t_pending = name; }
const char* prof_pending() { return t_pending; }

bool prof_take(const char* name, hipEvent_t* start, hipEvent_t* stop) {
    ProfState& P = state();
    std::lock_guard<std::mutex> g(P.mu);
    if (P.capacity == 0 || P.recs.size() >= P.capacity) return false;
    const size_t i = P.recs.size();
    Record r{name, P.pool[2 * i], P.pool[2 * i + 1]};
    P.recs.push_back(r);
    *start = r.start;
    *stop = r.stop;
    return true;
}

}  // namespace coli

using namespace coli;

extern "C" {

COLI_API coli_status coli_profile_enable(int32_t max_records) {
    ProfState& P = state();
    std::lock_guard<std::mutex> g(P.mu);
    for (hipEvent_t e : P.pool) (void)hipEventDestroy(e);
    P.pool.clear();
    P.recs.clear();
    P.capacity = 0;
    if (max_records <= 0) return COLI_OK;
    P.pool.resize(2 * (size_t)max_records);
    for (auto& e : P.pool) COLI_CHECK_HIP(hipEventCreate(&e));
    P.capacity = (size_t)max_records;
    return COLI_OK;
}

COLI_API coli_status coli_profile_clear(void) {
    ProfState& P = state();
    std::lock_guard<std::mutex> g(P.mu);
    P.recs.clear();
    return COLI_OK;
}

COLI_API coli_status coli_profile_summary(const char* name, int64_t* count, double* total_ms) {
    if (!name || !count || !total_ms) return fail(COLI_EINVAL, "profile_summary: NULL pointer");
    ProfState& P = state();
    std::lock_guard<std::mutex> g(P.mu);
    int64_t n = 0;
    double ms = 0.0;
    for (const Record& r : P.recs) {
        if (!r.name || std::string(r.name) != name) continue;
        COLI_CHECK_HIP(hipEventSynchronize(r.stop));
        float t = 0.f;
        COLI_CHECK_HIP(hipEventElapsedTime(&t, r.start, r.stop));
        ms += t;
        ++n;
    }
    *count = n;
    *total_ms = ms;
    return COLI_OK;
}

}  // extern "C"
