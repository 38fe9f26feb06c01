// Expert cache (placeholder entry points until the cache lands).
#include "layer.h"

extern "C" {
coli_status coli_expert_cache_create(const coli_cache_cfg*, struct coli_expert_cache**) {
    return coli::fail(COLI_EUNSUPPORTED, "expert cache not available yet");
}
coli_status coli_expert_cache_destroy(struct coli_expert_cache*) { return COLI_OK; }
coli_status coli_expert_cache_ensure(struct coli_expert_cache*, int32_t, const int32_t*, int32_t, int32_t*) {
    return coli::fail(COLI_EUNSUPPORTED, "expert cache not available yet");
}
coli_status coli_expert_cache_wait(struct coli_expert_cache*, int32_t, void*) {
    return coli::fail(COLI_EUNSUPPORTED, "expert cache not available yet");
}
coli_status coli_expert_cache_release(struct coli_expert_cache*, int32_t, void*) {
    return coli::fail(COLI_EUNSUPPORTED, "expert cache not available yet");
}
coli_status coli_expert_cache_table(struct coli_expert_cache*, int32_t, const void* const**) {
    return coli::fail(COLI_EUNSUPPORTED, "expert cache not available yet");
}
coli_status coli_expert_cache_stats(struct coli_expert_cache*, coli_cache_stats*) {
    return coli::fail(COLI_EUNSUPPORTED, "expert cache not available yet");
}
coli_status coli_expert_cache_reset(struct coli_expert_cache*) {
    return coli::fail(COLI_EUNSUPPORTED, "expert cache not available yet");
}
}
