// Library-wide entry points of the verification ABI (version, status text).
#include "ttv_device.h"

extern "C" TTV_API int32_t ttv_version(void) { return 100; }  // 0.1.0

extern "C" TTV_API const char* ttv_status_string(int32_t status) {
    switch (status) {
        case TTV_OK: return "ok";
        case TTV_EINVAL: return "invalid argument (nothing launched)";
        case TTV_EHIP: return "HIP launch failure";
        case TTV_ENOSPC: return "workspace too small (nothing launched)";
        default: return "unknown status";
    }
}

#ifdef TTV_DEBUG
// One reader per translation unit (TTV_DEBUG_TU at the end of each source).
extern "C" int ttv_debug_take_build(unsigned int*, int);
extern "C" int ttv_debug_take_attention(unsigned int*, int);
extern "C" int ttv_debug_take_accept(unsigned int*, int);
extern "C" int ttv_debug_take_commit(unsigned int*, int);
extern "C" int ttv_debug_take_stochastic(unsigned int*, int);
extern "C" int ttv_debug_take_mask(unsigned int*, int);
extern "C" int ttv_debug_take_ddtree(unsigned int*, int);
extern "C" int ttv_debug_take_merge(unsigned int*, int);
#endif

extern "C" TTV_API int ttv_debug_report(uint32_t* violations, int32_t* first_site, int32_t reset) {
    if (!violations || !first_site) return TTV_EINVAL;
    *violations = 0;
    *first_site = 0;
#ifdef TTV_DEBUG
    int (*const take[])(unsigned int*, int) = {
        ttv_debug_take_build, ttv_debug_take_attention, ttv_debug_take_accept, ttv_debug_take_commit,
        ttv_debug_take_stochastic, ttv_debug_take_mask, ttv_debug_take_ddtree, ttv_debug_take_merge};
    for (auto f : take) {
        unsigned int w[2] = {0u, 0u};
        const int st = f(w, reset);
        if (st != TTV_OK) return st;
        *violations += w[0];
        if (w[0] != 0 && *first_site == 0) *first_site = (int32_t)w[1];
    }
    return TTV_OK;
#else
    (void)reset;
    return TTV_EINVAL;
#endif
}
