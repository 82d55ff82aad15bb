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
