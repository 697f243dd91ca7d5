// Library-wide entry points: workspace sizing, status strings, device facts.
#include "common.h"

namespace moe {

size_t pre_reorder_ws_bytes(int64_t T, int32_t topk, int32_t num_local);
size_t act_requant_ws_bytes();

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cached[dev] = n;
    return n;
}

}  // namespace moe

extern "C" size_t moe_workspace_bytes(int64_t T, int32_t topk, int32_t num_local) {
    if (T < 0) T = 0;
    if (topk < 1) topk = 1;
    if (num_local < 0) num_local = 0;
    const size_t a = moe::pre_reorder_ws_bytes(T, topk, num_local);
    const size_t b = moe::act_requant_ws_bytes();
    return a > b ? a : b;
}

extern "C" const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: argument out of range or misaligned";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: buffer size does not match the mode";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: combination not implemented";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error at launch";
        default: return "unknown moe_status";
    }
}
