// The plan object behind hyena_plan_t and small host helpers shared by the
// C-ABI translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hyena.h"
#include "kernels.hpp"

struct hyena_plan_s {
    int64_t L = 0, D = 0;
    int order = 0;
    int logL = 0;            // log2 of the sequence length
    int logT = 0;            // log2 of the packed complex transform length (logL - circular)
    bool circular = false;   // circular convolution instead of zero padding to 2L
    hyena_dtype_t dtype = HYENA_F32;
    hyena_path_t path = HYENA_PATH_AUTO;
    int device = -1;
    float2* dtab = nullptr;  // all twiddle tables, one device allocation
    // LDS path
    const float2* tw = nullptr;
    const float2* wpair = nullptr;
    // four-step path
    int log1 = 0, log2 = 0;
    hy::FsTables fs{};
    // state of the operator entry points (projection GEMM handles and descriptors),
    // attached on their first call and released with the plan
    void* op = nullptr;
    void (*op_free)(void*) = nullptr;
};

namespace hy {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The plan's device must be the current one.
inline hyena_status_t check_device(const hyena_plan_t plan) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HYENA_ERR_DEVICE;
    return dev == plan->device ? HYENA_OK : HYENA_ERR_DEVICE;
}

}  // namespace hy
