// Output projection of the Hyena operator on the bf16 matrix cores (outproj.hip):
// out[b][t][n] = sum_k y[b][k][t] w_out[n][k] + b_out[n], y channels-first, out tokens-first.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hy {

// D a multiple of 64 and L a multiple of 8
bool outproj_supported(int64_t D, int64_t L);
// One launch over all B sequences on `st`; hipErrorInvalidValue for unsupported
// shapes or when a sequence of y or out (L*D*2 bytes) or w_out reaches 2 GiB.
hipError_t launch_outproj(const uint16_t* y, const uint16_t* w, const uint16_t* bo, uint16_t* out, int64_t B,
                          int64_t L, int64_t D, hipStream_t st);

}  // namespace hy
