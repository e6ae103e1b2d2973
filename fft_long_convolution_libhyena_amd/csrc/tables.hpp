// Host-side twiddle tables shared by the C-ABI translation units: every value is
// computed in fp64 after an exact integer reduction of its angle and rounded
// once to fp32.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <vector>

namespace hy {

// exp(-2 pi i num / den) computed in fp64 after an exact integer reduction.
inline float2 wfwd(int64_t num, int64_t den) {
    constexpr double kTwoPi = 6.283185307179586476925286766559;
    int64_t r = num % den;
    if (r < 0) r += den;
    const double a = -kTwoPi * (double)r / (double)den;
    return make_float2((float)cos(a), (float)sin(a));
}

// Stockham per-pass tables for a length-n transform, in the order the device
// schedule reads them: pass 0 (NS = 1) needs none; pass p >= 1 (radix R,
// NS = 16^p) holds W_{NS*R}^{r*k} at [(r-1)*NS + k], r = 1..R-1, k = 0..NS-1.
// Returns the index at which the table starts.
inline size_t append_stockham(std::vector<float2>& out, int logn) {
    const size_t start = out.size();
    const int full = logn / 4, rem = logn % 4;
    const int npass = full + (rem ? 1 : 0);
    int64_t ns = 1;
    for (int p = 0; p < npass; ++p) {
        const int R = p < full ? 16 : (1 << rem);
        if (p > 0)
            for (int r = 1; r < R; ++r)
                for (int64_t k = 0; k < ns; ++k) out.push_back(wfwd((int64_t)r * k, ns * R));
        ns *= R;
    }
    return start;
}

}  // namespace hy
