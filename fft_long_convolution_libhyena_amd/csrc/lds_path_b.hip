// Instantiations of the LDS path for log2 L in {11, 12}.
#include "lds_path.hpp"

namespace hy {
template hipError_t launch_lds_forward_t<11>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<11>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
template hipError_t launch_lds_forward_t<12>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<12>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
}  // namespace hy
