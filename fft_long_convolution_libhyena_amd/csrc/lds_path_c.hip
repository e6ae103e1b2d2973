// Instantiations of the LDS path for log2 L in {13}.
#include "lds_path.hpp"

namespace hy {
template hipError_t launch_lds_forward_t<13>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<13>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
}  // namespace hy
