// Instantiations of the LDS path for log2 L in {4, 5, 6, 7, 8, 9, 10}.
#include "lds_path.hpp"

namespace hy {
template hipError_t launch_lds_forward_t<4>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<4>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
template hipError_t launch_lds_forward_t<5>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<5>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
template hipError_t launch_lds_forward_t<6>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<6>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
template hipError_t launch_lds_forward_t<7>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<7>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
template hipError_t launch_lds_forward_t<8>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<8>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
template hipError_t launch_lds_forward_t<9>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<9>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
template hipError_t launch_lds_forward_t<10>(const LdsArgs&, hipStream_t);
template hipError_t launch_lds_spectrum_t<10>(const float*, float2*, int64_t, const float2*, const float2*, hipStream_t, bool);
}  // namespace hy
