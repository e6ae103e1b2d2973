// Instantiations of the LDS-path backward for log2 L in {11, 12}.
#include "lds_backward.hpp"

namespace hy {
template hipError_t launch_lds_backward_t<11>(const LdsBwdArgs&, hipStream_t);
template hipError_t launch_lds_backward_t<12>(const LdsBwdArgs&, hipStream_t);
}  // namespace hy
