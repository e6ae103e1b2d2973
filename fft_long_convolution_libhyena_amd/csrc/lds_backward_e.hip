// Instantiations of the LDS-path backward for log2 L in {7, 8}.
#include "lds_backward.hpp"

namespace hy {
template hipError_t launch_lds_backward_t<7>(const LdsBwdArgs&, hipStream_t);
template hipError_t launch_lds_backward_t<8>(const LdsBwdArgs&, hipStream_t);
}  // namespace hy
