// Instantiations of the LDS-path backward for log2 L in {9, 10}.
#include "lds_backward.hpp"

namespace hy {
template hipError_t launch_lds_backward_t<9>(const LdsBwdArgs&, hipStream_t);
template hipError_t launch_lds_backward_t<10>(const LdsBwdArgs&, hipStream_t);
}  // namespace hy
