// Instantiations of the LDS-path backward for log2 L in {14}.
#include "lds_backward.hpp"

namespace hy {
template hipError_t launch_lds_backward_t<14>(const LdsBwdArgs&, hipStream_t);
}  // namespace hy
