// Instantiations of the LDS-path backward for log2 L in {4, 5, 6}, and the
// dispatch over sizes.
#include "lds_backward.hpp"

namespace hy {
// instantiated in lds_backward_b.hip .. lds_backward_f.hip
extern template hipError_t launch_lds_backward_t<7>(const LdsBwdArgs&, hipStream_t);
extern template hipError_t launch_lds_backward_t<8>(const LdsBwdArgs&, hipStream_t);
extern template hipError_t launch_lds_backward_t<9>(const LdsBwdArgs&, hipStream_t);
extern template hipError_t launch_lds_backward_t<10>(const LdsBwdArgs&, hipStream_t);
extern template hipError_t launch_lds_backward_t<11>(const LdsBwdArgs&, hipStream_t);
extern template hipError_t launch_lds_backward_t<12>(const LdsBwdArgs&, hipStream_t);
extern template hipError_t launch_lds_backward_t<13>(const LdsBwdArgs&, hipStream_t);
extern template hipError_t launch_lds_backward_t<14>(const LdsBwdArgs&, hipStream_t);

template hipError_t launch_lds_backward_t<4>(const LdsBwdArgs&, hipStream_t);
template hipError_t launch_lds_backward_t<5>(const LdsBwdArgs&, hipStream_t);
template hipError_t launch_lds_backward_t<6>(const LdsBwdArgs&, hipStream_t);

hipError_t launch_lds_backward(int logL, const LdsBwdArgs& a, hipStream_t st) {
    switch (logL) {
        case 4: return launch_lds_backward_t<4>(a, st);
        case 5: return launch_lds_backward_t<5>(a, st);
        case 6: return launch_lds_backward_t<6>(a, st);
        case 7: return launch_lds_backward_t<7>(a, st);
        case 8: return launch_lds_backward_t<8>(a, st);
        case 9: return launch_lds_backward_t<9>(a, st);
        case 10: return launch_lds_backward_t<10>(a, st);
        case 11: return launch_lds_backward_t<11>(a, st);
        case 12: return launch_lds_backward_t<12>(a, st);
        case 13: return launch_lds_backward_t<13>(a, st);
        case 14: return launch_lds_backward_t<14>(a, st);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace hy
