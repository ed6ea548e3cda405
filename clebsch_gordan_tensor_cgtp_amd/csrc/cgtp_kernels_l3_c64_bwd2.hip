// cgtp_kernels_l3_c64_bwd2.hip -- the double-backward (sender side) and
// per-path-output backward kernels of the degree-3, 64-lane x 1-slice
// geometry (see cgtp_kernels_l3_c64.hip).
#include "cgtp_kernels.h"

namespace cgtp {

KernelSet kernels_l3_c64_bwd2() { return make_set_bwd2<3, 64, 1>(); }

}  // namespace cgtp
