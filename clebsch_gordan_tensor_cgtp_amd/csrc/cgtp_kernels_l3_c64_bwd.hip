// cgtp_kernels_l3_c64_bwd.hip -- the plain and fused-SH backward kernels of
// the degree-3, 64-lane x 1-slice geometry (see cgtp_kernels_l3_c64.hip).
#include "cgtp_kernels.h"

namespace cgtp {

KernelSet kernels_l3_c64_bwd1() { return make_set_bwd1<3, 64, 1>(); }

}  // namespace cgtp
