// cgtp_kernels_l3_c64.hip -- degree-3 convolution kernels for 64 channels.
#include "cgtp_kernels.h"

namespace cgtp {

KernelSet conv_set_l3_c64() { return make_conv_set<3, 64>(); }

}  // namespace cgtp
