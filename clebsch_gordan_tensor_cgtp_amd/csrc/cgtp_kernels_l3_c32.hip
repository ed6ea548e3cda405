// cgtp_kernels_l3_c32.hip -- degree-3 convolution kernels for 32 channels.
#include "cgtp_kernels.h"

namespace cgtp {

KernelSet conv_set_l3_c32() { return make_conv_set<3, 32>(); }

}  // namespace cgtp
