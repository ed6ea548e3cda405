// cgtp_kernels_l3_c16.hip -- degree-3 convolution kernels for 16 channels.
#include "cgtp_kernels.h"

namespace cgtp {

KernelSet conv_set_l3_c16() { return make_conv_set<3, 16>(); }

}  // namespace cgtp
