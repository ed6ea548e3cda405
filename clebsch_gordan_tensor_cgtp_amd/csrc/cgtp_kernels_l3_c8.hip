// cgtp_kernels_l3_c8.hip -- degree-3 convolution kernels for 8 channels.
#include "cgtp_kernels.h"

namespace cgtp {

KernelSet conv_set_l3_c8() { return make_conv_set<3, 8>(); }

}  // namespace cgtp
