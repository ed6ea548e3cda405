// cgtp_kernels_l2_wide.hip -- degree-2 kernels (paths of l_in, l_sh, l_out <= 2)
// for 33 to 128 channels.
#include "cgtp_kernels.h"

namespace cgtp {

// host-side table of this unit's kernels: geometries 3 (64 lanes) and 4 (2 x 64)
const KernelSet* kernels_l2_wide(int g)
{
    static const KernelSet sets[2] = {make_set<2, 64, 1>(), make_set<2, 64, 2>()};
    return &sets[g - 3];
}

}  // namespace cgtp
