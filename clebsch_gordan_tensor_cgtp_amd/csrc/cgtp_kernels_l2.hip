// cgtp_kernels_l2.hip -- degree-2 kernels (paths of l_in, l_sh, l_out <= 2)
// for up to 32 channels.
#include "cgtp_kernels.h"

namespace cgtp {

// host-side table of this unit's kernels: geometries 0..2 (8, 16, 32 lanes)
const KernelSet* kernels_l2_narrow(int g)
{
    static const KernelSet sets[3] = {make_set<2, 8, 1>(), make_set<2, 16, 1>(), make_set<2, 32, 1>()};
    return &sets[g];
}

}  // namespace cgtp
