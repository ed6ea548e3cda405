// cgtp_kernels_l1.hip -- degree-1 kernels (paths of l_in, l_sh, l_out <= 1),
// every lane geometry.
#include "cgtp_kernels.h"

namespace cgtp {

// host-side table of this unit's kernels, indexed by lane geometry
const KernelSet* kernels_l1(int g)
{
    static const KernelSet sets[5] = {make_set<1, 8, 1>(), make_set<1, 16, 1>(), make_set<1, 32, 1>(),
                                      make_set<1, 64, 1>(), make_set<1, 64, 2>()};
    return &sets[g];
}

}  // namespace cgtp
