// cgtp_kernels_l3_c128.hip -- degree-3 kernels (paths of l_in, l_sh, l_out <= 3)
// for channel counts served by 64 lanes x 2 slice(s); one unit per lane
// geometry so the degree-3 builds run in parallel.
#include "cgtp_kernels.h"

namespace cgtp {

const KernelSet* kernels_l3_c128()
{
    static const KernelSet set = make_set<3, 64, 2>();
    return &set;
}

}  // namespace cgtp
