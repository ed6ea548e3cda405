// cgtp_kernels_l3_c64.hip -- degree-3 kernels (paths of l_in, l_sh, l_out <= 3)
// for channel counts served by 64 lanes x 1 slice(s); one unit per lane
// geometry so the degree-3 builds run in parallel.  This geometry's backward
// kernels (path-split and single-wave forms), the slowest to compile, sit in
// units of their own: cgtp_kernels_l3_c64_bwd.hip (plain and fused-SH forms)
// and cgtp_kernels_l3_c64_bwd2.hip (double-backward and per-path forms).
#include "cgtp_kernels.h"

namespace cgtp {

KernelSet kernels_l3_c64_bwd1();
KernelSet kernels_l3_c64_bwd2();

const KernelSet* kernels_l3_c64()
{
    static const KernelSet set = merge_sets(make_set_fwd<3, 64, 1>(), kernels_l3_c64_bwd1(), kernels_l3_c64_bwd2());
    return &set;
}

}  // namespace cgtp
