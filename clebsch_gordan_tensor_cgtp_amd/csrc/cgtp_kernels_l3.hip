// cgtp_kernels_l3.hip -- degree-3 specialisations (features, SH and outputs l = 0..3).
#include "cgtp_kernels.h"

namespace cgtp {

static const KernelSet kSets[] = {
    make_set<3, 8>(),
    make_set<3, 16>(),
    make_set<3, 32>(),
    make_set<3, 64>(),
};

const KernelSet* kernels_l3(int channels)
{
    for (const KernelSet& k : kSets)
        if (k.channels == channels) return &k;
    return nullptr;
}

bool table_l3(int path, double* dense) { return copy_table<3, 3, 3>(path, dense); }

}  // namespace cgtp
