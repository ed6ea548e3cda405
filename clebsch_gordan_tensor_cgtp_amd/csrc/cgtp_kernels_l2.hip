// cgtp_kernels_l2.hip -- degree-2 specialisations (features, SH and outputs l = 0..2).
#include "cgtp_kernels.h"

namespace cgtp {

static const KernelSet kSets[] = {
    make_set<2, 8>(),
    make_set<2, 16>(),
    make_set<2, 32>(),
    make_set<2, 64>(),
    make_set<2, 128>(),
};

const KernelSet* kernels_l2(int channels)
{
    for (const KernelSet& k : kSets)
        if (k.channels == channels) return &k;
    return nullptr;
}

bool table_l2(int path, double* dense) { return copy_table<2, 2, 2>(path, dense); }

}  // namespace cgtp
