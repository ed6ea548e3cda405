// cgtp_kernels_l1.hip -- degree-1 specialisations (features, SH and outputs l = 0..1).
#include "cgtp_kernels.h"

namespace cgtp {

static const KernelSet kSets[] = {
    make_set<1, 8>(),
    make_set<1, 16>(),
    make_set<1, 32>(),
    make_set<1, 64>(),
    make_set<1, 128>(),
};

const KernelSet* kernels_l1(int channels)
{
    for (const KernelSet& k : kSets)
        if (k.channels == channels) return &k;
    return nullptr;
}

bool table_l1(int path, double* dense) { return copy_table<1, 1, 1>(path, dense); }

}  // namespace cgtp
