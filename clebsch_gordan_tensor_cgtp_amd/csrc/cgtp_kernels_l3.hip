// cgtp_kernels_l3.hip -- degree-3 registry (features, SH and outputs l = 0..3).
// The convolution kernels of each channel count are compiled in a translation
// unit of their own (cgtp_kernels_l3_c<C>.hip) so the builds run in parallel.
#include "cgtp_kernels.h"

namespace cgtp {

KernelSet conv_set_l3_c8();
KernelSet conv_set_l3_c16();
KernelSet conv_set_l3_c32();
KernelSet conv_set_l3_c64();

static KernelSet with_sh(KernelSet k)
{
    k.sh = &launch_sh<3>;
    return k;
}

const KernelSet* kernels_l3(int channels)
{
    static const KernelSet sets[] = {with_sh(conv_set_l3_c8()), with_sh(conv_set_l3_c16()),
                                     with_sh(conv_set_l3_c32()), with_sh(conv_set_l3_c64())};
    for (const KernelSet& k : sets)
        if (k.channels == channels) return &k;
    return nullptr;
}

bool table_l3(int path, double* dense) { return copy_table<3, 3, 3>(path, dense); }

}  // namespace cgtp
