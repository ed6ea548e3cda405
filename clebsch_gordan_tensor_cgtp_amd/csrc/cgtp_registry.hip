// cgtp_registry.hip -- the spherical-harmonics launchers and the table of
// compiled convolution kernels (one entry per degree and lane geometry).
#include "cgtp_kernels.h"

namespace cgtp {

const KernelSet* kernels_l1(int g);
const KernelSet* kernels_l2_narrow(int g);
const KernelSet* kernels_l2_wide(int g);
const KernelSet* kernels_l3_c8();
const KernelSet* kernels_l3_c16();
const KernelSet* kernels_l3_c32();
const KernelSet* kernels_l3_c64();
const KernelSet* kernels_l3_c128();

// lane geometry serving C channels: 0..3 -> 8, 16, 32, 64 lanes x 1 slice;
// 4 -> 64 lanes x 2 slices; -1 if C is out of range
static int geometry(int C)
{
    if (C < 1) return -1;
    if (C <= 8) return 0;
    if (C <= 16) return 1;
    if (C <= 32) return 2;
    if (C <= 64) return 3;
    if (C <= 128) return 4;
    return -1;
}

const KernelSet* find_kernels(int lm, int channels)
{
    const int g = geometry(channels);
    if (g < 0) return nullptr;
    switch (lm) {
        case 1: return kernels_l1(g);
        case 2: return g < 3 ? kernels_l2_narrow(g) : kernels_l2_wide(g);
        case 3: {
            switch (g) {
                case 0: return kernels_l3_c8();
                case 1: return kernels_l3_c16();
                case 2: return kernels_l3_c32();
                case 3: return kernels_l3_c64();
                default: return kernels_l3_c128();
            }
        }
        default: return nullptr;
    }
}

ShLaunch find_sh(int l)
{
    switch (l) {
        case 0: return &launch_sh<0>;
        case 1: return &launch_sh<1>;
        case 2: return &launch_sh<2>;
        case 3: return &launch_sh<3>;
        default: return nullptr;
    }
}

bool host_cg_table(int lm, int path, double* dense)
{
    switch (lm) {
        case 1: return copy_table<1>(path, dense);
        case 2: return copy_table<2>(path, dense);
        case 3: return copy_table<3>(path, dense);
        default: return false;
    }
}

}  // namespace cgtp
