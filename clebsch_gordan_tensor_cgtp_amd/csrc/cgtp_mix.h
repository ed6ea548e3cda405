// cgtp_mix.h -- the fully connected ("uvw") mixing of the per-path outputs
// (kernels in cgtp_mix.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "cgtp_internal.h"

namespace cgtp {

// Shapes of one mixing: N nodes, C input and Co output channels, the plan's
// P paths with their output degree l3[p] and first per-path row o[p];
// Dmid = sum_p (2*l3+1) per-path rows, Dout = (l_out+1)^2 summed rows.
struct MixShape {
    int32_t N, C, Co, P, Dmid, Dout;
    int32_t l3[kMaxPaths], o[kMaxPaths];
};

// Splits of the weight gradient's sum: path p's N*(2*l3+1) (row, node)
// pairs are cut into runs of `rows` (a whole number of 32-row chunks), runs
// off[p] .. off[p+1]-1 of all paths' runs; each run is one block per tile.
struct MixSplit {
    int32_t rows;
    int32_t off[kMaxPaths + 1];
};
MixSplit mix_split(const MixShape& m);

// workspace of the weight gradient: the fp64 partial of every run
size_t mix_workspace_bytes(const MixShape& m);

// out [N][Dout][Co] from mid [N][Dmid][C] and Wmix [P][C][Co]
hipError_t launch_mix_fwd(const MixShape& m, const float* mid, const float* Wmix, float* out, hipStream_t s);

// d_mid [N][Dmid][C] and dW [P][C][Co] (either may be nullptr); part: the
// workspace of mix_workspace_bytes(m)
hipError_t launch_mix_bwd(const MixShape& m, const float* mid, const float* Wmix, const float* G, float* dmid,
                          float* dW, double* part, hipStream_t s);

}  // namespace cgtp
