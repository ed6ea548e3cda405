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

// node-range splits of the weight gradient, and its workspace
int32_t mix_splits(int64_t N, int32_t P, int32_t C, int32_t Co);
size_t mix_workspace_bytes(int64_t N, int32_t P, int32_t C, int32_t Co);

// out [N][Dout][Co] from mid [N][Dmid][C] and Wmix [P][C][Co]
hipError_t launch_mix_fwd(const MixShape& m, const float* mid, const float* Wmix, float* out, hipStream_t s);

// d_mid [N][Dmid][C] and dW [P][C][Co] (either may be nullptr); part: the
// workspace of mix_workspace_bytes
hipError_t launch_mix_bwd(const MixShape& m, const float* mid, const float* Wmix, const float* G, float* dmid,
                          float* dW, double* part, hipStream_t s);

}  // namespace cgtp
