// cgtp_forces.hip -- the spherical-harmonics backward and the per-node
// gradient: the path from the convolution's grad_Y to the forces on atoms.
//
// The backward's grad_Y term is what feeds the force computation of an
// interatomic potential: grad_Y -> grad_r (this file, k_sh_bwd) -> the
// gradient with respect to each atom position (k_node_grad).  The AccelNet
// review (Referee Report) validates exactly such analytic forces against
// finite differences; the tests do the same against the oracle.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cgtp_internal.h"
#include "cgtp_math.h"
#include "cgtp_sh.h"

namespace cgtp {

namespace {

__device__ __forceinline__ int32_t clampi(int32_t v, int32_t lo, int32_t hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

}  // namespace

// grad_r[e] = sum_k grad_Y[e][k] dY_k/dr for degrees 0..L.  Y_k is a
// polynomial of the unit vector u = r/|r|; with q = sum_k grad_Y[e][k] grad_u
// of that polynomial, dY/dr = (I - u u^T)/|r| gives grad_r = (q - u (u.q))/|r|.
// One thread per edge, fp64 arithmetic on fp32 data.
template <int L>
__global__ void __launch_bounds__(256) k_sh_bwd(int64_t E, const float* __restrict__ r,
                                                 const float* __restrict__ gY, float* __restrict__ gr)
{
    constexpr int D = (L + 1) * (L + 1);
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    double x, y, z, inv;
    shf::unit(r[3 * e + 0], r[3 * e + 1], r[3 * e + 2], x, y, z, inv);
    double w[D];
#pragma unroll
    for (int k = 0; k < D; ++k) w[k] = (double)gY[e * D + k];
    double qx = 0.0, qy = 0.0, qz = 0.0;
    if constexpr (L >= 1) shf::grad_degree<1>(x, y, z, w + 1, qx, qy, qz);
    if constexpr (L >= 2) shf::grad_degree<2>(x, y, z, w + 4, qx, qy, qz);
    if constexpr (L >= 3) shf::grad_degree<3>(x, y, z, w + 9, qx, qy, qz);
    double g[3];
    shf::tangent(x, y, z, inv, qx, qy, qz, g);
    gr[3 * e + 0] = (float)g[0];
    gr[3 * e + 1] = (float)g[1];
    gr[3 * e + 2] = (float)g[2];
}

template <int L>
hipError_t launch_sh_bwd(int64_t E, const float* r, const float* gY, float* gr, hipStream_t s)
{
    if (E == 0) return hipSuccess;
    hipLaunchKernelGGL(k_sh_bwd<L>, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, E, r, gY, gr);
    return hipGetLastError();
}

ShBwdLaunch find_sh_bwd(int l)
{
    switch (l) {
        case 0: return &launch_sh_bwd<0>;
        case 1: return &launch_sh_bwd<1>;
        case 2: return &launch_sh_bwd<2>;
        case 3: return &launch_sh_bwd<3>;
        default: return nullptr;
    }
}

// gpos[n] = sum of grad_r over the out-edges of n (r = pos[src] - pos[dst]
// grows with pos[src]) minus the sum over its in-edges.  One wave per node,
// atomic-free: the out-edges come from the sender-sorted view, the in-edges
// from the CSR segment; lane l takes entries l, l+64, ... and the wave adds
// its lanes in a fixed butterfly order, so the result is deterministic.
__global__ void __launch_bounds__(256) k_node_grad(int32_t N, int32_t E, const int32_t* __restrict__ row_ptr,
                                                    const int32_t* __restrict__ srow, const int32_t* __restrict__ perm,
                                                    const float* __restrict__ gr, float* __restrict__ gpos)
{
    const int32_t n = (int32_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (n >= N) return;
    double ax = 0.0, ay = 0.0, az = 0.0;
    const int32_t q0 = clampi(srow[n], 0, E), q1 = clampi(srow[n + 1], q0, E);
    for (int32_t q = q0 + lane; q < q1; q += 64) {
        const int32_t e = perm[q];
        if ((uint32_t)e >= (uint32_t)E) continue;  // a view not prepared for this graph
        ax += gr[3 * (int64_t)e + 0];
        ay += gr[3 * (int64_t)e + 1];
        az += gr[3 * (int64_t)e + 2];
    }
    const int32_t e0 = clampi(row_ptr[n], 0, E), e1 = clampi(row_ptr[n + 1], e0, E);
    for (int32_t e = e0 + lane; e < e1; e += 64) {
        ax -= gr[3 * (int64_t)e + 0];
        ay -= gr[3 * (int64_t)e + 1];
        az -= gr[3 * (int64_t)e + 2];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        ax += __shfl_xor(ax, off, 64);
        ay += __shfl_xor(ay, off, 64);
        az += __shfl_xor(az, off, 64);
    }
    if (lane == 0) {
        gpos[3 * (int64_t)n + 0] = (float)ax;
        gpos[3 * (int64_t)n + 1] = (float)ay;
        gpos[3 * (int64_t)n + 2] = (float)az;
    }
}

hipError_t launch_node_grad(int32_t N, int32_t E, const int32_t* row_ptr, const GraphView& g, const float* gr,
                            float* gpos, hipStream_t s)
{
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(k_node_grad, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, N, E, row_ptr, g.srow, g.perm,
                       gr, gpos);
    return hipGetLastError();
}

}  // namespace cgtp
