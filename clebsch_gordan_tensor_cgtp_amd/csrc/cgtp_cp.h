// cgtp_cp.h -- arguments, workspace layout and launcher table of the
// CP-decomposed tensor-product convolution (kernels in cgtp_cp.hip, the fit of
// the factors in cgtp_cp_fit.cpp).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "cgtp_internal.h"

namespace cgtp {

constexpr int kMaxCpRank = 64;

// rank padded to the compiled size (16, 32 or 64)
int cp_padded_rank(int R);

// Byte offsets, after the graph view, of the CP buffers in the workspace:
//   xb  [N][RP][C] f64   B^T x per sender node
//   ga  [N][RP][C] f64   A^T grad_out per receiver node
//   yc  [E][RP]    f64   C^T Y per edge
//   dyc [E][H][RP] f64   per-edge gradient for C^T Y, one row per channel slice
//   dwa [E][C]     f64   grad_W summed over the backward's passes (only when
//                        the backward walks the edges more than once: rank
//                        above 32, or above 16 with C <= 32)
// All are fp64: the projection by A (or B) sums rank terms of mixed sign,
// and a rounded intermediate would be amplified by that cancellation.
struct CpWsLayout {
    size_t xb, ga, yc, dyc, dwa, total;
};

inline CpWsLayout cp_ws_layout(int64_t N, int64_t E, int RP, int C)
{
    CpWsLayout w{};
    const size_t n1 = (size_t)(N > 0 ? N : 1), e1 = (size_t)(E > 0 ? E : 1);
    const int H = C > 64 ? 2 : 1;
    size_t o = ws_layout(N, E).total;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += align256(bytes);
        return at;
    };
    w.xb = take(sizeof(double) * n1 * RP * (size_t)C);
    w.ga = take(sizeof(double) * n1 * RP * (size_t)C);
    w.yc = take(sizeof(double) * e1 * RP);
    w.dyc = take(sizeof(double) * e1 * H * RP);
    const bool passes = C > 32 ? RP > 32 : RP > 16;
    w.dwa = take(passes ? sizeof(double) * e1 * (size_t)C : 0);
    w.total = o;
    return w;
}

struct CpFwdArgs {
    int32_t N, E, C, R, d3;
    int64_t n_order;          // entries of `order` (conv_grid(N))
    const int32_t* order;     // receivers, longest segment first (-1: idle)
    const int32_t* row_ptr;
    const int32_t* src;
    const float* W;           // [E][C]
    const float* A;           // [d3][R]
    const double* xb;         // [N][RP][C]
    const double* yc;         // [E][RP]
    float* out;               // [N][d3][C]
};

struct CpBwdArgs {
    int32_t N, E, C, R, d1;
    int64_t n_order;
    const int32_t* order;     // senders, longest first (-1: idle)
    const int32_t* srow;      // sender-sorted view
    const int32_t* perm;
    const int32_t* sdst;
    const float* W;           // [E][C]
    const float* B;           // [d1][R]
    const double* xb;         // [N][RP][C]
    const double* ga;         // [N][RP][C]
    const double* yc;         // [E][RP]
    float* dx;                // [N][d1][C] or nullptr
    float* dW;                // [E][C] or nullptr
    double* dyc;              // [E][H][RP] or nullptr
    double* dwa;              // [E][C]: grad_W between passes
};

using CpFwdLaunch = hipError_t (*)(const CpFwdArgs& a, hipStream_t s);
using CpBwdLaunch = hipError_t (*)(const CpBwdArgs& a, hipStream_t s);
using CpProjRows = hipError_t (*)(int64_t rows, int32_t D, int32_t R, int32_t C, const float* M, const float* in,
                                  double* out, hipStream_t s);
using CpProjEdge = hipError_t (*)(int64_t E, int32_t D, int32_t R, const float* Cf, const float* Y, double* yc,
                                  hipStream_t s);
using CpEdgeBack = hipError_t (*)(int64_t E, int32_t D, int32_t R, int32_t H, const float* Cf, const double* dyc,
                                  float* dY, hipStream_t s);

// The kernels of one padded rank RP and one lane geometry (LPE lanes per
// node, H waves per node).
struct CpKernelSet {
    int rp, lpe, h;
    CpFwdLaunch fwd;
    CpBwdLaunch bwd;
    CpProjRows proj_rows;
    CpProjEdge proj_edge;
    CpEdgeBack edge_back;
};

// kernels for rank R (1..64) and channel count C (1..128), or nullptr
const CpKernelSet* find_cp_kernels(int rank, int channels);

// Alternating least squares for the rank-R factors of the coupling tensor M
// [d1][d2][d3] (row-major): A [d3][R], B [d1][R], Cf [d2][R] are the start on
// entry and the fit on return.  Per sweep B, then Cf, then A is replaced by
// the exact least-squares solution with the other two fixed (normal matrix:
// Hadamard product of their Gram matrices, plus ridge * trace / R on the
// diagonal, solved by Cholesky).  Returns false if a normal matrix is not
// positive definite.  *rel_err: ||M - [[A, B, Cf]]|| / ||M|| at the end.
bool cp_als_fit(const double* M, int d1, int d2, int d3, int R, int sweeps, double ridge, double* A, double* B,
                double* Cf, double* rel_err);

}  // namespace cgtp
