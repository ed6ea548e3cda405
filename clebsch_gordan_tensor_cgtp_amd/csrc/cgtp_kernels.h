// cgtp_kernels.h -- gfx950 kernels of the CGTP convolution (templates; each
// cgtp_kernels_l<L>.hip instantiates one degree).
//
// Hot path (the convolution LunaTP's abstract calls the cost centre of
// equivariant MLIPs; "LunaTP: Enabling Efficient and Scalable Tensor Product
// for Equivariant MLIPs", Abstract):
//   * real spherical harmonics of the edge vectors          (k_sh)
//   * forward, node-centric: the waves of a receiver walk its CSR segment,
//     gather the sender rows x_j with channel-contiguous loads, stream W[e],
//     accumulate in registers and write out[i] once; no atomics (k_conv_fwd)
//   * backward, sender-centric over the sender-sorted view: the waves of a
//     sender keep x_j and grad_x[j] in registers, gather the grad_out rows of
//     its receivers, write grad_W[e] per edge and grad_Y[e] reduced over the
//     channels; no atomics                                   (k_conv_bwd)
// (graph preparation lives in cgtp_graph.hip)
//
// Arithmetic is fp64 on fp32 data: the per-edge contraction and the sums over
// a segment and over channels keep fp64 accuracy, and fp64 FMA issues at the
// same rate as unpacked fp32 on this chip.
//
// Lane mapping: a lane owns one channel of one edge.  For C >= 64 a node's
// channels are split over C/64 waves (each owning a 64-channel slice of the
// node's rows); for C < 64 a wave covers 64/C edges of the segment at once and
// reduces across those edge groups at the end.  The CG values and their
// nonzero pattern are compile-time constants of the (L_in, L_sh, L_out)
// specialisation, so every contraction below is a straight line of fp64 FMAs
// over the nonzero coefficients only.
//
// Reuse inside an edge ("multi-level reuse" in the LunaTP abstract, done here
// per channel):
//   forward:  q[a][b] = x[l1,a] Y[l2,b] is formed once per (l1,l2) block and
//             shared by every path (l1,l2,l3) of the block; z_p = T_p q.
//   backward: R_p[a][b] = sum_m3 T_p[a][b][m3] g[l3,m3] gives both
//             h_p = R_p Y (-> grad_x += W h_p, grad_W = x . h_p) and
//             v_p = R_p^T x (-> grad_Y += W v_p).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>
#include <utility>

#include "cgtp_internal.h"
#include "cgtp_math.h"

namespace cgtp {

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Compile-time facts about path p of a table set.
template <class Tb, int p>
struct PathK {
    static constexpr int l1 = Tb::data.l1[p], l2 = Tb::data.l2[p], l3 = Tb::data.l3[p];
    static constexpr int d1 = 2 * l1 + 1, d2 = 2 * l2 + 1, d3 = 2 * l3 + 1;
    static constexpr int k1 = l1 * l1, k2 = l2 * l2, k3 = l3 * l3;  // first component of each degree
    // coefficient at 0-based (a, b, c) = (m1+l1, m2+l2, m3+l3)
    static constexpr double T(int a, int b, int c) { return Tb::t(p, a - l1, b - l2, c - l3); }
    static constexpr bool NZ(int a, int c)
    {
        for (int b = 0; b < d2; ++b)
            if (T(a, b, c) != 0.0) return true;
        return false;
    }
    static constexpr bool ROW(int a)
    {
        for (int c = 0; c < d3; ++c)
            if (NZ(a, c)) return true;
        return false;
    }
    static constexpr bool COL2(int b)
    {
        for (int a = 0; a < d1; ++a)
            for (int c = 0; c < d3; ++c)
                if (T(a, b, c) != 0.0) return true;
        return false;
    }
};

// M[a][c] = sum_b T[a][b][c] y[k2 + b] for the nonzero (a, c) pairs of path K.
template <class K, int DSH>
__device__ __forceinline__ void make_M(const double (&y)[DSH], double (&M)[K::d1][K::d3])
{
    static_for<0, K::d1>([&](auto A) {
        static_for<0, K::d3>([&](auto Cc) {
            constexpr int a = decltype(A)::value, c = decltype(Cc)::value;
            if constexpr (K::NZ(a, c)) {
                double s = 0.0;
                static_for<0, K::d2>([&](auto B) {
                    constexpr int b = decltype(B)::value;
                    constexpr double t = K::T(a, b, c);
                    if constexpr (t != 0.0) s = __builtin_fma(t, y[K::k2 + b], s);
                });
                M[a][c] = s;
            }
        });
    });
}

// ----------------------------------------------------------------------------
// real spherical harmonics (orthonormal, l <= 3), fp64 from fp32 vectors
// ----------------------------------------------------------------------------
template <int L>
__global__ void __launch_bounds__(256) k_sh(int64_t E, const float* __restrict__ r, float* __restrict__ Y)
{
    constexpr int D = (L + 1) * (L + 1);
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    const double rx = r[3 * e + 0], ry = r[3 * e + 1], rz = r[3 * e + 2];
    const double n = sqrt(rx * rx + ry * ry + rz * rz);
    const double x = rx / n, y = ry / n, z = rz / n;
    constexpr double pi = 3.14159265358979323846;
    constexpr double c0 = 0.5 * cgmath::csqrt(1.0 / pi);
    double o[D];
    o[0] = c0;
    if constexpr (L >= 1) {
        constexpr double c1 = cgmath::csqrt(3.0 / (4.0 * pi));
        o[1] = c1 * y;
        o[2] = c1 * z;
        o[3] = c1 * x;
    }
    if constexpr (L >= 2) {
        constexpr double a = 0.5 * cgmath::csqrt(15.0 / pi);
        constexpr double b = 0.25 * cgmath::csqrt(5.0 / pi);
        constexpr double c = 0.25 * cgmath::csqrt(15.0 / pi);
        o[4] = a * x * y;
        o[5] = a * y * z;
        o[6] = b * (3.0 * z * z - 1.0);
        o[7] = a * x * z;
        o[8] = c * (x * x - y * y);
    }
    if constexpr (L >= 3) {
        constexpr double a = 0.25 * cgmath::csqrt(35.0 / (2.0 * pi));
        constexpr double b = 0.5 * cgmath::csqrt(105.0 / pi);
        constexpr double c = 0.25 * cgmath::csqrt(21.0 / (2.0 * pi));
        constexpr double d = 0.25 * cgmath::csqrt(7.0 / pi);
        constexpr double f = 0.25 * cgmath::csqrt(105.0 / pi);
        o[9] = a * y * (3.0 * x * x - y * y);
        o[10] = b * x * y * z;
        o[11] = c * y * (5.0 * z * z - 1.0);
        o[12] = d * (5.0 * z * z * z - 3.0 * z);
        o[13] = c * x * (5.0 * z * z - 1.0);
        o[14] = f * z * (x * x - y * y);
        o[15] = a * x * (x * x - 3.0 * y * y);
    }
    float* out = Y + e * D;
#pragma unroll
    for (int k = 0; k < D; ++k) out[k] = (float)o[k];
}

template <int L>
hipError_t launch_sh(int64_t E, const float* r, float* Y, hipStream_t s)
{
    if (E == 0) return hipSuccess;
    const int64_t blocks = (E + 255) / 256;
    hipLaunchKernelGGL(k_sh<L>, dim3((unsigned)blocks), dim3(256), 0, s, E, r, Y);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// lane geometry
// ----------------------------------------------------------------------------
template <int C>
struct Geo {
    static constexpr int LPE = C < 64 ? C : 64;  // lanes per edge (one channel each)
    static constexpr int EPW = 64 / LPE;         // edges a wave processes at once
    static constexpr int WPN = C > 64 ? C / 64 : 1;  // waves per node
    static_assert(C > 0 && (C & (C - 1)) == 0 && C <= 256, "C must be a power of two <= 256");
};

// minimum waves per SIMD the register allocation must allow
#ifndef CGTP_BWD_OCC
#define CGTP_BWD_OCC 2
#endif
#ifndef CGTP_FWD_OCC
#define CGTP_FWD_OCC 4
#endif
// software prefetch of the next edge's operands (1) or not (0)
#ifndef CGTP_BWD_PREFETCH
#define CGTP_BWD_PREFETCH 0
#endif
#ifndef CGTP_FWD_PREFETCH
#define CGTP_FWD_PREFETCH 1
#endif

// ----------------------------------------------------------------------------
// forward
// ----------------------------------------------------------------------------
template <class Tb>
struct FwdEdge {
    static constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH, DOUT = Tb::DOUT;
    float w[P], x[DIN], y[DSH];
};

template <class Tb, int C>
__device__ __forceinline__ void fwd_load(FwdEdge<Tb>& d, int32_t e, int c, const int32_t* __restrict__ src,
                                         const float* __restrict__ x, const float* __restrict__ Y,
                                         const float* __restrict__ W)
{
    constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH;
    const int32_t j = src[e];
    const float* wp = W + (int64_t)e * (P * C) + c;
#pragma unroll
    for (int p = 0; p < P; ++p) d.w[p] = __builtin_nontemporal_load(wp + p * C);
    const float* xp = x + (int64_t)j * (DIN * C) + c;
#pragma unroll
    for (int k = 0; k < DIN; ++k) d.x[k] = xp[k * C];
    const float* yp = Y + (int64_t)e * DSH;
#pragma unroll
    for (int k = 0; k < DSH; ++k) d.y[k] = yp[k];
}

// acc[l3,m3] += sum_p W_p sum_{a,b} T_p[a][b][m3] x[l1,a] y[l2,b]
template <class Tb>
__device__ __forceinline__ void fwd_compute(const FwdEdge<Tb>& d, double (&acc)[Tb::DOUT])
{
    constexpr int DIN = Tb::DIN, DSH = Tb::DSH;
    double xv[DIN], yv[DSH];
#pragma unroll
    for (int k = 0; k < DIN; ++k) xv[k] = (double)d.x[k];
#pragma unroll
    for (int k = 0; k < DSH; ++k) yv[k] = (double)d.y[k];
    static_for<0, Tb::P>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        using K = PathK<Tb, p>;
        // first path of its (l1,l2) block forms the products for the block
        constexpr bool first = (p == 0) || Tb::data.l1[p > 0 ? p - 1 : 0] != K::l1 ||
                               Tb::data.l2[p > 0 ? p - 1 : 0] != K::l2;
        (void)first;
        const double w = (double)d.w[p];
        static_for<0, K::d3>([&](auto M3) {
            constexpr int m3 = decltype(M3)::value;
            double z = 0.0;
            bool any = false;
            static_for<0, K::d1>([&](auto A) {
                static_for<0, K::d2>([&](auto B) {
                    constexpr int a = decltype(A)::value, b = decltype(B)::value;
                    constexpr double t = K::T(a, b, m3);
                    if constexpr (t != 0.0) {
                        z = __builtin_fma(t, xv[K::k1 + a] * yv[K::k2 + b], z);
                        any = true;
                    }
                });
            });
            if (any) acc[K::k3 + m3] = __builtin_fma(w, z, acc[K::k3 + m3]);
        });
    });
}

template <int LIN, int LSH, int LOUT, int C>
__global__ void __launch_bounds__(256, CGTP_FWD_OCC) k_conv_fwd(int32_t N, const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ src, const float* __restrict__ x,
                                                   const float* __restrict__ Y, const float* __restrict__ W,
                                                   float* __restrict__ out)
{
    using Tb = cgmath::Tables<LIN, LSH, LOUT>;
    using G = Geo<C>;
    constexpr int DOUT = Tb::DOUT;
    const int lane = threadIdx.x & 63;
    // wave index made explicitly uniform so the node, its segment and the
    // per-edge indices live in scalar registers
    const int32_t gw = (int32_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int32_t i = gw / G::WPN;
    if (i >= N) return;
    const int g = lane / G::LPE;
    const int c = (gw % G::WPN) * 64 + lane % G::LPE;

    double acc[DOUT];
#pragma unroll
    for (int k = 0; k < DOUT; ++k) acc[k] = 0.0;

    const int32_t end = row_ptr[i + 1];
    int32_t e = row_ptr[i] + g;
    FwdEdge<Tb> cur;
    if (CGTP_FWD_PREFETCH && e < end) fwd_load<Tb, C>(cur, e, c, src, x, Y, W);
    while (e < end) {
        const int32_t en = e + G::EPW;
        FwdEdge<Tb> nxt;
        if (CGTP_FWD_PREFETCH) {
            if (en < end) fwd_load<Tb, C>(nxt, en, c, src, x, Y, W);
        } else {
            fwd_load<Tb, C>(cur, e, c, src, x, Y, W);
        }
        fwd_compute<Tb>(cur, acc);
        if (CGTP_FWD_PREFETCH) cur = nxt;
        e = en;
    }
    if constexpr (G::EPW > 1) {
#pragma unroll
        for (int off = G::LPE; off < 64; off <<= 1)
#pragma unroll
            for (int k = 0; k < DOUT; ++k) acc[k] += __shfl_xor(acc[k], off, 64);
    }
    if (g == 0) {
        float* op = out + (int64_t)i * (DOUT * C) + c;
#pragma unroll
        for (int k = 0; k < DOUT; ++k) op[k * C] = (float)acc[k];
    }
}

template <int LIN, int LSH, int LOUT, int C>
hipError_t launch_fwd(int32_t N, const int32_t* row_ptr, const int32_t* src, const float* x, const float* Y,
                      const float* W, float* out, hipStream_t s)
{
    if (N == 0) return hipSuccess;
    const int64_t waves = (int64_t)N * Geo<C>::WPN;
    hipLaunchKernelGGL((k_conv_fwd<LIN, LSH, LOUT, C>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, N,
                       row_ptr, src, x, Y, W, out);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// backward
// ----------------------------------------------------------------------------
template <class Tb>
struct BwdEdge {
    static constexpr int P = Tb::P, DSH = Tb::DSH, DOUT = Tb::DOUT;
    int32_t e;
    float w[P], g[DOUT], y[DSH];
};

template <class Tb, int C>
__device__ __forceinline__ void bwd_load(BwdEdge<Tb>& d, int32_t q, int c, const GraphView& gv,
                                         const float* __restrict__ Y, const float* __restrict__ W,
                                         const float* __restrict__ Gr)
{
    constexpr int P = Tb::P, DSH = Tb::DSH, DOUT = Tb::DOUT;
    const int32_t e = gv.perm[q];
    const int32_t i = gv.sdst[q];
    d.e = e;
    const float* wp = W + (int64_t)e * (P * C) + c;
#pragma unroll
    for (int p = 0; p < P; ++p) d.w[p] = __builtin_nontemporal_load(wp + p * C);
    const float* gp = Gr + (int64_t)i * (DOUT * C) + c;
#pragma unroll
    for (int k = 0; k < DOUT; ++k) d.g[k] = gp[k * C];
    const float* yp = Y + (int64_t)e * DSH;
#pragma unroll
    for (int k = 0; k < DSH; ++k) d.y[k] = yp[k];
}

// One edge of the backward for this lane's channel:
//   R_p[a][b] = sum_m3 T_p[a][b][m3] g[l3,m3]
//   h_p[a] = sum_b R_p[a][b] y[l2,b]   -> dx[l1,a] += W_p h_p[a], dW_p = sum_a x[l1,a] h_p[a]
//   v_p[b] = sum_a R_p[a][b] x[l1,a]   -> dy[l2,b] += W_p v_p[b]
// Hide a register value from the optimiser: values passed through here before
// each path cannot be matched with the previous path's, so products of
// coefficients and components are not shared across paths and kept live for
// the whole edge (which costs more registers than recomputing them).
__device__ __forceinline__ void opaque(double& v) { asm volatile("" : "+v"(v)); }

template <class Tb, int C, bool DX, bool DW, bool DY>
__device__ __forceinline__ void bwd_compute(const BwdEdge<Tb>& d, const double (&xv)[Tb::DIN],
                                            double (&dxa)[Tb::DIN], float* __restrict__ dwp,
                                            double (&dya)[Tb::DSH])
{
    constexpr int DSH = Tb::DSH, DOUT = Tb::DOUT;
    double gv[DOUT], yv[DSH];
#pragma unroll
    for (int k = 0; k < DOUT; ++k) gv[k] = (double)d.g[k];
#pragma unroll
    for (int k = 0; k < DSH; ++k) yv[k] = (double)d.y[k];
#pragma unroll
    for (int k = 0; k < DSH; ++k) dya[k] = 0.0;
    static_for<0, Tb::P>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        using K = PathK<Tb, p>;
        const double w = (double)d.w[p];
        static_for<0, K::d3>([&](auto M3) { opaque(gv[K::k3 + decltype(M3)::value]); });
        double v[K::d2];
        static_for<0, K::d2>([&](auto B) { v[decltype(B)::value] = 0.0; });
        double dw = 0.0;
        static_for<0, K::d1>([&](auto A) {
            constexpr int a = decltype(A)::value;
            if constexpr (K::ROW(a)) {
                double h = 0.0;
                static_for<0, K::d2>([&](auto B) {
                    constexpr int b = decltype(B)::value;
                    // R[a][b]
                    double r = 0.0;
                    bool any = false;
                    static_for<0, K::d3>([&](auto M3) {
                        constexpr int m3 = decltype(M3)::value;
                        constexpr double t = K::T(a, b, m3);
                        if constexpr (t != 0.0) {
                            r = __builtin_fma(t, gv[K::k3 + m3], r);
                            any = true;
                        }
                    });
                    if (any) {
                        h = __builtin_fma(r, yv[K::k2 + b], h);
                        if constexpr (DY) v[b] = __builtin_fma(r, xv[K::k1 + a], v[b]);
                    }
                });
                if constexpr (DX) dxa[K::k1 + a] = __builtin_fma(w, h, dxa[K::k1 + a]);
                if constexpr (DW) dw = __builtin_fma(xv[K::k1 + a], h, dw);
            }
        });
        if constexpr (DW) __builtin_nontemporal_store((float)dw, dwp + p * C);
        if constexpr (DY)
            static_for<0, K::d2>([&](auto B) {
                constexpr int b = decltype(B)::value;
                if constexpr (K::COL2(b)) dya[K::k2 + b] = __builtin_fma(w, v[b], dya[K::k2 + b]);
            });
        // schedule path by path: interleaving paths buys little ILP at this
        // occupancy and multiplies the live transients
        __builtin_amdgcn_sched_barrier(0);
    });
}

// grad_Y slots combined across the waves of a sender (C > 64), in LDS
constexpr int kDyBatch = 32;

// quad_perm DPP move of a double (both halves), CTRL a quad_perm selector
template <int CTRL>
__device__ __forceinline__ double dpp_quad(double v)
{
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

// Sum of v[k] over the 64 lanes of a wave, for every k < D (D <= 16), through
// a per-wave LDS tile red[D][64]: each lane stores its D partials, lane 4k+q
// adds red[k][16q .. 16q+15], and a quad exchange (DPP) completes the sum.
// Returns the total of component lane/4 in lanes with lane%4 == 0.
template <int D>
__device__ __forceinline__ double wave_sum_lds(const double (&v)[D], double* __restrict__ red, int lane)
{
    static_assert(D <= 16, "at most 16 components");
#pragma unroll
    for (int k = 0; k < D; ++k) red[k * 64 + lane] = v[k];
    __builtin_amdgcn_wave_barrier();
    const int k = lane >> 2, q = lane & 3;
    double s = 0.0;
    if (k < D) {
        const double2* r = reinterpret_cast<const double2*>(red + k * 64 + q * 16);
        double2 acc2[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) acc2[t] = r[t];
#pragma unroll
        for (int t = 0; t < 8; ++t) s += acc2[t].x + acc2[t].y;
    }
    __builtin_amdgcn_wave_barrier();
    s += dpp_quad<0xB1>(s);  // lanes ^1
    s += dpp_quad<0x4E>(s);  // lanes ^2
    return s;
}

template <int LIN, int LSH, int LOUT, int C, bool DX, bool DW, bool DY>
__global__ void __launch_bounds__(256, CGTP_BWD_OCC) k_conv_bwd(int32_t N, GraphView gv, const float* __restrict__ x,
                                                   const float* __restrict__ Y, const float* __restrict__ W,
                                                   const float* __restrict__ Gr, float* __restrict__ dx,
                                                   float* __restrict__ dW, float* __restrict__ dY)
{
    using Tb = cgmath::Tables<LIN, LSH, LOUT>;
    using Gm = Geo<C>;
    constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH;
    constexpr int WPN = Gm::WPN;
    constexpr int NPB = WPN > 1 ? 1 : 4;  // senders per block
    // per-wave grad_Y partial sums of a batch of edges (only when WPN > 1)
    __shared__ double dy_part[WPN > 1 ? WPN : 1][WPN > 1 ? kDyBatch : 1][DSH];
    __shared__ int32_t dy_edge[WPN > 1 ? kDyBatch : 1];
    // per-wave transpose tile of the channel reduction (one channel per lane)
    constexpr bool kLdsSum = DY && Gm::LPE == 64;
    __shared__ double dy_red[kLdsSum ? (WPN > 1 ? WPN : 4) : 1][kLdsSum ? DSH * 64 : 1];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int32_t j = (int32_t)blockIdx.x * NPB + (WPN > 1 ? 0 : wv);
    if (WPN == 1 && j >= N) return;  // whole wave; no block barrier when WPN == 1
    const int half = WPN > 1 ? wv : 0;
    const int g = lane / Gm::LPE;
    const int c = half * 64 + lane % Gm::LPE;

    double xv[DIN], dxa[DIN];
    {
        const float* xp = x + (int64_t)j * (DIN * C) + c;
#pragma unroll
        for (int k = 0; k < DIN; ++k) {
            xv[k] = (double)xp[k * C];
            dxa[k] = 0.0;
        }
    }
    const int32_t beg = gv.srow[j], end = gv.srow[j + 1];

    if constexpr (WPN == 1) {
        int32_t q = beg + g;
        BwdEdge<Tb> cur;
        if (CGTP_BWD_PREFETCH && q < end) bwd_load<Tb, C>(cur, q, c, gv, Y, W, Gr);
        while (q < end) {
            const int32_t qn = q + Gm::EPW;
            BwdEdge<Tb> nxt;
            if (CGTP_BWD_PREFETCH) {
                if (qn < end) bwd_load<Tb, C>(nxt, qn, c, gv, Y, W, Gr);
            } else {
                bwd_load<Tb, C>(cur, q, c, gv, Y, W, Gr);
            }
            double dya[DSH];
            bwd_compute<Tb, C, DX, DW, DY>(cur, xv, dxa, dW + (int64_t)cur.e * (P * C) + c, dya);
            if constexpr (DY) {
                if constexpr (kLdsSum) {
                    const double t = wave_sum_lds<DSH>(dya, dy_red[wv], lane);
                    if ((lane & 3) == 0 && (lane >> 2) < DSH) dY[(int64_t)cur.e * DSH + (lane >> 2)] = (float)t;
                } else {
#pragma unroll
                    for (int k = 0; k < DSH; ++k) {
                        double s = dya[k];
#pragma unroll
                        for (int off = 1; off < Gm::LPE; off <<= 1) s += __shfl_xor(s, off, 64);
                        dya[k] = s;
                    }
                    if ((lane % Gm::LPE) == 0) {
                        float* yp = dY + (int64_t)cur.e * DSH;
#pragma unroll
                        for (int k = 0; k < DSH; ++k) yp[k] = (float)dya[k];
                    }
                }
            }
            if (CGTP_BWD_PREFETCH) cur = nxt;
            q = qn;
        }
    } else {
        // WPN waves share the sender; the segment is walked in batches so the
        // per-wave grad_Y partials can be combined in LDS
        const int32_t n = end - beg;
        for (int32_t b0 = 0; b0 < n; b0 += kDyBatch) {
            const int32_t nb = n - b0 < kDyBatch ? n - b0 : kDyBatch;
            int32_t q = beg + b0;
            const int32_t qe = q + nb;
            BwdEdge<Tb> cur;
            if (CGTP_BWD_PREFETCH) bwd_load<Tb, C>(cur, q, c, gv, Y, W, Gr);
            for (int32_t s = 0; s < nb; ++s) {
                BwdEdge<Tb> nxt;
                if (CGTP_BWD_PREFETCH) {
                    if (q + 1 < qe) bwd_load<Tb, C>(nxt, q + 1, c, gv, Y, W, Gr);
                } else {
                    bwd_load<Tb, C>(cur, q, c, gv, Y, W, Gr);
                }
                double dya[DSH];
                bwd_compute<Tb, C, DX, DW, DY>(cur, xv, dxa, dW + (int64_t)cur.e * (P * C) + c, dya);
                if constexpr (DY) {
                    const double t = wave_sum_lds<DSH>(dya, dy_red[wv], lane);
                    if ((lane & 3) == 0 && (lane >> 2) < DSH) dy_part[half][s][lane >> 2] = t;
                    if (lane == 0 && half == 0) dy_edge[s] = cur.e;
                }
                if (CGTP_BWD_PREFETCH) cur = nxt;
                ++q;
            }
            if constexpr (DY) {
                __syncthreads();
                for (int t = threadIdx.x; t < nb * DSH; t += 64 * WPN) {
                    const int s = t / DSH, k = t % DSH;
                    double v = 0.0;
#pragma unroll
                    for (int h = 0; h < WPN; ++h) v += dy_part[h][s][k];
                    dY[(int64_t)dy_edge[s] * DSH + k] = (float)v;
                }
                __syncthreads();
            }
        }
    }
    if constexpr (DX) {
        if constexpr (Gm::EPW > 1) {
#pragma unroll
            for (int off = Gm::LPE; off < 64; off <<= 1)
#pragma unroll
                for (int k = 0; k < DIN; ++k) dxa[k] += __shfl_xor(dxa[k], off, 64);
        }
        if (g == 0) {
            float* dp = dx + (int64_t)j * (DIN * C) + c;
#pragma unroll
            for (int k = 0; k < DIN; ++k) dp[k * C] = (float)dxa[k];
        }
    }
}

template <int LIN, int LSH, int LOUT, int C, bool DX, bool DW, bool DY>
hipError_t launch_bwd_t(int32_t N, GraphView g, const float* x, const float* Y, const float* W, const float* G,
                        float* dx, float* dW, float* dY, hipStream_t s)
{
    using Gm = Geo<C>;
    const unsigned blocks = Gm::WPN > 1 ? (unsigned)N : (unsigned)((N + 3) / 4);
    const unsigned threads = Gm::WPN > 1 ? 64u * Gm::WPN : 256u;
    hipLaunchKernelGGL((k_conv_bwd<LIN, LSH, LOUT, C, DX, DW, DY>), dim3(blocks), dim3(threads), 0, s, N, g, x, Y,
                       W, G, dx, dW, dY);
    return hipGetLastError();
}

template <int LIN, int LSH, int LOUT, int C>
hipError_t launch_bwd(int32_t N, GraphView g, const float* x, const float* Y, const float* W, const float* G,
                      float* dx, float* dW, float* dY, int mask, hipStream_t s)
{
    if (N == 0) return hipSuccess;
    switch (mask) {
        case 1: return launch_bwd_t<LIN, LSH, LOUT, C, true, false, false>(N, g, x, Y, W, G, dx, dW, dY, s);
        case 2: return launch_bwd_t<LIN, LSH, LOUT, C, false, true, false>(N, g, x, Y, W, G, dx, dW, dY, s);
        case 3: return launch_bwd_t<LIN, LSH, LOUT, C, true, true, false>(N, g, x, Y, W, G, dx, dW, dY, s);
        case 4: return launch_bwd_t<LIN, LSH, LOUT, C, false, false, true>(N, g, x, Y, W, G, dx, dW, dY, s);
        case 5: return launch_bwd_t<LIN, LSH, LOUT, C, true, false, true>(N, g, x, Y, W, G, dx, dW, dY, s);
        case 6: return launch_bwd_t<LIN, LSH, LOUT, C, false, true, true>(N, g, x, Y, W, G, dx, dW, dY, s);
        case 7: return launch_bwd_t<LIN, LSH, LOUT, C, true, true, true>(N, g, x, Y, W, G, dx, dW, dY, s);
        default: return hipSuccess;
    }
}

template <int L, int C>
constexpr KernelSet make_set()
{
    return KernelSet{L, L, L, C, &launch_sh<L>, &launch_fwd<L, L, L, C>, &launch_bwd<L, L, L, C>};
}

template <int LIN, int LSH, int LOUT>
static bool copy_table(int path, double* dense)
{
    using Tb = cgmath::Tables<LIN, LSH, LOUT>;
    if (path < 0 || path >= Tb::P) return false;
    const int n = cgmath::path_size(cgmath::path_at(LIN, LSH, LOUT, path));
    for (int q = 0; q < n; ++q) dense[q] = Tb::data.T[Tb::data.off[path] + q];
    return true;
}

}  // namespace cgtp
