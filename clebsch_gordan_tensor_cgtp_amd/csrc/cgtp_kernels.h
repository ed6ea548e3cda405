// cgtp_kernels.h -- gfx950 kernels of the CGTP convolution (templates; each
// cgtp_kernels_l<L>.hip instantiates one degree).
//
// Hot path (the convolution LunaTP's abstract calls the cost centre of
// equivariant MLIPs; "LunaTP: Enabling Efficient and Scalable Tensor Product
// for Equivariant MLIPs", Abstract):
//   * real spherical harmonics of the edge vectors          (k_sh)
//   * sender-sorted view of the receiver CSR                (graph prep)
//   * forward, node-centric: one wavefront owns a receiver, walks its CSR
//     segment, gathers the sender rows x_j with channel-contiguous loads,
//     streams W[e], accumulates in registers and writes out[i] once; no
//     atomics                                               (k_conv_fwd)
//   * backward, sender-centric over the sender-sorted view: one wavefront owns
//     a sender j, keeps x_j and grad_x[j] in registers, gathers grad_out rows
//     of the receivers, writes grad_W[e] and a cross-lane-reduced grad_Y[e]
//     per edge; no atomics                                  (k_conv_bwd)
//
// Arithmetic is fp64 on fp32 data: the per-edge contraction and the sums over
// a segment and over channels keep fp64 accuracy, and fp64 FMA issues at the
// same rate as unpacked fp32 on this chip.
//
// Within an edge, the CG contraction is reused across channels: for each path
// p = (l1,l2,l3) the matrix M_p[m1][m3] = sum_m2 T_p[m1][m2][m3] Y[e][l2,m2]
// depends only on the edge, so it is formed once per edge (per lane, shared by
// the lane's channels) and each channel then needs M_p x (forward) or M_p g
// (backward).  The CG values and their nonzero pattern are compile-time
// constants of the (L_in, L_sh, L_out) specialisation.
//
// Lane mapping: a lane owns CPL adjacent channels of one edge; LPE = C/CPL
// lanes cover an edge, so a wave processes 64/LPE edges of its segment at once
// and reduces across those edge groups at the end.
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
// channel I/O helpers: CPL adjacent fp32 channels
// ----------------------------------------------------------------------------
template <int CPL>
__device__ __forceinline__ void load_ch(const float* __restrict__ p, float (&v)[CPL])
{
    if constexpr (CPL == 2) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        v[0] = t.x;
        v[1] = t.y;
    } else if constexpr (CPL == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        v[0] = t.x;
        v[1] = t.y;
        v[2] = t.z;
        v[3] = t.w;
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = p[c];
    }
}

template <int CPL>
__device__ __forceinline__ void store_ch(float* __restrict__ p, const double (&v)[CPL])
{
    if constexpr (CPL == 2) {
        *reinterpret_cast<float2*>(p) = make_float2((float)v[0], (float)v[1]);
    } else if constexpr (CPL == 4) {
        *reinterpret_cast<float4*>(p) = make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) p[c] = (float)v[c];
    }
}

// ----------------------------------------------------------------------------
// forward
// ----------------------------------------------------------------------------
template <int LIN, int LSH, int LOUT, int CPL, int LPE>
__global__ void __launch_bounds__(256) k_conv_fwd(int32_t N, const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ src, const float* __restrict__ x,
                                                   const float* __restrict__ Y, const float* __restrict__ W,
                                                   float* __restrict__ out)
{
    using Tb = cgmath::Tables<LIN, LSH, LOUT>;
    constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH, DOUT = Tb::DOUT;
    constexpr int C = CPL * LPE;
    constexpr int EPW = 64 / LPE;  // edges in flight per wave
    const int lane = threadIdx.x & 63;
    const int32_t i = (int32_t)blockIdx.x * 4 + (int32_t)(threadIdx.x >> 6);
    if (i >= N) return;
    const int g = lane / LPE;
    const int c0 = (lane % LPE) * CPL;

    double acc[DOUT][CPL];
#pragma unroll
    for (int k = 0; k < DOUT; ++k)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[k][c] = 0.0;

    const int32_t beg = row_ptr[i], end = row_ptr[i + 1];
    for (int32_t e = beg + g; e < end; e += EPW) {
        const int32_t j = src[e];
        double y[DSH];
#pragma unroll
        for (int k = 0; k < DSH; ++k) y[k] = (double)Y[(int64_t)e * DSH + k];
        float wv[P][CPL];
        const float* wp = W + (int64_t)e * (P * C) + c0;
#pragma unroll
        for (int p = 0; p < P; ++p) load_ch<CPL>(wp + p * C, wv[p]);
        float xf[DIN][CPL];
        const float* xp = x + (int64_t)j * (DIN * C) + c0;
#pragma unroll
        for (int k = 0; k < DIN; ++k) load_ch<CPL>(xp + k * C, xf[k]);
        double xv[DIN][CPL];
#pragma unroll
        for (int k = 0; k < DIN; ++k)
#pragma unroll
            for (int c = 0; c < CPL; ++c) xv[k][c] = (double)xf[k][c];

        static_for<0, P>([&](auto PI) {
            using K = PathK<Tb, decltype(PI)::value>;
            constexpr int p = decltype(PI)::value;
            double M[K::d1][K::d3];
            make_M<K>(y, M);
            static_for<0, CPL>([&](auto CI) {
                constexpr int c = decltype(CI)::value;
                const double w = (double)wv[p][c];
                static_for<0, K::d3>([&](auto M3) {
                    constexpr int m3 = decltype(M3)::value;
                    double z = 0.0;
                    bool any = false;
                    static_for<0, K::d1>([&](auto A) {
                        constexpr int a = decltype(A)::value;
                        if constexpr (K::NZ(a, m3)) {
                            z = __builtin_fma(M[a][m3], xv[K::k1 + a][c], z);
                            any = true;
                        }
                    });
                    if (any) acc[K::k3 + m3][c] = __builtin_fma(w, z, acc[K::k3 + m3][c]);
                });
            });
        });
    }
    if constexpr (EPW > 1) {
#pragma unroll
        for (int off = LPE; off < 64; off <<= 1)
#pragma unroll
            for (int k = 0; k < DOUT; ++k)
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[k][c] += __shfl_xor(acc[k][c], off, 64);
    }
    if (g == 0) {
        float* op = out + (int64_t)i * (DOUT * C) + c0;
#pragma unroll
        for (int k = 0; k < DOUT; ++k) store_ch<CPL>(op + k * C, acc[k]);
    }
}

template <int LIN, int LSH, int LOUT, int CPL, int LPE>
hipError_t launch_fwd(int32_t N, const int32_t* row_ptr, const int32_t* src, const float* x, const float* Y,
                      const float* W, float* out, hipStream_t s)
{
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL((k_conv_fwd<LIN, LSH, LOUT, CPL, LPE>), dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, N,
                       row_ptr, src, x, Y, W, out);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// backward
// ----------------------------------------------------------------------------
template <int LIN, int LSH, int LOUT, int CPL, int LPE>
__global__ void __launch_bounds__(256) k_conv_bwd(int32_t N, GraphView gv, const float* __restrict__ x,
                                                   const float* __restrict__ Y, const float* __restrict__ W,
                                                   const float* __restrict__ G, float* __restrict__ dx,
                                                   float* __restrict__ dW, float* __restrict__ dY, int mask)
{
    using Tb = cgmath::Tables<LIN, LSH, LOUT>;
    constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH, DOUT = Tb::DOUT;
    constexpr int C = CPL * LPE;
    constexpr int EPW = 64 / LPE;
    const int lane = threadIdx.x & 63;
    const int32_t j = (int32_t)blockIdx.x * 4 + (int32_t)(threadIdx.x >> 6);
    if (j >= N) return;
    const int g = lane / LPE;
    const int c0 = (lane % LPE) * CPL;
    const bool want_dx = (mask & kGradX) != 0;
    const bool want_dW = (mask & kGradW) != 0;
    const bool want_dY = (mask & kGradY) != 0;

    double xv[DIN][CPL];
    {
        float xf[DIN][CPL];
        const float* xp = x + (int64_t)j * (DIN * C) + c0;
#pragma unroll
        for (int k = 0; k < DIN; ++k) load_ch<CPL>(xp + k * C, xf[k]);
#pragma unroll
        for (int k = 0; k < DIN; ++k)
#pragma unroll
            for (int c = 0; c < CPL; ++c) xv[k][c] = (double)xf[k][c];
    }
    double dxa[DIN][CPL];
#pragma unroll
    for (int k = 0; k < DIN; ++k)
#pragma unroll
        for (int c = 0; c < CPL; ++c) dxa[k][c] = 0.0;

    const int32_t beg = gv.srow[j], end = gv.srow[j + 1];
    for (int32_t q = beg + g; q < end; q += EPW) {
        const int32_t e = gv.perm[q];
        const int32_t i = gv.sdst[q];
        double y[DSH];
#pragma unroll
        for (int k = 0; k < DSH; ++k) y[k] = (double)Y[(int64_t)e * DSH + k];
        float wv[P][CPL];
        const float* wp = W + (int64_t)e * (P * C) + c0;
#pragma unroll
        for (int p = 0; p < P; ++p) load_ch<CPL>(wp + p * C, wv[p]);
        double gg[DOUT][CPL];
        {
            float gf[DOUT][CPL];
            const float* gp = G + (int64_t)i * (DOUT * C) + c0;
#pragma unroll
            for (int k = 0; k < DOUT; ++k) load_ch<CPL>(gp + k * C, gf[k]);
#pragma unroll
            for (int k = 0; k < DOUT; ++k)
#pragma unroll
                for (int c = 0; c < CPL; ++c) gg[k][c] = (double)gf[k][c];
        }
        double dya[DSH];
#pragma unroll
        for (int k = 0; k < DSH; ++k) dya[k] = 0.0;
        float* dwp = dW + (int64_t)e * (P * C) + c0;

        static_for<0, P>([&](auto PI) {
            using K = PathK<Tb, decltype(PI)::value>;
            constexpr int p = decltype(PI)::value;
            double M[K::d1][K::d3];
            make_M<K>(y, M);
            double dwc[CPL];
            static_for<0, CPL>([&](auto CI) {
                constexpr int c = decltype(CI)::value;
                const double w = (double)wv[p][c];
                // h[a] = sum_m3 M[a][m3] g[m3]
                double h[K::d1];
                double dw = 0.0;
                static_for<0, K::d1>([&](auto A) {
                    constexpr int a = decltype(A)::value;
                    if constexpr (K::ROW(a)) {
                        double s = 0.0;
                        static_for<0, K::d3>([&](auto M3) {
                            constexpr int m3 = decltype(M3)::value;
                            if constexpr (K::NZ(a, m3)) s = __builtin_fma(M[a][m3], gg[K::k3 + m3][c], s);
                        });
                        h[a] = s;
                        dw = __builtin_fma(xv[K::k1 + a][c], s, dw);
                        if (want_dx) dxa[K::k1 + a][c] = __builtin_fma(w, s, dxa[K::k1 + a][c]);
                    }
                });
                dwc[c] = dw;
                if (want_dY) {
                    // v[b] = sum_{a,m3} T[a][b][m3] x[a] g[m3]; dY[b] += w v[b]
                    double v[K::d2];
                    static_for<0, K::d2>([&](auto B) { v[decltype(B)::value] = 0.0; });
                    static_for<0, K::d1>([&](auto A) {
                        static_for<0, K::d3>([&](auto M3) {
                            constexpr int a = decltype(A)::value, m3 = decltype(M3)::value;
                            if constexpr (K::NZ(a, m3)) {
                                const double pr = xv[K::k1 + a][c] * gg[K::k3 + m3][c];
                                static_for<0, K::d2>([&](auto B) {
                                    constexpr int b = decltype(B)::value;
                                    constexpr double t = K::T(a, b, m3);
                                    if constexpr (t != 0.0) v[b] = __builtin_fma(t, pr, v[b]);
                                });
                            }
                        });
                    });
                    static_for<0, K::d2>([&](auto B) {
                        constexpr int b = decltype(B)::value;
                        if constexpr (K::COL2(b)) dya[K::k2 + b] = __builtin_fma(w, v[b], dya[K::k2 + b]);
                    });
                }
            });
            if (want_dW) store_ch<CPL>(dwp + p * C, dwc);
        });

        if (want_dY) {
#pragma unroll
            for (int k = 0; k < DSH; ++k) {
                double v = dya[k];
#pragma unroll
                for (int off = 1; off < LPE; off <<= 1) v += __shfl_xor(v, off, 64);
                dya[k] = v;
            }
            if ((lane % LPE) == 0) {
                float* yp = dY + (int64_t)e * DSH;
#pragma unroll
                for (int k = 0; k < DSH; ++k) yp[k] = (float)dya[k];
            }
        }
    }
    if (want_dx) {
        if constexpr (EPW > 1) {
#pragma unroll
            for (int off = LPE; off < 64; off <<= 1)
#pragma unroll
                for (int k = 0; k < DIN; ++k)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) dxa[k][c] += __shfl_xor(dxa[k][c], off, 64);
        }
        if (g == 0) {
            float* dp = dx + (int64_t)j * (DIN * C) + c0;
#pragma unroll
            for (int k = 0; k < DIN; ++k) store_ch<CPL>(dp + k * C, dxa[k]);
        }
    }
}

template <int LIN, int LSH, int LOUT, int CPL, int LPE>
hipError_t launch_bwd(int32_t N, GraphView g, const float* x, const float* Y, const float* W, const float* G,
                      float* dx, float* dW, float* dY, int mask, hipStream_t s)
{
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL((k_conv_bwd<LIN, LSH, LOUT, CPL, LPE>), dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, N,
                       g, x, Y, W, G, dx, dW, dY, mask);
    return hipGetLastError();
}


template <int L, int C, int CPL>
constexpr KernelSet make_set()
{
    return KernelSet{L, L, L, C, &launch_sh<L>, &launch_fwd<L, L, L, CPL, C / CPL>, &launch_bwd<L, L, L, CPL, C / CPL>};
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
