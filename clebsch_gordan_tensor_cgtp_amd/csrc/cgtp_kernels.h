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
// work decomposition
// ----------------------------------------------------------------------------
// One 256-thread block (four waves) per node.  A lane owns one channel of an
// edge: LPE = min(C, 64) lanes cover a 64-channel slice, and for C > 64 the
// H = C/64 slices of a node go to different waves, so every wave carries the
// state of a single slice (the register budget decides occupancy here).  The
// node's edges are interleaved over the block's S edge streams (stream s takes
// the node's edges s, s+S, s+2S, ...), which keeps a long segment from
// serialising on one wave; the streams' partial sums are combined in LDS in a
// fixed order at the end (atomic-free, deterministic).
template <int C>
struct Geo {
    static_assert(C > 0 && (C & (C - 1)) == 0 && C <= 256, "C must be a power of two <= 256");
    static constexpr int LPE = C < 64 ? C : 64;      // lanes per edge slice
    static constexpr int H = C / LPE;                // channel slices (waves) per edge
    static_assert(H <= 4, "at most four slices per block");
    static constexpr int S = (4 / H) * (64 / LPE);   // edge streams per block
};

// position of this thread: channel slice, channel within the slice, stream
template <int C>
struct Pos {
    int h, cl, s;
    __device__ __forceinline__ explicit Pos(int tid)
    {
        using G = Geo<C>;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        h = wave % G::H;
        cl = (tid & 63) % G::LPE;
        if constexpr (G::LPE == 64) s = wave / G::H;  // wave-uniform
        else s = (wave / G::H) * (64 / G::LPE) + (tid & 63) / G::LPE;
    }
    __device__ __forceinline__ int channel() const { return h * Geo<C>::LPE + cl; }
};

// Per-specialisation tuning: the minimum waves per SIMD the register
// allocation must allow, and whether the next edge's operands are loaded
// before the current edge is computed.  Chosen so that no specialisation
// spills vector registers (a spill costs far more than the occupancy it buys).
template <int L, int C>
struct Tune {
    static constexpr int fwd_occ = L <= 2 ? 4 : 2;
    static constexpr int bwd_occ = L == 1 || (L == 2 && C >= 64) ? 4 : (L == 2 ? 3 : 2);
    static constexpr bool fwd_prefetch = L <= 2;
    static constexpr bool bwd_prefetch = false;
};

// An empty asm that takes a register value and hands it back: the optimiser
// must materialise the value at that point and cannot match it with values
// computed before it.  Used to keep accumulations in path order (otherwise
// they are sunk to the end of the edge and every path's intermediates stay
// live) and to keep per-path products from being shared across paths.
__device__ __forceinline__ void opaque(double& v) { asm volatile("" : "+v"(v)); }

// fp64 value known to be equal in every lane, moved to a scalar register pair
__device__ __forceinline__ double uniform(double v)
{
    const int lo = __builtin_amdgcn_readfirstlane(__double2loint(v));
    const int hi = __builtin_amdgcn_readfirstlane(__double2hiint(v));
    return __hiloint2double(hi, lo);
}

// the edge's spherical harmonics in fp64; held in scalar registers when the
// whole wave works on one edge (they are then the same in every lane)
template <int DSH, int LPE>
__device__ __forceinline__ void edge_sh(const float (&y)[DSH], double (&yv)[DSH])
{
#pragma unroll
    for (int k = 0; k < DSH; ++k) {
        yv[k] = (double)y[k];
        if constexpr (LPE == 64) yv[k] = uniform(yv[k]);
    }
}

// ----------------------------------------------------------------------------
// forward
// ----------------------------------------------------------------------------
template <class Tb>
struct FwdEdge {
    static constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH;
    float w[P], x[DIN], y[DSH];
};

// operands of edge e for channel ch
template <class Tb, int C>
__device__ __forceinline__ void fwd_load(FwdEdge<Tb>& d, int32_t e, int ch, const int32_t* __restrict__ src,
                                         const float* __restrict__ x, const float* __restrict__ Y,
                                         const float* __restrict__ W)
{
    constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH;
    const int32_t j = src[e];
    const float* wp = W + (int64_t)e * (P * C) + ch;
#pragma unroll
    for (int p = 0; p < P; ++p) d.w[p] = __builtin_nontemporal_load(wp + p * C);
    const float* xp = x + (int64_t)j * (DIN * C) + ch;
#pragma unroll
    for (int k = 0; k < DIN; ++k) d.x[k] = xp[k * C];
    const float* yp = Y + (int64_t)e * DSH;
#pragma unroll
    for (int k = 0; k < DSH; ++k) d.y[k] = yp[k];
}

// acc[l3,m3] += sum_p W_p sum_{a,b} T_p[a][b][m3] x[l1,a] y[l2,b] for one channel
template <class Tb>
__device__ __forceinline__ void fwd_slice(const float (&w)[Tb::P], const float (&x)[Tb::DIN],
                                          const double (&yv)[Tb::DSH], double (&acc)[Tb::DOUT])
{
    double xv[Tb::DIN];
#pragma unroll
    for (int k = 0; k < Tb::DIN; ++k) xv[k] = (double)x[k];
    static_for<0, Tb::P>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        using K = PathK<Tb, p>;
        const double wd = (double)w[p];
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
            if (any) acc[K::k3 + m3] = __builtin_fma(wd, z, acc[K::k3 + m3]);
        });
        // keep the accumulation in path order (see opaque)
        static_for<0, K::d3>([&](auto M3) { opaque(acc[K::k3 + decltype(M3)::value]); });
    });
}

template <int LIN, int LSH, int LOUT, int C>
__global__ void __launch_bounds__(256, (Tune<LIN, C>::fwd_occ)) k_conv_fwd(int32_t N, const int32_t* __restrict__ row_ptr,
                                                                         const int32_t* __restrict__ src,
                                                                         const int32_t* __restrict__ rorder,
                                                                         const float* __restrict__ x,
                                                                         const float* __restrict__ Y,
                                                                         const float* __restrict__ W,
                                                                         float* __restrict__ out)
{
    using Tb = cgmath::Tables<LIN, LSH, LOUT>;
    using Gm = Geo<C>;
    constexpr int DSH = Tb::DSH, DOUT = Tb::DOUT, S = Gm::S;
    constexpr bool kPf = Tune<LIN, C>::fwd_prefetch;
    // LDS: the streams' partial sums [stream][k][channel]
    __shared__ double red[S * DOUT * C];

    const int tid = threadIdx.x;
    const Pos<C> ps(tid);
    const int ch = ps.channel();
    const int32_t i = rorder[blockIdx.x];
    if ((uint32_t)i >= (uint32_t)N) return;  // unprepared workspace: never index with it
    const int32_t end = row_ptr[i + 1];

    double acc[DOUT];
#pragma unroll
    for (int k = 0; k < DOUT; ++k) acc[k] = 0.0;

    // with prefetch, the stream's next edge is loaded before the current one
    // is computed (the copy `cur = nxt` costs fewer registers than
    // alternating two named buffers, which would spill at this occupancy)
    int32_t e = row_ptr[i] + ps.s;
    FwdEdge<Tb> cur;
    if (kPf && e < end) fwd_load<Tb, C>(cur, e, ch, src, x, Y, W);
    while (e < end) {
        const int32_t en = e + S;
        FwdEdge<Tb> nxt;
        if constexpr (kPf) {
            if (en < end) fwd_load<Tb, C>(nxt, en, ch, src, x, Y, W);
        } else {
            fwd_load<Tb, C>(cur, e, ch, src, x, Y, W);
        }
        double yv[DSH];
        edge_sh<DSH, Gm::LPE>(cur.y, yv);
        fwd_slice<Tb>(cur.w, cur.x, yv, acc);
        if constexpr (kPf) cur = nxt;
        e = en;
    }

    // combine the streams in a fixed order; out[i] has this block as its only writer
#pragma unroll
    for (int k = 0; k < DOUT; ++k) red[(ps.s * DOUT + k) * C + ch] = acc[k];
    __syncthreads();
    float* op = out + (int64_t)i * (DOUT * C);
    for (int t = tid; t < DOUT * C; t += 256) {
        double v = 0.0;
#pragma unroll
        for (int q = 0; q < S; ++q) v += red[q * DOUT * C + t];
        op[t] = (float)v;
    }
}

template <int LIN, int LSH, int LOUT, int C>
hipError_t launch_fwd(int32_t N, const int32_t* row_ptr, const int32_t* src, const int32_t* rorder, const float* x,
                      const float* Y, const float* W, float* out, hipStream_t s)
{
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL((k_conv_fwd<LIN, LSH, LOUT, C>), dim3((unsigned)N), dim3(256), 0, s, N, row_ptr, src, rorder,
                       x, Y, W, out);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// backward
// ----------------------------------------------------------------------------
template <class Tb>
struct BwdEdge {
    static constexpr int P = Tb::P, DSH = Tb::DSH, DOUT = Tb::DOUT;
    int32_t e;
    bool ok;  // the view entry names a valid edge and receiver
    float w[P], g[DOUT], y[DSH];
};

// operands of the q-th edge of the sender-sorted view for channel ch; a
// corrupt entry (possible only if the view was not prepared for this graph)
// is read as edge 0 / receiver 0 and flagged, never used out of bounds
template <class Tb, int C>
__device__ __forceinline__ void bwd_load(BwdEdge<Tb>& d, int32_t q, int ch, int32_t N, const GraphView& gv,
                                         const float* __restrict__ Y, const float* __restrict__ W,
                                         const float* __restrict__ Gr)
{
    constexpr int P = Tb::P, DSH = Tb::DSH, DOUT = Tb::DOUT;
    int32_t e = gv.perm[q];
    int32_t i = gv.sdst[q];
    d.ok = (uint32_t)e < (uint32_t)gv.n_edges && (uint32_t)i < (uint32_t)N;
    if (!d.ok) e = i = 0;
    d.e = e;
    const float* wp = W + (int64_t)e * (P * C) + ch;
#pragma unroll
    for (int p = 0; p < P; ++p) d.w[p] = __builtin_nontemporal_load(wp + p * C);
    const float* gp = Gr + (int64_t)i * (DOUT * C) + ch;
#pragma unroll
    for (int k = 0; k < DOUT; ++k) d.g[k] = gp[k * C];
    const float* yp = Y + (int64_t)e * DSH;
#pragma unroll
    for (int k = 0; k < DSH; ++k) d.y[k] = yp[k];
}

// One edge of the backward for one channel:
//   R_p[a][b] = sum_m3 T_p[a][b][m3] g[l3,m3]
//   h_p[a] = sum_b R_p[a][b] y[l2,b]   -> dx[l1,a] += W_p h_p[a], dW_p = sum_a x[l1,a] h_p[a]
//   v_p[b] = sum_a R_p[a][b] x[l1,a]   -> dy[l2,b] += W_p v_p[b]
// The paths are taken grouped by l2, so only one degree's grad_Y partials
// are live at a time; flush_y(k2, dy) receives each degree's partials
// (components k2 .. k2+2*l2) as soon as its last path is done.
template <class Tb, int C, bool DX, bool DW, bool DY, class FlushY>
__device__ __forceinline__ void bwd_slice(const float (&w)[Tb::P], const float (&g)[Tb::DOUT],
                                          const double (&yv)[Tb::DSH], const double (&xv)[Tb::DIN],
                                          double (&dxa)[Tb::DIN], float* __restrict__ dwp, FlushY&& flush_y)
{
    constexpr int DOUT = Tb::DOUT;
    double gv[DOUT];
#pragma unroll
    for (int k = 0; k < DOUT; ++k) gv[k] = (double)g[k];
    static_for<0, 4>([&](auto L2I) {
        constexpr int l2 = decltype(L2I)::value;
        constexpr int d2 = 2 * l2 + 1, k2 = l2 * l2;
        if constexpr ((l2 + 1) * (l2 + 1) <= Tb::DSH) {
            double dyb[d2];
#pragma unroll
            for (int b = 0; b < d2; ++b) dyb[b] = 0.0;
            static_for<0, Tb::P>([&](auto PI) {
                constexpr int p = decltype(PI)::value;
                using K = PathK<Tb, p>;
                if constexpr (K::l2 == l2) {
                    const double wd = (double)w[p];
                    static_for<0, K::d3>([&](auto M3) { opaque(gv[K::k3 + decltype(M3)::value]); });
                    double v[d2];
                    static_for<0, d2>([&](auto B) { v[decltype(B)::value] = 0.0; });
                    double dw = 0.0;
                    static_for<0, K::d1>([&](auto A) {
                        constexpr int a = decltype(A)::value;
                        if constexpr (K::ROW(a)) {
                            double h = 0.0;
                            static_for<0, d2>([&](auto B) {
                                constexpr int b = decltype(B)::value;
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
                                    h = __builtin_fma(r, yv[k2 + b], h);
                                    if constexpr (DY) v[b] = __builtin_fma(r, xv[K::k1 + a], v[b]);
                                }
                            });
                            if constexpr (DX) dxa[K::k1 + a] = __builtin_fma(wd, h, dxa[K::k1 + a]);
                            if constexpr (DW) dw = __builtin_fma(xv[K::k1 + a], h, dw);
                        }
                    });
                    if constexpr (DW) __builtin_nontemporal_store((float)dw, dwp + p * C);
                    if constexpr (DY)
                        static_for<0, d2>([&](auto B) {
                            constexpr int b = decltype(B)::value;
                            if constexpr (K::COL2(b)) dyb[b] = __builtin_fma(wd, v[b], dyb[b]);
                        });
                    // Pin this path's accumulator updates here: without it the
                    // compiler sinks every accumulation to the end of the edge
                    // and keeps all paths' h and v values live at once.
                    if constexpr (DX)
                        static_for<0, K::d1>([&](auto A) {
                            if constexpr (K::ROW(decltype(A)::value)) opaque(dxa[K::k1 + decltype(A)::value]);
                        });
                    if constexpr (DY)
                        static_for<0, d2>([&](auto B) {
                            if constexpr (K::COL2(decltype(B)::value)) opaque(dyb[decltype(B)::value]);
                        });
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
            if constexpr (DY) flush_y(std::integral_constant<int, k2>{}, dyb);
        }
    });
}

// quad_perm DPP move of a double (both halves), CTRL a quad_perm selector
template <int CTRL>
__device__ __forceinline__ double dpp_quad(double v)
{
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

// Sum over the 64 lanes of a wave of the per-wave LDS tile red[D][64]
// (D <= 16; row k holds every lane's partial of component k, written by the
// caller): lane 4k+q adds red[k][16q .. 16q+15], and a quad exchange (DPP)
// completes the sum.  Returns the total of component lane/4 in lanes with
// lane%4 == 0.
template <int D>
__device__ __forceinline__ double wave_sum_tile(const double* __restrict__ red, int lane)
{
    static_assert(D <= 16, "at most 16 components");
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
__global__ void __launch_bounds__(256, (Tune<LIN, C>::bwd_occ)) k_conv_bwd(int32_t N, GraphView gv,
                                                                         const float* __restrict__ x,
                                                                         const float* __restrict__ Y,
                                                                         const float* __restrict__ W,
                                                                         const float* __restrict__ Gr,
                                                                         float* __restrict__ dx,
                                                                         float* __restrict__ dW,
                                                                         float* __restrict__ dY)
{
    using Tb = cgmath::Tables<LIN, LSH, LOUT>;
    using Gm = Geo<C>;
    constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH, S = Gm::S, LPE = Gm::LPE, H = Gm::H;
    constexpr bool kPf = Tune<LIN, C>::bwd_prefetch;
    // LDS: per-wave grad_Y transpose tiles during the edge loop, then the
    // streams' grad_x partials
    constexpr bool kLdsSum = DY && LPE == 64;
    constexpr int kTiles = kLdsSum ? 4 * DSH * 64 : 0;
    constexpr int kDx = DX ? S * DIN * C : 0;
    constexpr int kLds = (kTiles > kDx ? kTiles : kDx) > 0 ? (kTiles > kDx ? kTiles : kDx) : 1;
    __shared__ double lds[kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const Pos<C> ps(tid);
    const int ch = ps.channel();
    const int32_t j = gv.sorder[blockIdx.x];
    if ((uint32_t)j >= (uint32_t)N) return;  // unprepared workspace: never index with it

    double xv[DIN], dxa[DIN];
    {
        const float* xp = x + (int64_t)j * (DIN * C) + ch;
#pragma unroll
        for (int k = 0; k < DIN; ++k) {
            xv[k] = (double)xp[k * C];
            dxa[k] = 0.0;
        }
    }
    const int32_t end = gv.srow[j + 1];
    int32_t q = gv.srow[j] + ps.s;
    // One edge: with prefetch, load the stream's next edge into `nxt` before
    // computing `cur`.  The loop alternates the two buffers (no copies).
    auto step = [&](BwdEdge<Tb>& cur, BwdEdge<Tb>& nxt) {
        const int32_t qn = q + S;
        if constexpr (kPf) {
            if (qn < end) bwd_load<Tb, C>(nxt, qn, ch, N, gv, Y, W, Gr);
        } else {
            bwd_load<Tb, C>(cur, q, ch, N, gv, Y, W, Gr);
        }
        q = qn;
        if (!cur.ok) return;
        double yv[DSH];
        edge_sh<DSH, LPE>(cur.y, yv);
        float* dwp = dW + (int64_t)cur.e * (P * C) + ch;
        if constexpr (kLdsSum) {
            // grad_Y partials go to this wave's LDS tile degree by degree
            double* tile = lds + (tid >> 6) * (DSH * 64);
            bwd_slice<Tb, C, DX, DW, DY>(cur.w, cur.g, yv, xv, dxa, dwp, [&](auto K2, const auto& dyb) {
                constexpr int k2 = decltype(K2)::value;
#pragma unroll
                for (int b = 0; b < (int)(sizeof(dyb) / sizeof(double)); ++b) tile[(k2 + b) * 64 + lane] = dyb[b];
            });
            const double t = wave_sum_tile<DSH>(tile, lane);
            if ((lane & 3) == 0 && (lane >> 2) < DSH) {
                if constexpr (H == 1) dY[(int64_t)cur.e * DSH + (lane >> 2)] = (float)t;
                else gv.dyp[((int64_t)cur.e * H + ps.h) * DSH + (lane >> 2)] = t;
            }
        } else {
            // an edge spans LPE < 64 lanes: reduce each degree's partials over them
            float* yp = dY + (int64_t)cur.e * DSH;
            bwd_slice<Tb, C, DX, DW, DY>(cur.w, cur.g, yv, xv, dxa, dwp, [&](auto K2, const auto& dyb) {
                constexpr int k2 = decltype(K2)::value;
#pragma unroll
                for (int b = 0; b < (int)(sizeof(dyb) / sizeof(double)); ++b) {
                    double v = dyb[b];
#pragma unroll
                    for (int off = 1; off < LPE; off <<= 1) v += __shfl_xor(v, off, 64);
                    if (ps.cl == 0) yp[k2 + b] = (float)v;
                }
            });
        }
    };
    BwdEdge<Tb> ea, eb;
    if (kPf && q < end) bwd_load<Tb, C>(ea, q, ch, N, gv, Y, W, Gr);
    while (q < end) {
        step(ea, eb);
        if (q >= end) break;
        step(eb, ea);
    }
    if constexpr (DX) {
        // combine the streams in a fixed order; dx[j] has this block as its only writer
        if constexpr (kLdsSum) __syncthreads();  // every wave is done with its grad_Y tile
#pragma unroll
        for (int k = 0; k < DIN; ++k) lds[(ps.s * DIN + k) * C + ch] = dxa[k];
        __syncthreads();
        float* dp = dx + (int64_t)j * (DIN * C);
        for (int t = tid; t < DIN * C; t += 256) {
            double v = 0.0;
#pragma unroll
            for (int r = 0; r < S; ++r) v += lds[r * DIN * C + t];
            dp[t] = (float)v;
        }
    }
}

// grad_Y of an edge = the sum of its H slice partials (fixed order)
template <int DSH, int H>
__global__ void __launch_bounds__(256) k_dy_combine(int32_t E, const double* __restrict__ dyp, float* __restrict__ dY)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)E * DSH) return;
    const int64_t e = t / DSH;
    const int k = (int)(t % DSH);
    double v = 0.0;
#pragma unroll
    for (int h = 0; h < H; ++h) v += dyp[(e * H + h) * DSH + k];
    dY[t] = (float)v;
}

template <int LIN, int LSH, int LOUT, int C, bool DX, bool DW, bool DY>
hipError_t launch_bwd_t(int32_t N, GraphView g, const float* x, const float* Y, const float* W, const float* G,
                        float* dx, float* dW, float* dY, hipStream_t s)
{
    hipLaunchKernelGGL((k_conv_bwd<LIN, LSH, LOUT, C, DX, DW, DY>), dim3((unsigned)N), dim3(256), 0, s, N, g, x, Y,
                       W, G, dx, dW, dY);
    if constexpr (DY && Geo<C>::H > 1) {
        constexpr int DSH = (LSH + 1) * (LSH + 1);
        const int64_t n = (int64_t)g.n_edges * DSH;
        if (n > 0)
            hipLaunchKernelGGL((k_dy_combine<DSH, Geo<C>::H>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                               g.n_edges, g.dyp, dY);
    }
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
    return KernelSet{L, L, L, C, Geo<C>::H > 1 ? Geo<C>::H * (L + 1) * (L + 1) : 0, &launch_sh<L>,
                     &launch_fwd<L, L, L, C>, &launch_bwd<L, L, L, C>};
}

// the convolution kernels of one (L, C) without the SH launcher, for a
// translation unit of its own (the SH kernel is instantiated once per degree
// by the degree's registry)
template <int L, int C>
constexpr KernelSet make_conv_set()
{
    return KernelSet{L, L, L, C, Geo<C>::H > 1 ? Geo<C>::H * (L + 1) * (L + 1) : 0, nullptr,
                     &launch_fwd<L, L, L, C>, &launch_bwd<L, L, L, C>};
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
