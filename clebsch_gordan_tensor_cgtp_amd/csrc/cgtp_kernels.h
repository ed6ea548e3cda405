// cgtp_kernels.h -- gfx950 kernels of the CGTP convolution (templates; the
// cgtp_kernels_l<L>*.hip units instantiate them).
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
//   * at degree 3 with one 64-lane slice per edge, the backward and both
//     sides of the double backward give each edge to a pair of waves that
//     split its paths by degree (the abstract's path-group parallelism),
//     halving each wave's registers
// (graph preparation lives in cgtp_graph.hip)
//
// Arithmetic is fp64 on fp32 data: the per-edge contraction and the sums over
// a segment and over channels keep fp64 accuracy, and fp64 FMA issues at the
// same rate as unpacked fp32 on this chip.
//
// Lane mapping: a lane owns one channel of one edge.  A kernel is compiled
// for LPE lanes per edge slice and H slices per edge: for C <= 64 a wave
// covers 64/LPE edges at once (LPE the smallest power of two >= C); for
// 64 < C <= 128 a node's channels are split over two waves (H = 2).  The
// channel count itself is a run-time value; lanes past C load channel 0, take
// no part in any sum and store nothing.
//
// Degrees: each unit is compiled for the complete path set of one degree LM
// (l_in = l_sh = l_out = LM).  A plan with l_in, l_sh, l_out <= LM, not all
// equal to LM, runs the SUB variant: it uses the same compiled contraction,
// gives every path the plan does not have the weight 0 and stores no grad_W
// for it, and reads feature, SH and output rows of the plan's own widths
// (components past a width are read at the last valid index and only ever
// meet a zero weight).  The CG values and their nonzero pattern are
// compile-time constants, so every contraction below is a straight line of
// fp64 FMAs over the nonzero coefficients only.
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
#include "cgtp_sh.h"

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

__device__ __forceinline__ int32_t clampi(int32_t v, int32_t lo, int32_t hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

// element of `row` at byte offset `lb` (a lane's channel times 4): written as
// a pointer plus a zero-extended 32-bit byte offset so that a row pointer
// equal in every lane becomes the scalar base of the load or store.  The
// offset must be defined where it is used (see lane_offset), or the
// compiler hoists its 64-bit extension and adds it with vector instructions.
template <class T>
__device__ __forceinline__ T* at_lane(T* row, uint32_t lb)
{
    using B = typename std::conditional<std::is_const<T>::value, const char, char>::type;
    return (T*)((B*)row + lb);
}

// Read a value that is the same for every lane of the wave (a uniform
// address) through the scalar data cache into scalar registers, where a vector
// load would spend a vector register per lane and a read-first-lane move.
// Only data no kernel writes while this one runs is read this way.
template <class T>
__device__ __forceinline__ T scalar_load(const T* p)
{
    return *(const __attribute__((address_space(4))) T*)p;
}

// the lane's byte offset, re-defined at this point (an empty asm the
// optimiser cannot see through) for at_lane
__device__ __forceinline__ uint32_t lane_offset(uint32_t lb)
{
    asm volatile("" : "+v"(lb));
    return lb;
}

// the channel count, re-defined at this point: the row offsets p*C of an
// edge are then formed per edge with scalar arithmetic instead of being
// hoisted out of the edge loop, where they would hold 30 scalar registers
// and push others into spills
__device__ __forceinline__ int32_t edge_stride(int32_t C)
{
    asm volatile("" : "+s"(C));
    return C;
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
    double o[D];
    shf::values<L>(rx / n, ry / n, rz / n, o);
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
// One 256-thread block (four waves) per node.  LPE lanes cover a slice of up
// to LPE channels, and for H = 2 the two slices of a node go to different
// waves, so every wave carries the state of a single slice (the register
// budget decides occupancy here).  The node's edges are interleaved over the
// block's S edge streams (stream s takes the node's edges s, s+S, s+2S, ...),
// which keeps a long segment from serialising on one wave; the streams'
// partial sums are combined in LDS in a fixed order at the end (atomic-free,
// deterministic).
template <int LPE, int H>
struct Geo {
    static_assert(LPE == 8 || LPE == 16 || LPE == 32 || LPE == 64, "lanes per edge slice");
    static_assert(H == 1 || (H == 2 && LPE == 64), "two slices only with full waves");
    static constexpr int CP = LPE * H;               // padded channel count
    static constexpr int S = (4 / H) * (64 / LPE);   // edge streams per block
};

// position of this thread: channel slice, channel within the slice, stream
template <int LPE, int H>
struct Pos {
    int h, cl, s;
    __device__ __forceinline__ explicit Pos(int tid)
    {
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        h = wave % H;
        cl = (tid & 63) % LPE;
        if constexpr (LPE == 64) s = wave / H;  // wave-uniform
        else s = wave * (64 / LPE) + (tid & 63) / LPE;
    }
    __device__ __forceinline__ int channel() const { return h * LPE + cl; }
};

// Per-specialisation tuning: the minimum waves per SIMD the register
// allocation must allow, and whether the forward loads the next edge's
// operands before the current edge is computed.  Chosen so that no
// specialisation spills vector registers (a spill costs far more than the
// occupancy it buys), with one measured exception below.  From degree 2 on
// the forward is bound by fp64 issue, and the copies that rotate a prefetched
// edge into place cost more than the latency they hide (measured: 4% slower
// on the 50,000-atom layer), so only degree 1 prefetches.
// The double-backward kernels carry a second set of operands (the
// cotangents) and run at lower occupancy.  At degree 2 the receiver side fits
// 3 waves per SIMD without spilling.  The sender side needs 171 registers for
// 2 waves; held to 3 waves it spills 12-20 bytes per lane with one 64-lane
// slice per edge and is still 7-8% faster (2000- and 4000-atom layers), while
// narrower slices would spill 80-100 bytes and keep 2.
// The path-split kernels (degree 3, one 64-lane slice, two waves per edge)
// hold half of a single wave's per-edge state: the backward fits 3 waves per
// SIMD (168 registers and a 4-byte spill, measured 6% faster than 2 waves
// with the whole path set), both sides of the double backward 2 (from 1).
template <int LM, int LPE>
struct Tune {
    static constexpr int fwd_occ = LM <= 2 ? 4 : 2;
    static constexpr int bwd_occ = LM == 1 || (LM == 2 && LPE == 64) ? 4 : (LM == 2 ? 3 : 2);
    static constexpr bool fwd_prefetch = LM == 1;
    static constexpr int ps_bwd_occ = 3;
    static constexpr int dbl_ps_bwd_occ = 2;
    static constexpr int dbl_ps_fwd_occ = 2;
    static constexpr int dbl_fwd_occ = LM == 1 ? 4 : (LM == 2 ? 3 : 1);
    static constexpr int dbl_bwd_occ = LM == 1 ? 4 : (LM == 2 ? (LPE == 64 ? 3 : 2) : 1);
};

// acc += a*b, where the first term of a sum (`started` false, known at
// compile time after unrolling) is a plain product: a product with a unit CG
// coefficient then folds to a copy or a sign flip instead of an FMA with 0.
__device__ __forceinline__ void mac(double& acc, double a, double b, bool& started)
{
    acc = started ? __builtin_fma(a, b, acc) : a * b;
    started = true;
}

// An empty asm that takes a register value and hands it back: the optimiser
// must materialise the value at that point and cannot match it with values
// computed before it.  Used to keep accumulations in path order (otherwise
// they are sunk to the end of the edge and every path's intermediates stay
// live) and to keep per-path products from being shared across paths.
__device__ __forceinline__ void opaque(double& v) { asm volatile("" : "+v"(v)); }

// ---- CG coefficients in scalar registers -----------------------------------
// A coefficient other than an inline constant of the instruction set (+-1,
// +-0.5, +-2, +-4) is an fp64 value the FMAs read from a scalar register
// pair.  Left to itself the compiler materialises every distinct coefficient
// of a kernel once, before the edge loop; at degree 3 (42 distinct
// magnitudes) that is more scalar registers than a wave has, and the excess is
// spilled into vector-register lanes, which costs a vector instruction per
// read inside the loop.  Instead each path materialises its own few
// magnitudes (at most 9 at degree 3) where it starts, two scalar moves each
// that cannot be hoisted out of the loop: scalar issue has room here, vector
// issue is the bound.  Signs become operand modifiers.  Up to degree 2 the
// compiler's own placement is kept (the extra moves measured 1-2% slower in
// the degree-2 forward), except in the double backward (ALL), whose operand
// sets leave fewer scalar registers (1-2.5% faster there).
constexpr double cabs(double v) { return v < 0.0 ? -v : v; }
constexpr bool inline_coef(double m) { return m == 1.0 || m == 0.5 || m == 2.0 || m == 4.0; }

template <class Tb, int p, bool ALL = false>
struct PathMags {
    using K = PathK<Tb, p>;
    struct M {
        double v[64];
        int n;
    };
    static constexpr M make()
    {
        M m{};
        m.n = 0;
        for (int a = 0; a < K::d1; ++a)
            for (int b = 0; b < K::d2; ++b)
                for (int c = 0; c < K::d3; ++c) {
                    const double t = cabs(K::T(a, b, c));
                    if (t == 0.0 || inline_coef(t) || (Tb::DIN < 16 && !ALL)) continue;
                    bool seen = false;
                    for (int i = 0; i < m.n; ++i) seen = seen || m.v[i] == t;
                    if (!seen) m.v[m.n++] = t;
                }
        return m;
    }
    static constexpr M mags = make();
    static constexpr int N = mags.n;
    static_assert(N <= 64, "distinct coefficient magnitudes of a path");
    // slot of coefficient t, or -1 for an inline constant
    static constexpr int slot(double t)
    {
        for (int i = 0; i < N; ++i)
            if (mags.v[i] == cabs(t)) return i;
        return -1;
    }
};

// 32-bit value in a scalar register, defined here (never hoisted or merged)
template <uint32_t V>
__device__ __forceinline__ uint32_t sreg32()
{
    uint32_t r;
    asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(V));
    return r;
}

// the magnitudes of path p's coefficients, in scalar registers
template <class Tb, int p, bool ALL = false>
struct PathCoefs {
    using Mg = PathMags<Tb, p, ALL>;
    double c[Mg::N > 0 ? Mg::N : 1];
    __device__ __forceinline__ PathCoefs()
    {
        static_for<0, Mg::N>([&](auto I) {
            constexpr uint64_t bits = __builtin_bit_cast(uint64_t, Mg::mags.v[decltype(I)::value]);
            const uint32_t lo = sreg32<(uint32_t)bits>(), hi = sreg32<(uint32_t)(bits >> 32)>();
            c[decltype(I)::value] = __hiloint2double((int)hi, (int)lo);
        });
    }
    // acc += t * v for the coefficient t at (a, b, m3) of the path (the first
    // term of a sum a plain product; see mac)
    template <int a, int b, int m3>
    __device__ __forceinline__ void mac(double& acc, double v, bool& started) const
    {
        constexpr double t = PathK<Tb, p>::T(a, b, m3);
        constexpr int i = Mg::slot(t);
        if constexpr (i < 0) {
            cgtp::mac(acc, t, v, started);
        } else if constexpr (t > 0.0) {
            cgtp::mac(acc, c[i], v, started);
        } else {
            cgtp::mac(acc, -c[i], v, started);
        }
    }
};

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

// the edge's spherical harmonics evaluated from its vector r (the fused-SH
// kernels), fp64; in scalar registers when the whole wave works on one edge
template <int LM, int DSH, int LPE>
__device__ __forceinline__ void edge_sh_r(const float (&r)[3], double (&yv)[DSH])
{
    double x, y, z, inv;
    shf::unit(r[0], r[1], r[2], x, y, z, inv);
    shf::values<LM>(x, y, z, yv);
    if constexpr (LPE == 64)
#pragma unroll
        for (int k = 0; k < DSH; ++k) yv[k] = uniform(yv[k]);
}

// grad_r = sum_k w[k] dY_k/dr of the edge vector r (degrees 0..LM), the
// weights w[0 .. (LM+1)^2) read from LDS one degree at a time; components
// k >= d_sh (past the plan's SH width) count as zero
template <int LM>
__device__ __forceinline__ void edge_r_grad(const float (&r)[3], const double* w, int32_t d_sh, double (&g)[3])
{
    double x, y, z, inv;
    shf::unit(r[0], r[1], r[2], x, y, z, inv);
    double qx = 0.0, qy = 0.0, qz = 0.0;
    static_for<1, LM + 1>([&](auto LI) {
        constexpr int l = decltype(LI)::value;
        double wl[2 * l + 1];
#pragma unroll
        for (int b = 0; b < 2 * l + 1; ++b) wl[b] = l * l + b < d_sh ? w[l * l + b] : 0.0;
        shf::grad_degree<l>(x, y, z, wl, qx, qy, qz);
    });
    shf::tangent(x, y, z, inv, qx, qy, qz, g);
}

// Row widths and weight offsets of a launch: compile-time for the complete
// degree set, run-time (from the Shape) for a SUB plan.
template <class Tb, bool SUB>
struct Dims {
    int32_t d_in, d_sh, d_out, P;  // P: weight rows per edge
    __device__ __forceinline__ explicit Dims(const Shape& s)
    {
        if constexpr (SUB) {
            d_in = s.d_in;
            d_sh = s.d_sh;
            d_out = s.d_out;
            P = s.P;
        } else {
            d_in = Tb::DIN;
            d_sh = Tb::DSH;
            d_out = Tb::DOUT;
            P = Tb::P;
        }
    }
    // component k of a row of width d (SUB: clamped to the last valid one)
    template <int k>
    __device__ __forceinline__ static int32_t comp(int32_t d)
    {
        if constexpr (SUB) return k < d ? k : d - 1;
        else return k;
    }
};

// ----------------------------------------------------------------------------
// forward
// ----------------------------------------------------------------------------
template <class Tb>
struct FwdEdge {
    static constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH;
    float w[P], x[DIN], y[DSH];
    float r[3];  // the edge vector (fused-SH kernels, which load it instead of y)
};

// operands of edge e for the lane at byte offset chl (an in-range channel
// times 4).  Every row is
// addressed as a row pointer (uniform when the whole wave works on one edge)
// plus the lane's channel as an unsigned 32-bit index, which the compiler
// turns into scalar-base + lane-offset loads without 64-bit vector adds.
// (L3M: the weights only of the paths whose l3 is in the mask)
template <class Tb, bool SUB, bool UNI, bool FSH = false, int L3M = 0xF>
__device__ __forceinline__ void fwd_load(FwdEdge<Tb>& d, int32_t e, uint32_t chl, const FwdArgs& a,
                                         const Dims<Tb, SUB>& dm)
{
    constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH;
    const int32_t C = edge_stride(a.sh.C);
    chl = lane_offset(chl);
    int32_t j = UNI ? scalar_load(a.src + e) : a.src[e];
    j = (uint32_t)j < (uint32_t)a.sh.N ? j : 0;  // a sender outside [0, N) breaks the CSR contract
    const float* wrow = a.W + (int64_t)e * (dm.P * C);
    static_for<0, P>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        if constexpr (!((L3M >> Tb::data.l3[p]) & 1)) {
            d.w[p] = 0.0f;  // another wave's path
        } else if constexpr (SUB) {
            const float v = __builtin_nontemporal_load(at_lane(wrow + a.sh.woff[p], chl));
            d.w[p] = ((a.sh.active >> p) & 1) ? v : 0.0f;
        } else {
            d.w[p] = __builtin_nontemporal_load(at_lane(wrow + p * C, chl));
        }
    });
    const float* xrow = a.x + (int64_t)j * (dm.d_in * C);
    static_for<0, DIN>([&](auto K) { d.x[K] = *at_lane(xrow + Dims<Tb, SUB>::template comp<decltype(K)::value>(dm.d_in) * C, chl); });
    // (the edge's SH stay vector loads here: held across the prefetch, they
    // would occupy scalar registers the contraction needs)
    if constexpr (FSH) {
        const float* rp = a.r + 3 * (int64_t)e;
#pragma unroll
        for (int k = 0; k < 3; ++k) d.r[k] = rp[k];
    } else {
        const float* yp = a.Y + (int64_t)e * dm.d_sh;
        static_for<0, DSH>([&](auto K) { d.y[K] = yp[Dims<Tb, SUB>::template comp<decltype(K)::value>(dm.d_sh)]; });
    }
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
        const PathCoefs<Tb, p> cf;
        static_for<0, K::d3>([&](auto M3) {
            constexpr int m3 = decltype(M3)::value;
            double z = 0.0;
            bool any = false;
            static_for<0, K::d1>([&](auto A) {
                static_for<0, K::d2>([&](auto B) {
                    constexpr int a = decltype(A)::value, b = decltype(B)::value;
                    constexpr double t = K::T(a, b, m3);
                    if constexpr (t != 0.0) cf.template mac<a, b, m3>(z, xv[K::k1 + a] * yv[K::k2 + b], any);
                });
            });
            if (any) acc[K::k3 + m3] = __builtin_fma(wd, z, acc[K::k3 + m3]);
        });
        // keep the accumulation in path order (see opaque)
        static_for<0, K::d3>([&](auto M3) { opaque(acc[K::k3 + decltype(M3)::value]); });
    });
}

// ---- double backward, receiver side ----------------------------------------
// The gradient of S = <ggx, grad_x> + <ggW, grad_W> + <ggY, grad_Y> with
// respect to grad_out is the forward applied to the three products that are
// linear in one cotangent each:
//   d_out[i] = sum_e W (ggx_j (x) Y) + W (x_j (x) ggY) + ggW (x_j (x) Y).
// It runs on the forward's work decomposition with these operands added.
template <class Tb>
struct FwdEdgeD : FwdEdge<Tb> {
    float gw[Tb::P], gx[Tb::DIN], gy[Tb::DSH];
};

// the cotangent rows of edge e (zero where the caller passed none)
template <class Tb, bool SUB, bool UNI, int L3M = 0xF>
__device__ __forceinline__ void fwd_load_dbl(FwdEdgeD<Tb>& d, int32_t e, uint32_t chl, const FwdArgs& a,
                                             const Dims<Tb, SUB>& dm)
{
    fwd_load<Tb, SUB, UNI, false, L3M>(d, e, chl, a, dm);
    constexpr int P = Tb::P, DIN = Tb::DIN, DSH = Tb::DSH;
    const int32_t C = edge_stride(a.sh.C);
    chl = lane_offset(chl);
    int32_t j = UNI ? scalar_load(a.src + e) : a.src[e];
    j = (uint32_t)j < (uint32_t)a.sh.N ? j : 0;
    if (a.ggW) {
        const float* wrow = a.ggW + (int64_t)e * (dm.P * C);
        static_for<0, P>([&](auto PI) {
            constexpr int p = decltype(PI)::value;
            if constexpr (!((L3M >> Tb::data.l3[p]) & 1)) {
                d.gw[p] = 0.0f;  // another wave's path
            } else if constexpr (SUB) {
                const float v = __builtin_nontemporal_load(at_lane(wrow + a.sh.woff[p], chl));
                d.gw[p] = ((a.sh.active >> p) & 1) ? v : 0.0f;
            } else {
                d.gw[p] = __builtin_nontemporal_load(at_lane(wrow + p * C, chl));
            }
        });
    } else {
#pragma unroll
        for (int p = 0; p < P; ++p) d.gw[p] = 0.0f;
    }
    if (a.ggx) {
        const float* xrow = a.ggx + (int64_t)j * (dm.d_in * C);
        static_for<0, DIN>([&](auto K) { d.gx[K] = *at_lane(xrow + Dims<Tb, SUB>::template comp<decltype(K)::value>(dm.d_in) * C, chl); });
    } else {
#pragma unroll
        for (int k = 0; k < DIN; ++k) d.gx[k] = 0.0f;
    }
    if (a.ggY) {
        const float* yp = a.ggY + (int64_t)e * dm.d_sh;
        static_for<0, DSH>([&](auto K) { d.gy[K] = yp[Dims<Tb, SUB>::template comp<decltype(K)::value>(dm.d_sh)]; });
    } else {
#pragma unroll
        for (int k = 0; k < DSH; ++k) d.gy[k] = 0.0f;
    }
}

// acc[l3,m3] += sum_p sum_{a,b} T_p[a][b][m3] (W_p (ggx[a] y[b] + x[a] ggy[b]) + ggW_p x[a] y[b])
// over the paths whose l3 is in the mask L3M
template <class Tb, int L3M = 0xF>
__device__ __forceinline__ void fwd_slice_dbl(const FwdEdgeD<Tb>& d, const double (&yv)[Tb::DSH],
                                              const double (&gyv)[Tb::DSH], double (&acc)[Tb::DOUT])
{
    double xv[Tb::DIN], gxv[Tb::DIN];
#pragma unroll
    for (int k = 0; k < Tb::DIN; ++k) {
        xv[k] = (double)d.x[k];
        gxv[k] = (double)d.gx[k];
    }
    static_for<0, Tb::P>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        using K = PathK<Tb, p>;
        if constexpr (!((L3M >> K::l3) & 1)) return;  // another wave's path
        const double wd = (double)d.w[p], gwd = (double)d.gw[p];
        const PathCoefs<Tb, p, true> cf;
        static_for<0, K::d3>([&](auto M3) {
            constexpr int m3 = decltype(M3)::value;
            double z1 = 0.0, z2 = 0.0;
            bool any1 = false, any2 = false;
            static_for<0, K::d1>([&](auto A) {
                static_for<0, K::d2>([&](auto B) {
                    constexpr int a = decltype(A)::value, b = decltype(B)::value;
                    constexpr double t = K::T(a, b, m3);
                    if constexpr (t != 0.0) {
                        const double x = xv[K::k1 + a], y = yv[K::k2 + b];
                        cf.template mac<a, b, m3>(z1, __builtin_fma(x, gyv[K::k2 + b], gxv[K::k1 + a] * y), any1);
                        cf.template mac<a, b, m3>(z2, x * y, any2);
                    }
                });
            });
            if (any1) acc[K::k3 + m3] = __builtin_fma(wd, z1, __builtin_fma(gwd, z2, acc[K::k3 + m3]));
        });
        static_for<0, K::d3>([&](auto M3) { opaque(acc[K::k3 + decltype(M3)::value]); });
    });
}

// the two halves of a path-group split (degree masks): l = 1, 2 and l = 0, 3
constexpr int kPsMask0 = 0x6, kPsMask1 = 0x9;

// degree l of component k (k < 16)
constexpr int degree_of(int k) { return k < 1 ? 0 : (k < 4 ? 1 : (k < 9 ? 2 : 3)); }

// Geometry of a forward block: with PS (the path-group split, see the
// backward) two waves serve each edge and its 64 channels, one taking the
// paths whose output degree l3 is in {1, 2}, the other those in {0, 3}; each
// holds the accumulators of its own degrees and the weights of its own paths,
// and every output row keeps one writer.  Used by the receiver side of the
// degree-3 double backward with one 64-lane slice.
template <int LM, int LPE, int H, bool PS>
struct FwdGeo {
    using Tb = cgmath::Tables<LM, LM, LM>;
    static constexpr int HW = PS ? 2 : H;  // waves per edge
    using Gm = Geo<LPE, HW>;
    static constexpr int S = Gm::S, CP = PS ? LPE : Gm::CP, DOUT = Tb::DOUT;
    static constexpr int kRed = S * DOUT * CP;
};

template <int LM, int LPE, bool DBL, bool PS>
constexpr int fwd_bound()
{
    if (PS) return Tune<LM, LPE>::dbl_ps_fwd_occ;
    return DBL ? Tune<LM, LPE>::dbl_fwd_occ : Tune<LM, LPE>::fwd_occ;
}

// The forward of one block over the paths whose l3 is in L3M; red: the LDS
// of the streams' partial sums [stream][k][channel].
template <int LM, int LPE, int H, bool SUB, bool DBL, bool FSH, bool PS, int L3M>
__device__ __forceinline__ void fwd_body(const FwdArgs& a, double* __restrict__ red)
{
    static_assert(!(DBL && FSH), "the double backward takes Y");
    static_assert(!PS || (DBL && LPE == 64 && H == 1), "path split: double backward, one slice");
    using Tb = cgmath::Tables<LM, LM, LM>;
    using Fg = FwdGeo<LM, LPE, H, PS>;
    constexpr int DSH = Tb::DSH, DOUT = Tb::DOUT, S = Fg::S, CP = Fg::CP;
    constexpr bool kPf = Tune<LM, LPE>::fwd_prefetch && !DBL;
    using Edge = std::conditional_t<DBL, FwdEdgeD<Tb>, FwdEdge<Tb>>;

    const int tid = threadIdx.x;
    const Pos<LPE, Fg::HW> ps(tid);
    const int ch = PS ? ps.cl : ps.channel();
    const int32_t C = a.sh.C;
    const uint32_t chl = ch < C ? 4u * ch : 0u;  // byte offset; lanes past C read channel 0 and store nothing
    const Dims<Tb, SUB> dm(a.sh);
    const int32_t i = a.rorder[blockIdx.x];
    if ((uint32_t)i >= (uint32_t)a.sh.N) return;  // idle block (or an unprepared schedule)
    const int32_t E = a.sh.E;
    const int32_t e0 = clampi(a.row_ptr[i], 0, E);
    const int32_t end = clampi(a.row_ptr[i + 1], e0, E);

    double acc[DOUT];
#pragma unroll
    for (int k = 0; k < DOUT; ++k) acc[k] = 0.0;

    // with prefetch, the stream's next edge is loaded before the current one
    // is computed (the copy `cur = nxt` costs fewer registers than
    // alternating two named buffers, which would spill at this occupancy)
    int32_t e = e0 + ps.s;
    Edge cur;
    if (kPf && e < end) fwd_load<Tb, SUB, LPE == 64, FSH>(cur, e, chl, a, dm);
    while (e < end) {
        const int32_t en = e + S;
        Edge nxt;
        if constexpr (kPf) {
            if (en < end) fwd_load<Tb, SUB, LPE == 64, FSH>(nxt, en, chl, a, dm);
        } else if constexpr (DBL) {
            fwd_load_dbl<Tb, SUB, LPE == 64, L3M>(cur, e, chl, a, dm);
        } else {
            fwd_load<Tb, SUB, LPE == 64, FSH>(cur, e, chl, a, dm);
        }
        double yv[DSH];
        if constexpr (FSH) edge_sh_r<LM, DSH, LPE>(cur.r, yv);
        else edge_sh<DSH, LPE>(cur.y, yv);
        if constexpr (DBL) {
            double gyv[DSH];
            edge_sh<DSH, LPE>(cur.gy, gyv);
            fwd_slice_dbl<Tb, L3M>(cur, yv, gyv, acc);
        } else {
            fwd_slice<Tb>(cur.w, cur.x, yv, acc);
        }
        if constexpr (kPf) cur = nxt;
        e = en;
    }

    // combine the streams in a fixed order; out[i] has this block as its only writer
    // (with the path split each wave writes the components of its degrees)
    static_for<0, DOUT>([&](auto Kc) {
        constexpr int k = decltype(Kc)::value;
        if constexpr ((L3M >> degree_of(k)) & 1) red[(ps.s * DOUT + k) * CP + ch] = acc[k];
    });
    __syncthreads();
    float* op = a.out + (int64_t)i * (dm.d_out * C);
    for (int t = tid; t < DOUT * CP; t += 256) {
        const int k = t / CP, c = t % CP;
        if (k < dm.d_out && c < C) {
            double v = 0.0;
#pragma unroll
            for (int q = 0; q < S; ++q) v += red[q * DOUT * CP + t];
            op[k * C + c] = (float)v;
        }
    }
}

template <int LM, int LPE, int H, bool SUB, bool DBL = false, bool FSH = false, bool PS = false>
__global__ void __launch_bounds__(256, (fwd_bound<LM, LPE, DBL, PS>())) k_conv_fwd(FwdArgs a)
{
    __shared__ double red[FwdGeo<LM, LPE, H, PS>::kRed];
    if constexpr (PS) {
        // the pair's first wave (even wave index) takes the l3 = 1, 2 paths
        if ((__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1) == 0)
            fwd_body<LM, LPE, H, SUB, DBL, FSH, PS, kPsMask0>(a, red);
        else
            fwd_body<LM, LPE, H, SUB, DBL, FSH, PS, kPsMask1>(a, red);
    } else {
        fwd_body<LM, LPE, H, SUB, DBL, FSH, PS, 0xF>(a, red);
    }
}

template <int LM, int LPE, int H, bool SUB, bool DBL = false, bool FSH = false, bool PS = false>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s)
{
    if (a.sh.N == 0) return hipSuccess;
    hipLaunchKernelGGL((k_conv_fwd<LM, LPE, H, SUB, DBL, FSH, PS>), dim3((unsigned)conv_grid(a.sh.N)), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}

// the double backward's receiver side; at degree 3 with one 64-lane slice
// the path-split form
template <int LM, int LPE, int H>
hipError_t launch_fwd_dbl(const FwdArgs& a, hipStream_t s)
{
    return launch_fwd<LM, LPE, H, true, true, false, (LM == 3 && LPE == 64 && H == 1)>(a, s);
}

// ----------------------------------------------------------------------------
// forward with per-path outputs
// ----------------------------------------------------------------------------
// Every path writes its own 2*l3+1 output rows instead of adding into the l3
// slot (the summed output is the sum of these blocks over the paths of each
// l3).  The compiled paths are cut into consecutive groups of at most kMidRows
// output rows; one launch serves one group, so a lane's accumulators stay at
// the summed forward's count at degree 3 (16) and the groups' outputs are
// disjoint (no partial sums across launches).  Each launch gathers x_j and Y
// again and reads only its paths' weights.
constexpr int kMidRows = 16;

template <class Tb>
struct PathGroups {
    struct Info {
        int n;
        int begin[kMaxPaths + 1];
    };
    static constexpr Info make()
    {
        Info r{};
        int g = 0, rows = 0;
        r.begin[0] = 0;
        for (int p = 0; p < Tb::P; ++p) {
            const int d3 = 2 * Tb::data.l3[p] + 1;
            if (rows + d3 > kMidRows) {
                r.begin[++g] = p;
                rows = 0;
            }
            rows += d3;
        }
        r.n = g + 1;
        r.begin[r.n] = Tb::P;
        return r;
    }
    static constexpr Info info = make();
    static constexpr int NG = info.n;
    // rows of group g before path p (p inside the group), and the group's rows
    static constexpr int row_of(int g, int p)
    {
        int r = 0;
        for (int q = info.begin[g]; q < p; ++q) r += 2 * Tb::data.l3[q] + 1;
        return r;
    }
    static constexpr int rows(int g) { return row_of(g, info.begin[g + 1]); }
};

template <class Tb, int G>
struct MidEdge {
    static constexpr int P0 = PathGroups<Tb>::info.begin[G], P1 = PathGroups<Tb>::info.begin[G + 1];
    float w[P1 - P0], x[Tb::DIN], y[Tb::DSH];
};

template <class Tb, int G, bool UNI>
__device__ __forceinline__ void fwd_load_mid(MidEdge<Tb, G>& d, int32_t e, uint32_t chl, const FwdArgs& a,
                                             const Dims<Tb, true>& dm)
{
    using M = MidEdge<Tb, G>;
    constexpr int DIN = Tb::DIN, DSH = Tb::DSH;
    const int32_t C = edge_stride(a.sh.C);
    chl = lane_offset(chl);
    int32_t j = UNI ? scalar_load(a.src + e) : a.src[e];
    j = (uint32_t)j < (uint32_t)a.sh.N ? j : 0;  // a sender outside [0, N) breaks the CSR contract
    const float* wrow = a.W + (int64_t)e * (dm.P * C);
    static_for<M::P0, M::P1>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        const float v = __builtin_nontemporal_load(at_lane(wrow + a.sh.woff[p], chl));
        d.w[p - M::P0] = ((a.sh.active >> p) & 1) ? v : 0.0f;
    });
    const float* xrow = a.x + (int64_t)j * (dm.d_in * C);
    static_for<0, DIN>([&](auto K) { d.x[K] = *at_lane(xrow + Dims<Tb, true>::template comp<decltype(K)::value>(dm.d_in) * C, chl); });
    const float* yp = a.Y + (int64_t)e * dm.d_sh;
    static_for<0, DSH>([&](auto K) { d.y[K] = yp[Dims<Tb, true>::template comp<decltype(K)::value>(dm.d_sh)]; });
}

template <int LM, int LPE, int H, int G>
__global__ void __launch_bounds__(256, (Tune<LM, LPE>::fwd_occ)) k_conv_fwd_mid(FwdArgs a)
{
    using Tb = cgmath::Tables<LM, LM, LM>;
    using Gm = Geo<LPE, H>;
    using PG = PathGroups<Tb>;
    using M = MidEdge<Tb, G>;
    constexpr int DSH = Tb::DSH, S = Gm::S, CP = Gm::CP;
    constexpr int DG = PG::rows(G);
    __shared__ double red[S * DG * CP];

    const int tid = threadIdx.x;
    const Pos<LPE, H> ps(tid);
    const int ch = ps.channel();
    const int32_t C = a.sh.C;
    const uint32_t chl = ch < C ? 4u * ch : 0u;
    const Dims<Tb, true> dm(a.sh);
    const int32_t i = a.rorder[blockIdx.x];
    if ((uint32_t)i >= (uint32_t)a.sh.N) return;
    const int32_t E = a.sh.E;
    const int32_t e0 = clampi(a.row_ptr[i], 0, E);
    const int32_t end = clampi(a.row_ptr[i + 1], e0, E);

    double acc[DG];
#pragma unroll
    for (int k = 0; k < DG; ++k) acc[k] = 0.0;
    for (int32_t e = e0 + ps.s; e < end; e += S) {
        M cur;
        fwd_load_mid<Tb, G, LPE == 64>(cur, e, chl, a, dm);
        double yv[DSH], xv[Tb::DIN];
        edge_sh<DSH, LPE>(cur.y, yv);
#pragma unroll
        for (int k = 0; k < Tb::DIN; ++k) xv[k] = (double)cur.x[k];
        static_for<M::P0, M::P1>([&](auto PI) {
            constexpr int p = decltype(PI)::value;
            using K = PathK<Tb, p>;
            constexpr int r0 = PG::row_of(G, p);
            const double wd = (double)cur.w[p - M::P0];
            static_for<0, K::d3>([&](auto M3) {
                constexpr int m3 = decltype(M3)::value;
                double z = 0.0;
                bool any = false;
                static_for<0, K::d1>([&](auto A) {
                    static_for<0, K::d2>([&](auto B) {
                        constexpr int a_ = decltype(A)::value, b = decltype(B)::value;
                        constexpr double t = K::T(a_, b, m3);
                        if constexpr (t != 0.0) mac(z, t, xv[K::k1 + a_] * yv[K::k2 + b], any);
                    });
                });
                if (any) acc[r0 + m3] = __builtin_fma(wd, z, acc[r0 + m3]);
            });
            static_for<0, K::d3>([&](auto M3) { opaque(acc[r0 + decltype(M3)::value]); });
        });
    }

    // combine the streams in a fixed order; each path's rows have this block as their only writer
#pragma unroll
    for (int k = 0; k < DG; ++k) red[(ps.s * DG + k) * CP + ch] = acc[k];
    __syncthreads();
    float* op = a.out + (int64_t)i * (dm.d_out * C);
    for (int t = tid; t < DG * CP; t += 256) {
        const int k = t / CP, c = t % CP;
        // output row of local row k: the owning path's block
        int32_t row = -1;
        static_for<M::P0, M::P1>([&](auto PI) {
            constexpr int p = decltype(PI)::value;
            constexpr int r0 = PG::row_of(G, p), d3 = 2 * Tb::data.l3[p] + 1;
            if (k >= r0 && k < r0 + d3 && a.sh.moff[p] >= 0) row = a.sh.moff[p] + (k - r0);
        });
        if (row >= 0 && row < dm.d_out && c < C) {
            double v = 0.0;
#pragma unroll
            for (int q = 0; q < S; ++q) v += red[q * DG * CP + t];
            op[row * C + c] = (float)v;
        }
    }
}

// launches of groups G, G+1, ... in order
template <int LM, int LPE, int H, int G>
hipError_t launch_fwd_mid_from(const FwdArgs& a, hipStream_t s)
{
    if constexpr (G < PathGroups<cgmath::Tables<LM, LM, LM>>::NG) {
        hipLaunchKernelGGL((k_conv_fwd_mid<LM, LPE, H, G>), dim3((unsigned)conv_grid(a.sh.N)), dim3(256), 0, s, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        return launch_fwd_mid_from<LM, LPE, H, G + 1>(a, s);
    } else {
        return hipSuccess;
    }
}

template <int LM, int LPE, int H>
hipError_t launch_fwd_mid(const FwdArgs& a, hipStream_t s)
{
    if (a.sh.N == 0) return hipSuccess;
    return launch_fwd_mid_from<LM, LPE, H, 0>(a, s);
}

// ----------------------------------------------------------------------------
// backward
// ----------------------------------------------------------------------------
template <class Tb>
struct BwdEdge {
    static constexpr int P = Tb::P, DSH = Tb::DSH, DOUT = Tb::DOUT;
    int32_t e, i;
    bool ok;  // the view entry names a valid edge and receiver
    float w[P], g[DOUT], y[DSH];
    float r[3];  // the edge vector (fused-SH kernels, which load it instead of y)
};

// operands of the q-th edge of the sender-sorted view for the lane at byte
// offset chl (the weights only of the paths whose l1 is in the mask L1M); a
// corrupt entry (possible only if the view was not prepared for this graph)
// is read as edge 0 / receiver 0 and flagged, never used out of bounds
template <class Tb, bool SUB, bool UNI, bool LOADG = true, bool FSH = false, int L1M = 0xF>
__device__ __forceinline__ void bwd_load(BwdEdge<Tb>& d, int32_t q, uint32_t chl, const BwdArgs& a,
                                         const Dims<Tb, SUB>& dm)
{
    constexpr int P = Tb::P, DSH = Tb::DSH, DOUT = Tb::DOUT;
    const int32_t C = edge_stride(a.sh.C);
    chl = lane_offset(chl);
    int32_t e = UNI ? scalar_load(a.g.perm + q) : a.g.perm[q];
    int32_t i = UNI ? scalar_load(a.g.sdst + q) : a.g.sdst[q];
    d.ok = (uint32_t)e < (uint32_t)a.sh.E && (uint32_t)i < (uint32_t)a.sh.N;
    if (!d.ok) e = i = 0;
    d.e = e;
    d.i = i;
    const float* wrow = a.W + (int64_t)e * (dm.P * C);
    static_for<0, P>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        if constexpr (!((L1M >> Tb::data.l1[p]) & 1)) {
            d.w[p] = 0.0f;  // another wave's path
        } else if constexpr (SUB) {
            const float v = __builtin_nontemporal_load(at_lane(wrow + a.sh.woff[p], chl));
            d.w[p] = ((a.sh.active >> p) & 1) ? v : 0.0f;
        } else {
            d.w[p] = __builtin_nontemporal_load(at_lane(wrow + p * C, chl));
        }
    });
    if constexpr (LOADG) {
        const float* grow = a.G + (int64_t)i * (dm.d_out * C);
        static_for<0, DOUT>([&](auto K) { d.g[K] = *at_lane(grow + Dims<Tb, SUB>::template comp<decltype(K)::value>(dm.d_out) * C, chl); });
    }
    if constexpr (FSH) {
        const float* rp = a.r + 3 * (int64_t)e;
#pragma unroll
        for (int k = 0; k < 3; ++k) d.r[k] = UNI ? scalar_load(rp + k) : rp[k];
    } else {
        const float* yp = a.Y + (int64_t)e * dm.d_sh;
        static_for<0, DSH>([&](auto K) {
            const float* p = yp + Dims<Tb, SUB>::template comp<decltype(K)::value>(dm.d_sh);
            d.y[K] = UNI ? scalar_load(p) : *p;
        });
    }
}

// One edge of the backward for one channel:
//   R_p[a][b] = sum_m3 T_p[a][b][m3] g[l3,m3]
//   h_p[a] = sum_b R_p[a][b] y[l2,b]   -> dx[l1,a] += W_p h_p[a], dW_p = sum_a x[l1,a] h_p[a]
//   v_p[b] = sum_a R_p[a][b] x[l1,a]   -> dy[l2,b] += W_p v_p[b]
// The paths are taken grouped by l2, so only one degree's grad_Y partials
// are live at a time; flush_y(k2, dy) receives each degree's partials
// (components k2 .. k2+2*l2) as soon as its last path is done.  store_w(p, v)
// receives grad_W of path p.  Only the paths whose l1 is in the mask L1M are
// taken (path-group split: the other paths belong to another wave).
template <class Tb, int L1M = 0xF, class StoreW, class FlushY>
__device__ __forceinline__ void bwd_slice(const float (&w)[Tb::P], const float (&g)[Tb::DOUT],
                                          const double (&yv)[Tb::DSH], const double (&xv)[Tb::DIN],
                                          double (&dxa)[Tb::DIN], StoreW&& store_w, FlushY&& flush_y)
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
            bool dys[d2];
#pragma unroll
            for (int b = 0; b < d2; ++b) {
                dyb[b] = 0.0;
                dys[b] = false;
            }
            static_for<0, Tb::P>([&](auto PI) {
                constexpr int p = decltype(PI)::value;
                using K = PathK<Tb, p>;
                if constexpr (K::l2 == l2 && ((L1M >> K::l1) & 1)) {
                    const double wd = (double)w[p];
                    static_for<0, K::d3>([&](auto M3) { opaque(gv[K::k3 + decltype(M3)::value]); });
                    const PathCoefs<Tb, p> cf;
                    double v[d2];
                    bool vs[d2];
                    static_for<0, d2>([&](auto B) {
                        v[decltype(B)::value] = 0.0;
                        vs[decltype(B)::value] = false;
                    });
                    double dw = 0.0;
                    bool dws = false;
                    static_for<0, K::d1>([&](auto A) {
                        constexpr int a = decltype(A)::value;
                        if constexpr (K::ROW(a)) {
                            double h = 0.0;
                            bool hs = false;
                            static_for<0, d2>([&](auto B) {
                                constexpr int b = decltype(B)::value;
                                double r = 0.0;
                                bool any = false;
                                static_for<0, K::d3>([&](auto M3) {
                                    constexpr int m3 = decltype(M3)::value;
                                    constexpr double t = K::T(a, b, m3);
                                    if constexpr (t != 0.0) cf.template mac<a, b, m3>(r, gv[K::k3 + m3], any);
                                });
                                if (any) {
                                    mac(h, r, yv[k2 + b], hs);
                                    mac(v[b], r, xv[K::k1 + a], vs[b]);
                                }
                            });
                            dxa[K::k1 + a] = __builtin_fma(wd, h, dxa[K::k1 + a]);
                            mac(dw, xv[K::k1 + a], h, dws);
                        }
                    });
                    store_w(std::integral_constant<int, p>{}, dw);
                    static_for<0, d2>([&](auto B) {
                        constexpr int b = decltype(B)::value;
                        if constexpr (K::COL2(b)) mac(dyb[b], wd, v[b], dys[b]);
                    });
                    // Pin this path's accumulator updates here: without it the
                    // compiler sinks every accumulation to the end of the edge
                    // and keeps all paths' h and v values live at once.
                    static_for<0, K::d1>([&](auto A) {
                        if constexpr (K::ROW(decltype(A)::value)) opaque(dxa[K::k1 + decltype(A)::value]);
                    });
                    static_for<0, d2>([&](auto B) {
                        if constexpr (K::COL2(decltype(B)::value)) opaque(dyb[decltype(B)::value]);
                    });
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
            flush_y(std::integral_constant<int, k2>{}, dyb);
        }
    });
}

// ---- double backward, sender side -------------------------------------------
// The gradients of S = <ggx, grad_x> + <ggW, grad_W> + <ggY, grad_Y> with
// respect to x, W and Y, for one edge and channel, with R_p as in bwd_slice:
//   h_p = R_p y,  k_p = R_p ggy
//   d_x[l1,a] += W_p k_p[a] + ggW_p h_p[a]
//   d_W_p      = sum_a ggx[l1,a] h_p[a] + x[l1,a] k_p[a]
//   d_y[l2,b] += sum_a R_p[a][b] (W_p ggx[l1,a] + ggW_p x[l1,a])
// They run on the backward's work decomposition with these operands added.
template <class Tb>
struct BwdEdgeD : BwdEdge<Tb> {
    float gw[Tb::P], gy[Tb::DSH];
};

template <class Tb, bool SUB, bool UNI, int L1M = 0xF>
__device__ __forceinline__ void bwd_load_dbl(BwdEdgeD<Tb>& d, int32_t q, uint32_t chl, const BwdArgs& a,
                                             const Dims<Tb, SUB>& dm)
{
    bwd_load<Tb, SUB, UNI, true, false, L1M>(d, q, chl, a, dm);
    constexpr int P = Tb::P, DSH = Tb::DSH;
    const int32_t C = edge_stride(a.sh.C);
    chl = lane_offset(chl);
    const int32_t e = d.e;
    if (a.ggW) {
        const float* wrow = a.ggW + (int64_t)e * (dm.P * C);
        static_for<0, P>([&](auto PI) {
            constexpr int p = decltype(PI)::value;
            if constexpr (!((L1M >> Tb::data.l1[p]) & 1)) {
                d.gw[p] = 0.0f;  // another wave's path
            } else if constexpr (SUB) {
                const float v = __builtin_nontemporal_load(at_lane(wrow + a.sh.woff[p], chl));
                d.gw[p] = ((a.sh.active >> p) & 1) ? v : 0.0f;
            } else {
                d.gw[p] = __builtin_nontemporal_load(at_lane(wrow + p * C, chl));
            }
        });
    } else {
#pragma unroll
        for (int p = 0; p < P; ++p) d.gw[p] = 0.0f;
    }
    if (a.ggY) {
        const float* yp = a.ggY + (int64_t)e * dm.d_sh;
        static_for<0, DSH>([&](auto K) {
            const float* p = yp + Dims<Tb, SUB>::template comp<decltype(K)::value>(dm.d_sh);
            d.gy[K] = UNI ? scalar_load(p) : *p;
        });
    } else {
#pragma unroll
        for (int k = 0; k < DSH; ++k) d.gy[k] = 0.0f;
    }
}

template <class Tb, int L1M = 0xF, class StoreW, class FlushY>
__device__ __forceinline__ void bwd_slice_dbl(const BwdEdgeD<Tb>& d, const double (&yv)[Tb::DSH],
                                              const double (&gyv)[Tb::DSH], const double (&xv)[Tb::DIN],
                                              const double (&gxv)[Tb::DIN], double (&dxa)[Tb::DIN],
                                              StoreW&& store_w, FlushY&& flush_y)
{
    constexpr int DOUT = Tb::DOUT;
    double gv[DOUT];
#pragma unroll
    for (int k = 0; k < DOUT; ++k) gv[k] = (double)d.g[k];
    static_for<0, 4>([&](auto L2I) {
        constexpr int l2 = decltype(L2I)::value;
        constexpr int d2 = 2 * l2 + 1, k2 = l2 * l2;
        if constexpr ((l2 + 1) * (l2 + 1) <= Tb::DSH) {
            double dyb[d2];
            bool dys[d2];
#pragma unroll
            for (int b = 0; b < d2; ++b) {
                dyb[b] = 0.0;
                dys[b] = false;
            }
            static_for<0, Tb::P>([&](auto PI) {
                constexpr int p = decltype(PI)::value;
                using K = PathK<Tb, p>;
                if constexpr (K::l2 == l2 && ((L1M >> K::l1) & 1)) {
                    const double wd = (double)d.w[p], gwd = (double)d.gw[p];
                    static_for<0, K::d3>([&](auto M3) { opaque(gv[K::k3 + decltype(M3)::value]); });
                    const PathCoefs<Tb, p, true> cf;
                    double v[d2];
                    bool vs[d2];
                    static_for<0, d2>([&](auto B) {
                        v[decltype(B)::value] = 0.0;
                        vs[decltype(B)::value] = false;
                    });
                    double dw = 0.0;
                    bool dws = false;
                    static_for<0, K::d1>([&](auto A) {
                        constexpr int a = decltype(A)::value;
                        if constexpr (K::ROW(a)) {
                            const double xm = __builtin_fma(gwd, xv[K::k1 + a], wd * gxv[K::k1 + a]);
                            double h = 0.0, k = 0.0;
                            bool hs = false, ks = false;
                            static_for<0, d2>([&](auto B) {
                                constexpr int b = decltype(B)::value;
                                double r = 0.0;
                                bool any = false;
                                static_for<0, K::d3>([&](auto M3) {
                                    constexpr int m3 = decltype(M3)::value;
                                    constexpr double t = K::T(a, b, m3);
                                    if constexpr (t != 0.0) cf.template mac<a, b, m3>(r, gv[K::k3 + m3], any);
                                });
                                if (any) {
                                    mac(h, r, yv[k2 + b], hs);
                                    mac(k, r, gyv[k2 + b], ks);
                                    mac(v[b], r, xm, vs[b]);
                                }
                            });
                            dxa[K::k1 + a] = __builtin_fma(wd, k, __builtin_fma(gwd, h, dxa[K::k1 + a]));
                            mac(dw, gxv[K::k1 + a], h, dws);
                            dw = __builtin_fma(xv[K::k1 + a], k, dw);
                        }
                    });
                    store_w(std::integral_constant<int, p>{}, dw);
                    static_for<0, d2>([&](auto B) {
                        constexpr int b = decltype(B)::value;
                        if constexpr (K::COL2(b)) {
                            dyb[b] = dys[b] ? dyb[b] + v[b] : v[b];
                            dys[b] = true;
                        }
                    });
                    static_for<0, K::d1>([&](auto A) {
                        if constexpr (K::ROW(decltype(A)::value)) opaque(dxa[K::k1 + decltype(A)::value]);
                    });
                    static_for<0, d2>([&](auto B) {
                        if constexpr (K::COL2(decltype(B)::value)) opaque(dyb[decltype(B)::value]);
                    });
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
            flush_y(std::integral_constant<int, k2>{}, dyb);
        }
    });
}

// ---- per-path outputs, sender side ------------------------------------------
// The backward of the per-path-output forward: as bwd_slice, with path p's
// R_p formed from its own block of grad_out (rows moff[p] ..) instead of the
// l3 slot.  Those rows are gathered per path, some paths ahead of the one
// that uses them (kMidPrefetch), so their latency overlaps the arithmetic of
// the paths in between.
template <class Tb, int L1M = 0xF>
struct L2Order {
    struct O {
        int p[kMaxPaths];
        int n;
    };
    // the paths whose l1 is in L1M, grouped by l2
    static constexpr O make()
    {
        O o{};
        int k = 0;
        for (int l2 = 0; l2 < 4; ++l2)
            for (int p = 0; p < Tb::P; ++p)
                if (Tb::data.l2[p] == l2 && ((L1M >> Tb::data.l1[p]) & 1)) o.p[k++] = p;
        o.n = k;
        return o;
    }
    static constexpr O ord = make();
    static constexpr int N = ord.n;
};

// paths a per-path backward loads grad_out rows ahead (degree 3 holds up to
// 156 rows per edge and has no registers to spare)
template <class Tb>
constexpr int kMidPrefetch = Tb::DIN <= 9 ? 4 : 1;

template <class Tb, int p>
__device__ __forceinline__ void load_mid_rows(float (&g)[7], const float* grow, int32_t Cs, uint32_t chl,
                                              const Shape& sh)
{
    constexpr int d3 = 2 * Tb::data.l3[p] + 1;
    // a path the plan lacks reads the node's first rows (its weight is 0);
    // every row index stays inside the node's d_out rows
    const int32_t r0 = sh.moff[p] >= 0 ? sh.moff[p] : 0;
#pragma unroll
    for (int m = 0; m < d3; ++m) {
        const int32_t r = r0 + m < sh.d_out ? r0 + m : sh.d_out - 1;
        g[m] = *at_lane(grow + r * Cs, chl);
    }
}

template <class Tb, int L1M = 0xF, class StoreW, class FlushY>
__device__ __forceinline__ void bwd_slice_mid(const float (&w)[Tb::P], const float* grow, int32_t Cs, uint32_t chl,
                                              const Shape& sh, const double (&yv)[Tb::DSH],
                                              const double (&xv)[Tb::DIN], double (&dxa)[Tb::DIN],
                                              StoreW&& store_w, FlushY&& flush_y)
{
    // the paths whose l1 is in L1M (path-group split), grouped by l2; a degree
    // l2 none of them has gets no grad_Y partials from this wave (zeros below)
    using Ord = L2Order<Tb, L1M>;
    constexpr int NP = Ord::N;
    static_for<0, 4>([&](auto L2I) {
        constexpr int l2 = decltype(L2I)::value;
        constexpr bool has = [] {
            for (int k = 0; k < NP; ++k)
                if (Tb::data.l2[Ord::ord.p[k]] == l2) return true;
            return false;
        }();
        if constexpr (!has && (l2 + 1) * (l2 + 1) <= Tb::DSH) {
            double out[2 * l2 + 1];
#pragma unroll
            for (int b = 0; b < 2 * l2 + 1; ++b) out[b] = 0.0;
            flush_y(std::integral_constant<int, l2 * l2>{}, out);
        }
    });
    // rows of path k are loaded PD paths ahead of its computation (every
    // path's gather would otherwise wait out its own latency)
    constexpr int PD = kMidPrefetch<Tb>;
    float gb[NP][7];
    static_for<0, (PD < NP ? PD : NP)>([&](auto KI) {
        constexpr int k = decltype(KI)::value;
        load_mid_rows<Tb, Ord::ord.p[k]>(gb[k], grow, Cs, chl, sh);
    });
    double dyb[7];
    bool dys[7];
    static_for<0, NP>([&](auto KI) {
        constexpr int k = decltype(KI)::value;
        constexpr int p = Ord::ord.p[k];
        const float(&gcur)[7] = gb[k];
        using K = PathK<Tb, p>;
        constexpr int l2 = K::l2, d2 = 2 * l2 + 1, k2 = l2 * l2;
        constexpr bool first = k == 0 || Tb::data.l2[Ord::ord.p[k > 0 ? k - 1 : 0]] != l2;
        constexpr bool last = k + 1 == NP || Tb::data.l2[Ord::ord.p[k + 1 < NP ? k + 1 : k]] != l2;
        if constexpr (first) {
#pragma unroll
            for (int b = 0; b < 7; ++b) {
                dyb[b] = 0.0;
                dys[b] = false;
            }
        }
        if constexpr (k + PD < NP) load_mid_rows<Tb, Ord::ord.p[k + PD < NP ? k + PD : k]>(gb[k + PD < NP ? k + PD : k], grow, Cs, chl, sh);
        const double wd = (double)w[p];
        double gv[K::d3];
#pragma unroll
        for (int m = 0; m < K::d3; ++m) gv[m] = (double)gcur[m];
        double v[d2];
        bool vs[d2];
        static_for<0, d2>([&](auto B) {
            v[decltype(B)::value] = 0.0;
            vs[decltype(B)::value] = false;
        });
        double dw = 0.0;
        bool dws = false;
        static_for<0, K::d1>([&](auto A) {
            constexpr int a = decltype(A)::value;
            if constexpr (K::ROW(a)) {
                double h = 0.0;
                bool hs = false;
                static_for<0, d2>([&](auto B) {
                    constexpr int b = decltype(B)::value;
                    double r = 0.0;
                    bool any = false;
                    static_for<0, K::d3>([&](auto M3) {
                        constexpr int m3 = decltype(M3)::value;
                        constexpr double t = K::T(a, b, m3);
                        if constexpr (t != 0.0) mac(r, t, gv[m3], any);
                    });
                    if (any) {
                        mac(h, r, yv[k2 + b], hs);
                        mac(v[b], r, xv[K::k1 + a], vs[b]);
                    }
                });
                dxa[K::k1 + a] = __builtin_fma(wd, h, dxa[K::k1 + a]);
                mac(dw, xv[K::k1 + a], h, dws);
            }
        });
        store_w(std::integral_constant<int, p>{}, dw);
        static_for<0, d2>([&](auto B) {
            constexpr int b = decltype(B)::value;
            if constexpr (K::COL2(b)) mac(dyb[b], wd, v[b], dys[b]);
        });
        static_for<0, K::d1>([&](auto A) {
            if constexpr (K::ROW(decltype(A)::value)) opaque(dxa[K::k1 + decltype(A)::value]);
        });
        static_for<0, d2>([&](auto B) {
            if constexpr (K::COL2(decltype(B)::value)) opaque(dyb[decltype(B)::value]);
        });
        if constexpr (last) {
            double out[d2];
#pragma unroll
            for (int b = 0; b < d2; ++b) out[b] = dys[b] ? dyb[b] : 0.0;
            flush_y(std::integral_constant<int, k2>{}, out);
        }
        __builtin_amdgcn_sched_barrier(0);
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

// Order this wave's LDS writes before its lanes read what other lanes wrote
// (and, used again afterwards, the reads before the next overwrite).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum over the 64 lanes of a wave of the per-wave LDS tile red[D][64]
// (D <= 16; row k holds every lane's partial of component k, written by the
// caller): lane 4k+q adds red[k][16q .. 16q+15], and a quad exchange (DPP)
// completes the sum.  Returns the total of component lane/4 in lanes with
// lane%4 == 0.  The tile may be overwritten once this returns.
template <int D>
__device__ __forceinline__ double wave_sum_tile(const double* __restrict__ red, int lane)
{
    static_assert(D <= 16, "at most 16 components");
    wave_lds_sync();
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
    wave_lds_sync();
    s += dpp_quad<0xB1>(s);  // lanes ^1
    s += dpp_quad<0x4E>(s);  // lanes ^2
    return s;
}

// Edges per stream between two grad_Y combines of the two channel slices of
// a C > 64 backward block.
constexpr int kDyChunk = 64;

// fp64 value of lane `l` of the wave (l uniform)
__device__ __forceinline__ double readlane_d(double v, int l)
{
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
    return __hiloint2double(hi, lo);
}

// With FSH (the fused-SH backward) the kernel reads the edge vectors r
// instead of Y, evaluates the harmonics itself, and where the plain kernel
// stores an edge's grad_Y (once it is summed over the channels) it stores
// grad_r = sum_k grad_Y[k] dY_k/dr instead.
// Occupancy bound of a backward specialisation.  The fused-SH backward of a
// SUB plan at degree 2 with one full-wave slice per edge holds a few more
// scalar values than 4 waves per SIMD leave registers for (it would spill to
// memory), so it runs at 3.
template <int LM, int LPE, int H, bool SUB, bool DBL, bool FSH, bool PS = false>
constexpr int bwd_bound()
{
    if (PS) return DBL ? Tune<LM, LPE>::dbl_ps_bwd_occ : Tune<LM, LPE>::ps_bwd_occ;
    if (DBL) return Tune<LM, LPE>::dbl_bwd_occ;
    if (FSH && SUB && LM == 2 && LPE == 64 && H == 1) return 3;
    return Tune<LM, LPE>::bwd_occ;
}

// Path-group split of the backward (the path-group parallelism of the LunaTP
// abstract): with PS the two waves of a pair serve the same edge and the same
// 64 channels, each taking the paths of a set of input degrees l1 (l1 in
// {1, 2} and l1 in {0, 3} at degree 3, near equal halves of the work).  A
// wave then holds x and grad_x of its own degrees only and the weights of its
// own paths, which roughly halves its registers and raises occupancy; the
// two waves' grad_Y partials of an edge meet in LDS like the two channel
// slices of a C > 64 block.  The degree-3 backward with one slice per edge
// uses it, and so does the sender side of its double backward (which also
// holds the cotangent row ggx and ggW) unless the plan shares one weight over
// all paths: that grad_W sums every path, which the split spreads over two
// waves.

// LDS of a backward block: per-wave grad_Y transpose tiles and, with two
// waves per edge, the two waves' per-edge grad_Y sums of the current chunk
// [wave of the pair][stream][edge][k] during the edge loop; the streams'
// grad_x partials at the end
template <int LM, int LPE, int H, bool FSH, bool PS>
struct BwdLds {
    using Tb = cgmath::Tables<LM, LM, LM>;
    static constexpr int HW = PS ? 2 : H;  // waves per edge
    using Gm = Geo<LPE, HW>;
    static constexpr int DIN = Tb::DIN, DSH = Tb::DSH, S = Gm::S;
    static constexpr int CP = PS ? LPE : Gm::CP;  // padded channels of a node row
    // edges per stream between two grad_Y combines of a pair (smaller with
    // PS, so that three blocks fit a CU's LDS)
    static constexpr int K = PS ? kDyChunk / 2 : kDyChunk;
    static constexpr bool kTile = LPE == 64;
    static constexpr int kTiles = kTile ? 4 * DSH * 64 : 0;
    static constexpr int kDyl = HW == 2 ? 2 * S * K * DSH : 0;
    static constexpr int kDx = S * DIN * CP;
    static constexpr int kMain = kTiles + kDyl;
    static constexpr int kLds = kMain > kDx ? kMain : kDx;
    static constexpr int kEslot = HW == 2 ? S * K : 1;
    // FSH with LPE < 64: one grad_Y slot per edge a wave holds at a time (apart
    // from lds: the first waves to finish write their grad_x partials there)
    static constexpr int kStage = FSH && !kTile ? 4 * (64 / LPE) * DSH : 1;
};


// The backward of one block; the paths are those whose l1 is in L1M.
template <int LM, int LPE, int H, bool SUB, bool DBL, bool MID, bool FSH, bool PS, int L1M>
__device__ __forceinline__ void bwd_body(const BwdArgs& a, double* __restrict__ lds, int32_t* __restrict__ eslot,
                                         double* __restrict__ stage)
{
    static_assert(!(FSH && (DBL || MID)), "the fused-SH form is the plain backward's");
    static_assert(!PS || (LPE == 64 && H == 1), "path split: one 64-lane slice per edge");
    using Tb = cgmath::Tables<LM, LM, LM>;
    using Lz = BwdLds<LM, LPE, H, FSH, PS>;
    constexpr int HW = Lz::HW;
    constexpr int DIN = Tb::DIN, DSH = Tb::DSH, S = Lz::S, CP = Lz::CP;
    constexpr int K = Lz::K;
    constexpr bool kTile = Lz::kTile;
    constexpr int kTiles = Lz::kTiles;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const Pos<LPE, HW> ps(tid);
    const int ch = PS ? ps.cl : ps.channel();
    const int32_t C = a.sh.C, N = a.sh.N, E = a.sh.E;
    const bool live = ch < C;
    const uint32_t chl = live ? 4u * ch : 0u;  // byte offset of the lane's channel
    // every lane of this wave holds a channel below C (uniform)
    const bool full_c = C >= (PS ? 1 : ps.h + 1) * LPE;
    const Dims<Tb, SUB> dm(a.sh);
    // want_dy: grad_Y, or with FSH grad_r
    const bool want_dx = a.dx != nullptr, want_dw = a.dW != nullptr, want_dy = (FSH ? a.dr : a.dY) != nullptr;
    const int32_t j = a.g.sorder[blockIdx.x];
    if ((uint32_t)j >= (uint32_t)N) return;  // idle block (or an unprepared schedule)

    using Edge = std::conditional_t<DBL, BwdEdgeD<Tb>, BwdEdge<Tb>>;
    double xv[DIN], dxa[DIN];
    double gxv[DBL ? DIN : 1];  // the sender's cotangent row ggx[j] (double backward)
    {
        const float* xrow = a.x + (int64_t)j * (dm.d_in * C);
        static_for<0, DIN>([&](auto Kc) {
            constexpr int k = decltype(Kc)::value;
            if constexpr ((L1M >> degree_of(k)) & 1)
                xv[k] = (double)*at_lane(xrow + Dims<Tb, SUB>::template comp<k>(dm.d_in) * C, chl);
            else
                xv[k] = 0.0;  // another wave's degree: never read
            dxa[k] = 0.0;
        });
        if constexpr (DBL) {
            const float* grow = a.ggx ? a.ggx + (int64_t)j * (dm.d_in * C) : nullptr;
            static_for<0, DIN>([&](auto Kc) {
                constexpr int k = decltype(Kc)::value;
                if constexpr ((L1M >> degree_of(k)) & 1)
                    gxv[k] = grow ? (double)*at_lane(grow + Dims<Tb, SUB>::template comp<k>(dm.d_in) * C, chl) : 0.0;
                else
                    gxv[k] = 0.0;  // another wave's degree: never read
            });
        }
    }
    // the sender's range of the view, clamped to the view's bounds
    const int32_t q0 = clampi(a.g.srow[j], 0, E);
    const int32_t end = clampi(a.g.srow[j + 1], q0, E);
    const int32_t T = (end - q0 + S - 1) / S;  // edges per stream (block-uniform bound)
    double* tile = lds + (tid >> 6) * (DSH * 64);
    double* dyl = lds + kTiles;

    for (int32_t t0 = 0; t0 < T; t0 += (HW == 2 ? K : T)) {
        const int32_t t1 = HW == 2 ? (t0 + K < T ? t0 + K : T) : T;
        for (int32_t t = t0; t < t1; ++t) {
            const int32_t q = q0 + ps.s + S * t;
            if (q >= end) continue;  // uniform over the lanes of one edge
            Edge cur;
            if constexpr (DBL) bwd_load_dbl<Tb, SUB, LPE == 64, L1M>(cur, q, chl, a, dm);
            else bwd_load<Tb, SUB, LPE == 64, !MID, FSH, L1M>(cur, q, chl, a, dm);
            if constexpr (HW == 2)
                if (ps.h == 0 && lane == 0) eslot[ps.s * K + (t - t0)] = cur.ok ? cur.e : -1;
            if (!cur.ok) continue;
            double yv[DSH];
            if constexpr (FSH) edge_sh_r<LM, DSH, LPE>(cur.r, yv);
            else edge_sh<DSH, LPE>(cur.y, yv);
            double gyv[DBL ? DSH : 1];
            if constexpr (DBL) edge_sh<DSH, LPE>(cur.gy, gyv);
            // the edge's contraction (the backward's, or the double backward's)
            auto slice = [&](auto&& store_w, auto&& flush_y) {
                if constexpr (DBL) {
                    bwd_slice_dbl<Tb, L1M>(cur, yv, gyv, xv, gxv, dxa, store_w, flush_y);
                } else if constexpr (MID) {
                    const int32_t Cg = edge_stride(C);
                    bwd_slice_mid<Tb, L1M>(cur.w, a.G + (int64_t)cur.i * (dm.d_out * Cg), Cg, lane_offset(chl), a.sh,
                                           yv, xv, dxa, store_w, flush_y);
                } else {
                    bwd_slice<Tb, L1M>(cur.w, cur.g, yv, xv, dxa, store_w, flush_y);
                }
            };
            const int32_t Ce = edge_stride(C);
            float* dwrow = a.dW + (int64_t)cur.e * (dm.P * Ce);
            const uint32_t chs = lane_offset(chl);
            double dwsum = 0.0;  // shared path weights: grad_W is the sum over the paths
            auto store_w = [&](auto PI, double dw) {
                constexpr int p = decltype(PI)::value;
                bool keep = want_dw && (full_c || live);
                if constexpr (SUB) {
                    keep = keep && ((a.sh.active >> p) & 1);
                    if (a.sh.shared) {
                        if (keep) dwsum += dw;
                        return;
                    }
                }
                if (keep) __builtin_nontemporal_store((float)dw, at_lane(dwrow + (SUB ? a.sh.woff[p] : p * Ce), chs));
            };
            auto store_shared = [&]() {
                if constexpr (SUB)
                    if (a.sh.shared && want_dw && (full_c || live))
                        __builtin_nontemporal_store((float)dwsum, at_lane(dwrow, chs));
            };
            if constexpr (kTile) {
                // grad_Y partials go to this wave's LDS tile degree by degree
                slice(store_w, [&](auto K2, const auto& dyb) {
                    constexpr int k2 = decltype(K2)::value;
#pragma unroll
                    for (int b = 0; b < (int)(sizeof(dyb) / sizeof(double)); ++b)
                        tile[(k2 + b) * 64 + lane] = dyb[b];
                });
                store_shared();
                // lanes past C hold channel 0's terms: they leave the sum
                if (!full_c && !live)
#pragma unroll
                    for (int k = 0; k < DSH; ++k) tile[k * 64 + lane] = 0.0;
                const double s = wave_sum_tile<DSH>(tile, lane);
                const int k = lane >> 2;
                if ((lane & 3) == 0 && k < DSH) {
                    if constexpr (HW == 1) {
                        if constexpr (!FSH)
                            if (want_dy && k < dm.d_sh) a.dY[(int64_t)cur.e * dm.d_sh + k] = (float)s;
                    } else {
                        dyl[((ps.h * S + ps.s) * K + (t - t0)) * DSH + k] = s;
                    }
                }
                if constexpr (FSH && HW == 1) {
                    // component k's sum sits in lane 4k: read degree by degree
                    // (uniform) straight into the SH Jacobian
                    if (want_dy) {
                        // r again (cached) rather than held through the contraction
                        const float* rp = a.r + 3 * (int64_t)cur.e;
                        double x, y, z, inv;
                        shf::unit(scalar_load(rp), scalar_load(rp + 1), scalar_load(rp + 2), x, y, z, inv);
                        double qx = 0.0, qy = 0.0, qz = 0.0;
                        static_for<1, LM + 1>([&](auto LI) {
                            constexpr int l = decltype(LI)::value;
                            double wl[2 * l + 1];
                            static_for<0, 2 * l + 1>([&](auto B) {
                                constexpr int kk = l * l + decltype(B)::value;
                                const double v = readlane_d(s, 4 * kk);
                                wl[decltype(B)::value] = kk < dm.d_sh ? v : 0.0;
                            });
                            shf::grad_degree<l>(x, y, z, wl, qx, qy, qz);
                        });
                        double g[3];
                        shf::tangent(x, y, z, inv, qx, qy, qz, g);
                        if (lane == 0) {
                            float* o = a.dr + 3 * (int64_t)cur.e;
                            o[0] = (float)g[0];
                            o[1] = (float)g[1];
                            o[2] = (float)g[2];
                        }
                    }
                }
            } else {
                // an edge spans LPE < 64 lanes: reduce each degree's partials over them
                float* yp = a.dY + (int64_t)cur.e * dm.d_sh;
                // FSH: the first lane of the edge keeps each degree's summed
                // grad_Y in its own LDS slot until the edge is done (it alone
                // writes and reads the slot), then applies the SH Jacobian
                double* slot = stage + ((tid >> 6) * (64 / LPE) + (lane / LPE)) * DSH;
                slice(store_w, [&](auto K2, const auto& dyb) {
                    constexpr int k2 = decltype(K2)::value;
#pragma unroll
                    for (int b = 0; b < (int)(sizeof(dyb) / sizeof(double)); ++b) {
                        double v = (full_c || live) ? dyb[b] : 0.0;  // lanes past C leave the sum
#pragma unroll
                        for (int off = 1; off < LPE; off <<= 1) v += __shfl_xor(v, off, 64);
                        if constexpr (FSH) {
                            if (ps.cl == 0) slot[k2 + b] = v;
                        } else if (want_dy && ps.cl == 0 && k2 + b < dm.d_sh) {
                            yp[k2 + b] = (float)v;
                        }
                    }
                });
                store_shared();
                if constexpr (FSH) {
                    if (want_dy && ps.cl == 0) {
                        // r again (cached) rather than held through the contraction
                        const float* rp = a.r + 3 * (int64_t)cur.e;
                        const float rv[3] = {rp[0], rp[1], rp[2]};
                        double g[3];
                        edge_r_grad<LM>(rv, slot, dm.d_sh, g);
                        float* o = a.dr + 3 * (int64_t)cur.e;
                        o[0] = (float)g[0];
                        o[1] = (float)g[1];
                        o[2] = (float)g[2];
                    }
                }
            }
        }
        if constexpr (HW == 2 && FSH) {
            // grad_r of the chunk's edges: grad_Y is the two slices' sums, added
            // in a fixed order, then the SH Jacobian (one thread per edge)
            __syncthreads();
            if (want_dy)
                for (int idx = tid; idx < S * K; idx += 256) {
                    const int s = idx / K, tt = idx % K;
                    const int32_t t = t0 + tt;
                    if (t >= t1 || q0 + s + S * t >= end) continue;
                    const int32_t e = eslot[s * K + tt];
                    if (e < 0) continue;
                    // the two slices' sums, into the first slice's entries
                    double* w = dyl + ((0 * S + s) * K + tt) * DSH;
#pragma unroll
                    for (int k = 0; k < DSH; ++k) w[k] += dyl[((1 * S + s) * K + tt) * DSH + k];
                    const float* rp = a.r + 3 * (int64_t)e;
                    const float rv[3] = {rp[0], rp[1], rp[2]};
                    double g[3];
                    edge_r_grad<LM>(rv, w, dm.d_sh, g);
                    float* o = a.dr + 3 * (int64_t)e;
                    o[0] = (float)g[0];
                    o[1] = (float)g[1];
                    o[2] = (float)g[2];
                }
            __syncthreads();
        } else if constexpr (HW == 2) {
            // grad_Y of the chunk's edges: the two slices' sums, added in a fixed order
            __syncthreads();
            if (want_dy)
                for (int idx = tid; idx < S * K * DSH; idx += 256) {
                    const int s = idx / (K * DSH), tt = (idx / DSH) % K, k = idx % DSH;
                    const int32_t t = t0 + tt;
                    if (t >= t1 || q0 + s + S * t >= end || k >= dm.d_sh) continue;
                    const int32_t e = eslot[s * K + tt];
                    if (e < 0) continue;
                    a.dY[(int64_t)e * dm.d_sh + k] =
                        (float)(dyl[((0 * S + s) * K + tt) * DSH + k] + dyl[((1 * S + s) * K + tt) * DSH + k]);
                }
            __syncthreads();
        }
    }
    if (want_dx) {
        // combine the streams in a fixed order; dx[j] has this block as its only writer
        if constexpr (kTile && HW == 1) __syncthreads();  // every wave is done with its grad_Y tile
        // (with the path split each wave writes the components of its degrees)
        static_for<0, DIN>([&](auto Kc) {
            constexpr int k = decltype(Kc)::value;
            if constexpr ((L1M >> degree_of(k)) & 1) lds[(ps.s * DIN + k) * CP + ch] = dxa[k];
        });
        __syncthreads();
        float* dp = a.dx + (int64_t)j * (dm.d_in * C);
        for (int t = tid; t < DIN * CP; t += 256) {
            const int k = t / CP, c = t % CP;
            if (k < dm.d_in && c < C) {
                double v = 0.0;
#pragma unroll
                for (int r = 0; r < S; ++r) v += lds[r * DIN * CP + t];
                dp[k * C + c] = (float)v;
            }
        }
    }
}

template <int LM, int LPE, int H, bool SUB, bool DBL = false, bool MID = false, bool FSH = false, bool PS = false>
__global__ void __launch_bounds__(256, (bwd_bound<LM, LPE, H, SUB, DBL, FSH, PS>()))
    k_conv_bwd(BwdArgs a)
{
    using Lz = BwdLds<LM, LPE, H, FSH, PS>;
    __shared__ double lds[Lz::kLds];
    __shared__ int32_t eslot[Lz::kEslot];
    __shared__ double stage[Lz::kStage];
    if constexpr (PS) {
        // the pair's first wave (even wave index) takes the l1 = 1, 2 paths
        if ((__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1) == 0)
            bwd_body<LM, LPE, H, SUB, DBL, MID, FSH, PS, kPsMask0>(a, lds, eslot, stage);
        else
            bwd_body<LM, LPE, H, SUB, DBL, MID, FSH, PS, kPsMask1>(a, lds, eslot, stage);
    } else {
        bwd_body<LM, LPE, H, SUB, DBL, MID, FSH, PS, 0xF>(a, lds, eslot, stage);
    }
}

template <int LM, int LPE, int H, bool SUB, bool DBL = false, bool MID = false, bool FSH = false, bool PS = false>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s)
{
    if (a.sh.N == 0) return hipSuccess;
    hipLaunchKernelGGL((k_conv_bwd<LM, LPE, H, SUB, DBL, MID, FSH, PS>), dim3((unsigned)conv_grid(a.sh.N)), dim3(256),
                       0, s, a);
    return hipGetLastError();
}

// A backward launch (plain, SUB, double backward, per-path or fused-SH form).
// At degree 3 with one 64-lane slice it is the path-split kernel, unless the
// plan shares one weight over all paths: that grad_W sums every path, which
// the split spreads over two waves.
template <int LM, int LPE, int H, bool SUB, bool DBL = false, bool MID = false, bool FSH = false>
hipError_t launch_bwd_any(const BwdArgs& a, hipStream_t s)
{
    if constexpr (LM == 3 && LPE == 64 && H == 1) {
        if constexpr (SUB)
            if (a.sh.shared) return launch_bwd<LM, LPE, H, SUB, DBL, MID, FSH, false>(a, s);
        return launch_bwd<LM, LPE, H, SUB, DBL, MID, FSH, true>(a, s);
    } else {
        return launch_bwd<LM, LPE, H, SUB, DBL, MID, FSH, false>(a, s);
    }
}

// The forward launchers of a lane geometry (backward fields null) and its
// backward launchers in two parts (other fields null): a geometry's kernels
// can be compiled in units that run in parallel.
template <int LM, int LPE, int H>
constexpr KernelSet make_set_fwd()
{
    KernelSet k{};
    k.lm = LM;
    k.lpe = LPE;
    k.h = H;
    k.fwd[0] = &launch_fwd<LM, LPE, H, false>;
    k.fwd[1] = &launch_fwd<LM, LPE, H, true>;
    k.fwd_dbl = &launch_fwd_dbl<LM, LPE, H>;
    k.fwd_mid = &launch_fwd_mid<LM, LPE, H>;
    k.fwd_sh[0] = &launch_fwd<LM, LPE, H, false, false, true>;
    k.fwd_sh[1] = &launch_fwd<LM, LPE, H, true, false, true>;
    return k;
}

// the backward launchers: the plain and fused-SH forms (part 1) and the
// double-backward and per-path forms (part 2)
template <int LM, int LPE, int H>
constexpr KernelSet make_set_bwd1()
{
    KernelSet k{};
    k.lm = LM;
    k.lpe = LPE;
    k.h = H;
    k.bwd[0] = &launch_bwd_any<LM, LPE, H, false>;
    k.bwd[1] = &launch_bwd_any<LM, LPE, H, true>;
    k.bwd_sh[0] = &launch_bwd_any<LM, LPE, H, false, false, false, true>;
    k.bwd_sh[1] = &launch_bwd_any<LM, LPE, H, true, false, false, true>;
    return k;
}

template <int LM, int LPE, int H>
constexpr KernelSet make_set_bwd2()
{
    KernelSet k{};
    k.lm = LM;
    k.lpe = LPE;
    k.h = H;
    k.bwd_dbl = &launch_bwd_any<LM, LPE, H, true, true>;
    k.bwd_mid = &launch_bwd_any<LM, LPE, H, true, false, true>;
    return k;
}

// the forward fields of f, the plain and fused-SH backward fields of b1 and
// the double-backward and per-path backward fields of b2
constexpr KernelSet merge_sets(const KernelSet& f, const KernelSet& b1, const KernelSet& b2)
{
    KernelSet k = f;
    k.bwd[0] = b1.bwd[0];
    k.bwd[1] = b1.bwd[1];
    k.bwd_sh[0] = b1.bwd_sh[0];
    k.bwd_sh[1] = b1.bwd_sh[1];
    k.bwd_dbl = b2.bwd_dbl;
    k.bwd_mid = b2.bwd_mid;
    return k;
}

template <int LM, int LPE, int H>
constexpr KernelSet make_set()
{
    return merge_sets(make_set_fwd<LM, LPE, H>(), make_set_bwd1<LM, LPE, H>(), make_set_bwd2<LM, LPE, H>());
}

template <int LM>
static bool copy_table(int path, double* dense)
{
    using Tb = cgmath::Tables<LM, LM, LM>;
    if (path < 0 || path >= Tb::P) return false;
    const int n = cgmath::path_size(cgmath::path_at(LM, LM, LM, path));
    for (int q = 0; q < n; ++q) dense[q] = Tb::data.T[Tb::data.off[path] + q];
    return true;
}

}  // namespace cgtp
