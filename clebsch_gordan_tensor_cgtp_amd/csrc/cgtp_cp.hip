// cgtp_cp.hip -- gfx950 kernels of the CP-decomposed tensor-product
// convolution ("Tensor Decomposition Networks for Accelerating Machine
// Learning Force Field Computations", authors' rebuttal to reviewer S6y1:
// Equation (3) and the gradients derived after it).
//
// The coupling of x (d1 components) and y (d2) into z (d3) is the rank-R
// product z = A (B^T x (.) C^T y), A [d3][R], B [d1][R], C [d2][R].  Over the
// graph, for edge e = j -> i and channel u with one weight W[e][u]:
//   out[i][:,u] = sum_e W[e][u] A (B^T x[j][:,u] (.) C^T Y[e])
// Because A is linear it is applied once per receiver, after the edge sum,
// and B^T x once per sender node, before it:
//   xb[j][r][u] = sum_k B[k][r] x[j][k][u]          (k_cp_proj_rows)
//   yc[e][r]    = sum_k C[k][r] Y[e][k]             (k_cp_proj_edge)
//   acc[i][r][u] = sum_e W[e][u] yc[e][r] xb[j][r][u],  out = A acc  (k_cp_fwd)
// The backward (gradients after Equation (3), with the edge weight and the
// channel sum) runs sender-centric over the prepared sender-sorted view, with
// ga[i][r][u] = sum_k A[k][r] G[i][k][u] projected once per receiver:
//   t[r]        = yc[e][r] ga[i][r][u]
//   dxb[j][r]  += W[e][u] t[r]          -> dx[j] = B dxb[j]
//   dW[e][u]    = sum_r xb[j][r][u] t[r]
//   dyc[e][r]   = sum_u W[e][u] xb[j][r][u] ga[i][r][u]  -> dY[e] = C dyc[e]
//                                                          (k_cp_bwd, k_cp_edge_back)
// Arithmetic is fp64, and so are the projected rows xb, ga, yc, dyc: the
// projection by A (or B) sums R terms of mixed sign, and an fp32 intermediate
// would be amplified by that cancellation beyond the accuracy of the exact
// path.
//
// Work decomposition: the rank is padded to RP in {16, 32, 64} (columns past
// R are zero).  A group of LPE lanes holds one node's channels (LPE = 16, 32,
// 64; for 64 < C <= 128 two waves share a node, H = 2); a wave holds 64/LPE
// nodes.  Each group walks its node's whole edge segment, so the per-node
// projection by A (forward) or B (backward) runs once per node and channel and
// no partial sums are combined across waves.  Nodes are taken in the order of
// the prepared schedule (longest segment first).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cgtp_cp.h"
#include "cgtp_kernels.h"

namespace cgtp {
namespace {

constexpr int kThreads = 256;

// ---- projections -----------------------------------------------------------
// Rank columns are handled in chunks of kChunk: a chunk's loads and
// arithmetic are scheduled together, so only one chunk's operands are live
// (the whole rank at once would not fit the registers at rank 64).
constexpr int kChunk = 16;
constexpr int kMaxD = 16;  // (l+1)^2 for l <= 3

// out[n][r][u] = sum_{k < D} M[k][r] in[n][k][u] for r < R, 0 for R <= r < RP
template <int RP>
__global__ void __launch_bounds__(kThreads) k_cp_proj_rows(int64_t rows, int32_t D, int32_t R, int32_t C,
                                                           const float* __restrict__ M, const float* __restrict__ in,
                                                           double* __restrict__ out)
{
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= rows * C) return;
    const int64_t n = t / C;
    const int32_t u = (int32_t)(t - n * C);
    const float* ip = in + n * D * C + u;
    double v[kMaxD];
#pragma unroll
    for (int k = 0; k < kMaxD; ++k) v[k] = k < D ? (double)ip[(int64_t)(k < D ? k : D - 1) * C] : 0.0;
    double* op = out + n * RP * C + u;
#pragma unroll
    for (int c0 = 0; c0 < RP; c0 += kChunk) {
#pragma unroll
        for (int r = c0; r < c0 + kChunk; ++r) {
            double acc = 0.0;
            const int rc = r < R ? r : R - 1;  // every read stays inside M
#pragma unroll
            for (int k = 0; k < kMaxD; ++k) {
                const int kc = k < D ? k : D - 1;
                const double m = (k < D && r < R) ? (double)M[(int64_t)kc * R + rc] : 0.0;
                acc = __builtin_fma(m, v[k], acc);
            }
            op[(int64_t)r * C] = acc;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// yc[e][r] = sum_{k < D} Cf[k][r] Y[e][k] (fp64), 0 for R <= r < RP
template <int RP>
__global__ void __launch_bounds__(kThreads) k_cp_proj_edge(int64_t E, int32_t D, int32_t R,
                                                           const float* __restrict__ Cf, const float* __restrict__ Y,
                                                           double* __restrict__ yc)
{
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= E * RP) return;
    const int64_t e = t / RP;
    const int32_t r = (int32_t)(t - e * RP);
    double s = 0.0;
    if (r < R)
        for (int32_t k = 0; k < D; ++k) s = __builtin_fma((double)Cf[(int64_t)k * R + r], (double)Y[e * D + k], s);
    yc[t] = s;
}

// dY[e][k] = sum_{h < H} sum_{r < R} Cf[k][r] dyc[e][h][r]
template <int RP>
__global__ void __launch_bounds__(kThreads) k_cp_edge_back(int64_t E, int32_t D, int32_t R, int32_t H,
                                                           const float* __restrict__ Cf,
                                                           const double* __restrict__ dyc, float* __restrict__ dY)
{
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= E * D) return;
    const int64_t e = t / D;
    const int32_t k = (int32_t)(t - e * D);
    double s = 0.0;
    for (int32_t h = 0; h < H; ++h) {
        const double* v = dyc + (e * H + h) * RP;
        for (int32_t r = 0; r < R; ++r) s = __builtin_fma((double)Cf[(int64_t)k * R + r], v[r], s);
    }
    dY[t] = (float)s;
}

// ---- lane geometry ---------------------------------------------------------
template <int LPE, int H>
struct CpGeo {
    static_assert(LPE == 16 || LPE == 32 || LPE == 64, "lanes per node");
    static_assert(H == 1 || (H == 2 && LPE == 64), "two waves per node only with full waves");
    static constexpr int G = 64 / LPE;                    // nodes per wave
    static constexpr int NPB = H == 2 ? 2 : 4 * G;       // nodes per block
};

// this thread's node slot in the block, channel slice and channel
template <int LPE, int H>
struct CpPos {
    int slot, h, ch, q;  // q: position inside the lane group
    __device__ __forceinline__ explicit CpPos(int tid)
    {
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        q = lane % LPE;
        if constexpr (H == 2) {
            h = wave & 1;
            slot = wave >> 1;
        } else {
            h = 0;
            slot = wave * CpGeo<LPE, H>::G + lane / LPE;
        }
        ch = h * 64 + q;
    }
};

// the largest of a per-group count over the wave's groups (wave-uniform)
template <int LPE>
__device__ __forceinline__ int32_t wave_max_groups(int32_t n)
{
#pragma unroll
    for (int off = LPE; off < 64; off <<= 1) {
        const int32_t o = __shfl_xor(n, off, 64);
        n = o > n ? o : n;
    }
    return n;
}

// Reduce-scatter of v[0..RP) over the LPE lanes of a group: each halving
// step sends half of the remaining values to the partner lane (offset O) and
// keeps the sum of the other half.  On return v[0 .. max(1, RP/LPE)) hold the
// group totals of components base, base+1, ... (lanes that differ only in the
// offsets left after the halving hold the same totals).  The order of the
// additions is fixed, so the result is reproducible.
template <int N, int O, int RP>
__device__ __forceinline__ void reduce_scatter(double (&v)[RP], int q, int& base)
{
    if constexpr (O > 0) {
        if constexpr (N > 1) {
            constexpr int Hh = N / 2;
            const bool up = (q & O) != 0;
#pragma unroll
            for (int k = 0; k < Hh; ++k) {
                const double send = up ? v[k] : v[k + Hh];
                const double keep = up ? v[k + Hh] : v[k];
                v[k] = keep + __shfl_xor(send, O, 64);
            }
            base += up ? Hh : 0;
            reduce_scatter<Hh, O / 2, RP>(v, q, base);
        } else {
            v[0] += __shfl_xor(v[0], O, 64);
            reduce_scatter<1, O / 2, RP>(v, q, base);
        }
    }
}

// Rank columns live in registers during one walk over a node's edges: RH =
// 32 with whole waves per node, 16 with smaller groups (whose per-lane
// addresses take more registers) and in the backward beyond rank 32 (where
// the pass sums of dx take registers too).  A larger padded rank walks the
// edges again for each further block of RH columns.
template <int RP, int LPE, bool BWD>
struct CpPass {
    static constexpr int LIM = LPE == 64 && !(BWD && RP > 32) ? 32 : 16;
    static constexpr int RH = RP < LIM ? RP : LIM;
    static constexpr int NP = RP / RH;
};

// ---- forward ---------------------------------------------------------------
template <int RP, int LPE, int H>
__global__ void __launch_bounds__(kThreads, 2) k_cp_fwd(CpFwdArgs a)
{
    using Gm = CpGeo<LPE, H>;
    constexpr int RH = CpPass<RP, LPE, false>::RH, NP = CpPass<RP, LPE, false>::NP;
    const CpPos<LPE, H> ps(threadIdx.x);
    const int32_t C = a.C, N = a.N, E = a.E;
    const bool live = ps.ch < C;
    const uint32_t chl = live ? 4u * ps.ch : 0u;
    const int64_t qn = (int64_t)blockIdx.x * Gm::NPB + ps.slot;
    const int32_t i = qn < a.n_order ? a.order[qn] : -1;
    const bool valid = (uint32_t)i < (uint32_t)N;
    int32_t e0 = 0, cnt = 0;
    if (valid) {
        e0 = clampi(a.row_ptr[i], 0, E);
        cnt = clampi(a.row_ptr[i + 1], e0, E) - e0;
    }
    int32_t n = cnt;
    if constexpr (Gm::G > 1) n = wave_max_groups<LPE>(cnt);
    const int32_t Cs = edge_stride(C);
    const int32_t d3 = a.d3;

    double outa[NP > 1 ? kMaxD : 1];  // out, summed over the passes
#pragma unroll
    for (int k = 0; k < (NP > 1 ? kMaxD : 1); ++k) outa[k] = 0.0;
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int r0 = pass * RH;
        double acc[RH];
#pragma unroll
        for (int r = 0; r < RH; ++r) acc[r] = 0.0;
        for (int32_t t = 0; t < n; ++t) {
            if (t < cnt) {
                const int32_t e = e0 + t;
                int32_t j = LPE == 64 ? scalar_load(a.src + e) : a.src[e];
                j = (uint32_t)j < (uint32_t)N ? j : 0;  // a sender outside [0, N) breaks the CSR contract
                const uint32_t lo = lane_offset(chl);
                const double w = (double)__builtin_nontemporal_load(at_lane(a.W + (int64_t)e * Cs, lo));
                const double* xr = a.xb + (int64_t)j * (RP * Cs);
                const double* yr = a.yc + (int64_t)e * RP;
#pragma unroll
                for (int c0 = 0; c0 < RH; c0 += kChunk) {
#pragma unroll
                    for (int r = c0; r < c0 + kChunk; ++r) {
                        const double y = LPE == 64 ? scalar_load(yr + r0 + r) : yr[r0 + r];
                        acc[r] = __builtin_fma(w * y, *at_lane(xr + (r0 + r) * Cs, 2 * lo), acc[r]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if (!valid) continue;
        // out[i][k][u] (+)= sum_r A[k][r] acc[r] over this pass's columns
        float* op = a.out + (int64_t)i * d3 * C;
#pragma unroll
        for (int k = 0; k < kMaxD; ++k) {
            if (k < d3) {
                const float* ar = a.A + (int64_t)(k < d3 ? k : d3 - 1) * a.R;
                double s = 0.0;
#pragma unroll
                for (int r = 0; r < RH; ++r) {
                    const int rc = r0 + r < a.R ? r0 + r : a.R - 1;  // every read stays inside A
                    const double m = r0 + r < a.R ? (double)ar[rc] : 0.0;
                    s = __builtin_fma(m, acc[r], s);
                }
                if constexpr (NP > 1) {
                    outa[k] += s;
                } else if (live) {
                    op[k * C + ps.ch] = (float)s;
                }
            }
        }
    }
    if constexpr (NP > 1) {
        if (valid && live) {
            float* op = a.out + (int64_t)i * d3 * C;
#pragma unroll
            for (int k = 0; k < kMaxD; ++k)
                if (k < d3) op[k * C + ps.ch] = (float)outa[k];
        }
    }
}

// ---- backward --------------------------------------------------------------
template <int RP, int LPE, int H>
__global__ void __launch_bounds__(kThreads, 2) k_cp_bwd(CpBwdArgs a)
{
    using Gm = CpGeo<LPE, H>;
    constexpr int RH = CpPass<RP, LPE, true>::RH, NP = CpPass<RP, LPE, true>::NP;
    const CpPos<LPE, H> ps(threadIdx.x);
    const int32_t C = a.C, N = a.N, E = a.E;
    const bool live = ps.ch < C;
    const uint32_t chl = live ? 4u * ps.ch : 0u;
    const int64_t qn = (int64_t)blockIdx.x * Gm::NPB + ps.slot;
    const int32_t j = qn < a.n_order ? a.order[qn] : -1;
    const bool valid = (uint32_t)j < (uint32_t)N;
    int32_t q0 = 0, cnt = 0;
    if (valid) {
        q0 = clampi(a.srow[j], 0, E);
        cnt = clampi(a.srow[j + 1], q0, E) - q0;
    }
    int32_t n = cnt;
    if constexpr (Gm::G > 1) n = wave_max_groups<LPE>(cnt);
    const int32_t Cs = edge_stride(C);
    const int32_t d1 = a.d1;
    const bool want_dw = a.dW != nullptr, want_dy = a.dyc != nullptr;
    const double* xrow = a.xb + (int64_t)(valid ? j : 0) * (RP * Cs);

    double dxa[NP > 1 ? kMaxD : 1];  // dx, summed over the passes
#pragma unroll
    for (int k = 0; k < (NP > 1 ? kMaxD : 1); ++k) dxa[k] = 0.0;
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int r0 = pass * RH;
        // gradients of this pass's columns of the sender's projected row (the
        // row itself is re-read per edge: it stays in the vector cache)
        double dxb[RH];
#pragma unroll
        for (int r = 0; r < RH; ++r) dxb[r] = 0.0;
        for (int32_t t = 0; t < n; ++t) {
            if (t < cnt) {
                const int32_t qv = q0 + t;
                int32_t e = LPE == 64 ? scalar_load(a.perm + qv) : a.perm[qv];
                int32_t i = LPE == 64 ? scalar_load(a.sdst + qv) : a.sdst[qv];
                const bool ok = (uint32_t)e < (uint32_t)E && (uint32_t)i < (uint32_t)N;
                if (!ok) e = i = 0;  // a corrupt view entry is read as edge 0 and contributes nothing
                const uint32_t lo = lane_offset(chl);
                const double w = ok ? (double)__builtin_nontemporal_load(at_lane(a.W + (int64_t)e * Cs, lo)) : 0.0;
                const double* gr = a.ga + (int64_t)i * (RP * Cs);
                const double* yr = a.yc + (int64_t)e * RP;
                double* dp = a.dyc + ((int64_t)e * H + ps.h) * RP + r0;
                double dw = 0.0;
#pragma unroll
                for (int c0 = 0; c0 < RH; c0 += kChunk) {
                    double pv[kChunk];
#pragma unroll
                    for (int r = c0; r < c0 + kChunk; ++r) {
                        const double y = LPE == 64 ? scalar_load(yr + r0 + r) : yr[r0 + r];
                        const double g = *at_lane(gr + (r0 + r) * Cs, 2 * lo);
                        const double x = *at_lane(xrow + (r0 + r) * Cs, 2 * lo);
                        const double tt = y * g;
                        dxb[r] = __builtin_fma(w, tt, dxb[r]);
                        dw = __builtin_fma(x, tt, dw);
                        pv[r - c0] = live ? w * (x * g) : 0.0;  // lanes past C leave the channel sum
                    }
                    if (want_dy) {
                        // the chunk's channel sums, reduce-scattered over the group
                        int base = 0;
                        reduce_scatter<kChunk, LPE / 2, kChunk>(pv, ps.q, base);
                        constexpr int kDup = kChunk >= LPE ? 1 : LPE / kChunk;  // lanes holding the same total
                        constexpr int kOut = kChunk >= LPE ? kChunk / LPE : 1;
                        if (ok && (ps.q % kDup) == 0)
#pragma unroll
                            for (int k = 0; k < kOut; ++k) dp[c0 + base + k] = pv[k];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (ok && live && want_dw) {
                    if constexpr (NP > 1) {
                        // the passes' partial sums meet in fp64 in the workspace (same lane, same address)
                        double* ap = at_lane(a.dwa + (int64_t)e * Cs, 2 * lo);
                        if (pass > 0) dw += *ap;
                        if (pass + 1 < NP) *ap = dw;
                    }
                    if (pass + 1 == NP) __builtin_nontemporal_store((float)dw, at_lane(a.dW + (int64_t)e * Cs, lo));
                }
            }
        }
        if (!valid || a.dx == nullptr) continue;
        // dx[j][k][u] (+)= sum_r B[k][r] dxb[r] over this pass's columns
        float* dp = a.dx + (int64_t)j * d1 * C;
#pragma unroll
        for (int k = 0; k < kMaxD; ++k) {
            if (k < d1) {
                const float* br = a.B + (int64_t)(k < d1 ? k : d1 - 1) * a.R;
                double s = 0.0;
#pragma unroll
                for (int r = 0; r < RH; ++r) {
                    const int rc = r0 + r < a.R ? r0 + r : a.R - 1;  // every read stays inside B
                    const double m = r0 + r < a.R ? (double)br[rc] : 0.0;
                    s = __builtin_fma(m, dxb[r], s);
                }
                if constexpr (NP > 1) {
                    dxa[k] += s;
                } else if (live) {
                    dp[k * C + ps.ch] = (float)s;
                }
            }
        }
    }
    if constexpr (NP > 1) {
        if (valid && live && a.dx != nullptr) {
            float* dp = a.dx + (int64_t)j * d1 * C;
#pragma unroll
            for (int k = 0; k < kMaxD; ++k)
                if (k < d1) dp[k * C + ps.ch] = (float)dxa[k];
        }
    }
}

// ---- launchers -------------------------------------------------------------
inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + kThreads - 1) / kThreads); }

template <int RP, int LPE, int H>
hipError_t launch_cp_fwd(const CpFwdArgs& a, hipStream_t s)
{
    const int64_t nb = (a.n_order + CpGeo<LPE, H>::NPB - 1) / CpGeo<LPE, H>::NPB;
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL((k_cp_fwd<RP, LPE, H>), dim3((unsigned)nb), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int RP, int LPE, int H>
hipError_t launch_cp_bwd(const CpBwdArgs& a, hipStream_t s)
{
    const int64_t nb = (a.n_order + CpGeo<LPE, H>::NPB - 1) / CpGeo<LPE, H>::NPB;
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL((k_cp_bwd<RP, LPE, H>), dim3((unsigned)nb), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int RP>
hipError_t launch_proj_rows(int64_t rows, int32_t D, int32_t R, int32_t C, const float* M, const float* in,
                            double* out, hipStream_t s)
{
    if (rows * C == 0) return hipSuccess;
    hipLaunchKernelGGL((k_cp_proj_rows<RP>), dim3(blocks_for(rows * C)), dim3(kThreads), 0, s, rows, D, R, C, M,
                       in, out);
    return hipGetLastError();
}

template <int RP>
hipError_t launch_proj_edge(int64_t E, int32_t D, int32_t R, const float* Cf, const float* Y, double* yc,
                            hipStream_t s)
{
    if (E == 0) return hipSuccess;
    hipLaunchKernelGGL((k_cp_proj_edge<RP>), dim3(blocks_for(E * RP)), dim3(kThreads), 0, s, E, D, R, Cf, Y, yc);
    return hipGetLastError();
}

template <int RP>
hipError_t launch_edge_back(int64_t E, int32_t D, int32_t R, int32_t H, const float* Cf, const double* dyc,
                            float* dY, hipStream_t s)
{
    if (E * D == 0) return hipSuccess;
    hipLaunchKernelGGL((k_cp_edge_back<RP>), dim3(blocks_for(E * D)), dim3(kThreads), 0, s, E, D, R, H, Cf, dyc,
                       dY);
    return hipGetLastError();
}

template <int RP, int LPE, int H>
constexpr CpKernelSet cp_set()
{
    return CpKernelSet{RP, LPE, H, &launch_cp_fwd<RP, LPE, H>, &launch_cp_bwd<RP, LPE, H>, &launch_proj_rows<RP>,
                       &launch_proj_edge<RP>, &launch_edge_back<RP>};
}

template <int RP>
const CpKernelSet* cp_for_channels(int C)
{
    static const CpKernelSet s16 = cp_set<RP, 16, 1>(), s32 = cp_set<RP, 32, 1>(), s64 = cp_set<RP, 64, 1>(),
                             s128 = cp_set<RP, 64, 2>();
    if (C <= 16) return &s16;
    if (C <= 32) return &s32;
    if (C <= 64) return &s64;
    if (C <= 128) return &s128;
    return nullptr;
}

}  // namespace

int cp_padded_rank(int R) { return R <= 16 ? 16 : (R <= 32 ? 32 : 64); }

const CpKernelSet* find_cp_kernels(int rank, int channels)
{
    if (rank < 1 || rank > kMaxCpRank || channels < 1) return nullptr;
    switch (cp_padded_rank(rank)) {
        case 16: return cp_for_channels<16>(channels);
        case 32: return cp_for_channels<32>(channels);
        default: return cp_for_channels<64>(channels);
    }
}

}  // namespace cgtp
