// cgtp_mix.hip -- the fully connected ("uvw") mixing of the per-path outputs
// on the fp64 matrix cores.
//
// The fully connected CG tensor product (the cost-dominating kernel of the
// "Tensor Decomposition Networks ..." rebuttal, reply to cmnz) couples every
// input channel with every output channel per path.  With weights shared over
// the edges it factors into the per-path-output convolution followed by one
// dense channel matrix per path:
//   out[i][k(l3,m)][w] = sum_{p: l3_p = l3} sum_u mid[i][o_p + m][u] Wmix[p][u][w]
// and its backward
//   d_mid[i][o_p + m][u] = sum_w G[i][k(l3_p,m)][w] Wmix[p][u][w]
//   d_Wmix[p][u][w]      = sum_i sum_m mid[i][o_p + m][u] G[i][k(l3_p,m)][w]
// All three are dense contractions, run as 16x16x4 fp64 MFMA tiles (fp32
// operands widened on load, fp64 accumulation).  A 256-thread block holds four
// waves; a wave owns 16 rows and 64 columns (four MFMA tiles sharing the row
// operand).  The weight gradient sums over all nodes: the node range is split
// over blocks, each writes its fp64 partial to the workspace, and a second
// kernel adds the partials in a fixed order.
//
// Lane layout of v_mfma_f64_16x16x4_f64 (checked on the device): A[i][k] in
// lane i + 16k, B[k][j] in lane j + 16k, D[i][j] in element r of lane l with
// i = 4r + l/16, j = l%16.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cgtp_internal.h"
#include "cgtp_mix.h"

namespace cgtp {
namespace {

typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kRows = 16, kCols = 64, kWaves = 4;

__device__ __forceinline__ int32_t clamp_idx(int32_t v, int32_t n) { return v < n ? v : n - 1; }

// degree of output slot s (s in [l*l, (l+1)*(l+1)))
__device__ __forceinline__ int32_t slot_degree(int32_t s)
{
    int32_t l = 0;
    while ((l + 1) * (l + 1) <= s) ++l;
    return l;
}

// out[i][s][w] for the block's 64 nodes x 64 output channels of slot s
__global__ void __launch_bounds__(256) k_mix_fwd(MixShape m, const float* __restrict__ mid,
                                                 const float* __restrict__ Wmix, float* __restrict__ out)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t n0 = (int32_t)blockIdx.x * (kRows * kWaves) + kRows * wave;
    const int32_t c0 = (int32_t)blockIdx.y * kCols;
    const int32_t s = (int32_t)blockIdx.z;
    const int32_t l3 = slot_degree(s), mm = s - l3 * l3;
    const int i = lane % 16, kk = lane / 16;
    const int32_t node = n0 + i, nodec = clamp_idx(node, m.N);
    v4d acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4d{0.0, 0.0, 0.0, 0.0};
    for (int32_t p = 0; p < m.P; ++p) {
        if (m.l3[p] != l3) continue;
        const float* arow = mid + ((int64_t)nodec * m.Dmid + m.o[p] + mm) * m.C;
        const float* wp = Wmix + (int64_t)p * m.C * m.Co;
        for (int32_t u0 = 0; u0 < m.C; u0 += 4) {
            const int32_t u = u0 + kk, uc = clamp_idx(u, m.C);
            const double a = (node < m.N && u < m.C) ? (double)arow[uc] : 0.0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int32_t col = c0 + 16 * t + i;
                const double b = (u < m.C && col < m.Co) ? (double)wp[(int64_t)uc * m.Co + clamp_idx(col, m.Co)] : 0.0;
                acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[t], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int32_t nd = n0 + 4 * r + kk, col = c0 + 16 * t + i;
            if (nd < m.N && col < m.Co) out[((int64_t)nd * m.Dout + s) * m.Co + col] = (float)acc[t][r];
        }
}

// d_mid[i][row][u] for the block's 64 nodes x 64 input channels of per-path row `row`
__global__ void __launch_bounds__(256) k_mix_bwd_data(MixShape m, const float* __restrict__ G,
                                                      const float* __restrict__ Wmix, float* __restrict__ dmid)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t n0 = (int32_t)blockIdx.x * (kRows * kWaves) + kRows * wave;
    const int32_t c0 = (int32_t)blockIdx.y * kCols;
    const int32_t row = (int32_t)blockIdx.z;
    int32_t p = 0;
    while (p + 1 < m.P && m.o[p + 1] <= row) ++p;
    const int32_t s = m.l3[p] * m.l3[p] + (row - m.o[p]);
    const int i = lane % 16, kk = lane / 16;
    const int32_t node = n0 + i, nodec = clamp_idx(node, m.N);
    const float* grow = G + ((int64_t)nodec * m.Dout + s) * m.Co;
    const float* wp = Wmix + (int64_t)p * m.C * m.Co;
    v4d acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4d{0.0, 0.0, 0.0, 0.0};
    for (int32_t w0 = 0; w0 < m.Co; w0 += 4) {
        const int32_t w = w0 + kk, wc = clamp_idx(w, m.Co);
        const double a = (node < m.N && w < m.Co) ? (double)grow[wc] : 0.0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int32_t u = c0 + 16 * t + i;
            const double b = (w < m.Co && u < m.C) ? (double)wp[(int64_t)clamp_idx(u, m.C) * m.Co + wc] : 0.0;
            acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[t], 0, 0, 0);
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int32_t nd = n0 + 4 * r + kk, u = c0 + 16 * t + i;
            if (nd < m.N && u < m.C) dmid[((int64_t)nd * m.Dmid + row) * m.C + u] = (float)acc[t][r];
        }
}

// part[sp][p][u][w]: path p's weight gradient over the nodes of split sp
__global__ void __launch_bounds__(256) k_mix_bwd_weight(MixShape m, int32_t nsplit, int32_t chunk,
                                                        const float* __restrict__ mid, const float* __restrict__ G,
                                                        double* __restrict__ part)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t r0 = (int32_t)blockIdx.x * (kRows * kWaves) + kRows * wave;  // input channels u
    const int32_t c0 = (int32_t)blockIdx.y * kCols;                             // output channels w
    const int32_t p = (int32_t)blockIdx.z / nsplit, sp = (int32_t)blockIdx.z % nsplit;
    const int32_t nb = sp * chunk, ne = nb + chunk < m.N ? nb + chunk : m.N;
    const int i = lane % 16, kk = lane / 16;
    const int32_t u = r0 + i, uc = clamp_idx(u, m.C);
    const int32_t d3 = 2 * m.l3[p] + 1, s0 = m.l3[p] * m.l3[p];
    v4d acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4d{0.0, 0.0, 0.0, 0.0};
    for (int32_t mm = 0; mm < d3; ++mm) {
        for (int32_t i0 = nb; i0 < ne; i0 += 4) {
            const int32_t node = i0 + kk, nodec = clamp_idx(node, m.N);
            const bool in = node < ne;
            const double a = (in && u < m.C) ? (double)mid[((int64_t)nodec * m.Dmid + m.o[p] + mm) * m.C + uc] : 0.0;
            const float* grow = G + ((int64_t)nodec * m.Dout + s0 + mm) * m.Co;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int32_t col = c0 + 16 * t + i;
                const double b = (in && col < m.Co) ? (double)grow[clamp_idx(col, m.Co)] : 0.0;
                acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[t], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int32_t uu = r0 + 4 * r + kk, col = c0 + 16 * t + i;
            if (uu < m.C && col < m.Co) part[(((int64_t)sp * m.P + p) * m.C + uu) * m.Co + col] = acc[t][r];
        }
}

// dWmix[p][u][w] = sum over the splits, in order
__global__ void __launch_bounds__(256) k_mix_reduce(int64_t n, int32_t nsplit, const double* __restrict__ part,
                                                    float* __restrict__ dW)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= n) return;
    double v = 0.0;
    for (int32_t sp = 0; sp < nsplit; ++sp) v += part[(int64_t)sp * n + q];
    dW[q] = (float)v;
}

// dst[0 .. n) = 0 (a kernel, not a memset, so the call can sit in a captured graph)
__global__ void __launch_bounds__(256) k_zero(int64_t n, float* __restrict__ dst)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q < n) dst[q] = 0.0f;
}

inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

// Node-range splits of the weight gradient: enough blocks to fill the chip
// (about 4096 with the tiles of every path) and at most 512 nodes per split,
// but at least 16 nodes per split and at most 256 splits.
int32_t mix_splits(int64_t N, int32_t P, int32_t C, int32_t Co)
{
    const int64_t tiles = (int64_t)P * ((C + 63) / 64) * ((Co + 63) / 64);
    int64_t n = (4096 + tiles - 1) / (tiles > 0 ? tiles : 1);
    if (n < (N + 511) / 512) n = (N + 511) / 512;
    const int64_t by_nodes = (N + 15) / 16;
    if (n > by_nodes) n = by_nodes;
    if (n > 256) n = 256;
    return (int32_t)(n < 1 ? 1 : n);
}

size_t mix_workspace_bytes(int64_t N, int32_t P, int32_t C, int32_t Co)
{
    return sizeof(double) * (size_t)mix_splits(N, P, C, Co) * (size_t)P * (size_t)C * (size_t)Co;
}

hipError_t launch_mix_fwd(const MixShape& m, const float* mid, const float* Wmix, float* out, hipStream_t s)
{
    if (m.N == 0) return hipSuccess;
    hipLaunchKernelGGL(k_mix_fwd, dim3(cdiv(m.N, kRows * kWaves), cdiv(m.Co, kCols), (unsigned)m.Dout), dim3(256), 0,
                       s, m, mid, Wmix, out);
    return hipGetLastError();
}

hipError_t launch_mix_bwd(const MixShape& m, const float* mid, const float* Wmix, const float* G, float* dmid,
                          float* dW, double* part, hipStream_t s)
{
    if (m.N == 0) {
        // no nodes: the weight gradient is zero
        const int64_t n = (int64_t)m.P * m.C * m.Co;
        if (dW && n > 0) {
            hipLaunchKernelGGL(k_zero, dim3(cdiv(n, 256)), dim3(256), 0, s, n, dW);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    if (dmid && m.N > 0) {
        hipLaunchKernelGGL(k_mix_bwd_data, dim3(cdiv(m.N, kRows * kWaves), cdiv(m.C, kCols), (unsigned)m.Dmid),
                           dim3(256), 0, s, m, G, Wmix, dmid);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (dW) {
        const int32_t nsplit = mix_splits(m.N, m.P, m.C, m.Co);
        const int32_t chunk = (int32_t)((m.N + nsplit - 1) / nsplit);
        hipLaunchKernelGGL(k_mix_bwd_weight, dim3(cdiv(m.C, kRows * kWaves), cdiv(m.Co, kCols), (unsigned)(m.P * nsplit)),
                           dim3(256), 0, s, m, nsplit, chunk > 0 ? chunk : 1, mid, G, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t n = (int64_t)m.P * m.C * m.Co;
        hipLaunchKernelGGL(k_mix_reduce, dim3(cdiv(n, 256)), dim3(256), 0, s, n, nsplit, part, dW);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace cgtp
