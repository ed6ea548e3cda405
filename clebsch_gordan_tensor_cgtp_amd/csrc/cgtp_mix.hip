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
// operands staged through LDS, widened when read, fp64 accumulation).  A
// 256-thread block computes a 64 x 64 output tile; each of its four waves owns
// 16 rows (four MFMA tiles sharing the row operand).  The weight gradient sums over all nodes: the node range is split
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

__device__ __forceinline__ int32_t clamp_idx(int32_t v, int32_t n) { return v < n ? v : n - 1; }

// degree of output slot s (s in [l*l, (l+1)*(l+1)))
__device__ __forceinline__ int32_t slot_degree(int32_t s)
{
    int32_t l = 0;
    while ((l + 1) * (l + 1) <= s) ++l;
    return l;
}

// ---- LDS-tiled MFMA GEMM ----------------------------------------------------
// A block computes a 64 x 64 tile of D = sum over K-chunks of A (64 x 32) B
// (32 x 64).  Every thread brings eight elements of each operand chunk from
// global memory (runs of eight consecutive addresses, 16-byte loads where the
// rows allow), the chunk goes to one of two LDS buffers, and each wave runs
// its 16 x 64 strip as 8 k-steps x 4 MFMA tiles out of it.  The next chunk's
// global loads are issued before the current chunk's MFMAs; with two buffers
// one barrier per chunk keeps writers and readers apart.  Row strides of 36
// and 80 words put the 64 lanes of each MFMA operand read on distinct banks.
constexpr int kTM = 64, kTN = 64, kTK = 32;
constexpr int kSA = kTK + 4, kSB = kTN + 16;

struct Tile {
    float a[kTM][kSA];  // [row][k]
    float b[kTK][kSB];  // [k][col]
};

// one chunk: the thread's eight A and eight B elements
struct Chunk {
    float av[8], bv[8];
};

// v[0..7] = p[0..7] where idx0 + j < lim (else 0), 16-byte loads when the
// whole run is in range and vec (rows of a multiple of four floats) holds
__device__ __forceinline__ void load8(float (&v)[8], const float* __restrict__ p, int32_t idx0, int32_t lim, bool ok,
                                      bool vec)
{
    if (ok && vec && idx0 + 8 <= lim) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (ok && idx0 + j < lim) ? p[j] : 0.0f;
    }
}

// MFMAs of one staged chunk for this wave's 16 rows
__device__ __forceinline__ void mfma_chunk(const Tile& T, int wave, int lane, v4d (&acc)[4])
{
    const int i = lane % 16, kk = lane / 16;
#pragma unroll
    for (int ks = 0; ks < kTK / 4; ++ks) {
        const double a = (double)T.a[16 * wave + i][4 * ks + kk];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const double b = (double)T.b[4 * ks + kk][16 * t + i];
            acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[t], 0, 0, 0);
        }
    }
}

// Runs chunks 0 .. n-1 through the two buffers starting at T[*buf]:
// load(c, ch) fills the thread's elements of chunk c, put(ch, T) writes them
// to LDS.  *buf tracks the buffer parity across calls.
template <class Load, class Put>
__device__ __forceinline__ void gemm_chunks(int32_t n, Tile (&T)[2], int& buf, Load&& load, Put&& put,
                                            v4d (&acc)[4])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (n <= 0) return;
    Chunk cur;
    load(0, cur);
    for (int32_t c = 0; c < n; ++c) {
        // T[buf] was last read two chunks ago; every wave has passed the
        // barrier after that
        put(cur, T[buf]);
        __syncthreads();
        if (c + 1 < n) load(c + 1, cur);
        mfma_chunk(T[buf], wave, lane, acc);
        buf ^= 1;
    }
}

// store of D's 16 x 64 strip of this wave: row index r, column index col
template <class Store>
__device__ __forceinline__ void store_strip(const v4d (&acc)[4], Store&& store)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane % 16, kk = lane / 16;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) store(16 * wave + 4 * r + kk, 16 * t + i, acc[t][r]);
}

// out[i][s][w]: rows = 64 nodes, cols = 64 output channels, K = (paths of
// l3) x C.  The highest slots, whose degrees have the most paths, go first.
__global__ void __launch_bounds__(256) k_mix_fwd(MixShape m, bool vec, const float* __restrict__ mid,
                                                 const float* __restrict__ Wmix, float* __restrict__ out)
{
    __shared__ Tile T[2];
    const int tid = threadIdx.x;
    const int32_t n0 = (int32_t)blockIdx.x * kTM, c0 = (int32_t)blockIdx.y * kTN;
    const int32_t s = m.Dout - 1 - (int32_t)blockIdx.z;
    const int32_t l3 = slot_degree(s), mm = s - l3 * l3;
    const int32_t kc = (m.C + kTK - 1) / kTK;  // chunks per path
    v4d acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4d{0.0, 0.0, 0.0, 0.0};
    // A: row tid/4, k (tid%4)*8 + j; B: k tid/8, col (tid%8)*8 + j
    const int ar = tid / 4, ak = (tid % 4) * 8, bk = tid / 8, bc = (tid % 8) * 8;
    const int32_t node = n0 + ar, nodec = clamp_idx(node, m.N), col = c0 + bc;
    int buf = 0;
    for (int32_t p = 0; p < m.P; ++p) {
        if (m.l3[p] != l3) continue;
        const float* arow = mid + ((int64_t)nodec * m.Dmid + m.o[p] + mm) * m.C;
        const float* wp = Wmix + (int64_t)p * m.C * m.Co;
        auto load = [&](int32_t c, Chunk& ch) {
            const int32_t u = c * kTK + ak, ub = c * kTK + bk;
            load8(ch.av, arow + (u < m.C ? u : 0), u, m.C, node < m.N, vec);
            load8(ch.bv, wp + (int64_t)clamp_idx(ub, m.C) * m.Co + (col < m.Co ? col : 0), col, m.Co, ub < m.C,
                  vec);
        };
        auto put = [&](const Chunk& ch, Tile& t) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                t.a[ar][ak + j] = ch.av[j];
                t.b[bk][bc + j] = ch.bv[j];
            }
        };
        gemm_chunks(kc, T, buf, load, put, acc);
    }
    store_strip(acc, [&](int r, int cidx, double v) {
        const int32_t nd = n0 + r, cc = c0 + cidx;
        if (nd < m.N && cc < m.Co) out[((int64_t)nd * m.Dout + s) * m.Co + cc] = (float)v;
    });
}

// d_mid[i][row][u]: rows = 64 nodes, cols = 64 input channels, K = C_out
__global__ void __launch_bounds__(256) k_mix_bwd_data(MixShape m, bool vec, const float* __restrict__ G,
                                                      const float* __restrict__ Wmix, float* __restrict__ dmid)
{
    __shared__ Tile T[2];
    const int tid = threadIdx.x;
    const int32_t n0 = (int32_t)blockIdx.x * kTM, c0 = (int32_t)blockIdx.y * kTN;
    const int32_t row = (int32_t)blockIdx.z;
    int32_t p = 0;
    while (p + 1 < m.P && m.o[p + 1] <= row) ++p;
    const int32_t s = m.l3[p] * m.l3[p] + (row - m.o[p]);
    v4d acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4d{0.0, 0.0, 0.0, 0.0};
    // A (G rows, contiguous in w): row tid/4, k (tid%4)*8 + j; B (Wmix[p][u][w],
    // contiguous in w): col u = tid/4, k (tid%4)*8 + j, stored transposed
    const int ar = tid / 4, ak = (tid % 4) * 8;
    const int32_t node = n0 + ar, nodec = clamp_idx(node, m.N);
    const float* grow = G + ((int64_t)nodec * m.Dout + s) * m.Co;
    const int32_t ucol = c0 + ar;
    const float* wrow = Wmix + ((int64_t)p * m.C + clamp_idx(ucol, m.C)) * m.Co;
    auto load = [&](int32_t c, Chunk& ch) {
        const int32_t w = c * kTK + ak, wo = w < m.Co ? w : 0;
        load8(ch.av, grow + wo, w, m.Co, node < m.N, vec);
        load8(ch.bv, wrow + wo, w, m.Co, ucol < m.C, vec);
    };
    auto put = [&](const Chunk& ch, Tile& t) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            t.a[ar][ak + j] = ch.av[j];
            t.b[ak + j][ar] = ch.bv[j];
        }
    };
    int buf = 0;
    gemm_chunks((m.Co + kTK - 1) / kTK, T, buf, load, put, acc);
    store_strip(acc, [&](int r, int cidx, double v) {
        const int32_t nd = n0 + r, u = c0 + cidx;
        if (nd < m.N && u < m.C) dmid[((int64_t)nd * m.Dmid + row) * m.C + u] = (float)v;
    });
}

// part[g][u][w] of run g (path p's runs are g = off[p] .. off[p+1]-1):
// rows = 64 input channels, cols = 64 output channels, K = the run's (m, node)
// pairs, m-major (pair r is component m = r / N of node r % N)
__global__ void __launch_bounds__(256) k_mix_bwd_weight(MixShape m, MixSplit sp, bool vec,
                                                        const float* __restrict__ mid, const float* __restrict__ G,
                                                        double* __restrict__ part)
{
    __shared__ Tile T[2];
    const int tid = threadIdx.x;
    const int32_t r0 = (int32_t)blockIdx.x * kTM, c0 = (int32_t)blockIdx.y * kTN;
    const int32_t g = (int32_t)blockIdx.z;
    int32_t p = 0;
    while (p + 1 < m.P && sp.off[p + 1] <= g) ++p;
    const int32_t s0 = m.l3[p] * m.l3[p];
    const int64_t pairs = (int64_t)m.N * (2 * m.l3[p] + 1);
    const int64_t rb = (int64_t)(g - sp.off[p]) * sp.rows;
    const int64_t re = rb + sp.rows < pairs ? rb + sp.rows : pairs;
    const int32_t nch = re > rb ? (int32_t)((re - rb + kTK - 1) / kTK) : 0;
    v4d acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4d{0.0, 0.0, 0.0, 0.0};
    // A (mid rows, contiguous in u): pair k = tid/8, u (tid%8)*8 + j, stored
    // transposed; B (G rows, contiguous in w): pair k = tid/8, w (tid%8)*8 + j
    const int kr = tid / 8, c8 = (tid % 8) * 8;
    const int32_t u = r0 + c8, w = c0 + c8;
    auto load = [&](int32_t c, Chunk& ch) {
        const int64_t r = rb + (int64_t)c * kTK + kr;
        const bool in = r < re;
        const int32_t mm = in ? (int32_t)(r / m.N) : 0;
        const int32_t node = in ? (int32_t)(r - (int64_t)mm * m.N) : 0;
        load8(ch.av, mid + ((int64_t)node * m.Dmid + m.o[p] + mm) * m.C + (u < m.C ? u : 0), u, m.C, in, vec);
        load8(ch.bv, G + ((int64_t)node * m.Dout + s0 + mm) * m.Co + (w < m.Co ? w : 0), w, m.Co, in, vec);
    };
    auto put = [&](const Chunk& ch, Tile& t) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            t.a[c8 + j][kr] = ch.av[j];
            t.b[kr][c8 + j] = ch.bv[j];
        }
    };
    int buf = 0;
    gemm_chunks(nch, T, buf, load, put, acc);
    store_strip(acc, [&](int r, int cidx, double v) {
        const int32_t uu = r0 + r, col = c0 + cidx;
        if (uu < m.C && col < m.Co) part[((int64_t)g * m.C + uu) * m.Co + col] = v;
    });
}

// dWmix[p][u][w] = sum of path p's runs, in order
__global__ void __launch_bounds__(256) k_mix_reduce(MixShape m, MixSplit sp, const double* __restrict__ part,
                                                    float* __restrict__ dW)
{
    const int64_t n = (int64_t)m.C * m.Co;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)m.P * n) return;
    const int32_t p = (int32_t)(q / n);
    const int64_t r = q - (int64_t)p * n;
    double v = 0.0;
    for (int32_t g = sp.off[p]; g < sp.off[p + 1]; ++g) v += part[(int64_t)g * n + r];
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

// Runs of the weight gradient: about four blocks per compute unit over the
// output tiles, the (m, node) pairs of all paths cut into runs of equal length
// (a whole number of chunks, at least two), so every block has the same work.
MixSplit mix_split(const MixShape& m)
{
    MixSplit sp{};
    const int64_t tiles = (int64_t)((m.C + kTM - 1) / kTM) * ((m.Co + kTN - 1) / kTN);
    int64_t pairs = 0;
    for (int p = 0; p < m.P; ++p) pairs += (int64_t)m.N * (2 * m.l3[p] + 1);
    const int64_t target = (1024 + tiles - 1) / (tiles > 0 ? tiles : 1);
    int64_t rows = (pairs + target - 1) / target;
    rows = (rows + kTK - 1) / kTK * kTK;
    if (rows < 2 * kTK) rows = 2 * kTK;
    sp.rows = (int32_t)rows;
    sp.off[0] = 0;
    for (int p = 0; p < m.P; ++p)
        sp.off[p + 1] = sp.off[p] + (int32_t)(((int64_t)m.N * (2 * m.l3[p] + 1) + rows - 1) / rows);
    return sp;
}

size_t mix_workspace_bytes(const MixShape& m)
{
    return sizeof(double) * (size_t)mix_split(m).off[m.P] * (size_t)m.C * (size_t)m.Co;
}

// 16-byte operand loads need rows of a multiple of four floats (the entry
// points only take 16-byte aligned arrays)
static bool vec_ok(const MixShape& m) { return m.C % 4 == 0 && m.Co % 4 == 0; }

hipError_t launch_mix_fwd(const MixShape& m, const float* mid, const float* Wmix, float* out, hipStream_t s)
{
    if (m.N == 0) return hipSuccess;
    hipLaunchKernelGGL(k_mix_fwd, dim3(cdiv(m.N, kTM), cdiv(m.Co, kTN), (unsigned)m.Dout), dim3(256), 0,
                       s, m, vec_ok(m), mid, Wmix, out);
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
        hipLaunchKernelGGL(k_mix_bwd_data, dim3(cdiv(m.N, kTM), cdiv(m.C, kTN), (unsigned)m.Dmid),
                           dim3(256), 0, s, m, vec_ok(m), G, Wmix, dmid);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (dW) {
        const MixSplit sp = mix_split(m);
        hipLaunchKernelGGL(k_mix_bwd_weight, dim3(cdiv(m.C, kTM), cdiv(m.Co, kTN), (unsigned)sp.off[m.P]),
                           dim3(256), 0, s, m, sp, vec_ok(m), mid, G, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t n = (int64_t)m.P * m.C * m.Co;
        hipLaunchKernelGGL(k_mix_reduce, dim3(cdiv(n, 256)), dim3(256), 0, s, m, sp, part, dW);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace cgtp
