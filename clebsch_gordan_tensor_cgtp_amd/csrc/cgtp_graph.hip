// cgtp_graph.hip -- graph preparation (sender-sorted view of the receiver CSR)
// and the registry of compiled kernel specialisations.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cgtp_internal.h"

namespace cgtp {

// ----------------------------------------------------------------------------
// graph preparation: sender-sorted view of the receiver CSR
// ----------------------------------------------------------------------------
// zero the padded per-sender counters and cursors
__global__ void __launch_bounds__(256) k_zero_counters(int32_t n, int32_t* __restrict__ cnt,
                                                        int32_t* __restrict__ cursor)
{
    const int32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) {
        cnt[(int64_t)t * kCounterStride] = 0;
        cursor[(int64_t)t * kCounterStride] = 0;
    }
}

constexpr int kDegBins = 1024;  // degrees at or above kDegBins-1 share the first bin

// Inclusive prefix sum of one value per thread over a 1024-thread block:
// shuffle scans inside each wave, then the 16 wave totals.  `tot` is LDS
// scratch of 16 ints; ends with a barrier.
__device__ __forceinline__ int32_t block_scan_1024(int32_t v, int32_t* tot)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    if (lane == 63) tot[w] = v;
    __syncthreads();
    int32_t base = 0;
    for (int k = 0; k < w; ++k) base += tot[k];
    __syncthreads();  // tot may be reused after this
    return v + base;
}

// Sender offsets and block orders, run by one block of 1024 threads, each
// owning a contiguous chunk of nodes:
//   srow[0] = 0, srow[j+1] = srow[j] + cnt[j]  (sender offsets);
//   rorder / sorder: nodes ordered by in-degree / out-degree, longest first, so
//   the convolution kernels start the longest segments first (ties in any
//   order: the order only schedules blocks, every output has a fixed sum order).
__device__ void offsets_and_orders(int32_t N, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ cnt,
                                   int32_t* __restrict__ srow, int32_t* __restrict__ rorder,
                                   int32_t* __restrict__ sorder)
{
    __shared__ int32_t hin[kDegBins], hout[kDegBins], tot[16];
    const int t = threadIdx.x;
    const int32_t chunk = (N + 1023) / 1024;
    const int32_t b = t * chunk;
    const int32_t end = b + chunk < N ? b + chunk : N;
    auto bin = [](int32_t deg) { return kDegBins - 1 - (deg < kDegBins - 1 ? deg : kDegBins - 1); };
    hin[t] = 0;
    hout[t] = 0;
    __syncthreads();
    // one pass: this chunk's out-degree total and both degree histograms
    int32_t s = 0;
    for (int32_t j = b; j < end; ++j) {
        const int32_t c = cnt[(int64_t)j * kCounterStride];
        s += c;
        atomicAdd(&hin[bin(row_ptr[j + 1] - row_ptr[j])], 1);
        atomicAdd(&hout[bin(c)], 1);
    }
    __syncthreads();  // histograms complete before they are scanned
    const int32_t run0 = block_scan_1024(s, tot) - s;  // exclusive prefix of this chunk
    const int32_t hi = hin[t], ho = hout[t];
    const int32_t hi_incl = block_scan_1024(hi, tot), ho_incl = block_scan_1024(ho, tot);
    hin[t] = hi_incl - hi;  // exclusive bin starts
    hout[t] = ho_incl - ho;
    __syncthreads();
    int32_t run = run0;
    if (t == 0) srow[0] = 0;
    for (int32_t j = b; j < end; ++j) {
        const int32_t c = cnt[(int64_t)j * kCounterStride];
        run += c;
        srow[j + 1] = run;
        rorder[atomicAdd(&hin[bin(row_ptr[j + 1] - row_ptr[j])], 1)] = j;
        sorder[atomicAdd(&hout[bin(c)], 1)] = j;
    }
}

// out-degree histogram (integer atomics: the counts do not depend on order)
__global__ void __launch_bounds__(256) k_outdeg(int32_t E, const int32_t* __restrict__ src, int32_t* cnt)
{
    const int32_t e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < E) atomicAdd(&cnt[(int64_t)src[e] * kCounterStride], 1);
}

// sender offsets and block orders: a single block of 1024 threads
__global__ void __launch_bounds__(1024) k_offsets(int32_t N, const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ cnt, int32_t* __restrict__ srow,
                                                   int32_t* __restrict__ rorder, int32_t* __restrict__ sorder)
{
    offsets_and_orders(N, row_ptr, cnt, srow, rorder, sorder);
}

// Place every edge in its sender's bucket (arbitrary order within a bucket),
// one wave per receiver, recording the receiver beside the edge.
__global__ void __launch_bounds__(256) k_scatter(int32_t N, const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ src, const int32_t* __restrict__ srow,
                                                  int32_t* cursor, int32_t* __restrict__ perm,
                                                  int32_t* __restrict__ sdst)
{
    const int32_t i = (int32_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= N) return;
    const int32_t end = row_ptr[i + 1];
    for (int32_t e = row_ptr[i] + (threadIdx.x & 63); e < end; e += 64) {
        const int32_t j = src[e];
        const int32_t k = srow[j] + atomicAdd(&cursor[(int64_t)j * kCounterStride], 1);
        perm[k] = e;
        sdst[k] = i;
    }
}

constexpr int kBucketLds = 1024;  // bucket entries a wave sorts in LDS

// One wave per sender: order its bucket's (edge, receiver) pairs by edge id,
// so the view is the stable counting sort of the edges by sender.  Buckets up
// to kBucketLds are ranked in LDS (edge ids are distinct, so rank = number of
// smaller ids); longer ones fall back to a serial insertion sort by lane 0.
__global__ void __launch_bounds__(256) k_sort_buckets(int32_t N, const int32_t* __restrict__ srow,
                                                       int32_t* __restrict__ perm, int32_t* __restrict__ sdst)
{
    __shared__ int32_t ebuf[4][kBucketLds], ibuf[4][kBucketLds];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int32_t j = (int32_t)blockIdx.x * 4 + w;
    if (j >= N) return;  // whole wave; no block-level barrier below
    const int32_t b = srow[j], n = srow[j + 1] - b;
    if (n <= kBucketLds) {
        int32_t* se = ebuf[w];
        int32_t* si = ibuf[w];
        for (int32_t k = lane; k < n; k += 64) {
            se[k] = perm[b + k];
            si[k] = sdst[b + k];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int32_t k = lane; k < n; k += 64) {
            const int32_t v = se[k];
            int32_t rank = 0;
            for (int32_t t = 0; t < n; ++t) rank += se[t] < v ? 1 : 0;
            perm[b + rank] = v;
            sdst[b + rank] = si[k];
        }
        return;
    }
    if (lane == 0) {
        int32_t* a = perm + b;
        int32_t* r = sdst + b;
        for (int32_t q = 1; q < n; ++q) {
            const int32_t v = a[q], vr = r[q];
            int32_t p = q - 1;
            while (p >= 0 && a[p] > v) {
                a[p + 1] = a[p];
                r[p + 1] = r[p];
                --p;
            }
            a[p + 1] = v;
            r[p + 1] = vr;
        }
    }
}

hipError_t launch_graph_prepare(int32_t N, int32_t E, const int32_t* row_ptr, const int32_t* src, void* ws,
                                hipStream_t s)
{
    const WsLayout L = ws_layout(N, E);
    char* base = (char*)ws;
    int32_t* srow = (int32_t*)(base + L.srow);
    int32_t* perm = (int32_t*)(base + L.perm);
    int32_t* sdst = (int32_t*)(base + L.sdst);
    int32_t* cnt = (int32_t*)(base + L.cnt);
    int32_t* cursor = (int32_t*)(base + L.cursor);
    int32_t* rorder = (int32_t*)(base + L.rorder);
    int32_t* sorder = (int32_t*)(base + L.sorder);
    const unsigned bN = (unsigned)((N + 255) / 256), bE = (unsigned)((E + 255) / 256);
    if (N > 0) hipLaunchKernelGGL(k_zero_counters, dim3(bN), dim3(256), 0, s, N, cnt, cursor);
    if (E > 0) hipLaunchKernelGGL(k_outdeg, dim3(bE), dim3(256), 0, s, E, src, cnt);
    hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, s, N, row_ptr, cnt, srow, rorder, sorder);
    if (E > 0 && N > 0) {
        const unsigned b4 = (unsigned)((N + 3) / 4);
        hipLaunchKernelGGL(k_scatter, dim3(b4), dim3(256), 0, s, N, row_ptr, src, srow, cursor, perm, sdst);
        hipLaunchKernelGGL(k_sort_buckets, dim3(b4), dim3(256), 0, s, N, srow, perm, sdst);
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// registry
// ----------------------------------------------------------------------------
const KernelSet* kernels_l1(int channels);
const KernelSet* kernels_l2(int channels);
const KernelSet* kernels_l3(int channels);
bool table_l1(int path, double* dense);
bool table_l2(int path, double* dense);
bool table_l3(int path, double* dense);

const KernelSet* find_kernels(int l_in, int l_sh, int l_out, int channels)
{
    if (l_in != l_sh || l_sh != l_out) return nullptr;
    switch (l_in) {
        case 1: return kernels_l1(channels);
        case 2: return kernels_l2(channels);
        case 3: return kernels_l3(channels);
        default: return nullptr;
    }
}

bool host_cg_table(int l_in, int l_sh, int l_out, int path, double* dense)
{
    if (l_in != l_sh || l_sh != l_out) return false;
    switch (l_in) {
        case 1: return table_l1(path, dense);
        case 2: return table_l2(path, dense);
        case 3: return table_l3(path, dense);
        default: return false;
    }
}

}  // namespace cgtp
