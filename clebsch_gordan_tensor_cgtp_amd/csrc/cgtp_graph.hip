// cgtp_graph.hip -- graph preparation (sender-sorted view of the receiver CSR)
// and the registry of compiled kernel specialisations.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cgtp_internal.h"

namespace cgtp {

// ----------------------------------------------------------------------------
// graph preparation: sender-sorted view of the receiver CSR
// ----------------------------------------------------------------------------
// zero the padded per-sender counters
__global__ void __launch_bounds__(256) k_zero_counters(int32_t n, int32_t* __restrict__ p)
{
    const int32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) p[(int64_t)t * kCounterStride] = 0;
}

// out-degree histogram (integer atomics: the counts do not depend on order)
__global__ void __launch_bounds__(256) k_outdeg(int32_t E, const int32_t* __restrict__ src, int32_t* cnt)
{
    const int32_t e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < E) atomicAdd(&cnt[(int64_t)src[e] * kCounterStride], 1);
}

constexpr int kDegBins = 1024;  // degrees at or above kDegBins-1 share the first bin

// One block of 1024 threads, each owning a contiguous chunk of nodes:
//   srow[0] = 0, srow[j+1] = srow[j] + cnt[j]  (sender offsets), cursors cleared;
//   rorder / sorder: nodes ordered by in-degree / out-degree, longest first, so
//   the convolution kernels start the longest segments first (ties in any
//   order: the order only schedules blocks, every output has a fixed sum order).
__global__ void __launch_bounds__(1024) k_scan(int32_t N, const int32_t* __restrict__ row_ptr,
                                                const int32_t* __restrict__ cnt, int32_t* __restrict__ srow,
                                                int32_t* __restrict__ cursor, int32_t* __restrict__ rorder,
                                                int32_t* __restrict__ sorder)
{
    __shared__ int32_t part[1024];
    __shared__ int32_t hin[kDegBins], hout[kDegBins];
    const int t = threadIdx.x;
    const int32_t chunk = (N + 1023) / 1024;
    const int32_t b = t * chunk;
    const int32_t end = b + chunk < N ? b + chunk : N;
    auto bin = [](int32_t deg) { return kDegBins - 1 - (deg < kDegBins - 1 ? deg : kDegBins - 1); };
    hin[t] = 0;
    hout[t] = 0;
    int32_t s = 0;
    for (int32_t j = b; j < end; ++j) s += cnt[(int64_t)j * kCounterStride];
    part[t] = s;
    __syncthreads();
    for (int32_t j = b; j < end; ++j) {
        atomicAdd(&hin[bin(row_ptr[j + 1] - row_ptr[j])], 1);
        atomicAdd(&hout[bin(cnt[(int64_t)j * kCounterStride])], 1);
    }
    __syncthreads();  // histograms complete before the scan reads them
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = t >= off ? part[t - off] : 0;
        const int32_t vi = t >= off ? hin[t - off] : 0;
        const int32_t vo = t >= off ? hout[t - off] : 0;
        __syncthreads();
        part[t] += v;
        hin[t] += vi;
        hout[t] += vo;
        __syncthreads();
    }
    // exclusive bin starts
    const int32_t hi_excl = t > 0 ? hin[t - 1] : 0, ho_excl = t > 0 ? hout[t - 1] : 0;
    __syncthreads();
    hin[t] = hi_excl;
    hout[t] = ho_excl;
    __syncthreads();
    int32_t run = part[t] - s;  // exclusive prefix of this chunk
    if (t == 0) srow[0] = 0;
    for (int32_t j = b; j < end; ++j) {
        const int32_t c = cnt[(int64_t)j * kCounterStride];
        run += c;
        srow[j + 1] = run;
        cursor[(int64_t)j * kCounterStride] = 0;
        rorder[atomicAdd(&hin[bin(row_ptr[j + 1] - row_ptr[j])], 1)] = j;
        sorder[atomicAdd(&hout[bin(c)], 1)] = j;
    }
}

// place every edge in its sender's bucket (arbitrary order within a bucket)
__global__ void __launch_bounds__(256) k_scatter(int32_t E, const int32_t* __restrict__ src,
                                                  const int32_t* __restrict__ srow, int32_t* cursor,
                                                  int32_t* __restrict__ perm)
{
    const int32_t e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    const int32_t j = src[e];
    const int32_t k = atomicAdd(&cursor[(int64_t)j * kCounterStride], 1);
    perm[srow[j] + k] = e;
}

// receiver of edge e: the last i with row_ptr[i] <= e
__device__ __forceinline__ int32_t receiver_of(int32_t e, int32_t N, const int32_t* __restrict__ row_ptr)
{
    int32_t lo = 0, hi = N - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (row_ptr[mid] <= e) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

constexpr int kBucketLds = 1024;  // bucket entries a wave sorts in LDS

// One wave per sender: order its bucket by edge id (so the view is the stable
// counting sort of the edges by sender) and record the receiver of each
// permuted edge.  Buckets up to kBucketLds are ranked in LDS (edge ids are
// distinct, so rank = number of smaller ids); longer ones fall back to a
// serial insertion sort by lane 0.
__global__ void __launch_bounds__(256) k_sort_buckets(int32_t N, const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ srow, int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ sdst)
{
    __shared__ int32_t buf[4][kBucketLds];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int32_t j = (int32_t)blockIdx.x * 4 + w;
    if (j >= N) return;  // whole wave; no block-level barrier below
    const int32_t b = srow[j], n = srow[j + 1] - b;
    if (n <= kBucketLds) {
        int32_t* sb = buf[w];
        for (int32_t k = lane; k < n; k += 64) sb[k] = perm[b + k];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int32_t k = lane; k < n; k += 64) {
            const int32_t v = sb[k];
            int32_t rank = 0;
            for (int32_t t = 0; t < n; ++t) rank += sb[t] < v ? 1 : 0;
            perm[b + rank] = v;
            sdst[b + rank] = receiver_of(v, N, row_ptr);
        }
        return;
    }
    if (lane == 0) {
        int32_t* a = perm + b;
        for (int32_t q = 1; q < n; ++q) {
            const int32_t v = a[q];
            int32_t r = q - 1;
            while (r >= 0 && a[r] > v) {
                a[r + 1] = a[r];
                --r;
            }
            a[r + 1] = v;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int32_t k = lane; k < n; k += 64) sdst[b + k] = receiver_of(perm[b + k], N, row_ptr);
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
    if (N > 0) hipLaunchKernelGGL(k_zero_counters, dim3(bN), dim3(256), 0, s, N, cnt);
    if (E > 0) hipLaunchKernelGGL(k_outdeg, dim3(bE), dim3(256), 0, s, E, src, cnt);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, N, row_ptr, cnt, srow, cursor, rorder, sorder);
    if (E > 0) hipLaunchKernelGGL(k_scatter, dim3(bE), dim3(256), 0, s, E, src, srow, cursor, perm);
    if (E > 0) hipLaunchKernelGGL(k_sort_buckets, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, N, row_ptr, srow,
                                  perm, sdst);
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
