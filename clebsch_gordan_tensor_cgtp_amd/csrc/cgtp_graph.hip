// cgtp_graph.hip -- graph preparation (sender-sorted view of the receiver CSR)
// and the registry of compiled kernel specialisations.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cgtp_internal.h"

namespace cgtp {

// ----------------------------------------------------------------------------
// graph preparation: sender-sorted view of the receiver CSR
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_fill_i32(int32_t n, int32_t* __restrict__ p, int32_t v)
{
    const int32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) p[t] = v;
}

// recv[e] = receiver of edge e; one thread per receiver writes its segment
__global__ void __launch_bounds__(256) k_recv(int32_t N, const int32_t* __restrict__ row_ptr,
                                               int32_t* __restrict__ recv)
{
    const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) recv[e] = i;
}

// out-degree histogram (integer atomics: order-independent result)
__global__ void __launch_bounds__(256) k_outdeg(int32_t E, const int32_t* __restrict__ src, int32_t* cnt)
{
    const int32_t e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < E) atomicAdd(&cnt[src[e]], 1);
}

// srow[0] = 0, srow[j+1] = srow[j] + cnt[j]; one block of 1024 threads, each
// scanning a contiguous chunk
__global__ void __launch_bounds__(1024) k_scan(int32_t N, const int32_t* __restrict__ cnt,
                                                int32_t* __restrict__ srow)
{
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    const int32_t chunk = (N + 1023) / 1024;
    const int32_t b = t * chunk;
    const int32_t end = b + chunk < N ? b + chunk : N;
    int32_t s = 0;
    for (int32_t j = b; j < end; ++j) s += cnt[j];
    part[t] = s;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int32_t run = part[t] - s;  // exclusive prefix of this chunk
    if (t == 0) srow[0] = 0;
    for (int32_t j = b; j < end; ++j) {
        run += cnt[j];
        srow[j + 1] = run;
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
    const int32_t k = atomicAdd(&cursor[j], 1);
    perm[srow[j] + k] = e;
}

// sort each sender bucket by edge id (heap sort, one thread per sender), so the
// view is the stable counting sort of the edges by sender, then record the
// receiver of each permuted edge
__global__ void __launch_bounds__(256) k_sort_buckets(int32_t N, const int32_t* __restrict__ srow,
                                                       int32_t* __restrict__ perm)
{
    const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= N) return;
    int32_t* a = perm + srow[j];
    const int32_t n = srow[j + 1] - srow[j];
    if (n < 2) return;
    if (n <= 32) {  // insertion sort
        for (int32_t q = 1; q < n; ++q) {
            const int32_t v = a[q];
            int32_t r = q - 1;
            while (r >= 0 && a[r] > v) {
                a[r + 1] = a[r];
                --r;
            }
            a[r + 1] = v;
        }
        return;
    }
    auto sift = [&](int32_t root, int32_t len) {
        while (true) {
            int32_t c = 2 * root + 1;
            if (c >= len) break;
            if (c + 1 < len && a[c + 1] > a[c]) ++c;
            if (a[root] >= a[c]) break;
            const int32_t t = a[root];
            a[root] = a[c];
            a[c] = t;
            root = c;
        }
    };
    for (int32_t r = n / 2 - 1; r >= 0; --r) sift(r, n);
    for (int32_t len = n - 1; len > 0; --len) {
        const int32_t t = a[0];
        a[0] = a[len];
        a[len] = t;
        sift(0, len);
    }
}

__global__ void __launch_bounds__(256) k_sdst(int32_t E, const int32_t* __restrict__ perm,
                                               const int32_t* __restrict__ recv, int32_t* __restrict__ sdst)
{
    const int32_t k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k < E) sdst[k] = recv[perm[k]];
}

hipError_t launch_graph_prepare(int32_t N, int32_t E, const int32_t* row_ptr, const int32_t* src, void* ws,
                                hipStream_t s)
{
    const WsLayout L = ws_layout(N, E);
    char* base = (char*)ws;
    int32_t* srow = (int32_t*)(base + L.srow);
    int32_t* perm = (int32_t*)(base + L.perm);
    int32_t* sdst = (int32_t*)(base + L.sdst);
    int32_t* recv = (int32_t*)(base + L.recv);
    int32_t* cnt = (int32_t*)(base + L.cnt);
    const unsigned bN = (unsigned)((N + 255) / 256), bE = (unsigned)((E + 255) / 256);
    if (N > 0) hipLaunchKernelGGL(k_fill_i32, dim3(bN), dim3(256), 0, s, N, cnt, 0);
    if (E > 0) hipLaunchKernelGGL(k_outdeg, dim3(bE), dim3(256), 0, s, E, src, cnt);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, N, cnt, srow);
    if (N > 0) hipLaunchKernelGGL(k_fill_i32, dim3(bN), dim3(256), 0, s, N, cnt, 0);
    if (N > 0) hipLaunchKernelGGL(k_recv, dim3(bN), dim3(256), 0, s, N, row_ptr, recv);
    if (E > 0) hipLaunchKernelGGL(k_scatter, dim3(bE), dim3(256), 0, s, E, src, srow, cnt, perm);
    if (N > 0) hipLaunchKernelGGL(k_sort_buckets, dim3(bN), dim3(256), 0, s, N, srow, perm);
    if (E > 0) hipLaunchKernelGGL(k_sdst, dim3(bE), dim3(256), 0, s, E, perm, recv, sdst);
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
