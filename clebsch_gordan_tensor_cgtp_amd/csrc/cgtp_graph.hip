// cgtp_graph.hip -- graph preparation: the sender-sorted view of the receiver
// CSR that the backward walks, and the block schedules of both convolution
// kernels.
//
// The view is the stable counting sort of the edges by sender (per sender,
// edges in ascending id), so the backward's grad_x sums run in a fixed order.
//
// The schedules decide which node each block of a convolution launch serves.
// By default every node is placed by degree, longest segment first: blocks
// are dealt to the eight XCDs in turn (block b runs on XCD b % 8), so each XCD
// receives the same mix of long and short segments and the last blocks to
// start are short.
//
// The locality schedule (CGTP_FLAG_LOCALITY) instead gives each XCD, with its
// own L2, a compact piece of the atomic system, so the rows its blocks gather
// (x_j in the forward, grad_out_i in the backward) are shared through that L2
// instead of fetched again by every XCD.  The caller's node ids carry no
// spatial order, so it is read off the graph itself with two rounds of
// min-hash clustering: every node draws a pseudo-random key, key1(i) is the
// smallest key in the closed neighbourhood of i, and the cluster centre of i
// is the node holding the smallest key1 over the closed neighbourhood of i
// (nodes within two hops share it).  Nodes are ordered by centre and cut into
// eight ranges of ceil(N/8), range x served by the blocks b = x, x+8, ...;
// inside a range the blocks run longest segment first.  It cuts the gathered
// bytes but not the kernel time on this chip (the re-fetched rows come from
// the 256 MB last-level cache), and with skewed degrees the clusters can
// leave the ranges unequal in edges, hence it is not the default.
//
// Either order only schedules blocks: every output row has one writer and a
// fixed summation order, so results do not depend on it (placement inside a
// degree bin comes from integer atomics and may differ between runs).
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include "cgtp_internal.h"

namespace cgtp {

namespace {

__device__ __forceinline__ int32_t clampi(int32_t v, int32_t lo, int32_t hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

// a sender id outside [0, N) breaks the CSR contract; it is read as node 0 so
// every count and index below stays in range
__device__ __forceinline__ int32_t valid_node(int32_t j, int32_t N) { return (uint32_t)j < (uint32_t)N ? j : 0; }

// segment [e0, e1) of receiver i, clamped to [0, E]
__device__ __forceinline__ void segment(const int32_t* __restrict__ row_ptr, int32_t i, int32_t E, int32_t& e0,
                                        int32_t& e1)
{
    e0 = clampi(row_ptr[i], 0, E);
    e1 = clampi(row_ptr[i + 1], e0, E);
}

// pseudo-random 32-bit key of node j (an invertible multiply / xor-shift
// mix), paired with j so keys are distinct and ties cannot occur
__device__ __forceinline__ uint64_t node_key(int32_t j)
{
    uint32_t h = (uint32_t)j * 0x9E3779B1u;
    h ^= h >> 15;
    h *= 0x85EBCA77u;
    h ^= h >> 13;
    return ((uint64_t)h << 32) | (uint32_t)j;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o < v ? o : v;
    }
    return v;
}

__device__ __forceinline__ int deg_bin(int32_t d) { return kDegBins - 1 - (d < kDegBins - 1 ? d : kDegBins - 1); }

// Inclusive prefix sum of one value per thread over a 1024-thread block:
// shuffle scans inside each wave, then the 16 wave totals.  `tot` is LDS
// scratch of 16 ints; *total receives the block's sum.  Ends with a barrier.
__device__ __forceinline__ int32_t block_scan_1024(int32_t v, int32_t* tot, int32_t* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    if (lane == 63) tot[w] = v;
    __syncthreads();
    int32_t base = 0, all = 0;
    for (int k = 0; k < 16; ++k) {
        base += k < w ? tot[k] : 0;
        all += tot[k];
    }
    __syncthreads();  // tot may be reused after this
    *total = all;
    return v + base;
}

}  // namespace

// Step 1, one wave per receiver i: clear i's counters (used from step 2 on;
// block 0 also clears the global degree bins of step 3) and, for the
// clustered schedule, key1(i) = min node_key over i and its
// senders.
__global__ void __launch_bounds__(256) k_prep_keys(int32_t N, int32_t E, const int32_t* __restrict__ row_ptr,
                                                    const int32_t* __restrict__ src, int32_t locality,
                                                    uint64_t* __restrict__ key1, int32_t* __restrict__ cnt,
                                                    int32_t* __restrict__ ccnt, int32_t* __restrict__ bins)
{
    if (blockIdx.x == 0)
        for (int k = threadIdx.x; k < 4 * kDegBins; k += 256) bins[k] = 0;
    const int32_t i = (int32_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (i >= N) return;
    if (lane == 0) {
        cnt[(int64_t)i * kCounterStride] = 0;
        ccnt[i] = 0;
    }
    if (!locality) return;
    int32_t e0, e1;
    segment(row_ptr, i, E, e0, e1);
    uint64_t m = node_key(i);
    for (int32_t e = e0 + lane; e < e1; e += 64) {
        const uint64_t k = node_key(valid_node(src[e], N));
        m = k < m ? k : m;
    }
    m = wave_min_u64(m);
    if (lane == 0) key1[i] = m;
}

// Step 2, one wave per receiver i: the out-degree count of every sender, with
// each in-edge's rank among its sender's edges (the value the count's atomic
// returns, in arrival order) kept in urank, and, for the locality schedule,
// i's cluster centre and its rank inside the cluster (integer atomics).
__global__ void __launch_bounds__(256) k_prep_centers(int32_t N, int32_t E, const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ src, int32_t locality,
                                                       const uint64_t* __restrict__ key1, int32_t* __restrict__ center,
                                                       int32_t* __restrict__ crank, int32_t* ccnt, int32_t* cnt,
                                                       int32_t* __restrict__ urank)
{
    const int32_t i = (int32_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (i >= N) return;
    int32_t e0, e1;
    segment(row_ptr, i, E, e0, e1);
    if (locality) {
        uint64_t m = key1[i];
        for (int32_t e = e0 + lane; e < e1; e += 64) {
            const uint64_t k = key1[valid_node(src[e], N)];
            m = k < m ? k : m;
        }
        const int32_t c = (int32_t)(uint32_t)wave_min_u64(m);
        if (lane == 0) {
            center[i] = c;
            crank[i] = atomicAdd(&ccnt[c], 1);
        }
    }
    for (int32_t e = e0 + lane; e < e1; e += 64)
        urank[e] = atomicAdd(&cnt[(int64_t)valid_node(src[e], N) * kCounterStride], 1);
}

// Step 3 of the locality schedule (and of an empty graph), one block of 1024
// threads: the sender offsets srow (prefix sum of the out-degrees) and the two
// block schedules.  (The longest-first schedule of a non-empty graph runs
// k_prep_hist and k_prep_place below instead; this kernel still implements it
// as one range of all N nodes, longest first, block b serving entry b.)
// Locality: node i's place in the cluster order is g = coff[centre] +
// rank (coff the prefix sum of the cluster sizes), its range is x = g / Q,
// and inside a range the nodes go longest first by LDS histograms of
// (range, degree bin); block x + 8s serves entry s of range x.
__global__ void __launch_bounds__(1024) k_prep_orders(int32_t N, int32_t E, int32_t locality,
                                                       const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ cnt, const int32_t* __restrict__ ccnt,
                                                       const int32_t* __restrict__ center,
                                                       const int32_t* __restrict__ crank, int32_t* __restrict__ srow,
                                                       int32_t* __restrict__ coff, int32_t* __restrict__ rorder,
                                                       int32_t* __restrict__ sorder)
{
    __shared__ int32_t hin[kXcds * kDegBins], hout[kXcds * kDegBins], tot[16], xbase[2][kXcds];
    const int t = threadIdx.x;
    if (t == 0) srow[0] = 0;
    if (N == 0) return;
    const int32_t nr = locality ? kXcds : 1;  // ranges
    const int32_t Q = (N + nr - 1) / nr;       // nodes per range
    // prefix sums over each thread's contiguous chunk of nodes
    {
        const int32_t ch = (N + 1023) / 1024;
        const int32_t b = t * ch < N ? t * ch : N, e = b + ch < N ? b + ch : N;
        int32_t so = 0, sc = 0;
        for (int32_t i = b; i < e; ++i) {
            so += cnt[(int64_t)i * kCounterStride];
            sc += locality ? ccnt[i] : 0;
        }
        int32_t tt;
        int32_t ro = block_scan_1024(so, tot, &tt) - so;
        int32_t rc = block_scan_1024(sc, tot, &tt) - sc;
        for (int32_t i = b; i < e; ++i) {
            if (locality) {
                const int32_t c = ccnt[i];
                coff[i] = rc;
                rc += c;
            }
            ro += cnt[(int64_t)i * kCounterStride];
            srow[i + 1] = ro;
        }
    }
    for (int k = t; k < kXcds * kDegBins; k += 1024) {
        hin[k] = 0;
        hout[k] = 0;
    }
    __syncthreads();  // srow and coff (global) and the cleared histograms are visible block-wide
    auto place = [&](int32_t i, int& hi, int& ho) {
        int32_t x = 0;
        if (locality) {
            const int32_t g = clampi(coff[clampi(center[i], 0, N - 1)] + crank[i], 0, N - 1);
            x = g / Q;
        }
        const int32_t e0 = clampi(row_ptr[i], 0, E), e1 = clampi(row_ptr[i + 1], e0, E);
        hi = x * kDegBins + deg_bin(e1 - e0);
        ho = x * kDegBins + deg_bin(srow[i + 1] - srow[i]);
    };
    for (int32_t i = t; i < N; i += 1024) {
        int hi, ho;
        place(i, hi, ho);
        atomicAdd(&hin[hi], 1);
        atomicAdd(&hout[ho], 1);
    }
    __syncthreads();
    // exclusive bin starts inside each range: one scan over all kXcds*kDegBins
    // bins (thread t owns bins 8t .. 8t+7, all in range t / 128), minus the
    // range's own start
    static_assert(kXcds * kDegBins == 8 * 1024, "eight bins per thread");
    {
        int32_t vi[8], vo[8], si = 0, so = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            vi[k] = hin[8 * t + k];
            vo[k] = hout[8 * t + k];
            si += vi[k];
            so += vo[k];
        }
        int32_t tt;
        int32_t pi = block_scan_1024(si, tot, &tt) - si;
        int32_t po = block_scan_1024(so, tot, &tt) - so;
        if ((t & 127) == 0) {
            xbase[0][t >> 7] = pi;
            xbase[1][t >> 7] = po;
        }
        __syncthreads();
        pi -= xbase[0][t >> 7];
        po -= xbase[1][t >> 7];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            hin[8 * t + k] = pi;
            hout[8 * t + k] = po;
            pi += vi[k];
            po += vo[k];
        }
    }
    __syncthreads();
    for (int32_t i = t; i < N; i += 1024) {
        int hi, ho;
        place(i, hi, ho);
        const int32_t x = hi / kDegBins;
        rorder[x + nr * atomicAdd(&hin[hi], 1)] = i;
        sorder[x + nr * atomicAdd(&hout[ho], 1)] = i;
    }
    // blocks past the end of a short range, or past N, are idle
    const int32_t grid = kXcds * ((N + kXcds - 1) / kXcds);
    for (int32_t b = t; b < grid; b += 1024) {
        const int32_t x = b % nr, s = b / nr;
        const int32_t nx = clampi(N - x * Q, 0, Q);
        if (s >= nx) {
            rorder[b] = -1;
            sorder[b] = -1;
        }
    }
}

// Step 3 of the longest-first schedule over several blocks, part 1: block b
// takes nodes [b*1024, (b+1)*1024), one per thread.  It writes the sum of
// their out-degrees to bsum[b] and adds its LDS histograms of in-degree and
// out-degree bins to the global bins (one integer atomic per non-empty bin).
__global__ void __launch_bounds__(kOrderBlock) k_prep_hist(int32_t N, int32_t E, const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ cnt, int32_t* bins,
                                                            int32_t* __restrict__ bsum)
{
    static_assert(kOrderBlock == 1024 && kDegBins == 1024, "one node and one bin per thread");
    __shared__ int32_t hin[kDegBins], hout[kDegBins], tot[16];
    const int t = threadIdx.x;
    const int64_t i64 = (int64_t)blockIdx.x * kOrderBlock + t;
    const int32_t i = i64 < N ? (int32_t)i64 : N;  // i == N: no node
    hin[t] = 0;
    hout[t] = 0;
    __syncthreads();
    int32_t dout = 0;
    if (i < N) {
        const int32_t e0 = clampi(row_ptr[i], 0, E), e1 = clampi(row_ptr[i + 1], e0, E);
        dout = cnt[(int64_t)i * kCounterStride];
        atomicAdd(&hin[deg_bin(e1 - e0)], 1);
        atomicAdd(&hout[deg_bin(dout)], 1);
    }
    int32_t total;
    block_scan_1024(dout, tot, &total);  // ends with a barrier: the histograms are complete
    if (t == 0) bsum[blockIdx.x] = total;
    if (hin[t] > 0) atomicAdd(&bins[t], hin[t]);
    if (hout[t] > 0) atomicAdd(&bins[kDegBins + t], hout[t]);
}

// Part 2, the same blocks: srow (the block's base is the sum of bsum over
// the blocks before it, then a scan inside the block), the start of every bin
// (a scan of the global bins), and the schedules: the block claims a run of
// each non-empty bin with one atomic on the bin's cursor and places its nodes
// in it through LDS atomics.  Block b of a convolution serves entry b; the
// entries past N (up to the next multiple of kXcds) are idle blocks (-1).
__global__ void __launch_bounds__(kOrderBlock) k_prep_place(int32_t N, int32_t E, const int32_t* __restrict__ row_ptr,
                                                             const int32_t* __restrict__ cnt, int32_t* bins,
                                                             const int32_t* __restrict__ bsum, int32_t* __restrict__ srow,
                                                             int32_t* __restrict__ rorder, int32_t* __restrict__ sorder)
{
    __shared__ int32_t hin[kDegBins], hout[kDegBins], bin_in[kDegBins], bin_out[kDegBins], tot[16];
    const int t = threadIdx.x;
    const int32_t blk = (int32_t)blockIdx.x;
    const int64_t i64 = (int64_t)blk * kOrderBlock + t;
    const int32_t i = i64 < N ? (int32_t)i64 : N;  // i == N: no node
    hin[t] = 0;
    hout[t] = 0;
    // sender offsets
    int32_t before = 0;
    for (int32_t k = t; k < blk; k += kOrderBlock) before += bsum[k];
    int32_t base;
    block_scan_1024(before, tot, &base);
    int32_t din = 0, dout = 0;
    if (i < N) {
        const int32_t e0 = clampi(row_ptr[i], 0, E), e1 = clampi(row_ptr[i + 1], e0, E);
        din = e1 - e0;
        dout = cnt[(int64_t)i * kCounterStride];
    }
    int32_t tt;
    const int32_t incl = block_scan_1024(dout, tot, &tt);
    if (i < N) srow[i + 1] = base + incl;
    if (i == 0) srow[0] = 0;
    // exclusive start of bin t in each schedule
    const int32_t gi = bins[t], go = bins[kDegBins + t];
    const int32_t si = block_scan_1024(gi, tot, &tt) - gi;
    const int32_t so = block_scan_1024(go, tot, &tt) - go;
    if (i < N) {
        atomicAdd(&hin[deg_bin(din)], 1);
        atomicAdd(&hout[deg_bin(dout)], 1);
    }
    __syncthreads();
    // this block's run of bin t, then hin/hout count the places taken in it
    bin_in[t] = hin[t] > 0 ? si + atomicAdd(&bins[2 * kDegBins + t], hin[t]) : 0;
    bin_out[t] = hout[t] > 0 ? so + atomicAdd(&bins[3 * kDegBins + t], hout[t]) : 0;
    hin[t] = 0;
    hout[t] = 0;
    __syncthreads();
    if (i < N) {
        const int bi = deg_bin(din), bo = deg_bin(dout);
        const int32_t pi = bin_in[bi] + atomicAdd(&hin[bi], 1), po = bin_out[bo] + atomicAdd(&hout[bo], 1);
        if ((uint32_t)pi < (uint32_t)N) rorder[pi] = i;
        if ((uint32_t)po < (uint32_t)N) sorder[po] = i;
    }
    if (blk == (int32_t)gridDim.x - 1) {
        const int64_t grid = kXcds * (((int64_t)N + kXcds - 1) / kXcds);
        if ((int64_t)N + t < grid) {
            rorder[N + t] = -1;
            sorder[N + t] = -1;
        }
    }
}

// Step 4, one wave per receiver i: place every in-edge of i in its sender's
// bucket of the unsorted view at the rank step 2 gave it (arrival order
// inside a bucket), with i beside it.
__global__ void __launch_bounds__(256) k_prep_scatter(int32_t N, int32_t E, const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ src, const int32_t* __restrict__ srow,
                                                       const int32_t* __restrict__ urank, int32_t* __restrict__ uperm,
                                                       int32_t* __restrict__ usdst)
{
    const int32_t i = (int32_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= N) return;
    int32_t e0, e1;
    segment(row_ptr, i, E, e0, e1);
    for (int32_t e = e0 + (threadIdx.x & 63); e < e1; e += 64) {
        const int32_t j = valid_node(src[e], N);
        const int32_t k = srow[j] + urank[e];
        if ((uint32_t)k < (uint32_t)E) {
            uperm[k] = e;
            usdst[k] = i;
        }
    }
}

constexpr int kBucketLds = 1024;  // bucket entries a wave ranks in one LDS tile

// Order this wave's LDS writes before its lanes read what other lanes wrote.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Step 5, one wave per sender j: write j's bucket of the view ordered by edge
// id (edge ids are distinct, so an entry's place is the number of smaller
// ids in the bucket).  A bucket of up to kBucketLds entries is ranked against
// itself in LDS; a longer one (a hub) ranks each 1024-entry chunk against the
// whole bucket one LDS tile at a time, O(n^2/64) steps per wave.
__global__ void __launch_bounds__(256) k_prep_sort(int32_t N, int32_t E, const int32_t* __restrict__ srow,
                                                    const int32_t* __restrict__ uperm,
                                                    const int32_t* __restrict__ usdst, int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ sdst)
{
    __shared__ int32_t ebuf[4][kBucketLds], ibuf[4][kBucketLds];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int32_t j = (int32_t)blockIdx.x * 4 + w;
    if (j >= N) return;  // whole wave; no block-level barrier below
    const int32_t b = clampi(srow[j], 0, E);
    const int32_t n = clampi(srow[j + 1], b, E) - b;
    int32_t* se = ebuf[w];
    if (n <= kBucketLds) {
        int32_t* si = ibuf[w];
        for (int32_t k = lane; k < n; k += 64) {
            se[k] = uperm[b + k];
            si[k] = usdst[b + k];
        }
        wave_lds_sync();
        for (int32_t k = lane; k < n; k += 64) {
            const int32_t v = se[k];
            int32_t rank = 0;
            for (int32_t t = 0; t < n; ++t) rank += se[t] < v ? 1 : 0;
            perm[b + rank] = v;
            sdst[b + rank] = si[k];
        }
        return;
    }
    constexpr int kPer = kBucketLds / 64;  // entries of a chunk per lane
    for (int32_t c = 0; c < n; c += kBucketLds) {
        int32_t v[kPer], r[kPer], rank[kPer];
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int32_t idx = c + lane + 64 * t;
            v[t] = idx < n ? uperm[b + idx] : INT_MAX;
            r[t] = idx < n ? usdst[b + idx] : 0;
            rank[t] = 0;
        }
        for (int32_t c2 = 0; c2 < n; c2 += kBucketLds) {
            const int32_t m = n - c2 < kBucketLds ? n - c2 : kBucketLds;
            wave_lds_sync();  // the previous tile's reads are done
            for (int32_t k = lane; k < m; k += 64) se[k] = uperm[b + c2 + k];
            wave_lds_sync();
            for (int32_t u = 0; u < m; ++u) {
                const int32_t y = se[u];
#pragma unroll
                for (int t = 0; t < kPer; ++t) rank[t] += y < v[t] ? 1 : 0;
            }
        }
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int32_t idx = c + lane + 64 * t;
            if (idx < n && (uint32_t)rank[t] < (uint32_t)n) {
                perm[b + rank[t]] = v[t];
                sdst[b + rank[t]] = r[t];
            }
        }
    }
}

hipError_t launch_graph_prepare(int32_t N, int32_t E, const int32_t* row_ptr, const int32_t* src, void* ws,
                                bool locality, hipStream_t s)
{
    const WsLayout L = ws_layout(N, E);
    char* base = (char*)ws;
    auto at = [&](size_t off) { return (int32_t*)(base + off); };
    int32_t *srow = at(L.srow), *perm = at(L.perm), *sdst = at(L.sdst), *uperm = at(L.uperm), *usdst = at(L.usdst);
    int32_t *cnt = at(L.cnt), *center = at(L.center), *crank = at(L.crank);
    // the edges' ranks inside their senders' buckets live in perm until step 5
    // writes the sorted view over them
    int32_t* urank = perm;
    int32_t *ccnt = at(L.ccnt), *coff = at(L.coff), *rorder = at(L.rorder), *sorder = at(L.sorder);
    uint64_t* key1 = (uint64_t*)(base + L.key1);
    const unsigned b4 = (unsigned)((N + 3) / 4);
    const int32_t loc = locality ? 1 : 0;
    int32_t *bins = at(L.bins), *bsum = at(L.bsum);
    if (N > 0) {
        hipLaunchKernelGGL(k_prep_keys, dim3(b4), dim3(256), 0, s, N, E, row_ptr, src, loc, key1, cnt, ccnt, bins);
        hipLaunchKernelGGL(k_prep_centers, dim3(b4), dim3(256), 0, s, N, E, row_ptr, src, loc, key1, center, crank,
                           ccnt, cnt, urank);
    }
    if (N > 0 && !locality) {
        const unsigned nb = (unsigned)((N + kOrderBlock - 1) / kOrderBlock);
        hipLaunchKernelGGL(k_prep_hist, dim3(nb), dim3(kOrderBlock), 0, s, N, E, row_ptr, cnt, bins, bsum);
        hipLaunchKernelGGL(k_prep_place, dim3(nb), dim3(kOrderBlock), 0, s, N, E, row_ptr, cnt, bins, bsum, srow,
                           rorder, sorder);
    } else {
        hipLaunchKernelGGL(k_prep_orders, dim3(1), dim3(1024), 0, s, N, E, loc, row_ptr, cnt, ccnt, center, crank,
                           srow, coff, rorder, sorder);
    }
    if (E > 0 && N > 0) {
        hipLaunchKernelGGL(k_prep_scatter, dim3(b4), dim3(256), 0, s, N, E, row_ptr, src, srow, urank, uperm, usdst);
        hipLaunchKernelGGL(k_prep_sort, dim3(b4), dim3(256), 0, s, N, E, srow, uperm, usdst, perm, sdst);
    }
    return hipGetLastError();
}

}  // namespace cgtp
