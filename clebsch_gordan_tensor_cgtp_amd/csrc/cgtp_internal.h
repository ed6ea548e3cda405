// cgtp_internal.h -- launcher table shared by the C-ABI layer and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace cgtp {

// Byte offsets of the sender-sorted graph view inside the workspace.
struct WsLayout {
    size_t srow, perm, sdst, cnt, cursor, rorder, sorder, dyp, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// the per-sender counters and cursors of the graph preparation are spaced one
// 128-byte cache line apart, so their atomic updates do not serialise on
// shared lines
constexpr int kCounterStride = 32;

// dyp_per_edge: fp64 values per edge of the grad_Y slice partials (0 when the
// plan's channels fit one 64-lane slice)
inline WsLayout ws_layout(int64_t N, int64_t E, int64_t dyp_per_edge = 0)
{
    WsLayout w{};
    size_t o = 0;
    w.srow = o;
    o += align256(sizeof(int32_t) * (size_t)(N + 1));
    w.perm = o;
    o += align256(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    w.sdst = o;
    o += align256(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    w.cnt = o;
    o += align256(sizeof(int32_t) * kCounterStride * (size_t)(N > 0 ? N : 1));
    w.cursor = o;
    o += align256(sizeof(int32_t) * kCounterStride * (size_t)(N > 0 ? N : 1));
    w.rorder = o;
    o += align256(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
    w.sorder = o;
    o += align256(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
    w.dyp = o;
    o += align256(sizeof(double) * (size_t)(E > 0 ? E : 0) * (size_t)dyp_per_edge);
    w.total = o;
    return w;
}

struct GraphView {
    const int32_t* srow;    // [N+1] sender offsets
    const int32_t* perm;    // [E]  edge ids grouped by sender
    const int32_t* sdst;    // [E]  receiver of perm[k]
    const int32_t* sorder;  // [N]  senders, longest out-edge list first
    double* dyp;            // [E][H][D_sh] grad_Y slice partials (C > 64 only)
    int32_t n_edges;        // E
};

enum GradMask : int { kGradX = 1, kGradW = 2, kGradY = 4 };

using ShLaunch = hipError_t (*)(int64_t E, const float* r, float* Y, hipStream_t s);
using FwdLaunch = hipError_t (*)(int32_t N, const int32_t* row_ptr, const int32_t* src, const int32_t* rorder,
                                 const float* x, const float* Y, const float* W, float* out, hipStream_t s);
using BwdLaunch = hipError_t (*)(int32_t N, GraphView g, const float* x, const float* Y, const float* W,
                                 const float* G, float* dx, float* dW, float* dY, int mask, hipStream_t s);

struct KernelSet {
    int l_in, l_sh, l_out, channels;
    int dyp_per_edge;  // workspace fp64 values per edge for grad_Y slice partials
    ShLaunch sh;
    FwdLaunch fwd;
    BwdLaunch bwd;
};

// Kernels compiled for (l_in, l_sh, l_out, C), or nullptr.
const KernelSet* find_kernels(int l_in, int l_sh, int l_out, int channels);

// Graph preparation into `ws` (layout ws_layout(N, E)).
hipError_t launch_graph_prepare(int32_t N, int32_t E, const int32_t* row_ptr, const int32_t* src, void* ws,
                                hipStream_t s);

// Host copy of the real CG table for a path (the same constexpr tables the
// kernels are compiled with).
bool host_cg_table(int l_in, int l_sh, int l_out, int path, double* dense);

}  // namespace cgtp
