// cgtp_internal.h -- workspace layout, kernel arguments and the launcher
// table shared by the C-ABI layer, the graph preparation and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace cgtp {

// Blocks of one launch are dealt to the chip's eight XCDs in turn (block b
// runs on XCD b % 8), each XCD with its own L2.
constexpr int kXcds = 8;

// Largest path count of any compiled degree set (l_in = l_sh = l_out = 3).
constexpr int kMaxPaths = 34;

// Byte offsets of the graph view inside the caller's workspace.
struct WsLayout {
    size_t srow, perm, sdst, uperm, usdst, cnt, key1, center, crank, ccnt, coff, rorder, sorder, bins, bsum,
        total;
};

// degree bins of the longest-first block schedules (degrees >= kDegBins-1
// share the first bin), and the nodes per block of the multi-block schedule
// kernels
constexpr int kDegBins = 1024;
constexpr int kOrderBlock = 1024;

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// the per-sender counters of the graph preparation are spaced one 128-byte
// cache line apart, so their atomic updates do not serialise on shared lines
constexpr int kCounterStride = 32;

// grid size of the convolution kernels: N rounded up to a multiple of kXcds
// (the locality schedule splits the nodes into kXcds ranges of ceil(N/kXcds))
inline int64_t conv_grid(int64_t N) { return kXcds * ((N + kXcds - 1) / kXcds); }

inline WsLayout ws_layout(int64_t N, int64_t E)
{
    WsLayout w{};
    const size_t n1 = (size_t)(N > 0 ? N : 1), e1 = (size_t)(E > 0 ? E : 1);
    const size_t grid = (size_t)(conv_grid(N) > 0 ? conv_grid(N) : 1);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += align256(bytes);
        return at;
    };
    w.srow = take(sizeof(int32_t) * (n1 + 1));
    w.perm = take(sizeof(int32_t) * e1);
    w.sdst = take(sizeof(int32_t) * e1);
    w.uperm = take(sizeof(int32_t) * e1);  // the view before its buckets are sorted
    w.usdst = take(sizeof(int32_t) * e1);
    w.cnt = take(sizeof(int32_t) * kCounterStride * n1);
    w.key1 = take(sizeof(uint64_t) * n1);
    w.center = take(sizeof(int32_t) * n1);
    w.crank = take(sizeof(int32_t) * n1);
    w.ccnt = take(sizeof(int32_t) * n1);
    w.coff = take(sizeof(int32_t) * n1);
    w.rorder = take(sizeof(int32_t) * grid);
    w.sorder = take(sizeof(int32_t) * grid);
    // global degree-bin counts and claim cursors (receiver and sender
    // schedules), and the out-degree sum of every kOrderBlock nodes
    w.bins = take(sizeof(int32_t) * 4 * kDegBins);
    w.bsum = take(sizeof(int32_t) * ((n1 + kOrderBlock - 1) / kOrderBlock));
    w.total = o;
    return w;
}

// The sender-sorted view of the receiver CSR and the block schedules.
struct GraphView {
    const int32_t* srow;    // [N+1] sender offsets
    const int32_t* perm;    // [E]  edge ids grouped by sender, ascending within a sender
    const int32_t* sdst;    // [E]  receiver of perm[k]
    const int32_t* rorder;  // [conv_grid(N)] receiver of each forward block (-1: idle block)
    const int32_t* sorder;  // [conv_grid(N)] sender of each backward block (-1: idle block)
};

// Degrees and channel count of a launch.  The kernels are compiled for the
// full path set of degree LM (l_in = l_sh = l_out = LM); a plan with smaller
// degrees runs the paths it has (bit p of `active`) and reads path p's
// weights at element offset woff[p] (a multiple of C) inside the edge's
// [P][C] weight row.  With path-weight sharing the row is [1][C]: every
// woff[p] is 0 and the backward sums grad_W over the paths.
//
// With per-path outputs (mid = 1) the output and grad_out rows are not summed
// per l3: path p owns rows moff[p] .. moff[p] + 2*l3 of a node's d_out =
// sum_p (2*l3 + 1) rows (moff[p] = -1 for a compiled path the plan lacks).
struct Shape {
    int32_t N, E, C;
    int32_t d_in, d_sh, d_out;  // row widths: (l+1)^2 of the plan's degrees (d_out: per-path rows when mid)
    int32_t P;                  // weight rows per edge: the plan's path count, or 1 when shared
    int32_t shared;             // 1: one weight per edge and channel for every path
    int32_t mid;                // 1: one output block per path
    uint64_t active;            // compiled paths the plan uses
    int32_t woff[kMaxPaths];    // weight offset of every compiled path (clamped for inactive ones)
    int32_t moff[kMaxPaths];    // per-path outputs: first output row of every compiled path, or -1
};

enum GradMask : int { kGradX = 1, kGradW = 2, kGradY = 4 };

// The double-backward launches read the cotangents ggx, ggY, ggW as well
// (nullptr: zero); the others leave them unset.
struct FwdArgs {
    Shape sh;
    const int32_t* row_ptr;
    const int32_t* src;
    const int32_t* rorder;
    const float* x;
    const float* Y;
    const float* W;
    float* out;
    const float* ggx;
    const float* ggY;
    const float* ggW;
    const float* r;  // edge vectors [E][3] of the fused-SH kernels (Y is then unused)
};

struct BwdArgs {
    Shape sh;
    GraphView g;
    const float* x;
    const float* Y;
    const float* W;
    const float* G;
    float* dx;
    float* dW;
    float* dY;
    const float* ggx;
    const float* ggY;
    const float* ggW;
    const float* r;  // edge vectors [E][3] of the fused-SH kernels (Y, dY are then unused)
    float* dr;       // their gradient [E][3]
};

using ShLaunch = hipError_t (*)(int64_t E, const float* r, float* Y, hipStream_t s);
using FwdLaunch = hipError_t (*)(const FwdArgs& a, hipStream_t s);
using BwdLaunch = hipError_t (*)(const BwdArgs& a, hipStream_t s);

// The kernels of one compiled degree LM and one lane geometry: LPE lanes per
// edge slice and H slices (waves) per edge; they serve every channel count C
// with LPE*(H-1) < C <= LPE*H (lanes beyond C idle).
struct KernelSet {
    int lm, lpe, h;
    FwdLaunch fwd[2];  // [0]: complete degree set; [1]: SUB (smaller or mixed degrees)
    BwdLaunch bwd[2];
    // double backward (every degree set, SUB form): fwd_dbl writes the
    // gradient for grad_out into `out`, bwd_dbl those for x, W and Y into
    // dx, dW and dY
    FwdLaunch fwd_dbl;
    BwdLaunch bwd_dbl;
    // per-path outputs (SUB form): fwd_mid writes every path's block of
    // `out` (one launch per group of paths), bwd_mid reads every path's block
    // of grad_out
    FwdLaunch fwd_mid;
    BwdLaunch bwd_mid;
    // spherical harmonics evaluated inside the kernels from the edge vectors r
    // ([0] complete degree set, [1] SUB): fwd_sh reads r instead of Y, bwd_sh
    // writes grad_r (through the SH Jacobian) instead of grad_Y
    FwdLaunch fwd_sh[2];
    BwdLaunch bwd_sh[2];
};

// Kernels for compiled degree lm and channel count C, or nullptr.
const KernelSet* find_kernels(int lm, int channels);

// Real spherical harmonics of degrees 0..l (l <= 3), or nullptr.
ShLaunch find_sh(int l);

// Their backward: grad_r[E][3] from grad_Y[E][(l+1)^2] (l <= 3), or nullptr.
using ShBwdLaunch = hipError_t (*)(int64_t E, const float* r, const float* gY, float* gr, hipStream_t s);
ShBwdLaunch find_sh_bwd(int l);

// Per-node gradient gpos[N][3] = sum over out-edges of grad_r - sum over
// in-edges, over the prepared view g.
hipError_t launch_node_grad(int32_t N, int32_t E, const int32_t* row_ptr, const GraphView& g, const float* gr,
                            float* gpos, hipStream_t s);

// Graph preparation into `ws` (layout ws_layout(N, E)).  `locality` selects
// the cluster-ordered block schedule (false: longest first), see cgtp_graph.hip.
hipError_t launch_graph_prepare(int32_t N, int32_t E, const int32_t* row_ptr, const int32_t* src, void* ws,
                                bool locality, hipStream_t s);

// Host copy of the real CG table of path `path` of the compiled degree lm
// (the same constexpr tables the kernels are compiled with).
bool host_cg_table(int lm, int path, double* dense);

}  // namespace cgtp
