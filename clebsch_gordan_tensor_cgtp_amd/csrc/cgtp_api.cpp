// cgtp_api.cpp -- the C ABI of libcgtp.so (see include/cgtp.h): plans,
// argument checks, workspace sizing and records, and dispatch to the gfx950
// kernels.
#include "cgtp.h"

#include <hip/hip_runtime.h>

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "cgtp_cp.h"
#include "cgtp_internal.h"
#include "cgtp_math.h"
#include "cgtp_mix.h"

struct cgtp_plan_s {
    int l_in, l_sh, l_out, channels;
    unsigned flags;
    int P, d_in, d_sh, d_out;
    int lm;                         // compiled degree serving this plan
    bool sub;                       // degrees other than (lm, lm, lm)
    bool mid;                       // per-path outputs
    int d_mid;                      // their row count, sum of 2*l3+1
    std::vector<int> paths;         // [P][3]
    std::vector<int> super_index;   // [P]: index of each path in the compiled degree's path list
    cgtp::Shape shape;              // N and E filled in per call
    const cgtp::KernelSet* ks;
    cgtp::ShLaunch sh;
    cgtp::ShBwdLaunch sh_bwd;
};

namespace {

constexpr unsigned kKnownFlags =
    CGTP_FLAG_VALIDATE | CGTP_FLAG_LOCALITY | CGTP_FLAG_SHARED_WEIGHTS | CGTP_FLAG_PATH_OUTPUTS;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

cgtp_status_t hip_status(hipError_t e) { return e == hipSuccess ? CGTP_OK : CGTP_ERR_HIP; }

// synchronous host-side CSR check (CGTP_FLAG_VALIDATE only)
cgtp_status_t validate_graph(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src)
{
    std::vector<int32_t> rp((size_t)N + 1), s((size_t)(E > 0 ? E : 1));
    if (hipMemcpy(rp.data(), row_ptr, sizeof(int32_t) * (size_t)(N + 1), hipMemcpyDeviceToHost) != hipSuccess)
        return CGTP_ERR_HIP;
    if (E > 0 && hipMemcpy(s.data(), src, sizeof(int32_t) * (size_t)E, hipMemcpyDeviceToHost) != hipSuccess)
        return CGTP_ERR_HIP;
    if (rp[0] != 0 || rp[(size_t)N] != E) return CGTP_ERR_GRAPH;
    for (int64_t i = 0; i < N; ++i)
        if (rp[(size_t)i + 1] < rp[(size_t)i]) return CGTP_ERR_GRAPH;
    for (int64_t e = 0; e < E; ++e)
        if (s[(size_t)e] < 0 || s[(size_t)e] >= N) return CGTP_ERR_GRAPH;
    return CGTP_OK;
}

cgtp_status_t check_graph_args(const cgtp_plan_s* plan, int64_t N, int64_t E, const int32_t* row_ptr,
                               const int32_t* src)
{
    if (!plan) return CGTP_ERR_INVALID_ARG;
    if (N < 0 || E < 0 || N >= (int64_t)INT32_MAX || E >= (int64_t)INT32_MAX) return CGTP_ERR_INVALID_ARG;
    if (!row_ptr || !aligned16(row_ptr)) return CGTP_ERR_INVALID_ARG;
    if (E > 0 && (!src || !aligned16(src))) return CGTP_ERR_INVALID_ARG;
    if (plan->flags & CGTP_FLAG_VALIDATE) return validate_graph(N, E, row_ptr, src);
    return CGTP_OK;
}

cgtp_status_t check_ws(int64_t N, int64_t E, const void* ws, size_t ws_bytes)
{
    if (!ws || ws_bytes < cgtp::ws_layout(N, E).total) return CGTP_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return CGTP_ERR_INVALID_ARG;
    return CGTP_OK;
}

// ---- records of prepared workspaces -----------------------------------------
// A workspace counts as prepared for a graph when the last preparation into
// it (on the same device) was for the same sizes and graph arrays and the
// same schedule kind.
struct Prepared {
    int64_t N, E;
    const void* row_ptr;
    const void* src;
    bool locality;
    int device;
};

std::mutex g_mu;
std::unordered_map<const void*, Prepared>& records()
{
    static std::unordered_map<const void*, Prepared> m;
    return m;
}

cgtp_status_t prepare_into(const cgtp_plan_s* plan, int64_t N, int64_t E, const int32_t* row_ptr,
                           const int32_t* src, void* ws, hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CGTP_ERR_HIP;
    const bool loc = (plan->flags & CGTP_FLAG_LOCALITY) != 0;
    const hipError_t e = cgtp::launch_graph_prepare((int32_t)N, (int32_t)E, row_ptr, src, ws, loc, stream);
    std::lock_guard<std::mutex> lk(g_mu);
    if (e != hipSuccess) {
        records().erase(ws);
        return CGTP_ERR_HIP;
    }
    records()[ws] = Prepared{N, E, row_ptr, src, loc, dev};
    return CGTP_OK;
}

// run the preparation unless `ws` already holds this graph's view
cgtp_status_t ensure_prepared(const cgtp_plan_s* plan, int64_t N, int64_t E, const int32_t* row_ptr,
                              const int32_t* src, void* ws, hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CGTP_ERR_HIP;
    const bool loc = (plan->flags & CGTP_FLAG_LOCALITY) != 0;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = records().find(ws);
        if (it != records().end()) {
            const Prepared& r = it->second;
            if (r.N == N && r.E == E && r.row_ptr == row_ptr && r.src == src && r.locality == loc && r.device == dev)
                return CGTP_OK;
        }
    }
    return prepare_into(plan, N, E, row_ptr, src, ws, stream);
}

// ---- the allocation-free backward's scratch --------------------------------
// A file-scope device array holds the graph view for cgtp_conv_bwd_noalloc.
// Host code never passes `scratch` itself (in host code the name is only a
// stand-in for the symbol): each device's copy is looked up once with
// hipGetSymbolAddress and that address is used.  The record of which graph
// the scratch holds is a fixed per-device slot, so this path allocates
// nothing, host or device.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchSlot {
    void* ptr;        // this device's copy of `scratch`, or nullptr until set up
    bool valid;       // rec holds the graph last prepared into it
    Prepared rec;
};
ScratchSlot g_scratch[kMaxDevices];

// this device's scratch address (looked up on its first use, with the device current)
cgtp_status_t scratch_ptr(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return CGTP_ERR_UNSUPPORTED;
    ScratchSlot& s = g_scratch[dev];
    if (!s.ptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CGTP_ERR_HIP;
        s.ptr = p;
    }
    *out = s.ptr;
    return CGTP_OK;
}

cgtp::Shape launch_shape(const cgtp_plan_s* plan, int64_t N, int64_t E)
{
    cgtp::Shape s = plan->shape;
    s.N = (int32_t)N;
    s.E = (int32_t)E;
    return s;
}

}  // namespace

extern "C" {

cgtp_status_t cgtp_plan_create(cgtp_plan_t* plan, int l_in, int l_sh, int l_out, int channels, unsigned flags)
{
    if (!plan) return CGTP_ERR_INVALID_ARG;
    *plan = nullptr;
    if (l_in < 0 || l_sh < 0 || l_out < 0 || channels <= 0) return CGTP_ERR_INVALID_ARG;
    if (flags & ~kKnownFlags) return CGTP_ERR_INVALID_ARG;
    if (l_in > cgtp::cgmath::kMaxL || l_sh > cgtp::cgmath::kMaxL || l_out > cgtp::cgmath::kMaxL)
        return CGTP_ERR_UNSUPPORTED;
    const int lm = std::max(1, std::max(l_in, std::max(l_sh, l_out)));
    const cgtp::KernelSet* ks = cgtp::find_kernels(lm, channels);
    const cgtp::ShLaunch sh = cgtp::find_sh(l_sh);
    const cgtp::ShBwdLaunch sh_bwd = cgtp::find_sh_bwd(l_sh);
    if (!ks || !sh || !sh_bwd) return CGTP_ERR_UNSUPPORTED;
    cgtp_plan_s* p = new (std::nothrow) cgtp_plan_s();
    if (!p) return CGTP_ERR_ALLOC;
    p->l_in = l_in;
    p->l_sh = l_sh;
    p->l_out = l_out;
    p->channels = channels;
    p->flags = flags;
    p->lm = lm;
    const bool shared = (flags & CGTP_FLAG_SHARED_WEIGHTS) != 0;
    p->mid = (flags & CGTP_FLAG_PATH_OUTPUTS) != 0;
    p->sub = shared || !(l_in == lm && l_sh == lm && l_out == lm);
    p->P = cgtp::cgmath::num_paths(l_in, l_sh, l_out);
    p->d_in = (l_in + 1) * (l_in + 1);
    p->d_sh = (l_sh + 1) * (l_sh + 1);
    p->d_out = (l_out + 1) * (l_out + 1);
    p->paths.resize(3 * (size_t)p->P);
    for (int q = 0; q < p->P; ++q) {
        const cgtp::cgmath::Path t = cgtp::cgmath::path_at(l_in, l_sh, l_out, q);
        p->paths[3 * q + 0] = t.l1;
        p->paths[3 * q + 1] = t.l2;
        p->paths[3 * q + 2] = t.l3;
    }
    // the compiled degree's paths this plan has, and where each one's weights sit
    cgtp::Shape s{};
    s.C = channels;
    s.d_in = p->d_in;
    s.d_sh = p->d_sh;
    s.d_out = p->d_out;
    s.P = shared ? 1 : p->P;
    s.shared = shared ? 1 : 0;
    const int Pm = cgtp::cgmath::num_paths(lm, lm, lm);
    int q = 0, rows = 0;
    for (int k = 0; k < Pm; ++k) {
        const cgtp::cgmath::Path t = cgtp::cgmath::path_at(lm, lm, lm, k);
        const bool mine = t.l1 <= l_in && t.l2 <= l_sh && t.l3 <= l_out;
        if (mine) {
            s.active |= uint64_t(1) << k;
            p->super_index.push_back(k);
        }
        // an inactive path reads a valid row (and gets weight 0)
        s.woff[k] = shared ? 0 : std::min(q, p->P - 1) * channels;
        // per-path outputs: the path's first row, in the plan's path order
        s.moff[k] = mine ? rows : -1;
        if (mine) {
            ++q;
            rows += 2 * t.l3 + 1;
        }
    }
    p->d_mid = rows;
    if (p->mid) {
        s.mid = 1;
        s.d_out = rows;
    }
    p->shape = s;
    p->ks = ks;
    p->sh = sh;
    p->sh_bwd = sh_bwd;
    *plan = p;
    return CGTP_OK;
}

cgtp_status_t cgtp_plan_destroy(cgtp_plan_t plan)
{
    delete plan;
    return CGTP_OK;
}

cgtp_status_t cgtp_plan_info(cgtp_plan_t plan, int* num_paths, int* paths_l1l2l3, int* dim_in, int* dim_sh,
                             int* dim_out)
{
    if (!plan) return CGTP_ERR_INVALID_ARG;
    if (num_paths) *num_paths = plan->P;
    if (paths_l1l2l3) memcpy(paths_l1l2l3, plan->paths.data(), sizeof(int) * plan->paths.size());
    if (dim_in) *dim_in = plan->d_in;
    if (dim_sh) *dim_sh = plan->d_sh;
    if (dim_out) *dim_out = plan->mid ? plan->d_mid : plan->d_out;
    return CGTP_OK;
}

cgtp_status_t cgtp_plan_export_cg(cgtp_plan_t plan, int path, double* dense)
{
    if (!plan || !dense || path < 0 || path >= plan->P) return CGTP_ERR_INVALID_ARG;
    return cgtp::host_cg_table(plan->lm, plan->super_index[(size_t)path], dense) ? CGTP_OK : CGTP_ERR_UNSUPPORTED;
}

cgtp_status_t cgtp_workspace_size(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, size_t* bytes)
{
    if (!plan || !bytes || n_nodes < 0 || n_edges < 0) return CGTP_ERR_INVALID_ARG;
    *bytes = cgtp::ws_layout(n_nodes, n_edges).total;
    return CGTP_OK;
}

cgtp_status_t cgtp_sh_fwd(cgtp_plan_t plan, int64_t n_edges, const float* r, float* Y, hipStream_t stream)
{
    if (!plan || n_edges < 0) return CGTP_ERR_INVALID_ARG;
    if (n_edges == 0) return CGTP_OK;
    if (!r || !Y || !aligned16(Y) || !aligned16(r)) return CGTP_ERR_INVALID_ARG;
    return hip_status(plan->sh(n_edges, r, Y, stream));
}

cgtp_status_t cgtp_sh_bwd(cgtp_plan_t plan, int64_t n_edges, const float* r, const float* grad_Y, float* grad_r,
                          hipStream_t stream)
{
    if (!plan || n_edges < 0) return CGTP_ERR_INVALID_ARG;
    if (n_edges == 0) return CGTP_OK;
    if (!r || !grad_Y || !grad_r || !aligned16(r) || !aligned16(grad_Y) || !aligned16(grad_r))
        return CGTP_ERR_INVALID_ARG;
    return hip_status(plan->sh_bwd(n_edges, r, grad_Y, grad_r, stream));
}

cgtp_status_t cgtp_node_grad(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                             const int32_t* src, const float* grad_r, float* grad_pos, void* ws, size_t ws_bytes,
                             hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    st = check_ws(n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    if (n_nodes == 0) return CGTP_OK;
    if (!grad_pos || !aligned16(grad_pos)) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && (!grad_r || !aligned16(grad_r))) return CGTP_ERR_INVALID_ARG;
    st = ensure_prepared(plan, n_nodes, n_edges, row_ptr, src, ws, stream);
    if (st != CGTP_OK) return st;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges);
    const char* base = (const char*)ws;
    const cgtp::GraphView g{(const int32_t*)(base + L.srow), (const int32_t*)(base + L.perm),
                            (const int32_t*)(base + L.sdst), (const int32_t*)(base + L.rorder),
                            (const int32_t*)(base + L.sorder)};
    return hip_status(
        cgtp::launch_node_grad((int32_t)n_nodes, (int32_t)n_edges, row_ptr, g, grad_r, grad_pos, stream));
}

cgtp_status_t cgtp_graph_prepare(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                                 const int32_t* src, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    st = check_ws(n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    return prepare_into(plan, n_nodes, n_edges, row_ptr, src, ws, stream);
}

cgtp_status_t cgtp_conv_fwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const float* x, const float* Y, const float* W, float* out,
                            void* ws, size_t ws_bytes, hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    st = check_ws(n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    if (n_nodes == 0) return CGTP_OK;
    if (!out || !aligned16(out) || !x || !aligned16(x)) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && (!Y || !W || !aligned16(W) || !aligned16(Y))) return CGTP_ERR_INVALID_ARG;
    st = ensure_prepared(plan, n_nodes, n_edges, row_ptr, src, ws, stream);
    if (st != CGTP_OK) return st;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges);
    cgtp::FwdArgs a{};
    a.sh = launch_shape(plan, n_nodes, n_edges);
    a.row_ptr = row_ptr;
    a.src = src;
    a.rorder = (const int32_t*)((const char*)ws + L.rorder);
    a.x = x;
    a.Y = Y;
    a.W = W;
    a.out = out;
    if (plan->mid) return hip_status(plan->ks->fwd_mid(a, stream));
    return hip_status(plan->ks->fwd[plan->sub ? 1 : 0](a, stream));
}

cgtp_status_t cgtp_conv_bwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const float* x, const float* Y, const float* W,
                            const float* grad_out, float* grad_x, float* grad_W, float* grad_Y, void* ws,
                            size_t ws_bytes, hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    st = check_ws(n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    if ((!grad_x && !grad_W && !grad_Y) || n_nodes == 0) return CGTP_OK;
    if (!x || !aligned16(x) || !grad_out || !aligned16(grad_out)) return CGTP_ERR_INVALID_ARG;
    if (grad_x && !aligned16(grad_x)) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && (!Y || !W || !aligned16(W) || !aligned16(Y))) return CGTP_ERR_INVALID_ARG;
    if (grad_W && !aligned16(grad_W)) return CGTP_ERR_INVALID_ARG;
    if (grad_Y && !aligned16(grad_Y)) return CGTP_ERR_INVALID_ARG;
    st = ensure_prepared(plan, n_nodes, n_edges, row_ptr, src, ws, stream);
    if (st != CGTP_OK) return st;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges);
    const char* base = (const char*)ws;
    cgtp::BwdArgs a{};
    a.sh = launch_shape(plan, n_nodes, n_edges);
    a.g = cgtp::GraphView{(const int32_t*)(base + L.srow), (const int32_t*)(base + L.perm),
                          (const int32_t*)(base + L.sdst), (const int32_t*)(base + L.rorder),
                          (const int32_t*)(base + L.sorder)};
    a.x = x;
    a.Y = Y;
    a.W = W;
    a.G = grad_out;
    a.dx = grad_x;
    a.dW = grad_W;
    a.dY = grad_Y;
    if (plan->mid) return hip_status(plan->ks->bwd_mid(a, stream));
    return hip_status(plan->ks->bwd[plan->sub ? 1 : 0](a, stream));
}

cgtp_status_t cgtp_conv_fwd_sh(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                               const int32_t* src, const float* x, const float* r, const float* W, float* out,
                               void* ws, size_t ws_bytes, hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    if (plan->mid) return CGTP_ERR_UNSUPPORTED;
    st = check_ws(n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    if (n_nodes == 0) return CGTP_OK;
    if (!out || !aligned16(out) || !x || !aligned16(x)) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && (!r || !W || !aligned16(W) || !aligned16(r))) return CGTP_ERR_INVALID_ARG;
    st = ensure_prepared(plan, n_nodes, n_edges, row_ptr, src, ws, stream);
    if (st != CGTP_OK) return st;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges);
    cgtp::FwdArgs a{};
    a.sh = launch_shape(plan, n_nodes, n_edges);
    a.row_ptr = row_ptr;
    a.src = src;
    a.rorder = (const int32_t*)((const char*)ws + L.rorder);
    a.x = x;
    a.r = r;
    a.W = W;
    a.out = out;
    return hip_status(plan->ks->fwd_sh[plan->sub ? 1 : 0](a, stream));
}

cgtp_status_t cgtp_conv_bwd_sh(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                               const int32_t* src, const float* x, const float* r, const float* W,
                               const float* grad_out, float* grad_x, float* grad_W, float* grad_r, void* ws,
                               size_t ws_bytes, hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    if (plan->mid) return CGTP_ERR_UNSUPPORTED;
    st = check_ws(n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    if ((!grad_x && !grad_W && !grad_r) || n_nodes == 0) return CGTP_OK;
    if (!x || !aligned16(x) || !grad_out || !aligned16(grad_out)) return CGTP_ERR_INVALID_ARG;
    if (grad_x && !aligned16(grad_x)) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && (!r || !W || !aligned16(W) || !aligned16(r))) return CGTP_ERR_INVALID_ARG;
    if (grad_W && !aligned16(grad_W)) return CGTP_ERR_INVALID_ARG;
    if (grad_r && !aligned16(grad_r)) return CGTP_ERR_INVALID_ARG;
    st = ensure_prepared(plan, n_nodes, n_edges, row_ptr, src, ws, stream);
    if (st != CGTP_OK) return st;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges);
    const char* base = (const char*)ws;
    cgtp::BwdArgs a{};
    a.sh = launch_shape(plan, n_nodes, n_edges);
    a.g = cgtp::GraphView{(const int32_t*)(base + L.srow), (const int32_t*)(base + L.perm),
                          (const int32_t*)(base + L.sdst), (const int32_t*)(base + L.rorder),
                          (const int32_t*)(base + L.sorder)};
    a.x = x;
    a.r = r;
    a.W = W;
    a.G = grad_out;
    a.dx = grad_x;
    a.dW = grad_W;
    a.dr = grad_r;
    return hip_status(plan->ks->bwd_sh[plan->sub ? 1 : 0](a, stream));
}

cgtp_status_t cgtp_conv_bwd_bwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                                const int32_t* src, const float* x, const float* Y, const float* W,
                                const float* grad_out, const float* gg_x, const float* gg_Y, const float* gg_W,
                                float* dd_x, float* dd_Y, float* dd_W, float* dd_out, void* ws, size_t ws_bytes,
                                hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    if (plan->mid) return CGTP_ERR_UNSUPPORTED;
    st = check_ws(n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    if ((!dd_x && !dd_Y && !dd_W && !dd_out) || n_nodes == 0) return CGTP_OK;
    if (!x || !aligned16(x) || !grad_out || !aligned16(grad_out)) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && (!Y || !W || !aligned16(W) || !aligned16(Y))) return CGTP_ERR_INVALID_ARG;
    for (const void* p : {(const void*)gg_x, (const void*)gg_Y, (const void*)gg_W, (const void*)dd_x,
                          (const void*)dd_Y, (const void*)dd_W, (const void*)dd_out})
        if (p && !aligned16(p)) return CGTP_ERR_INVALID_ARG;
    st = ensure_prepared(plan, n_nodes, n_edges, row_ptr, src, ws, stream);
    if (st != CGTP_OK) return st;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges);
    const char* base = (const char*)ws;
    if (dd_out) {
        cgtp::FwdArgs a{};
        a.sh = launch_shape(plan, n_nodes, n_edges);
        a.row_ptr = row_ptr;
        a.src = src;
        a.rorder = (const int32_t*)(base + L.rorder);
        a.x = x;
        a.Y = Y;
        a.W = W;
        a.out = dd_out;
        a.ggx = gg_x;
        a.ggY = gg_Y;
        a.ggW = gg_W;
        st = hip_status(plan->ks->fwd_dbl(a, stream));
        if (st != CGTP_OK) return st;
    }
    if (dd_x || dd_Y || dd_W) {
        cgtp::BwdArgs a{};
        a.sh = launch_shape(plan, n_nodes, n_edges);
        a.g = cgtp::GraphView{(const int32_t*)(base + L.srow), (const int32_t*)(base + L.perm),
                              (const int32_t*)(base + L.sdst), (const int32_t*)(base + L.rorder),
                              (const int32_t*)(base + L.sorder)};
        a.x = x;
        a.Y = Y;
        a.W = W;
        a.G = grad_out;
        a.dx = dd_x;
        a.dW = dd_W;
        a.dY = dd_Y;
        a.ggx = gg_x;
        a.ggY = gg_Y;
        a.ggW = gg_W;
        st = hip_status(plan->ks->bwd_dbl(a, stream));
    }
    return st;
}

// ---- fully connected mixing of the per-path outputs ----------------------------
namespace {

constexpr int kMaxMixOut = 1024;

cgtp::MixShape mix_shape(const cgtp_plan_s* plan, int64_t n_nodes, int c_out)
{
    cgtp::MixShape m{};
    m.N = (int32_t)n_nodes;
    m.C = plan->channels;
    m.Co = c_out;
    m.P = plan->P;
    m.Dmid = plan->d_mid;
    m.Dout = plan->d_out;
    int o = 0;
    for (int p = 0; p < plan->P; ++p) {
        m.l3[p] = plan->paths[3 * p + 2];
        m.o[p] = o;
        o += 2 * m.l3[p] + 1;
    }
    return m;
}

}  // namespace

cgtp_status_t cgtp_path_mix_workspace_size(cgtp_plan_t plan, int64_t n_nodes, int c_out, size_t* bytes)
{
    if (!plan || !bytes || n_nodes < 0 || n_nodes >= (int64_t)INT32_MAX || c_out < 1) return CGTP_ERR_INVALID_ARG;
    if (c_out > kMaxMixOut) return CGTP_ERR_UNSUPPORTED;
    *bytes = cgtp::mix_workspace_bytes(mix_shape(plan, n_nodes, c_out));
    return CGTP_OK;
}

cgtp_status_t cgtp_path_mix_fwd(cgtp_plan_t plan, int64_t n_nodes, int c_out, const float* mid, const float* Wmix,
                                float* out, hipStream_t stream)
{
    if (!plan || n_nodes < 0 || n_nodes >= (int64_t)INT32_MAX || c_out < 1) return CGTP_ERR_INVALID_ARG;
    if (c_out > kMaxMixOut) return CGTP_ERR_UNSUPPORTED;
    if (!Wmix || !aligned16(Wmix)) return CGTP_ERR_INVALID_ARG;
    if (n_nodes == 0) return CGTP_OK;
    if (!mid || !out || !aligned16(mid) || !aligned16(out)) return CGTP_ERR_INVALID_ARG;
    return hip_status(cgtp::launch_mix_fwd(mix_shape(plan, n_nodes, c_out), mid, Wmix, out, stream));
}

cgtp_status_t cgtp_path_mix_bwd(cgtp_plan_t plan, int64_t n_nodes, int c_out, const float* mid, const float* Wmix,
                                const float* grad_out, float* grad_mid, float* grad_Wmix, void* ws, size_t ws_bytes,
                                hipStream_t stream)
{
    if (!plan || n_nodes < 0 || n_nodes >= (int64_t)INT32_MAX || c_out < 1) return CGTP_ERR_INVALID_ARG;
    if (c_out > kMaxMixOut) return CGTP_ERR_UNSUPPORTED;
    if (!grad_mid && !grad_Wmix) return CGTP_OK;
    if (!Wmix || !aligned16(Wmix)) return CGTP_ERR_INVALID_ARG;
    if (grad_Wmix) {
        if (!aligned16(grad_Wmix)) return CGTP_ERR_INVALID_ARG;
        if (!ws || ws_bytes < cgtp::mix_workspace_bytes(mix_shape(plan, n_nodes, c_out)))
            return CGTP_ERR_WORKSPACE;
        if (((uintptr_t)ws & 255u) != 0) return CGTP_ERR_INVALID_ARG;
    }
    if (n_nodes > 0) {
        if (!mid || !grad_out || !aligned16(mid) || !aligned16(grad_out)) return CGTP_ERR_INVALID_ARG;
        if (grad_mid && !aligned16(grad_mid)) return CGTP_ERR_INVALID_ARG;
    }
    return hip_status(cgtp::launch_mix_bwd(mix_shape(plan, n_nodes, c_out), mid, Wmix, grad_out, grad_mid,
                                           grad_Wmix, (double*)ws, stream));
}

// ---- CP-decomposed tensor product ------------------------------------------
cgtp_status_t cgtp_cp_workspace_size(cgtp_plan_t plan, int rank, int64_t n_nodes, int64_t n_edges, size_t* bytes)
{
    if (!plan || !bytes || n_nodes < 0 || n_edges < 0 || rank < 1) return CGTP_ERR_INVALID_ARG;
    if (rank > cgtp::kMaxCpRank) return CGTP_ERR_UNSUPPORTED;
    *bytes = cgtp::cp_ws_layout(n_nodes, n_edges, cgtp::cp_padded_rank(rank), plan->channels).total;
    return CGTP_OK;
}

cgtp_status_t cgtp_cp_fit(cgtp_plan_t plan, int rank, int sweeps, double ridge, double* A, double* B, double* C,
                          double* rel_err)
{
    if (!plan || rank < 1 || sweeps < 0 || !(ridge >= 0.0) || !A || !B || !C) return CGTP_ERR_INVALID_ARG;
    const int d1 = plan->d_in, d2 = plan->d_sh, d3 = plan->d_out;
    std::vector<double> M((size_t)d1 * d2 * d3, 0.0), T;
    for (int p = 0; p < plan->P; ++p) {
        const int l1 = plan->paths[3 * p], l2 = plan->paths[3 * p + 1], l3 = plan->paths[3 * p + 2];
        const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
        T.assign((size_t)n1 * n2 * n3, 0.0);
        if (!cgtp::host_cg_table(plan->lm, plan->super_index[(size_t)p], T.data())) return CGTP_ERR_UNSUPPORTED;
        for (int a = 0; a < n1; ++a)
            for (int b = 0; b < n2; ++b)
                for (int c = 0; c < n3; ++c)
                    M[((size_t)(l1 * l1 + a) * d2 + (l2 * l2 + b)) * d3 + (l3 * l3 + c)] =
                        T[((size_t)a * n2 + b) * n3 + c];
    }
    return cgtp::cp_als_fit(M.data(), d1, d2, d3, rank, sweeps, ridge, A, B, C, rel_err) ? CGTP_OK
                                                                                          : CGTP_ERR_NUMERIC;
}

namespace {

// shared checks of the two CP convolution calls
cgtp_status_t cp_prepare(const cgtp_plan_s* plan, int rank, int64_t n_nodes, int64_t n_edges,
                         const int32_t* row_ptr, const int32_t* src, void* ws, size_t ws_bytes,
                         const cgtp::CpKernelSet** ks, cgtp::CpWsLayout* CL)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    if (rank < 1) return CGTP_ERR_INVALID_ARG;
    *ks = cgtp::find_cp_kernels(rank, plan->channels);
    if (!*ks) return CGTP_ERR_UNSUPPORTED;
    *CL = cgtp::cp_ws_layout(n_nodes, n_edges, (*ks)->rp, plan->channels);
    if (!ws || ws_bytes < CL->total) return CGTP_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return CGTP_ERR_INVALID_ARG;
    return CGTP_OK;
}

bool all_aligned(std::initializer_list<const void*> ps)
{
    for (const void* p : ps)
        if (!p || !aligned16(p)) return false;
    return true;
}

}  // namespace

cgtp_status_t cgtp_cp_conv_fwd(cgtp_plan_t plan, int rank, int64_t n_nodes, int64_t n_edges,
                               const int32_t* row_ptr, const int32_t* src, const float* x, const float* Y,
                               const float* W, const float* A, const float* B, const float* C, float* out,
                               void* ws, size_t ws_bytes, hipStream_t stream)
{
    const cgtp::CpKernelSet* ks = nullptr;
    cgtp::CpWsLayout CL{};
    cgtp_status_t st = cp_prepare(plan, rank, n_nodes, n_edges, row_ptr, src, ws, ws_bytes, &ks, &CL);
    if (st != CGTP_OK) return st;
    if (n_nodes == 0) return CGTP_OK;
    if (!all_aligned({x, out, A, B})) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && !all_aligned({Y, W, C})) return CGTP_ERR_INVALID_ARG;
    st = ensure_prepared(plan, n_nodes, n_edges, row_ptr, src, ws, stream);
    if (st != CGTP_OK) return st;
    char* base = (char*)ws;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges);
    const int Cn = plan->channels;
    double* xb = (double*)(base + CL.xb);
    double* yc = (double*)(base + CL.yc);
    st = hip_status(ks->proj_rows(n_nodes, plan->d_in, rank, Cn, B, x, xb, stream));
    if (st == CGTP_OK) st = hip_status(ks->proj_edge(n_edges, plan->d_sh, rank, C, Y, yc, stream));
    if (st != CGTP_OK) return st;
    cgtp::CpFwdArgs a{};
    a.N = (int32_t)n_nodes;
    a.E = (int32_t)n_edges;
    a.C = Cn;
    a.R = rank;
    a.d3 = plan->d_out;
    a.n_order = cgtp::conv_grid(n_nodes);
    a.order = (const int32_t*)(base + L.rorder);
    a.row_ptr = row_ptr;
    a.src = src;
    a.W = W;
    a.A = A;
    a.xb = xb;
    a.yc = yc;
    a.out = out;
    return hip_status(ks->fwd(a, stream));
}

cgtp_status_t cgtp_cp_conv_bwd(cgtp_plan_t plan, int rank, int64_t n_nodes, int64_t n_edges,
                               const int32_t* row_ptr, const int32_t* src, const float* x, const float* Y,
                               const float* W, const float* A, const float* B, const float* C,
                               const float* grad_out, float* grad_x, float* grad_W, float* grad_Y, void* ws,
                               size_t ws_bytes, hipStream_t stream)
{
    const cgtp::CpKernelSet* ks = nullptr;
    cgtp::CpWsLayout CL{};
    cgtp_status_t st = cp_prepare(plan, rank, n_nodes, n_edges, row_ptr, src, ws, ws_bytes, &ks, &CL);
    if (st != CGTP_OK) return st;
    if ((!grad_x && !grad_W && !grad_Y) || n_nodes == 0) return CGTP_OK;
    if (!all_aligned({x, grad_out, A, B})) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && !all_aligned({Y, W, C})) return CGTP_ERR_INVALID_ARG;
    for (const void* p : {(const void*)grad_x, (const void*)grad_W, (const void*)grad_Y})
        if (p && !aligned16(p)) return CGTP_ERR_INVALID_ARG;
    st = ensure_prepared(plan, n_nodes, n_edges, row_ptr, src, ws, stream);
    if (st != CGTP_OK) return st;
    char* base = (char*)ws;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges);
    const int Cn = plan->channels;
    double* xb = (double*)(base + CL.xb);
    double* ga = (double*)(base + CL.ga);
    double* yc = (double*)(base + CL.yc);
    double* dyc = (double*)(base + CL.dyc);
    st = hip_status(ks->proj_rows(n_nodes, plan->d_in, rank, Cn, B, x, xb, stream));
    if (st == CGTP_OK) st = hip_status(ks->proj_rows(n_nodes, plan->d_out, rank, Cn, A, grad_out, ga, stream));
    if (st == CGTP_OK) st = hip_status(ks->proj_edge(n_edges, plan->d_sh, rank, C, Y, yc, stream));
    if (st != CGTP_OK) return st;
    cgtp::CpBwdArgs a{};
    a.N = (int32_t)n_nodes;
    a.E = (int32_t)n_edges;
    a.C = Cn;
    a.R = rank;
    a.d1 = plan->d_in;
    a.n_order = cgtp::conv_grid(n_nodes);
    a.order = (const int32_t*)(base + L.sorder);
    a.srow = (const int32_t*)(base + L.srow);
    a.perm = (const int32_t*)(base + L.perm);
    a.sdst = (const int32_t*)(base + L.sdst);
    a.W = W;
    a.B = B;
    a.xb = xb;
    a.ga = ga;
    a.yc = yc;
    a.dx = grad_x;
    a.dW = grad_W;
    a.dyc = grad_Y ? dyc : nullptr;
    a.dwa = (double*)(base + CL.dwa);
    st = hip_status(ks->bwd(a, stream));
    if (st != CGTP_OK || !grad_Y) return st;
    return hip_status(ks->edge_back(n_edges, plan->d_sh, rank, ks->h, C, dyc, grad_Y, stream));
}

cgtp_status_t cgtp_conv_bwd_noalloc(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                                    const int32_t* src, const float* x, const float* Y, const float* W,
                                    const float* grad_out, float* grad_x, float* grad_W, float* grad_Y,
                                    hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    if (cgtp::ws_layout(n_nodes, n_edges).total > kScratchBytes) return CGTP_ERR_WORKSPACE;
    if ((!grad_x && !grad_W && !grad_Y) || n_nodes == 0) return CGTP_OK;
    if (!x || !aligned16(x) || !grad_out || !aligned16(grad_out)) return CGTP_ERR_INVALID_ARG;
    if (grad_x && !aligned16(grad_x)) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && (!Y || !W || !aligned16(W) || !aligned16(Y))) return CGTP_ERR_INVALID_ARG;
    if (grad_W && !aligned16(grad_W)) return CGTP_ERR_INVALID_ARG;
    if (grad_Y && !aligned16(grad_Y)) return CGTP_ERR_INVALID_ARG;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CGTP_ERR_HIP;
    void* ws = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        st = scratch_ptr(dev, &ws);
        if (st != CGTP_OK) return st;
        ScratchSlot& s = g_scratch[dev];
        const bool loc = (plan->flags & CGTP_FLAG_LOCALITY) != 0;
        const bool same = s.valid && s.rec.N == n_nodes && s.rec.E == n_edges && s.rec.row_ptr == row_ptr &&
                          s.rec.src == src && s.rec.locality == loc;
        if (!same) {
            s.valid = false;
            if (cgtp::launch_graph_prepare((int32_t)n_nodes, (int32_t)n_edges, row_ptr, src, ws, loc, stream) !=
                hipSuccess)
                return CGTP_ERR_HIP;
            s.rec = Prepared{n_nodes, n_edges, row_ptr, src, loc, dev};
            s.valid = true;
        }
    }
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges);
    const char* base = (const char*)ws;
    cgtp::BwdArgs a{};
    a.sh = launch_shape(plan, n_nodes, n_edges);
    a.g = cgtp::GraphView{(const int32_t*)(base + L.srow), (const int32_t*)(base + L.perm),
                          (const int32_t*)(base + L.sdst), (const int32_t*)(base + L.rorder),
                          (const int32_t*)(base + L.sorder)};
    a.x = x;
    a.Y = Y;
    a.W = W;
    a.G = grad_out;
    a.dx = grad_x;
    a.dW = grad_W;
    a.dY = grad_Y;
    if (plan->mid) return hip_status(plan->ks->bwd_mid(a, stream));
    return hip_status(plan->ks->bwd[plan->sub ? 1 : 0](a, stream));
}

const char* cgtp_status_string(cgtp_status_t status)
{
    switch (status) {
        case CGTP_OK: return "ok";
        case CGTP_ERR_INVALID_ARG: return "invalid argument";
        case CGTP_ERR_UNSUPPORTED: return "unsupported degrees or channel count";
        case CGTP_ERR_WORKSPACE: return "workspace missing or too small";
        case CGTP_ERR_HIP: return "HIP error";
        case CGTP_ERR_ALLOC: return "host allocation failed";
        case CGTP_ERR_GRAPH: return "malformed CSR graph";
        case CGTP_ERR_NUMERIC: return "CP fit: normal matrix not positive definite";
    }
    return "unknown status";
}

}  // extern "C"
