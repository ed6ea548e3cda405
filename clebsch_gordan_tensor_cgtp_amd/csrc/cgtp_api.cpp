// cgtp_api.cpp -- the C ABI of libcgtp.so (see include/cgtp.h): plans,
// argument checks, workspace sizing and dispatch to the gfx950 kernels.
#include "cgtp.h"

#include <hip/hip_runtime.h>

#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "cgtp_internal.h"
#include "cgtp_math.h"

struct cgtp_plan_s {
    int l_in, l_sh, l_out, channels;
    unsigned flags;
    int P, d_in, d_sh, d_out;
    std::vector<int> paths;  // [P][3]
    const cgtp::KernelSet* ks;
};

namespace {

bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }

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
    if (!row_ptr) return CGTP_ERR_INVALID_ARG;
    if (E > 0 && !src) return CGTP_ERR_INVALID_ARG;
    if (plan->flags & CGTP_FLAG_VALIDATE) return validate_graph(N, E, row_ptr, src);
    return CGTP_OK;
}

cgtp_status_t check_ws(const cgtp_plan_s* plan, int64_t N, int64_t E, const void* ws, size_t ws_bytes)
{
    const cgtp::WsLayout L = cgtp::ws_layout(N, E, plan->ks->dyp_per_edge);
    if (!ws || ws_bytes < L.total) return CGTP_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return CGTP_ERR_INVALID_ARG;
    return CGTP_OK;
}

}  // namespace

extern "C" {

cgtp_status_t cgtp_plan_create(cgtp_plan_t* plan, int l_in, int l_sh, int l_out, int channels, unsigned flags)
{
    if (!plan) return CGTP_ERR_INVALID_ARG;
    *plan = nullptr;
    if (l_in < 0 || l_sh < 0 || l_out < 0 || channels <= 0) return CGTP_ERR_INVALID_ARG;
    if (flags & ~CGTP_FLAG_VALIDATE) return CGTP_ERR_INVALID_ARG;
    const cgtp::KernelSet* ks = cgtp::find_kernels(l_in, l_sh, l_out, channels);
    if (!ks) return CGTP_ERR_UNSUPPORTED;
    cgtp_plan_s* p = new (std::nothrow) cgtp_plan_s();
    if (!p) return CGTP_ERR_ALLOC;
    p->l_in = l_in;
    p->l_sh = l_sh;
    p->l_out = l_out;
    p->channels = channels;
    p->flags = flags;
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
    p->ks = ks;
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
    if (dim_out) *dim_out = plan->d_out;
    return CGTP_OK;
}

cgtp_status_t cgtp_plan_export_cg(cgtp_plan_t plan, int path, double* dense)
{
    if (!plan || !dense || path < 0 || path >= plan->P) return CGTP_ERR_INVALID_ARG;
    return cgtp::host_cg_table(plan->l_in, plan->l_sh, plan->l_out, path, dense) ? CGTP_OK
                                                                                   : CGTP_ERR_UNSUPPORTED;
}

cgtp_status_t cgtp_workspace_size(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, size_t* bytes)
{
    if (!plan || !bytes || n_nodes < 0 || n_edges < 0) return CGTP_ERR_INVALID_ARG;
    *bytes = cgtp::ws_layout(n_nodes, n_edges, plan->ks->dyp_per_edge).total;
    return CGTP_OK;
}

cgtp_status_t cgtp_sh_fwd(cgtp_plan_t plan, int64_t n_edges, const float* r, float* Y, hipStream_t stream)
{
    if (!plan || n_edges < 0) return CGTP_ERR_INVALID_ARG;
    if (n_edges == 0) return CGTP_OK;
    if (!r || !Y || !aligned8(Y) || ((uintptr_t)r & 3u)) return CGTP_ERR_INVALID_ARG;
    return hip_status(plan->ks->sh(n_edges, r, Y, stream));
}

cgtp_status_t cgtp_graph_prepare(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                                 const int32_t* src, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    st = check_ws(plan, n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    return hip_status(cgtp::launch_graph_prepare((int32_t)n_nodes, (int32_t)n_edges, row_ptr, src, ws, stream));
}

cgtp_status_t cgtp_conv_fwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const float* x, const float* Y, const float* W, float* out,
                            const void* ws, size_t ws_bytes, hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    st = check_ws(plan, n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    if (n_nodes == 0) return CGTP_OK;
    if (!out || !aligned8(out) || !x || !aligned8(x)) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && (!Y || !W || !aligned8(W) || ((uintptr_t)Y & 3u))) return CGTP_ERR_INVALID_ARG;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges, plan->ks->dyp_per_edge);
    const int32_t* rorder = (const int32_t*)((const char*)ws + L.rorder);
    return hip_status(plan->ks->fwd((int32_t)n_nodes, row_ptr, src, rorder, x, Y, W, out, stream));
}

cgtp_status_t cgtp_conv_bwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const float* x, const float* Y, const float* W,
                            const float* grad_out, float* grad_x, float* grad_W, float* grad_Y, void* ws,
                            size_t ws_bytes, hipStream_t stream)
{
    cgtp_status_t st = check_graph_args(plan, n_nodes, n_edges, row_ptr, src);
    if (st != CGTP_OK) return st;
    st = check_ws(plan, n_nodes, n_edges, ws, ws_bytes);
    if (st != CGTP_OK) return st;
    int mask = (grad_x ? cgtp::kGradX : 0) | (grad_W ? cgtp::kGradW : 0) | (grad_Y ? cgtp::kGradY : 0);
    if (mask == 0 || n_nodes == 0) return CGTP_OK;
    if (!x || !aligned8(x) || !grad_out || !aligned8(grad_out)) return CGTP_ERR_INVALID_ARG;
    if (grad_x && !aligned8(grad_x)) return CGTP_ERR_INVALID_ARG;
    if (n_edges > 0 && (!Y || !W || !aligned8(W) || ((uintptr_t)Y & 3u))) return CGTP_ERR_INVALID_ARG;
    if (grad_W && !aligned8(grad_W)) return CGTP_ERR_INVALID_ARG;
    if (grad_Y && ((uintptr_t)grad_Y & 3u)) return CGTP_ERR_INVALID_ARG;
    const cgtp::WsLayout L = cgtp::ws_layout(n_nodes, n_edges, plan->ks->dyp_per_edge);
    char* base = (char*)ws;
    cgtp::GraphView g{(const int32_t*)(base + L.srow), (const int32_t*)(base + L.perm),
                      (const int32_t*)(base + L.sdst), (const int32_t*)(base + L.sorder),
                      (double*)(base + L.dyp), (int32_t)n_edges};
    return hip_status(
        plan->ks->bwd((int32_t)n_nodes, g, x, Y, W, grad_out, grad_x, grad_W, grad_Y, mask, stream));
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
    }
    return "unknown status";
}

}  // extern "C"
