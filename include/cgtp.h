/*
 * cgtp.h -- C ABI of libcgtp.so: the Clebsch-Gordan tensor-product (CGTP)
 * convolution of equivariant interatomic potentials on AMD MI355X (gfx950).
 *
 * The operation.  The LunaTP abstract ("LunaTP: Enabling Efficient and
 * Scalable Tensor Product for Equivariant MLIPs", Abstract) names the CGTP
 * convolution as the cost that limits equivariant MLIPs.  For every edge
 * j -> i of a neighbour graph, the irreps of node j (degrees l = 0..L_in, C
 * channels) are coupled with the real spherical harmonics of the edge vector
 * (degrees 0..L_sh) through the real-basis Clebsch-Gordan coefficients, one
 * coupling per path (l1, l2, l3) allowed by the selection rules
 * |l1-l2| <= l3 <= l1+l2, m3 = m1+m2 ("Tensor Decomposition Networks ...",
 * rebuttal to reviewer S6y1, first answer), scaled by a weight per edge, path
 * and channel ("uvu"), and summed into node i:
 *
 *   out[i][k(l3,m3)][u] = sum_{e: j->i} sum_{p=(l1,l2,l3)} W[e][p][u]
 *                         sum_{m1,m2} T_p[m1][m2][m3] x[j][k(l1,m1)][u] Y[e][k(l2,m2)]
 *
 * with k(l,m) = l*l + l + m.  The backward returns the gradients of
 * L = <grad_out, out> with respect to x, W and Y, the bilinear-map gradients
 * of the TDN rebuttal to S6y1 (formulas after Equation (3)) applied to each
 * argument of this trilinear map.
 *
 * Conventions shared by every entry point:
 *   - paths (l1,l2,l3) in lexicographic order, every triangle-valid path
 *     (no parity filter); the path count P is reported by cgtp_plan_info.
 *   - T_p is the real part (even l1+l2+l3) or the imaginary part (odd) of the
 *     complex CG tensor (Condon-Shortley phase) carried to the real basis
 *     Y_{l,m} = sqrt2 (-1)^m Im Y_l^|m| (m<0), Y_l^0, sqrt2 (-1)^m Re Y_l^m (m>0).
 *   - layouts, all row-major fp32, channels fastest:
 *       x, grad_x       [N][(L_in+1)^2][C]
 *       out, grad_out   [N][(L_out+1)^2][C]
 *       Y, grad_Y       [E][(L_sh+1)^2]
 *       W, grad_W       [E][P][C]
 *       r               [E][3]
 *   - the graph is a receiver-sorted CSR: row_ptr[N+1] (int32, row_ptr[0] = 0,
 *     non-decreasing, row_ptr[N] = E) and src[E] (int32 sender of each edge,
 *     in [0, N)).  Well-formedness is a precondition, checked only when the
 *     plan was created with CGTP_FLAG_VALIDATE.
 *   - every array argument is a DEVICE pointer owned by the caller; calls are
 *     asynchronous on the given stream; outputs are overwritten, never
 *     accumulated; a NULL gradient pointer skips that gradient.
 *   - arithmetic is fp64 inside the kernels; inputs and outputs are fp32.
 *   - every function returns a status and never aborts.  Only host-side
 *     checks are made (null handles and pointers, sizes, 8-byte alignment of
 *     the channel arrays, workspace size); a HIP launch error returns
 *     CGTP_ERR_HIP.
 */
#ifndef CGTP_H
#define CGTP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cgtp_plan_s* cgtp_plan_t;

typedef enum {
    CGTP_OK = 0,
    CGTP_ERR_INVALID_ARG = -1,  /* null handle/pointer, negative size, misalignment */
    CGTP_ERR_UNSUPPORTED = -2,  /* degrees or channel count without a compiled kernel */
    CGTP_ERR_WORKSPACE = -3,    /* workspace missing or smaller than cgtp_workspace_size */
    CGTP_ERR_HIP = -4,          /* a HIP call or kernel launch failed */
    CGTP_ERR_ALLOC = -5,        /* host allocation failed */
    CGTP_ERR_GRAPH = -6         /* CGTP_FLAG_VALIDATE found a malformed CSR */
} cgtp_status_t;

/* Validate the CSR (on a host copy, synchronously) in every call taking a graph. */
#define CGTP_FLAG_VALIDATE 1u

/* Create a plan for degrees (l_in, l_sh, l_out) and C channels.
 * Supported: l_in = l_sh = l_out = L with L in {1, 2} and C in {8, 16, 32, 64, 128},
 * or L = 3 and C in {8, 16, 32, 64}.  Host-only: no HIP call is made.
 * On success *plan owns host memory released by cgtp_plan_destroy. */
cgtp_status_t cgtp_plan_create(cgtp_plan_t* plan, int l_in, int l_sh, int l_out, int channels,
                               unsigned flags);

/* Release a plan (NULL is accepted). */
cgtp_status_t cgtp_plan_destroy(cgtp_plan_t plan);

/* Path count and dimensions.  paths_l1l2l3, if not NULL, receives [P][3]
 * (l1, l2, l3) in the order the weights use.  Any output pointer may be NULL. */
cgtp_status_t cgtp_plan_info(cgtp_plan_t plan, int* num_paths, int* paths_l1l2l3, int* dim_in,
                             int* dim_sh, int* dim_out);

/* Test hook: the real CG tensor of path `path` exactly as the kernels use it,
 * dense [(2l1+1)][(2l2+1)][(2l3+1)] fp64 into host memory `dense`. */
cgtp_status_t cgtp_plan_export_cg(cgtp_plan_t plan, int path, double* dense);

/* Bytes of device workspace for N nodes and E edges: the sender-sorted view
 * of the CSR and its temporaries, degree-ordered block schedules, and for
 * C > 64 a scratch section of 8*E*(C/64)*(l_sh+1)^2 bytes for the backward. */
cgtp_status_t cgtp_workspace_size(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, size_t* bytes);

/* Real spherical harmonics, degrees 0..l_sh, of r[e]/|r[e]|: Y[E][(l_sh+1)^2].
 * A zero-length r[e] is a precondition violation (the result is unspecified). */
cgtp_status_t cgtp_sh_fwd(cgtp_plan_t plan, int64_t n_edges, const float* r, float* Y, hipStream_t stream);

/* Graph preparation: writes into `ws` the sender-sorted view of the CSR
 * (sender offsets, edge permutation stable in edge id, receiver of each
 * permuted edge).  Must run, on the same stream or earlier, before
 * cgtp_conv_fwd / cgtp_conv_bwd are called with this (row_ptr, src, ws); a
 * prepared workspace can serve any number of such calls for the same graph. */
cgtp_status_t cgtp_graph_prepare(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges,
                                 const int32_t* row_ptr, const int32_t* src, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Forward: out[N][(l_out+1)^2][C] from x, Y, W over the CSR.  Node-centric and
 * atomic-free: each receiver's output row has exactly one writer. ws is the
 * workspace prepared by cgtp_graph_prepare for this graph. */
cgtp_status_t cgtp_conv_fwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const float* x, const float* Y, const float* W, float* out,
                            const void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of L = <grad_out, out>: grad_x [N][(l_in+1)^2][C],
 * grad_W [E][P][C], grad_Y [E][(l_sh+1)^2]; each may be NULL to skip it.
 * Sender-centric and atomic-free over the prepared workspace `ws`.  For
 * C > 64 the backward also writes per-slice grad_Y partial sums into the
 * workspace's scratch section, so two backward calls in flight at the same
 * time must not share one workspace (the graph view itself is only read). */
cgtp_status_t cgtp_conv_bwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const float* x, const float* Y, const float* W,
                            const float* grad_out, float* grad_x, float* grad_W, float* grad_Y,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Static text for a status code. */
const char* cgtp_status_string(cgtp_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* CGTP_H */
