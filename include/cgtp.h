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
 *   - paths (l1,l2,l3) in lexicographic order, every triangle-valid path with
 *     l1 <= l_in, l2 <= l_sh, l3 <= l_out (no parity filter); the path count
 *     P and the list are reported by cgtp_plan_info.
 *   - T_p is the real part (even l1+l2+l3) or the imaginary part (odd) of the
 *     complex CG tensor (Condon-Shortley phase) carried to the real basis
 *     Y_{l,m} = sqrt2 (-1)^m Im Y_l^|m| (m<0), Y_l^0, sqrt2 (-1)^m Re Y_l^m (m>0).
 *   - layouts, all row-major fp32, channels fastest:
 *       x, grad_x       [N][(l_in+1)^2][C]
 *       out, grad_out   [N][(l_out+1)^2][C]   ([N][D_mid][C] with CGTP_FLAG_PATH_OUTPUTS)
 *       Y, grad_Y       [E][(l_sh+1)^2]
 *       W, grad_W       [E][P][C]   ([E][C] with CGTP_FLAG_SHARED_WEIGHTS)
 *       r               [E][3]
 *   - the graph is a receiver-sorted CSR: row_ptr[N+1] (int32, row_ptr[0] = 0,
 *     non-decreasing, row_ptr[N] = E) and src[E] (int32 sender of each edge,
 *     in [0, N)).  Well-formedness is a precondition, checked (on a host copy,
 *     synchronously) only when the plan was created with CGTP_FLAG_VALIDATE.
 *     A malformed graph never makes a kernel read or write out of bounds: the
 *     kernels clamp every CSR and view index; the values are then unspecified.
 *   - every array argument is a DEVICE pointer owned by the caller and aligned
 *     to 16 bytes; calls are asynchronous on the given stream; outputs are
 *     overwritten, never accumulated; a NULL gradient pointer skips that
 *     gradient.
 *   - arithmetic is fp64 inside the kernels; inputs and outputs are fp32.
 *     Every floating-point sum has a fixed order: results are bitwise
 *     reproducible run to run (no floating-point atomics).
 *   - every function returns a status and never aborts.  Only host-side
 *     checks are made (null handles and pointers, sizes, alignment, workspace
 *     size); a HIP launch error returns CGTP_ERR_HIP.
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
    CGTP_ERR_UNSUPPORTED = -2,  /* degrees or channel count outside the compiled range */
    CGTP_ERR_WORKSPACE = -3,    /* workspace missing or smaller than cgtp_workspace_size */
    CGTP_ERR_HIP = -4,          /* a HIP call or kernel launch failed */
    CGTP_ERR_ALLOC = -5,        /* host allocation failed */
    CGTP_ERR_GRAPH = -6,        /* CGTP_FLAG_VALIDATE found a malformed CSR */
    CGTP_ERR_NUMERIC = -7       /* the CP fit met a normal matrix that is not positive definite */
} cgtp_status_t;

/* Validate the CSR (on a host copy, synchronously) in every call taking a graph. */
#define CGTP_FLAG_VALIDATE 1u
/* Schedule convolution blocks by graph-derived clusters, one compact range
 * per XCD, instead of longest segment first over the whole graph (results
 * are identical; only the L2 reuse of gathered rows and the balance differ). */
#define CGTP_FLAG_LOCALITY 2u
/* Path-weight sharing ("Tensor Decomposition Networks ...", rebuttal to
 * reviewer oXft: one weight matrix shared across the paths): W and grad_W are
 * [E][C], one weight per edge and channel used by every path, and
 * grad_W[e][u] = sum over the paths of dL/dW[e][p][u]. */
#define CGTP_FLAG_SHARED_WEIGHTS 4u
/* Per-path (concatenated) outputs: every path keeps its own 2*l3+1 output
 * rows instead of adding into the l3 slot ("irreps_mid").  out and grad_out
 * are [N][D_mid][C] with D_mid = sum over the paths of (2*l3+1); path p owns
 * rows o_p .. o_p + 2*l3_p with o_p = sum over earlier paths of (2*l3+1), in
 * the path order of cgtp_plan_info (which reports D_mid as dim_out).  The
 * summed output is the sum of these blocks over the paths of each l3.  The
 * per-path blocks are what a fully connected ("uvw") product mixes over
 * channels per path (TDN rebuttal to cmnz: the fully connected CG tensor
 * product as the cost-dominating kernel).  Combines with
 * CGTP_FLAG_SHARED_WEIGHTS; cgtp_conv_bwd_bwd returns CGTP_ERR_UNSUPPORTED
 * for such plans. */
#define CGTP_FLAG_PATH_OUTPUTS 8u

/* Create a plan for degrees (l_in, l_sh, l_out) and C channels: the path list
 * under the selection rules (TDN rebuttal to S6y1, first answer) and the real
 * CG tables (TDN rebuttal to 7Mvd: the coordinates of the SO(3) tensor
 * product in the coupled basis).
 * Supported: 0 <= l_in, l_sh, l_out <= 3 and 1 <= C <= 128.  Host-only: no
 * HIP call is made.  flags: CGTP_FLAG_* or 0; unknown bits -> INVALID_ARG.
 * On success *plan owns host memory released by cgtp_plan_destroy; a plan
 * is immutable and may be shared by threads. */
cgtp_status_t cgtp_plan_create(cgtp_plan_t* plan, int l_in, int l_sh, int l_out, int channels,
                               unsigned flags);

/* Release a plan (NULL is accepted). */
cgtp_status_t cgtp_plan_destroy(cgtp_plan_t plan);

/* Path count and dimensions of a plan (TDN rebuttal to S6y1, first answer:
 * which (l1, l2, l3) couple).  paths_l1l2l3, if not NULL, receives [P][3]
 * (l1, l2, l3) in the order the weights use.  Any output pointer may be NULL.
 * dim_* = (l+1)^2 of each degree (dim_out = D_mid with CGTP_FLAG_PATH_OUTPUTS). */
cgtp_status_t cgtp_plan_info(cgtp_plan_t plan, int* num_paths, int* paths_l1l2l3, int* dim_in,
                             int* dim_sh, int* dim_out);

/* Test hook: the real CG tensor of path `path` exactly as the kernels use it
 * (TDN rebuttal to 7Mvd), dense [(2l1+1)][(2l2+1)][(2l3+1)] fp64 into HOST
 * memory `dense` (caller-owned, at least that many doubles). */
cgtp_status_t cgtp_plan_export_cg(cgtp_plan_t plan, int path, double* dense);

/* Bytes of device workspace for N nodes and E edges (independent of the
 * plan's degrees): the sender-sorted view of the CSR and its temporaries and
 * the block schedules, about 16*E + 170*N + 16384 bytes. */
cgtp_status_t cgtp_workspace_size(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, size_t* bytes);

/* Real spherical harmonics Y_l(r/|r|), degrees 0..l_sh, orthonormal, of every
 * edge vector (the SH that couple to the node features in the CGTP
 * convolution, LunaTP Abstract): r[E][3] -> Y[E][(l_sh+1)^2].
 * A zero-length r[e] is a precondition violation (the result is unspecified). */
cgtp_status_t cgtp_sh_fwd(cgtp_plan_t plan, int64_t n_edges, const float* r, float* Y, hipStream_t stream);

/* Backward of the spherical harmonics: grad_r[e] = sum_k grad_Y[e][k] dY_k/dr
 * evaluated at r[e], for degrees 0..l_sh: r[E][3], grad_Y[E][(l_sh+1)^2] ->
 * grad_r[E][3].  This is the path by which the convolution backward's grad_Y
 * term feeds the forces of an interatomic potential (analytic forces checked
 * by finite differences, AccelNet review, Referee Report).  Since Y depends on
 * the direction only, grad_r is orthogonal to r.  A zero-length r[e] is a
 * precondition violation. */
cgtp_status_t cgtp_sh_bwd(cgtp_plan_t plan, int64_t n_edges, const float* r, const float* grad_Y, float* grad_r,
                          hipStream_t stream);

/* Per-node gradient from per-edge gradients of the edge vectors
 * r[e] = pos[src e] - pos[dst e] (the forces on atoms are its negative):
 *   grad_pos[n] = sum_{e: src e = n} grad_r[e] - sum_{e: dst e = n} grad_r[e],
 * grad_r[E][3] -> grad_pos[N][3].  One writer per node, fixed summation
 * order (the out-edges through the sender-sorted view in `ws`, prepared here
 * first unless cgtp_graph_prepare already did, see there). */
cgtp_status_t cgtp_node_grad(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                             const int32_t* src, const float* grad_r, float* grad_pos, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* Graph preparation (LunaTP Abstract: node-centric execution needs each
 * node's edges together): writes into `ws` the sender-sorted view of the CSR
 * (sender offsets, edge permutation stable in edge id, receiver of each
 * permuted edge) and the block schedules of both convolution kernels.  The
 * library records that `ws` now holds the view of (n_nodes, n_edges,
 * row_ptr, src); cgtp_conv_fwd / cgtp_conv_bwd called with the same four
 * values and `ws` use it as it is, and otherwise run this preparation
 * themselves first.  The record is by pointer: after rewriting the contents
 * of row_ptr or src in place, or when the workspace memory has held anything
 * else since it was prepared (for instance freed and allocated again at the
 * same address), call cgtp_graph_prepare again.  ws must be
 * 256-byte aligned and at least cgtp_workspace_size bytes. */
cgtp_status_t cgtp_graph_prepare(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges,
                                 const int32_t* row_ptr, const int32_t* src, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Forward of the CGTP convolution (LunaTP Abstract; the formula above):
 * out[N][(l_out+1)^2][C] from x, Y, W over the CSR.  Node-centric and
 * atomic-free: each receiver's output row has exactly one writer, and a
 * receiver without in-edges gets zeros.  ws: the workspace of this graph
 * (prepared here first unless cgtp_graph_prepare already did, see there). */
cgtp_status_t cgtp_conv_fwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const float* x, const float* Y, const float* W, float* out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of L = <grad_out, out> (TDN rebuttal to S6y1, the gradients after
 * Equation (3), one per argument of the trilinear map):
 *   grad_x [N][(l_in+1)^2][C]   (a sender without out-edges gets zeros)
 *   grad_W [E][P][C]
 *   grad_Y [E][(l_sh+1)^2]      (summed over the channels)
 * each may be NULL to skip it.  Sender-centric and atomic-free over the
 * sender-sorted view in `ws` (prepared here first unless cgtp_graph_prepare
 * already did).  The view is only read, so backward and forward calls of one
 * graph may share a workspace. */
cgtp_status_t cgtp_conv_bwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                            const int32_t* src, const float* x, const float* Y, const float* W,
                            const float* grad_out, float* grad_x, float* grad_W, float* grad_Y,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Forward with the spherical harmonics evaluated inside the kernel: as
 * cgtp_conv_fwd with Y = the real SH of degrees 0..l_sh of r[e]/|r[e]|,
 * taken from the edge vectors r [E][3] in fp64 (not rounded to fp32 as
 * cgtp_sh_fwd's output is) instead of read from memory.  Evaluating the
 * harmonics where they are used saves writing Y and reading it back in both
 * passes, and (cgtp_conv_bwd_sh) writing grad_Y and reading it back for the
 * SH backward: 4*(l_sh+1)^2 bytes per edge each.  A zero-length r[e] is a
 * precondition violation.  Not for CGTP_FLAG_PATH_OUTPUTS plans
 * (CGTP_ERR_UNSUPPORTED). */
cgtp_status_t cgtp_conv_fwd_sh(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                               const int32_t* src, const float* x, const float* r, const float* W, float* out,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of L = <grad_out, out> of cgtp_conv_fwd_sh, with respect to x, W
 * and the edge vectors:
 *   grad_x [N][(l_in+1)^2][C], grad_W [E][P][C] as cgtp_conv_bwd's,
 *   grad_r [E][3] = sum_k grad_Y[e][k] dY_k/dr, the SH backward of
 *                   cgtp_sh_bwd applied inside the kernel to the grad_Y that
 *                   cgtp_conv_bwd would return (which never reaches memory);
 *                   the per-edge gradient that cgtp_node_grad turns into
 *                   forces (AccelNet review, Referee Report).
 * Each may be NULL to skip it.  Same workspace, schedule and determinism as
 * cgtp_conv_bwd; not for CGTP_FLAG_PATH_OUTPUTS plans. */
cgtp_status_t cgtp_conv_bwd_sh(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                               const int32_t* src, const float* x, const float* r, const float* W,
                               const float* grad_out, float* grad_x, float* grad_W, float* grad_r,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Double backward (the higher-order derivatives LunaTP's abstract names;
 * training on forces differentiates the backward once more).  With
 * (grad_x, grad_W, grad_Y) = cgtp_conv_bwd(x, Y, W, grad_out) and cotangents
 * gg_x [N][(l_in+1)^2][C], gg_W [E][P][C], gg_Y [E][(l_sh+1)^2] of those
 * three results, this computes the gradients of
 *   S = <gg_x, grad_x> + <gg_W, grad_W> + <gg_Y, grad_Y>
 * with respect to each input of the backward:
 *   dd_x   [N][(l_in+1)^2][C]   (with respect to x)
 *   dd_Y   [E][(l_sh+1)^2]      (with respect to Y, summed over the channels)
 *   dd_W   [E][P][C]            (with respect to W)
 *   dd_out [N][(l_out+1)^2][C]  (with respect to grad_out)
 * A NULL cotangent counts as zero; a NULL result is skipped; results are
 * overwritten.  With CGTP_FLAG_SHARED_WEIGHTS, W, gg_W and dd_W are [E][1][C].
 * S is linear in each input, so every result is a sum of three (dd_out) or
 * two (the others) backward- or forward-like contractions, formed in one pass
 * per side: dd_out on the receiver side as the forward is, the others on the
 * sender side over the view in `ws` as the backward is (prepared here first
 * unless cgtp_graph_prepare already did).  Same alignment rules as the other
 * calls. */
cgtp_status_t cgtp_conv_bwd_bwd(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                                const int32_t* src, const float* x, const float* Y, const float* W,
                                const float* grad_out, const float* gg_x, const float* gg_Y, const float* gg_W,
                                float* dd_x, float* dd_Y, float* dd_W, float* dd_out, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* ---- fully connected ("uvw") mixing ----------------------------------------
 * The fully connected CG tensor product ("Tensor Decomposition Networks ...",
 * rebuttal to cmnz: the cost-dominating kernel) couples every input channel
 * with every output channel per path.  With its weights shared over the edges
 * it is the per-path-output convolution (CGTP_FLAG_PATH_OUTPUTS) followed by
 * one dense channel matrix per path, summed over the paths of each l3:
 *   out[i][k(l3,m)][w] = sum_{p: l3_p = l3} sum_u mid[i][o_p + m][u] Wmix[p][u][w]
 * mid [N][D_mid][C] (the per-path outputs, layout of CGTP_FLAG_PATH_OUTPUTS,
 * C the plan's channels), Wmix [P][C][c_out], out [N][(l_out+1)^2][c_out];
 * 1 <= c_out <= 1024.  Runs on the fp64 matrix cores; any plan of the degree
 * set may be used (only its path list and C matter). */

/* Workspace bytes of cgtp_path_mix_bwd (the weight gradient's per-block
 * partial sums). */
cgtp_status_t cgtp_path_mix_workspace_size(cgtp_plan_t plan, int64_t n_nodes, int c_out, size_t* bytes);

/* out = the mixing above (overwritten). */
cgtp_status_t cgtp_path_mix_fwd(cgtp_plan_t plan, int64_t n_nodes, int c_out, const float* mid, const float* Wmix,
                                float* out, hipStream_t stream);

/* Backward of L = <grad_out, out>:
 *   grad_mid[i][o_p + m][u] = sum_w grad_out[i][k(l3_p,m)][w] Wmix[p][u][w]
 *   grad_Wmix[p][u][w]      = sum_i sum_m mid[i][o_p + m][u] grad_out[i][k(l3_p,m)][w]
 * Either output may be NULL.  The weight gradient sums over the nodes in a
 * fixed order (node ranges per block, partials in ws, added in order). */
cgtp_status_t cgtp_path_mix_bwd(cgtp_plan_t plan, int64_t n_nodes, int c_out, const float* mid, const float* Wmix,
                                const float* grad_out, float* grad_mid, float* grad_Wmix, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* ---- CP-decomposed tensor product ----------------------------------------
 * The approximate product of "Tensor Decomposition Networks for Accelerating
 * Machine Learning Force Field Computations" (authors' rebuttal to S6y1,
 * Equation (3)): the coupling of x (d1 = (l_in+1)^2 components) and y
 * (d2 = (l_sh+1)^2) into z (d3 = (l_out+1)^2) is z = A (B^T x (.) C^T y)
 * with rank-R factors A [d3][R], B [d1][R], C [d2][R] (row-major), which
 * approximate the whole coupling tensor M of the plan's degrees (every
 * path's real CG block at its components).  Over the graph, with one weight
 * per edge and channel:
 *   out[i][:,u] = sum_{e = j->i} W[e][u] A (B^T x[j][:,u] (.) C^T Y[e])
 * W is [E][C] whatever the plan's weight flags.  Ranks 1..64; the plan's
 * degrees and channel count (1..128) apply. */

/* Workspace of the CP calls: the graph view of cgtp_workspace_size followed
 * by the projected rows (B^T x and A^T grad_out per node, C^T Y and its
 * gradient per edge).  One such workspace serves cgtp_graph_prepare and the
 * CP calls of one graph. */
cgtp_status_t cgtp_cp_workspace_size(cgtp_plan_t plan, int rank, int64_t n_nodes, int64_t n_edges,
                                     size_t* bytes);

/* Data-free fit of the factors (same rebuttal, reply on Figure 3: minimise
 * the Frobenius norm between the exact and the approximate product over
 * standard-normal inputs, once, before training).  Over independent
 * standard-normal x, y the expected squared error equals ||M - [[A,B,C]]||_F^2,
 * so this runs alternating least squares on M: per sweep B, then C, then A
 * is replaced by its exact least-squares solution with the other two fixed
 * (normal matrix plus ridge * trace / R on its diagonal; ridge 0 is allowed).
 * A [d3][rank], B [d1][rank], C [d2][rank] are host fp64 arrays: the starting
 * point on entry (the caller draws it, e.g. standard normal), the fit on
 * return.  *rel_err (may be NULL) = ||M - [[A,B,C]]||_F / ||M||_F.  Host
 * computation, no GPU.  CGTP_ERR_NUMERIC if a normal matrix is not positive
 * definite (raise ridge). */
cgtp_status_t cgtp_cp_fit(cgtp_plan_t plan, int rank, int sweeps, double ridge, double* A, double* B, double* C,
                          double* rel_err);

/* Forward of the CP convolution: out [N][d3][C] (a receiver without in-edges
 * gets zeros).  A, B, C: the factors as fp32 device arrays.  Node-centric and
 * atomic-free; B^T x is formed once per node and A applied once per receiver
 * (inside `ws`, prepared here first unless cgtp_graph_prepare already did). */
cgtp_status_t cgtp_cp_conv_fwd(cgtp_plan_t plan, int rank, int64_t n_nodes, int64_t n_edges,
                               const int32_t* row_ptr, const int32_t* src, const float* x, const float* Y,
                               const float* W, const float* A, const float* B, const float* C, float* out,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of L = <grad_out, out> for the CP convolution, by the closed forms
 * after Equation (3) (g_x = (g_z A (.) C^T y) B^T, g_y = (g_z A (.) B^T x) C^T,
 * here with the edge weight and the sum over channels):
 *   grad_x [N][d1][C], grad_W [E][C], grad_Y [E][d2]; each may be NULL.
 * Sender-centric and atomic-free over the view in `ws`. */
cgtp_status_t cgtp_cp_conv_bwd(cgtp_plan_t plan, int rank, int64_t n_nodes, int64_t n_edges,
                               const int32_t* row_ptr, const int32_t* src, const float* x, const float* Y,
                               const float* W, const float* A, const float* B, const float* C,
                               const float* grad_out, float* grad_x, float* grad_W, float* grad_Y, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * backward exactly as cgtp_conv_bwd computes it, with the graph view held in
 * a static device array of the library (64 MiB per GPU, held from the
 * library's first use of that GPU until the process ends) instead of a
 * caller workspace.  Calls no allocating routine.  The array is prepared by
 * this call for (n_nodes, n_edges, row_ptr, src) unless the previous call on
 * this GPU prepared it for the same four values (the record is by pointer, as
 * for cgtp_graph_prepare); the preparation clears every counter it uses.
 * Returns CGTP_ERR_WORKSPACE when the graph's workspace
 * (cgtp_workspace_size) exceeds 64 MiB.  Every call on one GPU shares the
 * array: calls that overlap on one GPU (other streams or threads) race and
 * must be ordered by the caller. */
cgtp_status_t cgtp_conv_bwd_noalloc(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr,
                                    const int32_t* src, const float* x, const float* Y, const float* W,
                                    const float* grad_out, float* grad_x, float* grad_W, float* grad_Y,
                                    hipStream_t stream);

/* Static text for a status code. */
const char* cgtp_status_string(cgtp_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* CGTP_H */
