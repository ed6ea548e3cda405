/*
 * cgtp_oracle.c -- fp64 CPU oracle for the Clebsch-Gordan tensor-product (CGTP)
 * convolution of equivariant interatomic potentials.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * (libcgtp.so) shares no code, header, table or constant with this file.
 *
 * What it computes and where that is stated:
 *   - the CG selection rules |l1-l2| <= l3 <= l1+l2, m3 = m1+m2 ("Tensor
 *     Decomposition Networks ...", rebuttal to reviewer S6y1, first answer);
 *     the CG tensor as the coordinates of the SO(3) tensor product in the
 *     coupled basis (same page, rebuttal to reviewer 7Mvd, last answer);
 *   - the CGTP convolution whose cost LunaTP attacks ("LunaTP: Enabling
 *     Efficient and Scalable Tensor Product for Equivariant MLIPs",
 *     Abstract): for every edge j->i, node features of j are coupled with the
 *     spherical harmonics of the edge through the real-basis CG coefficients,
 *     scaled by per-edge, per-path, per-channel weights and summed into i;
 *   - the gradient of a bilinear map with respect to each of its inputs
 *     (TDN rebuttal to S6y1, the backward formulas after Equation (3)),
 *     applied to the trilinear form <G, out(x, Y, W)>.
 * Formulas the pages leave open are textbook: Racah's closed formula for the
 * complex CG coefficients (Condon-Shortley phase), the unitary change from the
 * complex to the real spherical-harmonic basis, and the closed forms of the
 * orthonormal real spherical harmonics for l <= 3.
 *
 * Conventions:
 *   component index k(l,m) = l*l + l + m, m = -l..l
 *   paths (l1,l2,l3) in lexicographic order, no parity filter
 *   x[N][D_in][C], Y[E][D_sh], W[E][P][C], out/G/dx[N][D][C], dW[E][P][C],
 *   dY[E][D_sh]; receiver-sorted CSR row_ptr[N+1], src[E] (int64 here).
 * Everything is fp64.  Loops are the plain definition: no blocking, fusion or
 * reordering.  OpenMP only splits independent output rows across threads
 * (per-thread buffers for the scattered dx, summed at the end).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_MAXL 6

static double orc_fact(int n)
{
    double r = 1.0;
    for (int i = 2; i <= n; ++i) r *= (double)i;
    return r;
}

/* <j1 m1 j2 m2 | J M> in the complex basis (Racah's closed formula). */
double orc_cg_complex(int j1, int m1, int j2, int m2, int J, int M)
{
    if (M != m1 + m2) return 0.0;
    if (j1 < 0 || j2 < 0 || J < 0) return 0.0;
    if (J < abs(j1 - j2) || J > j1 + j2) return 0.0;
    if (abs(m1) > j1 || abs(m2) > j2 || abs(M) > J) return 0.0;
    double pre = sqrt((2.0 * J + 1.0) * orc_fact(J + j1 - j2) * orc_fact(J - j1 + j2) *
                      orc_fact(j1 + j2 - J) / orc_fact(j1 + j2 + J + 1));
    pre *= sqrt(orc_fact(J + M) * orc_fact(J - M) * orc_fact(j1 - m1) * orc_fact(j1 + m1) *
                orc_fact(j2 - m2) * orc_fact(j2 + m2));
    double sum = 0.0;
    for (int k = 0; k <= j1 + j2 + J; ++k) {
        int a = j1 + j2 - J - k, b = j1 - m1 - k, c = j2 + m2 - k;
        int d = J - j2 + m1 + k, e = J - j1 - m2 + k;
        if (a < 0 || b < 0 || c < 0 || d < 0 || e < 0) continue;
        double term = 1.0 / (orc_fact(k) * orc_fact(a) * orc_fact(b) * orc_fact(c) *
                             orc_fact(d) * orc_fact(e));
        sum += (k & 1) ? -term : term;
    }
    return pre * sum;
}

/* Row m (real), column mu (complex) of the unitary complex->real change of
 * basis for degree l, so that Y_real[m] = sum_mu U[m][mu] Y_complex[mu]. */
static void orc_U(int l, int m, int mu, double* re, double* im)
{
    const double s = 1.0 / sqrt(2.0);
    const double sgn = (abs(m) & 1) ? -1.0 : 1.0; /* (-1)^m */
    *re = 0.0;
    *im = 0.0;
    (void)l;
    if (m == 0) {
        if (mu == 0) *re = 1.0;
    } else if (m > 0) {
        if (mu == m) *re = sgn * s;
        else if (mu == -m) *re = s;
    } else {
        if (mu == m) *im = s;
        else if (mu == -m) *im = -sgn * s;
    }
}

/* Real-basis coupling tensor of path (l1,l2,l3) before taking a real part:
 * S[m1][m2][m3] = sum U1[m1][mu1] U2[m2][mu2] conj(U3[m3][mu3]) <l1 mu1 l2 mu2|l3 mu3>.
 * Dense, index ((m1+l1)*(2l2+1) + (m2+l2))*(2l3+1) + (m3+l3). */
void orc_real_cg_parts(int l1, int l2, int l3, double* re_out, double* im_out)
{
    const int d1 = 2 * l1 + 1, d2 = 2 * l2 + 1, d3 = 2 * l3 + 1;
    for (int m1 = -l1; m1 <= l1; ++m1)
        for (int m2 = -l2; m2 <= l2; ++m2)
            for (int m3 = -l3; m3 <= l3; ++m3) {
                double sre = 0.0, sim = 0.0;
                for (int u1 = -l1; u1 <= l1; ++u1)
                    for (int u2 = -l2; u2 <= l2; ++u2) {
                        int u3 = u1 + u2;
                        if (u3 < -l3 || u3 > l3) continue;
                        double cg = orc_cg_complex(l1, u1, l2, u2, l3, u3);
                        if (cg == 0.0) continue;
                        double ar, ai, br, bi, cr, ci;
                        orc_U(l1, m1, u1, &ar, &ai);
                        orc_U(l2, m2, u2, &br, &bi);
                        orc_U(l3, m3, u3, &cr, &ci);
                        ci = -ci; /* conjugate */
                        /* (a*b) */
                        double abr = ar * br - ai * bi, abi = ar * bi + ai * br;
                        /* (a*b)*c */
                        double pr = abr * cr - abi * ci, pi = abr * ci + abi * cr;
                        sre += pr * cg;
                        sim += pi * cg;
                    }
                int idx = ((m1 + l1) * d2 + (m2 + l2)) * d3 + (m3 + l3);
                re_out[idx] = sre;
                im_out[idx] = sim;
            }
    (void)d1;
}

/* Real CG tensor T of path (l1,l2,l3): Re S for even l1+l2+l3, Im S for odd;
 * entries below 1e-14 in magnitude are set to exactly zero. */
void orc_real_cg(int l1, int l2, int l3, double* T)
{
    const int n = (2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1);
    double* re = (double*)malloc(sizeof(double) * n);
    double* im = (double*)malloc(sizeof(double) * n);
    orc_real_cg_parts(l1, l2, l3, re, im);
    const int odd = (l1 + l2 + l3) & 1;
    for (int i = 0; i < n; ++i) {
        double v = odd ? im[i] : re[i];
        T[i] = fabs(v) < 1e-14 ? 0.0 : v;
    }
    free(re);
    free(im);
}

/* Paths (l1,l2,l3), l1<=lin, l2<=lsh, l3<=lout, |l1-l2|<=l3<=l1+l2, in
 * lexicographic order.  Writes [P][3] into paths when non-NULL; returns P. */
int orc_paths(int lin, int lsh, int lout, int* paths)
{
    int P = 0;
    for (int l1 = 0; l1 <= lin; ++l1)
        for (int l2 = 0; l2 <= lsh; ++l2)
            for (int l3 = 0; l3 <= lout; ++l3) {
                if (l3 < abs(l1 - l2) || l3 > l1 + l2) continue;
                if (paths) {
                    paths[3 * P + 0] = l1;
                    paths[3 * P + 1] = l2;
                    paths[3 * P + 2] = l3;
                }
                ++P;
            }
    return P;
}

/* Orthonormal real spherical harmonics (Condon-Shortley phase folded into the
 * real basis), degrees 0..L (L <= 3), of the unit vector along each r[e].
 * Y[e][l*l+l+m]. */
void orc_sh(int L, int64_t E, const double* r, double* Y)
{
    const double pi = 3.14159265358979323846;
    const int D = (L + 1) * (L + 1);
    for (int64_t e = 0; e < E; ++e) {
        double rx = r[3 * e + 0], ry = r[3 * e + 1], rz = r[3 * e + 2];
        double n = sqrt(rx * rx + ry * ry + rz * rz);
        double x = rx / n, y = ry / n, z = rz / n;
        double* o = Y + e * D;
        o[0] = 0.5 * sqrt(1.0 / pi);
        if (L >= 1) {
            double c1 = sqrt(3.0 / (4.0 * pi));
            o[1] = c1 * y;
            o[2] = c1 * z;
            o[3] = c1 * x;
        }
        if (L >= 2) {
            o[4] = 0.5 * sqrt(15.0 / pi) * x * y;
            o[5] = 0.5 * sqrt(15.0 / pi) * y * z;
            o[6] = 0.25 * sqrt(5.0 / pi) * (3.0 * z * z - 1.0);
            o[7] = 0.5 * sqrt(15.0 / pi) * x * z;
            o[8] = 0.25 * sqrt(15.0 / pi) * (x * x - y * y);
        }
        if (L >= 3) {
            o[9] = 0.25 * sqrt(35.0 / (2.0 * pi)) * y * (3.0 * x * x - y * y);
            o[10] = 0.5 * sqrt(105.0 / pi) * x * y * z;
            o[11] = 0.25 * sqrt(21.0 / (2.0 * pi)) * y * (5.0 * z * z - 1.0);
            o[12] = 0.25 * sqrt(7.0 / pi) * (5.0 * z * z * z - 3.0 * z);
            o[13] = 0.25 * sqrt(21.0 / (2.0 * pi)) * x * (5.0 * z * z - 1.0);
            o[14] = 0.25 * sqrt(105.0 / pi) * z * (x * x - y * y);
            o[15] = 0.25 * sqrt(35.0 / (2.0 * pi)) * x * (x * x - 3.0 * y * y);
        }
    }
}

/* Gradient of the spherical harmonics with respect to the edge vector:
 *   dr[e][a] = sum_k dY[e][k] dY_k(r[e]) / dr_a,   k over degrees 0..L (L <= 3).
 * Each Y_k is a polynomial P_k(u) of the unit vector u = r/|r| (the closed
 * forms of orc_sh).  With g_b = sum_k dY[e][k] dP_k/du_b (the gradient of
 * the polynomial, x, y, z taken as independent) and du_b/dr_a =
 * (delta_ab - u_a u_b)/|r|, the chain rule gives dr = (g - u (u.g)) / |r|:
 * only the part of g tangent to the sphere survives, so any polynomial that
 * agrees with Y_k on the sphere gives the same result.  This is the edge
 * term of the forces that the convolution backward's grad_Y feeds (the
 * finite-difference-validated analytic forces of the AccelNet review,
 * Referee Report). */
void orc_sh_bwd(int L, int64_t E, const double* r, const double* dY, double* dr)
{
    const double pi = 3.14159265358979323846;
    const int D = (L + 1) * (L + 1);
    for (int64_t e = 0; e < E; ++e) {
        double rx = r[3 * e + 0], ry = r[3 * e + 1], rz = r[3 * e + 2];
        double n = sqrt(rx * rx + ry * ry + rz * rz);
        double x = rx / n, y = ry / n, z = rz / n;
        const double* w = dY + e * D;
        double gx = 0.0, gy = 0.0, gz = 0.0;
        if (L >= 1) {
            double c1 = sqrt(3.0 / (4.0 * pi));
            gy += w[1] * c1; /* c1 y */
            gz += w[2] * c1; /* c1 z */
            gx += w[3] * c1; /* c1 x */
        }
        if (L >= 2) {
            double a = 0.5 * sqrt(15.0 / pi), b = 0.25 * sqrt(5.0 / pi), c = 0.25 * sqrt(15.0 / pi);
            gx += w[4] * a * y;  gy += w[4] * a * x;                       /* a x y */
            gy += w[5] * a * z;  gz += w[5] * a * y;                       /* a y z */
            gz += w[6] * 6.0 * b * z;                                      /* b (3 z^2 - 1) */
            gx += w[7] * a * z;  gz += w[7] * a * x;                       /* a x z */
            gx += w[8] * 2.0 * c * x;  gy -= w[8] * 2.0 * c * y;           /* c (x^2 - y^2) */
        }
        if (L >= 3) {
            double a = 0.25 * sqrt(35.0 / (2.0 * pi)), b = 0.5 * sqrt(105.0 / pi);
            double c = 0.25 * sqrt(21.0 / (2.0 * pi)), d = 0.25 * sqrt(7.0 / pi), f = 0.25 * sqrt(105.0 / pi);
            /* a y (3 x^2 - y^2) */
            gx += w[9] * 6.0 * a * x * y;  gy += w[9] * 3.0 * a * (x * x - y * y);
            /* b x y z */
            gx += w[10] * b * y * z;  gy += w[10] * b * x * z;  gz += w[10] * b * x * y;
            /* c y (5 z^2 - 1) */
            gy += w[11] * c * (5.0 * z * z - 1.0);  gz += w[11] * 10.0 * c * y * z;
            /* d (5 z^3 - 3 z) */
            gz += w[12] * d * (15.0 * z * z - 3.0);
            /* c x (5 z^2 - 1) */
            gx += w[13] * c * (5.0 * z * z - 1.0);  gz += w[13] * 10.0 * c * x * z;
            /* f z (x^2 - y^2) */
            gx += w[14] * 2.0 * f * x * z;  gy -= w[14] * 2.0 * f * y * z;  gz += w[14] * f * (x * x - y * y);
            /* a x (x^2 - 3 y^2) */
            gx += w[15] * 3.0 * a * (x * x - y * y);  gy -= w[15] * 6.0 * a * x * y;
        }
        double ug = x * gx + y * gy + z * gz;
        dr[3 * e + 0] = (gx - x * ug) / n;
        dr[3 * e + 1] = (gy - y * ug) / n;
        dr[3 * e + 2] = (gz - z * ug) / n;
    }
}

/* Per-node gradient from per-edge gradients of the edge vectors
 * r[e] = pos[src e] - pos[dst e]:
 *   dpos[j] = sum_{e: src e = j} dr[e] - sum_{e: dst e = j} dr[e].
 * (The force on atom j is -dpos[j].)  dpos is overwritten. */
void orc_node_grad(int64_t N, int64_t E, const int64_t* row_ptr, const int64_t* src, const double* dr,
                   double* dpos)
{
    (void)E;
    for (int64_t q = 0; q < 3 * N; ++q) dpos[q] = 0.0;
    for (int64_t i = 0; i < N; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e)
            for (int a = 0; a < 3; ++a) {
                dpos[3 * src[e] + a] += dr[3 * e + a];
                dpos[3 * i + a] -= dr[3 * e + a];
            }
}

/* Per-plan tables: path list and dense real CG tensors. */
typedef struct {
    int P;
    int paths[3 * 64];
    double* T[64];
} orc_tables;

static int orc_tables_make(int lin, int lsh, int lout, orc_tables* t)
{
    if (lin < 0 || lsh < 0 || lout < 0 || lin > ORC_MAXL || lsh > ORC_MAXL || lout > ORC_MAXL)
        return -1;
    t->P = orc_paths(lin, lsh, lout, NULL);
    if (t->P > 64) return -1;
    orc_paths(lin, lsh, lout, t->paths);
    for (int p = 0; p < t->P; ++p) {
        int l1 = t->paths[3 * p], l2 = t->paths[3 * p + 1], l3 = t->paths[3 * p + 2];
        t->T[p] = (double*)malloc(sizeof(double) * (2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1));
        orc_real_cg(l1, l2, l3, t->T[p]);
    }
    return 0;
}

static void orc_tables_free(orc_tables* t)
{
    for (int p = 0; p < t->P; ++p) free(t->T[p]);
}

/* Forward:
 * out[i][k(l3,m3)][u] = sum_{e in seg(i)} sum_{p=(l1,l2,l3)} W[e][p][u]
 *     sum_{m1,m2} T_p[m1][m2][m3] x[src e][k(l1,m1)][u] Y[e][k(l2,m2)].
 * out is overwritten.  Returns 0, or -1 on unsupported degrees. */
int orc_conv_fwd(int lin, int lsh, int lout, int C, int64_t N, int64_t E,
                 const int64_t* row_ptr, const int64_t* src, const double* x,
                 const double* Y, const double* W, double* out)
{
    orc_tables t;
    if (orc_tables_make(lin, lsh, lout, &t)) return -1;
    const int Din = (lin + 1) * (lin + 1), Dsh = (lsh + 1) * (lsh + 1);
    const int Dout = (lout + 1) * (lout + 1);
    const int P = t.P;
    (void)E;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < N; ++i) {
        double* o = out + i * Dout * C;
        for (int q = 0; q < Dout * C; ++q) o[q] = 0.0;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            const int64_t j = src[e];
            for (int p = 0; p < P; ++p) {
                const int l1 = t.paths[3 * p], l2 = t.paths[3 * p + 1], l3 = t.paths[3 * p + 2];
                const double* T = t.T[p];
                for (int u = 0; u < C; ++u) {
                    const double w = W[(e * P + p) * C + u];
                    for (int m1 = -l1; m1 <= l1; ++m1)
                        for (int m2 = -l2; m2 <= l2; ++m2)
                            for (int m3 = -l3; m3 <= l3; ++m3) {
                                double c = T[((m1 + l1) * (2 * l2 + 1) + (m2 + l2)) * (2 * l3 + 1) +
                                             (m3 + l3)];
                                if (c == 0.0) continue;
                                double xv = x[(j * Din + l1 * l1 + l1 + m1) * C + u];
                                double yv = Y[e * Dsh + l2 * l2 + l2 + m2];
                                o[(l3 * l3 + l3 + m3) * C + u] += w * c * xv * yv;
                            }
                }
            }
        }
    }
    orc_tables_free(&t);
    return 0;
}

/* Backward of L = <G, out>:
 *   dx[j][k(l1,m1)][u] = sum_{e: src e = j} sum_p W[e][p][u]
 *                          sum_{m2,m3} T_p[m1][m2][m3] Y[e][k(l2,m2)] G[dst e][k(l3,m3)][u]
 *   dW[e][p][u]       = sum_{m1,m2,m3} T x[src e][k(l1,m1)][u] Y[e][k(l2,m2)] G[dst e][k(l3,m3)][u]
 *   dY[e][k(l2,m2)]   = sum_u sum_p W[e][p][u] sum_{m1,m3} T x[src e][.][u] G[dst e][.][u]
 * Any of dx, dW, dY may be NULL (skipped).  Outputs are overwritten. */
int orc_conv_bwd(int lin, int lsh, int lout, int C, int64_t N, int64_t E,
                 const int64_t* row_ptr, const int64_t* src, const double* x,
                 const double* Y, const double* W, const double* G, double* dx,
                 double* dW, double* dY)
{
    orc_tables t;
    if (orc_tables_make(lin, lsh, lout, &t)) return -1;
    const int Din = (lin + 1) * (lin + 1), Dsh = (lsh + 1) * (lsh + 1);
    const int Dout = (lout + 1) * (lout + 1);
    const int P = t.P;

    /* receiver of every edge, from the CSR */
    int64_t* dst = (int64_t*)malloc(sizeof(int64_t) * (E > 0 ? E : 1));
    for (int64_t i = 0; i < N; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) dst[e] = i;

    /* dW and dY: independent per edge */
    if (dW || dY) {
#pragma omp parallel for schedule(dynamic, 64)
        for (int64_t e = 0; e < E; ++e) {
            const int64_t j = src[e], i = dst[e];
            if (dY)
                for (int q = 0; q < Dsh; ++q) dY[e * Dsh + q] = 0.0;
            for (int p = 0; p < P; ++p) {
                const int l1 = t.paths[3 * p], l2 = t.paths[3 * p + 1], l3 = t.paths[3 * p + 2];
                const double* T = t.T[p];
                for (int u = 0; u < C; ++u) {
                    const double w = W[(e * P + p) * C + u];
                    double acc = 0.0;
                    for (int m1 = -l1; m1 <= l1; ++m1)
                        for (int m2 = -l2; m2 <= l2; ++m2)
                            for (int m3 = -l3; m3 <= l3; ++m3) {
                                double c = T[((m1 + l1) * (2 * l2 + 1) + (m2 + l2)) * (2 * l3 + 1) +
                                             (m3 + l3)];
                                if (c == 0.0) continue;
                                double xv = x[(j * Din + l1 * l1 + l1 + m1) * C + u];
                                double yv = Y[e * Dsh + l2 * l2 + l2 + m2];
                                double gv = G[(i * Dout + l3 * l3 + l3 + m3) * C + u];
                                acc += c * xv * yv * gv;
                                if (dY) dY[e * Dsh + l2 * l2 + l2 + m2] += w * c * xv * gv;
                            }
                    if (dW) dW[(e * P + p) * C + u] = acc;
                }
            }
        }
    }

    /* dx: scatter over edges into per-thread buffers, then sum */
    if (dx) {
        const int64_t rowlen = (int64_t)Din * C;
        for (int64_t q = 0; q < N * rowlen; ++q) dx[q] = 0.0;
#pragma omp parallel
        {
            double* mine = dx;
            int nthr = 1;
#ifdef _OPENMP
            nthr = omp_get_num_threads();
#endif
            if (nthr > 1) mine = (double*)calloc((size_t)(N * rowlen > 0 ? N * rowlen : 1), sizeof(double));
#pragma omp for schedule(static)
            for (int64_t e = 0; e < E; ++e) {
                const int64_t j = src[e], i = dst[e];
                for (int p = 0; p < P; ++p) {
                    const int l1 = t.paths[3 * p], l2 = t.paths[3 * p + 1], l3 = t.paths[3 * p + 2];
                    const double* T = t.T[p];
                    for (int u = 0; u < C; ++u) {
                        const double w = W[(e * P + p) * C + u];
                        for (int m1 = -l1; m1 <= l1; ++m1)
                            for (int m2 = -l2; m2 <= l2; ++m2)
                                for (int m3 = -l3; m3 <= l3; ++m3) {
                                    double c = T[((m1 + l1) * (2 * l2 + 1) + (m2 + l2)) * (2 * l3 + 1) +
                                                 (m3 + l3)];
                                    if (c == 0.0) continue;
                                    double yv = Y[e * Dsh + l2 * l2 + l2 + m2];
                                    double gv = G[(i * Dout + l3 * l3 + l3 + m3) * C + u];
                                    mine[(j * Din + l1 * l1 + l1 + m1) * C + u] += w * c * yv * gv;
                                }
                    }
                }
            }
            if (nthr > 1) {
#pragma omp critical
                for (int64_t q = 0; q < N * rowlen; ++q) dx[q] += mine[q];
                free(mine);
            }
        }
    }
    free(dst);
    orc_tables_free(&t);
    return 0;
}

/* Per-path (concatenated) outputs: path p keeps its own 2*l3+1 rows,
 * rows o_p .. o_p + 2*l3 with o_p = sum over earlier paths of (2*l3+1), so
 * out_mid [N][D_mid][C], D_mid = sum_p (2*l3+1):
 *   out_mid[i][o_p + l3 + m3][u] = sum_{e in seg(i)} W[e][p][u]
 *       sum_{m1,m2} T_p[m1][m2][m3] x[src e][k(l1,m1)][u] Y[e][k(l2,m2)].
 * Summing the blocks of the paths of each l3 gives orc_conv_fwd. */
int orc_conv_fwd_mid(int lin, int lsh, int lout, int C, int64_t N, const int64_t* row_ptr, const int64_t* src,
                     const double* x, const double* Y, const double* W, double* out)
{
    orc_tables t;
    if (orc_tables_make(lin, lsh, lout, &t)) return -1;
    const int Din = (lin + 1) * (lin + 1), Dsh = (lsh + 1) * (lsh + 1), P = t.P;
    int o[64], Dmid = 0;
    for (int p = 0; p < P; ++p) {
        o[p] = Dmid;
        Dmid += 2 * t.paths[3 * p + 2] + 1;
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < N; ++i) {
        double* op = out + i * Dmid * C;
        for (int q = 0; q < Dmid * C; ++q) op[q] = 0.0;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            const int64_t j = src[e];
            for (int p = 0; p < P; ++p) {
                const int l1 = t.paths[3 * p], l2 = t.paths[3 * p + 1], l3 = t.paths[3 * p + 2];
                for (int u = 0; u < C; ++u) {
                    const double w = W[(e * P + p) * C + u];
                    for (int m1 = -l1; m1 <= l1; ++m1)
                        for (int m2 = -l2; m2 <= l2; ++m2)
                            for (int m3 = -l3; m3 <= l3; ++m3) {
                                double c = t.T[p][((m1 + l1) * (2 * l2 + 1) + (m2 + l2)) * (2 * l3 + 1) + (m3 + l3)];
                                if (c == 0.0) continue;
                                op[(o[p] + l3 + m3) * C + u] += w * c * x[(j * Din + l1 * l1 + l1 + m1) * C + u] *
                                                                Y[e * Dsh + l2 * l2 + l2 + m2];
                            }
                }
            }
        }
    }
    orc_tables_free(&t);
    return 0;
}

/* Backward of L = <G_mid, out_mid> (G_mid [N][D_mid][C]): as orc_conv_bwd,
 * with path p coupled to its own block G_mid[dst e][o_p + l3 + m3] instead
 * of the l3 slot.  A NULL output is skipped; outputs are overwritten. */
int orc_conv_bwd_mid(int lin, int lsh, int lout, int C, int64_t N, int64_t E, const int64_t* row_ptr,
                     const int64_t* src, const double* x, const double* Y, const double* W, const double* G,
                     double* dx, double* dW, double* dY)
{
    orc_tables t;
    if (orc_tables_make(lin, lsh, lout, &t)) return -1;
    const int Din = (lin + 1) * (lin + 1), Dsh = (lsh + 1) * (lsh + 1), P = t.P;
    int o[64], Dmid = 0;
    for (int p = 0; p < P; ++p) {
        o[p] = Dmid;
        Dmid += 2 * t.paths[3 * p + 2] + 1;
    }
    int64_t* dst = (int64_t*)malloc(sizeof(int64_t) * (E > 0 ? E : 1));
    for (int64_t i = 0; i < N; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) dst[e] = i;
    if (dx)
        for (int64_t q = 0; q < N * Din * C; ++q) dx[q] = 0.0;
    /* per edge: dW, dY; dx scattered serially (plain and order-independent in exact arithmetic) */
    for (int64_t e = 0; e < E; ++e) {
        const int64_t j = src[e], i = dst[e];
        if (dY)
            for (int q = 0; q < Dsh; ++q) dY[e * Dsh + q] = 0.0;
        for (int p = 0; p < P; ++p) {
            const int l1 = t.paths[3 * p], l2 = t.paths[3 * p + 1], l3 = t.paths[3 * p + 2];
            for (int u = 0; u < C; ++u) {
                const double w = W[(e * P + p) * C + u];
                double acc = 0.0;
                for (int m1 = -l1; m1 <= l1; ++m1)
                    for (int m2 = -l2; m2 <= l2; ++m2)
                        for (int m3 = -l3; m3 <= l3; ++m3) {
                            double c = t.T[p][((m1 + l1) * (2 * l2 + 1) + (m2 + l2)) * (2 * l3 + 1) + (m3 + l3)];
                            if (c == 0.0) continue;
                            const double xv = x[(j * Din + l1 * l1 + l1 + m1) * C + u];
                            const double yv = Y[e * Dsh + l2 * l2 + l2 + m2];
                            const double gv = G[(i * Dmid + o[p] + l3 + m3) * C + u];
                            acc += c * xv * yv * gv;
                            if (dx) dx[(j * Din + l1 * l1 + l1 + m1) * C + u] += w * c * yv * gv;
                            if (dY) dY[e * Dsh + l2 * l2 + l2 + m2] += w * c * xv * gv;
                        }
                if (dW) dW[(e * P + p) * C + u] = acc;
            }
        }
    }
    free(dst);
    orc_tables_free(&t);
    return 0;
}

/* Double backward: the gradients of
 *   S = <ggx, dx> + <ggW, dW> + <ggY, dY>,   (dx, dW, dY) = orc_conv_bwd(x, Y, W, G),
 * with respect to x, Y, W and G (the higher-order derivatives LunaTP's
 * abstract names; force training differentiates the backward again).  The
 * loss L(x, Y, W, G) = <G, out(x, Y, W)> is linear in each argument, so
 * S = L(ggx, Y, W, G) + L(x, Y, ggW, G) + L(x, ggY, W, G) and every term of
 * its gradients is read off the single coupling c = T_p[m1][m2][m3] of one
 * edge, path, channel and (m1, m2, m3):
 *   dG[i][k3][u] += c (ggx Y W + x ggY W + x Y ggW)
 *   dx[j][k1][u] += c (ggY W G + Y ggW G)
 *   dW[e][p][u]  += c (ggx Y G + x ggY G)
 *   dY[e][k2]    += sum_u c (ggx W G + x ggW G)
 * (x, ggx at the sender j, G at the receiver i).  A NULL cotangent counts as
 * zero; a NULL output is skipped; outputs are overwritten. */
int orc_conv_bwd_bwd(int lin, int lsh, int lout, int C, int64_t N, int64_t E, const int64_t* row_ptr,
                     const int64_t* src, const double* x, const double* Y, const double* W, const double* G,
                     const double* ggx, const double* ggY, const double* ggW, double* dx, double* dY,
                     double* dW, double* dG)
{
    orc_tables t;
    if (orc_tables_make(lin, lsh, lout, &t)) return -1;
    const int Din = (lin + 1) * (lin + 1), Dsh = (lsh + 1) * (lsh + 1);
    const int Dout = (lout + 1) * (lout + 1);
    const int P = t.P;
    int64_t* dst = (int64_t*)malloc(sizeof(int64_t) * (E > 0 ? E : 1));
    for (int64_t i = 0; i < N; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) dst[e] = i;
#define ORC_X(a) x[(j * Din + (a)) * C + u]
#define ORC_GX(a) (ggx ? ggx[(j * Din + (a)) * C + u] : 0.0)
#define ORC_Y(b) Y[e * Dsh + (b)]
#define ORC_GY(b) (ggY ? ggY[e * Dsh + (b)] : 0.0)
#define ORC_W W[(e * P + p) * C + u]
#define ORC_GW (ggW ? ggW[(e * P + p) * C + u] : 0.0)
#define ORC_G(c3) G[(i * Dout + (c3)) * C + u]
    /* dG: per receiver */
    if (dG) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < N; ++i) {
            double* o = dG + i * Dout * C;
            for (int q = 0; q < Dout * C; ++q) o[q] = 0.0;
            for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
                const int64_t j = src[e];
                for (int p = 0; p < P; ++p) {
                    const int l1 = t.paths[3 * p], l2 = t.paths[3 * p + 1], l3 = t.paths[3 * p + 2];
                    for (int u = 0; u < C; ++u)
                        for (int m1 = -l1; m1 <= l1; ++m1)
                            for (int m2 = -l2; m2 <= l2; ++m2)
                                for (int m3 = -l3; m3 <= l3; ++m3) {
                                    double c = t.T[p][((m1 + l1) * (2 * l2 + 1) + (m2 + l2)) * (2 * l3 + 1) + (m3 + l3)];
                                    if (c == 0.0) continue;
                                    int a = l1 * l1 + l1 + m1, b = l2 * l2 + l2 + m2;
                                    o[(l3 * l3 + l3 + m3) * C + u] +=
                                        c * (ORC_GX(a) * ORC_Y(b) * ORC_W + ORC_X(a) * ORC_GY(b) * ORC_W +
                                             ORC_X(a) * ORC_Y(b) * ORC_GW);
                                }
                }
            }
        }
    }
    /* dW, dY: per edge */
    if (dW || dY) {
#pragma omp parallel for schedule(dynamic, 64)
        for (int64_t e = 0; e < E; ++e) {
            const int64_t j = src[e], i = dst[e];
            if (dY)
                for (int q = 0; q < Dsh; ++q) dY[e * Dsh + q] = 0.0;
            for (int p = 0; p < P; ++p) {
                const int l1 = t.paths[3 * p], l2 = t.paths[3 * p + 1], l3 = t.paths[3 * p + 2];
                for (int u = 0; u < C; ++u) {
                    double acc = 0.0;
                    for (int m1 = -l1; m1 <= l1; ++m1)
                        for (int m2 = -l2; m2 <= l2; ++m2)
                            for (int m3 = -l3; m3 <= l3; ++m3) {
                                double c = t.T[p][((m1 + l1) * (2 * l2 + 1) + (m2 + l2)) * (2 * l3 + 1) + (m3 + l3)];
                                if (c == 0.0) continue;
                                int a = l1 * l1 + l1 + m1, b = l2 * l2 + l2 + m2, k3 = l3 * l3 + l3 + m3;
                                acc += c * (ORC_GX(a) * ORC_Y(b) + ORC_X(a) * ORC_GY(b)) * ORC_G(k3);
                                if (dY) dY[e * Dsh + b] += c * (ORC_GX(a) * ORC_W + ORC_X(a) * ORC_GW) * ORC_G(k3);
                            }
                    if (dW) dW[(e * P + p) * C + u] = acc;
                }
            }
        }
    }
    /* dx: scattered over edges into per-thread buffers, then summed */
    if (dx) {
        const int64_t rowlen = (int64_t)Din * C;
        for (int64_t q = 0; q < N * rowlen; ++q) dx[q] = 0.0;
#pragma omp parallel
        {
            double* mine = dx;
            int nthr = 1;
#ifdef _OPENMP
            nthr = omp_get_num_threads();
#endif
            if (nthr > 1) mine = (double*)calloc((size_t)(N * rowlen > 0 ? N * rowlen : 1), sizeof(double));
#pragma omp for schedule(static)
            for (int64_t e = 0; e < E; ++e) {
                const int64_t j = src[e], i = dst[e];
                for (int p = 0; p < P; ++p) {
                    const int l1 = t.paths[3 * p], l2 = t.paths[3 * p + 1], l3 = t.paths[3 * p + 2];
                    for (int u = 0; u < C; ++u)
                        for (int m1 = -l1; m1 <= l1; ++m1)
                            for (int m2 = -l2; m2 <= l2; ++m2)
                                for (int m3 = -l3; m3 <= l3; ++m3) {
                                    double c = t.T[p][((m1 + l1) * (2 * l2 + 1) + (m2 + l2)) * (2 * l3 + 1) + (m3 + l3)];
                                    if (c == 0.0) continue;
                                    int a = l1 * l1 + l1 + m1, b = l2 * l2 + l2 + m2, k3 = l3 * l3 + l3 + m3;
                                    mine[(j * Din + a) * C + u] +=
                                        c * (ORC_GY(b) * ORC_W + ORC_Y(b) * ORC_GW) * ORC_G(k3);
                                }
                }
            }
            if (nthr > 1) {
#pragma omp critical
                for (int64_t q = 0; q < N * rowlen; ++q) dx[q] += mine[q];
                free(mine);
            }
        }
    }
#undef ORC_X
#undef ORC_GX
#undef ORC_Y
#undef ORC_GY
#undef ORC_W
#undef ORC_GW
#undef ORC_G
    free(dst);
    orc_tables_free(&t);
    return 0;
}

/* CP-decomposed tensor-product convolution ("Tensor Decomposition Networks
 * ...", rebuttal to S6y1: Equation (3) and the gradients derived after it).
 * The coupling of x (d1 components) and y (d2) into z (d3) is approximated by
 * rank-R factors A [d3][R], B [d1][R], Cf [d2][R] (row-major):
 *   z = A (B^T x  (.)  Cf^T y).
 * Per edge e = j->i and channel u, with one weight W[e][u]:
 *   out[i][:,u] += W[e][u] * A (B^T x[j][:,u] (.) Cf^T Y[e]).
 * out is overwritten. */
void orc_cp_conv_fwd(int d1, int d2, int d3, int R, int C, int64_t N, const int64_t* row_ptr,
                     const int64_t* src, const double* x, const double* Y, const double* W, const double* A,
                     const double* B, const double* Cf, double* out)
{
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (R > 0 ? R : 1));
        double* t = (double*)malloc(sizeof(double) * (R > 0 ? R : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < N; ++i) {
            double* o = out + i * d3 * C;
            for (int q = 0; q < d3 * C; ++q) o[q] = 0.0;
            for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
                const int64_t j = src[e];
                for (int r = 0; r < R; ++r) {
                    t[r] = 0.0;
                    for (int b = 0; b < d2; ++b) t[r] += Cf[b * R + r] * Y[e * d2 + b];
                }
                for (int u = 0; u < C; ++u) {
                    for (int r = 0; r < R; ++r) {
                        s[r] = 0.0;
                        for (int a = 0; a < d1; ++a) s[r] += B[a * R + r] * x[(j * d1 + a) * C + u];
                    }
                    const double w = W[e * C + u];
                    for (int c = 0; c < d3; ++c) {
                        double z = 0.0;
                        for (int r = 0; r < R; ++r) z += A[c * R + r] * s[r] * t[r];
                        o[c * C + u] += w * z;
                    }
                }
            }
        }
        free(s);
        free(t);
    }
}

/* Its backward for L = <G, out>, by the closed forms after Equation (3)
 * (g_x = (g_z A (.) Cf^T y) B^T and g_y = (g_z A (.) B^T x) Cf^T, here with
 * the edge weight and the channel sum): with g = G[i][:,u] for edge e = j->i,
 *   dx[j][:,u] += W[e][u] B (A^T g (.) Cf^T Y[e])
 *   dY[e]      += sum_u W[e][u] Cf (A^T g (.) B^T x[j][:,u])
 *   dW[e][u]    = <g, A (B^T x[j][:,u] (.) Cf^T Y[e])>
 * A NULL output is skipped; outputs are overwritten. */
void orc_cp_conv_bwd(int d1, int d2, int d3, int R, int C, int64_t N, int64_t E, const int64_t* row_ptr,
                     const int64_t* src, const double* x, const double* Y, const double* W, const double* A,
                     const double* B, const double* Cf, const double* G, double* dx, double* dY, double* dW)
{
    int64_t* dst = (int64_t*)malloc(sizeof(int64_t) * (E > 0 ? E : 1));
    for (int64_t i = 0; i < N; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) dst[e] = i;
    const int64_t rowlen = (int64_t)d1 * C;
    if (dx)
        for (int64_t q = 0; q < N * rowlen; ++q) dx[q] = 0.0;
#pragma omp parallel
    {
        const int Rm = R > 0 ? R : 1;
        double* s = (double*)malloc(sizeof(double) * Rm);
        double* t = (double*)malloc(sizeof(double) * Rm);
        double* ga = (double*)malloc(sizeof(double) * Rm);
        double* mine = dx;
        int nthr = 1;
#ifdef _OPENMP
        nthr = omp_get_num_threads();
#endif
        if (dx && nthr > 1) mine = (double*)calloc((size_t)(N * rowlen > 0 ? N * rowlen : 1), sizeof(double));
#pragma omp for schedule(static)
        for (int64_t e = 0; e < E; ++e) {
            const int64_t j = src[e], i = dst[e];
            for (int r = 0; r < R; ++r) {
                t[r] = 0.0;
                for (int b = 0; b < d2; ++b) t[r] += Cf[b * R + r] * Y[e * d2 + b];
            }
            if (dY)
                for (int b = 0; b < d2; ++b) dY[e * d2 + b] = 0.0;
            for (int u = 0; u < C; ++u) {
                const double w = W[e * C + u];
                for (int r = 0; r < R; ++r) {
                    s[r] = 0.0;
                    for (int a = 0; a < d1; ++a) s[r] += B[a * R + r] * x[(j * d1 + a) * C + u];
                    ga[r] = 0.0;
                    for (int c = 0; c < d3; ++c) ga[r] += A[c * R + r] * G[(i * d3 + c) * C + u];
                }
                if (dx)
                    for (int a = 0; a < d1; ++a) {
                        double v = 0.0;
                        for (int r = 0; r < R; ++r) v += B[a * R + r] * ga[r] * t[r];
                        mine[(j * d1 + a) * C + u] += w * v;
                    }
                if (dY)
                    for (int b = 0; b < d2; ++b) {
                        double v = 0.0;
                        for (int r = 0; r < R; ++r) v += Cf[b * R + r] * ga[r] * s[r];
                        dY[e * d2 + b] += w * v;
                    }
                if (dW) {
                    double v = 0.0;
                    for (int r = 0; r < R; ++r) v += ga[r] * s[r] * t[r];
                    dW[e * C + u] = v;
                }
            }
        }
        if (dx && nthr > 1) {
#pragma omp critical
            for (int64_t q = 0; q < N * rowlen; ++q) dx[q] += mine[q];
            free(mine);
        }
        free(s);
        free(t);
        free(ga);
    }
    free(dst);
}

/* Sender-sorted view of a receiver-sorted CSR (the graph preparation the
 * backward needs): a stable counting sort of the edges by sender.
 *   srow_ptr[N+1]  offsets of each sender's out-edges
 *   perm[E]        edge ids, grouped by sender, ascending edge id within a sender
 *   sdst[E]        receiver of edge perm[k]                                    */
void orc_graph_transpose(int64_t N, int64_t E, const int64_t* row_ptr, const int64_t* src,
                         int64_t* srow_ptr, int64_t* perm, int64_t* sdst)
{
    for (int64_t j = 0; j <= N; ++j) srow_ptr[j] = 0;
    for (int64_t e = 0; e < E; ++e) srow_ptr[src[e] + 1] += 1;
    for (int64_t j = 0; j < N; ++j) srow_ptr[j + 1] += srow_ptr[j];
    int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
    for (int64_t j = 0; j < N; ++j) cursor[j] = srow_ptr[j];
    for (int64_t i = 0; i < N; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            int64_t k = cursor[src[e]]++;
            perm[k] = e;
            sdst[k] = i;
        }
    free(cursor);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
