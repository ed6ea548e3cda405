// cgtp_math.h -- compile-time path lists and real-basis Clebsch-Gordan tables.
//
// The selection rules |l1-l2| <= l3 <= l1+l2 and m3 = m1+m2 decide which
// triples couple at all ("Tensor Decomposition Networks ...", rebuttal to
// reviewer S6y1, first answer); the CG tensor is the coordinate form of the
// SO(3) tensor product in the coupled basis (same page, rebuttal to reviewer
// 7Mvd).  The pages give no formula for the coefficients; this file uses the
// textbook Racah formula for the Wigner 3j symbol (Condon-Shortley phase),
// converts it to CG, and changes basis to real spherical harmonics
//     Y_{l,m} = sqrt2 (-1)^m Im Y_l^{|m|} (m<0), Y_l^0, sqrt2 (-1)^m Re Y_l^m (m>0)
// by scattering every complex coefficient onto the real indices +-|mu|.
// The real tensor is the real part of the result for even l1+l2+l3 and the
// imaginary part for odd l1+l2+l3 (the other part vanishes).
//
// Everything is constexpr: the kernels are specialised on (L_in, L_sh, L_out)
// and read the coefficients as compile-time constants, so the nonzero pattern
// is resolved by the compiler and the values become scalar operands of the
// fp64 FMAs.  The host plan calls the same functions at run time to report the
// tables.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define CGTP_HD __host__ __device__
#else
#define CGTP_HD
#endif

namespace cgtp {
namespace cgmath {

constexpr int kMaxL = 3;

CGTP_HD constexpr int iabs(int v) { return v < 0 ? -v : v; }

// sqrt by Newton's iteration in double (exact to an ulp; usable in constexpr)
CGTP_HD constexpr double csqrt(double v)
{
    if (v <= 0.0) return 0.0;
    double x = v > 1.0 ? v : 1.0;
    for (int it = 0; it < 200; ++it) {
        double nx = 0.5 * (x + v / x);
        if (nx == x) break;
        x = nx;
    }
    // settle a possible 1-ulp oscillation on the smaller candidate
    double nx = 0.5 * (x + v / x);
    return nx < x ? nx : x;
}

CGTP_HD constexpr double factorial(int n)
{
    double r = 1.0;
    for (int i = 2; i <= n; ++i) r *= (double)i;
    return r;
}

// Wigner 3j symbol ( j1 j2 j3 ; m1 m2 m3 ), Racah's formula.
CGTP_HD constexpr double wigner3j(int j1, int j2, int j3, int m1, int m2, int m3)
{
    if (m1 + m2 + m3 != 0) return 0.0;
    if (j3 < iabs(j1 - j2) || j3 > j1 + j2) return 0.0;
    if (iabs(m1) > j1 || iabs(m2) > j2 || iabs(m3) > j3) return 0.0;
    const double tri = factorial(j1 + j2 - j3) * factorial(j1 - j2 + j3) * factorial(-j1 + j2 + j3) /
                       factorial(j1 + j2 + j3 + 1);
    const double pre = csqrt(tri * factorial(j1 + m1) * factorial(j1 - m1) * factorial(j2 + m2) *
                             factorial(j2 - m2) * factorial(j3 + m3) * factorial(j3 - m3));
    // t runs over the integers keeping every factorial argument non-negative
    int tmin = 0;
    if (j2 - j3 - m1 > tmin) tmin = j2 - j3 - m1;
    if (j1 - j3 + m2 > tmin) tmin = j1 - j3 + m2;
    int tmax = j1 + j2 - j3;
    if (j1 - m1 < tmax) tmax = j1 - m1;
    if (j2 + m2 < tmax) tmax = j2 + m2;
    double s = 0.0;
    for (int t = tmin; t <= tmax; ++t) {
        const double den = factorial(t) * factorial(j3 - j2 + t + m1) * factorial(j3 - j1 + t - m2) *
                           factorial(j1 + j2 - j3 - t) * factorial(j1 - t - m1) * factorial(j2 - t + m2);
        s += ((t & 1) ? -1.0 : 1.0) / den;
    }
    const int ph = j1 - j2 - m3;
    return (((ph % 2) + 2) % 2 ? -1.0 : 1.0) * pre * s;
}

// <j1 m1 j2 m2 | J M> = (-1)^(j1-j2+M) sqrt(2J+1) ( j1 j2 J ; m1 m2 -M )
CGTP_HD constexpr double clebsch(int j1, int m1, int j2, int m2, int J, int M)
{
    if (M != m1 + m2) return 0.0;
    const int ph = j1 - j2 + M;
    return (((ph % 2) + 2) % 2 ? -1.0 : 1.0) * csqrt(2.0 * J + 1.0) * wigner3j(j1, j2, J, m1, m2, -M);
}

// Entry U[m][mu] of the complex -> real change of basis as (re, im); only
// |m| == |mu| is nonzero.
struct cplx {
    double re, im;
};
CGTP_HD constexpr cplx cmul(cplx a, cplx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }

CGTP_HD constexpr cplx basis_entry(int m, int mu)
{
    const double h = 0.70710678118654752440;  // 1/sqrt2
    const double sg = (iabs(m) & 1) ? -1.0 : 1.0;
    if (m == 0) return {mu == 0 ? 1.0 : 0.0, 0.0};
    if (m > 0) {
        if (mu == m) return {sg * h, 0.0};
        if (mu == -m) return {h, 0.0};
        return {0.0, 0.0};
    }
    if (mu == m) return {0.0, h};
    if (mu == -m) return {0.0, -sg * h};
    return {0.0, 0.0};
}

// ---- path lists -----------------------------------------------------------

struct Path {
    int l1, l2, l3;
};

CGTP_HD constexpr bool coupled(int l1, int l2, int l3) { return l3 >= iabs(l1 - l2) && l3 <= l1 + l2; }

CGTP_HD constexpr int num_paths(int lin, int lsh, int lout)
{
    int P = 0;
    for (int a = 0; a <= lin; ++a)
        for (int b = 0; b <= lsh; ++b)
            for (int c = 0; c <= lout; ++c)
                if (coupled(a, b, c)) ++P;
    return P;
}

CGTP_HD constexpr Path path_at(int lin, int lsh, int lout, int p)
{
    int q = 0;
    for (int a = 0; a <= lin; ++a)
        for (int b = 0; b <= lsh; ++b)
            for (int c = 0; c <= lout; ++c)
                if (coupled(a, b, c)) {
                    if (q == p) return {a, b, c};
                    ++q;
                }
    return {-1, -1, -1};
}

CGTP_HD constexpr int path_size(Path p) { return (2 * p.l1 + 1) * (2 * p.l2 + 1) * (2 * p.l3 + 1); }

// Every real-basis coefficient is +-sqrt(q) with q a small rational.  Snapping
// to that form (continued fraction of v*v, then one square root) makes equal
// coefficients bit-identical whatever route computed them, so a kernel needs
// only one register constant per distinct magnitude.
CGTP_HD constexpr double canonical(double v)
{
    const double x = v * v;
    int64_t h0 = 0, h1 = 1, k0 = 1, k1 = 0;
    double r = x;
    for (int it = 0; it < 40; ++it) {
        const int64_t a = (int64_t)r;
        const int64_t h2 = a * h1 + h0, k2 = a * k1 + k0;
        h0 = h1;
        h1 = h2;
        k0 = k1;
        k1 = k2;
        const double approx = (double)h1 / (double)k1;
        const double err = approx > x ? approx - x : x - approx;
        if (err <= 1e-13 * x || k1 > 100000000) break;
        const double frac = r - (double)a;
        if (frac < 1e-12) break;
        r = 1.0 / frac;
    }
    const double q = csqrt((double)h1 / (double)k1);
    return v < 0.0 ? -q : q;
}

// real-basis coefficient T_p[m1][m2][m3], computed by scattering every
// complex coefficient <l1 mu1 l2 mu2 | l3 mu1+mu2> onto the real indices
// m_i = +-|mu_i| that it feeds.
CGTP_HD constexpr double real_cg(int l1, int l2, int l3, int m1, int m2, int m3)
{
    double re = 0.0, im = 0.0;
    for (int s1 = 0; s1 < 2; ++s1) {
        const int mu1 = s1 ? -m1 : m1;
        if (s1 && m1 == 0) continue;
        for (int s2 = 0; s2 < 2; ++s2) {
            const int mu2 = s2 ? -m2 : m2;
            if (s2 && m2 == 0) continue;
            const int mu3 = mu1 + mu2;
            if (iabs(mu3) != iabs(m3)) continue;
            const double c = clebsch(l1, mu1, l2, mu2, l3, mu3);
            if (c == 0.0) continue;
            cplx u3 = basis_entry(m3, mu3);
            u3.im = -u3.im;
            const cplx t = cmul(cmul(basis_entry(m1, mu1), basis_entry(m2, mu2)), u3);
            re += c * t.re;
            im += c * t.im;
        }
    }
    const double v = ((l1 + l2 + l3) & 1) ? im : re;
    return (v < 1e-14 && v > -1e-14) ? 0.0 : canonical(v);
}

// ---- compile-time tables ---------------------------------------------------

template <int LIN, int LSH, int LOUT>
struct Tables {
    static constexpr int P = num_paths(LIN, LSH, LOUT);
    static constexpr int DIN = (LIN + 1) * (LIN + 1);
    static constexpr int DSH = (LSH + 1) * (LSH + 1);
    static constexpr int DOUT = (LOUT + 1) * (LOUT + 1);
    static constexpr int total()
    {
        int n = 0;
        for (int p = 0; p < P; ++p) n += path_size(path_at(LIN, LSH, LOUT, p));
        return n;
    }
    static constexpr int SIZE = total();
    struct Data {
        int l1[P], l2[P], l3[P], off[P];
        double T[SIZE];
    };
    static constexpr Data build()
    {
        Data d{};
        int o = 0;
        for (int p = 0; p < P; ++p) {
            const Path q = path_at(LIN, LSH, LOUT, p);
            d.l1[p] = q.l1;
            d.l2[p] = q.l2;
            d.l3[p] = q.l3;
            d.off[p] = o;
            for (int a = -q.l1; a <= q.l1; ++a)
                for (int b = -q.l2; b <= q.l2; ++b)
                    for (int c = -q.l3; c <= q.l3; ++c)
                        d.T[o + ((a + q.l1) * (2 * q.l2 + 1) + (b + q.l2)) * (2 * q.l3 + 1) + (c + q.l3)] =
                            real_cg(q.l1, q.l2, q.l3, a, b, c);
            o += path_size(q);
        }
        return d;
    }
    static constexpr Data data = build();

    // coefficient of path p at (m1, m2, m3)
    CGTP_HD static constexpr double t(int p, int m1, int m2, int m3)
    {
        return data.T[data.off[p] + ((m1 + data.l1[p]) * (2 * data.l2[p] + 1) + (m2 + data.l2[p])) *
                                        (2 * data.l3[p] + 1) +
                      (m3 + data.l3[p])];
    }
    // does the (m1, m3) pair of path p have any nonzero coefficient?
    CGTP_HD static constexpr bool pair_nz(int p, int m1, int m3)
    {
        for (int m2 = -data.l2[p]; m2 <= data.l2[p]; ++m2)
            if (t(p, m1, m2, m3) != 0.0) return true;
        return false;
    }
};

}  // namespace cgmath
}  // namespace cgtp
