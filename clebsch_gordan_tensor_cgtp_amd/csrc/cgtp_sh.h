// cgtp_sh.h -- real spherical harmonics of degrees 0..3 as polynomials of the
// unit vector u = r/|r| (orthonormal, components m = -l..l of each degree in
// the order y, z, x for l = 1), and the gradient of sum_k w_k Y_k(r) with
// respect to r; fp64 device code shared by the SH kernels and the
// convolution kernels that evaluate the harmonics themselves.
//
// The harmonics are the textbook real forms (the coupled basis of the TDN
// rebuttal's reply to 7Mvd needs the same real basis as the CG tables).
// Since Y depends on the direction only, dY/dr = (I - u u^T) grad_u Y / |r|.
#pragma once

#include <hip/hip_runtime.h>

#include "cgtp_math.h"

namespace cgtp {
namespace shf {

constexpr double kPi = 3.14159265358979323846;

// Y_0 .. Y_{(L+1)^2 - 1} at the unit vector (x, y, z)
template <int L, int D>
__device__ __forceinline__ void values(double x, double y, double z, double (&o)[D])
{
    static_assert(D >= (L + 1) * (L + 1), "room for degrees 0..L");
    (void)x, (void)y, (void)z;
    constexpr double c0 = 0.5 * cgmath::csqrt(1.0 / kPi);
    o[0] = c0;
    if constexpr (L >= 1) {
        constexpr double c1 = cgmath::csqrt(3.0 / (4.0 * kPi));
        o[1] = c1 * y;
        o[2] = c1 * z;
        o[3] = c1 * x;
    }
    if constexpr (L >= 2) {
        constexpr double a = 0.5 * cgmath::csqrt(15.0 / kPi);
        constexpr double b = 0.25 * cgmath::csqrt(5.0 / kPi);
        constexpr double c = 0.25 * cgmath::csqrt(15.0 / kPi);
        o[4] = a * x * y;
        o[5] = a * y * z;
        o[6] = b * (3.0 * z * z - 1.0);
        o[7] = a * x * z;
        o[8] = c * (x * x - y * y);
    }
    if constexpr (L >= 3) {
        constexpr double a = 0.25 * cgmath::csqrt(35.0 / (2.0 * kPi));
        constexpr double b = 0.5 * cgmath::csqrt(105.0 / kPi);
        constexpr double c = 0.25 * cgmath::csqrt(21.0 / (2.0 * kPi));
        constexpr double d = 0.25 * cgmath::csqrt(7.0 / kPi);
        constexpr double f = 0.25 * cgmath::csqrt(105.0 / kPi);
        o[9] = a * y * (3.0 * x * x - y * y);
        o[10] = b * x * y * z;
        o[11] = c * y * (5.0 * z * z - 1.0);
        o[12] = d * (5.0 * z * z * z - 3.0 * z);
        o[13] = c * x * (5.0 * z * z - 1.0);
        o[14] = f * z * (x * x - y * y);
        o[15] = a * x * (x * x - 3.0 * y * y);
    }
}

// q += grad_u of sum_b w[b] Y_{l,b}(u), w the 2l+1 weights of degree l
// (degree 0 is constant and adds nothing)
template <int l>
__device__ __forceinline__ void grad_degree(double x, double y, double z, const double* w, double& qx, double& qy,
                                            double& qz)
{
    (void)x, (void)y, (void)z, (void)w, (void)qx, (void)qy, (void)qz;
    if constexpr (l == 1) {
        // sqrt(3/4pi) (y, z, x)
        constexpr double c = cgmath::csqrt(3.0 / (4.0 * kPi));
        qx += c * w[2];
        qy += c * w[0];
        qz += c * w[1];
    } else if constexpr (l == 2) {
        constexpr double s15 = cgmath::csqrt(15.0 / kPi), s5 = cgmath::csqrt(5.0 / kPi);
        // s15/2 xy, s15/2 yz, s5/4 (3z^2-1), s15/2 xz, s15/4 (x^2-y^2)
        const double h = 0.5 * s15;
        qx += h * (w[0] * y + w[3] * z + w[4] * x);
        qy += h * (w[0] * x + w[1] * z - w[4] * y);
        qz += h * (w[1] * y + w[3] * x) + 1.5 * s5 * w[2] * z;
    } else if constexpr (l == 3) {
        constexpr double k9 = 0.25 * cgmath::csqrt(35.0 / (2.0 * kPi));   // y(3x^2-y^2), x(x^2-3y^2)
        constexpr double k10 = 0.5 * cgmath::csqrt(105.0 / kPi);          // xyz
        constexpr double k11 = 0.25 * cgmath::csqrt(21.0 / (2.0 * kPi));  // y(5z^2-1), x(5z^2-1)
        constexpr double k12 = 0.25 * cgmath::csqrt(7.0 / kPi);           // 5z^3-3z
        constexpr double k14 = 0.25 * cgmath::csqrt(105.0 / kPi);         // z(x^2-y^2)
        const double xx = x * x, yy = y * y, zz = z * z;
        const double t = 5.0 * zz - 1.0;
        qx += k9 * (6.0 * x * y * w[0] + 3.0 * (xx - yy) * w[6]) + k10 * y * z * w[1] + k11 * t * w[4] +
              k14 * 2.0 * x * z * w[5];
        qy += k9 * (3.0 * (xx - yy) * w[0] - 6.0 * x * y * w[6]) + k10 * x * z * w[1] + k11 * t * w[2] -
              k14 * 2.0 * y * z * w[5];
        qz += k10 * x * y * w[1] + k11 * 10.0 * z * (y * w[2] + x * w[4]) + k12 * (15.0 * zz - 3.0) * w[3] +
              k14 * (xx - yy) * w[5];
    }
}

// unit vector and 1/|r| of an edge vector (rsqrt: the hardware estimate and
// one refinement, a third of the instructions of a square root and a division)
__device__ __forceinline__ void unit(double rx, double ry, double rz, double& x, double& y, double& z, double& inv)
{
    inv = rsqrt(rx * rx + ry * ry + rz * rz);
    x = rx * inv;
    y = ry * inv;
    z = rz * inv;
}

// grad_r = (q - u (u.q)) / |r| from the unit-vector gradient q
__device__ __forceinline__ void tangent(double x, double y, double z, double inv, double qx, double qy, double qz,
                                        double (&g)[3])
{
    const double uq = x * qx + y * qy + z * qz;
    g[0] = (qx - x * uq) * inv;
    g[1] = (qy - y * uq) * inv;
    g[2] = (qz - z * uq) * inv;
}

}  // namespace shf
}  // namespace cgtp
