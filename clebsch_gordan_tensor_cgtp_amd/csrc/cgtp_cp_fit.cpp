// cgtp_cp_fit.cpp -- the data-free fit of the CP factors ("Tensor
// Decomposition Networks ...", rebuttal to S6y1, reply on Figure 3: the factors
// are fitted once, before any training, by minimising the Frobenius norm
// between the exact and the approximate product over standard-normal inputs).
//
// For independent standard-normal x and y the expected squared error of the
// two products equals the squared Frobenius norm of M - [[A, B, C]], so the
// fit is a CP fit of the coupling tensor M itself; alternating least squares
// solves it one factor at a time, each step exactly.  Host code, run once when
// a model is set up; the convolution itself runs in the kernels.
#include <math.h>
#include <string.h>

#include <vector>

#include "cgtp_cp.h"

namespace cgtp {
namespace {

// In place: V (n x n, symmetric positive definite) = L L^T, lower triangle.
bool cholesky(std::vector<double>& V, int n)
{
    for (int j = 0; j < n; ++j) {
        double d = V[(size_t)j * n + j];
        for (int k = 0; k < j; ++k) d -= V[(size_t)j * n + k] * V[(size_t)j * n + k];
        if (!(d > 0.0)) return false;
        const double l = sqrt(d);
        V[(size_t)j * n + j] = l;
        for (int i = j + 1; i < n; ++i) {
            double s = V[(size_t)i * n + j];
            for (int k = 0; k < j; ++k) s -= V[(size_t)i * n + k] * V[(size_t)j * n + k];
            V[(size_t)i * n + j] = s / l;
        }
    }
    return true;
}

// rows of X (m x n) replaced by the solutions z of z (L L^T) = x
void solve_rows(const std::vector<double>& Lf, int n, double* X, int m)
{
    std::vector<double> z((size_t)n);
    for (int row = 0; row < m; ++row) {
        double* x = X + (size_t)row * n;
        // L y = x
        for (int i = 0; i < n; ++i) {
            double s = x[i];
            for (int k = 0; k < i; ++k) s -= Lf[(size_t)i * n + k] * z[k];
            z[i] = s / Lf[(size_t)i * n + i];
        }
        // L^T w = y
        for (int i = n - 1; i >= 0; --i) {
            double s = z[i];
            for (int k = i + 1; k < n; ++k) s -= Lf[(size_t)k * n + i] * x[k];
            x[i] = s / Lf[(size_t)i * n + i];
        }
    }
}

// G = F^T F for F (rows x R)
void gram(const double* F, int rows, int R, double* G)
{
    for (int a = 0; a < R; ++a)
        for (int b = 0; b < R; ++b) {
            double s = 0.0;
            for (int k = 0; k < rows; ++k) s += F[(size_t)k * R + a] * F[(size_t)k * R + b];
            G[(size_t)a * R + b] = s;
        }
}

}  // namespace

bool cp_als_fit(const double* M, int d1, int d2, int d3, int R, int sweeps, double ridge, double* A, double* B,
                double* Cf, double* rel_err)
{
    std::vector<double> G1((size_t)R * R), G2((size_t)R * R), V((size_t)R * R);
    std::vector<double> K((size_t)(d1 > d2 ? (d1 > d3 ? d1 : d3) : (d2 > d3 ? d2 : d3)) * R);
    auto at = [&](int a, int b, int c) { return M[((size_t)a * d2 + b) * d3 + c]; };
    // F = K V^-1 with V = G1 (.) G2 (+ ridge), F and K of `rows` rows
    auto update = [&](double* F, int rows) -> bool {
        double tr = 0.0;
        for (int r = 0; r < R; ++r) tr += G1[(size_t)r * R + r] * G2[(size_t)r * R + r];
        for (size_t q = 0; q < V.size(); ++q) V[q] = G1[q] * G2[q];
        for (int r = 0; r < R; ++r) V[(size_t)r * R + r] += ridge * tr / R;
        if (!cholesky(V, R)) return false;
        solve_rows(V, R, K.data(), rows);
        memcpy(F, K.data(), sizeof(double) * (size_t)rows * R);
        return true;
    };
    for (int sweep = 0; sweep < sweeps; ++sweep) {
        // B: K[a][r] = sum_{b,c} M[a][b][c] Cf[b][r] A[c][r]
        for (int a = 0; a < d1; ++a)
            for (int r = 0; r < R; ++r) {
                double s = 0.0;
                for (int b = 0; b < d2; ++b)
                    for (int c = 0; c < d3; ++c) s += at(a, b, c) * Cf[(size_t)b * R + r] * A[(size_t)c * R + r];
                K[(size_t)a * R + r] = s;
            }
        gram(Cf, d2, R, G1.data());
        gram(A, d3, R, G2.data());
        if (!update(B, d1)) return false;
        // Cf: K[b][r] = sum_{a,c} M[a][b][c] B[a][r] A[c][r]
        for (int b = 0; b < d2; ++b)
            for (int r = 0; r < R; ++r) {
                double s = 0.0;
                for (int a = 0; a < d1; ++a)
                    for (int c = 0; c < d3; ++c) s += at(a, b, c) * B[(size_t)a * R + r] * A[(size_t)c * R + r];
                K[(size_t)b * R + r] = s;
            }
        gram(B, d1, R, G1.data());
        gram(A, d3, R, G2.data());
        if (!update(Cf, d2)) return false;
        // A: K[c][r] = sum_{a,b} M[a][b][c] B[a][r] Cf[b][r]
        for (int c = 0; c < d3; ++c)
            for (int r = 0; r < R; ++r) {
                double s = 0.0;
                for (int a = 0; a < d1; ++a)
                    for (int b = 0; b < d2; ++b) s += at(a, b, c) * B[(size_t)a * R + r] * Cf[(size_t)b * R + r];
                K[(size_t)c * R + r] = s;
            }
        gram(B, d1, R, G1.data());
        gram(Cf, d2, R, G2.data());
        if (!update(A, d3)) return false;
    }
    if (rel_err) {
        double num = 0.0, den = 0.0;
        for (int a = 0; a < d1; ++a)
            for (int b = 0; b < d2; ++b)
                for (int c = 0; c < d3; ++c) {
                    double v = 0.0;
                    for (int r = 0; r < R; ++r)
                        v += B[(size_t)a * R + r] * Cf[(size_t)b * R + r] * A[(size_t)c * R + r];
                    const double m = at(a, b, c);
                    num += (m - v) * (m - v);
                    den += m * m;
                }
        *rel_err = den > 0.0 ? sqrt(num / den) : sqrt(num);
    }
    return true;
}

}  // namespace cgtp
