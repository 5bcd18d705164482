// Host-side rotation from prefill vectors ("MosaicKV 阅读笔记" reading notes,
// Eq. 4 and 6-8; paper summary section 2.3): R = V^T with X^T X = V S^2 V^T.
//
// G = X^T X is accumulated in float64 (partial Gram matrices over fixed token
// ranges, added in a fixed order), reduced to tridiagonal form by Householder reflections and
// diagonalised by the implicit symmetric QR iteration with Wilkinson shifts
// (Golub and Van Loan, "Matrix Computations", sections 8.3.1 and 8.3.3).
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "../../include/mkv.h"
#include "host_la.h"

namespace mkv {

double host_elem(const void *x, int32_t dtype, int64_t i) {
    if (dtype == MKV_F32) return (double)static_cast<const float *>(x)[i];
    uint32_t u = (uint32_t) static_cast<const uint16_t *>(x)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

}  // namespace mkv

namespace {

using mkv::host_elem;

// Upper triangle of X^T X, X given row-major [T][d] in the storage dtype.
// The tokens are cut into GRAM_PARTS contiguous ranges of whole 64-token
// chunks; each range sums its chunks in order into its own partial, and the
// partials are added in range order. Neither depends on the thread count, so
// G (and R) is bitwise the same on every host.
constexpr int GRAM_PARTS = 64;

void gram(const void *x, int32_t dtype, int64_t T, int d, std::vector<double> &G) {
    const int64_t chunk = 64;
    const int64_t nchunk = (T + chunk - 1) / chunk;
    std::vector<std::vector<double>> partial(GRAM_PARTS);
    const int nthr = std::max(1, std::min(omp_get_max_threads(), GRAM_PARTS));
#pragma omp parallel num_threads(nthr)
    {
        std::vector<double> xt((size_t)d * chunk);  // chunk transposed: [d][chunk]
#pragma omp for schedule(dynamic)
        for (int p = 0; p < GRAM_PARTS; ++p) {
            const int64_t c0 = nchunk * p / GRAM_PARTS, c1 = nchunk * (p + 1) / GRAM_PARTS;
            if (c0 >= c1) continue;
            std::vector<double> &acc = partial[p];
            acc.assign((size_t)d * d, 0.0);
            for (int64_t ci = c0; ci < c1; ++ci) {
                const int64_t t0 = ci * chunk;
                const int64_t n = std::min<int64_t>(chunk, T - t0);
                for (int64_t t = 0; t < n; ++t)
                    for (int c = 0; c < d; ++c) xt[(size_t)c * chunk + t] = host_elem(x, dtype, (t0 + t) * d + c);
                for (int i = 0; i < d; ++i) {
                    const double *xi = &xt[(size_t)i * chunk];
                    for (int j = i; j < d; ++j) {
                        const double *xj = &xt[(size_t)j * chunk];
                        double s = 0.0;
                        for (int64_t t = 0; t < n; ++t) s += xi[t] * xj[t];
                        acc[(size_t)i * d + j] += s;
                    }
                }
            }
        }
    }
    G.assign((size_t)d * d, 0.0);
    for (int p = 0; p < GRAM_PARTS; ++p)
        if (!partial[p].empty())
            for (size_t k = 0; k < G.size(); ++k) G[k] += partial[p][k];
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < i; ++j) G[(size_t)i * d + j] = G[(size_t)j * d + i];
}

// A (n x n symmetric, row-major) -> Q T Q^T with T tridiagonal (diag a, off b).
void tridiagonalize(int n, std::vector<double> &A, std::vector<double> &a, std::vector<double> &b,
                    std::vector<double> &Q) {
    Q.assign((size_t)n * n, 0.0);
    for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
    std::vector<double> v(n), u(n), w(n);
    for (int k = 0; k + 2 < n; ++k) {
        double nrm = 0.0;
        for (int i = k + 1; i < n; ++i) nrm += A[(size_t)i * n + k] * A[(size_t)i * n + k];
        nrm = sqrt(nrm);
        if (nrm == 0.0) continue;
        const double x0 = A[(size_t)(k + 1) * n + k];
        const double alpha = x0 > 0 ? -nrm : nrm;  // reflect onto -sign(x0) |x| e1
        std::fill(v.begin(), v.end(), 0.0);
        for (int i = k + 1; i < n; ++i) v[i] = A[(size_t)i * n + k];
        v[k + 1] -= alpha;
        double vv = 0.0;
        for (int i = k + 1; i < n; ++i) vv += v[i] * v[i];
        if (vv == 0.0) continue;
        const double beta = 2.0 / vv;
        // u = beta A v ; K = beta/2 v^T u ; w = u - K v ; A <- A - v w^T - w v^T
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int j = k + 1; j < n; ++j) s += A[(size_t)i * n + j] * v[j];
            u[i] = beta * s;
        }
        double K = 0.0;
        for (int i = k + 1; i < n; ++i) K += v[i] * u[i];
        K *= beta / 2.0;
        for (int i = 0; i < n; ++i) w[i] = u[i] - K * v[i];
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) A[(size_t)i * n + j] -= v[i] * w[j] + w[i] * v[j];
        // Q <- Q H, H = I - beta v v^T
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int j = k + 1; j < n; ++j) s += Q[(size_t)i * n + j] * v[j];
            s *= beta;
            for (int j = k + 1; j < n; ++j) Q[(size_t)i * n + j] -= s * v[j];
        }
    }
    a.resize(n);
    b.assign(n > 1 ? n - 1 : 0, 0.0);
    for (int i = 0; i < n; ++i) a[i] = A[(size_t)i * n + i];
    for (int i = 0; i + 1 < n; ++i) b[i] = A[(size_t)(i + 1) * n + i];
}

// Implicit symmetric QR with Wilkinson shift on (a, b); rotations accumulate
// into the columns of Z. Returns false if it fails to converge.
bool tridiag_qr(int n, std::vector<double> &a, std::vector<double> &b, std::vector<double> &Z) {
    const double eps = 2.220446049250313e-16;
    int iters = 0;
    int hi = n - 1;
    while (hi > 0) {
        // deflate negligible off-diagonal entries
        for (int i = 0; i < hi; ++i)
            if (fabs(b[i]) <= eps * (fabs(a[i]) + fabs(a[i + 1]))) b[i] = 0.0;
        while (hi > 0 && b[hi - 1] == 0.0) --hi;
        if (hi == 0) break;
        int lo = hi - 1;
        while (lo > 0 && b[lo - 1] != 0.0) --lo;
        if (++iters > 60 * n) return false;
        // Wilkinson shift from the trailing 2x2 of the unreduced block
        const double dd = 0.5 * (a[hi - 1] - a[hi]);
        const double bb = b[hi - 1];
        const double den = dd + (dd >= 0 ? 1.0 : -1.0) * hypot(dd, bb);
        const double mu = den != 0.0 ? a[hi] - bb * bb / den : a[hi] - fabs(bb);
        double x = a[lo] - mu, z = b[lo];
        for (int k = lo; k < hi; ++k) {
            const double rr = hypot(x, z);
            const double c = rr == 0.0 ? 1.0 : x / rr;
            const double s = rr == 0.0 ? 0.0 : z / rr;
            if (k > lo) b[k - 1] = rr;  // the bulge folds into the off-diagonal
            const double ak = a[k], ak1 = a[k + 1], bk = b[k];
            a[k] = c * c * ak + 2.0 * c * s * bk + s * s * ak1;
            a[k + 1] = s * s * ak - 2.0 * c * s * bk + c * c * ak1;
            b[k] = c * s * (ak1 - ak) + (c * c - s * s) * bk;
            if (k + 1 < hi) {
                x = b[k];
                z = s * b[k + 1];
                b[k + 1] = c * b[k + 1];
            }
            for (int i = 0; i < n; ++i) {
                const double zk = Z[(size_t)i * n + k], zk1 = Z[(size_t)i * n + k + 1];
                Z[(size_t)i * n + k] = c * zk + s * zk1;
                Z[(size_t)i * n + k + 1] = -s * zk + c * zk1;
            }
        }
    }
    return true;
}

}  // namespace

mkv_status mkv::rotation_from_gram(std::vector<double> &G, int d, float *R_out, double *sigma_out) {
    std::vector<double> a, b, Q;
    tridiagonalize(d, G, a, b, Q);
    if (!tridiag_qr(d, a, b, Q)) return MKV_ERR_NOCONVERGE;
    std::vector<int> order(d);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int i, int j) { return a[i] > a[j]; });
    for (int c = 0; c < d; ++c) {
        const int col = order[c];
        int best = 0;
        for (int j = 1; j < d; ++j)
            if (fabs(Q[(size_t)j * d + col]) > fabs(Q[(size_t)best * d + col])) best = j;
        const double sg = Q[(size_t)best * d + col] < 0.0 ? -1.0 : 1.0;
        for (int j = 0; j < d; ++j) R_out[(size_t)c * d + j] = (float)(sg * Q[(size_t)j * d + col]);
        if (sigma_out) sigma_out[c] = sqrt(a[col] > 0.0 ? a[col] : 0.0);
    }
    return MKV_OK;
}

extern "C" mkv_status mkv_rotation_from_prefill(const void *x_host, int32_t dtype, int64_t T, int32_t d,
                                                float *R_out, double *sigma_out) {
    if (!R_out || d < 1 || d > 256 || T < 0 || (T > 0 && !x_host)) return MKV_ERR_ARG;
    if (dtype != MKV_F32 && dtype != MKV_BF16) return MKV_ERR_ARG;
    std::vector<double> G;
    if (T > 0) {
        gram(x_host, dtype, T, d, G);
    } else {
        G.assign((size_t)d * d, 0.0);
    }
    return mkv::rotation_from_gram(G, d, R_out, sigma_out);
}
