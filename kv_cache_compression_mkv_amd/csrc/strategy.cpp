// Segment strategy generation (paper summary "MosaicKV: Serving Long-Context
// LLM with Dynamic Two-D KV Cache Compression", sections 4.3 and 5.5): where
// a request's token stream is cut into segments, and each finished segment's
// rotation and kept-channel count.
//
// Loss of a set of tokens under a strategy (R, r): the energy of their rotated
// vectors x' = R x outside each vector's own r largest magnitudes (what the
// per-vector top-r of the reading notes' Eq. 9 and Algorithm 1 drops), over
// their total rotated energy, summed over the request's KV heads and over keys
// and values. A segment ends at a 16-token block boundary once it holds
// min_len tokens and its loss under the strategy in force exceeds cut_loss,
// or when it holds max_len tokens. A finished segment's rotations come from
// the Gram matrices accumulated while its tokens were scanned (the paper's
// incremental covariance; eigenvectors as at prefill, reading notes Eq. 4,
// 6, 7), and its r is the smallest in [r_min, r_max] whose loss under them is
// at most keep_loss; that strategy is in force for the next segment (the
// paper's section 5.4 compresses the current segment with the previous
// strategy until it is finished).
//
// Work is split over (matrix, KV head) units, each summed in token order on
// one thread; units are combined in a fixed order (keys of every head, then
// values), so results do not depend on the thread count.
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <vector>

#include "../../include/mkv.h"
#include "host_la.h"

namespace {

constexpr int64_t BLOCK = 16;

struct Stream {
    const void *k, *v;
    int32_t dtype;
    int d, H;
    int64_t stride;
    // unit u: keys of head u for u < H, values of head u - H after
    const void *base(int u) const { return u < H ? k : v; }
    int64_t row(int u, int64_t t) const { return ((int64_t)(u % H) * stride + t) * d; }
};

// rotation of unit u inside a [H][2][d][d] table
const float *unit_rot(const float *rot, int u, int H, int d) {
    return rot + ((size_t)(u % H) * 2 + (u < H ? 0 : 1)) * d * d;
}

// token t of unit u rotated by R: x (input, binary64), e (squared rotated elements); returns their sum
double rotated_energy(const Stream &S, int u, int64_t t, const float *R, double *x, double *e) {
    const int d = S.d;
    const void *b = S.base(u);
    const int64_t r0 = S.row(u, t);
    for (int c = 0; c < d; ++c) x[c] = mkv::host_elem(b, S.dtype, r0 + c);
    double tot = 0.0;
    for (int c = 0; c < d; ++c) {
        double s = 0.0;
        for (int j = 0; j < d; ++j) s += (double)R[(size_t)c * d + j] * x[j];
        e[c] = s * s;
        tot += e[c];
    }
    return tot;
}

// L(r) for r = 0 .. d of tokens [t0, t1) under rotations rot [H][2][d][d]
void loss_curve(const Stream &S, int64_t t0, int64_t t1, const float *rot, double *loss) {
    const int d = S.d, U = 2 * S.H;
    std::vector<std::vector<double>> col(U, std::vector<double>(d, 0.0));
#pragma omp parallel num_threads(std::max(1, std::min(U, omp_get_max_threads())))
    {
        std::vector<double> x(d), e(d);
#pragma omp for schedule(static)
        for (int u = 0; u < U; ++u) {
            const float *R = unit_rot(rot, u, S.H, d);
            for (int64_t t = t0; t < t1; ++t) {
                rotated_energy(S, u, t, R, x.data(), e.data());
                std::sort(e.begin(), e.end(), std::greater<double>());
                for (int i = 0; i < d; ++i) col[u][i] += e[i];
            }
        }
    }
    std::vector<double> dropped(d + 1, 0.0);
    double total = 0.0;
    for (int u = 0; u < U; ++u) {
        double tail = 0.0;
        for (int i = d - 1; i >= 0; --i) {
            tail += col[u][i];
            dropped[i] += tail;
        }
        for (int i = 0; i < d; ++i) total += col[u][i];
    }
    for (int r = 0; r <= d; ++r) loss[r] = total > 0.0 ? dropped[r] / total : 0.0;
}

bool stream_ok(const void *k, const void *v, int32_t dtype, int32_t d, int32_t H, int64_t n, int64_t stride) {
    if (d < 1 || d > 256 || H < 1 || n < 0 || stride < n) return false;
    if (dtype != MKV_F32 && dtype != MKV_BF16) return false;
    return n == 0 || (k && v);
}

}  // namespace

extern "C" mkv_status mkv_strategy_loss_curve(const void *k_host, const void *v_host, int32_t dtype, int32_t d,
                                              int32_t n_kv_heads, int64_t n_tokens, int64_t row_stride,
                                              const float *rot, double *loss_out) {
    if (!stream_ok(k_host, v_host, dtype, d, n_kv_heads, n_tokens, row_stride) || !rot || !loss_out)
        return MKV_ERR_ARG;
    const Stream S{k_host, v_host, dtype, d, n_kv_heads, row_stride};
    loss_curve(S, 0, n_tokens, rot, loss_out);
    return MKV_OK;
}

extern "C" mkv_status mkv_strategy_segments(const void *k_host, const void *v_host, int32_t dtype, int32_t d,
                                           int32_t n_kv_heads, int64_t n_tokens, int64_t row_stride,
                                           const float *rot0, int32_t r0, double cut_loss, double keep_loss,
                                           int32_t r_min, int32_t r_max, int64_t min_len, int64_t max_len,
                                           int64_t seg_cap, int64_t *seg_end, int32_t *seg_r, float *seg_rot,
                                           int64_t *n_seg) {
    if (!stream_ok(k_host, v_host, dtype, d, n_kv_heads, n_tokens, row_stride) || !rot0 || !seg_end ||
        !seg_r || !n_seg || seg_cap < 1)
        return MKV_ERR_ARG;
    if (r0 < 0 || r0 > d || r_min < 0 || r_min > r_max || r_max > d || min_len < 0 || max_len < BLOCK ||
        max_len % BLOCK || isnan(cut_loss) || isnan(keep_loss))
        return MKV_ERR_ARG;
    const int H = n_kv_heads, U = 2 * H;
    const size_t dd = (size_t)d * d;
    const Stream S{k_host, v_host, dtype, d, H, row_stride};
    std::vector<float> cur(rot0, rot0 + (size_t)H * 2 * dd), next((size_t)H * 2 * dd);
    int r = r0;
    int64_t start = 0, ns = 0;
    *n_seg = 0;
    std::vector<std::vector<double>> G(U);
    std::vector<double> part_dropped(U), part_total(U);
    const int nthr = std::max(1, std::min(U, omp_get_max_threads()));
    while (start < n_tokens) {
        for (int u = 0; u < U; ++u) G[u].assign(dd, 0.0);
        double num = 0.0, den = 0.0;
        int64_t pos = start, end = n_tokens;
        while (pos < n_tokens) {
            const int64_t stop = std::min(pos + BLOCK, n_tokens);
#pragma omp parallel num_threads(nthr)
            {
                std::vector<double> x(d), e(d);
#pragma omp for schedule(static)
                for (int u = 0; u < U; ++u) {
                    const float *R = unit_rot(cur.data(), u, H, d);
                    double dr = 0.0, tt = 0.0;
                    std::vector<double> &g = G[u];
                    for (int64_t t = pos; t < stop; ++t) {
                        tt += rotated_energy(S, u, t, R, x.data(), e.data());
                        // energy outside the r largest: the d - r smallest elements
                        std::nth_element(e.begin(), e.begin() + r, e.end(), std::greater<double>());
                        for (int i = r; i < d; ++i) dr += e[i];
                        for (int i = 0; i < d; ++i) {  // Gram matrix, upper triangle
                            const double xi = x[i];
                            double *gi = &g[(size_t)i * d];
                            for (int j = i; j < d; ++j) gi[j] += xi * x[j];
                        }
                    }
                    part_dropped[u] = dr;
                    part_total[u] = tt;
                }
            }
            for (int u = 0; u < U; ++u) {
                num += part_dropped[u];
                den += part_total[u];
            }
            pos = stop;
            const int64_t len = pos - start;
            if (len >= max_len || (len >= min_len && num > cut_loss * den)) {
                end = pos;
                break;
            }
        }
        // the finished segment's own rotations and r
        mkv_status st = MKV_OK;
#pragma omp parallel for num_threads(nthr) schedule(static)
        for (int u = 0; u < U; ++u) {
            std::vector<double> &g = G[u];
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < i; ++j) g[(size_t)i * d + j] = g[(size_t)j * d + i];
            float *R = next.data() + ((size_t)(u % H) * 2 + (u < H ? 0 : 1)) * dd;
            if (mkv::rotation_from_gram(g, d, R, nullptr) != MKV_OK) {
#pragma omp critical
                st = MKV_ERR_NOCONVERGE;
            }
        }
        if (st != MKV_OK) return st;
        std::vector<double> L(d + 1);
        loss_curve(S, start, end, next.data(), L.data());
        int rs = r_max;
        for (int q = r_min; q <= r_max; ++q)
            if (L[q] <= keep_loss) {
                rs = q;
                break;
            }
        if (ns == seg_cap) {
            *n_seg = ns;
            return MKV_ERR_CAPACITY;
        }
        seg_end[ns] = end;
        seg_r[ns] = rs;
        if (seg_rot) memcpy(seg_rot + (size_t)ns * H * 2 * dd, next.data(), sizeof(float) * H * 2 * dd);
        ++ns;
        cur.swap(next);
        r = rs;
        start = end;
    }
    *n_seg = ns;
    return MKV_OK;
}
