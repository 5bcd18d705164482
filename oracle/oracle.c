/* oracle.c -- plain, slow, fp64 CPU oracle of MosaicKV's decode hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; it is used by the tests, by the smoke check and by the benchmark's
 * CPU-baseline leg. It shares no code with the HIP library.
 *
 * Sources (the pages this follows; see each function):
 *   [N] "MosaicKV 阅读笔记" (reading notes on MosaicKV, zhongzhuzhou.org):
 *       Eq. 1 (attention), Eq. 4/6/7/8 (SVD rotation), Eq. 5 (energy),
 *       Eq. 9 and Algorithm 1 (per-vector top-r), Eq. 12-14 (block score,
 *       compressed attention, inverse rotation), the Quest paragraph of the
 *       sequence-compression background (per-block min/max keys), the d=4
 *       example of the SVD background section.
 *   [S] paperlayer.ai summary of arXiv 2607.00760 ("MosaicKV: Serving
 *       Long-Context LLM with Dynamic Two-D KV Cache Compression"):
 *       section 4.2 (two-stage compression: top-r elements, then top-k token
 *       blocks by query-to-block-key scores), 5.2 (per-block keys), 5.3
 *       (PackedAttention; inverse rotation merged into the query), 5.4
 *       (heterogeneous double compression buffering: a finished segment is
 *       recompressed on the CPU with its own SVD rotation and swapped in),
 *       6.3 (Quest per-block keys at block size 16).
 *   [N] also describes the double buffering (its heterogeneous double
 *       buffering section and Fig. 4): the swapped-in segment is packed with
 *       a per-segment rotation.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - rotation arithmetic: x'_c = sum_j R[c][j] x_j in fp64, j ascending;
 *   - storage rounding: one direct round-to-nearest-even from fp64;
 *   - top-r ranks unrounded |x'|, ties to the lower channel, stored ascending;
 *   - per-block min/max over the sparse-reconstructed stored keys (0 at dropped
 *     channels), min/max taken in IEEE totalOrder (-0 < +0);
 *   - block score (1/sqrt(d)) sum_c max(q'_c mx_c, q'_c mn_c), over the
 *     leading key_ch rotated channels of a segment whose block keys are
 *     channel-compressed ([S] 5.2 channel-compresses the per-block keys; the
 *     rotation orders channels by descending singular value, so the leading
 *     ones carry the most energy), over all d channels otherwise;
 *   - k = ceil(keep_ppm * n / 1e6) in integers (or k_abs), clamped to [1, n];
 *   - top-k per query head and per packed segment, ties to the lower block;
 *   - dense segments are always attended.
 *
 * Parity unpinned: no value printed on the pages fixes these conventions, so
 * only the agreement of this oracle with the GPU path checks them -- block
 * keys taken from the stored sparse keys, the ascending stored order of kept
 * channels, the integer ceil of the keep ratio, top-k per packed segment with
 * dense segments always attended, per-query-head selection read once per KV
 * group, rotated dense storage, partial tail blocks, the serving layout with
 * one packed segment after the sink, totalOrder on signed zeros, block keys
 * of decode-time appends, and the input generator.
 *
 * All floating point is IEEE binary64; built with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };
enum { ORC_DENSE = 0, ORC_PACKED = 1 };

/* ------------------------------------------------------------------------- */
/* Rounding to the storage type                                               */
/* ------------------------------------------------------------------------- */

/* Round a binary64 value to the nearest value of a binary format with 8
 * exponent bits (bias 127) and `mbits` stored mantissa bits (23: binary32,
 * 7: bfloat16), ties to even, in one step from the exact binary64 value
 * (IEEE 754 roundTiesToEven). Returns the target bit pattern. */
uint32_t orc_round_e8(double x, int mbits) {
    uint64_t b;
    memcpy(&b, &x, 8);
    const uint32_t sign_bit = (uint32_t)(b >> 63) << (8 + mbits);
    const int e = (int)((b >> 52) & 0x7ff);
    const uint64_t m = b & 0xFFFFFFFFFFFFFull;
    const uint32_t inf = 0xFFu << mbits;
    if (e == 0x7ff) return sign_bit | inf | (m ? (1u << (mbits - 1)) : 0u); /* inf / quiet nan */
    if (e == 0) return sign_bit; /* zero or binary64 subnormal: far below the target's range */
    const int E = e - 1023;               /* value = sig * 2^(E-52), sig in [2^52, 2^53) */
    const uint64_t sig = m | (1ull << 52);
    const int q = (E >= -126) ? E - mbits : -126 - mbits; /* exponent of the target ulp */
    const int shift = q - (E - 52);
    if (shift >= 64) return sign_bit;
    uint64_t kept = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (kept & 1))) kept++;
    uint64_t mag;
    if (E >= -126)
        mag = ((uint64_t)(E + 126) << mbits) + kept; /* kept includes the hidden bit */
    else
        mag = kept; /* subnormal; a carry lands on the smallest normal */
    if (mag >= inf) mag = inf;
    return sign_bit | (uint32_t)mag;
}

double orc_decode_e8(uint32_t bits, int mbits) {
    const int neg = (bits >> (8 + mbits)) & 1;
    const int ex = (int)((bits >> mbits) & 0xFF);
    const uint32_t man = bits & ((1u << mbits) - 1);
    double v;
    if (ex == 0xFF) v = man ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)man, -126 - mbits);
    else v = ldexp((double)(man | (1u << mbits)), ex - 127 - mbits);
    return neg ? -v : v;
}

static double store_value(double x, int dtype) {
    if (dtype == ORC_F64) return x;
    const int mb = dtype == ORC_F32 ? 23 : 7;
    return orc_decode_e8(orc_round_e8(x, mb), mb);
}

void orc_round_array(const double *x, int64_t n, int dtype, double *out, uint32_t *bits) {
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == ORC_F64) {
            out[i] = x[i];
            if (bits) bits[i] = 0;
            continue;
        }
        const int mb = dtype == ORC_F32 ? 23 : 7;
        uint32_t u = orc_round_e8(x[i], mb);
        out[i] = orc_decode_e8(u, mb);
        if (bits) bits[i] = u;
    }
}

/* IEEE totalOrder key for finite values: -0 sorts below +0. */
static uint64_t total_key(double x) {
    uint64_t b;
    memcpy(&b, &x, 8);
    return (b >> 63) ? ~b : (b | (1ull << 63));
}

/* ------------------------------------------------------------------------- */
/* Rotation from prefill keys/values: [N] Eq. 4, 6, 7, 8; [S] section 2.3    */
/* ------------------------------------------------------------------------- */

/* G = X^T X (no centering), eigen-decomposed by cyclic Jacobi (Golub & Van
 * Loan, "Matrix Computations", symmetric Schur rotations). Row c of R is the
 * eigenvector of the c-th largest eigenvalue, sigma_c = sqrt(max(lambda_c, 0)).
 * Sign: the entry of largest magnitude in each row is made positive (ties to
 * the lower index). Returns 0, or 5 if Jacobi did not converge. */
int orc_rotation(const double *X, int64_t T, int d, double *R, double *sigma, int nthreads) {
    double *G = (double *)calloc((size_t)d * d, sizeof(double));
    double *V = (double *)calloc((size_t)d * d, sizeof(double));
    int *order = (int *)malloc(sizeof(int) * d);
    if (!G || !V || !order) {
        free(G); free(V); free(order);
        return 1;
    }
#pragma omp parallel for schedule(dynamic) num_threads(nthreads)
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            double s = 0.0;
            for (int64_t t = 0; t < T; ++t) s += X[t * d + i] * X[t * d + j];
            G[i * d + j] = s;
        }
    for (int i = 0; i < d; ++i) V[i * d + i] = 1.0;

    double fro = 0.0;
    for (int i = 0; i < d * d; ++i) fro += G[i] * G[i];
    fro = sqrt(fro);
    int converged = 0;
    for (int sweep = 0; sweep < 100 && !converged; ++sweep) {
        double off = 0.0;
        for (int p = 0; p < d; ++p)
            for (int q = 0; q < d; ++q)
                if (p != q) off += G[p * d + q] * G[p * d + q];
        if (sqrt(off) <= 1e-15 * fro || fro == 0.0) {
            converged = 1;
            break;
        }
        for (int p = 0; p < d - 1; ++p)
            for (int q = p + 1; q < d; ++q) {
                const double apq = G[p * d + q];
                if (apq == 0.0) continue;
                const double tau = (G[q * d + q] - G[p * d + p]) / (2.0 * apq);
                const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
                const double c = 1.0 / sqrt(1.0 + t * t);
                const double s = t * c;
                for (int k = 0; k < d; ++k) { /* G <- G J */
                    const double gkp = G[k * d + p], gkq = G[k * d + q];
                    G[k * d + p] = c * gkp - s * gkq;
                    G[k * d + q] = s * gkp + c * gkq;
                }
                for (int k = 0; k < d; ++k) { /* G <- J^T G */
                    const double gpk = G[p * d + k], gqk = G[q * d + k];
                    G[p * d + k] = c * gpk - s * gqk;
                    G[q * d + k] = s * gpk + c * gqk;
                }
                for (int k = 0; k < d; ++k) { /* V <- V J */
                    const double vkp = V[k * d + p], vkq = V[k * d + q];
                    V[k * d + p] = c * vkp - s * vkq;
                    V[k * d + q] = s * vkp + c * vkq;
                }
            }
    }
    if (!converged) {
        free(G); free(V); free(order);
        return 5;
    }
    /* order eigenvalues descending (stable: equal values keep index order) */
    for (int i = 0; i < d; ++i) order[i] = i;
    for (int i = 1; i < d; ++i)
        for (int j = i; j > 0 && G[order[j] * d + order[j]] > G[order[j - 1] * d + order[j - 1]]; --j) {
            int tmp = order[j];
            order[j] = order[j - 1];
            order[j - 1] = tmp;
        }
    for (int c = 0; c < d; ++c) {
        const int col = order[c];
        const double lam = G[col * d + col];
        if (sigma) sigma[c] = sqrt(lam > 0.0 ? lam : 0.0);
        int best = 0;
        for (int j = 1; j < d; ++j)
            if (fabs(V[j * d + col]) > fabs(V[best * d + col])) best = j;
        const double sg = V[best * d + col] < 0.0 ? -1.0 : 1.0;
        for (int j = 0; j < d; ++j) R[c * d + j] = sg * V[j * d + col];
    }
    free(G); free(V); free(order);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Compression of one (request, KV head) unit                                 */
/* ------------------------------------------------------------------------- */

/* [N] Eq. 7 / 8: x' = x R^T, i.e. x'_c = sum_j R[c][j] x_j (j ascending). */
static void rotate(const double *R, const double *x, int d, double *xr) {
    for (int c = 0; c < d; ++c) {
        double s = 0.0;
        for (int j = 0; j < d; ++j) s += R[c * d + j] * x[j];
        xr[c] = s;
    }
}

typedef struct {
    double mag;
    int c;
} ranked;

static int by_magnitude(const void *a, const void *b) {
    const ranked *x = (const ranked *)a, *y = (const ranked *)b;
    if (x->mag > y->mag) return -1;
    if (x->mag < y->mag) return 1;
    return x->c - y->c;
}

static int ascending_int(const void *a, const void *b) { return *(const int *)a - *(const int *)b; }

/* [N] Eq. 9 / Algorithm 1: I = argtopk(|x'|, r); kept channels returned in
 * ascending channel order. */
void orc_topr(const double *xr, int d, int r, int *idx) {
    ranked tmp[256];
    for (int c = 0; c < d; ++c) {
        tmp[c].mag = fabs(xr[c]);
        tmp[c].c = c;
    }
    qsort(tmp, (size_t)d, sizeof(ranked), by_magnitude);
    for (int m = 0; m < r; ++m) idx[m] = tmp[m].c;
    qsort(idx, (size_t)r, sizeof(int), ascending_int);
}

/* [S] 5.1 (and 4.3's element-group size): a position bitmap with one bit per
 * group of g adjacent channels keeps whole groups. Reading taken: the r / g
 * groups i (channels g i .. g i + g - 1) of largest energy
 *   e_i = sum_{m < g} x'^2_{g i + m}
 * (binary64, each square and each sum rounded, m ascending), ties to the
 * lower group -- the choice that drops the least energy; kept channels
 * returned in ascending order. g divides d and r. */
void orc_topr_groups(const double *xr, int d, int r, int g, int *idx) {
    ranked tmp[256];
    const int ng = d / g;
    for (int i = 0; i < ng; ++i) {
        double e = 0.0;
        for (int m = 0; m < g; ++m) {
            const double v = xr[g * i + m];
            e += v * v;
        }
        tmp[i].mag = e;
        tmp[i].c = i;
    }
    qsort(tmp, (size_t)ng, sizeof(ranked), by_magnitude);
    int n = 0;
    for (int k = 0; k < r / g; ++k)
        for (int m = 0; m < g; ++m) idx[n++] = g * tmp[k].c + m;
    qsort(idx, (size_t)n, sizeof(int), ascending_int);
}

static int find_segment(int nseg, const int64_t *t_begin, const int64_t *t_cap, int64_t t) {
    for (int j = 0; j < nseg; ++j)
        if (t >= t_begin[j] && t < t_begin[j] + t_cap[j]) return j;
    return -1;
}

static int64_t seg_filled(int64_t len, int64_t tb, int64_t cap) {
    int64_t f = len - tb;
    if (f < 0) f = 0;
    if (f > cap) f = cap;
    return f;
}

/* Number of blocks of `block` tokens that a segment holding `filled` tokens has. */
static int64_t n_blocks_of(int64_t filled, int block) { return (filled + block - 1) / block; }

/* Compress tokens [t_from, len) of a unit and rebuild the per-block keys of
 * every block holding one of them (tokens before t_from are already stored).
 *   Kraw, Vraw [len][d]: stored raw inputs (as exact doubles)
 *   Rk, Rv [d][d]: the unit's rotation
 *   segR (nullable): per segment, NULL or its own [2][d][d] rotation (R_k then
 *        R_v) that replaces Rk, Rv for the tokens of that segment (the paper's
 *        per-segment SVD of recompressed segments, section 5.4; the reading
 *        notes' heterogeneous double buffering)
 *   group (nullable): per segment, the channels per kept group (0 or 1: single
 *        channels, orc_topr; else orc_topr_groups)
 *   Khat, Vhat [len][d]: stored values, 0 at dropped channels
 *   Kidx, Vidx [len][d]: kept channels ascending, then -1 (dense tokens: 0..d-1)
 *   meta: packed segments one after the other, each [ceil(t_cap/block)][2][d] (mn, mx)
 * Returns 0, or 1 when a token falls outside every segment. */
int orc_compress_unit(int d, int64_t len, int64_t t_from, int dtype, int block,
                      const double *Kraw, const double *Vraw, const double *Rk, const double *Rv,
                      const double *const *segR, int nseg, const int32_t *kind, const int64_t *t_begin,
                      const int64_t *t_cap, const int32_t *r, const int32_t *group, double *Khat, double *Vhat,
                      int16_t *Kidx,
                      int16_t *Vidx, double *meta, int nthreads) {
    if (t_from < 0) t_from = 0;
    for (int64_t t = t_from; t < len; ++t)
        if (find_segment(nseg, t_begin, t_cap, t) < 0) return 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t t = t_from; t < len; ++t) {
        const int j = find_segment(nseg, t_begin, t_cap, t);
        for (int which = 0; which < 2; ++which) {
            const double *x = (which == 0 ? Kraw : Vraw) + t * d;
            const double *R = (segR && segR[j]) ? segR[j] + (int64_t)which * d * d : (which == 0 ? Rk : Rv);
            double *hat = (which == 0 ? Khat : Vhat) + t * d;
            int16_t *ix = (which == 0 ? Kidx : Vidx) + t * d;
            double xr[256];
            int keep[256];
            rotate(R, x, d, xr);
            int nk;
            if (kind[j] == ORC_PACKED) {
                nk = r[j];
                if (group && group[j] > 1) orc_topr_groups(xr, d, nk, group[j], keep);
                else orc_topr(xr, d, nk, keep);
            } else {
                nk = d;
                for (int c = 0; c < d; ++c) keep[c] = c;
            }
            for (int c = 0; c < d; ++c) {
                hat[c] = 0.0;
                ix[c] = -1;
            }
            for (int m = 0; m < nk; ++m) {
                hat[keep[m]] = store_value(xr[keep[m]], dtype);
                ix[m] = (int16_t)keep[m];
            }
        }
    }
    /* per-block keys: [N] Quest background paragraph; [S] 4.2, 5.2, 6.3 */
    int64_t off = 0;
    for (int j = 0; j < nseg; ++j) {
        if (kind[j] != ORC_PACKED) continue;
        const int64_t filled = seg_filled(len, t_begin[j], t_cap[j]);
        const int64_t nb = n_blocks_of(filled, block);
        const int64_t from = t_from > t_begin[j] ? (t_from - t_begin[j]) / block : 0;
        for (int64_t l = from; l < nb; ++l) {
            double *mn = meta + (off + l) * 2 * d, *mx = mn + d;
            const int64_t t0 = t_begin[j] + l * block;
            int64_t t1 = t0 + block;
            if (t1 > t_begin[j] + filled) t1 = t_begin[j] + filled;
            for (int c = 0; c < d; ++c) {
                double lo = Khat[t0 * d + c], hi = lo;
                for (int64_t t = t0 + 1; t < t1; ++t) {
                    const double v = Khat[t * d + c];
                    if (total_key(v) < total_key(lo)) lo = v;
                    if (total_key(v) > total_key(hi)) hi = v;
                }
                mn[c] = lo;
                mx[c] = hi;
            }
        }
        off += n_blocks_of(t_cap[j], block);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Decode attention of the query heads of one unit                            */
/* ------------------------------------------------------------------------- */

/* Blocks kept per packed segment: k_abs if positive (at most n), else
 * ceil(keep_ppm * n / 10^6) in integers, clamped to [1, n]; 0 when n = 0. */
int64_t orc_block_keep(int64_t n, int32_t keep_ppm, int32_t k_abs) {
    if (n <= 0) return 0;
    int64_t k;
    if (k_abs > 0) k = k_abs < n ? k_abs : n;
    else k = ((int64_t)keep_ppm * n + 999999) / 1000000;
    if (k < 1) k = 1;
    if (k > n) k = n;
    return k;
}

typedef struct {
    double s;
    int64_t l;
} scored;

static int by_score(const void *a, const void *b) {
    const scored *x = (const scored *)a, *y = (const scored *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return x->l < y->l ? -1 : (x->l > y->l ? 1 : 0);
}

static int ascending_i32(const void *a, const void *b) {
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

/* For each of the G query heads of a unit:
 *   q' = R_k q                                   ([N] Eq. 12 text; [S] 5.3)
 *   score of block l = (1/sqrt d) sum_{c < m_j} max(q'_c mx_c, q'_c mn_c),
 *     m_j = key_ch[j] channels of packed segment j (d when key_ch is NULL,
 *     or key_ch[j] <= 0 or > d)
 *   top-k blocks per packed segment (ties -> lower block), ascending
 *   z_i = (1/sqrt d) q'[I_i]^T k^_i over dense tokens and selected blocks
 *   o = softmax(z) V^                            ([N] Eq. 13)
 *   out_j = sum_c R_v[c][j] o_c                  ([N] Eq. 14)
 * A segment with its own rotation (segR[j] != NULL, [2][d][d]) stores its
 * tokens in its own rotated space: its scores and logits use q'_j = R_k,j q,
 * and its share of o is rotated back by its own R_v,j. Since the softmax
 * weights are shared and the inverse rotation is linear,
 *   out = sum over segments j of R_v,j^T (sum_{i in j} p_i v^_i).
 * forced_sel (nullable) replaces the top-k by a given selection.
 * Outputs: qrot [G][d], scores [G][nsum], sel [G][ksum], tau [G][npacked]
 * (the k-th largest score; NAN when k = 0), out [G][d]. */
int orc_decode_unit(int d, int64_t len, int G, int block, const double *Khat, const double *Vhat,
                    const int16_t *Kidx, const int16_t *Vidx, const double *meta, const double *const *segR,
                    int nseg,
                    const int32_t *kind, const int64_t *t_begin, const int64_t *t_cap,
                    const int32_t *r, const int32_t *keep_ppm, const int32_t *k_abs, const int32_t *key_ch,
                    const double *q, const double *Rk, const double *Rv, const int32_t *forced_sel, double *qrot,
                    double *scores, int32_t *sel, double *tau, double *out, int nthreads) {
    (void)r;
    int64_t nsum = 0, ksum = 0;
    int npacked = 0;
    for (int j = 0; j < nseg; ++j) {
        if (kind[j] != ORC_PACKED) continue;
        const int64_t nb = n_blocks_of(seg_filled(len, t_begin[j], t_cap[j]), block);
        nsum += nb;
        ksum += orc_block_keep(nb, keep_ppm[j], k_abs[j]);
        npacked++;
    }
    const double scale = 1.0 / sqrt((double)d);
    int status = 0;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads)
    for (int h = 0; h < G; ++h) {
        double *qr = qrot + (int64_t)h * d;
        rotate(Rk, q + (int64_t)h * d, d, qr);
        /* q' in the rotated space of each segment: the unit's, or its own */
        double *qseg = (double *)malloc(sizeof(double) * (size_t)nseg * d);
        if (!qseg) {
            status = 1;
            continue;
        }
        for (int j = 0; j < nseg; ++j) {
            if (segR && segR[j]) rotate(segR[j], q + (int64_t)h * d, d, qseg + (int64_t)j * d);
            else memcpy(qseg + (int64_t)j * d, qr, sizeof(double) * d);
        }
        double *sc = scores + h * nsum;
        int32_t *sh = sel + h * ksum;
        scored *tmp = (scored *)malloc(sizeof(scored) * (size_t)(nsum > 0 ? nsum : 1));
        char *chosen = (char *)calloc((size_t)(nsum > 0 ? nsum : 1), 1);
        if (!tmp || !chosen) {
            status = 1;
            free(tmp); free(chosen); free(qseg);
            continue;
        }
        int64_t noff = 0, koff = 0, moff = 0;
        int pj = 0;
        for (int j = 0; j < nseg; ++j) {
            if (kind[j] != ORC_PACKED) continue;
            const int64_t nb = n_blocks_of(seg_filled(len, t_begin[j], t_cap[j]), block);
            const int64_t k = orc_block_keep(nb, keep_ppm[j], k_abs[j]);
            const double *qj = qseg + (int64_t)j * d;
            const int m = (key_ch && key_ch[j] > 0 && key_ch[j] < d) ? key_ch[j] : d;
            for (int64_t l = 0; l < nb; ++l) {
                const double *mn = meta + (moff + l) * 2 * d, *mx = mn + d;
                double s = 0.0;
                for (int c = 0; c < m; ++c) {
                    const double a = qj[c] * mx[c], b = qj[c] * mn[c];
                    s += a > b ? a : b;
                }
                sc[noff + l] = s * scale;
                tmp[l].s = s * scale;
                tmp[l].l = l;
            }
            qsort(tmp, (size_t)nb, sizeof(scored), by_score);
            tau[h * npacked + pj] = k > 0 ? tmp[k - 1].s : NAN;
            if (forced_sel) {
                for (int64_t i = 0; i < k; ++i) sh[koff + i] = forced_sel[h * ksum + koff + i];
            } else {
                for (int64_t i = 0; i < k; ++i) sh[koff + i] = (int32_t)tmp[i].l;
                qsort(sh + koff, (size_t)k, sizeof(int32_t), ascending_i32);
            }
            for (int64_t i = 0; i < k; ++i) {
                const int32_t l = sh[koff + i];
                if (l >= 0 && l < nb) chosen[noff + l] = 1;
            }
            noff += nb;
            koff += k;
            moff += n_blocks_of(t_cap[j], block);
            pj++;
        }
        /* token set in position order: every filled dense token and every
         * valid token of every selected block */
        double *z = (double *)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
        char *att = (char *)calloc((size_t)(len > 0 ? len : 1), 1);
        if (!z || !att) {
            status = 1;
            free(z); free(att); free(tmp); free(chosen); free(qseg);
            continue;
        }
        noff = 0;
        for (int j = 0; j < nseg; ++j) {
            const int64_t filled = seg_filled(len, t_begin[j], t_cap[j]);
            if (kind[j] == ORC_DENSE) {
                for (int64_t t = t_begin[j]; t < t_begin[j] + filled; ++t) att[t] = 1;
            } else {
                const int64_t nb = n_blocks_of(filled, block);
                for (int64_t l = 0; l < nb; ++l) {
                    if (!chosen[noff + l]) continue;
                    const int64_t t0 = t_begin[j] + l * block;
                    for (int64_t t = t0; t < t0 + block && t < t_begin[j] + filled; ++t) att[t] = 1;
                }
                noff += nb;
            }
        }
        double zmax = -INFINITY;
        for (int64_t t = 0; t < len; ++t) {
            if (!att[t]) continue;
            const double *qj = qseg + (int64_t)find_segment(nseg, t_begin, t_cap, t) * d;
            double s = 0.0;
            const int16_t *ix = Kidx + t * d;
            for (int m = 0; m < d && ix[m] >= 0; ++m) s += qj[ix[m]] * Khat[t * d + ix[m]];
            z[t] = s * scale;
            if (z[t] > zmax) zmax = z[t];
        }
        /* o_j: the weighted sum of segment j's stored values, in its space */
        double *o = (double *)calloc((size_t)nseg * d, sizeof(double));
        if (!o) {
            status = 1;
            free(z); free(att); free(tmp); free(chosen); free(qseg);
            continue;
        }
        double denom = 0.0;
        for (int64_t t = 0; t < len; ++t) {
            if (!att[t]) continue;
            const double w = exp(z[t] - zmax);
            denom += w;
            double *oj = o + (int64_t)find_segment(nseg, t_begin, t_cap, t) * d;
            const int16_t *ix = Vidx + t * d;
            for (int m = 0; m < d && ix[m] >= 0; ++m) oj[ix[m]] += w * Vhat[t * d + ix[m]];
        }
        for (int jj = 0; jj < d; ++jj) out[(int64_t)h * d + jj] = 0.0;
        for (int j = 0; j < nseg; ++j) {
            const double *Rvj = (segR && segR[j]) ? segR[j] + (int64_t)d * d : Rv;
            const double *oj = o + (int64_t)j * d;
            for (int jj = 0; jj < d; ++jj) {
                double s = 0.0;
                for (int c = 0; c < d; ++c) s += Rvj[c * d + jj] * (denom > 0.0 ? oj[c] / denom : 0.0);
                out[(int64_t)h * d + jj] += s;
            }
        }
        free(o); free(z); free(att); free(tmp); free(chosen); free(qseg);
    }
    return status;
}
