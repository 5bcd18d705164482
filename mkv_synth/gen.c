/* Bulk synthetic key/value rows for the MosaicKV decode-path workloads.
 *
 * Input generation only: nothing here belongs to the method (no rotation by
 * the cache's R, no selection, packing, scoring or attention).
 *
 * Random numbers come from SplitMix64 used as a counter-based generator
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014): the i-th output of a stream with seed s is
 * mix64(s + (i + 1) * GAMMA). Each token owns 256 counters, so any token
 * range can be produced independently and in parallel.
 *
 * Per token t: 128 standard normals (Box-Muller on counters 0..127),
 * x = z * M (M = diag(exp(-i/24)) Q^T supplied by the caller), then 4 distinct
 * channels offset by +/-6 (counters 128..135), then the value is rounded to the
 * storage type: float32 by the C conversion, bf16 by nearest-even on the
 * float32 bit pattern.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t seed, uint64_t i) { return mix64(seed + (i + 1) * GAMMA); }

/* uniform in (0, 1] */
static inline double unit(uint64_t r) { return ((double)(r >> 11) + 1.0) * (1.0 / 9007199254740992.0); }

uint64_t mkv_gen_seed(int64_t a, int64_t b, int64_t c, int64_t d) {
    uint64_t s = mix64((uint64_t)a * GAMMA + 1);
    s = mix64(s + (uint64_t)b * GAMMA + 2);
    s = mix64(s + (uint64_t)c * GAMMA + 3);
    s = mix64(s + (uint64_t)d * GAMMA + 4);
    return s;
}

static inline uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u = u + 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* dtype: 0 = float32 rows written to out (float*), 1 = bf16 rows (uint16_t*),
 * 2 = unrounded float64 rows (double*). d <= 256. */
int mkv_gen_kv(uint64_t seed, const double *M, int d, int64_t t0, int64_t t1, int dtype,
               void *out, int nthreads) {
    if (d <= 0 || d > 256 || (d & 1) || t1 < t0) return 1;
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t t = t0; t < t1; ++t) {
        double z[256], x[256];
        uint64_t base = (uint64_t)t * 256u;
        for (int i = 0; i < d; i += 2) {
            double u1 = unit(draw(seed, base + (uint64_t)i));
            double u2 = unit(draw(seed, base + (uint64_t)i + 1));
            double rad = sqrt(-2.0 * log(u1));
            z[i] = rad * cos(two_pi * u2);
            z[i + 1] = rad * sin(two_pi * u2);
        }
        for (int c = 0; c < d; ++c) x[c] = 0.0;
        for (int i = 0; i < d; ++i) {
            const double zi = z[i];
            const double *row = M + (int64_t)i * d;
            for (int c = 0; c < d; ++c) x[c] += zi * row[c];
        }
        int chosen[4];
        for (int k = 0; k < 4; ++k) {
            int u = (int)(draw(seed, base + 128u + (uint64_t)k) % (uint64_t)(d - k));
            /* map u past the channels already taken, in ascending order */
            int sorted[4];
            for (int j = 0; j < k; ++j) sorted[j] = chosen[j];
            for (int a = 1; a < k; ++a)
                for (int b = a; b > 0 && sorted[b - 1] > sorted[b]; --b) {
                    int tmp = sorted[b];
                    sorted[b] = sorted[b - 1];
                    sorted[b - 1] = tmp;
                }
            for (int j = 0; j < k; ++j)
                if (u >= sorted[j]) ++u;
            chosen[k] = u;
            double sign = (draw(seed, base + 132u + (uint64_t)k) & 1u) ? 6.0 : -6.0;
            x[u] += sign;
        }
        int64_t o = (t - t0) * (int64_t)d;
        if (dtype == 0) {
            float *dst = (float *)out + o;
            for (int c = 0; c < d; ++c) dst[c] = (float)x[c];
        } else if (dtype == 1) {
            uint16_t *dst = (uint16_t *)out + o;
            for (int c = 0; c < d; ++c) dst[c] = bf16_of((float)x[c]);
        } else {
            double *dst = (double *)out + o;
            for (int c = 0; c < d; ++c) dst[c] = x[c];
        }
    }
    return 0;
}
