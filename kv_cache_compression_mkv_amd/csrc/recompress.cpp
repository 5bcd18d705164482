// Exact recompression of a finished packed segment on the host: the CPU side
// of heterogeneous double compression buffering (paper summary section 5.4;
// "MosaicKV 阅读笔记" reading notes, heterogeneous double buffering section
// and Fig. 4). The segment's tokens are re-packed with rotations computed from
// the segment itself, with the arithmetic of the GPU append:
//   x'_c = sum_j R[c][j] x_j   binary64, exact products (binary32 x bfloat16
//                               or binary32 x binary32 fit in 53 bits), j ascending
//   the r largest |x'_c| kept (ties to the lower channel) -- or, with element
//   groups of g adjacent channels, the r / g groups of largest energy
//   sum_m x'^2 (binary64, each square and sum rounded, m ascending; ties to the
//   lower group) -- stored in ascending channel order, each rounded once to
//   nearest even to the storage type;
//   per-block min/max keys of the stored sparse keys (0 at dropped channels)
//   in IEEE totalOrder.
// The result is written in the documented device layouts (include/mkv.h), so
// it can be copied to the device as is and swapped in by mkv_swap_segment.
#include <omp.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/mkv.h"

namespace {

constexpr int BT = MKV_BLOCK_TOKENS;

double raw_value(const void *x, int32_t dtype, int64_t i) {
    if (dtype == MKV_F32) return (double)static_cast<const float *>(x)[i];
    const uint32_t u = (uint32_t) static_cast<const uint16_t *>(x)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

// binary64 -> bfloat16 bits, nearest even, through a binary32 rounded to odd
// (truncated, with the last bit set when anything nonzero was cut off): an
// intermediate with at least two more significand bits, rounded to odd, makes
// the second nearest-even rounding equal to a direct one (Boldo and
// Melquiond, IEEE Trans. Computers 57(4), 2008).
uint16_t to_bf16(double x) {
    uint64_t b;
    memcpy(&b, &x, 8);
    const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    const int ex = (int)((b >> 52) & 0x7ff);
    const uint64_t m = b & 0xFFFFFFFFFFFFFull;
    if (ex == 0x7ff) return (uint16_t)(sign | (m ? 0x7FC0u : 0x7F80u));
    const int E = ex - 1023;
    uint32_t f;
    if (ex == 0) {
        f = m ? 1u : 0u;
    } else if (E > 127) {
        f = 0x7F7FFFFFu;
    } else if (E >= -126) {
        f = ((uint32_t)(E + 127) << 23) | (uint32_t)(m >> 29) | (uint32_t)((m & 0x1FFFFFFFull) != 0);
    } else {
        const uint64_t sig = m | (1ull << 52);
        const int sh = -97 - E;
        f = sh >= 64 ? 1u : (uint32_t)(sig >> sh) | (uint32_t)((sig & ((1ull << sh) - 1)) != 0);
    }
    return (uint16_t)(sign | ((f + 0x7FFFu + ((f >> 16) & 1u)) >> 16));
}

uint32_t to_f32(double x) {
    const float f = (float)x;  // the conversion rounds to nearest even
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

// totalOrder key of stored bits (s bytes): unsigned order = value order, -0 < +0
uint32_t order_key(uint32_t v, int s) {
    if (s == 2) return (v & 0x8000u) ? (~v & 0xFFFFu) : (v | 0x8000u);
    return (v & 0x80000000u) ? ~v : (v | 0x80000000u);
}

}  // namespace

extern "C" mkv_status mkv_recompress_segment(const void *k_host, const void *v_host, int32_t dtype, int32_t d,
                                             int32_t n_kv_heads, int64_t n_tokens, int64_t t_cap, int32_t kind,
                                             int32_t r, int32_t key_ch, int32_t group, void *data_out,
                                             void *meta_out, float *rot_out) {
    if (!k_host || !v_host || !data_out || !meta_out || !rot_out || n_kv_heads < 1 || t_cap < 1 || n_tokens < 1 ||
        n_tokens > t_cap || r < 1 || r > d || (kind != MKV_SEG_PACKED && kind != MKV_SEG_BITMAP) || key_ch < 0 ||
        key_ch > d || key_ch % 8 || (group != 0 && group != 1 && group != 2 && group != 4 && group != 8))
        return MKV_ERR_ARG;
    const int gs = group > 1 ? group : 1;  // channels per kept group
    if (r % gs) return MKV_ERR_ARG;
    if (d != MKV_HEAD_DIM) return MKV_ERR_UNSUPPORTED;
    if (dtype != MKV_F32 && dtype != MKV_BF16) return MKV_ERR_UNSUPPORTED;
    if ((t_cap + BT - 1) / BT > MKV_MAX_PACKED_BLOCKS) return MKV_ERR_UNSUPPORTED;
    const int s = dtype == MKV_BF16 ? 2 : 4;
    const int64_t nbcap = (t_cap + BT - 1) / BT, nb = (n_tokens + BT - 1) / BT;
    const bool bitmap = kind == MKV_SEG_BITMAP;
    // record: K values, V values, then K and V positions (u8 indices [16][r]
    // each, or 16-byte bitmaps [16] each)
    const int64_t pos_bytes = bitmap ? (int64_t)BT * (d / 8 / gs) : (int64_t)BT * r;
    const int64_t rec = (int64_t)BT * r * 2 * s + 2 * pos_bytes;
    const int64_t ntile = (nbcap + 63) / 64;
    const int kch = key_ch > 0 ? key_ch : d;  // channels of the block keys
    const int cpg = 16 / (2 * s), ng = kch / cpg;  // channels per meta 16-byte group, groups per block
    const int64_t mhead = ntile * ng * 64 * 16;
    const size_t xsz = (size_t)n_tokens * d;

    // rotations of each KV head from the segment's own vectors
    for (int g = 0; g < n_kv_heads; ++g)
        for (int kv = 0; kv < 2; ++kv) {
            const char *x = static_cast<const char *>(kv ? v_host : k_host) + (size_t)g * xsz * s;
            const mkv_status st =
                mkv_rotation_from_prefill(x, dtype, n_tokens, d, rot_out + ((size_t)g * 2 + kv) * d * d, nullptr);
            if (st != MKV_OK) return st;
        }

    char *data = static_cast<char *>(data_out);
    char *meta = static_cast<char *>(meta_out);
    memset(data, 0, (size_t)n_kv_heads * nbcap * rec);
    memset(meta, 0, (size_t)n_kv_heads * mhead);

    // records: one (KV head, block) per iteration
#pragma omp parallel
    {
        std::vector<double> xr(d), energy(d);
        std::vector<int> order(d), kept(r);
#pragma omp for schedule(dynamic, 16) collapse(2)
        for (int g = 0; g < n_kv_heads; ++g)
            for (int64_t l = 0; l < nb; ++l) {
                char *blk = data + ((size_t)g * nbcap + l) * rec;
                uint32_t kmn[MKV_HEAD_DIM], kmx[MKV_HEAD_DIM];
                for (int c = 0; c < d; ++c) {
                    kmn[c] = 0xFFFFFFFFu;
                    kmx[c] = 0u;
                }
                const int64_t t0 = l * BT, t1 = std::min<int64_t>(t0 + BT, n_tokens);
                for (int64_t t = t0; t < t1; ++t) {
                    const int slot = (int)(t - t0);
                    for (int kv = 0; kv < 2; ++kv) {
                        const void *x = kv ? v_host : k_host;
                        const float *R = rot_out + ((size_t)g * 2 + kv) * d * d;
                        const int64_t row = ((int64_t)g * n_tokens + t) * d;
                        for (int c = 0; c < d; ++c) {
                            double a = 0.0;
                            for (int j = 0; j < d; ++j) a += (double)R[(size_t)c * d + j] * raw_value(x, dtype, row + j);
                            xr[c] = a;
                        }
                        if (gs == 1) {
                            for (int c = 0; c < d; ++c) order[c] = c;
                            std::partial_sort(order.begin(), order.begin() + r, order.end(), [&](int a, int b) {
                                const double ma = xr[a] < 0 ? -xr[a] : xr[a], mb = xr[b] < 0 ? -xr[b] : xr[b];
                                return ma > mb || (ma == mb && a < b);
                            });
                            std::copy(order.begin(), order.begin() + r, kept.begin());
                        } else {
                            const int ng = d / gs;
                            for (int i = 0; i < ng; ++i) {
                                double e = 0.0;
                                for (int m = 0; m < gs; ++m) {
                                    const double v = xr[gs * i + m];
                                    const double sq = v * v;  // ISO C++ mode: no contraction
                                    e += sq;
                                }
                                energy[i] = e;
                                order[i] = i;
                            }
                            std::partial_sort(order.begin(), order.begin() + r / gs, order.begin() + ng,
                                              [&](int a, int b) {
                                                  return energy[a] > energy[b] || (energy[a] == energy[b] && a < b);
                                              });
                            for (int k = 0; k < r / gs; ++k)
                                for (int m = 0; m < gs; ++m) kept[k * gs + m] = gs * order[k] + m;
                        }
                        std::sort(kept.begin(), kept.end());
                        char *vals = blk + (size_t)kv * BT * r * s + (size_t)slot * r * s;
                        uint8_t *pos = reinterpret_cast<uint8_t *>(blk + (size_t)2 * BT * r * s + kv * pos_bytes +
                                                                   (size_t)slot * (bitmap ? d / 8 / gs : r));
                        uint32_t stored[MKV_HEAD_DIM] = {0};
                        for (int m = 0; m < r; ++m) {
                            const int c = kept[m];
                            const uint32_t bits = s == 2 ? (uint32_t)to_bf16(xr[c]) : to_f32(xr[c]);
                            if (s == 2) {
                                const uint16_t h = (uint16_t)bits;
                                memcpy(vals + (size_t)m * 2, &h, 2);
                            } else {
                                memcpy(vals + (size_t)m * 4, &bits, 4);
                            }
                            if (bitmap) {
                                if (c % gs == 0) pos[c / gs / 8] |= (uint8_t)(1u << ((c / gs) % 8));
                            } else {
                                pos[m] = (uint8_t)c;
                            }
                            stored[c] = bits;
                        }
                        if (kv == 0)
                            for (int c = 0; c < d; ++c) {
                                const uint32_t key = order_key(stored[c], s);
                                kmn[c] = std::min(kmn[c], key);
                                kmx[c] = std::max(kmx[c], key);
                            }
                    }
                }
                // block keys: lane l % 64 of tile l / 64, group c / cpg, (min, max) of channel c < kch
                char *tile = meta + (size_t)g * mhead + (size_t)(l / 64) * ng * 64 * 16;
                for (int c = 0; c < kch; ++c) {
                    char *pr = tile + ((size_t)(c / cpg) * 64 + l % 64) * 16 + (size_t)(c % cpg) * 2 * s;
                    for (int w = 0; w < 2; ++w) {
                        const uint32_t key = w ? kmx[c] : kmn[c];
                        uint32_t bits;
                        if (s == 2) bits = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
                        else bits = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
                        if (s == 2) {
                            const uint16_t h = (uint16_t)bits;
                            memcpy(pr + (size_t)w * 2, &h, 2);
                        } else {
                            memcpy(pr + (size_t)w * 4, &bits, 4);
                        }
                    }
                }
            }
    }
    return MKV_OK;
}
