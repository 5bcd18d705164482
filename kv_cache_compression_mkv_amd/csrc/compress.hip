// Compression of new K/V vectors into dense or packed segments, and the bulk
// recomputation of per-block min/max keys.
//
// Per vector ("MosaicKV 阅读笔记" reading notes, Eq. 7-9 and Algorithm 1;
// paper summary sections 4.2 and 5.2):
//   x'_c = sum_j R[c][j] x_j          float64, exact products, j ascending
//   keep the r channels of largest |x'_c| (ties to the lower channel)
//   store (channel, round(x'_c)) pairs in ascending channel order
// Packed segments also keep per-block min/max keys of the stored sparse key
// vectors up to date (the Quest-style block keys of the reading notes' Quest
// paragraph and the paper's section 5.2).
//
// One wave per matrix handles one block of one (request, segment, KV head):
// the keys, and (in the same or another workgroup) the values. Lane l owns channels l and l+64,
// so the top-r selection is a wave-wide radix search with ballots and the
// packing order falls out of a ballot prefix count.
#include <algorithm>

#include "device_util.hpp"
#include "mkv_internal.h"
#include "qrot.hpp"

namespace mkv {

namespace {

// Compute x' = R x for one token (xs: its input as doubles in LDS, exact
// copies of the stored values). R is staged in LDS with rows padded to D + 1
// floats, so the 64 lanes reading 64 rows at one column hit distinct banks.
// Lane owns channels lane and lane + 64; each sum is one fp64 chain over j
// ascending, and every product of two floats is exact in fp64.
__device__ __forceinline__ void rotate_f64_lds(const float (*Rs)[D + 1], const double *xs, int lane, double &a0,
                                               double &a1) {
    double p0 = 0.0, p1 = 0.0;
#pragma unroll 8
    for (int j = 0; j < D; ++j) {
        const double x = xs[j];
        p0 = fma((double)Rs[lane][j], x, p0);
        p1 = fma((double)Rs[lane + 64][j], x, p1);
    }
    a0 = p0;
    a1 = p1;
}

// ---- bulk rotation: inputs in registers, broadcast across lanes by DPP ----
// Lane l owns channels l and l + 64. In row q (16 lanes) lane n holds inputs
// 8n .. 8n + 7 of each token, one per register (the four rows hold the same
// copy), so input j = 8n + m is register m of lane n of every row; the
// fused multiply-add reads it with a row broadcast of lane n, and no input
// goes through LDS. R is held in LDS as binary64 pairs (R[c][j], R[c+64][j])
// at [j][c], one 16-byte read per column per lane.
//
// The multiply-adds are written as ordered assembly statements because the
// compiler does not fuse the broadcast into the f64 multiply-add. A DPP read
// needs two wait states after a vector-ALU write of any register it reads:
// inputs are fenced by dpp_fence after their conversion, R values come from
// LDS reads, zeroed accumulators are fenced too, and an accumulator is
// rewritten only 2 NT statements later.
template <int N>
__device__ __forceinline__ void fma_row_bcast(double &acc, double x, double r) {
    asm volatile("v_fmac_f64_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc)
                 : "v"(x), "v"(r), "n"(N));
}

__device__ __forceinline__ void dpp_fence(double (&X)[8]) {
    asm volatile("s_nop 1"
                 : "+v"(X[0]), "+v"(X[1]), "+v"(X[2]), "+v"(X[3]), "+v"(X[4]), "+v"(X[5]), "+v"(X[6]), "+v"(X[7]));
}

// one token's inputs 8n .. 8n + 7 (raw storage words) and their binary64 values
template <typename ST>
struct Row8 {
    uint4 w[ST::bytes / 2];
};

template <typename ST>
__device__ __forceinline__ void row8_load(Row8<ST> &raw, const typename ST::bits_t *xr, int n) {
    const uint4 *p = reinterpret_cast<const uint4 *>(xr) + n * (ST::bytes / 2);
#pragma unroll
    for (int k = 0; k < ST::bytes / 2; ++k) raw.w[k] = p[k];
}

__device__ __forceinline__ void row8_f64(const Row8<Bf16> &raw, double (&X)[8]) {
    const uint32_t u[4] = {raw.w[0].x, raw.w[0].y, raw.w[0].z, raw.w[0].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        X[2 * k] = (double)bf16_lo(u[k]);
        X[2 * k + 1] = (double)bf16_hi(u[k]);
    }
}

__device__ __forceinline__ void row8_f64(const Row8<F32> &raw, double (&X)[8]) {
    const uint32_t u[8] = {raw.w[0].x, raw.w[0].y, raw.w[0].z, raw.w[0].w,
                           raw.w[1].x, raw.w[1].y, raw.w[1].z, raw.w[1].w};
#pragma unroll
    for (int k = 0; k < 8; ++k) X[k] = (double)__uint_as_float(u[k]);
}

// columns 8n .. 8n + 7 of the rotation of NT tokens (one fp64 chain per
// channel and token, j ascending across calls)
template <int NT, int N, int PF>
__device__ __forceinline__ void rotate_cols8(const double2 *Rl, double2 (&ring)[PF], const double (&X)[NT][8],
                                             double (&a0)[NT], double (&a1)[NT]) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int j = 8 * N + m;
        const double2 rc = ring[j % PF];
        if (j + PF < D) ring[j % PF] = Rl[(j + PF) * 64];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            fma_row_bcast<N>(a0[t], X[t][m], rc.x);
            fma_row_bcast<N>(a1[t], X[t][m], rc.y);
        }
    }
}

template <int NT>
__device__ __forceinline__ void rotate_regs(const double2 *Rl, const double (&X)[NT][8], double (&a0)[NT],
                                            double (&a1)[NT]) {
    constexpr int PF = 3;  // columns of R in flight
    static_assert(NT == 8, "fences cover 8 accumulators each");
#pragma unroll
    for (int t = 0; t < NT; ++t) a0[t] = a1[t] = 0.0;
    dpp_fence(a0);
    dpp_fence(a1);
    double2 ring[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) ring[k] = Rl[k * 64];
    rotate_cols8<NT, 0, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 1, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 2, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 3, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 4, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 5, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 6, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 7, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 8, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 9, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 10, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 11, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 12, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 13, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 14, PF>(Rl, ring, X, a0, a1);
    rotate_cols8<NT, 15, PF>(Rl, ring, X, a0, a1);
}

// Keys are the magnitude bit patterns (63 bits; order = magnitude order).
// The threshold is found bit by bit with ballot counts, from the leading bit
// of the largest key down (higher bits are zero in every key). It keeps the
// invariant that at least r keys are >= thr; once exactly r are (cnt == r)
// they are the kept set and lower bits cannot change it, so the search stops.
__device__ __forceinline__ void topr_keep(double v0, double v1, int r, int lane, bool &keep0,
                                          bool &keep1) {
    const uint64_t k0 = (uint64_t)__double_as_longlong(v0) & 0x7FFFFFFFFFFFFFFFull;
    const uint64_t k1 = (uint64_t)__double_as_longlong(v1) & 0x7FFFFFFFFFFFFFFFull;
    // wave max of the keys' high words (DPP row max, then the four rows)
    uint32_t hm = (uint32_t)(max(k0, k1) >> 32);
    hm = max(hm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hm, 0x121, 0xf, 0xf, false));
    hm = max(hm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hm, 0x122, 0xf, 0xf, false));
    hm = max(hm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hm, 0x124, 0xf, 0xf, false));
    hm = max(hm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hm, 0x128, 0xf, 0xf, false));
    hm = max(max((uint32_t)__builtin_amdgcn_readlane((int)hm, 0), (uint32_t)__builtin_amdgcn_readlane((int)hm, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)hm, 32), (uint32_t)__builtin_amdgcn_readlane((int)hm, 48)));
    uint64_t thr = 0;
    int cnt = 2 * 64;  // keys >= thr
    for (int bit = hm ? 63 - __clz(hm) : 31; bit >= 0 && cnt > r; --bit) {
        const uint64_t cand = thr | (1ull << bit);
        const int c = popc64(ballot(k0 >= cand)) + popc64(ballot(k1 >= cand));
        if (c >= r) {
            thr = cand;
            cnt = c;
        }
    }
    const bool gt0 = k0 > thr, gt1 = k1 > thr;
    const int need = r - popc64(ballot(gt0)) - popc64(ballot(gt1));
    const uint64_t e0 = ballot(k0 == thr), e1 = ballot(k1 == thr);
    const uint64_t below = lanes_below(lane);
    const int rank0 = popc64(e0 & below);
    const int rank1 = popc64(e0) + popc64(e1 & below);
    keep0 = gt0 || ((k0 == thr) && rank0 < need);
    keep1 = gt1 || ((k1 == thr) && rank1 < need);
}

// The same selection for NT tokens at once (v0/v1[t]: token t's channels
// lane and lane + 64; tokens t >= nt are padding), with the same kept set.
// The threshold is the largest key T with at least r keys >= T, found in
// three steps that each fix more of its bits: its exponent (scanning down
// from the largest exponent present), the 20 mantissa bits of the keys' high
// words (compares of high words only), then, only while some token still has
// more than r keys >= its threshold, the low words. The NT searches run side
// by side, so each token's ballot-to-scalar latency is covered by the others;
// a token with exactly r keys >= its threshold is settled (later steps cannot
// change its kept set).
template <int NT>
__device__ __forceinline__ void topr_keep_nt(const double (&v0)[NT], const double (&v1)[NT], int nt, int r, int lane,
                                             bool (&keep0)[NT], bool (&keep1)[NT]) {
    uint64_t k0[NT], k1[NT];
    uint32_t h0[NT], h1[NT], th[NT];
    int cnt[NT];
    uint32_t hm = 0, found = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        k0[t] = (uint64_t)__double_as_longlong(v0[t]) & 0x7FFFFFFFFFFFFFFFull;
        k1[t] = (uint64_t)__double_as_longlong(v1[t]) & 0x7FFFFFFFFFFFFFFFull;
        h0[t] = (uint32_t)(k0[t] >> 32);
        h1[t] = (uint32_t)(k1[t] >> 32);
        hm = max(hm, max(h0[t], h1[t]));
        th[t] = 0;
        cnt[t] = t < nt ? 2 * 64 : r;  // padding tokens count as settled
        found |= (t < nt ? 0u : 1u) << t;
    }
    hm = max(hm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hm, 0x121, 0xf, 0xf, false));
    hm = max(hm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hm, 0x122, 0xf, 0xf, false));
    hm = max(hm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hm, 0x124, 0xf, 0xf, false));
    hm = max(hm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hm, 0x128, 0xf, 0xf, false));
    hm = max(max((uint32_t)__builtin_amdgcn_readlane((int)hm, 0), (uint32_t)__builtin_amdgcn_readlane((int)hm, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)hm, 32), (uint32_t)__builtin_amdgcn_readlane((int)hm, 48)));
    // exponent: every key is >= 0, so the scan ends at exponent 0 at the latest
    constexpr uint32_t ALL = (1u << NT) - 1;
    for (int e = (int)(hm >> 20); e >= 0 && found != ALL; --e) {
        const uint32_t cand = (uint32_t)e << 20;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int c = popc64(ballot(h0[t] >= cand)) + popc64(ballot(h1[t] >= cand));
            const bool take = !((found >> t) & 1u) && c >= r;
            th[t] = take ? cand : th[t];
            cnt[t] = take ? c : cnt[t];
            found |= (take ? 1u : 0u) << t;
        }
    }
    int excess = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) excess += cnt[t] - r;
    // high-word mantissa bits (k >= T with T's low word zero iff high(k) >= high(T))
    for (int bit = 19; bit >= 0 && excess > 0; --bit) {
        excess = 0;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t cand = th[t] | (1u << bit);
            const int c = popc64(ballot(h0[t] >= cand)) + popc64(ballot(h1[t] >= cand));
            const bool take = c >= r;
            th[t] = take ? cand : th[t];
            cnt[t] = take ? c : cnt[t];
            excess += cnt[t] - r;
        }
    }
    uint64_t thr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) thr[t] = (uint64_t)th[t] << 32;
    for (int bit = 31; bit >= 0 && excess > 0; --bit) {
        excess = 0;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint64_t cand = thr[t] | (1ull << bit);
            const int c = popc64(ballot(k0[t] >= cand)) + popc64(ballot(k1[t] >= cand));
            const bool take = c >= r;
            thr[t] = take ? cand : thr[t];
            cnt[t] = take ? c : cnt[t];
            excess += cnt[t] - r;
        }
    }
    if (excess == 0) {  // every token has exactly r keys >= its threshold
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            keep0[t] = k0[t] >= thr[t];
            keep1[t] = k1[t] >= thr[t];
        }
        return;
    }
    const uint64_t below = lanes_below(lane);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const bool gt0 = k0[t] > thr[t], gt1 = k1[t] > thr[t];
        const int need = r - popc64(ballot(gt0)) - popc64(ballot(gt1));
        const uint64_t e0 = ballot(k0[t] == thr[t]), e1 = ballot(k1[t] == thr[t]);
        const int rank0 = popc64(e0 & below);
        const int rank1 = popc64(e0) + popc64(e1 & below);
        keep0[t] = gt0 || ((k0[t] == thr[t]) && rank0 < need);
        keep1[t] = gt1 || ((k1[t] == thr[t]) && rank1 < need);
    }
}

// Element groups (g > 1 adjacent channels kept or dropped together). The
// energy of group `lane` (channels g lane .. g lane + g - 1) from the rotated
// channels held as v0 (channel lane) and v1 (channel lane + 64) of every lane:
// binary64, each square and each sum rounded, channels ascending; 0 on lanes
// >= D / g. Those zero keys sit above every group's slot, so the top-r search's
// tie rule (lower slot first) never prefers them to a group of energy 0.
__device__ __forceinline__ double group_energy(double v0, double v1, int g, int lane) {
#pragma clang fp contract(off)
    double e = 0.0;
    for (int m = 0; m < g; ++m) {
        const int c = g * lane + m;
        const double a = __shfl(v0, c & 63, 64), b = __shfl(v1, c & 63, 64);
        const double x = c < 64 ? a : b;
        e = e + x * x;
    }
    return lane < D / g ? e : 0.0;
}

// kept flags of channels lane and lane + 64 from the per-group flags (group i on lane i)
__device__ __forceinline__ void group_expand(bool kg, int g, int lane, bool &keep0, bool &keep1) {
    const int f = kg ? 1 : 0;
    keep0 = __shfl(f, lane / g, 64) != 0;
    keep1 = __shfl(f, (lane + 64) / g, 64) != 0;
}

// top-r of one token with element groups of g channels (g = 1: single channels)
__device__ __forceinline__ void topr_keep_g(double v0, double v1, int r, int g, int lane, bool &keep0,
                                            bool &keep1) {
    if (g <= 1) {
        topr_keep(v0, v1, r, lane, keep0, keep1);
        return;
    }
    bool kg, unused;
    topr_keep(group_energy(v0, v1, g, lane), 0.0, r / g, lane, kg, unused);
    group_expand(kg, g, lane, keep0, keep1);
}

template <int NT>
__device__ __forceinline__ void topr_keep_nt_g(const double (&v0)[NT], const double (&v1)[NT], int nt, int r, int g,
                                               int lane, bool (&keep0)[NT], bool (&keep1)[NT]) {
    if (g <= 1) {
        topr_keep_nt<NT>(v0, v1, nt, r, lane, keep0, keep1);
        return;
    }
    double e[NT], z[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        e[t] = group_energy(v0[t], v1[t], g, lane);
        z[t] = 0.0;
    }
    bool kg[NT], unused[NT];
    topr_keep_nt<NT>(e, z, nt, r / g, lane, kg, unused);
#pragma unroll
    for (int t = 0; t < NT; ++t) group_expand(kg[t], g, lane, keep0[t], keep1[t]);
}

// Per-block state of one wave's append into block blk of one (entry, KV head,
// matrix): destination pointers, the new slots [sa, se), the running keys of
// a packed segment's block (keys matrix only) and the first new row.
template <typename ST>
struct BlockJob {
    typename ST::bits_t *vals;
    uint8_t *idxs;
    char *meta_tile;
    const typename ST::bits_t *xin;
    int p0, sa, se, r, G16, cpg, kch, g;
    bool packed, bitmap, do_meta;
    uint32_t mn0, mx0, mn1, mx1;
    typename ST::bits_t x0, x1;  // row of the first new token (lane's channels; one-token appends)
};

// Pointers of block blk, its stored keys (when it already holds tokens) and
// the first new token's row: the loads are issued here, not waited for.
template <typename ST, bool BULK>
__device__ __forceinline__ void block_begin(BlockJob<ST> &J, const CompressArgs &A, const CompressEntry &E,
                                            size_t unit, int g, int blk, int wave, int lane) {
    using bits_t = typename ST::bits_t;
    const int p0 = blk * BT;
    const int sa = max(E.a, p0) - p0;
    const int se = min(E.e, p0 + BT) - p0;
    const bits_t *xin = reinterpret_cast<const bits_t *>(wave ? A.v_new : A.k_new) + unit * A.n_max * D;
    const bool packed = packed_kind(E.kind);
    const bool bitmap = E.kind == MKV_SEG_BITMAP;
    const int r = E.r;
    char *blkbase;
    if (packed) {
        const size_t rec = (size_t)record_bytes(E.kind, r, ST::bytes, E.group);
        blkbase = static_cast<char *>(E.data) + ((size_t)g * E.nbcap + blk) * rec;
    } else {
        blkbase = static_cast<char *>(E.data) + ((size_t)g * E.nbcap + blk) * 2 * BT * D * ST::bytes;
    }
    bits_t *vals = packed ? reinterpret_cast<bits_t *>(blkbase + (size_t)wave * BT * r * ST::bytes)
                          : reinterpret_cast<bits_t *>(blkbase + (size_t)wave * BT * D * ST::bytes);
    // u8 indices [16][r], or bitmaps [16][D / 8 / group], of this matrix
    uint8_t *idxs = packed ? reinterpret_cast<uint8_t *>(blkbase + (size_t)2 * BT * r * ST::bytes +
                                                         (size_t)wave * BT * pos_bytes(E.kind, r, E.group))
                           : nullptr;

    // per-block keys (keys wave, packed segments) of the leading kch
    // channels: running totalOrder min/max
    const bool do_meta = packed && wave == 0;
    const int kch = E.kch;
    const int G16 = 2 * kch * ST::bytes / 16;  // 16-byte groups per block
    const int cpg = 16 / (2 * ST::bytes);      // channels per group
    char *meta_tile = nullptr;
    uint32_t mn0 = 0xFFFFFFFFu, mx0 = 0u, mn1 = 0xFFFFFFFFu, mx1 = 0u;
    if (do_meta) {
        const int ntile = (E.nbcap + META_TILE - 1) / META_TILE;
        meta_tile = static_cast<char *>(E.meta) + ((size_t)g * ntile + blk / META_TILE) * G16 * META_TILE * 16;
        if (sa > 0) {  // block already holds tokens: start from its keys
            const int bl = blk % META_TILE;
            for (int h = 0; h < 2; ++h) {
                const int c = lane + 64 * h;
                if (c >= kch) continue;
                const bits_t *pr = reinterpret_cast<const bits_t *>(
                    meta_tile + ((size_t)(c / cpg) * META_TILE + bl) * 16 + (c % cpg) * 2 * ST::bytes);
                const uint32_t kmn = order_key<ST>(pr[0]), kmx = order_key<ST>(pr[1]);
                if (h == 0) { mn0 = kmn; mx0 = kmx; } else { mn1 = kmn; mx1 = kmx; }
            }
        }
    }

    // one-token appends: the first token's row is loaded before R is staged,
    // so that the two (and the block keys above) are in flight together (bulk
    // appends load their rows themselves)
    bits_t x0 = 0, x1 = 0;
    if (!BULK && sa < se) {
        const bits_t *xr = xin + (size_t)(E.row0 + (p0 + sa - E.a)) * D;
        x0 = xr[lane];
        x1 = xr[lane + 64];
    }
    J.vals = vals;
    J.idxs = idxs;
    J.meta_tile = meta_tile;
    J.xin = xin;
    J.p0 = p0;
    J.sa = sa;
    J.se = se;
    J.r = r;
    J.G16 = G16;
    J.cpg = cpg;
    J.kch = kch;
    J.g = E.group;
    J.packed = packed;
    J.bitmap = bitmap;
    J.do_meta = do_meta;
    J.mn0 = mn0; J.mx0 = mx0; J.mn1 = mn1; J.mx1 = mx1;
    J.x0 = x0;
    J.x1 = x1;
}

// Rounding and the stores of token `slot` of J's block from its rotated
// channels (lane: channels lane and lane + 64) and, for packed segments, its
// kept channels keep0/keep1; packed segments fold the stored key into the
// block's running min/max.
template <typename ST>
__device__ __forceinline__ void store_kept(BlockJob<ST> &J, int slot, double v0, double v1, bool keep0, bool keep1,
                                           int lane) {
    using bits_t = typename ST::bits_t;
    const bits_t s0 = round_store<ST>(v0), s1 = round_store<ST>(v1);
    if (J.packed) {
        const uint64_t m0 = ballot(keep0), m1 = ballot(keep1);
        const uint64_t below = lanes_below(lane);
        bits_t *vrow = J.vals + (size_t)slot * J.r;
        if (keep0) vrow[popc64(m0 & below)] = s0;
        if (keep1) vrow[popc64(m0) + popc64(m1 & below)] = s1;
        if (J.bitmap && J.g <= 1) {
            // bit c of the vector's bitmap: channel c kept (channels lane and lane + 64 of the ballots)
            if (lane == 0) {
                uint64_t *brow = reinterpret_cast<uint64_t *>(J.idxs + (size_t)slot * (D / 8));
                brow[0] = m0;
                brow[1] = m1;
            }
        } else if (J.bitmap) {
            // bit i: group i (channels g i ..) kept, read from its first channel's ballot bit
            const int c = J.g * lane;
            const bool kg = lane < D / J.g && (((c < 64 ? m0 >> c : m1 >> (c - 64)) & 1ull) != 0);
            const uint64_t gb = ballot(kg);
            if (lane == 0) {
                uint8_t *brow = J.idxs + (size_t)slot * (D / 8 / J.g);
                if (J.g == 2) *reinterpret_cast<uint64_t *>(brow) = gb;
                else if (J.g == 4) *reinterpret_cast<uint32_t *>(brow) = (uint32_t)gb;
                else *reinterpret_cast<uint16_t *>(brow) = (uint16_t)gb;
            }
        } else {
            uint8_t *irow = J.idxs + (size_t)slot * J.r;
            if (keep0) irow[popc64(m0 & below)] = (uint8_t)lane;
            if (keep1) irow[popc64(m0) + popc64(m1 & below)] = (uint8_t)(lane + 64);
        }
        if (J.do_meta) {
            const uint32_t q0 = order_key<ST>(keep0 ? s0 : (bits_t)0);
            const uint32_t q1 = order_key<ST>(keep1 ? s1 : (bits_t)0);
            J.mn0 = min(J.mn0, q0); J.mx0 = max(J.mx0, q0);
            J.mn1 = min(J.mn1, q1); J.mx1 = max(J.mx1, q1);
        }
    } else {
        bits_t *vrow = J.vals + (size_t)slot * D;
        vrow[lane] = s0;
        vrow[lane + 64] = s1;
    }
}

// top-r selection, then the stores, of one token
template <typename ST>
__device__ __forceinline__ void store_token(BlockJob<ST> &J, int slot, double v0, double v1, int lane) {
    bool keep0 = false, keep1 = false;
    if (J.packed) topr_keep_g(v0, v1, J.r, J.g, lane, keep0, keep1);
    store_kept<ST>(J, slot, v0, v1, keep0, keep1, lane);
}

// After a block's new tokens: clear the slots after its last token when this
// call started the block, and write the block keys back.
template <typename ST>
__device__ __forceinline__ void block_finish(const BlockJob<ST> &J, int blk, int lane) {
    using bits_t = typename ST::bits_t;
    if (J.sa == 0 && J.se < BT) {
        if (J.packed) {
            for (int i = J.se * J.r + lane; i < BT * J.r; i += 64) J.vals[i] = (bits_t)0;
            const int ib = J.bitmap ? D / 8 / J.g : J.r;  // position bytes per vector
            for (int i = J.se * ib + lane; i < BT * ib; i += 64) J.idxs[i] = 0;
        } else {
            for (int i = J.se * D + lane; i < BT * D; i += 64) J.vals[i] = (bits_t)0;
        }
    }
    if (J.do_meta && J.se > J.sa) {
        const int bl = blk % META_TILE;
        for (int h = 0; h < 2; ++h) {
            const int c = lane + 64 * h;
            if (c >= J.kch) continue;
            bits_t *pr = reinterpret_cast<bits_t *>(J.meta_tile + ((size_t)(c / J.cpg) * META_TILE + bl) * 16 +
                                                    (c % J.cpg) * 2 * ST::bytes);
            pr[0] = key_to_bits<ST>(h == 0 ? J.mn0 : J.mn1);
            pr[1] = key_to_bits<ST>(h == 0 ? J.mx0 : J.mx1);
        }
    }
}

// Rotate, rank, round and store the block's new tokens one at a time (R from
// LDS; xs is the wave's LDS row of doubles), the next row loading while one
// is rotated; then finish the block.
template <typename ST>
__device__ __forceinline__ void block_run(BlockJob<ST> &J, const CompressEntry &E, int blk, int lane,
                                          const float (*Rs)[D + 1], double (*xs)[D]) {
    using bits_t = typename ST::bits_t;
    bits_t x0 = J.x0, x1 = J.x1;
    for (int slot = J.sa; slot < J.se; ++slot) {
        xs[0][lane] = (double)bits_to_float<ST>(x0);
        xs[0][lane + 64] = (double)bits_to_float<ST>(x1);
        wave_lds_sync();
        if (slot + 1 < J.se) {
            const bits_t *xr = J.xin + (size_t)(E.row0 + (J.p0 + slot + 1 - E.a)) * D;
            x0 = xr[lane];
            x1 = xr[lane + 64];
        }
        double a0, a1;
        rotate_f64_lds(Rs, xs[0], lane, a0, a1);
        wave_lds_sync();
        store_token<ST>(J, slot, a0, a1, lane);
    }
    block_finish<ST>(J, blk, lane);
}

// One workgroup per (block, matrix) of an (entry, KV head), for appends of a
// token or two: its 256 threads copy R_k or R_v into LDS (rows padded to
// D + 1 floats, so the 64 lanes reading 64 rows at one column hit distinct
// banks) with one round of coalesced 16-byte loads; wave 0 then rotates the
// block's new tokens from LDS, a token at a time. The block's keys and first
// row are requested before the copy, so those loads overlap it; the K and V
// workgroups run side by side.
// Workgroups past the append table (z >= n_ent) rotate queries instead.
template <typename ST>
__global__ __launch_bounds__(256) void k_compress(const CompressArgs A) {
    if ((int)blockIdx.z >= A.n_ent) {
        if (blockIdx.x >= D / 32) return;
        __shared__ __align__(16) float qsh[4][D];
        const int b = (int)blockIdx.z - A.n_ent, g = (int)blockIdx.y, cb = (int)blockIdx.x;
        // the cache's rotation: q' slot 0 of the request
        const float *Rb = A.rot + (size_t)b * A.n_kv * 2 * D * D;
        const float *qb = A.q + (size_t)b * A.q_hq * D;
        float *qa = A.qa + (size_t)b * A.q_ns * A.q_hq * D;
        float *qs = A.qs + (size_t)b * A.q_ns * A.n_kv * D * 2 * A.q_G;
        switch (A.q_G) {
        case 1: qrot_block<1>(Rb, qb, qa, qs, g, cb, qsh); break;
        case 2: qrot_block<2>(Rb, qb, qa, qs, g, cb, qsh); break;
        default: qrot_block<4>(Rb, qb, qa, qs, g, cb, qsh); break;
        }
        return;
    }
    const CompressEntry &E = A.ent[blockIdx.z];
    const int bx = (int)blockIdx.x >> 1;  // block index within the entry's range
    if (bx >= E.nblk) return;
    const int mat = (int)blockIdx.x & 1;  // 0: keys (R_k), 1: values (R_v)
    const int g = (int)blockIdx.y;
    const int w = (int)(threadIdx.x >> 6);
    const int lane = lane_id();
    const size_t unit = (size_t)E.b * A.n_kv + g;
    __shared__ __align__(16) double xs[1][D];
    __shared__ float Rst[D][D + 1];
    BlockJob<ST> J;
    if (w == 0) block_begin<ST, false>(J, A, E, unit, g, E.blk0 + bx, mat, lane);
    {
        const float4 *Rg = reinterpret_cast<const float4 *>(E.rot + ((size_t)g * 2 + mat) * D * D);
        float4 v[D * D / 4 / 256];
#pragma unroll
        for (int k = 0; k < D * D / 4 / 256; ++k) v[k] = Rg[threadIdx.x + 256 * k];
#pragma unroll
        for (int k = 0; k < D * D / 4 / 256; ++k) {
            const int i = (int)threadIdx.x + 256 * k;
            const int c = i / (D / 4), j = (i % (D / 4)) * 4;
            Rst[c][j] = v[k].x;
            Rst[c][j + 1] = v[k].y;
            Rst[c][j + 2] = v[k].z;
            Rst[c][j + 3] = v[k].w;
        }
    }
    __syncthreads();
    if (w == 0) block_run<ST>(J, E, E.blk0 + bx, lane, Rst, xs);
}

// Bulk appends (prefill): one workgroup of 8 waves per (chunk of
// COMPRESS_CHUNK blocks, matrix) of an (entry, KV head). R is copied into LDS
// once per chunk, as binary64; wave w takes blocks w, w + 8, ... of the chunk
// and rotates their tokens BULK_NT at a time with inputs in registers; the
// rows of a wave's next pass (in the same or its next block) load while the
// current pass is ranked and stored.
constexpr int BULK_NT = 8;
constexpr int BULK_WAVES = 8;

template <typename ST>
__global__ __launch_bounds__(64 * BULK_WAVES) void k_compress_bulk(const CompressArgs A) {
    using bits_t = typename ST::bits_t;
    // a copy: the stores below would otherwise make the compiler reload entry fields
    const CompressEntry E = A.ent[blockIdx.z];
    const int c0 = ((int)blockIdx.x >> 1) * A.chunk_blocks;
    if (c0 >= E.nblk) return;
    const int c1 = min(c0 + A.chunk_blocks, E.nblk);
    const int mat = (int)blockIdx.x & 1;  // 0: keys (R_k), 1: values (R_v)
    const int g = (int)blockIdx.y;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = lane_id();
    const size_t unit = (size_t)E.b * A.n_kv + g;
    __shared__ __align__(16) double2 Rl[D * 64];  // [j][c]: (R[c][j], R[c + 64][j])
    {
        // thread: channel pair c, columns 16 jb .. 16 jb + 15
        const float *Rg = E.rot + ((size_t)g * 2 + mat) * D * D;
        const int c = (int)threadIdx.x & 63, jb = (int)threadIdx.x >> 6;
        const float4 *r0 = reinterpret_cast<const float4 *>(Rg + (size_t)c * D + 16 * jb);
        const float4 *r1 = reinterpret_cast<const float4 *>(Rg + (size_t)(c + 64) * D + 16 * jb);
        float4 u[4], v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            u[k] = r0[k];
            v[k] = r1[k];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = 16 * jb + 4 * k;
            Rl[(j + 0) * 64 + c] = make_double2(u[k].x, v[k].x);
            Rl[(j + 1) * 64 + c] = make_double2(u[k].y, v[k].y);
            Rl[(j + 2) * 64 + c] = make_double2(u[k].z, v[k].z);
            Rl[(j + 3) * 64 + c] = make_double2(u[k].w, v[k].w);
        }
    }
    __syncthreads();
    const double2 *Rlane = Rl + lane;
    const int n = lane & 15;
    const bits_t *xin = reinterpret_cast<const bits_t *>(mat ? A.v_new : A.k_new) + unit * A.n_max * D;
    auto row_of = [&](int blk, int slot) { return xin + (size_t)(E.row0 + (blk * BT + slot - E.a)) * D; };
    auto slots_of = [&](int blk, int &sa, int &se) {
        sa = max(E.a, blk * BT) - blk * BT;
        se = min(E.e, blk * BT + BT) - blk * BT;
    };
    // rows of the next pass: block blk, slots [slot, slot + BULK_NT)
    Row8<ST> raw[BULK_NT];
    // (slot < se; rows past the block's last new token repeat it and are not used)
    auto load_pass = [&](int blk, int slot, int se) {
#pragma unroll
        for (int t = 0; t < BULK_NT; ++t) row8_load<ST>(raw[t], row_of(blk, min(slot + t, se - 1)), n);
    };
    int bx = c0 + w;
    if (bx >= c1) return;
    {
        int sa, se;
        slots_of(E.blk0 + bx, sa, se);
        load_pass(E.blk0 + bx, sa, se);
    }
    for (; bx < c1; bx += BULK_WAVES) {
        const int blk = E.blk0 + bx;
        BlockJob<ST> J;
        block_begin<ST, true>(J, A, E, unit, g, blk, mat, lane);
        for (int slot = J.sa; slot < J.se; slot += BULK_NT) {
            const int nt = min(BULK_NT, J.se - slot);
            double X[BULK_NT][8];
#pragma unroll
            for (int t = 0; t < BULK_NT; ++t) {
                if (t < nt) {
                    row8_f64(raw[t], X[t]);
                } else {
#pragma unroll
                    for (int m = 0; m < 8; ++m) X[t][m] = 0.0;
                }
                dpp_fence(X[t]);
            }
            double a0[BULK_NT], a1[BULK_NT];
            rotate_regs<BULK_NT>(Rlane, X, a0, a1);
            // the next pass's rows: this block's next slots, else the next block's first
            if (slot + BULK_NT < J.se) {
                load_pass(blk, slot + BULK_NT, J.se);
            } else if (bx + BULK_WAVES < c1) {
                int sa2, se2;
                slots_of(blk + BULK_WAVES, sa2, se2);
                load_pass(blk + BULK_WAVES, sa2, se2);
            }
            bool keep0[BULK_NT], keep1[BULK_NT];
            if (J.packed) {
                topr_keep_nt_g<BULK_NT>(a0, a1, nt, J.r, J.g, lane, keep0, keep1);
            } else {
#pragma unroll
                for (int t = 0; t < BULK_NT; ++t) keep0[t] = keep1[t] = false;
            }
#pragma unroll
            for (int t = 0; t < BULK_NT; ++t)
                if (t < nt) store_kept<ST>(J, slot + t, a0[t], a1[t], keep0[t], keep1[t], lane);
        }
        block_finish<ST>(J, blk, lane);
    }
}

// Bulk recomputation of the per-block keys of one packed segment from the
// stored records. One wave per block: the kept values of each valid token are
// scattered into a zeroed dense row in LDS and folded into totalOrder min/max.
template <typename ST>
__global__ __launch_bounds__(64) void k_block_meta(const MetaArgs A) {
    using bits_t = typename ST::bits_t;
    const MetaEntry &E = A.ent[blockIdx.z];
    const int blk = (int)blockIdx.x;
    if (blk >= E.nb) return;
    const int g = (int)blockIdx.y;
    const int lane = lane_id();
    const int r = E.r;
    const bool bitmap = E.kind == MKV_SEG_BITMAP;
    const int gs = E.group;
    const size_t rec = (size_t)record_bytes(E.kind, r, ST::bytes, gs);
    const char *base = static_cast<const char *>(E.data) + ((size_t)g * E.nbcap + blk) * rec;
    const bits_t *kv = reinterpret_cast<const bits_t *>(base);
    const uint8_t *ki = reinterpret_cast<const uint8_t *>(base + (size_t)2 * BT * r * ST::bytes);
    const int nvalid = min(BT, E.filled - blk * BT);
    __shared__ bits_t row[D];
    uint32_t mn0 = 0xFFFFFFFFu, mx0 = 0u, mn1 = 0xFFFFFFFFu, mx1 = 0u;
    for (int t = 0; t < nvalid; ++t) {
        bits_t v0, v1;
        if (bitmap && gs > 1) {
            // channel c is kept with its group c / gs; its rank: gs per kept group before it, plus c % gs
            const uint8_t *gp = ki + (size_t)t * (D / 8 / gs);
            uint64_t gb = 0;
            for (int q = 0; q < D / 8 / gs; ++q) gb |= (uint64_t)gp[q] << (8 * q);
            const int i0 = lane / gs, i1 = (lane + 64) / gs;
            const int r0 = gs * popc64(gb & ((1ull << i0) - 1ull)) + lane % gs;
            const int r1 = gs * popc64(gb & ((i1 >= 64 ? 0ull : (1ull << i1)) - 1ull)) + (lane + 64) % gs;
            v0 = ((gb >> i0) & 1ull) ? kv[t * r + r0] : (bits_t)0;
            v1 = ((gb >> i1) & 1ull) ? kv[t * r + r1] : (bits_t)0;
        } else if (bitmap) {
            // channel c is the rank(c)-th kept element of the token
            const uint64_t *bm = reinterpret_cast<const uint64_t *>(ki + (size_t)t * (D / 8));
            const uint64_t m0 = bm[0], m1 = bm[1];
            const uint64_t below = lanes_below(lane);
            v0 = ((m0 >> lane) & 1ull) ? kv[t * r + popc64(m0 & below)] : (bits_t)0;
            v1 = ((m1 >> lane) & 1ull) ? kv[t * r + popc64(m0) + popc64(m1 & below)] : (bits_t)0;
        } else {
            row[lane] = 0;
            row[lane + 64] = 0;
            wave_lds_sync();
            for (int m = lane; m < r; m += 64) row[ki[t * r + m] & (D - 1)] = kv[t * r + m];
            wave_lds_sync();
            v0 = row[lane];
            v1 = row[lane + 64];
            wave_lds_sync();
        }
        const uint32_t q0 = order_key<ST>(v0), q1 = order_key<ST>(v1);
        mn0 = min(mn0, q0); mx0 = max(mx0, q0);
        mn1 = min(mn1, q1); mx1 = max(mx1, q1);
    }
    const int G16 = 2 * E.kch * ST::bytes / 16;
    const int cpg = 16 / (2 * ST::bytes);
    const int ntile = (E.nbcap + META_TILE - 1) / META_TILE;
    char *tile = static_cast<char *>(E.meta) + ((size_t)g * ntile + blk / META_TILE) * G16 * META_TILE * 16;
    const int bl = blk % META_TILE;
    for (int h = 0; h < 2; ++h) {
        const int c = lane + 64 * h;
        if (c >= E.kch) continue;
        bits_t *pr = reinterpret_cast<bits_t *>(tile + ((size_t)(c / cpg) * META_TILE + bl) * 16 +
                                                (c % cpg) * 2 * ST::bytes);
        pr[0] = key_to_bits<ST>(h == 0 ? mn0 : mn1);
        pr[1] = key_to_bits<ST>(h == 0 ? mx0 : mx1);
    }
}

}  // namespace

hipError_t launch_compress(const CompressArgs &a, int dtype, int max_blk, hipStream_t s) {
    if (a.n_ent <= 0 || max_blk <= 0) return a.q_req > 0 ? hipErrorInvalidValue : hipSuccess;
    const bool small = compress_stages(max_blk);
    // a query rotation rides along only on one-block-chunk launches
    if (a.q_req > 0 && (!small || !a.q || !a.qa || !a.qs || (a.q_G != 1 && a.q_G != 2 && a.q_G != 4) ||
                        a.q_hq != a.q_G * a.n_kv || a.q_ns < 1))
        return hipErrorInvalidValue;
    CompressArgs b = a;
    b.chunk_blocks = small ? 1 : COMPRESS_CHUNK;
    const int nchunk = (max_blk + b.chunk_blocks - 1) / b.chunk_blocks;
    const unsigned gx = (unsigned)std::max(2 * nchunk, a.q_req > 0 ? D / 32 : 0);
    const dim3 grid(gx, (unsigned)a.n_kv, (unsigned)(a.n_ent + std::max(a.q_req, 0)));
    if (dtype == MKV_BF16) {
        if (small) hipLaunchKernelGGL(k_compress<Bf16>, grid, dim3(256), 0, s, b);
        else hipLaunchKernelGGL(k_compress_bulk<Bf16>, grid, dim3(64 * BULK_WAVES), 0, s, b);
    } else {
        if (small) hipLaunchKernelGGL(k_compress<F32>, grid, dim3(256), 0, s, b);
        else hipLaunchKernelGGL(k_compress_bulk<F32>, grid, dim3(64 * BULK_WAVES), 0, s, b);
    }
    return hipGetLastError();
}

hipError_t launch_block_meta(const MetaArgs &a, int dtype, int max_nb, hipStream_t s) {
    if (a.n_ent <= 0 || max_nb <= 0) return hipSuccess;
    const dim3 grid((unsigned)max_nb, (unsigned)a.n_kv, (unsigned)a.n_ent);
    if (dtype == MKV_BF16)
        hipLaunchKernelGGL(k_block_meta<Bf16>, grid, dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL(k_block_meta<F32>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace mkv
