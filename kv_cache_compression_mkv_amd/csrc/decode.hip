// Decode attention computed straight from the compressed cache.
//
// Steps ("MosaicKV 阅读笔记" reading notes Eq. 12-14; paper summary sections
// 4.2 and 5.3, and the reading notes' Quest paragraph for the block keys):
//   q_rotate      : q' = R_k q for the G query heads of a KV head
//   score         : s_l = (1/sqrt d) sum_c max(q'_c mx_c, q'_c mn_c) per block
//   select        : per query head and packed segment, the k best blocks
//                   (ties to the lower block), plus a per-block head mask
//   attend        : split-KV attention over the dense (sink / recent) blocks
//                   and the union of the group's selected packed blocks
//   merge         : log-sum-exp merge of every split, then out = o R_v
//
// All of it is bandwidth-bound gather work: every kernel runs on the vector
// ALU (no MFMA); meta and record reads are 16-byte coalesced loads.
#include <math.h>

#include "device_util.hpp"
#include "mkv_internal.h"
#include "qrot.hpp"

namespace mkv {

namespace {

// 2^x with the hardware exponential (results below the smallest normal float
// flush to zero, which softmax weights tolerate: they are at most 2^8 times
// the running maximum's weight and such tiny ones do not change any sum)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ const DSeg &seg_of(const DecodeArgs &A, int bl, int si) {
    return A.seg[bl * A.nseg + si];
}

// packed j of a request takes the sliced select (nb > BIG_SEL_MIN)
__device__ __forceinline__ bool sliced(const DecodeArgs &A, int j, const DSeg &S) {
    return A.big_row[j] >= 0 && S.nb > BIG_SEL_MIN;
}

// ----------------------------------------------------------------------------
// q_rotate: four workgroups per (request, KV head), 32 channels each.
// ----------------------------------------------------------------------------
// the rotations [n_kv][2][D][D] of rotation slot `slot` for request bl of the
// launch: the cache's for slot 0 and for requests whose segment of that slot
// has no rotation of its own, else the segment's
__device__ __forceinline__ const float *slot_rot(const DecodeArgs &A, int bl, int slot) {
    const float *own = nullptr;
    if (slot > 0)
        for (int j = 0; j < A.nseg; ++j) {
            const DSeg &S = seg_of(A, bl, j);
            if (S.slot == slot) own = S.rot;
        }
    return own ? own : A.rot + (size_t)(A.b0 + bl) * A.hkv * 2 * D * D;
}

// q' of every rotation slot from qrot_from on: grid z = request * nslot + slot
template <int G>
__global__ __launch_bounds__(256) void k_qrot(const DecodeArgs A) {
    __shared__ __align__(16) float qsh[G][D];
    const int bl = (int)blockIdx.z / A.nslot, slot = (int)blockIdx.z % A.nslot;
    if (slot < A.qrot_from) return;
    const int b = A.b0 + bl;
    qrot_block<G>(slot_rot(A, bl, slot), A.q + (size_t)b * A.hq * D, A.qa + ((size_t)b * A.nslot + slot) * A.hq * D,
                  A.qs + ((size_t)b * A.nslot + slot) * A.hkv * D * 2 * G, (int)blockIdx.y, (int)blockIdx.x, qsh);
}

// DPP row (16-lane) reductions on integers; every lane of the row gets the result
#define MKV_RORI(v, ctrl) __builtin_amdgcn_update_dpp(0, (v), ctrl, 0xf, 0xf, false)
__device__ __forceinline__ int row_sum16_i(int v) {
    v += MKV_RORI(v, 0x121);
    v += MKV_RORI(v, 0x122);
    v += MKV_RORI(v, 0x124);
    v += MKV_RORI(v, 0x128);
    return v;
}
__device__ __forceinline__ uint32_t row_min16_u(uint32_t v) {
    v = min(v, (uint32_t)MKV_RORI((int)v, 0x121));
    v = min(v, (uint32_t)MKV_RORI((int)v, 0x122));
    v = min(v, (uint32_t)MKV_RORI((int)v, 0x124));
    v = min(v, (uint32_t)MKV_RORI((int)v, 0x128));
    return v;
}
__device__ __forceinline__ uint32_t row_max16_u(uint32_t v) {
    v = max(v, (uint32_t)MKV_RORI((int)v, 0x121));
    v = max(v, (uint32_t)MKV_RORI((int)v, 0x122));
    v = max(v, (uint32_t)MKV_RORI((int)v, 0x124));
    v = max(v, (uint32_t)MKV_RORI((int)v, 0x128));
    return v;
}
#undef MKV_RORI
__device__ __forceinline__ int lane_int(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// wave-uniform min / max of a per-lane value
__device__ __forceinline__ void wave_minmax_u(uint32_t &mn, uint32_t &mx) {
    const uint32_t a = row_min16_u(mn), b = row_max16_u(mx);
    mn = min(min((uint32_t)lane_int((int)a, 0), (uint32_t)lane_int((int)a, 16)),
             min((uint32_t)lane_int((int)a, 32), (uint32_t)lane_int((int)a, 48)));
    mx = max(max((uint32_t)lane_int((int)b, 0), (uint32_t)lane_int((int)b, 16)),
             max((uint32_t)lane_int((int)b, 32), (uint32_t)lane_int((int)b, 48)));
}

// ----------------------------------------------------------------------------
// score: one wave per tile of 64 blocks, one lane per block. The tile's keys
// are stored channel-group-major, so each 16-byte load of the wave covers
// 1 KB of contiguous meta. q' enters as wave-uniform (scalar) operands split
// into positive and negative parts: max(q mx, q mn) = q+ mx + q- mn. A
// segment whose keys cover its leading kch channels reads and sums only those
// groups.
// ----------------------------------------------------------------------------
// acc[i] = sum over the ng key groups of head i's q'+ mx + q'- mn (NGC > 0:
// ng == NGC, known at compile time)
template <typename ST, int G, int NGC>
__device__ __forceinline__ void score_groups(const uint4 *mt, const float *__restrict__ qs, int lane, float (&acc)[G],
                                             int ng) {
    constexpr int CPG = 16 / (2 * ST::bytes);
    if constexpr (NGC > 0) ng = NGC;
#pragma unroll
    for (int i = 0; i < G; ++i) acc[i] = 0.f;
#pragma unroll 8
    for (int grp = 0; grp < ng; ++grp) {
        const uint4 w = mt[grp * META_TILE + lane];
        float mn[CPG], mx[CPG];
        if constexpr (ST::bytes == 2) {
            mn[0] = bf16_lo(w.x); mx[0] = bf16_hi(w.x);
            mn[1] = bf16_lo(w.y); mx[1] = bf16_hi(w.y);
            mn[2] = bf16_lo(w.z); mx[2] = bf16_hi(w.z);
            mn[3] = bf16_lo(w.w); mx[3] = bf16_hi(w.w);
        } else {
            mn[0] = __uint_as_float(w.x); mx[0] = __uint_as_float(w.y);
            mn[1] = __uint_as_float(w.z); mx[1] = __uint_as_float(w.w);
        }
#pragma unroll
        for (int cc = 0; cc < CPG; ++cc) {
            const float *qc = qs + (size_t)(grp * CPG + cc) * 2 * G;
#pragma unroll
            for (int i = 0; i < G; ++i) {
                acc[i] = fmaf(qc[i], mx[cc], acc[i]);
                acc[i] = fmaf(qc[G + i], mn[cc], acc[i]);
            }
        }
    }
}

template <typename ST, int G>
__device__ __forceinline__ void score_tile(const DecodeArgs &A, int bl, int j, int g, int tile) {
    const int b = A.b0 + bl;
    const DSeg &S = seg_of(A, bl, A.pseg[j]);
    const int lane = lane_id();
    const int ntile = (S.nb + META_TILE - 1) / META_TILE;
    if (tile >= ntile) return;
    const int l = tile * META_TILE + lane;
    constexpr int CPG = 16 / (2 * ST::bytes);   // channels per 16-byte group
    const int ng = S.kch / CPG;                 // groups per block
    const int ntile_cap = (S.nbcap + META_TILE - 1) / META_TILE;
    const uint4 *mt = reinterpret_cast<const uint4 *>(static_cast<const char *>(S.meta) +
                                                      ((size_t)g * ntile_cap + tile) * ng * META_TILE * 16);
    const float *__restrict__ qs = A.qs + ((((size_t)b * A.nslot + S.slot) * A.hkv + g) * D) * 2 * G;
    float acc[G];
    // full keys: a compile-time trip count, as the common case; compressed keys: a run-time one
    constexpr int NG_FULL = D / CPG;
    if (ng == NG_FULL) score_groups<ST, G, NG_FULL>(mt, qs, lane, acc, NG_FULL);
    else score_groups<ST, G, 0>(mt, qs, lane, acc, ng);
    if (l < S.nb) {
        const int nbc = A.nbcap[j];
#pragma unroll
        for (int i = 0; i < G; ++i)
            A.scores[A.sc_off[j] + ((size_t)b * A.hq + g * G + i) * nbc + l] = acc[i];
        A.mask[A.mk_off[j] + ((size_t)b * A.hkv + g) * nbc + l] = 0u;
    }
    if (sliced(A, j, S)) {
        // the sliced select's inputs: each tile's key range per head, and
        // (tile 0) cleared histogram and candidate state of the group's heads
        const int ntc = (A.nbcap[j] + META_TILE - 1) / META_TILE;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const bool valid = l < S.nb;
            uint32_t mn = valid ? score_key(acc[i]) : 0xFFFFFFFFu, mx = valid ? score_key(acc[i]) : 0u;
            wave_minmax_u(mn, mx);
            uint32_t *tm = A.tmm + A.tm_off[j] + (((size_t)b * A.hq + g * G + i) * ntc + tile) * 2;
            if (lane == 0) {
                tm[0] = mn;
                tm[1] = mx;
            }
        }
        if (tile == 0) {
#pragma unroll
            for (int i = 0; i < G; ++i) {
                BigRow &R = A.big[A.big_row[j] + (size_t)b * A.hq + g * G + i];
                uint4 *hv = reinterpret_cast<uint4 *>(R.hist);
                for (int q = lane; q < BSEL_BINS / 4; q += 64) hv[q] = make_uint4(0u, 0u, 0u, 0u);
                if (lane == 0) {
                    R.bmn = 0xFFFFFFFFu;
                    R.bmx = 0u;
                    R.ncand = 0u;
                }
            }
        }
    }
}

constexpr int SEL_MAX_WAVES = 16;


// Cross-wave helpers (nw <= 16 waves): after the barrier, lane i of every
// wave reads wave i's entry and a DPP row reduction combines them.
// sum three wave-uniform values over the workgroup's waves
template <class SH>
__device__ __forceinline__ void xwave_sum3(SH &sh, int &ph, int nw, int &a, int &b, int &c) {
    if (nw == 1) return;
    const int w = (int)(threadIdx.x >> 6), lane = lane_id();
    if (lane == 0) {
        sh.v[ph][w][0] = a;
        sh.v[ph][w][1] = b;
        sh.v[ph][w][2] = c;
    }
    __syncthreads();
    // DPP row i (lanes 16 i .. 16 i + 15) sums value i over the waves
    const int wi = lane & 15, vi = lane >> 4;
    const int x = (vi < 3 && wi < nw) ? sh.v[ph][wi][vi] : 0;
    const int t = row_sum16_i(x);
    a = lane_int(t, 0);
    b = lane_int(t, 16);
    c = lane_int(t, 32);
    ph ^= 1;
}

// exclusive prefix over waves of a wave-uniform value
template <class SH>
__device__ __forceinline__ int xwave_excl(SH &sh, int &ph, int nw, int v) {
    if (nw == 1) return 0;
    const int w = (int)(threadIdx.x >> 6), lane = lane_id();
    if (lane == 0) sh.v[ph][w][0] = v;
    __syncthreads();
    const int x = lane < w ? sh.v[ph][lane][0] : 0;
    ph ^= 1;
    return lane_int(row_sum16_i(x), 0);
}

template <class SH>
__device__ __forceinline__ void xwave_minmax(SH &sh, int &ph, int nw, uint32_t &mn, uint32_t &mx) {
    wave_minmax_u(mn, mx);
    if (nw == 1) return;
    const int w = (int)(threadIdx.x >> 6), lane = lane_id();
    if (lane == 0) {
        sh.v[ph][w][0] = (int)mn;
        sh.v[ph][w][1] = (int)mx;
    }
    __syncthreads();
    uint32_t a = 0xFFFFFFFFu, b = 0u;
    if (lane < nw) {
        a = (uint32_t)sh.v[ph][lane][0];
        b = (uint32_t)sh.v[ph][lane][1];
    }
    mn = (uint32_t)lane_int((int)row_min16_u(a), 0);
    mx = (uint32_t)lane_int((int)row_max16_u(b), 0);
    ph ^= 1;
}

template <int KPT>
__device__ __forceinline__ int count_ge(const uint32_t (&key)[KPT], uint32_t cand) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) n += popc64(ballot(key[i] >= cand));
    return n;
}

// The nact (1..64) keys in [thr, thr + 2^(bit + 1)) go to LDS; wave 0 then
// finds, bit by bit with ballots and no barriers, the threshold t in that
// range with at least need of them >= t (largest such t, or one with exactly
// need), and every wave gets it back. With cnt_hi keys above the range and
// need = k - cnt_hi this is the threshold the workgroup-wide search reaches.
template <int KPT, class SH>
__device__ __forceinline__ uint32_t select_compact(SH &sh, int &ph, int nw, const uint32_t (&key)[KPT],
                                                   uint32_t thr, int bit, int nact, int need) {
    const int wave = (int)(threadIdx.x >> 6), lane = lane_id();
    const int sft = bit + 1;  // 1..31
    const uint32_t pre = thr >> sft;
    int cw = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) cw += popc64(ballot((key[i] >> sft) == pre));
    int base = xwave_excl(sh, ph, nw, cw);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const bool a = (key[i] >> sft) == pre;
        const uint64_t m = ballot(a);
        const int at = base + rank_below(m);
        if (a && at < 64) sh.act[at] = key[i];  // (never 64 or more: nact <= 64)
        base += popc64(m);
    }
    __syncthreads();
    if (wave == 0) {
        // inactive lanes hold 0, below every candidate (thr > 0)
        const uint32_t x = lane < nact ? sh.act[lane] : 0u;
        uint32_t t = thr;
        int c = nact, b = bit;
        while (b >= 0 && c != need) {
            if (b >= 1) {
                const uint32_t c1 = t | (1u << (b - 1)), c2 = t | (2u << (b - 1)), c3 = t | (3u << (b - 1));
                const int n1 = popc64(ballot(x >= c1)), n2 = popc64(ballot(x >= c2)), n3 = popc64(ballot(x >= c3));
                if (n3 >= need) { t = c3; c = n3; }
                else if (n2 >= need) { t = c2; c = n2; }
                else if (n1 >= need) { t = c1; c = n1; }
                b -= 2;
            } else {
                const int n1 = popc64(ballot(x >= (t | 1u)));
                if (n1 >= need) { t |= 1u; c = n1; }
                b -= 1;
            }
        }
        if (lane == 0) sh.thr = t;
    }
    __syncthreads();
    return sh.thr;
}

// Exact threshold of the k largest keys, 2 bits at a time, over keys known to
// lie in [kmn, kmx] from the k-th largest on (every key above kmx counts as
// kept): the largest t with at least k keys >= t. Counting uses ballots and
// one cross-wave sum per step; once at most 64 keys remain undecided one wave
// finishes with ballots and no barriers.
template <int KPT, class SH>
__device__ __forceinline__ uint32_t radix_threshold(SH &sh, int &ph, int nw, const uint32_t (&key)[KPT], uint32_t kmn,
                                                    uint32_t kmx, int k) {
    const uint32_t diff = kmn ^ kmx;
    int bit = diff ? 31 - __clz(diff) : -1;
    uint32_t thr = diff ? (kmx & ~((bit == 31) ? 0xFFFFFFFFu : ((2u << bit) - 1u))) : kmx;
    // Invariant: at least k keys are >= thr. Once exactly k are (cnt == k)
    // they are the selection, and the remaining bits cannot change it.
    // cnt_hi counts the keys at or above the range's upper end
    // thr + 2^(bit + 1), all of which are kept.
    // keys at or above the range's upper end (none when [kmn, kmx] spans
    // every key; keys of higher bins otherwise)
    const uint64_t upper = (uint64_t)thr + (bit >= 0 ? (2ull << bit) : 1ull);
    int cnt = -1, cnt_hi = upper > 0xFFFFFFFFull ? 0 : count_ge<KPT>(key, (uint32_t)upper);
    {
        int u1 = 0, u2 = 0;
        xwave_sum3(sh, ph, nw, cnt_hi, u1, u2);
    }
    while (bit >= 0 && cnt != k) {
        if (bit >= 1) {
            const uint32_t c1 = thr | (1u << (bit - 1)), c2 = thr | (2u << (bit - 1)), c3 = thr | (3u << (bit - 1));
            int n1 = count_ge<KPT>(key, c1), n2 = count_ge<KPT>(key, c2), n3 = count_ge<KPT>(key, c3);
            xwave_sum3(sh, ph, nw, n1, n2, n3);
            if (n3 >= k) { thr = c3; cnt = n3; }
            else if (n2 >= k) { thr = c2; cnt = n2; cnt_hi = n3; }
            else if (n1 >= k) { thr = c1; cnt = n1; cnt_hi = n2; }
            else cnt_hi = n1;
            bit -= 2;
        } else {
            int n1 = count_ge<KPT>(key, thr | 1u), n2 = 0, n3 = 0;
            xwave_sum3(sh, ph, nw, n1, n2, n3);
            if (n1 >= k) { thr |= 1u; cnt = n1; }
            else cnt_hi = n1;
            bit -= 1;
        }
        // at most 64 keys left undecided: one wave finishes the search
        if (nw > 1 && bit >= 0 && cnt > k && cnt - cnt_hi <= 64) {
            thr = select_compact<KPT>(sh, ph, nw, key, thr, bit, cnt - cnt_hi, k - cnt_hi);
            break;
        }
    }
    return thr;
}

// the score of an order key (inverse of score_key)
__device__ __forceinline__ float key_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// bin of a score between smin and smax: monotone in the score (a subtraction,
// a product by a positive factor and a truncation each preserve order), so
// every key of a higher bin exceeds every key of a lower one
__device__ __forceinline__ int score_bin(uint32_t key, float smin, float inv) {
    return min(255, (int)((key_score(key) - smin) * inv));
}

// ----------------------------------------------------------------------------
// select: one workgroup of up to 16 waves per (request, query head, packed
// segment). Lane l of wave w holds the keys of blocks (w * KPT + i) * 64 + l,
// so block order is (wave, i, lane) order. The k-th largest score is located
// in one histogram pass: scores are binned linearly between their minimum
// and maximum into 256 bins (per-wave histograms, LDS atomics), and one wave
// finds the bin holding the k-th largest from the top. Usually that bin's
// keys are all needed, or at most 64 of them remain; those are compacted to
// LDS and one wave finds the exact threshold with ballots. Otherwise (many
// near-equal scores) the exact 2-bit search runs from that bin's key range.
// Blocks above the threshold are kept, equal ones by ascending block index;
// ballot prefix counts give each kept block its place in the ascending output.
// ----------------------------------------------------------------------------
struct SelShared {
    int v[2][SEL_MAX_WAVES][3];
    uint32_t hist[SEL_MAX_WAVES][256];  // one histogram per wave (no cross-wave atomics)
    uint32_t act[64];                   // candidate keys handed to one wave
    uint32_t thr;
    int res[3];                         // bin, keys above it, keys in it
    int ncand;
};

template <int G, int KPT>
__global__ __launch_bounds__(1024) void k_select(const DecodeArgs A) {
    const int z = (int)blockIdx.z;
    const int bl = z / A.npk, j = z % A.npk;
    const int b = A.b0 + bl, g = (int)blockIdx.y, hi = (int)blockIdx.x;
    const int h = g * G + hi;
    const DSeg &S = seg_of(A, bl, A.pseg[j]);
    if (sliced(A, j, S)) return;
    const int n = S.nb, k = S.k;
    const int nbc = A.nbcap[j];
    const int nw = (int)(blockDim.x >> 6), lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    __shared__ SelShared sh;
    int ph = 0;

    // sel_out column offset of this packed segment for this request
    int coloff = 0;
    for (int jj = 0; jj < j; ++jj) coloff += seg_of(A, bl, A.pseg[jj]).k;
    int32_t *so = A.sel_out ? A.sel_out + ((size_t)b * A.hq + h) * A.sel_cols : nullptr;
    if (so && j == A.npk - 1) {
        for (int64_t c = coloff + k + (int)threadIdx.x; c < A.sel_cols; c += blockDim.x) so[c] = -1;
    }
    if (n <= 0 || k <= 0) return;

    // keys; 0 marks a missing block (every finite score has a key above
    // 0x007FFFFF). Every load is issued first (lanes past the last block
    // reread it), so they are in flight together.
    const float *sc = A.scores + A.sc_off[j] + ((size_t)b * A.hq + h) * nbc;
    uint32_t key[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) key[i] = __float_as_uint(sc[min((w * KPT + i) * 64 + lane, n - 1)]);
    for (int i = (int)threadIdx.x; i < nw * 256; i += (int)blockDim.x) (&sh.hist[0][0])[i] = 0u;
    if (threadIdx.x == 0) sh.ncand = 0;
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const bool valid = (w * KPT + i) * 64 + lane < n;
        key[i] = valid ? score_key(__uint_as_float(key[i])) : 0u;
        if (valid) {
            kmn = min(kmn, key[i]);
            kmx = max(kmx, key[i]);
        }
    }
    xwave_minmax(sh, ph, nw, kmn, kmx);
    if (nw == 1) wave_lds_sync();

    // Kept: every key above thr and the first (k - #above) equal to thr in
    // block order; or, when by_bin, every key in bin bstar or above.
    uint32_t thr = kmn;
    bool by_bin = false;
    int bstar = 0;
    float smin = 0.f, inv = 0.f;
    if (k < n && kmn != kmx) {
        smin = key_score(kmn);
        const float range = key_score(kmx) - smin;
        inv = 256.f / range;
        if (range > 0.f && inv > 0.f && inv < 3.0e38f) {
            uint32_t *hist = sh.hist[w];
#pragma unroll
            for (int i = 0; i < KPT; ++i)
                if (key[i] != 0u) atomicAdd(&hist[score_bin(key[i], smin, inv)], 1u);
            __syncthreads();
            if (w == 0) {
                // lane holds bins 4 lane .. 4 lane + 3, summed over the waves
                uint4 hv = make_uint4(0u, 0u, 0u, 0u);
                for (int v = 0; v < nw; ++v) {
                    const uint4 x = reinterpret_cast<const uint4 *>(sh.hist[v])[lane];
                    hv.x += x.x;
                    hv.y += x.y;
                    hv.z += x.z;
                    hv.w += x.w;
                }
                const uint32_t tot = hv.x + hv.y + hv.z + hv.w;
                uint32_t suf = tot;  // keys in the bins of lanes >= lane
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t y = __shfl_down(suf, o, 64);
                    if (lane + o < 64) suf += y;
                }
                const uint32_t a3 = suf - tot, s3 = a3 + hv.w, s2 = s3 + hv.z, s1 = s2 + hv.y, s0 = s1 + hv.x;
                // highest bin whose keys and those above it reach k
                const uint64_t m = ballot(s0 >= (uint32_t)k);
                const int L = 63 - __clzll(m);
                if (lane == L) {
                    int bin;
                    uint32_t above, cnt;
                    if (s3 >= (uint32_t)k) { bin = 4 * L + 3; above = a3; cnt = hv.w; }
                    else if (s2 >= (uint32_t)k) { bin = 4 * L + 2; above = s3; cnt = hv.z; }
                    else if (s1 >= (uint32_t)k) { bin = 4 * L + 1; above = s2; cnt = hv.y; }
                    else { bin = 4 * L; above = s1; cnt = hv.x; }
                    sh.res[0] = bin;
                    sh.res[1] = (int)above;
                    sh.res[2] = (int)cnt;
                }
            }
            __syncthreads();
            bstar = sh.res[0];
            const int above = sh.res[1], cnt = sh.res[2], need = k - above;
            if (cnt == need) {
                by_bin = true;
            } else if (cnt <= 64) {
                // the need-th largest of the bin's keys, found by one wave
#pragma unroll
                for (int i = 0; i < KPT; ++i)
                    if (key[i] != 0u && score_bin(key[i], smin, inv) == bstar) sh.act[atomicAdd(&sh.ncand, 1)] = key[i];
                __syncthreads();
                if (w == 0) {
                    const uint32_t x = lane < cnt ? sh.act[lane] : 0u;  // candidates are > 0
                    uint32_t t = 0u;
                    for (int bit = 31; bit >= 0; --bit) {
                        const uint32_t c = t | (1u << bit);
                        if (popc64(ballot(x >= c)) >= need) t = c;
                    }
                    if (lane == 0) sh.thr = t;
                }
                __syncthreads();
                thr = sh.thr;
            } else {
                // many near-equal scores: exact search over the bin's key range
                uint32_t cmn = 0xFFFFFFFFu, cmx = 0u;
#pragma unroll
                for (int i = 0; i < KPT; ++i)
                    if (key[i] != 0u && score_bin(key[i], smin, inv) == bstar) {
                        cmn = min(cmn, key[i]);
                        cmx = max(cmx, key[i]);
                    }
                xwave_minmax(sh, ph, nw, cmn, cmx);
                thr = radix_threshold<KPT>(sh, ph, nw, key, cmn, cmx, k);
            }
        } else {
            thr = radix_threshold<KPT>(sh, ph, nw, key, kmn, kmx, k);
        }
    }
    const uint64_t below = lanes_below(lane);
    uint64_t selm = 0;
    if (by_bin || k >= n) {
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if (key[i] != 0u && (k >= n || score_bin(key[i], smin, inv) >= bstar)) selm |= 1ull << i;
    } else {
        int ngt = 0, neq = 0, unused = 0;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            ngt += popc64(ballot(key[i] > thr));
            neq += popc64(ballot(key[i] == thr));
        }
        xwave_sum3(sh, ph, nw, ngt, neq, unused);
        const int need = k - ngt;
        if (neq <= need) {
#pragma unroll
            for (int i = 0; i < KPT; ++i)
                if (key[i] >= thr) selm |= 1ull << i;
        } else {
            int eqw = 0;
#pragma unroll
            for (int i = 0; i < KPT; ++i) eqw += popc64(ballot(key[i] == thr));
            int run = xwave_excl(sh, ph, nw, eqw);
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const uint64_t em = ballot(key[i] == thr);
                const int rank = run + popc64(em & below);
                if (key[i] > thr || (key[i] == thr && rank < need)) selm |= 1ull << i;
                run += popc64(em);
            }
        }
    }
    int cw = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) cw += popc64(ballot((selm >> i) & 1));
    int base = xwave_excl(sh, ph, nw, cw);
    int32_t *sl = A.sel + A.sl_off[j] + ((size_t)b * A.hq + h) * A.kcap[j];
    uint32_t *mk = A.mask + A.mk_off[j] + ((size_t)b * A.hkv + g) * nbc;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const bool sel = (selm >> i) & 1;
        const uint64_t m = ballot(sel);
        if (sel) {
            const int pos = base + popc64(m & below);
            if (pos < k) {
                const int blk = (w * KPT + i) * 64 + lane;
                sl[pos] = blk;
                if (so) so[coloff + pos] = blk;
                reinterpret_cast<uint8_t *>(mk + blk)[hi] = 1;  // byte hi: head hi chose it
            }
        }
        base += popc64(m);
    }
}

// ----------------------------------------------------------------------------
// Sliced select of a large packed segment (more than BIG_SEL_MIN blocks): one
// workgroup of 4 waves per (slice of BSL blocks, request, query head). Lane l
// of wave w holds the keys of blocks s BSL + (16 w + i) 64 + l, so block order
// is (slice, wave, i, lane) order.
//   1. histogram: the segment's key range [kmin, kmax] comes from the score
//      pass's per-tile ranges; keys fall into BSEL_BINS bins of width
//      2^sft in key space (monotone in the score); each slice adds its
//      counts to the row's histogram.
//   2. candidates: every slice finds the same threshold bin (the highest bin
//      whose keys and those above it reach k), records its own counts above
//      and in that bin, and appends its keys of the bin to the candidates.
//   3. output: every slice derives the same exact threshold (the k-th largest
//      key) from the candidates, the counts of the slices before it give its
//      first output position, and ties at the threshold go to the lowest
//      blocks; kept blocks are written in ascending order.
// ----------------------------------------------------------------------------
constexpr int BSEL_KPT = BSL / 256;

// shift of the key-space bins: (kmax - kmin) >> sft < BSEL_BINS
__device__ __forceinline__ int bsel_shift(uint32_t span) {
    const int bits = span ? 32 - __clz(span) : 0;
    return max(0, bits - 11);
}

struct BselRow {
    int z, bl, j, b, h, s, n, k;
    const DSeg *S;
};

// the launch's (slice, request, head, segment) of this workgroup; false when
// the segment does not take the sliced select
__device__ __forceinline__ bool bsel_row(const DecodeArgs &A, BselRow &r) {
    r.z = (int)blockIdx.z;
    r.bl = r.z / A.npk;
    r.j = r.z % A.npk;
    r.b = A.b0 + r.bl;
    r.h = (int)blockIdx.y;
    r.s = (int)blockIdx.x;
    r.S = &seg_of(A, r.bl, A.pseg[r.j]);
    r.n = r.S->nb;
    r.k = r.S->k;
    return sliced(A, r.j, *r.S);
}

// this slice's keys (0 for blocks past the segment's end); every load is
// issued before any is used
__device__ __forceinline__ void bsel_keys(const DecodeArgs &A, const BselRow &r, uint32_t (&key)[BSEL_KPT]) {
    const int w = (int)(threadIdx.x >> 6), lane = lane_id();
    const float *sc = A.scores + A.sc_off[r.j] + ((size_t)r.b * A.hq + r.h) * A.nbcap[r.j];
    const int base = r.s * BSL + w * BSEL_KPT * 64 + lane;
#pragma unroll
    for (int i = 0; i < BSEL_KPT; ++i) key[i] = __float_as_uint(sc[min(base + i * 64, r.n - 1)]);
#pragma unroll
    for (int i = 0; i < BSEL_KPT; ++i) key[i] = base + i * 64 < r.n ? score_key(__uint_as_float(key[i])) : 0u;
}

struct BselHistShared {
    int v[2][SEL_MAX_WAVES][3];
    uint32_t hist[BSEL_BINS];
};

template <int G>
__global__ __launch_bounds__(256) void k_bsel_hist(const DecodeArgs A) {
    BselRow r;
    if (!bsel_row(A, r) || r.k >= r.n || r.s * BSL >= r.n) return;
    BigRow &R = A.big[A.big_row[r.j] + (size_t)r.b * A.hq + r.h];
    __shared__ BselHistShared sh;
    int ph = 0;
    const int tid = (int)threadIdx.x;
    uint32_t key[BSEL_KPT];
    bsel_keys(A, r, key);
    // key range of the whole segment from its tiles' ranges
    const int ntile = (r.n + META_TILE - 1) / META_TILE, ntc = (A.nbcap[r.j] + META_TILE - 1) / META_TILE;
    const uint32_t *tm = A.tmm + A.tm_off[r.j] + ((size_t)r.b * A.hq + r.h) * ntc * 2;
    static_assert(MKV_MAX_PACKED_BLOCKS / META_TILE <= 4 * 256, "four tiles per thread at most");
    uint2 tv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) tv[q] = reinterpret_cast<const uint2 *>(tm)[min(tid + 256 * q, ntile - 1)];
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        kmn = min(kmn, tv[q].x);  // (repeated tiles change nothing)
        kmx = max(kmx, tv[q].y);
    }
    xwave_minmax(sh, ph, 4, kmn, kmx);
    if (r.s == 0 && tid == 0) {
        R.kmin = kmn;
        R.kmax = kmx;
    }
    if (kmn == kmx) return;  // every key equal: the output pass needs no histogram
    const int sft = bsel_shift(kmx - kmn);
    for (int i = tid; i < BSEL_BINS; i += 256) sh.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BSEL_KPT; ++i)
        if (key[i] != 0u) atomicAdd(&sh.hist[(key[i] - kmn) >> sft], 1u);
    __syncthreads();
    for (int i = tid; i < BSEL_BINS; i += 256) {
        const uint32_t c = sh.hist[i];
        if (c) atomicAdd(&R.hist[i], c);
    }
}

struct BselCandShared {
    int v[2][SEL_MAX_WAVES][3];
    int res[3];
};

template <int G>
__global__ __launch_bounds__(256) void k_bsel_cand(const DecodeArgs A) {
    BselRow r;
    if (!bsel_row(A, r) || r.k >= r.n || r.s * BSL >= r.n) return;
    BigRow &R = A.big[A.big_row[r.j] + (size_t)r.b * A.hq + r.h];
    __shared__ BselCandShared sh;
    int ph = 0;
    const int tid = (int)threadIdx.x, lane = lane_id(), w = (int)(threadIdx.x >> 6);
    // keys, key range and histogram are requested together
    uint32_t key[BSEL_KPT];
    bsel_keys(A, r, key);
    const uint2 kr = *reinterpret_cast<const uint2 *>(&R.kmin);
    const uint4 *hv = reinterpret_cast<const uint4 *>(R.hist) + 2 * tid;
    const uint4 x0 = hv[0], x1 = hv[1];
    const uint32_t kmn = kr.x, kmx = kr.y;
    if (kmn == kmx) return;
    // threshold bin: thread t holds bins 8t .. 8t + 7; suffix sums from the top
    uint32_t hb[8];
    hb[0] = x0.x; hb[1] = x0.y; hb[2] = x0.z; hb[3] = x0.w;
    hb[4] = x1.x; hb[5] = x1.y; hb[6] = x1.z; hb[7] = x1.w;
    int tsum = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) tsum += (int)hb[q];
    int suf = tsum;  // inclusive suffix within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += y;
    }
    if (lane == 0) sh.v[ph][w][0] = suf;  // the wave's total
    __syncthreads();
    int above_w = 0;
    for (int v = w + 1; v < 4; ++v) above_w += sh.v[ph][v][0];
    int run = suf - tsum + above_w;  // keys in the bins of higher threads
#pragma unroll
    for (int q = 7; q >= 0; --q) {
        const int c = (int)hb[q];
        if (run < r.k && run + c >= r.k) {
            sh.res[0] = 8 * tid + q;
            sh.res[1] = run;
            sh.res[2] = c;
        }
        run += c;
    }
    __syncthreads();
    ph ^= 1;
    const int bstar = sh.res[0];
    const int sft = bsel_shift(kmx - kmn);
    const uint64_t below = lanes_below(lane);
    int above_s = 0, in_s = 0;
    uint32_t cmn = 0xFFFFFFFFu, cmx = 0u;
#pragma unroll
    for (int i = 0; i < BSEL_KPT; ++i) {
        const bool valid = key[i] != 0u;
        const int bin = (int)((key[i] - kmn) >> sft);
        above_s += popc64(ballot(valid && bin > bstar));
        const bool inb = valid && bin == bstar;
        const uint64_t m = ballot(inb);
        if (m) {
            const int first = __builtin_ctzll(m);
            uint32_t base = 0u;
            if (lane == first) base = atomicAdd(&R.ncand, (uint32_t)popc64(m));
            base = (uint32_t)__builtin_amdgcn_readlane((int)base, first);
            const uint32_t pos = base + (uint32_t)popc64(m & below);
            if (inb && pos < (uint32_t)BSEL_CAP) {
                R.cand[pos][0] = key[i];
                R.cand[pos][1] = (uint32_t)r.s;
            }
            in_s += popc64(m);
        }
        if (inb) {
            cmn = min(cmn, key[i]);
            cmx = max(cmx, key[i]);
        }
    }
    wave_minmax_u(cmn, cmx);
    if (lane == 0 && cmx != 0u) {
        atomicMin(&R.bmn, cmn);
        atomicMax(&R.bmx, cmx);
    }
    int unused = 0;
    xwave_sum3(sh, ph, 4, above_s, in_s, unused);
    if (tid == 0) {
        R.slc[r.s][0] = above_s;
        R.slc[r.s][1] = in_s;
        if (r.s == 0) {
            R.bstar = bstar;
            R.above = sh.res[1];
            R.inbin = sh.res[2];
        }
    }
}

struct BselOutShared {
    int v[2][SEL_MAX_WAVES][3];
    int slc[BSEL_MAX_SLICES][2];
    uint32_t act[64];
    uint32_t thr;
    int gtc[BSEL_MAX_SLICES], eqc[BSEL_MAX_SLICES];
    int res[2];   // this slice's first output position, its quota of keys equal to the threshold
    uint32_t sub[256];  // candidates per sub-bin of the threshold bin
    int sres[3];        // sub-bin holding the need-th largest candidate, candidates above it, in it
    int nact;
};

// The need-th largest of the n candidate keys ck (thread t holds candidates
// t + 256 i; 0 pads), all in [bmn, bmx]: a 256-bin histogram of the
// candidates locates it; when at most 64 candidates share its sub-bin one
// wave finishes with ballots, else the exact 2-bit search runs.
__device__ __forceinline__ uint32_t bsel_cand_threshold(BselOutShared &sh, int &ph, const uint32_t (&ck)[BSEL_CAP / 256],
                                                        uint32_t bmn, uint32_t bmx, int need) {
    const int tid = (int)threadIdx.x, lane = lane_id(), w = (int)(threadIdx.x >> 6);
    const uint32_t span = bmx - bmn;
    const int bits = span ? 32 - __clz(span) : 0;
    const int sft = max(0, bits - 8);  // span >> sft < 256
    sh.sub[tid] = 0u;
    if (tid == 0) sh.nact = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BSEL_CAP / 256; ++i)
        if (ck[i] != 0u) atomicAdd(&sh.sub[(ck[i] - bmn) >> sft], 1u);
    __syncthreads();
    if (w == 0) {
        // lane holds sub-bins 4 lane .. 4 lane + 3; suffix counts from the top
        const uint4 hv = reinterpret_cast<const uint4 *>(sh.sub)[lane];
        const uint32_t tot = hv.x + hv.y + hv.z + hv.w;
        uint32_t suf = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_down(suf, o, 64);
            if (lane + o < 64) suf += y;
        }
        const uint32_t a3 = suf - tot, s3 = a3 + hv.w, s2 = s3 + hv.z, s1 = s2 + hv.y, s0 = s1 + hv.x;
        const uint64_t m = ballot(s0 >= (uint32_t)need);
        const int L = 63 - __clzll(m);
        if (lane == L) {
            if (s3 >= (uint32_t)need) { sh.sres[0] = 4 * L + 3; sh.sres[1] = (int)a3; sh.sres[2] = (int)hv.w; }
            else if (s2 >= (uint32_t)need) { sh.sres[0] = 4 * L + 2; sh.sres[1] = (int)s3; sh.sres[2] = (int)hv.z; }
            else if (s1 >= (uint32_t)need) { sh.sres[0] = 4 * L + 1; sh.sres[1] = (int)s2; sh.sres[2] = (int)hv.y; }
            else { sh.sres[0] = 4 * L; sh.sres[1] = (int)s1; sh.sres[2] = (int)hv.x; }
        }
    }
    __syncthreads();
    const int sb = sh.sres[0], above = sh.sres[1], cnt = sh.sres[2];
    if (cnt > 64) return radix_threshold<BSEL_CAP / 256>(sh, ph, 4, ck, bmn, bmx, need);
    const int nd = need - above;  // 1 .. cnt
#pragma unroll
    for (int i = 0; i < BSEL_CAP / 256; ++i)
        if (ck[i] != 0u && (int)((ck[i] - bmn) >> sft) == sb) sh.act[atomicAdd(&sh.nact, 1)] = ck[i];
    __syncthreads();
    if (w == 0) {
        const uint32_t x = lane < cnt ? sh.act[lane] : 0u;  // candidates are > 0
        uint32_t t = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = t | (1u << bit);
            if (popc64(ballot(x >= c)) >= nd) t = c;
        }
        if (lane == 0) sh.thr = t;
    }
    __syncthreads();
    return sh.thr;
}

// Keys counted over the whole segment (scores re-read from memory), for the
// rare threshold bins with more than BSEL_CAP keys: number of keys >= cand.
__device__ __forceinline__ int bsel_count_all(const DecodeArgs &A, const BselRow &r, BselOutShared &sh, int &ph,
                                              uint32_t cand) {
    const float *sc = A.scores + A.sc_off[r.j] + ((size_t)r.b * A.hq + r.h) * A.nbcap[r.j];
    int c = 0;
    for (int blk = (int)threadIdx.x; blk < r.n; blk += 256) c += score_key(sc[blk]) >= cand ? 1 : 0;
    const int rs = row_sum16_i(c);
    c = (lane_int(rs, 0) + lane_int(rs, 16)) + (lane_int(rs, 32) + lane_int(rs, 48));
    int u1 = 0, u2 = 0;
    xwave_sum3(sh, ph, 4, c, u1, u2);
    return c;
}

template <int G>
__global__ __launch_bounds__(256) void k_bsel_out(const DecodeArgs A) {
    BselRow r;
    if (!bsel_row(A, r)) return;
    const int n = r.n, k = r.k, j = r.j, b = r.b, h = r.h, s = r.s;
    const int g = h / G, hi = h % G;
    const int tid = (int)threadIdx.x, lane = lane_id(), w = (int)(threadIdx.x >> 6);
    int coloff = 0;
    for (int jj = 0; jj < j; ++jj) coloff += seg_of(A, r.bl, A.pseg[jj]).k;
    int32_t *so = A.sel_out ? A.sel_out + ((size_t)b * A.hq + h) * A.sel_cols : nullptr;
    if (so && j == A.npk - 1 && s == 0)
        for (int64_t c = coloff + k + tid; c < A.sel_cols; c += 256) so[c] = -1;
    if (k <= 0 || s * BSL >= n) return;
    __shared__ BselOutShared sh;
    int ph = 0;
    uint32_t key[BSEL_KPT];
    bsel_keys(A, r, key);
    const BigRow &R = A.big[A.big_row[j] + (size_t)b * A.hq + h];
    const int nsl = (n + BSL - 1) / BSL;
    // the row's header and per-slice counts, requested together
    const uint4 h0 = *reinterpret_cast<const uint4 *>(&R.kmin);   // kmin, kmax, bmn, bmx
    const uint4 h1 = *reinterpret_cast<const uint4 *>(&R.ncand);  // ncand, bstar, above, inbin
    if (tid < nsl && k < n) {
        const int2 c = *reinterpret_cast<const int2 *>(&R.slc[tid][0]);
        sh.slc[tid][0] = c.x;
        sh.slc[tid][1] = c.y;
    }
    // Kept: every valid key when k >= n; the first k blocks when every key is
    // equal; else keys above thr, and keys equal to thr while the slice's
    // quota lasts (by_bin: every key of bin bstar or above).
    int mode = 0;  // 0: all, 1: first k blocks, 2: by bin, 3: threshold
    uint32_t thr = 0u, kmn = 0u;
    int sft = 0, bstar = 0, base = 0, quota = 0;
    __syncthreads();
    if (k < n) {
        kmn = h0.x;
        const uint32_t kmx = h0.y;
        if (kmn == kmx) {
            mode = 1;
        } else {
            sft = bsel_shift(kmx - kmn);
            bstar = (int)h1.y;
            const int need = k - (int)h1.z, inbin = (int)h1.w;
            if (inbin == need) {
                mode = 2;
                if (tid == 0) {
                    int bs = 0;
                    for (int q = 0; q < s; ++q) bs += sh.slc[q][0] + sh.slc[q][1];
                    sh.res[0] = bs;
                }
            } else {
                mode = 3;
                for (int q = tid; q < nsl; q += 256) sh.gtc[q] = sh.eqc[q] = 0;
                const uint32_t bmn = h0.z, bmx = h0.w;
                if (bmn == bmx) {
                    // every key of the bin ties at the threshold
                    thr = bmn;
                    for (int q = tid; q < nsl; q += 256) sh.eqc[q] = sh.slc[q][1];
                } else if (inbin <= BSEL_CAP) {
                    // exact threshold among the candidates (padding keys 0 lie below them)
                    uint32_t ck[BSEL_CAP / 256];
#pragma unroll
                    for (int i = 0; i < BSEL_CAP / 256; ++i) {
                        const int at = tid + 256 * i;
                        ck[i] = at < inbin ? R.cand[at][0] : 0u;
                    }
                    thr = bsel_cand_threshold(sh, ph, ck, bmn, bmx, need);
                    __syncthreads();
#pragma unroll
                    for (int i = 0; i < BSEL_CAP / 256; ++i) {
                        const int at = tid + 256 * i;
                        if (at < inbin) {
                            const int q = min((int)R.cand[at][1], nsl - 1);
                            if (ck[i] > thr) atomicAdd(&sh.gtc[q], 1);
                            else if (ck[i] == thr) atomicAdd(&sh.eqc[q], 1);
                        }
                    }
                } else {
                    // more candidates than stored: bit search over every key of the segment
                    const uint32_t diff = bmn ^ bmx;
                    int bit = 31 - __clz(diff);
                    uint32_t t = bmx & ~((bit == 31) ? 0xFFFFFFFFu : ((2u << bit) - 1u));
                    int cnt = (int)h1.z + inbin;  // keys >= t (every key of the bin is >= bmn >= t)
                    for (; bit >= 0 && cnt != k; --bit) {
                        const uint32_t cand = t | (1u << bit);
                        const int c = bsel_count_all(A, r, sh, ph, cand);
                        if (c >= k) {
                            t = cand;
                            cnt = c;
                        }
                    }
                    thr = t;
                    __syncthreads();
                    const float *sc = A.scores + A.sc_off[j] + ((size_t)b * A.hq + h) * A.nbcap[j];
                    for (int blk = tid; blk < n; blk += 256) {
                        const uint32_t kk = score_key(sc[blk]);
                        const int q = blk / BSL;
                        if (((kk - kmn) >> sft) == (uint32_t)bstar && kk > thr) atomicAdd(&sh.gtc[q], 1);
                        else if (kk == thr) atomicAdd(&sh.eqc[q], 1);
                    }
                }
                __syncthreads();
                if (tid == 0) {
                    int gt_all = 0;
                    for (int q = 0; q < nsl; ++q) gt_all += sh.gtc[q];
                    int left = need - gt_all;  // keys equal to thr still to take, lowest blocks first
                    int bs = 0, mine = 0;
                    for (int q = 0; q <= s; ++q) {
                        const int tq = min(sh.eqc[q], max(left, 0));
                        if (q < s) bs += sh.slc[q][0] + sh.gtc[q] + tq;
                        else mine = tq;
                        left -= tq;
                    }
                    sh.res[0] = bs;
                    sh.res[1] = mine;
                }
            }
        }
    }
    __syncthreads();
    if (mode == 0) base = s * BSL;
    else if (mode == 2 || mode == 3) base = sh.res[0];
    if (mode == 3) quota = sh.res[1];
    const uint64_t below = lanes_below(lane);
    const int blk0 = s * BSL + w * BSEL_KPT * 64 + lane;
    uint32_t selm = 0u;
    if (mode == 3) {
        int eqw = 0;
#pragma unroll
        for (int i = 0; i < BSEL_KPT; ++i) eqw += popc64(ballot(key[i] != 0u && key[i] == thr));
        int erun = xwave_excl(sh, ph, 4, eqw);
#pragma unroll
        for (int i = 0; i < BSEL_KPT; ++i) {
            const bool eq = key[i] != 0u && key[i] == thr;
            const uint64_t em = ballot(eq);
            const int rank = erun + popc64(em & below);
            if (key[i] != 0u && (key[i] > thr || (eq && rank < quota))) selm |= 1u << i;
            erun += popc64(em);
        }
    } else {
#pragma unroll
        for (int i = 0; i < BSEL_KPT; ++i) {
            const bool valid = key[i] != 0u;
            bool kept = valid;
            if (mode == 1) kept = valid && blk0 + i * 64 < k;
            else if (mode == 2) kept = valid && (int)((key[i] - kmn) >> sft) >= bstar;
            if (kept) selm |= 1u << i;
        }
    }
    int cw = 0;
#pragma unroll
    for (int i = 0; i < BSEL_KPT; ++i) cw += popc64(ballot((selm >> i) & 1u));
    if (mode == 1) base = s * BSL;  // the first k blocks: position = block
    int pos0 = base + xwave_excl(sh, ph, 4, cw);
    int32_t *sl = A.sel + A.sl_off[j] + ((size_t)b * A.hq + h) * A.kcap[j];
    uint32_t *mk = A.mask + A.mk_off[j] + ((size_t)b * A.hkv + g) * A.nbcap[j];
#pragma unroll
    for (int i = 0; i < BSEL_KPT; ++i) {
        const bool sel = (selm >> i) & 1u;
        const uint64_t m = ballot(sel);
        if (sel) {
            const int pos = pos0 + popc64(m & below);
            if (pos < k) {
                const int blk = blk0 + i * 64;
                sl[pos] = blk;
                if (so) so[coloff + pos] = blk;
                reinterpret_cast<uint8_t *>(mk + blk)[hi] = 1;
            }
        }
        pos0 += popc64(m);
    }
}

// ----------------------------------------------------------------------------
// shared pieces of the attention kernels
// ----------------------------------------------------------------------------
// Reductions over the 16 lanes of a DPP row (every lane gets the result).
#define MKV_ROR(v, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xf, 0xf, false))
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, MKV_ROR(v, 0x121));
    v = fmaxf(v, MKV_ROR(v, 0x122));
    v = fmaxf(v, MKV_ROR(v, 0x124));
    v = fmaxf(v, MKV_ROR(v, 0x128));
    return v;
}
__device__ __forceinline__ float row_sum16(float v) {
    v += MKV_ROR(v, 0x121);
    v += MKV_ROR(v, 0x122);
    v += MKV_ROR(v, 0x124);
    v += MKV_ROR(v, 0x128);
    return v;
}
#undef MKV_ROR
__device__ __forceinline__ float lane_value(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// ----------------------------------------------------------------------------
// attend: four waves per workgroup, each wave one split of a (request, KV
// head) unit's work. The launch holds two kinds of workgroups: the first
// ceil(S_p / 4) in x take the packed union records, the rest the dense
// blocks, so the dense stream runs beside the latency-bound packed records.
// Every split carries one online softmax state per query head; merge combines
// them.
//
// Packed records: in union mode a workgroup takes an exact byte share of the
// unit's union (blocks some head of the group selected, with the mask of the
// heads that did) and splits it evenly over its waves; otherwise item (rank,
// head) of a packed segment is the rank-th block that head selected, an item
// whose block a lower head of the group also selected is dropped, and items
// are resolved 64 at a time into a compact list. Either way every union block
// is read once and serves each head that chose it.
//
// Dense blocks and packed records both stream through a two-deep register
// pipeline (the next one's loads are in flight while one is computed; a
// deeper pipeline costs more registers than the occupancy it displaces).
//
// Lane (t, p) = (lane / 4, lane % 4) owns part p of token t. For a packed
// record that is elements [p Q, min((p + 1) Q, r)) of the token's r,
// Q = ceil(r / 4), QM >= Q being the compile-time bound: the lane loads
// dword-aligned windows of the four regions of the record that cover its
// elements, so no lane's work crosses a token. For a dense block it is
// channels 32 p .. 32 p + 31 of token t's key.
//   K       z_h(t) = sum of q'_h[c] k_t[c] over the token's four parts (q' in
//           LDS; the parts add with DPP quad permutes);
//   softmax per head, running max over the wave that only moves when a block
//           exceeds it by 2^8 (so rescales are rare), p = exp2(z - m),
//           lane-private running sums;
//   V       lane l accumulates channels 2l, 2l + 1 over the 16 tokens, the
//           p_t broadcast through LDS. Dense rows are read
//           directly; packed values first scatter into the wave's dense tile
//           [16][128] (a token's kept channels are distinct, so no two lanes
//           of one token collide; window bytes past a lane's part go to the
//           lane's slot of a dummy row), which is cleared after use.
// ----------------------------------------------------------------------------
// Online-softmax state. Softmax lanes are head-major: lane h*16 + t holds
// token t of query head h, so each head is one DPP row.
template <int G>
struct WaveState {
    float m;  // running max (log2 units) of the lane's head, uniform within the row
    float l;  // lane-private partial sum of p
    __device__ __forceinline__ void init() {
        m = -INFINITY;
        l = 0.f;
    }
    __device__ __forceinline__ float head_max(int i) const { return lane_value(m, 16 * i); }
    __device__ __forceinline__ float head_sum(int i) const { return lane_value(row_sum16(l), 16 * i); }
};

// One online-softmax step over a block of 16 tokens. z is the logit of lane
// (h, t) = (lane / 16, lane % 16), valid marks real (token, head) pairs. The
// running max only moves when a block exceeds it by more than 2^8, so
// rescales are rare. Writes p to zb[t * G + h]; alpha[i] is head i's rescale.
template <int G>
__device__ __forceinline__ void softmax16(float z, bool valid, float *zb, WaveState<G> &st, float alpha[G]) {
    const int lane = lane_id();
    const float zz = valid ? z : -INFINITY;
    const float bm = row_max16(zz);
    const float mh = st.m;
    float mnew = mh, a = 1.f;
    if (bm != -INFINITY && (mh == -INFINITY || bm > mh + 8.f)) {
        a = (mh == -INFINITY) ? 0.f : fast_exp2(mh - bm);
        mnew = bm;
    }
    const float p = valid ? fast_exp2(zz - mnew) : 0.f;
    if (lane < 16 * G) {
        st.l = st.l * a + p;
        st.m = mnew;
        zb[(lane & 15) * G + (lane >> 4)] = p;
    }
#pragma unroll
    for (int i = 0; i < G; ++i) alpha[i] = lane_value(a, 16 * i);
}

// 8 consecutive stored values (bf16: one 16-byte load; f32: two)
template <typename ST>
struct Vals8;
template <>
struct Vals8<Bf16> {
    uint4 w;
    __device__ __forceinline__ void load(const char *p) { w = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void zero() { w = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void get(float v[8]) const {
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
        v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
    __device__ __forceinline__ void raw(uint16_t v[8]) const {
        v[0] = (uint16_t)w.x; v[1] = (uint16_t)(w.x >> 16);
        v[2] = (uint16_t)w.y; v[3] = (uint16_t)(w.y >> 16);
        v[4] = (uint16_t)w.z; v[5] = (uint16_t)(w.z >> 16);
        v[6] = (uint16_t)w.w; v[7] = (uint16_t)(w.w >> 16);
    }
};
template <>
struct Vals8<F32> {
    uint4 a, b;
    __device__ __forceinline__ void load(const char *p) {
        a = reinterpret_cast<const uint4 *>(p)[0];
        b = reinterpret_cast<const uint4 *>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = b = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void get(float v[8]) const {
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
        v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
        v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    }
    __device__ __forceinline__ void raw(uint32_t v[8]) const {
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

// wait until at most N vector-memory loads of this wave are outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] (7 = no wait) | lgkmcnt[11:8] (15 = no wait) | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

struct alignas(4) W4 { uint32_t x, y, z, w; };
struct alignas(4) W3 { uint32_t x, y, z; };
struct alignas(4) W2 { uint32_t x, y; };

// N consecutive dwords from a 4-byte aligned address, in 16-byte pieces
template <int N>
__device__ __forceinline__ void load_words(const char *p, uint32_t (&w)[N]) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
        const W4 v = *reinterpret_cast<const W4 *>(q + 4 * i);
        w[4 * i] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
    constexpr int b = N - N % 4;
    if constexpr (N % 4 == 3) {
        const W3 v = *reinterpret_cast<const W3 *>(q + b);
        w[b] = v.x;
        w[b + 1] = v.y;
        w[b + 2] = v.z;
    } else if constexpr (N % 4 == 2) {
        const W2 v = *reinterpret_cast<const W2 *>(q + b);
        w[b] = v.x;
        w[b + 1] = v.y;
    } else if constexpr (N % 4 == 1) {
        w[b] = q[b];
    }
}
template <int N>
constexpr int load_instrs() { return N / 4 + (N % 4 ? 1 : 0); }

// One record's windows for one lane. Bitmap records (BM) carry the token's
// K and V position bitmaps instead of the u8 index windows.
template <typename ST, int QM, bool BM>
struct PkWin {
    // values: a bf16 window may start 2 bytes before the lane's first element
    static constexpr int NV = ST::bytes == 2 ? (2 * QM + 5) / 4 : QM;
    // indices: the window may start up to 3 bytes early
    static constexpr int NI = (QM + 6) / 4;
    static constexpr int LOADS = 2 * load_instrs<NV>() + (BM ? 2 : 2 * load_instrs<NI>());
    uint32_t kv[NV], vv[NV], ki[NI], vi[NI];
    uint4 bk, bv;
};

// Per-lane constants of one packed segment.
template <typename ST, int QM>
struct PkGeom {
    uint32_t o_kv, o_vv, o_ki, o_vi;  // window offsets in the record
    uint32_t sv, si;                  // byte shifts of the value / index windows
    uint32_t o_bk, o_bv;              // bitmap records: the token's K and V bitmaps
    int g;                            // bitmap records: channels per position bit
    uint32_t l_ki, l_vi;              // bitmap records: index windows in the wave's LDS index buffer
    int cnt;                          // elements of this lane's part
    int row;                          // t * 128: this token's tile row
    __device__ __forceinline__ void init(int r, int gsz) {
        const int lane = lane_id();
        const int t = lane >> 2, p = lane & 3;
        const int Q = (r + 3) >> 2;
        const uint32_t e0 = (uint32_t)(t * r + p * Q);
        cnt = max(0, min(Q, r - p * Q));
        const uint32_t reg = (uint32_t)BT * r * ST::bytes;  // one value region
        const uint32_t vb = e0 * ST::bytes;
        sv = vb & 3u;
        si = e0 & 3u;
        o_kv = vb & ~3u;
        o_vv = reg + o_kv;
        o_ki = 2 * reg + (e0 & ~3u);
        o_vi = o_ki + (uint32_t)BT * r;
        g = gsz;
        const uint32_t vb_bytes = (uint32_t)(D / 8 / gsz);  // one vector's bitmap
        o_bk = 2 * reg + (uint32_t)t * vb_bytes;
        o_bv = o_bk + (uint32_t)BT * vb_bytes;
        l_ki = e0 & ~3u;
        l_vi = l_ki + (uint32_t)BT * r;
        row = t * D;
    }
};

template <typename ST, int QM, bool BM>
__device__ __forceinline__ void load_win(const char *rec, const PkGeom<ST, QM> &gm, PkWin<ST, QM, BM> &W) {
    load_words(rec + gm.o_kv, W.kv);
    load_words(rec + gm.o_vv, W.vv);
    if constexpr (BM) {
        // the 16-byte aligned window holding the token's bitmap (all of it for
        // one bit per channel; 8, 4 or 2 bytes of it with element groups)
        const W4 a = *reinterpret_cast<const W4 *>(rec + (gm.o_bk & ~15u));
        const W4 b = *reinterpret_cast<const W4 *>(rec + (gm.o_bv & ~15u));
        W.bk = make_uint4(a.x, a.y, a.z, a.w);
        W.bv = make_uint4(b.x, b.y, b.z, b.w);
    } else {
        load_words(rec + gm.o_ki, W.ki);
        load_words(rec + gm.o_vi, W.vi);
    }
}

// Bitmap records: lane p of a token writes the channels of the set bits of
// word p of the token's bitmap b (channels 32 p .. 32 p + 31) to dst, at their
// ranks among the token's kept elements, so dst holds the token's u8 indices
// in ascending channel order.
__device__ __forceinline__ void bitmap_positions(const uint4 b, int p, uint8_t *dst) {
    const int c0 = __popc(b.x), c1 = __popc(b.y), c2 = __popc(b.z);
    uint32_t w = p == 0 ? b.x : p == 1 ? b.y : p == 2 ? b.z : b.w;
    int pos = (p > 0 ? c0 : 0) + (p > 1 ? c1 : 0) + (p > 2 ? c2 : 0);
    while (w) {
        dst[pos++] = (uint8_t)(32 * p + __builtin_ctz(w));
        w &= w - 1u;
    }
}

// Bitmap records with element groups of g channels (bit i: channels g i ..
// g i + g - 1 kept): the token's group bits are the bytes at `off` (0..15) of
// the 16-byte window w. Lane p of a token writes the channels of its groups
// in channels 32 p .. 32 p + 31, g bytes per group as one aligned store (r is
// a multiple of g, so every group's rank is), at rank g * (groups before it).
// (The group size is a template argument: with it known, the shifts, masks
// and the store width fold away; a uniform switch picks the instance.)
template <int GS>
__device__ __forceinline__ uint64_t group_bits(const uint4 w, uint32_t off) {
    const uint64_t lo = ((uint64_t)w.y << 32) | w.x, hi = ((uint64_t)w.w << 32) | w.z;
    const uint64_t x = ((off & 8u) ? hi : lo) >> (8 * (off & 7u));
    constexpr int n = D / GS;  // bits
    if constexpr (n >= 64) return x;
    else return x & ((1ull << n) - 1ull);
}
template <int GS>
__device__ __forceinline__ void group_positions(uint64_t gb, int p, uint8_t *dst) {
    constexpr int gw = 32 / GS;  // groups per lane
    const int i0 = p * gw;       // the lane's first group
    uint32_t w = (uint32_t)((gb >> i0) & ((1ull << gw) - 1ull));
    int pos = GS * __popcll(gb & ((1ull << i0) - 1ull));
    while (w) {
        const uint32_t c = (uint32_t)(GS * (i0 + __builtin_ctz(w)));
        if constexpr (GS == 2) *reinterpret_cast<uint16_t *>(dst + pos) = (uint16_t)(c | ((c + 1u) << 8));
        else if constexpr (GS == 4) *reinterpret_cast<uint32_t *>(dst + pos) = c * 0x01010101u + 0x03020100u;
        else *reinterpret_cast<uint64_t *>(dst + pos) = (uint64_t)c * 0x0101010101010101ull + 0x0706050403020100ull;
        pos += GS;
        w &= w - 1u;
    }
}
template <int GS>
__device__ __forceinline__ void group_positions_kv(const uint4 &bk, const uint4 &bv, uint32_t ok, uint32_t ov, int p,
                                                   uint8_t *dk, uint8_t *dv) {
    group_positions<GS>(group_bits<GS>(bk, ok), p, dk);
    group_positions<GS>(group_bits<GS>(bv, ov), p, dv);
}

// N dwords from the wave's LDS index buffer (4-byte aligned)
template <int N>
__device__ __forceinline__ void lds_words(const uint8_t *p, uint32_t (&w)[N]) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = q[i];
}

// Per-wave LDS of the packed path: the dense V tile; row 16 absorbs masked writes.
template <typename ST, int G>
struct PkLds {
    typename ST::bits_t vt[BT + 1][D];
    float zb[G][BT];  // p of the current record, head-major
};

template <int G>
struct PkState {
    float acc[G][2];  // channels 2 lane, 2 lane + 1
    float l[G];       // lane-private sums of p (each token counted by its 4 lanes)
    float m[G];       // running max per head (wave-uniform)
};

#define MKV_DPP(v, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xf, 0xf, false))
__device__ __forceinline__ float quad_sum(float v) {
    v += MKV_DPP(v, 0xB1);  // quad_perm [1, 0, 3, 2]
    v += MKV_DPP(v, 0x4E);  // quad_perm [2, 3, 0, 1]
    return v;
}
// max over the wave of a value replicated within each quad
__device__ __forceinline__ float wave_max_quads(float v) {
    v = fmaxf(v, MKV_DPP(v, 0x124));  // row_ror 4
    v = fmaxf(v, MKV_DPP(v, 0x128));  // row_ror 8
    return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
#undef MKV_DPP
__device__ __forceinline__ float wave_sum_all(float v) {
    v = row_sum16(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// One online-softmax step of head h over a block of 16 tokens: z is this
// lane's part of token (lane / 4)'s logit (log2 units). Returns p, replicated
// over the token's four lanes.
template <int G>
__device__ __forceinline__ float softmax_step(float z, bool valid, PkState<G> &S, int h) {
    z = valid ? quad_sum(z) : -INFINITY;
    const float bm = wave_max_quads(z);
    const float mh = S.m[h];
    if (bm != -INFINITY && (mh == -INFINITY || bm > mh + 8.f)) {
        const float a = (mh == -INFINITY) ? 0.f : fast_exp2(mh - bm);
        S.m[h] = bm;
        S.acc[h][0] *= a;
        S.acc[h][1] *= a;
        S.l[h] *= a;
    }
    const float p = valid ? fast_exp2(z - S.m[h]) : 0.f;
    S.l[h] += p;
    return p;
}

// the 16 weights of one head, broadcast from LDS
__device__ __forceinline__ void read_p16(const float *zb, float (&p)[BT]) {
#pragma unroll
    for (int q = 0; q < BT / 4; ++q) {
        const float4 v = reinterpret_cast<const float4 *>(zb)[q];
        p[4 * q] = v.x;
        p[4 * q + 1] = v.y;
        p[4 * q + 2] = v.z;
        p[4 * q + 3] = v.w;
    }
}

// acc[I][*] += sum_t p_t * tile[t][2 lane, 2 lane + 1]
template <typename ST, int G, int I>
__device__ __forceinline__ void pk_accum(const PkLds<ST, G> &L, PkState<G> &S, int lane) {
    float p[BT];
    read_p16(L.zb[I], p);
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        float a, b;
        if constexpr (ST::bytes == 2) {
            const uint32_t w = reinterpret_cast<const uint32_t *>(&L.vt[t][0])[lane];
            a = bf16_lo(w);
            b = bf16_hi(w);
        } else {
            const uint2 w = reinterpret_cast<const uint2 *>(&L.vt[t][0])[lane];
            a = __uint_as_float(w.x);
            b = __uint_as_float(w.y);
        }
        S.acc[I][0] = fmaf(p[t], a, S.acc[I][0]);
        S.acc[I][1] = fmaf(p[t], b, S.acc[I][1]);
    }
}

// the I-th value of a lane's window (masked to 0 past its part for K)
template <typename ST, int NV>
__device__ __forceinline__ uint32_t win_word(const uint32_t (&w)[NV], int k, uint32_t sv) {
    if constexpr (ST::bytes == 2) return __builtin_amdgcn_alignbyte(w[k + 1], w[k], sv);
    else return w[k];
}

template <typename ST, int G, int QM, int WAITN, bool BM>
__device__ __forceinline__ void pk_proc(const PkWin<ST, QM, BM> &W, const PkGeom<ST, QM> &gm, int hm, int nv,
                                        const float (*qsh)[2 * D], PkLds<ST, G> &L, PkState<G> &S, uint8_t *ib,
                                        int r) {
    const int lane = lane_id();
    vm_wait<WAITN>();
    constexpr int NI = PkWin<ST, QM, BM>::NI;
    uint32_t wki[NI], wvi[NI];
    if constexpr (BM) {
        // the record's u8 indices, decoded from its bitmaps into the wave's
        // LDS buffer ([16][r] K then [16][r] V), then read as index windows
        const int t = lane >> 2, p = lane & 3;
        uint8_t *dk = ib + t * r, *dv = ib + BT * r + t * r;
        const uint32_t ok = gm.o_bk & 15u, ov = gm.o_bv & 15u;
        switch (gm.g) {
        case 2: group_positions_kv<2>(W.bk, W.bv, ok, ov, p, dk, dv); break;
        case 4: group_positions_kv<4>(W.bk, W.bv, ok, ov, p, dk, dv); break;
        case 8: group_positions_kv<8>(W.bk, W.bv, ok, ov, p, dk, dv); break;
        default:
            bitmap_positions(W.bk, p, dk);
            bitmap_positions(W.bv, p, dv);
        }
        wave_lds_sync();
        lds_words(ib + gm.l_ki, wki);
        lds_words(ib + gm.l_vi, wvi);
    } else {
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            wki[k] = W.ki[k];
            wvi[k] = W.vi[k];
        }
    }
    // indices: element j = byte j of the aligned index words
    constexpr int NIW = (QM + 3) / 4;
    uint32_t ki[NIW], vi[NIW];
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
        ki[k] = __builtin_amdgcn_alignbyte(wki[k + 1], wki[k], gm.si);
        vi[k] = __builtin_amdgcn_alignbyte(wvi[k + 1], wvi[k], gm.si);
    }
    // ---- V scatter first: its LDS writes drain while K is computed
#pragma unroll
    for (int j = 0; j < QM; ++j) {
        // past the lane's part the index byte belongs to other data: such
        // writes go to the lane's own slot of the dummy row
        // (bitmap records: bytes of tokens past the block's last one are stale, so masked to a channel)
        const int c = (int)((vi[j >> 2] >> (8 * (j & 3))) & (BM ? (uint32_t)(D - 1) : 0xFFu));
        const int at = j < gm.cnt ? gm.row + c : BT * D + lane;
        if constexpr (ST::bytes == 2) {
            const uint32_t w = win_word<ST>(W.vv, j >> 1, gm.sv);
            (&L.vt[0][0])[at] = (uint16_t)((j & 1) ? (w >> 16) : w);
        } else {
            (&L.vt[0][0])[at] = W.vv[j];
        }
    }
    // ---- K: this lane's partial logit per head
    float kval[QM];
    if constexpr (ST::bytes == 2) {
#pragma unroll
        for (int k = 0; k < QM / 2; ++k) {
            const uint32_t w = win_word<ST>(W.kv, k, gm.sv);
            kval[2 * k] = 2 * k < gm.cnt ? bf16_lo(w) : 0.f;
            kval[2 * k + 1] = 2 * k + 1 < gm.cnt ? bf16_hi(w) : 0.f;
        }
    } else {
#pragma unroll
        for (int j = 0; j < QM; ++j) kval[j] = j < gm.cnt ? __uint_as_float(W.kv[j]) : 0.f;
    }
    const bool valid = (lane >> 2) < nv;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (!((hm >> h) & 1)) continue;
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < QM; ++j) {
            const int c = (int)((ki[j >> 2] >> (8 * (j & 3))) & 0xFFu);
            z = fmaf(qsh[h][c], kval[j], z);
        }
        const float p = softmax_step<G>(z, valid, S, h);
        if ((lane & 3) == 0) L.zb[h][lane >> 2] = p;
    }
    wave_lds_sync();
    // ---- V accumulate over the 16 rows, then clear them
    if (hm & 1) pk_accum<ST, G, 0>(L, S, lane);
    if constexpr (G > 1) if (hm & 2) pk_accum<ST, G, 1>(L, S, lane);
    if constexpr (G > 2) if (hm & 4) pk_accum<ST, G, 2>(L, S, lane);
    if constexpr (G > 3) if (hm & 8) pk_accum<ST, G, 3>(L, S, lane);
    {
        constexpr int n16 = BT * D * ST::bytes / 16;  // 16-byte pieces of rows 0..15
        uint4 *v4 = reinterpret_cast<uint4 *>(&L.vt[0][0]);
#pragma unroll
        for (int i = 0; i < n16 / 64; ++i) v4[lane + 64 * i] = make_uint4(0, 0, 0, 0);
    }
}

// list entries are wave-uniform: read them into scalar registers, so each
// record load is a scalar base plus loop-invariant per-lane offsets
__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <typename ST, int G, int QM, bool BM>
__device__ __forceinline__ void pk_run(const int2 *list, int n, const char *seg_base, size_t rec, int r, int gsz,
                                       int filled, const float (*qsh)[2 * D], PkLds<ST, G> &L, PkState<G> &S,
                                       uint8_t *ib) {
    PkGeom<ST, QM> gm;
    gm.init(r, gsz);
    constexpr int WN = PkWin<ST, QM, BM>::LOADS;
    PkWin<ST, QM, BM> B0, B1;
    // a load past the end of the list repeats its last record, so every step
    // has exactly one record in flight behind the one it computes
    auto at = [&](int i) {
        return seg_base + (size_t)uniform_int(list[min(i, n - 1)].x) * rec;
    };
    auto nv_of = [&](int i) { return min(BT, filled - uniform_int(list[i].x) * BT); };
    load_win(at(0), gm, B0);
    for (int i = 0; i < n; i += 2) {
        load_win(at(i + 1), gm, B1);
        pk_proc<ST, G, QM, WN, BM>(B0, gm, uniform_int(list[i].y), nv_of(i), qsh, L, S, ib, r);
        if (i + 1 >= n) break;
        load_win(at(i + 2), gm, B0);
        pk_proc<ST, G, QM, WN, BM>(B1, gm, uniform_int(list[i + 1].y), nv_of(i + 1), qsh, L, S, ib, r);
    }
}

// the records of one packed segment, with the windows code of their r
// (BM: the cache's packed segments hold bitmap records; ib is the wave's LDS
// index buffer for them)
template <typename ST, int G, int QA, int QB, bool BM>
__device__ __forceinline__ void run_records(const int2 *list, int n, const char *seg_base, size_t rec, int r,
                                            int gsz, int filled, const float (*qsh)[2 * D], PkLds<ST, G> &L,
                                            PkState<G> &S, uint8_t *ib) {
    if (((r + 3) >> 2) <= QA) pk_run<ST, G, QA, BM>(list, n, seg_base, rec, r, gsz, filled, qsh, L, S, ib);
    else pk_run<ST, G, QB, BM>(list, n, seg_base, rec, r, gsz, filled, qsh, L, S, ib);
}

__device__ __forceinline__ int64_t packed_weight(int kind, int r, int gsz, int sb, int G) {
    const int64_t rec = record_bytes(kind, r, sb, gsz);
    return (G > 1 ? rec * 4 / 5 : rec) + 256;
}

// a split's partial (m, l, acc[128]) per head into dst [G][PART] (LDS)
template <typename ST, int G>
__device__ __forceinline__ void write_partial(float *dst, const PkState<G> &S) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const float li = wave_sum_all(S.l[i]) * 0.25f;
        float *pp = dst + i * PART;
        if (lane == 0) {
            pp[0] = S.m[i];
            pp[1] = li;
        }
        reinterpret_cast<float2 *>(pp + 2)[lane] = make_float2(S.acc[i][0], S.acc[i][1]);
    }
}

template <int G>
__device__ __forceinline__ void init_state(PkState<G> &S) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
        S.acc[i][0] = S.acc[i][1] = 0.f;
        S.l[i] = 0.f;
        S.m[i] = -INFINITY;
    }
}

// dense split s of S_d: an equal share of the unit's dense blocks. Lane
// (tg, ch) = (lane / 16, lane % 16) covers tokens tg, tg+4, tg+8, tg+12 on
// channels 8ch..8ch+7; the K and V loads of a block are issued together.
// Logits reduce over the 16 lanes of a token group (one DPP row); softmax
// lanes are head-major (lane h * 16 + t); the V sums stay in registers until
// the end, where the four token groups add up.
template <typename ST, int G>
__device__ __forceinline__ void attend_dense_split(const DecodeArgs &A, int bl, int g, int s,
                                                   const float (*qsh)[2 * D], float *zb, float *dst) {
    const int lane = lane_id();
    const int tg = lane >> 4, ch = lane & 15;
    float vacc[G][8];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) vacc[i][c] = 0.f;
    WaveState<G> st;
    st.init();

    constexpr int sb = ST::bytes;
    int64_t nblocks = 0;
    for (int si = 0; si < A.nseg; ++si) {
        const DSeg &S = seg_of(A, bl, si);
        if (S.kind == MKV_SEG_DENSE && S.slot == A.cur_slot) nblocks += S.nb;
    }
    const int64_t i0 = nblocks * s / A.S_d, i1 = nblocks * (s + 1) / A.S_d;
    int64_t before = 0;
    for (int si = 0; si < A.nseg; ++si) {
        const DSeg &S = seg_of(A, bl, si);
        if (S.kind != MKV_SEG_DENSE || S.slot != A.cur_slot) continue;
        const int64_t a0 = max(i0 - before, (int64_t)0), a1 = min(i1 - before, (int64_t)S.nb);
        before += S.nb;
        if (a0 >= a1) continue;
        const char *seg_base = static_cast<const char *>(S.data) + (size_t)g * S.nbcap * 2 * BT * D * sb;
        for (int64_t blk = a0; blk < a1; ++blk) {
            const int nv = min(BT, S.filled - (int)blk * BT);
            const char *kb = seg_base + (size_t)blk * 2 * BT * D * sb;
            const char *vb = kb + (size_t)BT * D * sb;
            Vals8<ST> kr[4], vr[4];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                kr[ii].load(kb + (size_t)((4 * ii + tg) * D + ch * 8) * sb);
                vr[ii].load(vb + (size_t)((4 * ii + tg) * D + ch * 8) * sb);
            }
            float part[4][G];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                float kv[8];
                kr[ii].get(kv);
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const float4 qa = *reinterpret_cast<const float4 *>(&qsh[i][ch * 8]);
                    const float4 qb = *reinterpret_cast<const float4 *>(&qsh[i][ch * 8 + 4]);
                    float a = qa.x * kv[0];
                    a = fmaf(qa.y, kv[1], a);
                    a = fmaf(qa.z, kv[2], a);
                    a = fmaf(qa.w, kv[3], a);
                    a = fmaf(qb.x, kv[4], a);
                    a = fmaf(qb.y, kv[5], a);
                    a = fmaf(qb.z, kv[6], a);
                    a = fmaf(qb.w, kv[7], a);
                    part[ii][i] = a;
                }
            }
            // a token group is one DPP row of 16 lanes
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
                for (int i = 0; i < G; ++i) part[ii][i] = row_sum16(part[ii][i]);
            if (ch < G) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    float v = part[ii][0];
#pragma unroll
                    for (int i = 1; i < G; ++i)
                        if (ch == i) v = part[ii][i];
                    zb[(4 * ii + tg) * G + ch] = v;
                }
            }
            wave_lds_sync();
            float alpha[G];
            {
                const int h = lane >> 4, t = lane & 15;
                const bool valid = h < G && t < nv;
                softmax16<G>(valid ? zb[t * G + h] : 0.f, valid, zb, st, alpha);
            }
#pragma unroll
            for (int i = 0; i < G; ++i)
                if (alpha[i] != 1.f) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) vacc[i][c] *= alpha[i];
                }
            wave_lds_sync();
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int tt = 4 * ii + tg;
                float vv[8];
                vr[ii].get(vv);
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const float p = zb[tt * G + i];
#pragma unroll
                    for (int c = 0; c < 8; ++c) vacc[i][c] = fmaf(p, vv[c], vacc[i][c]);
                }
            }
            wave_lds_sync();
        }
    }
    // partials: m, l and acc[h][c]; acc sums over the four token groups
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v = vacc[i][c];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            vacc[i][c] = v;
        }
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const float li = st.head_sum(i);
        const float mi = st.head_max(i);
        float *pp = dst + i * PART;
        if (lane == 0) {
            pp[0] = mi;
            pp[1] = li;
        }
        if (tg == 0) {
            float2 *d2 = reinterpret_cast<float2 *>(pp + 2 + ch * 8);  // partials are 8-byte aligned
#pragma unroll
            for (int c = 0; c < 8; c += 2) d2[c / 2] = make_float2(vacc[i][c], vacc[i][c + 1]);
        }
    }
}

// packed split s of S_p: an equal share (by bytes) of the unit's union records
template <typename ST, int G, int QA, int QB, bool BM>
__device__ __forceinline__ void attend_packed_split(const DecodeArgs &A, int bl, int b, int g, int s,
                                                    const float (*qsh)[2 * D], PkLds<ST, G> &L, int2 *list,
                                                    float *dst, uint8_t *ib) {
    constexpr int sb = ST::bytes;
    const int lane = lane_id();
    for (int i = lane; i < BT * D; i += 64) (&L.vt[0][0])[i] = 0;
    PkState<G> S;
    init_state<G>(S);
    int64_t W = 0;
    for (int si = 0; si < A.nseg; ++si) {
        const DSeg &Sg = seg_of(A, bl, si);
        if (packed_kind(Sg.kind) && Sg.slot == A.cur_slot)
            W += (int64_t)G * Sg.k * packed_weight(Sg.kind, Sg.r, Sg.group, sb, G);
    }
    const int64_t lo = W * s / A.S_p, hi = W * (s + 1) / A.S_p;
    int64_t Wb = 0;
    int pj = 0;
    for (int si = 0; si < A.nseg; ++si) {
        const DSeg &Sg = seg_of(A, bl, si);
        if (!packed_kind(Sg.kind)) continue;
        const int myj = pj++;
        if (Sg.slot != A.cur_slot) continue;
        const int64_t w = packed_weight(Sg.kind, Sg.r, Sg.group, sb, G);
        const int64_t items = (int64_t)G * Sg.k;
        int64_t i0 = lo - Wb, i1 = hi - Wb;
        i0 = i0 <= 0 ? 0 : (i0 + w - 1) / w;
        i1 = i1 <= 0 ? 0 : (i1 + w - 1) / w;
        i0 = min(i0, items);
        i1 = min(i1, items);
        Wb += items * w;
        if (i0 >= i1) continue;
        const int r = Sg.r;
        const size_t rec = (size_t)record_bytes(Sg.kind, r, sb, Sg.group);
        const char *seg_base = static_cast<const char *>(Sg.data) + (size_t)g * Sg.nbcap * rec;
        const int kc = A.kcap[myj];
        const int32_t *sel = A.sel + A.sl_off[myj] + ((size_t)b * A.hq + g * G) * kc;
        const uint32_t *mk = A.mask + A.mk_off[myj] + ((size_t)b * A.hkv + g) * A.nbcap[myj];
        for (int64_t base = i0; base < i1; base += 64) {
            // resolve up to 64 items into (block, head mask) pairs
            const int64_t it = base + lane;
            bool keep = false;
            int blk = 0, hm = 0;
            if (it < i1) {
                const int rank = (int)(it / G), hl = (int)(it % G);
                blk = sel[(size_t)hl * kc + rank];
                if ((unsigned)blk < (unsigned)Sg.nb) {
                    // byte i of the word is 1 if head i chose the block
                    const uint32_t bytes = mk[blk];
                    hm = (int)((bytes | (bytes >> 7) | (bytes >> 14) | (bytes >> 21)) & 0xFu);
                    keep = !(hm & ((1 << hl) - 1));
                }
            }
            const uint64_t km = ballot(keep);
            if (keep) list[popc64(km & lanes_below(lane))] = make_int2(blk, hm);
            const int n = popc64(km);
            wave_lds_sync();
            if (n > 0) run_records<ST, G, QA, QB, BM>(list, n, seg_base, rec, r, Sg.group, Sg.filled, qsh, L, S, ib);
            wave_lds_sync();
        }
    }
    write_partial<ST, G>(dst, S);
}

// ---- union mode: exact byte-balanced packed splits -------------------------
// For units whose (at most UNION_MAX_SEGS) packed segments hold at most
// UNION_SEG_BLOCKS blocks each, a packed workgroup takes an exact
// byte-weighted share of the unit's union records (blocks with a non-zero head
// mask; weight = record bytes + UNION_RECORD_FIXED) and gives each of its waves an equal
// quarter of it. The workgroup reads the union masks itself: wave v, lane l
// holds blocks 1024 v + 256 m + 4 l + k (m, k < 4; four coalesced 16-byte
// loads per segment), and union records are ranked in that order, segment by
// segment, by one workgroup prefix sum.
constexpr int UNION_SEG_BLOCKS = 4096;
constexpr int UNION_MAX_SEGS = 4;

struct UnionLds {
    uint32_t ent[UNION_CAP];  // block | head mask << 16, segment by segment
    uint64_t red[4];
};

__device__ __forceinline__ int union_block(int i) {
    return 1024 * (int)(threadIdx.x >> 6) + 256 * (i >> 2) + 4 * lane_id() + (i & 3);
}

// this thread's 16 union mask words of packed segment j of unit (b, g) (0
// past the stored blocks; byte h is 1 if head h chose the block)
__device__ __forceinline__ void union_words(const DecodeArgs &A, int j, int b, int g, int nb, uint32_t (&w)[16]) {
    const uint32_t *mk = A.mask + A.mk_off[j] + ((size_t)b * A.hkv + g) * A.nbcap[j];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int l0 = union_block(4 * m);
        uint32_t x[4];
        if (l0 + 3 < nb) {
            const W4 v = *reinterpret_cast<const W4 *>(mk + l0);  // 4-byte aligned
            x[0] = v.x;
            x[1] = v.y;
            x[2] = v.z;
            x[3] = v.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = l0 + k < nb ? mk[l0 + k] : 0u;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) w[4 * m + k] = x[k];
    }
}

// workgroup exclusive prefix of v (four 16-bit counts) in thread order, and
// the workgroup total
__device__ __forceinline__ uint64_t wg_excl64(uint64_t v, UnionLds &U, uint64_t &total) {
    const int wave = (int)(threadIdx.x >> 6), lane = lane_id();
    uint64_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) U.red[wave] = x;
    __syncthreads();
    uint64_t before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint64_t t = U.red[w];
        if (w < wave) before += t;
        total += t;
    }
    return before + x - v;
}

// first entry of a segment whose weighted start (Wb + e w) is >= pos
__device__ __forceinline__ int union_entry(uint32_t pos, uint32_t Wb, uint32_t w, int n) {
    const int e = pos <= Wb ? 0 : (int)((pos - Wb + w - 1) / w);
    return min(e, n);
}

// Weighted positions stay below 2^32 / 4: at most 4 segments x 4096 records
// x (record bytes + UNION_RECORD_FIXED <= 20480 + 16384) bytes (bitmap records
// are at most 16896 bytes).
template <typename ST, int G, int QA, int QB, bool BM>
__device__ __forceinline__ void attend_packed_union(const DecodeArgs &A, int bl, int b, int g, int xs, int wave,
                                                    const float (*qsh)[2 * D], PkLds<ST, G> &L, int2 *list,
                                                    float *dst, UnionLds &U, uint8_t *ib) {
    constexpr int sb = ST::bytes;
    const int lane = lane_id();
    const int npk = A.npk;
    // per packed segment: stored blocks, kept elements and record weight
    int nbj[UNION_MAX_SEGS], rj[UNION_MAX_SEGS];
    uint32_t wj[UNION_MAX_SEGS];
#pragma unroll
    for (int j = 0; j < UNION_MAX_SEGS; ++j) {
        const DSeg &Sg = seg_of(A, bl, A.pseg[min(j, npk - 1)]);
        nbj[j] = (j < npk && Sg.slot == A.cur_slot) ? Sg.nb : 0;
        rj[j] = Sg.r;
        wj[j] = (uint32_t)(record_bytes(Sg.kind, Sg.r, sb, Sg.group) + UNION_RECORD_FIXED);
    }
    uint32_t w[UNION_MAX_SEGS][16];
#pragma unroll
    for (int j = 0; j < UNION_MAX_SEGS; ++j)
        if (j < npk) union_words(A, j, b, g, nbj[j], w[j]);
    {
        uint4 *v4 = reinterpret_cast<uint4 *>(&L.vt[0][0]);  // rows 0..15 of the tile
#pragma unroll
        for (int i = 0; i < BT * D * sb / 16 / 64; ++i) v4[lane + 64 * i] = make_uint4(0, 0, 0, 0);
    }
    PkState<G> S;
    init_state<G>(S);
    // union records of each segment: this thread's rank base and the totals
    uint64_t cnt = 0;
#pragma unroll
    for (int j = 0; j < UNION_MAX_SEGS; ++j) {
        if (j >= npk) break;
        int c = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) c += w[j][i] != 0u;
        cnt |= (uint64_t)c << (16 * j);
    }
    uint64_t tot;
    const uint64_t pre = wg_excl64(cnt, U, tot);
    int nj[UNION_MAX_SEGS];
    uint32_t W = 0;
#pragma unroll
    for (int j = 0; j < UNION_MAX_SEGS; ++j) {
        nj[j] = j < npk ? (int)((tot >> (16 * j)) & 0xFFFFu) : 0;
        W += (uint32_t)nj[j] * wj[j];
    }
    const uint32_t P = (uint32_t)A.S_p / 4, q = W / P, rm = W % P;
    const uint32_t wlo = q * xs + rm * xs / P, whi = q * (xs + 1) + rm * (xs + 1) / P;
    const uint32_t vlo = wlo + (whi - wlo) * wave / 4, vhi = wlo + (whi - wlo) * (wave + 1) / 4;
    int e0[UNION_MAX_SEGS], e1[UNION_MAX_SEGS], off[UNION_MAX_SEGS];
    {
        uint32_t Wb = 0;
        int o = 0;
#pragma unroll
        for (int j = 0; j < UNION_MAX_SEGS; ++j) {
            e0[j] = union_entry(wlo, Wb, wj[j], nj[j]);
            e1[j] = union_entry(whi, Wb, wj[j], nj[j]);
            off[j] = o;
            o += e1[j] - e0[j];
            Wb += (uint32_t)nj[j] * wj[j];
        }
    }
    // the workgroup's entries into LDS, segment by segment (only the threads
    // whose records overlap the workgroup's share)
#pragma unroll
    for (int j = 0; j < UNION_MAX_SEGS; ++j) {
        if (j >= npk) break;
        int u = (int)((pre >> (16 * j)) & 0xFFFFu);
        const int c = (int)((cnt >> (16 * j)) & 0xFFFFu);
        if (u + c <= e0[j] || u >= e1[j]) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t x = w[j][i];
            if (x != 0u) {
                const int at = off[j] + u - e0[j];
                if (u >= e0[j] && u < e1[j] && at < UNION_CAP) {
                    const uint32_t hm = (x | (x >> 7) | (x >> 14) | (x >> 21)) & 0xFu;  // byte h -> bit h
                    U.ent[at] = (uint32_t)union_block(i) | (hm << 16);
                }
                ++u;
            }
        }
    }
    __syncthreads();
    // this wave's quarter, 64 entries at a time
    uint32_t Wb = 0;
#pragma unroll
    for (int j = 0; j < UNION_MAX_SEGS; ++j) {
        if (j >= npk) break;
        const int v0 = union_entry(vlo, Wb, wj[j], nj[j]), v1 = union_entry(vhi, Wb, wj[j], nj[j]);
        Wb += (uint32_t)nj[j] * wj[j];
        if (v0 >= v1) continue;
        const DSeg &Sg = seg_of(A, bl, A.pseg[j]);
        const int r = rj[j];
        const size_t rec = (size_t)record_bytes(Sg.kind, r, sb, Sg.group);
        const char *seg_base = static_cast<const char *>(Sg.data) + (size_t)g * Sg.nbcap * rec;
        for (int base = v0; base < v1; base += 64) {
            // (the host bounds the workgroup's entries by UNION_CAP; the clamp
            // only keeps reads inside the table)
            const int n = min(min(64, v1 - base), UNION_CAP - (off[j] + base - e0[j]));
            if (n <= 0) break;
            if (lane < n) {
                const uint32_t e = U.ent[off[j] + base - e0[j] + lane];
                list[lane] = make_int2((int)(e & 0xFFFFu), (int)(e >> 16));
            }
            wave_lds_sync();
            run_records<ST, G, QA, QB, BM>(list, n, seg_base, rec, r, Sg.group, Sg.filled, qsh, L, S, ib);
            wave_lds_sync();
        }
    }
    write_partial<ST, G>(dst, S);
}

// QA < QB: packed segments with ceil(r / 4) <= QA run the QA code, the others QB
// Occupancy floor: 4 waves per SIMD for bf16 records; fp32 windows are twice
// as wide and fit 3 (2 at r > 64). Bitmap launches hold 4 KB more LDS per
// wave: 3 workgroups per CU (bf16), 2 (fp32).
template <typename ST, int QB, bool BM>
constexpr int attend_min_waves() {
    return BM ? (ST::bytes == 2 ? 3 : 2) : (ST::bytes == 2 ? 4 : (QB > 16 ? 2 : 3));
}

// BM: the cache's packed segments hold bitmap records (each wave then has a
// 4 KB LDS index buffer)
constexpr int BM_IDX_BYTES = 2 * BT * D + 64;

template <typename ST, int G, int QA, int QB, bool BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attend_min_waves<ST, QB, BM>(), 8))) void k_attend(const DecodeArgs A) {
    const int bl = (int)blockIdx.z, g = (int)blockIdx.y;
    const int b = A.b0 + bl;
    // wave-uniform: the split bounds and their 64-bit arithmetic stay scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int px = (A.S_p + 3) / 4;
    // q' * log2(e) / sqrt(d) per head; channels 128..255 are zero so that any
    // index byte of a packed window gathers a finite value
    __shared__ __align__(16) float qsh[G][2 * D];
    __shared__ __align__(16) PkLds<ST, G> lds[4];
    __shared__ int2 lists[4][64];
    __shared__ __align__(16) uint8_t bmi[BM ? 4 : 1][BM ? BM_IDX_BYTES : 16];
    for (int i = (int)threadIdx.x; i < G * 2 * D; i += 256) {
        const int h = i / (2 * D), c = i % (2 * D);
        qsh[h][c] = c < D ? A.qa[(((size_t)b * A.nslot + A.cur_slot) * A.hq + g * G + h) * D + c] : 0.f;
    }
    __syncthreads();
    // each wave's split partial goes to its own LDS area once the wave is done with it
    float *mine = reinterpret_cast<float *>(&lds[wave]);
    static_assert(sizeof(PkLds<ST, G>) >= G * PART * sizeof(float), "partial fits the wave's LDS");
    const bool packed = (int)blockIdx.x < px;
    const int xs = packed ? (int)blockIdx.x : (int)blockIdx.x - px;  // workgroup index within its role
    const int S = packed ? A.S_p : A.S_d;
    const int s = xs * 4 + wave;
    if (packed && A.union_mode) {
        __shared__ UnionLds U;
        attend_packed_union<ST, G, QA, QB, BM>(A, bl, b, g, xs, wave, qsh, lds[wave], lists[wave], mine, U,
                                               BM ? bmi[wave] : nullptr);
    } else if (s < S) {
        if (packed)
            attend_packed_split<ST, G, QA, QB, BM>(A, bl, b, g, s, qsh, lds[wave], lists[wave], mine,
                                                   BM ? bmi[wave] : nullptr);
        else attend_dense_split<ST, G>(A, bl, g, s, qsh, lds[wave].zb[0], mine);
    }
    __syncthreads();
    // Log-sum-exp combine of the workgroup's splits (in wave order) into one
    // partial per head: wave h takes head h. Dense workgroups' partials come
    // first, then the packed ones'.
    const int nvalid = min(4, S - 4 * xs);
    const int P = packed ? (A.S_d + 3) / 4 + xs : xs;
    const int lane = lane_id();
    for (int h = wave; h < G; h += 4) {
        float mv[4];
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            mv[v] = v < nvalid ? reinterpret_cast<const float *>(&lds[v])[h * PART] : -INFINITY;
            M = fmaxf(M, mv[v]);
        }
        float L = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (v >= nvalid) break;
            const float *src = reinterpret_cast<const float *>(&lds[v]) + h * PART;
            const float w = (mv[v] == -INFINITY) ? 0.f : fast_exp2(mv[v] - M);
            const float2 x = reinterpret_cast<const float2 *>(src + 2)[lane];
            L = fmaf(w, src[1], L);
            a0 = fmaf(w, x.x, a0);
            a1 = fmaf(w, x.y, a1);
        }
        float *pp = A.part + ((((size_t)b * A.hq + g * G + h) * A.nslot + A.cur_slot) * MAX_PARTS + P) * PART;
        if (lane == 0) {
            pp[0] = M;
            pp[1] = L;
        }
        reinterpret_cast<float2 *>(pp + 2)[lane] = make_float2(a0, a1);
    }
}

template <typename ST, int G>
__global__ __launch_bounds__(256) void k_score(const DecodeArgs A) {
    const int z = (int)blockIdx.z;
    const int bl = z / A.npk, j = z % A.npk;
    score_tile<ST, G>(A, bl, j, (int)blockIdx.y, (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
}

// ----------------------------------------------------------------------------
// merge: one workgroup per (request, query head): log-sum-exp merge of the
// head's partials (one per attend workgroup: dense ones, then packed ones,
// rotation slot by rotation slot) in order, then out_j = sum over slots of
// sum_c R_v,slot[c][j] o_slot,c -- each slot's share is rotated back by its
// own R_v (one slot unless segments carry rotations of their own).
// Thread (cc, j4) = (t / 32, t % 32) loads rows 16 cc .. 16 cc + 15 of the
// cache's R_v at columns 4 j4 .. 4 j4 + 3 first, so those loads overlap the
// merge.
// ----------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void k_merge(const DecodeArgs A) {
    static_assert(MAX_PARTS <= 256, "one thread per partial");
    const int bl = (int)blockIdx.y, h = (int)blockIdx.x;
    const int b = A.b0 + bl, g = h / G;
    const int t = (int)threadIdx.x, lane = lane_id(), wave = (int)(threadIdx.x >> 6);
    const int ns = A.nslot;
    const float *pp = A.part + ((size_t)b * A.hq + h) * ns * MAX_PARTS * PART;
    if (A.npk == 0 && A.sel_out) {  // no packed segment, no select launch: all of sel_out is padding
        int32_t *so = A.sel_out + ((size_t)b * A.hq + h) * A.sel_cols;
        for (int64_t c = t; c < A.sel_cols; c += 256) so[c] = -1;
    }
    __shared__ float wsc[MAX_SLOTS * MAX_PARTS];
    __shared__ float red[2][4];
    __shared__ __align__(16) float part_o[8][D];
    __shared__ __align__(16) float osh[D];
    const int j4 = t & 31, cc = t >> 5;
    float4 rv[16];
    {
        const float4 *Rv4 = reinterpret_cast<const float4 *>(A.rot + (((size_t)b * A.hkv + g) * 2 + 1) * D * D);
#pragma unroll
        for (int u = 0; u < 16; ++u) rv[u] = Rv4[(size_t)(cc * 16 + u) * (D / 4) + j4];
    }

    // Every load of the first slot is issued before any result is used: the
    // partials' (m, l) (thread t takes partials t, t + 256, ...) and this
    // thread's accumulator words, channels 4 quad .. 4 quad + 3 of partials
    // grp, grp + 8, ... (grp, quad) = (t / 32, t % 32).
    constexpr int NML = (MAX_SLOTS * MAX_PARTS + 255) / 256;
    constexpr int NY = (MAX_PARTS + 7) / 8;
    const int quad = t & 31, grp = t >> 5;
    float mi[NML], li[NML];
#pragma unroll
    for (int u = 0; u < NML; ++u) {
        const int i = t + 256 * u;
        const bool ok = i < ns * MAX_PARTS && i % MAX_PARTS < A.nparts[i / MAX_PARTS];
        mi[u] = ok ? pp[(size_t)i * PART] : -INFINITY;
        li[u] = ok ? pp[(size_t)i * PART + 1] : 0.f;
    }
    float2 xa[NY], xb[NY];
    {
        const int np = A.nparts[0];
#pragma unroll
        for (int k = 0; k < NY; ++k) {
            const int y = grp + 8 * k;
            if (y < np) {
                const float *src = pp + (size_t)y * PART + 2 + quad * 4;  // 8-byte aligned
                xa[k] = *reinterpret_cast<const float2 *>(src);
                xb[k] = *reinterpret_cast<const float2 *>(src + 2);
            }
        }
    }
    // partial weights: w_p = exp2(m_p - M), L = sum_p w_p l_p over every slot
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < NML; ++u) m = fmaxf(m, mi[u]);
    {
        float v = row_max16(m);
        v = fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
        if (lane == 0) red[0][wave] = v;
    }
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    float wl = 0.f;
#pragma unroll
    for (int u = 0; u < NML; ++u) {
        const int i = t + 256 * u;
        if (i < ns * MAX_PARTS) {
            float w = 0.f;
            if (i % MAX_PARTS < A.nparts[i / MAX_PARTS]) {
                w = (mi[u] == -INFINITY) ? 0.f : fast_exp2(mi[u] - M);
                wl = fmaf(w, li[u], wl);
            }
            wsc[i] = w;
        }
    }
    {
        const float v = wave_sum(wl);
        if (lane == 0) red[1][wave] = v;
    }
    __syncthreads();
    const float L = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int slot = 0; slot < ns; ++slot) {
        const float *ps = pp + (size_t)slot * MAX_PARTS * PART;
        const int np = A.nparts[slot];
        {
            // thread (grp, quad): channels 4 quad .. 4 quad + 3 over partials grp, grp + 8, ...
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
            if (slot == 0) {
#pragma unroll
                for (int k = 0; k < NY; ++k) {
                    const int y = grp + 8 * k;
                    if (y < np) {
                        const float wy = wsc[y];
                        o.x = fmaf(wy, xa[k].x, o.x);
                        o.y = fmaf(wy, xa[k].y, o.y);
                        o.z = fmaf(wy, xb[k].x, o.z);
                        o.w = fmaf(wy, xb[k].y, o.w);
                    }
                }
            } else {
#pragma unroll 8
                for (int y = grp; y < np; y += 8) {
                    const float wy = wsc[slot * MAX_PARTS + y];
                    const float *src = ps + (size_t)y * PART + 2 + quad * 4;  // 8-byte aligned
                    const float2 x0 = *reinterpret_cast<const float2 *>(src);
                    const float2 x1 = *reinterpret_cast<const float2 *>(src + 2);
                    o.x = fmaf(wy, x0.x, o.x);
                    o.y = fmaf(wy, x0.y, o.y);
                    o.z = fmaf(wy, x1.x, o.z);
                    o.w = fmaf(wy, x1.y, o.w);
                }
            }
            *reinterpret_cast<float4 *>(&part_o[grp][quad * 4]) = o;
        }
        __syncthreads();
        if (t < D) {
            float o = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) o += part_o[k][t];
            osh[t] = L > 0.f ? o / L : 0.f;
        }
        __syncthreads();
        if (slot > 0) {
            const float4 *Rv4 = reinterpret_cast<const float4 *>(slot_rot(A, bl, slot) + ((size_t)g * 2 + 1) * D * D);
#pragma unroll
            for (int u = 0; u < 16; ++u) rv[u] = Rv4[(size_t)(cc * 16 + u) * (D / 4) + j4];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float oc = osh[cc * 16 + u];
            acc.x = fmaf(rv[u].x, oc, acc.x);
            acc.y = fmaf(rv[u].y, oc, acc.y);
            acc.z = fmaf(rv[u].z, oc, acc.z);
            acc.w = fmaf(rv[u].w, oc, acc.w);
        }
    }
    *reinterpret_cast<float4 *>(&part_o[cc][4 * j4]) = acc;
    __syncthreads();
    if (t < D) {
        float o = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) o += part_o[k][t];
        A.out[((size_t)b * A.hq + h) * D + t] = o;
    }
}

template <int G, int KPT>
hipError_t select_launch_kpt(const DecodeArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)G, (unsigned)a.hkv, (unsigned)(a.n_req * a.npk));
    hipLaunchKernelGGL((k_select<G, KPT>), grid, dim3(64 * a.sel_waves), 0, s, a);
    return hipGetLastError();
}

template <int G>
hipError_t select_launch(const DecodeArgs &a, hipStream_t s) {
    hipError_t e = hipSuccess;
    switch (a.sel_kpt) {
    case 0: break;  // every packed segment takes the sliced select
    case 4: e = select_launch_kpt<G, 4>(a, s); break;
    case 8: e = select_launch_kpt<G, 8>(a, s); break;
    case 16: e = select_launch_kpt<G, 16>(a, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || a.bsel_slices <= 0) return e;
    const dim3 grid((unsigned)a.bsel_slices, (unsigned)a.hq, (unsigned)(a.n_req * a.npk));
    hipLaunchKernelGGL((k_bsel_hist<G>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_bsel_cand<G>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_bsel_out<G>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qrot(const DecodeArgs &a, int G, hipStream_t s) {
    const dim3 grid(D / 32, (unsigned)a.hkv, (unsigned)(a.n_req * a.nslot));
    switch (G) {
    case 1: hipLaunchKernelGGL(k_qrot<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_qrot<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_qrot<4>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_score(const DecodeArgs &a, int dtype, int G, int max_tiles, hipStream_t s) {
    const dim3 grid((unsigned)((max_tiles + 3) / 4), (unsigned)a.hkv, (unsigned)(a.n_req * a.npk));
#define MKV_SCORE(ST, GG) hipLaunchKernelGGL((k_score<ST, GG>), grid, dim3(256), 0, s, a)
    if (dtype == MKV_BF16) {
        if (G == 1) MKV_SCORE(Bf16, 1); else if (G == 2) MKV_SCORE(Bf16, 2); else MKV_SCORE(Bf16, 4);
    } else {
        if (G == 1) MKV_SCORE(F32, 1); else if (G == 2) MKV_SCORE(F32, 2); else MKV_SCORE(F32, 4);
    }
#undef MKV_SCORE
    return hipGetLastError();
}

hipError_t launch_select(const DecodeArgs &a, int G, hipStream_t s) {
    if (a.npk == 0) return hipSuccess;
    if (G == 1) return select_launch<1>(a, s);
    if (G == 2) return select_launch<2>(a, s);
    return select_launch<4>(a, s);
}

hipError_t launch_merge(const DecodeArgs &a, int G, hipStream_t s) {
    const dim3 grid((unsigned)a.hq, (unsigned)a.n_req);
    switch (G) {
    case 1: hipLaunchKernelGGL(k_merge<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_merge<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_merge<4>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename ST, int G>
void attend_launch(const DecodeArgs &a, int qmax, dim3 grid, hipStream_t s) {
#define MKV_PK(QA, QB, BM) hipLaunchKernelGGL((k_attend<ST, G, QA, QB, BM>), grid, dim3(256), 0, s, a)
    if (a.has_bitmap) {  // bitmap records: two window shapes
        if (qmax <= 10) MKV_PK(8, 10, true);
        else MKV_PK(16, 32, true);
        return;
    }
    if (qmax <= 4) MKV_PK(4, 4, false);
    else if (qmax <= 8) MKV_PK(4, 8, false);
    else if (qmax <= 10) MKV_PK(8, 10, false);
    else if (qmax <= 16) MKV_PK(10, 16, false);
    else MKV_PK(16, 32, false);
#undef MKV_PK
}

// qmax = ceil(r_max / 4): elements per lane of the widest packed segment
hipError_t launch_attend(const DecodeArgs &a, int dtype, int G, int qmax, hipStream_t s) {
    const dim3 grid((unsigned)((a.S_p + 3) / 4 + (a.S_d + 3) / 4), (unsigned)a.hkv, (unsigned)a.n_req);
    if (dtype == MKV_BF16) {
        if (G == 1) attend_launch<Bf16, 1>(a, qmax, grid, s);
        else if (G == 2) attend_launch<Bf16, 2>(a, qmax, grid, s);
        else attend_launch<Bf16, 4>(a, qmax, grid, s);
    } else {
        if (G == 1) attend_launch<F32, 1>(a, qmax, grid, s);
        else if (G == 2) attend_launch<F32, 2>(a, qmax, grid, s);
        else attend_launch<F32, 4>(a, qmax, grid, s);
    }
    return hipGetLastError();
}

}  // namespace mkv
