// Decode attention computed straight from the compressed cache.
//
// Steps ("MosaicKV 阅读笔记" reading notes Eq. 12-14; paper summary sections
// 4.2 and 5.3, and the reading notes' Quest paragraph for the block keys):
//   q_rotate : q' = R_k q for the G query heads of a KV head
//   score    : s_l = (1/sqrt d) sum_c max(q'_c mx_c, q'_c mn_c) per block
//   select   : per query head and packed segment, the k best blocks
//              (ties to the lower block), plus a per-block head mask
//   attend   : split-KV attention over dense blocks and the union of the
//              group's selected packed blocks, online softmax in base 2
//   merge    : log-sum-exp merge of the splits, then out = o R_v
//
// All of it is bandwidth-bound gather work: every kernel runs on the vector
// ALU (no MFMA); meta and record reads are 16-byte coalesced loads.
#include <math.h>

#include "device_util.hpp"
#include "mkv_internal.h"

namespace mkv {

namespace {

constexpr float kRsqrtD = 0.08838834764831845f;  // 1 / sqrt(128)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ const DSeg &seg_of(const DecodeArgs &A, int bl, int si) {
    return A.seg[bl * A.nseg + si];
}

// ----------------------------------------------------------------------------
// q_rotate: one workgroup per (request, KV head); thread c computes q'_c.
// ----------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(128) void k_qrot(const DecodeArgs A) {
    const int bl = (int)blockIdx.y, g = (int)blockIdx.x;
    const int b = A.b0 + bl;
    const int c = (int)threadIdx.x;
    __shared__ __align__(16) float qsh[G][D];
    for (int i = 0; i < G; ++i) qsh[i][c] = A.q[((size_t)b * A.hq + g * G + i) * D + c];
    __syncthreads();
    const float4 *Rr = reinterpret_cast<const float4 *>(A.rot + (((size_t)b * A.hkv + g) * 2) * D * D +
                                                        (size_t)c * D);
    float acc[G];
#pragma unroll
    for (int i = 0; i < G; ++i) acc[i] = 0.f;
    for (int j = 0; j < D / 4; ++j) {
        const float4 r = Rr[j];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float4 x = reinterpret_cast<const float4 *>(qsh[i])[j];
            acc[i] = fmaf(r.x, x.x, acc[i]);
            acc[i] = fmaf(r.y, x.y, acc[i]);
            acc[i] = fmaf(r.z, x.z, acc[i]);
            acc[i] = fmaf(r.w, x.w, acc[i]);
        }
    }
    float *qs = A.qs + (((size_t)b * A.hkv + g) * D + c) * 2 * G;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        A.qa[((size_t)b * A.hq + g * G + i) * D + c] = acc[i] * (kRsqrtD * kLog2e);
        qs[i] = fmaxf(acc[i], 0.f) * kRsqrtD;
        qs[G + i] = fminf(acc[i], 0.f) * kRsqrtD;
    }
}

// ----------------------------------------------------------------------------
// score: one wave per tile of 64 blocks, one lane per block. The tile's keys
// are stored channel-group-major, so each 16-byte load of the wave covers
// 1 KB of contiguous meta. q' enters as wave-uniform (scalar) operands split
// into positive and negative parts: max(q mx, q mn) = q+ mx + q- mn.
// ----------------------------------------------------------------------------
template <typename ST, int G>
__global__ __launch_bounds__(256) void k_score(const DecodeArgs A) {
    const int z = (int)blockIdx.z;
    const int bl = z / A.npk, j = z % A.npk;
    const int b = A.b0 + bl, g = (int)blockIdx.y;
    const DSeg &S = seg_of(A, bl, A.pseg[j]);
    const int wave = (int)(threadIdx.x >> 6), lane = lane_id();
    const int tile = (int)blockIdx.x * 4 + wave;
    const int ntile = (S.nb + META_TILE - 1) / META_TILE;
    if (tile >= ntile) return;
    const int l = tile * META_TILE + lane;
    constexpr int NG = 2 * D * ST::bytes / 16;  // 16-byte groups per block
    constexpr int CPG = D / NG;                 // channels per group
    const int ntile_cap = (S.nbcap + META_TILE - 1) / META_TILE;
    const uint4 *mt = reinterpret_cast<const uint4 *>(static_cast<const char *>(S.meta) +
                                                      ((size_t)g * ntile_cap + tile) * NG * META_TILE * 16);
    const float *__restrict__ qs = A.qs + (((size_t)b * A.hkv + g) * D) * 2 * G;
    float acc[G];
#pragma unroll
    for (int i = 0; i < G; ++i) acc[i] = 0.f;
#pragma unroll 2
    for (int grp = 0; grp < NG; ++grp) {
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
    if (l < S.nb) {
        const int nbc = A.nbcap[j];
#pragma unroll
        for (int i = 0; i < G; ++i)
            A.scores[A.sc_off[j] + ((size_t)b * A.hq + g * G + i) * nbc + l] = acc[i];
        A.mask[A.mk_off[j] + ((size_t)b * A.hkv + g) * nbc + l] = 0u;
    }
}

// ----------------------------------------------------------------------------
// block-wide helpers for 1024-thread workgroups
// ----------------------------------------------------------------------------
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;

struct SelShared {
    int red[2][SEL_WAVES][3];
    uint32_t ured[2][SEL_WAVES][2];
    int scan[SEL_WAVES];
};

__device__ __forceinline__ void block_sum3(SelShared &sh, int &phase, int &a, int &b, int &c) {
    a = wave_sum_i(a);
    b = wave_sum_i(b);
    c = wave_sum_i(c);
    const int w = (int)(threadIdx.x >> 6);
    if (lane_id() == 0) {
        sh.red[phase][w][0] = a;
        sh.red[phase][w][1] = b;
        sh.red[phase][w][2] = c;
    }
    __syncthreads();
    a = b = c = 0;
#pragma unroll
    for (int i = 0; i < SEL_WAVES; ++i) {
        a += sh.red[phase][i][0];
        b += sh.red[phase][i][1];
        c += sh.red[phase][i][2];
    }
    phase ^= 1;
}

__device__ __forceinline__ void block_minmax(SelShared &sh, int &phase, uint32_t &mn, uint32_t &mx) {
    mn = wave_min_u(mn);
    mx = wave_max_u(mx);
    const int w = (int)(threadIdx.x >> 6);
    if (lane_id() == 0) {
        sh.ured[phase][w][0] = mn;
        sh.ured[phase][w][1] = mx;
    }
    __syncthreads();
    mn = 0xFFFFFFFFu;
    mx = 0u;
#pragma unroll
    for (int i = 0; i < SEL_WAVES; ++i) {
        mn = min(mn, sh.ured[phase][i][0]);
        mx = max(mx, sh.ured[phase][i][1]);
    }
    phase ^= 1;
}

// exclusive prefix sum over the workgroup (thread order)
__device__ __forceinline__ int block_excl_scan(SelShared &sh, int v, int &total) {
    const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    __syncthreads();  // sh.scan free
    if (lane == 63) sh.scan[w] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < SEL_WAVES; ++i) {
        const int s = sh.scan[i];
        if (i < w) before += s;
        total += s;
    }
    return before + incl - v;
}

// ----------------------------------------------------------------------------
// select: one 1024-thread workgroup per (request, query head, packed segment).
// Thread t holds the scores of blocks [t*KPT, t*KPT+KPT) as order-preserving
// keys. The k-th largest key is found two bits at a time (counting keys at or
// above three candidates), starting below the bits all keys share. Blocks
// above the threshold are kept, equal ones by ascending block index.
// ----------------------------------------------------------------------------
template <int G, int KPT>
__global__ __launch_bounds__(SEL_THREADS) void k_select(const DecodeArgs A) {
    const int z = (int)blockIdx.z;
    const int bl = z / A.npk, j = z % A.npk;
    const int b = A.b0 + bl, g = (int)blockIdx.y, hi = (int)blockIdx.x;
    const int h = g * G + hi;
    const DSeg &S = seg_of(A, bl, A.pseg[j]);
    const int n = S.nb, k = S.k;
    const int nbc = A.nbcap[j];
    __shared__ SelShared sh;
    int phase = 0;
    const int t = (int)threadIdx.x;

    // sel_out column offset of this packed segment for this request
    int coloff = 0;
    for (int jj = 0; jj < j; ++jj) coloff += seg_of(A, bl, A.pseg[jj]).k;
    int32_t *so = A.sel_out ? A.sel_out + ((size_t)b * A.hq + h) * A.sel_cols : nullptr;
    if (so && j == A.npk - 1) {
        for (int64_t c = coloff + k + t; c < A.sel_cols; c += SEL_THREADS) so[c] = -1;
    }
    if (n <= 0 || k <= 0) return;

    const float *sc = A.scores + A.sc_off[j] + ((size_t)b * A.hq + h) * nbc;
    uint32_t key[KPT];
    const int base = t * KPT;
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = base + i;
        key[i] = idx < n ? score_key(sc[idx]) : 0u;
        if (idx < n) {
            kmn = min(kmn, key[i]);
            kmx = max(kmx, key[i]);
        }
    }
    block_minmax(sh, phase, kmn, kmx);
    uint32_t thr;
    if (k >= n) {
        thr = kmn;
    } else {
        const uint32_t diff = kmn ^ kmx;
        int bit = diff ? 31 - __clz(diff) : -1;
        thr = diff ? (kmx & ~((bit == 31) ? 0xFFFFFFFFu : ((2u << bit) - 1u))) : kmx;
        while (bit >= 0) {
            if (bit >= 1) {
                const uint32_t c1 = thr | (1u << (bit - 1)), c2 = thr | (2u << (bit - 1)),
                               c3 = thr | (3u << (bit - 1));
                int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
                for (int i = 0; i < KPT; ++i) {
                    const bool v = base + i < n;
                    n1 += (v && key[i] >= c1);
                    n2 += (v && key[i] >= c2);
                    n3 += (v && key[i] >= c3);
                }
                block_sum3(sh, phase, n1, n2, n3);
                if (n3 >= k) thr = c3;
                else if (n2 >= k) thr = c2;
                else if (n1 >= k) thr = c1;
                bit -= 2;
            } else {
                const uint32_t c1 = thr | 1u;
                int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
                for (int i = 0; i < KPT; ++i) n1 += (base + i < n && key[i] >= c1);
                block_sum3(sh, phase, n1, n2, n3);
                if (n1 >= k) thr = c1;
                bit -= 1;
            }
        }
    }
    // keys above the threshold, and how many equal ones are needed
    int ngt = 0, neq = 0, dummy = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const bool v = base + i < n;
        ngt += (v && key[i] > thr);
        neq += (v && key[i] == thr);
    }
    int my_eq = neq;
    block_sum3(sh, phase, ngt, neq, dummy);
    const int need = k - ngt;
    int eq_before = 0;
    if (neq > need) {
        int tot;
        eq_before = block_excl_scan(sh, my_eq, tot);
    }
    int cnt = 0;
    uint32_t selbits = 0;  // bit i: block base+i kept (KPT <= 32 per word below)
    bool keepv[KPT];
    int eqr = eq_before;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const bool v = base + i < n;
        bool kp = v && key[i] > thr;
        if (v && key[i] == thr) {
            kp = (neq <= need) || (eqr < need);
            ++eqr;
        }
        keepv[i] = kp;
        cnt += kp;
    }
    (void)selbits;
    int tot;
    const int pos0 = block_excl_scan(sh, cnt, tot);
    int32_t *sl = A.sel + A.sl_off[j] + ((size_t)b * A.hq + h) * A.kcap[j];
    uint32_t *mk = A.mask + A.mk_off[j] + ((size_t)b * A.hkv + g) * nbc;
    int pos = pos0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if (keepv[i] && pos < k) {
            const int idx = base + i;
            sl[pos] = idx;
            if (so) so[coloff + pos] = idx;
            atomicOr(mk + idx, 1u << hi);
            ++pos;
        }
    }
}

// ----------------------------------------------------------------------------
// attend: four waves per workgroup, each wave an independent split of one
// (request, KV head) unit. The unit's work list is, segment by segment,
// dense blocks (all heads) and packed items (rank, head) in rank-major order;
// an item whose block a lower head of the group also selected is skipped, so
// each union block is read once and serves every head that chose it. Splits
// are equal shares of the list weighted by bytes.
// ----------------------------------------------------------------------------
template <typename ST>
struct Loader;
template <>
struct Loader<Bf16> {
    // 8 consecutive stored values starting at element e0 (16-byte aligned)
    __device__ __forceinline__ static void load8(const void *base, int e0, float v[8]) {
        const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const char *>(base) + (size_t)e0 * 2);
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
        v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
};
template <>
struct Loader<F32> {
    __device__ __forceinline__ static void load8(const void *base, int e0, float v[8]) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const char *>(base) + (size_t)e0 * 4);
        const float4 a = p[0], c = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
    }
};

__device__ __forceinline__ void load_idx8(const uint8_t *base, int e0, int ix[8]) {
    const uint2 w = *reinterpret_cast<const uint2 *>(base + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ix[i] = (int)((w.x >> (8 * i)) & (D - 1));
        ix[4 + i] = (int)((w.y >> (8 * i)) & (D - 1));
    }
}

template <int G>
struct WaveState {
    float m[G];   // running max (log2 units), uniform across the wave
    float l;      // lane-private partial sum for lane (t, h)
};

// Online-softmax step over the 16 logits of one block held in zb[t*G + h].
// Lanes t*G+h (< 16G) own one logit each. Returns per-head rescale factors
// (uniform) and leaves p in zb.
template <int G>
__device__ __forceinline__ void softmax_block(float *zb, int nv, int hm, WaveState<G> &st, float alpha[G]) {
    const int lane = lane_id();
    const int t = lane / G, h = lane % G;
    const bool own = lane < 16 * G;
    const bool valid = own && t < nv && ((hm >> h) & 1);
    const float z = valid ? zb[lane] : -INFINITY;
    float bm = z;
#pragma unroll
    for (int o = G; o < 16 * G; o <<= 1) bm = fmaxf(bm, __shfl_xor(bm, o, 64));
    // m for this lane's head
    float mh = st.m[0];
#pragma unroll
    for (int i = 1; i < G; ++i)
        if (h == i) mh = st.m[i];
    float mnew = mh, a = 1.f;
    if (bm != -INFINITY && (mh == -INFINITY || bm > mh + 8.f)) {
        a = (mh == -INFINITY) ? 0.f : exp2f(mh - bm);
        mnew = bm;
    }
    const float p = valid ? exp2f(z - mnew) : 0.f;
    if (own) {
        st.l = st.l * a + p;
        zb[lane] = p;
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
        alpha[i] = __shfl(a, i, 64);
        st.m[i] = __shfl(mnew, i, 64);
    }
}

template <typename ST, int G>
__global__ __launch_bounds__(256) void k_attend(const DecodeArgs A) {
    const int bl = (int)blockIdx.z, g = (int)blockIdx.y;
    const int b = A.b0 + bl;
    const int wave = (int)(threadIdx.x >> 6), lane = lane_id();
    const int s = (int)blockIdx.x * 4 + wave;
    const int S_ = A.S;

    __shared__ __align__(16) float qsh[G][D];
    __shared__ __align__(16) float accs[4][G][D];
    __shared__ __align__(16) float zbs[4][16 * G];
    for (int i = (int)threadIdx.x; i < G * D; i += 256)
        qsh[i / D][i % D] = A.qa[((size_t)b * A.hq + g * G) * D + i];
    __syncthreads();
    if (s >= S_) return;

    float *acc = &accs[wave][0][0];
    float *zb = zbs[wave];
    for (int i = lane; i < G * D; i += 64) acc[i] = 0.f;

    WaveState<G> st;
#pragma unroll
    for (int i = 0; i < G; ++i) st.m[i] = -INFINITY;
    st.l = 0.f;

    // dense-path registers: lane = (token group tg, channel chunk ch)
    const int tg = lane >> 4, ch = lane & 15;
    float qd[G][8], vacc[G][8];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            qd[i][c] = qsh[i][ch * 8 + c];
            vacc[i][c] = 0.f;
        }

    // ---- work partition ----
    const int sb = ST::bytes;
    int64_t W = 0;
    for (int si = 0; si < A.nseg; ++si) {
        const DSeg &S = seg_of(A, bl, si);
        if (S.kind == MKV_SEG_DENSE)
            W += (int64_t)S.nb * (2 * BT * D * sb + 256);
        else
            W += (int64_t)G * S.k * ((G > 1 ? (BT * S.r * 2 * (sb + 1) * 4) / 5 : BT * S.r * 2 * (sb + 1)) + 256);
    }
    const int64_t lo = W * s / S_, hi = W * (s + 1) / S_;
    wave_lds_sync();

    int64_t Wb = 0;
    int pj = 0;
    for (int si = 0; si < A.nseg; ++si) {
        const DSeg &S = seg_of(A, bl, si);
        const bool dense = S.kind == MKV_SEG_DENSE;
        const int64_t w = dense ? (int64_t)(2 * BT * D * sb + 256)
                                : (int64_t)((G > 1 ? (BT * S.r * 2 * (sb + 1) * 4) / 5 : BT * S.r * 2 * (sb + 1)) + 256);
        const int64_t items = dense ? (int64_t)S.nb : (int64_t)G * S.k;
        int64_t i0 = lo - Wb, i1 = hi - Wb;
        i0 = i0 <= 0 ? 0 : (i0 + w - 1) / w;
        i1 = i1 <= 0 ? 0 : (i1 + w - 1) / w;
        if (i0 > items) i0 = items;
        if (i1 > items) i1 = items;
        Wb += items * w;
        const int myj = pj;
        if (!dense) ++pj;
        if (i0 >= i1) continue;

        if (dense) {
            const char *seg_base = static_cast<const char *>(S.data) + (size_t)g * S.nbcap * 2 * BT * D * sb;
            for (int64_t it = i0; it < i1; ++it) {
                const int blk = (int)it;
                const int nv = min(BT, S.filled - blk * BT);
                const char *kb = seg_base + (size_t)blk * 2 * BT * D * sb;
                const char *vb = kb + (size_t)BT * D * sb;
                // logits: lane (tg, ch) covers tokens tg, tg+4, tg+8, tg+12 on channels 8ch..8ch+7
                float part[4][G];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int tt = 4 * ii + tg;
                    float kv[8];
                    Loader<ST>::load8(kb, tt * D + ch * 8, kv);
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        float a = 0.f;
#pragma unroll
                        for (int c = 0; c < 8; ++c) a = fmaf(qd[i][c], kv[c], a);
                        part[ii][i] = a;
                    }
                }
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        float v = part[ii][i];
                        v += __shfl_xor(v, 1, 64);
                        v += __shfl_xor(v, 2, 64);
                        v += __shfl_xor(v, 4, 64);
                        v += __shfl_xor(v, 8, 64);
                        part[ii][i] = v;
                    }
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
                softmax_block<G>(zb, nv, (1 << G) - 1, st, alpha);
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    if (alpha[i] != 1.f) {
                        for (int c = lane; c < D; c += 64) acc[i * D + c] *= alpha[i];
#pragma unroll
                        for (int c = 0; c < 8; ++c) vacc[i][c] *= alpha[i];
                    }
                }
                wave_lds_sync();
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int tt = 4 * ii + tg;
                    float vv[8];
                    Loader<ST>::load8(vb, tt * D + ch * 8, vv);
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        const float p = zb[tt * G + i];
#pragma unroll
                        for (int c = 0; c < 8; ++c) vacc[i][c] = fmaf(p, vv[c], vacc[i][c]);
                    }
                }
                wave_lds_sync();
            }
        } else {
            const int r = S.r;
            const size_t rec = (size_t)BT * r * 2 * (sb + 1);
            const char *seg_base = static_cast<const char *>(S.data) + (size_t)g * S.nbcap * rec;
            const int32_t *sel = A.sel + A.sl_off[myj] + ((size_t)b * A.hq + g * G) * A.kcap[myj];
            const uint32_t *mk = A.mask + A.mk_off[myj] + ((size_t)b * A.hkv + g) * A.nbcap[myj];
            const int nch = 2 * r;               // chunks of 8 elements per half-record
            const uint32_t mr = ((1u << 20) + (uint32_t)r - 1) / (uint32_t)r;  // e / r = (e * mr) >> 20
            for (int64_t it = i0; it < i1; ++it) {
                const int rank = (int)(it / G), hl = (int)(it % G);
                const int blk = sel[(size_t)hl * A.kcap[myj] + rank];
                if ((unsigned)blk >= (unsigned)S.nb) continue;  // never taken for a valid selection
                const int hm = (int)mk[blk];
                if (hm & ((1 << hl) - 1)) continue;  // a lower head already covers this block
                const int nv = min(BT, S.filled - blk * BT);
                const char *base = seg_base + (size_t)blk * rec;
                const void *kval = base;
                const void *vval = base + (size_t)BT * r * sb;
                const uint8_t *kidx = reinterpret_cast<const uint8_t *>(base + (size_t)2 * BT * r * sb);
                const uint8_t *vidx = kidx + BT * r;
                if (lane < 16 * G) zb[lane] = 0.f;
                wave_lds_sync();
                // ---- K: gather-dot into zb[t][h]
                for (int c = lane; c < nch; c += 64) {
                    const int e0 = c * 8;
                    float kv[8];
                    int ix[8];
                    Loader<ST>::load8(kval, e0, kv);
                    load_idx8(kidx, e0, ix);
                    const int t0 = (int)(((uint32_t)e0 * mr) >> 20);
                    if (r >= 8) {
                        const int tb = (t0 + 1) * r;
#pragma unroll
                        for (int i = 0; i < G; ++i) {
                            if (!((hm >> i) & 1)) continue;
                            float s0 = 0.f, s1 = 0.f;
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float pr = qsh[i][ix[e]] * kv[e];
                                if (e0 + e >= tb) s1 += pr; else s0 += pr;
                            }
                            atomicAdd(&zb[t0 * G + i], s0);
                            if (t0 + 1 < BT) atomicAdd(&zb[(t0 + 1) * G + i], s1);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < G; ++i) {
                            if (!((hm >> i) & 1)) continue;
                            int tt = t0, tb = (t0 + 1) * r;
                            float s0 = 0.f;
                            for (int e = 0; e < 8; ++e) {
                                if (e0 + e >= tb) {
                                    atomicAdd(&zb[tt * G + i], s0);
                                    s0 = 0.f;
                                    ++tt;
                                    tb += r;
                                }
                                s0 += qsh[i][ix[e]] * kv[e];
                            }
                            atomicAdd(&zb[tt * G + i], s0);
                        }
                    }
                }
                wave_lds_sync();
                float alpha[G];
                softmax_block<G>(zb, nv, hm, st, alpha);
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    if (alpha[i] != 1.f) {
                        for (int c = lane; c < D; c += 64) acc[i * D + c] *= alpha[i];
#pragma unroll
                        for (int c = 0; c < 8; ++c) vacc[i][c] *= alpha[i];
                    }
                }
                wave_lds_sync();
                // ---- V: scatter-add p * v into acc[h][channel]
                for (int c = lane; c < nch; c += 64) {
                    const int e0 = c * 8;
                    float vv[8];
                    int ix[8];
                    Loader<ST>::load8(vval, e0, vv);
                    load_idx8(vidx, e0, ix);
                    const int t0 = (int)(((uint32_t)e0 * mr) >> 20);
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        if (!((hm >> i) & 1)) continue;
                        int tt = t0, tb = (t0 + 1) * r;
                        float p = zb[tt * G + i];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            while (e0 + e >= tb) {
                                ++tt;
                                tb += r;
                                p = zb[min(tt, BT - 1) * G + i];
                            }
                            atomicAdd(&acc[i * D + ix[e]], p * vv[e]);
                        }
                    }
                }
                wave_lds_sync();
            }
        }
    }

    // fold the dense-path register accumulators into acc
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v = vacc[i][c];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            vacc[i][c] = v;
        }
    wave_lds_sync();
    if (tg == 0) {
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[i * D + ch * 8 + c] += vacc[i][c];
    }
    wave_lds_sync();
    // l per head: sum the lanes (t, h) over t
    float lsum = lane < 16 * G ? st.l : 0.f;
#pragma unroll
    for (int o = G; o < 64; o <<= 1) lsum += __shfl_xor(lsum, o, 64);
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const float li = __shfl(lsum, i, 64);
        float *pp = A.part + (((size_t)b * A.hq + g * G + i) * MAX_SPLITS + s) * PART;
        if (lane == 0) {
            pp[0] = st.m[i];
            pp[1] = li;
        }
        pp[2 + lane] = acc[i * D + lane];
        pp[2 + 64 + lane] = acc[i * D + 64 + lane];
    }
}

// ----------------------------------------------------------------------------
// merge: one workgroup per (request, KV head): combine the splits of each
// head (fixed order), normalise, then out_j = sum_c R_v[c][j] o_c.
// ----------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void k_merge(const DecodeArgs A) {
    const int bl = (int)blockIdx.y, g = (int)blockIdx.x;
    const int b = A.b0 + bl;
    const int t = (int)threadIdx.x;
    const int S_ = A.S;
    __shared__ float wsc[G][MAX_SPLITS];
    __shared__ float Ls[G];
    __shared__ __align__(16) float osh[G][D];
    for (int i = 0; i < G; ++i) {
        const float *pp = A.part + ((size_t)b * A.hq + g * G + i) * MAX_SPLITS * PART;
        if (t < 64) {
            float M = -INFINITY;
            for (int s = t; s < S_; s += 64) M = fmaxf(M, pp[(size_t)s * PART]);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
            float L = 0.f;
            for (int s = t; s < S_; s += 64) {
                const float m = pp[(size_t)s * PART];
                const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
                wsc[i][s] = w;
                L += w * pp[(size_t)s * PART + 1];
            }
            L = wave_sum(L);
            if (t == 0) Ls[i] = L;
        }
    }
    __syncthreads();
    for (int x = t; x < G * D; x += 256) {
        const int i = x / D, c = x % D;
        const float *pp = A.part + ((size_t)b * A.hq + g * G + i) * MAX_SPLITS * PART;
        float o = 0.f;
        for (int s = 0; s < S_; ++s) o = fmaf(wsc[i][s], pp[(size_t)s * PART + 2 + c], o);
        const float L = Ls[i];
        osh[i][c] = L > 0.f ? o / L : 0.f;
    }
    __syncthreads();
    if (t < D) {
        const float *Rv = A.rot + (((size_t)b * A.hkv + g) * 2 + 1) * D * D;
        float acc[G];
#pragma unroll
        for (int i = 0; i < G; ++i) acc[i] = 0.f;
        for (int c = 0; c < D; ++c) {
            const float r = Rv[(size_t)c * D + t];
#pragma unroll
            for (int i = 0; i < G; ++i) acc[i] = fmaf(r, osh[i][c], acc[i]);
        }
#pragma unroll
        for (int i = 0; i < G; ++i) A.out[((size_t)b * A.hq + g * G + i) * D + t] = acc[i];
    }
}

template <int G>
hipError_t select_launch(const DecodeArgs &a, int kpt, hipStream_t s) {
    const dim3 grid((unsigned)G, (unsigned)a.hkv, (unsigned)(a.n_req * a.npk));
    switch (kpt) {
    case 1: hipLaunchKernelGGL((k_select<G, 1>), grid, dim3(SEL_THREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_select<G, 4>), grid, dim3(SEL_THREADS), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_select<G, 16>), grid, dim3(SEL_THREADS), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_select<G, 64>), grid, dim3(SEL_THREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qrot(const DecodeArgs &a, int G, hipStream_t s) {
    const dim3 grid((unsigned)a.hkv, (unsigned)a.n_req);
    switch (G) {
    case 1: hipLaunchKernelGGL(k_qrot<1>, grid, dim3(128), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_qrot<2>, grid, dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_qrot<4>, grid, dim3(128), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_score(const DecodeArgs &a, int dtype, int G, int max_tiles, hipStream_t s) {
    if (a.npk == 0 || max_tiles <= 0) return hipSuccess;
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

hipError_t launch_select(const DecodeArgs &a, int G, int kpt, hipStream_t s) {
    if (a.npk == 0) return hipSuccess;
    if (G == 1) return select_launch<1>(a, kpt, s);
    if (G == 2) return select_launch<2>(a, kpt, s);
    return select_launch<4>(a, kpt, s);
}

hipError_t launch_attend(const DecodeArgs &a, int dtype, int G, hipStream_t s) {
    const dim3 grid((unsigned)((a.S + 3) / 4), (unsigned)a.hkv, (unsigned)a.n_req);
#define MKV_ATT(ST, GG) hipLaunchKernelGGL((k_attend<ST, GG>), grid, dim3(256), 0, s, a)
    if (dtype == MKV_BF16) {
        if (G == 1) MKV_ATT(Bf16, 1); else if (G == 2) MKV_ATT(Bf16, 2); else MKV_ATT(Bf16, 4);
    } else {
        if (G == 1) MKV_ATT(F32, 1); else if (G == 2) MKV_ATT(F32, 2); else MKV_ATT(F32, 4);
    }
#undef MKV_ATT
    return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs &a, int G, hipStream_t s) {
    const dim3 grid((unsigned)a.hkv, (unsigned)a.n_req);
    switch (G) {
    case 1: hipLaunchKernelGGL(k_merge<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_merge<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_merge<4>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mkv
