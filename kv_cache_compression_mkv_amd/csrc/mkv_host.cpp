// C ABI of the MosaicKV decode path: argument validation, launch planning and
// the optional kernel timing. All device work is in compress.hip / decode.hip.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "mkv_internal.h"

using namespace mkv;

namespace {

// ---------------------------------------------------------------- timing --
struct PendingPair {
    hipEvent_t a, b;
};
struct Timing {
    bool on = false;
    std::vector<PendingPair> pending[MKV_N_STAGES];
    std::vector<hipEvent_t> pool;
    std::mutex mu;
};
Timing &timing() {
    static Timing t;
    return t;
}

hipEvent_t take_event(Timing &t) {
    if (!t.pool.empty()) {
        hipEvent_t e = t.pool.back();
        t.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void give_back(Timing &t, hipEvent_t a, hipEvent_t b) {
    std::lock_guard<std::mutex> g(t.mu);
    if (a) t.pool.push_back(a);
    if (b) t.pool.push_back(b);
}

// Run one launch; while timing is enabled, bracket it with a pair of events on
// its stream. Every access to the shared timing state holds its mutex, and the
// events go back to the pool when a record or the launch fails.
template <class F>
mkv_status timed(int stage, hipStream_t s, F &&launch) {
    Timing &t = timing();
    hipEvent_t a = nullptr, b = nullptr;
    {
        std::lock_guard<std::mutex> g(t.mu);
        if (t.on) {
            a = take_event(t);
            b = a ? take_event(t) : nullptr;
            if (!a || !b) {
                if (a) t.pool.push_back(a);
                return MKV_ERR_HIP;
            }
        }
    }
    if (a && hipEventRecord(a, s) != hipSuccess) {
        give_back(t, a, b);
        return MKV_ERR_HIP;
    }
    if (launch() != hipSuccess) {
        give_back(t, a, b);
        return MKV_ERR_HIP;
    }
    if (a) {
        if (hipEventRecord(b, s) != hipSuccess) {
            give_back(t, a, b);
            return MKV_ERR_HIP;
        }
        std::lock_guard<std::mutex> g(t.mu);
        t.pending[stage].push_back({a, b});
    }
    return MKV_OK;
}

// ------------------------------------------------------------ validation --
int64_t keep_blocks(int64_t n, int32_t keep_ppm, int32_t k_abs) {
    if (n <= 0) return 0;
    int64_t k = k_abs > 0 ? std::min<int64_t>(k_abs, n) : ((int64_t)keep_ppm * n + 999999) / 1000000;
    return std::max<int64_t>(1, std::min(k, n));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int elem_bytes(int32_t dtype) { return dtype == MKV_BF16 ? 2 : 4; }

const mkv_segment &segof(const mkv_cache *c, int b, int j) { return c->segs[(size_t)b * c->n_segments + j]; }

int64_t seg_filled(const mkv_cache *c, int b, int j) {
    const mkv_segment &s = segof(c, b, j);
    return std::max<int64_t>(0, std::min<int64_t>(c->len[b] - s.t_begin, s.t_cap));
}

mkv_status check_cache(const mkv_cache *c) {
    if (!c || !c->segs || !c->len || !c->rot) return MKV_ERR_ARG;
    if (c->batch < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads)
        return MKV_ERR_ARG;
    if (c->n_segments < 1 || c->n_segments > MKV_MAX_SEGMENTS) return MKV_ERR_ARG;
    if (c->dtype != MKV_F32 && c->dtype != MKV_BF16) return MKV_ERR_UNSUPPORTED;
    if (c->head_dim != MKV_HEAD_DIM) return MKV_ERR_UNSUPPORTED;
    const int G = c->n_q_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4) return MKV_ERR_UNSUPPORTED;
    for (int b = 0; b < c->batch; ++b) {
        int64_t t = 0;
        for (int j = 0; j < c->n_segments; ++j) {
            const mkv_segment &s = segof(c, b, j);
            const mkv_segment &s0 = segof(c, 0, j);
            if (s.kind != MKV_SEG_DENSE && !packed_kind(s.kind)) return MKV_ERR_ARG;
            if (s.t_begin != t || s.t_cap < 1 || !s.data) return MKV_ERR_ARG;
            if (s.kind != s0.kind || s.r != s0.r || s.keep_ppm != s0.keep_ppm || s.k_abs != s0.k_abs ||
                s.key_ch != s0.key_ch || s.group != s0.group)
                return MKV_ERR_ARG;
            if (packed_kind(s.kind)) {
                // one position format per cache (u8 indices or bitmaps)
                for (int jj = 0; jj < j; ++jj)
                    if (packed_kind(segof(c, 0, jj).kind) && segof(c, 0, jj).kind != s.kind) return MKV_ERR_ARG;
                if (s.kind == MKV_SEG_BITMAP && c->head_dim != MKV_HEAD_DIM) return MKV_ERR_UNSUPPORTED;
                if (s.r < 1 || s.r > c->head_dim || !s.meta || s.k_abs < 0) return MKV_ERR_ARG;
                if (s.key_ch < 0 || s.key_ch > c->head_dim || s.key_ch % 8) return MKV_ERR_ARG;
                if (s.group != 0 && s.group != 1 && s.group != 2 && s.group != 4 && s.group != 8)
                    return MKV_ERR_ARG;
                if (s.r % group_size(s.group)) return MKV_ERR_ARG;
                if (s.k_abs == 0 && (s.keep_ppm < 1 || s.keep_ppm > 1000000)) return MKV_ERR_ARG;
                if (ceil_div(s.t_cap, BT) > MKV_MAX_PACKED_BLOCKS) return MKV_ERR_UNSUPPORTED;
            }
            if ((reinterpret_cast<uintptr_t>(s.data) & 15) || (reinterpret_cast<uintptr_t>(s.meta) & 15) ||
                (reinterpret_cast<uintptr_t>(s.rot) & 15))
                return MKV_ERR_ARG;
            t += s.t_cap;
        }
        if (t > INT32_MAX) return MKV_ERR_UNSUPPORTED;
        if (c->len[b] < 0 || c->len[b] > t) return MKV_ERR_ARG;
    }
    return MKV_OK;
}

// Rotation slots: slot 0 is the cache's rotation; every segment index whose
// segment carries its own rotation in some request gets a slot of its own
// (slot_of[j], 0 for the others). Returns the number of slots.
int rot_slots(const mkv_cache *c, int (&slot_of)[MKV_MAX_SEGMENTS]) {
    int ns = 1;
    for (int j = 0; j < c->n_segments; ++j) {
        slot_of[j] = 0;
        for (int b = 0; b < c->batch; ++b)
            if (segof(c, b, j).rot) {
                slot_of[j] = ns++;
                break;
            }
    }
    return ns;
}

// ---------------------------------------------------------- workspace map --
struct WsMap {
    size_t qa, qs, scores, mask, sel, part, big, tmm, total;
    int64_t sc_off[MKV_MAX_SEGMENTS], mk_off[MKV_MAX_SEGMENTS], sl_off[MKV_MAX_SEGMENTS];
    int64_t tm_off[MKV_MAX_SEGMENTS];
    int32_t big_row[MKV_MAX_SEGMENTS];
    int32_t nbcap[MKV_MAX_SEGMENTS], kcap[MKV_MAX_SEGMENTS], pseg[MKV_MAX_SEGMENTS];
    int npk;
    int nslot;
    int slot_of[MKV_MAX_SEGMENTS];
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsMap ws_map(const mkv_cache *c) {
    WsMap m{};
    const size_t B = c->batch, Hq = c->n_q_heads, Hkv = c->n_kv_heads;
    const int G = (int)(Hq / Hkv);
    int64_t sc = 0, mk = 0, sl = 0, rows = 0, tm = 0;
    m.npk = 0;
    m.nslot = rot_slots(c, m.slot_of);
    const size_t NS = (size_t)m.nslot;
    for (int j = 0; j < c->n_segments; ++j) {
        if (!packed_kind(segof(c, 0, j).kind)) continue;
        int64_t nbc = 0;
        for (int b = 0; b < c->batch; ++b) nbc = std::max<int64_t>(nbc, ceil_div(segof(c, b, j).t_cap, BT));
        const mkv_segment &s = segof(c, 0, j);
        const int p = m.npk++;
        m.pseg[p] = j;
        m.nbcap[p] = (int32_t)nbc;
        m.kcap[p] = (int32_t)keep_blocks(nbc, s.keep_ppm, s.k_abs);
        m.sc_off[p] = sc;
        m.mk_off[p] = mk;
        m.sl_off[p] = sl;
        sc += (int64_t)(B * Hq) * nbc;
        mk += (int64_t)(B * Hkv) * nbc;
        sl += (int64_t)(B * Hq) * m.kcap[p];
        // segments that can outgrow BIG_SEL_MIN blocks: state of the sliced select
        m.big_row[p] = -1;
        m.tm_off[p] = 0;
        if (nbc > BIG_SEL_MIN) {
            m.big_row[p] = (int32_t)rows;
            m.tm_off[p] = tm;
            rows += (int64_t)(B * Hq);
            tm += (int64_t)(B * Hq) * ceil_div(nbc, META_TILE) * 2;
        }
    }
    size_t off = 0;
    m.qa = off;
    off = align256(off + B * NS * Hq * D * 4);
    m.qs = off;
    off = align256(off + B * NS * Hkv * D * 2 * G * 4);
    m.scores = off;
    off = align256(off + (size_t)sc * 4);
    m.mask = off;
    off = align256(off + (size_t)mk * 4);
    m.sel = off;
    off = align256(off + (size_t)sl * 4);
    m.part = off;
    off = align256(off + B * Hq * NS * MAX_PARTS * PART * 4);
    m.big = off;
    off = align256(off + (size_t)rows * sizeof(BigRow));
    m.tmm = off;
    off = align256(off + (size_t)tm * 4);
    m.total = off;
    return m;
}

int64_t sel_cols_now(const mkv_cache *c) {
    int64_t best = 0;
    for (int b = 0; b < c->batch; ++b) {
        int64_t s = 0;
        for (int j = 0; j < c->n_segments; ++j) {
            const mkv_segment &sg = segof(c, b, j);
            if (!packed_kind(sg.kind)) continue;
            s += keep_blocks(ceil_div(seg_filled(c, b, j), BT), sg.keep_ppm, sg.k_abs);
        }
        best = std::max(best, s);
    }
    return best;
}

}  // namespace

namespace {

// Argument checks of an append; *any tells whether any request appends.
mkv_status append_check(const mkv_cache *c, const void *k_new, const void *v_new, const int32_t *n_new,
                        int32_t n_max, bool *any) {
    if (!n_new || n_max < 0) return MKV_ERR_ARG;
    *any = false;
    for (int b = 0; b < c->batch; ++b) {
        if (n_new[b] < 0 || n_new[b] > n_max) return MKV_ERR_ARG;
        int64_t cap = 0;
        for (int j = 0; j < c->n_segments; ++j) cap += segof(c, b, j).t_cap;
        if (c->len[b] + n_new[b] > cap) return MKV_ERR_CAPACITY;
        *any = *any || n_new[b] > 0;
    }
    if (*any && (!k_new || !v_new)) return MKV_ERR_ARG;
    return MKV_OK;
}

// Query rotation to run beside an append: q and the decode workspace's q'
// buffers (every request of the cache).
struct QrotFuse {
    const float *q;
    float *qa;
    float *qs;
    int nslot;
};

// Enqueue a checked, non-empty append and advance c->len. With `fuse`, the
// first launch also rotates the queries when it is a staged launch; *rotated
// then reports it.
mkv_status append_enqueue(mkv_cache *c, const void *k_new, const void *v_new, const int32_t *n_new, int32_t n_max,
                          hipStream_t s, const QrotFuse *fuse, bool *rotated) {
    if (rotated) *rotated = false;
    std::vector<CompressEntry> ents;
    for (int b = 0; b < c->batch; ++b) {
        const int64_t p0 = c->len[b], p1 = c->len[b] + n_new[b];
        for (int j = 0; j < c->n_segments; ++j) {
            const mkv_segment &sg = segof(c, b, j);
            const int64_t a = std::max(p0, sg.t_begin) - sg.t_begin;
            const int64_t e = std::min(p1, sg.t_begin + sg.t_cap) - sg.t_begin;
            if (e <= a) continue;
            CompressEntry E{};
            E.data = sg.data;
            E.meta = sg.meta;
            E.rot = sg.rot ? sg.rot : c->rot + (size_t)b * c->n_kv_heads * 2 * D * D;
            E.a = (int32_t)a;
            E.e = (int32_t)e;
            E.row0 = (int32_t)(sg.t_begin + a - p0);
            E.b = b;
            E.r = (uint8_t)sg.r;
            E.kind = (int8_t)sg.kind;
            E.group = (uint8_t)group_size(sg.group);
            E.kch = (uint8_t)key_channels(sg.key_ch);
            E.blk0 = (int32_t)(a / BT);
            E.nblk = (int32_t)((e - 1) / BT - a / BT + 1);
            E.nbcap = (int32_t)ceil_div(sg.t_cap, BT);
            ents.push_back(E);
        }
    }
    for (size_t i0 = 0; i0 < ents.size(); i0 += TABLE) {
        CompressArgs A;
        memset(&A, 0, sizeof(A));
        const size_t n = std::min<size_t>(TABLE, ents.size() - i0);
        int max_blk = 0;
        for (size_t i = 0; i < n; ++i) {
            A.ent[i] = ents[i0 + i];
            max_blk = std::max(max_blk, A.ent[i].nblk);
        }
        A.k_new = k_new;
        A.v_new = v_new;
        A.rot = c->rot;
        A.n_ent = (int32_t)n;
        A.n_kv = c->n_kv_heads;
        A.n_max = n_max;
        if (fuse && i0 == 0 && compress_stages(max_blk)) {
            A.q = fuse->q;
            A.qa = fuse->qa;
            A.qs = fuse->qs;
            A.q_req = c->batch;
            A.q_hq = c->n_q_heads;
            A.q_G = c->n_q_heads / c->n_kv_heads;
            A.q_ns = fuse->nslot;
            if (rotated) *rotated = true;
        }
        mkv_status st = timed(0, s, [&] { return launch_compress(A, c->dtype, max_blk, s); });
        if (st != MKV_OK) return st;
    }
    for (int b = 0; b < c->batch; ++b) c->len[b] += n_new[b];
    return MKV_OK;
}

// Argument checks of a decode at the cache's current lengths.
mkv_status decode_check(const mkv_cache *c, const float *q, const float *out, const int32_t *sel_out,
                        int64_t sel_cols, const void *workspace, size_t ws_bytes) {
    if (!q || !out) return MKV_ERR_ARG;
    if (sel_out && sel_cols < sel_cols_now(c)) return MKV_ERR_ARG;
    if (!workspace || ws_bytes < ws_map(c).total || (reinterpret_cast<uintptr_t>(workspace) & 255))
        return MKV_ERR_WORKSPACE;
    return MKV_OK;
}

// Attention splits of one rotation slot's launch: the dense and packed work of
// the segments in that slot, for every request of the launch.
void plan_splits(DecodeArgs &A, const mkv_cache *c, int slot, int G, int sb, int npk) {
    int max_nb = 0;
    int64_t Wmax = 0, Dmax = 0;
    int npk_slot = 0;
    for (int i = 0; i < A.n_req; ++i) {
        int64_t W = 0, Dn = 0;
        for (int j = 0; j < c->n_segments; ++j) {
            const DSeg &D_ = A.seg[i * c->n_segments + j];
            if (D_.slot != slot) continue;
            if (packed_kind(D_.kind)) {
                const int64_t rec = record_bytes(D_.kind, D_.r, sb, D_.group);
                W += (int64_t)G * D_.k * ((G > 1 ? rec * 4 / 5 : rec) + 256);
                max_nb = std::max(max_nb, D_.nb);
            } else {
                Dn += (int64_t)D_.nb * 2 * BT * D * sb;
            }
        }
        Wmax = std::max(Wmax, W);
        Dmax = std::max(Dmax, Dn);
    }
    for (int j = 0; j < c->n_segments; ++j)
        if (packed_kind(A.seg[j].kind) && A.seg[j].slot == slot) ++npk_slot;
    // splits of about 96 KB of packed and 128 KB of dense reads each: both
    // kinds fit one round of resident waves with room to spare (measured
    // on the 128K workload: 88-104 KB packed splits are the fastest; 64 KB
    // fills every wave slot and is slower, 128 KB leaves too few waves)
    A.S_d = (int32_t)std::max<int64_t>(1, std::min<int64_t>(64, ceil_div(Dmax, 128 * 1024)));
    A.S_p = (int32_t)std::max<int64_t>(1, std::min<int64_t>(MAX_SPLITS - A.S_d, ceil_div(Wmax, PACKED_SPLIT)));
    // Union mode (exact byte-balanced packed workgroups) when every packed
    // segment has at most 4096 blocks and a workgroup's share of the union
    // provably fits its UNION_CAP-entry table: a share holds at most
    // U w_max / (P w_min) + npk entries, U = max over requests of the sum
    // over packed segments of min(G k, nb).
    A.union_mode = 0;
    if (npk > 0 && npk <= 4 && max_nb <= 4096 && npk_slot > 0) {
        const int32_t sp4 = (int32_t)std::min<int64_t>(((int64_t)A.S_p + 3) / 4 * 4, (MAX_SPLITS - A.S_d) / 4 * 4);
        int64_t U = 0, wmin = INT64_MAX, wmax = 0;
        for (int i = 0; i < A.n_req; ++i) {
            int64_t u = 0;
            for (int j = 0; j < c->n_segments; ++j) {
                const DSeg &D_ = A.seg[i * c->n_segments + j];
                if (!packed_kind(D_.kind) || D_.slot != slot) continue;
                u += std::min<int64_t>((int64_t)G * D_.k, D_.nb);
                const int64_t w = record_bytes(D_.kind, D_.r, sb, D_.group) + UNION_RECORD_FIXED;
                wmin = std::min(wmin, w);
                wmax = std::max(wmax, w);
            }
            U = std::max(U, u);
        }
        const int64_t P = sp4 / 4;
        if (P >= 1 && ceil_div(U * wmax, P * wmin) + npk <= UNION_CAP) {
            A.union_mode = 1;
            A.S_p = sp4;
        }
    }
}

// Enqueue a checked decode; `rotated`: q' of slot 0 is already in the workspace.
mkv_status decode_enqueue(const mkv_cache *c, const float *q, float *out, int32_t *sel_out, int64_t sel_cols,
                          void *workspace, bool rotated, hipStream_t s) {
    const WsMap m = ws_map(c);
    const int G = c->n_q_heads / c->n_kv_heads;
    const int sb = elem_bytes(c->dtype);
    char *ws = static_cast<char *>(workspace);
    const int per_launch = std::max(1, TABLE / c->n_segments);

    for (int b0 = 0; b0 < c->batch; b0 += per_launch) {
        DecodeArgs A;
        memset(&A, 0, sizeof(A));
        const int n_req = std::min(per_launch, c->batch - b0);
        A.rot = c->rot;
        A.q = q;
        A.out = out;
        A.sel_out = sel_out;
        A.sel_cols = sel_cols;
        A.qa = reinterpret_cast<float *>(ws + m.qa);
        A.qs = reinterpret_cast<float *>(ws + m.qs);
        A.scores = reinterpret_cast<float *>(ws + m.scores);
        A.mask = reinterpret_cast<uint32_t *>(ws + m.mask);
        A.sel = reinterpret_cast<int32_t *>(ws + m.sel);
        A.part = reinterpret_cast<float *>(ws + m.part);
        for (int p = 0; p < m.npk; ++p) {
            A.sc_off[p] = m.sc_off[p];
            A.mk_off[p] = m.mk_off[p];
            A.sl_off[p] = m.sl_off[p];
            A.nbcap[p] = m.nbcap[p];
            A.kcap[p] = m.kcap[p];
            A.pseg[p] = m.pseg[p];
            A.big_row[p] = m.big_row[p];
            A.tm_off[p] = m.tm_off[p];
        }
        A.big = reinterpret_cast<BigRow *>(ws + m.big);
        A.tmm = reinterpret_cast<uint32_t *>(ws + m.tmm);
        A.b0 = b0;
        A.n_req = n_req;
        A.nseg = c->n_segments;
        A.npk = m.npk;
        A.hq = c->n_q_heads;
        A.hkv = c->n_kv_heads;
        A.nslot = m.nslot;
        int max_tiles = 0, max_nb = 0, max_r = 1;
        bool unsliced = false;  // some request's packed segment takes the one-workgroup select
        for (int i = 0; i < n_req; ++i) {
            for (int j = 0; j < c->n_segments; ++j) {
                const mkv_segment &sg = segof(c, b0 + i, j);
                DSeg &D_ = A.seg[i * c->n_segments + j];
                D_.data = sg.data;
                D_.meta = sg.meta;
                D_.rot = sg.rot;
                D_.kind = (int8_t)sg.kind;
                D_.group = (int8_t)group_size(sg.group);
                // a segment index with a slot of its own keeps that slot in
                // every request; requests whose segment has no own rotation
                // there use the cache's, through the slot's launch
                D_.slot = (int16_t)m.slot_of[j];
                D_.r = (int16_t)sg.r;
                D_.kch = (int16_t)key_channels(sg.key_ch);
                D_.filled = (int32_t)seg_filled(c, b0 + i, j);
                D_.nb = (int32_t)ceil_div(D_.filled, BT);
                D_.nbcap = (int32_t)ceil_div(sg.t_cap, BT);
                if (packed_kind(sg.kind)) {
                    D_.k = (int32_t)keep_blocks(D_.nb, sg.keep_ppm, sg.k_abs);
                    max_tiles = std::max(max_tiles, (int)ceil_div(D_.nb, META_TILE));
                    max_r = std::max(max_r, (int)sg.r);
                    // the same rule as the device's: sliced select past BIG_SEL_MIN blocks
                    int p = 0;
                    while (m.pseg[p] != j) ++p;
                    if (m.big_row[p] >= 0 && D_.nb > BIG_SEL_MIN)
                        A.bsel_slices = std::max(A.bsel_slices, (int32_t)ceil_div(D_.nb, BSL));
                    else {
                        max_nb = std::max(max_nb, D_.nb);
                        unsliced = true;
                    }
                }
            }
        }
        // select: the fewest keys per lane (4, 8 or 16) that 16 waves cover;
        // more waves with fewer keys each shorten every phase of this
        // latency-bound kernel. Larger segments take the sliced select.
        static_assert(BIG_SEL_MIN <= 16 * 64 * 16, "one select workgroup covers every unsliced segment");
        const int kpt = max_nb <= 16 * 64 * 4 ? 4 : max_nb <= 16 * 64 * 8 ? 8 : 16;
        A.sel_kpt = unsliced ? kpt : 0;  // 0: no one-workgroup select launch
        A.sel_waves = (int32_t)std::max<int64_t>(1, ceil_div(max_nb, 64 * kpt));

        mkv_status st = MKV_OK;
        A.qrot_from = rotated ? 1 : 0;
        if (A.qrot_from < m.nslot) {
            st = timed(2, s, [&] { return launch_qrot(A, G, s); });
            if (st != MKV_OK) return st;
        }
        if (m.npk > 0) {
            st = timed(3, s, [&] { return launch_score(A, c->dtype, G, max_tiles, s); });
            if (st != MKV_OK) return st;
            st = timed(4, s, [&] { return launch_select(A, G, s); });
            if (st != MKV_OK) return st;
        }
        // one attend launch per rotation slot, each over its slot's segments
        const int qmax = (max_r + 3) / 4;
        for (int slot = 0; slot < m.nslot; ++slot) {
            DecodeArgs As = A;
            As.cur_slot = slot;
            As.has_bitmap = 0;
            for (int j = 0; j < c->n_segments; ++j)
                if (segof(c, 0, j).kind == MKV_SEG_BITMAP) As.has_bitmap = 1;
            plan_splits(As, c, slot, G, sb, m.npk);
            if ((As.S_d + 3) / 4 + (As.S_p + 3) / 4 > MAX_PARTS) return MKV_ERR_UNSUPPORTED;  // (never: S_d + S_p <= 256)
            A.nparts[slot] = (As.S_d + 3) / 4 + (As.S_p + 3) / 4;
            st = timed(5, s, [&] { return launch_attend(As, c->dtype, G, qmax, s); });
            if (st != MKV_OK) return st;
        }
        st = timed(6, s, [&] { return launch_merge(A, G, s); });
        if (st != MKV_OK) return st;
    }
    return MKV_OK;
}

}  // namespace

extern "C" {

const char *mkv_status_str(mkv_status s) {
    switch (s) {
    case MKV_OK: return "ok";
    case MKV_ERR_ARG: return "invalid argument";
    case MKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case MKV_ERR_CAPACITY: return "append exceeds segment capacity";
    case MKV_ERR_WORKSPACE: return "workspace missing or too small";
    case MKV_ERR_NOCONVERGE: return "eigensolver did not converge";
    case MKV_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t mkv_segment_bytes(int32_t dtype, int32_t kind, int32_t r, int32_t d, int32_t n_kv_heads, int64_t t_cap,
                         int32_t key_ch, int32_t group, size_t *meta_bytes_out) {
    if (meta_bytes_out) *meta_bytes_out = 0;
    if ((dtype != MKV_F32 && dtype != MKV_BF16) || d < 1 || n_kv_heads < 1 || t_cap < 1) return 0;
    const size_t s = elem_bytes(dtype);
    const size_t nb = (size_t)ceil_div(t_cap, BT);
    if (kind == MKV_SEG_DENSE) return (size_t)n_kv_heads * nb * 2 * BT * d * s;
    if (!packed_kind(kind) || r < 1 || r > d || (kind == MKV_SEG_BITMAP && d != D)) return 0;
    if (key_ch < 0 || key_ch > d || key_ch % 8) return 0;
    if ((group != 0 && group != 1 && group != 2 && group != 4 && group != 8) || r % group_size(group)) return 0;
    if (meta_bytes_out) {
        const size_t ntile = ceil_div((int64_t)nb, META_TILE);
        *meta_bytes_out = (size_t)n_kv_heads * ntile * META_TILE * 2 * (key_ch > 0 ? key_ch : d) * s;
    }
    return (size_t)n_kv_heads * nb * record_bytes(kind, r, s, group) + MKV_PACKED_TAIL_BYTES;
}

mkv_status mkv_compress_append(mkv_cache *c, const void *k_new, const void *v_new, const int32_t *n_new,
                               int32_t n_max, void *stream) {
    mkv_status st = check_cache(c);
    if (st != MKV_OK) return st;
    bool any = false;
    st = append_check(c, k_new, v_new, n_new, n_max, &any);
    if (st != MKV_OK || !any) return st;
    return append_enqueue(c, k_new, v_new, n_new, n_max, static_cast<hipStream_t>(stream), nullptr, nullptr);
}

mkv_status mkv_block_meta(const mkv_cache *c, int32_t seg, void *stream) {
    mkv_status st = check_cache(c);
    if (st != MKV_OK) return st;
    if (seg < 0 || seg >= c->n_segments || !packed_kind(segof(c, 0, seg).kind)) return MKV_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int b0 = 0; b0 < c->batch; b0 += TABLE) {
        MetaArgs A;
        memset(&A, 0, sizeof(A));
        const int n = std::min(TABLE, c->batch - b0);
        int max_nb = 0;
        for (int i = 0; i < n; ++i) {
            const mkv_segment &sg = segof(c, b0 + i, seg);
            MetaEntry &E = A.ent[i];
            E.data = sg.data;
            E.meta = sg.meta;
            E.filled = (int32_t)seg_filled(c, b0 + i, seg);
            E.nb = (int32_t)ceil_div(E.filled, BT);
            E.r = sg.r;
            E.b = b0 + i;
            E.nbcap = (int32_t)ceil_div(sg.t_cap, BT);
            E.kind = sg.kind;
            E.kch = key_channels(sg.key_ch);
            E.group = group_size(sg.group);
            max_nb = std::max(max_nb, E.nb);
        }
        A.n_ent = n;
        A.n_kv = c->n_kv_heads;
        st = timed(1, s, [&] { return launch_block_meta(A, c->dtype, max_nb, s); });
        if (st != MKV_OK) return st;
    }
    return MKV_OK;
}

mkv_status mkv_swap_segment(mkv_cache *c, int32_t b, int32_t seg, void *data, void *meta, const float *rot,
                            void *ready_event, void *stream) {
    mkv_status st = check_cache(c);
    if (st != MKV_OK) return st;
    if (b < 0 || b >= c->batch || seg < 0 || seg >= c->n_segments) return MKV_ERR_ARG;
    mkv_segment &sg = c->segs[(size_t)b * c->n_segments + seg];
    if (!packed_kind(sg.kind) || !data || !meta || !rot) return MKV_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(data) & 15) || (reinterpret_cast<uintptr_t>(meta) & 15) ||
        (reinterpret_cast<uintptr_t>(rot) & 15))
        return MKV_ERR_ARG;
    if (c->len[b] < sg.t_begin + sg.t_cap) return MKV_ERR_ARG;  // only a finished segment is swapped
    if (ready_event &&
        hipStreamWaitEvent(static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ready_event), 0) != hipSuccess)
        return MKV_ERR_HIP;
    sg.data = data;
    sg.meta = meta;
    sg.rot = rot;
    return MKV_OK;
}

size_t mkv_decode_workspace_bytes(const mkv_cache *c) {
    if (check_cache(c) != MKV_OK) return 0;
    return ws_map(c).total;
}

int64_t mkv_decode_sel_cols(const mkv_cache *c) {
    if (check_cache(c) != MKV_OK) return -1;
    return sel_cols_now(c);
}

mkv_status mkv_decode_attn(const mkv_cache *c, const float *q, float *out, int32_t *sel_out, int64_t sel_cols,
                           void *workspace, size_t ws_bytes, void *stream) {
    mkv_status st = check_cache(c);
    if (st != MKV_OK) return st;
    st = decode_check(c, q, out, sel_out, sel_cols, workspace, ws_bytes);
    if (st != MKV_OK) return st;
    return decode_enqueue(c, q, out, sel_out, sel_cols, workspace, false, static_cast<hipStream_t>(stream));
}

mkv_status mkv_decode_attn_noalloc(const mkv_cache *c, const float *q, float *out, int32_t *sel_out,
                                   int64_t sel_cols, void *stream) {
    mkv_status st = check_cache(c);
    if (st != MKV_OK) return st;
    if (ws_map(c).total > MKV_SCRATCH_BYTES) return MKV_ERR_WORKSPACE;
    if (!q || !out) return MKV_ERR_ARG;
    if (sel_out && sel_cols < sel_cols_now(c)) return MKV_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (scratch_address(s, &ws) != hipSuccess) return MKV_ERR_HIP;
    st = decode_check(c, q, out, sel_out, sel_cols, ws, MKV_SCRATCH_BYTES);
    if (st != MKV_OK) return st;
    return decode_enqueue(c, q, out, sel_out, sel_cols, ws, false, s);
}

mkv_status mkv_append_decode(mkv_cache *c, const void *k_new, const void *v_new, const int32_t *n_new,
                             int32_t n_max, const float *q, float *out, int32_t *sel_out, int64_t sel_cols,
                             void *workspace, size_t ws_bytes, void *stream) {
    mkv_status st = check_cache(c);
    if (st != MKV_OK) return st;
    bool any = false;
    st = append_check(c, k_new, v_new, n_new, n_max, &any);
    if (st != MKV_OK) return st;
    // the decode's arguments are checked at the lengths after the append
    std::vector<int64_t> len0(c->len, c->len + c->batch);
    for (int b = 0; b < c->batch; ++b) c->len[b] += n_new[b];
    st = decode_check(c, q, out, sel_out, sel_cols, workspace, ws_bytes);
    for (int b = 0; b < c->batch; ++b) c->len[b] = len0[b];
    if (st != MKV_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool rotated = false;
    if (any) {
        const WsMap m = ws_map(c);
        char *ws = static_cast<char *>(workspace);
        const QrotFuse f{q, reinterpret_cast<float *>(ws + m.qa), reinterpret_cast<float *>(ws + m.qs), m.nslot};
        st = append_enqueue(c, k_new, v_new, n_new, n_max, s, &f, &rotated);
        if (st != MKV_OK) return st;
    }
    return decode_enqueue(c, q, out, sel_out, sel_cols, workspace, rotated, s);
}

mkv_status mkv_timing_enable(int32_t on) {
    Timing &t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    t.on = on != 0;
    return MKV_OK;
}

mkv_status mkv_timing_read(double *ms_out, int64_t *count_out, int32_t n_stages) {
    if (!ms_out || !count_out || n_stages < 0) return MKV_ERR_ARG;
    Timing &t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    mkv_status st = MKV_OK;
    for (int i = 0; i < MKV_N_STAGES; ++i) {
        double ms = 0.0;
        for (PendingPair &p : t.pending[i]) {
            float e = 0.f;
            if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&e, p.a, p.b) != hipSuccess)
                st = MKV_ERR_HIP;
            ms += e;
            t.pool.push_back(p.a);
            t.pool.push_back(p.b);
        }
        if (i < n_stages) {
            ms_out[i] = ms;
            count_out[i] = (int64_t)t.pending[i].size();
        }
        t.pending[i].clear();
    }
    return st;
}

const char *mkv_stage_name(int32_t stage) {
    static const char *names[MKV_N_STAGES] = {"compress", "block_meta", "q_rotate", "score",
                                              "select",   "attend",     "merge"};
    return (stage >= 0 && stage < MKV_N_STAGES) ? names[stage] : "unknown";
}

}  // extern "C"
