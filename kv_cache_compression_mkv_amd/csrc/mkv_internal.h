// Internal launch descriptors shared by the host library and the HIP kernels.
//
// Every kernel receives its whole per-launch table by value (kernel arguments
// stay below 4 KB), so no host-to-device copy precedes a launch and the calls
// never synchronise. Requests beyond one table are handled by further launches.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/mkv.h"

namespace mkv {

constexpr int D = MKV_HEAD_DIM;
constexpr int BT = MKV_BLOCK_TOKENS;
constexpr int TABLE = 64;       // (request, segment) entries per launch
constexpr int META_TILE = 64;   // blocks per meta tile

// packed segments of either position format
__host__ __device__ constexpr bool packed_kind(int kind) { return kind == MKV_SEG_PACKED || kind == MKV_SEG_BITMAP; }
// channels covered by a packed segment's block keys (0 means all)
__host__ __device__ constexpr int key_channels(int key_ch) { return key_ch > 0 ? key_ch : D; }
// channels per kept group (0 means single channels)
__host__ __device__ constexpr int group_size(int group) { return group > 1 ? group : 1; }
// position bytes of one vector: u8 indices, or a bitmap of one bit per group
__host__ __device__ constexpr int pos_bytes(int kind, int r, int g) {
    return kind == MKV_SEG_BITMAP ? D / 8 / group_size(g) : r;
}
// bytes of one packed block record (values, then u8 indices or bitmaps)
__host__ __device__ constexpr int64_t record_bytes(int kind, int r, int sb, int g = 1) {
    return (int64_t)BT * r * 2 * sb + (int64_t)2 * BT * pos_bytes(kind, r, g);
}
constexpr int MAX_SPLITS = 256; // attention splits per (request, KV head)
// Partials per (request, query head): one per attend workgroup of 4 splits.
// With S_d + S_p <= MAX_SPLITS there are ceil(S_d / 4) + ceil(S_p / 4) <= 65.
constexpr int MAX_PARTS = MAX_SPLITS / 4 + 1;
constexpr int PART = D + 2;     // floats per split partial: m, l, acc[D]
// Union-mode weight of a packed record: its bytes plus a fixed per-record
// cost. A wave holds about one record in flight, so a record's time is mostly
// its load latency and only a little its size; the constant is the measured
// balance point at 96 KB shares (its cost is worth about 3 KB of bytes).
constexpr int UNION_RECORD_FIXED = 3072;
constexpr int UNION_CAP = 1024;  // union records one packed workgroup can take
// Bytes of packed records per attention split.
constexpr int64_t PACKED_SPLIT = 96 * 1024;
static_assert(UNION_RECORD_FIXED <= 16384, "union weights of a unit stay below 2^32 / 4");

// ---- compression ----------------------------------------------------------
struct CompressEntry {
    void *data;       // segment data
    void *meta;       // packed meta or nullptr
    const float *rot; // the request's rotations [n_kv][2][D][D]: the segment's own or the cache's
    int32_t a, e;     // new tokens occupy local positions [a, e) of the segment
    int32_t row0;     // input row of local position a
    int32_t b;        // request
    int32_t blk0;     // first block touched
    int32_t nblk;     // blocks touched
    int32_t nbcap;    // block capacity of the segment
    uint8_t r;        // kept elements (packed)
    int8_t kind;      // MKV_SEG_*
    uint8_t kch;      // channels of the block keys (packed)
    uint8_t group;    // channels per kept group (1: single channels)
};  // 56 bytes

struct CompressArgs {
    CompressEntry ent[TABLE];
    const void *k_new;
    const void *v_new;
    const float *rot;
    int32_t n_ent, n_kv, n_max;
    int32_t chunk_blocks;  // blocks per workgroup (set by the launcher)
    // optional query rotation run beside the append (staged launches only):
    // workgroups z = n_ent .. n_ent + q_req - 1, x < 4, rotate request z - n_ent
    // with the cache's rotation (q' slot 0 of q_ns)
    const float *q;
    float *qa;
    float *qs;
    int32_t q_req, q_hq, q_G, q_ns;
};
static_assert(sizeof(CompressEntry) == 56, "compress entry layout");
static_assert(sizeof(CompressArgs) <= 4096, "kernel arguments stay below 4 KB");

struct MetaEntry {
    const void *data;
    void *meta;
    int32_t filled, nb, r, b, nbcap, kind;
    int32_t kch;       // channels of the block keys
    int32_t group;     // channels per kept group
};  // 48 bytes

struct MetaArgs {
    MetaEntry ent[TABLE];
    int32_t n_ent, n_kv;
};

// ---- decode ----------------------------------------------------------------
struct DSeg {
    const void *data;
    const void *meta;
    const float *rot; // the segment's own rotations [n_kv][2][D][D], or nullptr (the cache's)
    int8_t kind;
    int8_t group;     // channels per kept group (1: single channels)
    int16_t slot;     // rotation slot: 0 the cache's rotation, else that of the segment index
    int16_t r;
    int16_t kch;      // channels of the block keys (packed)
    int32_t filled;   // tokens stored
    int32_t nb;       // blocks stored
    int32_t k;        // blocks kept (packed)
    int32_t nbcap;    // block capacity (layout stride)
};  // 48 bytes

// ---- sliced select of large packed segments -----------------------------------
// A packed segment of more than BIG_SEL_MIN blocks (in one request, at decode
// time) is selected by slices of BSL blocks, one workgroup each, in three
// launches that share one BigRow per (request, query head, segment).
constexpr int BIG_SEL_MIN = 16384;
constexpr int BSL = 4096;               // blocks per slice: 4 waves x 16 keys per lane
constexpr int BSEL_BINS = 2048;         // key-space bins of the histogram pass
constexpr int BSEL_CAP = 2048;          // candidate keys kept for the exact threshold
constexpr int BSEL_MAX_SLICES = MKV_MAX_PACKED_BLOCKS / BSL;
static_assert(BSEL_MAX_SLICES * BSL == MKV_MAX_PACKED_BLOCKS, "slices cover the largest packed segment");
struct BigRow {
    uint32_t kmin, kmax;       // key range of the segment's scores
    uint32_t bmn, bmx;         // key range of the keys in the threshold bin
    uint32_t ncand;            // keys in the threshold bin (candidates past BSEL_CAP are not stored)
    int32_t bstar, above, inbin;  // threshold bin, keys in higher bins, keys in it
    uint32_t hist[BSEL_BINS];
    int32_t slc[BSEL_MAX_SLICES][2];  // per slice: keys in higher bins, keys in the threshold bin
    uint32_t cand[BSEL_CAP][2];       // (key, slice) of the threshold bin's keys
};
static_assert(sizeof(BigRow) % 16 == 0, "rows stay 16-byte aligned");

struct DecodeArgs {
    DSeg seg[TABLE];  // [n_req][nseg]
    const float *rot;
    const float *q;
    float *out;
    int32_t *sel_out;
    float *qa;        // [B][nslot][Hq][D] q' * log2(e) / sqrt(D), per rotation slot
    float *qs;        // [B][nslot][Hkv][D][2G] (max(q',0), min(q',0)) / sqrt(D)
    float *scores;    // per packed j: [B][Hq][nbcap_j]
    uint32_t *mask;   // per packed j: [B][Hkv][nbcap_j], byte i = 1 if head i of the group chose the block
    int32_t *sel;     // per packed j: [B][Hq][kcap_j]
    float *part;      // [B][Hq][nslot][MAX_PARTS][PART]: one partial per attend workgroup (of 4
                      // splits) of the slot's launch, dense first
    int64_t sel_cols;
    int64_t sc_off[MKV_MAX_SEGMENTS];
    int64_t mk_off[MKV_MAX_SEGMENTS];
    int64_t sl_off[MKV_MAX_SEGMENTS];
    int32_t nbcap[MKV_MAX_SEGMENTS];  // per packed j (max over requests)
    int32_t kcap[MKV_MAX_SEGMENTS];
    int32_t pseg[MKV_MAX_SEGMENTS];   // segment index of packed j
    int32_t b0, n_req, nseg, npk, hq, hkv;
    int32_t S_d;       // dense attention splits per unit (>= 1)
    int32_t S_p;       // packed attention splits per unit (>= 1), S_d + S_p <= MAX_SPLITS
    int32_t sel_kpt;   // keys per lane in select
    int32_t sel_waves; // waves per select workgroup
    int32_t union_mode; // packed workgroups take exact byte shares of the union (S_p a multiple of 4)
    int32_t nslot;      // rotation slots (1 + segment indices with own rotations)
    int32_t cur_slot;   // attend: the slot whose segments this launch attends
    int32_t qrot_from;  // q_rotate: first slot to rotate (1 when the append's launch did slot 0)
    int32_t nparts[MKV_MAX_SEGMENTS + 1];  // merge: partials per slot
    BigRow *big;      // sliced select: per packed j with big_row[j] >= 0, rows [B][Hq] from big_row[j]
    uint32_t *tmm;    // per such j: [B][Hq][ceil(nbcap_j / 64)][2] min and max score key of each 64-block tile
    int64_t tm_off[MKV_MAX_SEGMENTS];
    int32_t big_row[MKV_MAX_SEGMENTS];  // -1: packed j never takes the sliced select (nbcap <= BIG_SEL_MIN)
    int32_t bsel_slices;                // slices of the launch's largest sliced segment (0: none)
    int32_t has_bitmap;                 // attend: the cache's packed segments hold bitmap records
};

static_assert(sizeof(DSeg) == 48, "decode segment layout");
static_assert(sizeof(DecodeArgs) <= 4096, "kernel arguments stay below 4 KB");
constexpr int MAX_SLOTS = MKV_MAX_SEGMENTS + 1;

// Appends touching at most two blocks per (entry, KV head) take one block per
// workgroup and may carry a query rotation; larger ones take COMPRESS_CHUNK.
constexpr bool compress_stages(int max_blk) { return max_blk <= 2; }
constexpr int COMPRESS_CHUNK = 32;

// ---- launchers (defined in the .hip files) --------------------------------
hipError_t launch_compress(const CompressArgs &a, int dtype, int max_blk, hipStream_t s);
hipError_t launch_block_meta(const MetaArgs &a, int dtype, int max_nb, hipStream_t s);
hipError_t launch_qrot(const DecodeArgs &a, int G, hipStream_t s);
hipError_t launch_score(const DecodeArgs &a, int dtype, int G, int max_tiles, hipStream_t s);
hipError_t launch_select(const DecodeArgs &a, int G, hipStream_t s);
hipError_t launch_attend(const DecodeArgs &a, int dtype, int G, int qmax, hipStream_t s);
hipError_t launch_merge(const DecodeArgs &a, int G, hipStream_t s);

// ---- allocation-free decode (noalloc.hip) ----------------------------------
// Device address of the library's scratch array on the device of `stream`
// (looked up once per device, then cached). Bytes: MKV_SCRATCH_BYTES.
hipError_t scratch_address(hipStream_t stream, void **ptr);

}  // namespace mkv
