/* mkv.h -- C ABI of the MosaicKV decode hot path for AMD Instinct MI355X (gfx950).
 *
 * MosaicKV ("MosaicKV: Serving Long-Context LLM with Dynamic Two-D KV Cache
 * Compression", arXiv 2607.00760) compresses a KV cache in two dimensions:
 * every key/value vector is rotated by its head's SVD-derived orthogonal
 * matrix and keeps only its own r largest elements (or whole groups of
 * adjacent channels), stored as packed (channel index, value) pairs or as
 * values with a position bitmap; at decode time each query head scores blocks
 * of 16 tokens from per-block min/max keys, keeps the top-k blocks and runs
 * attention directly on the packed vectors, rotating the result back.
 *
 * Sources cited below:
 *   [N] "MosaicKV 阅读笔记" (reading notes, zhongzhuzhou.org): SVD background
 *       (Eq. 3-5), rotation (Eq. 6-8), per-vector selection (Eq. 9,
 *       Algorithm 1), block score / compressed attention / inverse rotation
 *       (Eq. 12-14), packed sparse attention section, Quest paragraph.
 *   [S] paperlayer.ai summary of the paper: sections 4.2, 4.3, 5.1-5.5, 6.3.
 *
 * Conventions for every call:
 *   - Arguments are validated on the host before anything is enqueued. On an
 *     error nothing is enqueued, no state changes, and a status is returned.
 *   - Device work is enqueued on the caller's HIP stream (`stream` is a
 *     hipStream_t; NULL is the null stream); calls return after the enqueue.
 *     Faults of enqueued work surface at the caller's next synchronisation.
 *   - The library allocates no device memory and keeps no state between calls
 *     apart from the optional kernel-timing facility below (thread-safe).
 *     The caller owns every buffer. Calls on distinct caches are thread-safe; one cache must be
 *     used from one stream at a time.
 *   - Inputs must be finite (NaN/Inf behaviour is unspecified).
 *   - The GPU path supports head_dim == 128, storage MKV_F32 or MKV_BF16, and
 *     1, 2 or 4 query heads per KV head.
 */
#ifndef MKV_H
#define MKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MKV_BLOCK_TOKENS 16        /* tokens per block ([S] 6.3: Quest block size 16) */
#define MKV_HEAD_DIM 128           /* the only head dimension of the GPU path */
#define MKV_MAX_GROUP 4            /* query heads per KV head */
#define MKV_MAX_SEGMENTS 8         /* segments per request */
#define MKV_MAX_PACKED_BLOCKS 65536 /* blocks of one packed segment (1,048,576 tokens) */
#define MKV_PACKED_TAIL_BYTES 256   /* bytes after the last record of a packed data buffer */

typedef enum {
    MKV_OK = 0,
    MKV_ERR_ARG = 1,         /* invalid argument or descriptor */
    MKV_ERR_UNSUPPORTED = 2, /* valid but not supported here (head_dim, dtype, group size) */
    MKV_ERR_CAPACITY = 3,    /* an append would pass a request's total capacity */
    MKV_ERR_WORKSPACE = 4,   /* workspace missing or too small */
    MKV_ERR_NOCONVERGE = 5,  /* eigensolver did not converge */
    MKV_ERR_HIP = 6          /* a HIP launch or event call failed */
} mkv_status;

typedef enum { MKV_F32 = 0, MKV_BF16 = 1 } mkv_dtype;
typedef enum { MKV_SEG_DENSE = 0, MKV_SEG_PACKED = 1, MKV_SEG_BITMAP = 2 } mkv_seg_kind;

/* One segment of one request ([S] 4.1, 4.3: the cache is split into segments,
 * each with its own channel retention and block retention).
 *
 * kind      MKV_SEG_DENSE: tokens are rotated and stored at full width and are
 *           always attended (attention-sink and recent-window segments).
 *           MKV_SEG_PACKED: tokens keep their own r largest rotated elements
 *           ([N] Eq. 9) and blocks are chosen per query head by top-k; each
 *           kept element's position is a u8 channel index.
 *           MKV_SEG_BITMAP: the same, with each vector's kept positions held
 *           as a d-bit bitmap ([S] 5.1: a position bitmap instead of per-element
 *           indices; one bit per channel). "Packed" below means either kind;
 *           the packed segments of one cache all use the same one.
 * r         kept elements per vector, 1..head_dim (packed only).
 * keep_ppm  block keep ratio in parts per million, 1..1000000 (packed only);
 *           k = ceil(keep_ppm * n_blocks / 1e6) in integers, clamped to [1, n].
 * k_abs     if > 0, keep min(k_abs, n_blocks) blocks instead.
 * t_begin   position of the segment's first token; segments of a request are
 *           contiguous and ordered: t_begin[0] = 0, t_begin[j+1] = t_begin[j] + t_cap[j].
 * t_cap     capacity in tokens (> 0).
 * data      device buffer of mkv_segment_bytes() bytes (layout below).
 * meta      device buffer of the meta bytes reported by mkv_segment_bytes()
 *           (packed only; NULL for dense).
 * rot       NULL: the segment's tokens are rotated by the cache's rotation of
 *           the request. Otherwise the segment's own rotation, device float32
 *           [n_kv_heads][2][d][d] (R_k then R_v per KV head, rows as for the
 *           cache's), 16-byte aligned: appends to the segment rotate by it,
 *           and decode scores and attends the segment with q' = R_k,seg q and
 *           rotates its share of the output back by its own R_v,seg ([S] 5.4:
 *           a finished segment recompressed with its own SVD rotation; see
 *           mkv_recompress_segment and mkv_swap_segment).
 * key_ch    packed only: the block keys cover the leading key_ch rotated
 *           channels ([S] 5.2 channel-compresses the per-block keys; the
 *           rotation orders channels by descending singular value), and block
 *           scores sum over those channels only. 0 means all head_dim
 *           channels; otherwise a multiple of 8 in 8..head_dim.
 * group     packed only: 0 or 1, each vector keeps its own r largest elements;
 *           2, 4 or 8 (dividing r), it keeps whole groups of `group` adjacent
 *           channels ([S] 5.1: one position bit per group of adjacent
 *           elements; [S] 4.3: the element-group size): the r / group groups
 *           i (channels group*i ...) of largest energy sum_m x'^2 (binary64,
 *           each square and sum rounded, m ascending), ties to the lower
 *           group. Bitmap records then hold one bit per group.
 * Across the requests of one cache, segment j must have the same kind, r,
 * keep_ppm, k_abs, key_ch and group; t_begin, t_cap and rot may differ per request.
 *
 * Device layouts (s = bytes per stored element, nb = ceil(t_cap / 16),
 * block l holds positions t_begin + 16 l .. t_begin + 16 l + 15, slot = position - block start):
 *   dense data : [n_kv_heads][nb][2][16][d] stored rotated K' (index 0) and V'.
 *   packed data: [n_kv_heads][nb][record], record of 16 * r * 2 * (s + 1) bytes =
 *                K values [16][r] | V values [16][r] | K indices [16][r] u8 |
 *                V indices [16][r] u8; each vector's kept channels in ascending
 *                channel order. Slots of a block past its last token are zero.
 *   bitmap data: [n_kv_heads][nb][record], record of 16 * r * 2 * s + 2 * 16 * n / 8
 *                bytes, n = d / max(group, 1) bits per vector = K values [16][r] |
 *                V values [16][r] | K bitmaps [16][n / 8] | V bitmaps [16][n / 8];
 *                bit i % 8 of byte i / 8 of a vector's bitmap is set iff channel i
 *                (group i) is kept; values in ascending channel order, as above.
 *                MKV_PACKED_TAIL_BYTES follow the last record: decode reads
 *                whole dwords around each record's fields and may touch them
 *                (their contents are never used, nothing writes them).
 *   packed meta: [n_kv_heads][ceil(nb / 64)][2 m s / 16][64][16 bytes] with
 *                m = key_ch (head_dim when 0): for the
 *                block l, lane l % 64 of tile l / 64 holds, per 16-byte group,
 *                the (min, max) pairs of 16 / (2 s) consecutive channels
 *                (bf16: channels 4g..4g+3, f32: 2g..2g+1), min first. min/max are
 *                taken over the block's tokens of the stored sparse keys (0 at
 *                dropped channels) in IEEE totalOrder (-0 < +0).
 */
typedef struct mkv_segment {
    int32_t kind;
    int32_t r;
    int32_t keep_ppm;
    int32_t k_abs;
    int64_t t_begin;
    int64_t t_cap;
    void *data;
    void *meta;
    const float *rot;
    int32_t key_ch;
    int32_t group;
} mkv_segment;

/* A compressed cache for one attention layer of a batch of requests.
 *   segs  host array [batch][n_segments], owned by the caller.
 *   len   host array [batch]: tokens stored per request. Host-authoritative:
 *         mkv_compress_append advances it after enqueueing, so no device-to-host
 *         synchronisation is ever needed.
 *   rot   device [batch][n_kv_heads][2][d][d] float32: R_k (index 0) and R_v,
 *         row c = c-th right singular vector ([N] Eq. 4, 6-8), e.g. from
 *         mkv_rotation_from_prefill. Query head h uses KV head h / (n_q_heads / n_kv_heads).
 */
typedef struct mkv_cache {
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t dtype;
    int32_t n_segments;
    mkv_segment *segs;
    int64_t *len;
    const float *rot;
} mkv_cache;

/* Human-readable name of a status code (static string). */
const char *mkv_status_str(mkv_status s);

/* Rotation of one head from its prefill vectors ([N] Eq. 4, 6-8; [S] 2.3).
 * x_host [T][d] on the host, in `dtype` (f32 values, or bf16 bit patterns as
 * uint16). Computes G = X^T X in float64 (no centering), its eigenvectors by
 * Householder tridiagonalisation and the implicit symmetric QR iteration
 * (Wilkinson shifts), orders them by descending
 * eigenvalue and makes the largest-magnitude entry of each row positive (ties
 * to the lower index). R_out [d][d] host float32 (row c = c-th vector),
 * sigma_out [d] host float64 (nullable) = sqrt(max(eigenvalue, 0)).
 * Synchronous host computation (OpenMP); d in 1..256, T >= 0. The Gram sums
 * run in a fixed order, so R and sigma are bitwise the same whatever the
 * number of host threads.
 * Errors: MKV_ERR_ARG, MKV_ERR_NOCONVERGE. */
mkv_status mkv_rotation_from_prefill(const void *x_host, int32_t dtype, int64_t T, int32_t d,
                                     float *R_out, double *sigma_out);

/* Bytes of the device buffers of one segment: returns the data bytes and
 * writes the meta bytes (0 for dense) to meta_bytes_out (nullable). key_ch and
 * group are those of mkv_segment, ignored for dense. Returns 0 for invalid
 * arguments. */
size_t mkv_segment_bytes(int32_t dtype, int32_t kind, int32_t r, int32_t d, int32_t n_kv_heads,
                         int64_t t_cap, int32_t key_ch, int32_t group, size_t *meta_bytes_out);

/* Compress and append new tokens ([N] Eq. 7-9, Algorithm 1; [S] 4.2, 5.2, 5.4:
 * new vectors are rotated by the head's R, keep their top-r elements and are
 * packed on arrival; prefill uses the same call with many tokens).
 * k_new, v_new: device [batch][n_kv_heads][n_max][d] in the cache dtype; request b
 * appends rows 0 .. n_new[b]-1 at positions len[b] ... (n_new host [batch], each
 * 0..n_max). Each vector is rotated in float64 with exact products (summed in
 * ascending input channel), ranked by the unrounded magnitudes (ties to the
 * lower channel) and rounded once, to nearest even, to the storage type.
 * Packed segments store each vector in their record format (u8 indices or a
 * position bitmap) and update the min/max keys (channels < key_ch) of the
 * blocks they touch.
 * Advances c->len on success.
 * Errors: MKV_ERR_ARG, MKV_ERR_UNSUPPORTED, MKV_ERR_CAPACITY, MKV_ERR_HIP. */
mkv_status mkv_compress_append(mkv_cache *c, const void *k_new, const void *v_new,
                               const int32_t *n_new, int32_t n_max, void *stream);

/* Recompute the per-block min/max keys of packed segment `seg` of every request
 * from its stored records ([N] Quest paragraph; [S] 5.2). The result equals the
 * keys kept up to date by mkv_compress_append, bit for bit.
 * Errors: MKV_ERR_ARG, MKV_ERR_UNSUPPORTED, MKV_ERR_HIP. */
mkv_status mkv_block_meta(const mkv_cache *c, int32_t seg, void *stream);

/* Workspace bytes mkv_decode_attn needs for this cache (sized from capacities,
 * so it does not change as the cache fills; it grows with the number of
 * segment indices whose segment carries its own rotation in some request, so
 * query it again after mkv_swap_segment gives a segment its first own one). */
size_t mkv_decode_workspace_bytes(const mkv_cache *c);

/* Columns of sel_out needed at the current lengths: max over requests of the
 * sum over packed segments of k. */
int64_t mkv_decode_sel_cols(const mkv_cache *c);

/* Decode attention straight from the compressed cache ([N] Eq. 12-14; [S] 4.2,
 * 5.3). For every request b and query head h, with q' = R_k q:
 *   score of block l = (1/sqrt d) sum_c max(q'_c mx_c, q'_c mn_c) over the
 *     block's min/max keys (channels c < key_ch of its segment, all when
 *     key_ch is 0), for every block of every packed segment;
 *   per packed segment, the k blocks of highest score (ties to the lower block);
 *   o = softmax(q' K^T / sqrt d) V^ over every stored dense token and every
 *     token of a selected block, with K^, V^ the packed sparse vectors;
 *   out = o R_v (the inverse rotation).
 * q [batch][n_q_heads][d] device float32; out [batch][n_q_heads][d] device float32.
 * sel_out (nullable) device int32 [batch][n_q_heads][sel_cols]: per packed
 *   segment in order, its k selected block indices (relative to the segment)
 *   ascending, then -1 up to sel_cols (>= mkv_decode_sel_cols()).
 * workspace: device buffer of at least mkv_decode_workspace_bytes() bytes.
 * Scores accumulate in float32, the softmax and the sums in float32. A head
 * with no stored token outputs zeros.
 * Errors: MKV_ERR_ARG, MKV_ERR_UNSUPPORTED, MKV_ERR_WORKSPACE, MKV_ERR_HIP. */
mkv_status mkv_decode_attn(const mkv_cache *c, const float *q, float *out, int32_t *sel_out,
                           int64_t sel_cols, void *workspace, size_t ws_bytes, void *stream);

/* One serving step in one call: mkv_compress_append(c, k_new, v_new, n_new,
 * n_max) and then mkv_decode_attn(c, q, out, sel_out, sel_cols, workspace,
 * ws_bytes), with the same arguments, meaning and results bit for bit ([N]
 * Eq. 7-9 and 12-14; [S] 4.2, 5.2-5.3). When the append is small (at most two
 * blocks per request and segment), the query rotation q' = R_k q runs in the
 * append's launch instead of a launch of its own. Every argument of both
 * parts is checked before anything is enqueued (the decode's at the lengths
 * after the append), so an argument error leaves the cache unchanged; after
 * MKV_ERR_HIP the append may have been enqueued and c->len advanced.
 * Errors: those of both calls. */
mkv_status mkv_append_decode(mkv_cache *c, const void *k_new, const void *v_new, const int32_t *n_new,
                             int32_t n_max, const float *q, float *out, int32_t *sel_out, int64_t sel_cols,
                             void *workspace, size_t ws_bytes, void *stream);

/* Exact recompression of one finished packed segment on the host: the
 * CPU side of the paper's heterogeneous double compression buffering ([S]
 * 5.4; [N] its double-buffering section and Fig. 4), where a segment first
 * compressed on arrival with the request's rotation is re-packed with a
 * rotation of its own and swapped in without blocking decode.
 * For each KV head g: R_k,g and R_v,g from the segment's raw keys and values
 * exactly as mkv_rotation_from_prefill computes them; then every token is
 * rotated in float64 with exact products (summed in ascending input channel),
 * keeps its r largest elements (ties to the lower channel), rounded once to
 * nearest even, and the per-block min/max keys are formed -- the arithmetic
 * of mkv_compress_append, so the result is what the GPU would store with
 * these rotations.
 * k_host, v_host: [n_kv_heads][n_tokens][d] in `dtype` (f32 values or bf16
 *   bit patterns), n_tokens in 1..t_cap.
 * Outputs in the documented device layouts, in host memory the caller owns:
 * kind: the segment's record format, MKV_SEG_PACKED or MKV_SEG_BITMAP;
 * key_ch, group: its block-key channels and element-group size, as in
 * mkv_segment.
 *   data_out [mkv_segment_bytes(dtype, kind, r, d, n_kv_heads, t_cap, key_ch, group)]
 *     (slots after the last token zero; the tail bytes are left as they are),
 *   meta_out [that call's meta bytes] (blocks past the last one zero),
 *   rot_out float32 [n_kv_heads][2][d][d].
 * Synchronous host computation (OpenMP); d == MKV_HEAD_DIM, dtype MKV_F32 or
 * MKV_BF16, r in 1..d. Errors: MKV_ERR_ARG, MKV_ERR_UNSUPPORTED,
 * MKV_ERR_NOCONVERGE. */
mkv_status mkv_recompress_segment(const void *k_host, const void *v_host, int32_t dtype, int32_t d,
                                  int32_t n_kv_heads, int64_t n_tokens, int64_t t_cap, int32_t kind, int32_t r,
                                  int32_t key_ch, int32_t group, void *data_out, void *meta_out, float *rot_out);

/* Segment strategy generation ([S] 4.3 and 5.5: output caches start a new
 * segment when the accumulated compression loss exceeds a threshold or at the
 * maximum length; each segment's strategy holds its rotation and retention;
 * the loss and the covariance are updated incrementally on the host).
 * Host-only, synchronous (OpenMP); meant to run beside decode, like the
 * recompression it feeds.
 *
 * Loss of a set of tokens under a strategy (R, r): the energy of the rotated
 * vectors x' = R x outside each vector's own r largest magnitudes (what the
 * top-r of [N] Eq. 9 drops), over their total rotated energy, summed over the
 * KV heads and over keys and values.
 *
 * k_host, v_host: host [n_kv_heads][row_stride][d] in `dtype` (f32, or bf16 bit
 * patterns as uint16); tokens 0 .. n_tokens-1 of each head (row_stride >= n_tokens).
 * rot, rot0, seg_rot: float32 [n_kv_heads][2][d][d] per strategy (R_k, R_v per
 * head, rows as mkv_rotation_from_prefill's), applied as stored.
 *
 * mkv_strategy_loss_curve: loss_out [d + 1] = the loss for r = 0 .. d of
 * every token under `rot`. */
mkv_status mkv_strategy_loss_curve(const void *k_host, const void *v_host, int32_t dtype, int32_t d,
                                   int32_t n_kv_heads, int64_t n_tokens, int64_t row_stride, const float *rot,
                                   double *loss_out);

/* mkv_strategy_segments: cut one request's token stream into segments and
 * give each its strategy. (rot0, r0) is the strategy in force at token 0
 * (e.g. the previous segment's). A segment ends at a 16-token block boundary
 * once it holds at least min_len tokens and its loss under the strategy in
 * force exceeds cut_loss, or when it holds max_len tokens (a positive
 * multiple of 16; [S] 4.3 uses 64K); the last segment ends with the data.
 * Each segment then gets, per KV head, R_k and R_v from the Gram matrices of
 * its own tokens (accumulated while they are scanned; eigenvectors ordered and
 * signed as in mkv_rotation_from_prefill), and the smallest r in
 * [r_min, r_max] whose loss under them is at most keep_loss (r_max if none);
 * that strategy is in force for the next segment ([S] 5.4: the current
 * segment is compressed with the previous strategy until it is finished).
 * Outputs (host): seg_end [seg_cap] exclusive end token, seg_r [seg_cap],
 * seg_rot [seg_cap][n_kv_heads][2][d][d] (nullable), *n_seg. Sums run in
 * token order per (head, matrix) and combine in a fixed order, so results do
 * not depend on the thread count.
 * Errors: MKV_ERR_ARG (sizes, 0 <= r_min <= r_max <= d, 0 <= r0 <= d,
 * max_len not a positive multiple of 16, NaN thresholds), MKV_ERR_CAPACITY
 * (more than seg_cap segments: the first seg_cap are written and *n_seg =
 * seg_cap), MKV_ERR_NOCONVERGE. */
mkv_status mkv_strategy_segments(const void *k_host, const void *v_host, int32_t dtype, int32_t d,
                                 int32_t n_kv_heads, int64_t n_tokens, int64_t row_stride, const float *rot0,
                                 int32_t r0, double cut_loss, double keep_loss, int32_t r_min, int32_t r_max,
                                 int64_t min_len, int64_t max_len, int64_t seg_cap, int64_t *seg_end,
                                 int32_t *seg_r, float *seg_rot, int64_t *n_seg);

/* Stream-ordered swap of packed segment `seg` of request b to new device
 * buffers (data, meta, rot: as mkv_segment's, e.g. mkv_recompress_segment's
 * outputs copied to the device), without any host wait: if ready_event (a
 * hipEvent_t, nullable) is given, `stream` is made to wait for it (e.g. the
 * end of the copies on another stream), then the descriptor of (b, seg) is
 * pointed at the new buffers. Work enqueued on `stream` before the call reads
 * the old buffers, work enqueued after it the new ones; the caller keeps the
 * old buffers alive until that earlier work is done. The segment must be
 * full (c->len[b] >= t_begin + t_cap) and keep its kind, r and capacity.
 * Errors: MKV_ERR_ARG, MKV_ERR_HIP (the wait could not be enqueued; nothing
 * changed). */
mkv_status mkv_swap_segment(mkv_cache *c, int32_t b, int32_t seg, void *data, void *meta, const float *rot,
                            void *ready_event, void *stream);

/* Decode attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, meaning and results, bit
 * for bit, as mkv_decode_attn with the workspace replaced by the library's own
 * scratch array of MKV_SCRATCH_BYTES bytes: a file-scope device array each
 * device holds from the library's first use on it until the process ends
 * (its address is looked up once per device, on the first call whose stream
 * belongs to that device). The call allocates and frees nothing.
 * Every call on one device shares that device's array, so calls that overlap
 * on one device (concurrent streams or threads) race and must be serialised
 * by the caller; the array keeps the last call's contents, and every byte a
 * call reads it has written earlier in the same call.
 * Errors: those of mkv_decode_attn; MKV_ERR_WORKSPACE when the cache needs
 * more than MKV_SCRATCH_BYTES (mkv_decode_workspace_bytes() tells), checked
 * before anything is enqueued. */
#define MKV_SCRATCH_BYTES (128ull << 20)
mkv_status mkv_decode_attn_noalloc(const mkv_cache *c, const float *q, float *out, int32_t *sel_out,
                                   int64_t sel_cols, void *stream);

/* Optional kernel timing (a diagnostic; process-wide, thread-safe): while
 * enabled, every kernel the library launches, from any thread, is bracketed
 * by HIP events on its stream. This is the library's only state kept between
 * calls: a pool of HIP events and the pairs not yet read.
 * mkv_timing_read synchronises those events and returns, per stage, the summed
 * milliseconds and the number of launches since the last read, then clears
 * them. Stages: 0 compress (with the query rotation when mkv_append_decode
 * runs it there), 1 block_meta, 2 q_rotate, 3 score, 4 select,
 * 5 attend (dense blocks and selected packed blocks), 6 merge (split merge +
 * inverse rotation). */
#define MKV_N_STAGES 7
mkv_status mkv_timing_enable(int32_t on);
mkv_status mkv_timing_read(double *ms_out, int64_t *count_out, int32_t n_stages);
const char *mkv_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif

#endif /* MKV_H */
