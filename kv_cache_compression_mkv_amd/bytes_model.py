"""Byte accounting for the compressed cache and for one decode call.

Host-side arithmetic used to report achieved bandwidth; no device work.

Layout facts (the library's documented storage, see include/mkv.h):
  * packed record of one 16-token block: K values, V values, K indices (u8),
    V indices (u8), each [16][r]  ->  16 * r * 2 * (s + 1) bytes;
  * per-block keys (min and max of each of the m = key_ch leading channels,
    all d when key_ch is 0): 2 * m * s bytes;
  * dense block of 16 tokens: 16 * 2 * d * s bytes.
"""
from __future__ import annotations

BLOCK = 16


def dense_kv_bytes(tokens: int, d: int, s: int) -> int:
    """K and V of `tokens` tokens of one head: Eq. 2 of the reading notes per layer and head."""
    return 2 * tokens * d * s


def packed_record_bytes(r: int, s: int, bitmap: bool = False, d: int = 128, group: int = 0) -> int:
    """One block record: K and V values, then u8 indices or (bitmap) position bitmaps of one
    bit per channel, or per group of `group` channels."""
    return BLOCK * r * 2 * s + (2 * BLOCK * (d // 8 // max(group, 1)) if bitmap else BLOCK * r * 2)


def meta_block_bytes(d: int, s: int, key_ch: int = 0) -> int:
    return 2 * (key_ch or d) * s


def quest_key_overhead(block: int = BLOCK) -> float:
    """Per-block min+max keys relative to the block's dense K+V (paper section 6.3)."""
    return meta_block_bytes(128, 2) / dense_kv_bytes(block, 128, 2)


def notes_compressed_bytes(tokens: int, r: int, alpha: float, s: int, idx_bytes: int) -> dict:
    """The reading notes' own accounting (Eq. 20-22): all-token K at r channels,
    exact K/V of the selected tokens, and one index per kept element."""
    k_all = tokens * r * s
    sel = int(round(alpha * tokens)) * r * s * 2
    idx = tokens * r * idx_bytes
    return dict(k_all=k_all, selected=sel, indices=idx, total=k_all + sel + idx)


def keep_blocks(n: int, keep_ppm: int, k_abs: int) -> int:
    """Blocks a packed segment keeps (the rule of include/mkv.h): k_abs if set,
    else ceil(keep_ppm * n / 1e6) in integers; clamped to [1, n]; 0 if n = 0."""
    if n <= 0:
        return 0
    k = min(k_abs, n) if k_abs > 0 else (keep_ppm * n + 999999) // 1000000
    return max(1, min(k, n))


def theoretical_speedup(alpha: float, beta: float) -> float:
    """T*d / (s_selected * r) = 1 / (alpha * beta) (reading notes, Eq. 15)."""
    return 1.0 / (alpha * beta)


def decode_call_bytes(d: int, s: int, hkv: int, batch: int, hq: int, seg_summary) -> dict:
    """Algorithmic bytes one decode call must read.

    seg_summary: list over requests of lists over segments of dicts with
      kind ('dense'|'packed'), filled tokens, r, n_blocks, union (the number of
      distinct blocks selected by the query heads of a KV head, summed over KV
      heads of the request).
    Counts: every block's keys (all KV heads), each union record once, every
    dense token, R_k and R_v per unit, plus the queries read and outputs written.
    """
    meta = records = dense = 0
    for req in seg_summary:
        for sg in req:
            if sg["kind"] == "packed":
                meta += sg["n_blocks"] * hkv * meta_block_bytes(d, s, sg.get("key_ch", 0))
                records += sg["union"] * packed_record_bytes(sg["r"], s, sg.get("bitmap", False), d,
                                                             sg.get("group", 0))
            else:
                dense += dense_kv_bytes(sg["filled"], d, s) * hkv
    rot = batch * hkv * 2 * d * d * 4
    qo = 2 * batch * hq * d * 4
    return dict(meta=meta, records=records, dense=dense, rot=rot, qo=qo,
                total=meta + records + dense + rot + qo)


def append_bytes(d: int, s: int, hkv: int, batch: int, r: int, bitmap: bool = False, key_ch: int = 0,
                 group: int = 0) -> int:
    """Algorithmic bytes of appending one token per request to a packed
    segment: per (request, KV head) read R_k and R_v (float32) and the raw key
    and value, write the two packed vectors (r values and r u8 indices, or a
    d-bit bitmap, each) and read and write the block's min/max keys."""
    pos = d // 8 // max(group, 1) if bitmap else r
    per_unit = 2 * d * d * 4 + 2 * d * s + 2 * (r * s + pos) + 2 * meta_block_bytes(d, s, key_ch)
    return batch * hkv * per_unit
