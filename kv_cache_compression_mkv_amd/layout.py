"""Host-side (numpy) readers of the documented device layouts (include/mkv.h).

Used to inspect what the library stored; no arithmetic of the method here.
"""
from __future__ import annotations

import numpy as np

BT = 16
TILE = 64


def _vals(raw: np.ndarray, dtype: str):
    if dtype == "bf16":
        bits = raw.view(np.uint16)
        return bits, (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bits = raw.view(np.uint32)
    return bits, bits.view(np.float32).astype(np.float64)


def unpack_packed(data: np.ndarray, hkv: int, nbcap: int, r: int, dtype: str):
    """-> dict of K/V values (float64), value bits and indices, each [hkv][nbcap][16][r]."""
    s = 2 if dtype == "bf16" else 4
    rec = BT * r * 2 * (s + 1)
    a = np.ascontiguousarray(data, np.uint8)[:hkv * nbcap * rec].reshape(hkv, nbcap, rec)
    kb, kv = _vals(np.ascontiguousarray(a[:, :, :BT * r * s]).reshape(-1), dtype)
    vb, vv = _vals(np.ascontiguousarray(a[:, :, BT * r * s:2 * BT * r * s]).reshape(-1), dtype)
    ki = a[:, :, 2 * BT * r * s:2 * BT * r * s + BT * r].reshape(hkv, nbcap, BT, r)
    vi = a[:, :, 2 * BT * r * s + BT * r:].reshape(hkv, nbcap, BT, r)
    shp = (hkv, nbcap, BT, r)
    return dict(kval=kv.reshape(shp), vval=vv.reshape(shp), kbits=kb.reshape(shp), vbits=vb.reshape(shp),
                kidx=ki, vidx=vi)


def record_bytes(kind: int, r: int, dtype: str, d: int = 128, group: int = 0) -> int:
    """Bytes of one packed block record (kind 1: u8 indices, kind 2: bitmaps of
    one bit per channel, or per group of `group` channels)."""
    s = 2 if dtype == "bf16" else 4
    return BT * r * 2 * s + (2 * BT * (d // 8 // max(group, 1)) if kind == 2 else 2 * BT * r)


def unpack_bitmap(data: np.ndarray, hkv: int, nbcap: int, r: int, dtype: str, d: int = 128, group: int = 0):
    """Bitmap records -> the fields of unpack_packed (indices are the kept
    channels in ascending order, 0-padded after a vector's last one) plus the
    kept channels as booleans [hkv][nbcap][16][d] (kbm, vbm; with element
    groups, every channel of a set group bit)."""
    s = 2 if dtype == "bf16" else 4
    g = max(group, 1)
    rec = record_bytes(2, r, dtype, d, group)
    a = np.ascontiguousarray(data, np.uint8)[:hkv * nbcap * rec].reshape(hkv, nbcap, rec)
    kb, kv = _vals(np.ascontiguousarray(a[:, :, :BT * r * s]).reshape(-1), dtype)
    vb, vv = _vals(np.ascontiguousarray(a[:, :, BT * r * s:2 * BT * r * s]).reshape(-1), dtype)
    nbm = BT * (d // 8 // g)
    def bits(x):
        gb = np.unpackbits(np.ascontiguousarray(x).reshape(hkv, nbcap, BT, d // 8 // g), axis=-1,
                           bitorder="little").astype(bool)
        return np.repeat(gb, g, axis=-1)
    kbm = bits(a[:, :, 2 * BT * r * s:2 * BT * r * s + nbm])
    vbm = bits(a[:, :, 2 * BT * r * s + nbm:2 * BT * r * s + 2 * nbm])
    def idx(bm):
        out = np.zeros(bm.shape[:3] + (r,), np.uint8)
        ch = np.arange(d)
        for pos in np.ndindex(*bm.shape[:3]):
            sel = ch[bm[pos]][:r]
            out[pos][:sel.size] = sel
        return out
    shp = (hkv, nbcap, BT, r)
    return dict(kval=kv.reshape(shp), vval=vv.reshape(shp), kbits=kb.reshape(shp), vbits=vb.reshape(shp),
                kidx=idx(kbm), vidx=idx(vbm), kbm=kbm, vbm=vbm)


def unpack_records(data: np.ndarray, hkv: int, nbcap: int, r: int, dtype: str, kind: int, d: int = 128,
                   group: int = 0):
    """unpack_packed or unpack_bitmap by segment kind."""
    if kind == 2:
        return unpack_bitmap(data, hkv, nbcap, r, dtype, d, group)
    return unpack_packed(data, hkv, nbcap, r, dtype)


def unpack_dense(data: np.ndarray, hkv: int, nbcap: int, dtype: str, d: int = 128):
    """-> (values float64, bits), each [hkv][nbcap][2][16][d]."""
    bits, vals = _vals(np.ascontiguousarray(data, np.uint8).reshape(-1), dtype)
    shp = (hkv, nbcap, 2, BT, d)
    return vals.reshape(shp), bits.reshape(shp)


def meta_groups(dtype: str, d: int = 128, key_ch: int = 0) -> int:
    """16-byte key groups per block of a packed segment whose keys cover key_ch channels (0: d)."""
    s = 2 if dtype == "bf16" else 4
    return 2 * (key_ch or d) * s // 16


def unpack_meta(meta: np.ndarray, hkv: int, nbcap: int, dtype: str, d: int = 128, key_ch: int = 0):
    """-> (values float64 [hkv][nbcap][2][m] (min, max), bits same shape), m = key_ch or d."""
    ng = meta_groups(dtype, d, key_ch)
    m = key_ch or d
    cpg = m // ng
    ntile = -(-nbcap // TILE)
    raw = np.ascontiguousarray(meta, np.uint8).reshape(hkv, ntile, ng, TILE, 16)
    bits, vals = _vals(np.ascontiguousarray(raw).reshape(-1), dtype)
    # [hkv][ntile][ng][TILE][cpg][2] -> [hkv][ntile*TILE][2][ng*cpg]
    shp = (hkv, ntile, ng, TILE, cpg, 2)
    def re(x):
        x = x.reshape(shp).transpose(0, 1, 3, 5, 2, 4).reshape(hkv, ntile * TILE, 2, ng * cpg)
        return x[:, :nbcap]
    return re(vals), re(bits)
