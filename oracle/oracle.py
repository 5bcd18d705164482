"""Python entry to the fp64 CPU oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The product library never does, and this module imports
nothing from the product package.

Every function here is marshalling around oracle.c; the arithmetic lives
there (see its header for the passages each step follows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_LIB = None

DTYPES = {"f32": 0, "bf16": 1, "f64": 2}
DENSE, PACKED, BITMAP = 0, 1, 2  # BITMAP: packed, positions stored as bitmaps (same kept set)
BLOCK = 16


def build(force: bool = True) -> str:
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC",
                               "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _LIB
    if _LIB is None:
        build(force=False)
        L = ctypes.CDLL(_SO)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.orc_round_e8.restype = ctypes.c_uint32
        L.orc_round_e8.argtypes = [ctypes.c_double, ctypes.c_int]
        L.orc_decode_e8.restype = ctypes.c_double
        L.orc_decode_e8.argtypes = [ctypes.c_uint32, ctypes.c_int]
        L.orc_round_array.restype = None
        L.orc_round_array.argtypes = [P, I64, ctypes.c_int, P, P]
        L.orc_rotation.restype = ctypes.c_int
        L.orc_rotation.argtypes = [P, I64, ctypes.c_int, P, P, ctypes.c_int]
        L.orc_topr.restype = None
        L.orc_topr.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
        L.orc_topr_groups.restype = None
        L.orc_topr_groups.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
        L.orc_block_keep.restype = I64
        L.orc_block_keep.argtypes = [I64, I32, I32]
        L.orc_compress_unit.restype = ctypes.c_int
        L.orc_compress_unit.argtypes = [ctypes.c_int, I64, I64, ctypes.c_int, ctypes.c_int, P, P, P, P, P,
                                        ctypes.c_int, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
        L.orc_decode_unit.restype = ctypes.c_int
        L.orc_decode_unit.argtypes = [ctypes.c_int, I64, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P,
                                      ctypes.c_int, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                      ctypes.c_int]
        _LIB = L
    return _LIB


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 64))


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# --------------------------------------------------------------------------
def round_to(x, dtype: str):
    """Stored value (as float64) of each element after one nearest-even rounding."""
    x = _c(x, np.float64)
    out = np.empty_like(x)
    bits = np.empty(x.shape, np.uint32)
    _lib().orc_round_array(x.ctypes.data, x.size, DTYPES[dtype], out.ctypes.data, bits.ctypes.data)
    return out


def round_bits(x, dtype: str):
    """Bit pattern (uint32; bf16 in the low 16 bits) of the rounded value."""
    x = _c(x, np.float64)
    out = np.empty_like(x)
    bits = np.empty(x.shape, np.uint32)
    _lib().orc_round_array(x.ctypes.data, x.size, DTYPES[dtype], out.ctypes.data, bits.ctypes.data)
    return bits


def rotation(X, nthreads: int | None = None):
    """(R [d][d] float64, sigma [d]) from prefill rows X [T][d]."""
    X = _c(X, np.float64)
    T, d = X.shape
    R = np.empty((d, d), np.float64)
    sig = np.empty(d, np.float64)
    rc = _lib().orc_rotation(X.ctypes.data, T, d, R.ctypes.data, sig.ctypes.data, nthreads or threads())
    if rc != 0:
        raise RuntimeError("oracle rotation failed (%d)" % rc)
    return R, sig


def topr(xr, r: int):
    xr = _c(xr, np.float64)
    idx = np.empty(r, np.int32)
    _lib().orc_topr(xr.ctypes.data, xr.size, r, idx.ctypes.data)
    return idx


def topr_groups(xr, r: int, g: int):
    """Kept channels (ascending) of the r / g highest-energy groups of g adjacent channels."""
    xr = _c(xr, np.float64)
    assert xr.size % g == 0 and r % g == 0
    idx = np.empty(r, np.int32)
    _lib().orc_topr_groups(xr.ctypes.data, xr.size, r, g, idx.ctypes.data)
    return idx


def _groups(segs):
    """Per segment: channels per kept group (1: single channels)."""
    for s in segs:
        g = s.get("group", 0) or 1
        if g > 1 and s["kind"] != DENSE and s["r"] % g:
            raise ValueError("group %d does not divide r = %d" % (g, s["r"]))
    return _c([s.get("group", 0) or 1 for s in segs], np.int32)


def block_keep(n: int, keep_ppm: int, k_abs: int) -> int:
    return int(_lib().orc_block_keep(n, keep_ppm, k_abs))


def _seg_arrays(segs):
    kind = _c([DENSE if s["kind"] == DENSE else PACKED for s in segs], np.int32)
    tb = _c([s["t_begin"] for s in segs], np.int64)
    cap = _c([s["t_cap"] for s in segs], np.int64)
    r = _c([s["r"] for s in segs], np.int32)
    keep = _c([s["keep_ppm"] for s in segs], np.int32)
    kabs = _c([s["k_abs"] for s in segs], np.int32)
    return kind, tb, cap, r, keep, kabs


def _key_channels(segs):
    """Per segment: the leading rotated channels its block keys cover (0: all)."""
    return _c([s.get("key_ch", 0) for s in segs], np.int32)


def seg_blocks(segs, length: int, block: int = BLOCK):
    """Per packed segment: (n_blocks, k) at the given request length."""
    out = []
    for s in segs:
        if s["kind"] == DENSE:
            continue
        filled = min(max(length - s["t_begin"], 0), s["t_cap"])
        nb = -(-filled // block)
        out.append((nb, block_keep(nb, s["keep_ppm"], s["k_abs"])))
    return out


def _seg_rot_table(seg_rot, nseg, d):
    """(ctypes pointer array, kept arrays) for per-segment rotations: seg_rot is
    None or a list (per segment) of None or (R_k, R_v) [d][d]."""
    if seg_rot is None:
        return None, []
    assert len(seg_rot) == nseg
    keep = [None if x is None else _c(np.stack([x[0], x[1]]), np.float64).reshape(2, d, d) for x in seg_rot]
    tab = (ctypes.c_void_p * nseg)(*[None if a is None else a.ctypes.data for a in keep])
    return tab, keep


def compress_unit(Kraw, Vraw, Rk, Rv, segs, length: int, dtype: str, block: int = BLOCK,
                  nthreads: int | None = None, state=None, seg_rot=None):
    """Compress one (request, KV head) unit. Returns a dict with Khat, Vhat, Kidx, Vidx
    ([len][d]) and meta: list (one per packed segment) of [n_blocks][2][d].

    state: a dict returned by an earlier call on the same unit; then only the
    tokens from its length on are compressed, into the same arrays (their row
    capacity is the row count of the raw inputs given the first time).
    seg_rot: per segment, None or its own (R_k, R_v), which then replace Rk, Rv
    for that segment's tokens (kept in the state for decode_unit)."""
    if Kraw.shape[0] < length or Vraw.shape[0] < length:
        raise ValueError("compress_unit: %d input rows for length %d" % (min(Kraw.shape[0], Vraw.shape[0]), length))
    d = Kraw.shape[1]
    Rk, Rv = _c(Rk, np.float64), _c(Rv, np.float64)
    kind, tb, cap, r, keep, kabs = _seg_arrays(segs)
    nbcaps = [-(-s["t_cap"] // block) for s in segs if s["kind"] != DENSE]
    if state is None:
        rows = max(Kraw.shape[0], length, 1)
        st = dict(Khat=np.zeros((rows, d)), Vhat=np.zeros((rows, d)), Kidx=np.full((rows, d), -1, np.int16),
                  Vidx=np.full((rows, d), -1, np.int16), meta_flat=np.zeros((max(sum(nbcaps), 1), 2, d)),
                  length=0, segs=segs, dtype=dtype, block=block, seg_rot=seg_rot)
    else:
        st = state
        if st["Khat"].shape[0] < length:
            raise ValueError("compress_unit: state holds %d rows, need %d" % (st["Khat"].shape[0], length))
        if seg_rot is not None:
            st["seg_rot"] = seg_rot
    tab, _rot_arrays = _seg_rot_table(st.get("seg_rot"), len(segs), d)
    t_from = st["length"]
    grp = _groups(segs)
    Kin = _c(Kraw[:length], np.float64)
    Vin = _c(Vraw[:length], np.float64)
    rc = _lib().orc_compress_unit(d, length, t_from, DTYPES[dtype], block, Kin.ctypes.data, Vin.ctypes.data,
                                  Rk.ctypes.data, Rv.ctypes.data, tab, len(segs), kind.ctypes.data,
                                  tb.ctypes.data, cap.ctypes.data, r.ctypes.data, grp.ctypes.data,
                                  st["Khat"].ctypes.data,
                                  st["Vhat"].ctypes.data, st["Kidx"].ctypes.data, st["Vidx"].ctypes.data,
                                  st["meta_flat"].ctypes.data, nthreads or threads())
    if rc != 0:
        raise RuntimeError("oracle compress failed (%d)" % rc)
    st["length"] = length
    metas, o = [], 0
    for (nb, _), nbc in zip(seg_blocks(segs, length, block), nbcaps):
        metas.append(st["meta_flat"][o:o + nb])
        o += nbc
    st["meta"] = metas
    return st


def decode_unit(comp, q, Rk, Rv, forced_sel=None, nthreads: int | None = None):
    """Decode attention for the G query heads q [G][d] of one compressed unit
    (with the per-segment rotations the unit was compressed with, if any).

    forced_sel: optional list (per packed segment) of [G][k] block lists that
    replace the top-k. Returns dict(qrot [G][d], scores [list per seg of [G][n]],
    sel [list per seg of [G][k]], tau [G][npacked], out [G][d])."""
    q = _c(q, np.float64)
    G, d = q.shape
    segs, length, block = comp["segs"], comp["length"], comp["block"]
    kind, tb, cap, r, keep, kabs = _seg_arrays(segs)
    kch = _key_channels(segs)
    nk = seg_blocks(segs, length, block)
    nsum = sum(n for n, _ in nk)
    ksum = sum(k for _, k in nk)
    npk = len(nk)
    qrot = np.empty((G, d)); out = np.empty((G, d))
    scores = np.empty((G, max(nsum, 1))); sel = np.empty((G, max(ksum, 1)), np.int32)
    tau = np.empty((G, max(npk, 1)))
    fs = None
    if forced_sel is not None:
        fs = np.concatenate([np.asarray(s, np.int32).reshape(G, -1) for s in forced_sel], axis=1) \
            if npk else np.zeros((G, 1), np.int32)
        fs = _c(fs, np.int32)
        assert fs.shape[1] == max(ksum, 1) or (ksum == 0)
    tab, _rot_arrays = _seg_rot_table(comp.get("seg_rot"), len(segs), d)
    rc = _lib().orc_decode_unit(d, length, G, block, comp["Khat"].ctypes.data, comp["Vhat"].ctypes.data,
                                comp["Kidx"].ctypes.data, comp["Vidx"].ctypes.data,
                                comp["meta_flat"].ctypes.data, tab, len(segs), kind.ctypes.data,
                                tb.ctypes.data, cap.ctypes.data, r.ctypes.data, keep.ctypes.data,
                                kabs.ctypes.data, kch.ctypes.data, q.ctypes.data, _c(Rk, np.float64).ctypes.data,
                                _c(Rv, np.float64).ctypes.data,
                                fs.ctypes.data if fs is not None else None, qrot.ctypes.data,
                                scores.ctypes.data, sel.ctypes.data, tau.ctypes.data, out.ctypes.data,
                                nthreads or threads())
    if rc != 0:
        raise RuntimeError("oracle decode failed (%d)" % rc)
    sc_list, sel_list, o1, o2 = [], [], 0, 0
    for n, k in nk:
        sc_list.append(scores[:, o1:o1 + n])
        sel_list.append(sel[:, o2:o2 + k])
        o1 += n
        o2 += k
    return dict(qrot=qrot, scores=sc_list, sel=sel_list, tau=tau[:, :npk], out=out)
