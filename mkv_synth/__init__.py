"""Seeded synthetic inputs and workload layouts for the MosaicKV decode path.

This module is shared by the oracle-side tests and by the GPU-side tests, the
benchmark and the smoke run. It produces *inputs only*: raw K/V vectors in the
storage dtype, queries, and the per-request segment tables of each workload. It
contains none of the method's arithmetic (no rotation, selection, packing,
scoring or attention).

Key/value recipe (one independent stream per request b, KV head g and K|V):
  Z ~ N(0,1)^{T x 128} in float64, D = diag(exp(-i/24)), Q Haar-orthogonal
  (QR of a Gaussian matrix, columns multiplied by sign(diag R)),
  X = Z D Q^T plus, per token, 4 distinct random channels set off by +/-6
  (sign +/- with probability 1/2), then rounded to the storage dtype.
  This stands in for the LLaMA-3.1-8B-class key/value caches that the pages
  measure on (their evaluation setup, MosaicKV paper section 6.1); no dataset
  or model weights are used.
Queries: q ~ N(0, I_128) per (request, query head, iteration); for bf16
  workloads they are rounded through bf16 and handed over as float32.

Random streams are counter-addressed (SplitMix64, see gen.c): token t of the
stream (cfg, b, g, kind) uses its own 256 counters, so any token range can be
generated on its own and prefixes agree. The mixing matrix Q comes from numpy
PCG64(SeedSequence([cfg, b, g, kind, 0])).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HEAD_DIM = 128
BLOCK_TOKENS = 16
N_SPIKES = 4
SPIKE = 6.0

DENSE = 0
PACKED = 1   # packed records with u8 channel indices
BITMAP = 2   # packed records with per-vector position bitmaps


def is_packed(kind) -> bool:
    return kind in (PACKED, BITMAP)


def as_bitmap(segs):
    """The same segment table with every packed segment holding bitmap records."""
    return [[dict(s, kind=BITMAP) if s["kind"] == PACKED else dict(s) for s in row] for row in segs]


# ----------------------------------------------------------------------------
# storage-dtype helpers used to *produce inputs* (not the method's rounding)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns (nearest-even on the f32 bits)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str):
    """Input preparation: float64 -> storage dtype.

    Returns (values_f32, bits) where values_f32 holds the exact stored values as
    float32 and bits is the uint16 pattern for bf16 (None for f32).
    """
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32, None
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return bf16_bits_to_f32(bits), bits
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# key / value generator (bulk work in gen.c, OpenMP over tokens)
# ----------------------------------------------------------------------------
_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmkvsynth.so")


def build(force: bool = True) -> str:
    """Compile gen.c into libmkvsynth.so next to this file."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _LIB
    if _LIB is None:
        build(force=False)
        lib = ctypes.CDLL(_SO)
        lib.mkv_gen_seed.restype = ctypes.c_uint64
        lib.mkv_gen_seed.argtypes = [ctypes.c_int64] * 4
        lib.mkv_gen_kv.restype = ctypes.c_int
        lib.mkv_gen_kv.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        _LIB = lib
    return _LIB


def host_threads() -> int:
    """Host threads to use: every CPU this process may run on, bounded by the
    OMP_NUM_THREADS the environment grants (a GPU job's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "").strip()
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _haar(cfg: int, b: int, g: int, kind: int, d: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, b, g, kind, 0])))
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def _mix(cfg: int, b: int, g: int, kind: int, d: int) -> np.ndarray:
    """M = diag(exp(-i/24)) Q^T, so that a token row is x = z M."""
    dscale = np.exp(-np.arange(d) / 24.0)
    return np.ascontiguousarray(dscale[:, None] * _haar(cfg, b, g, kind, d).T)


_DT = {"f32": (0, np.float32), "bf16": (1, np.uint16), "f64": (2, np.float64)}


def gen_kv_into(cfg, b, g, kind, t0, t1, dtype, out, d=HEAD_DIM):
    """Write rows [t0, t1) of stream (cfg, b, g, kind) into out ([t1-t0][d]).

    dtype 'f32' -> float32 values, 'bf16' -> uint16 bit patterns, 'f64' -> unrounded.
    """
    code, npdt = _DT[dtype]
    assert out.dtype == npdt and out.flags.c_contiguous and out.shape == (t1 - t0, d)
    if t1 <= t0:
        return out
    lib = _lib()
    mix = _mix(cfg, b, g, kind, d)
    seed = lib.mkv_gen_seed(cfg, b, g, kind)
    rc = lib.mkv_gen_kv(seed, mix.ctypes.data, d, t0, t1, code, out.ctypes.data, host_threads())
    if rc != 0:
        raise RuntimeError("mkv_gen_kv failed")
    return out


def gen_kv64(cfg: int, b: int, g: int, kind: int, t0: int, t1: int, d: int = HEAD_DIM) -> np.ndarray:
    """Unrounded float64 K (kind=0) or V (kind=1) rows for token positions [t0, t1)."""
    return gen_kv_into(cfg, b, g, kind, t0, t1, "f64", np.empty((max(t1 - t0, 0), d), np.float64), d)


def gen_kv(cfg: int, b: int, g: int, kind: int, t0: int, t1: int, dtype: str, d: int = HEAD_DIM):
    """Raw stored K/V rows for [t0, t1): (values as float32, bf16 bits or None)."""
    n = max(t1 - t0, 0)
    if dtype == "f32":
        v = gen_kv_into(cfg, b, g, kind, t0, t1, "f32", np.empty((n, d), np.float32), d)
        return v, None
    bits = gen_kv_into(cfg, b, g, kind, t0, t1, "bf16", np.empty((n, d), np.uint16), d)
    return bf16_bits_to_f32(bits), bits


def gen_q(cfg: int, it: int, batch: int, n_q_heads: int, dtype: str, d: int = HEAD_DIM) -> np.ndarray:
    """Queries [batch][n_q_heads][d] float32 (bf16-representable for bf16 workloads)."""
    q = np.empty((batch, n_q_heads, d), dtype=np.float64)
    for b in range(batch):
        for h in range(n_q_heads):
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, 1000 + it, b, h])))
            q[b, h] = rng.standard_normal(d)
    vals, _ = to_storage(q, dtype)
    return vals


# ----------------------------------------------------------------------------
# workload layouts
# ----------------------------------------------------------------------------
def seg(kind, t_begin, t_cap, r=0, keep_ppm=0, k_abs=0, key_ch=0):
    """key_ch: leading rotated channels covered by a packed segment's block keys (0: all)."""
    return dict(kind=kind, t_begin=int(t_begin), t_cap=int(t_cap), r=int(r),
                keep_ppm=int(keep_ppm), k_abs=int(k_abs), key_ch=int(key_ch))


def with_groups(segs, group: int):
    """The same segment table with every packed segment keeping whole groups of `group` channels."""
    return [[dict(s, group=int(group)) if is_packed(s["kind"]) else dict(s) for s in row] for row in segs]


def with_key_channels(segs, key_ch: int):
    """The same segment table with every packed segment's block keys over key_ch channels."""
    return [[dict(s, key_ch=int(key_ch)) if is_packed(s["kind"]) else dict(s) for s in row] for row in segs]


def _stack(parts):
    """parts: list of (kind, length, r, keep_ppm, k_abs) -> contiguous segment list."""
    out, t = [], 0
    for kind, n, r, keep, kabs in parts:
        out.append(seg(kind, t, n, r, keep, kabs))
        t += n
    return out


def serving_lengths(batch: int = 32, lo: int = 16384, hi: int = 98304) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5, 999])))
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def workload(cfg: int, scale: int = 1, extra_cap: int = 0, batch: int | None = None):
    """Describe one of the five workloads, by id (the id also seeds its streams):
    1 single head, T = 4096, fp32; 2 GQA 32/8 layer, T = 32768, bf16;
    3 the same layer at T = 131072, batch 4, two packed segments; 4 the same
    layer at T = 1048576 (one layer's share at million-token context);
    5 serving, batch 32, T uniform in [16384, 98304].

    scale divides every token count (1 = full size); extra_cap adds capacity to
    the last segment (decode-step growth). Returns a dict with keys:
    cfg, batch, n_q_heads, n_kv_heads, d, dtype, lengths [B], segs [B][n_seg].
    """
    d = HEAD_DIM
    if cfg == 1:
        B, hq, hk, dt = 1, 1, 1, "f32"
        T = 4096 // scale
        sink, recent = max(16 // scale, 1), max(64 // scale, 1)
        layouts = [_stack([(DENSE, sink, 0, 0, 0),
                           (PACKED, T - sink - recent, 32, 0, max(64 // scale, 1)),
                           (DENSE, recent + extra_cap, 0, 0, 0)])]
        lengths = [T]
    elif cfg == 2:
        B, hq, hk, dt = 1, 32, 8, "bf16"
        T = 32768 // scale
        sink, recent = max(64 // scale, 1), max(1024 // scale, 1)
        layouts = [_stack([(DENSE, sink, 0, 0, 0),
                           (PACKED, T - sink - recent, 38, 100000, 0),
                           (DENSE, recent + extra_cap, 0, 0, 0)])]
        lengths = [T]
    elif cfg == 3:
        B, hq, hk, dt = 4, 32, 8, "bf16"
        T = 131072 // scale
        sink, recent = max(64 // scale, 1), max(4096 // scale, 1)
        mid = T - sink - recent
        half = (mid // 2) // BLOCK_TOKENS * BLOCK_TOKENS
        layouts = [_stack([(DENSE, sink, 0, 0, 0),
                           (PACKED, half, 26, 50000, 0),
                           (PACKED, mid - half, 38, 100000, 0),
                           (DENSE, recent + extra_cap, 0, 0, 0)])] * B
        lengths = [T] * B
    elif cfg == 4:
        B, hq, hk, dt = 1, 32, 8, "bf16"
        T = 1048576 // scale
        sink, recent = max(64 // scale, 1), max(8192 // scale, 1)
        layouts = [_stack([(DENSE, sink, 0, 0, 0),
                           (PACKED, T - sink - recent, 32, 40000, 0),
                           (DENSE, recent + extra_cap, 0, 0, 0)])]
        lengths = [T]
    elif cfg == 5:
        B = 32 if batch is None else batch
        hq, hk, dt = 32, 8, "bf16"
        Ts = serving_lengths(32)[:B] // scale
        sink = max(64 // scale, 1)
        layouts = [_stack([(DENSE, sink, 0, 0, 0),
                           (PACKED, int(t) - sink + 256 + extra_cap, 38, 100000, 0)]) for t in Ts]
        lengths = [int(t) for t in Ts]
    else:
        raise ValueError(cfg)
    if batch is not None and cfg != 5:
        layouts = (layouts * batch)[:batch] if len(layouts) < batch else layouts[:batch]
        lengths = (lengths * batch)[:batch] if len(lengths) < batch else lengths[:batch]
        B = batch
    return dict(cfg=cfg, batch=B, n_q_heads=hq, n_kv_heads=hk, d=d, dtype=dt,
                lengths=np.asarray(lengths, dtype=np.int64), segs=[list(l) for l in layouts])


def with_update_segment(w: dict, cap: int, r: int = 38, keep_ppm: int = 100000) -> dict:
    """Append a packed update segment after each request's last segment.

    New decode-step tokens land there: they are rotated, top-r'd and packed on
    arrival, the GPU-side fast path of the pages' double buffering (MosaicKV
    paper section 5.4; the reading notes' Fig. 4).
    """
    segs = []
    for s in w["segs"]:
        last = s[-1]
        segs.append(list(s) + [seg(PACKED, last["t_begin"] + last["t_cap"], cap, r, keep_ppm, 0)])
    out = dict(w)
    out["segs"] = segs
    return out
