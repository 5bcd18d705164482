"""ctypes binding of libmkv.so (include/mkv.h). Argument marshalling only.

Every function has the name of the C entry point it calls. Errors raise
MkvError carrying the C status. The shared library must exist (built by
build.py / __graft_entry__.build()); if it cannot be loaded this module raises
at import time -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmkv.so")

MKV_OK, MKV_ERR_ARG, MKV_ERR_UNSUPPORTED, MKV_ERR_CAPACITY, MKV_ERR_WORKSPACE, MKV_ERR_NOCONVERGE, \
    MKV_ERR_HIP = range(7)
MKV_F32, MKV_BF16 = 0, 1
MKV_SEG_DENSE, MKV_SEG_PACKED, MKV_SEG_BITMAP = 0, 1, 2
MKV_BLOCK_TOKENS = 16
MKV_HEAD_DIM = 128
MKV_MAX_GROUP = 4
MKV_MAX_SEGMENTS = 8
MKV_MAX_PACKED_BLOCKS = 65536
MKV_PACKED_TAIL_BYTES = 256
MKV_N_STAGES = 7
MKV_SCRATCH_BYTES = 128 << 20

EXPORTS = ["mkv_status_str", "mkv_rotation_from_prefill", "mkv_segment_bytes", "mkv_compress_append",
           "mkv_block_meta", "mkv_decode_workspace_bytes", "mkv_decode_sel_cols", "mkv_decode_attn",
           "mkv_append_decode", "mkv_decode_attn_noalloc", "mkv_recompress_segment", "mkv_swap_segment",
           "mkv_strategy_loss_curve", "mkv_strategy_segments",
           "mkv_timing_enable", "mkv_timing_read", "mkv_stage_name"]


class mkv_segment(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("r", ctypes.c_int32), ("keep_ppm", ctypes.c_int32),
                ("k_abs", ctypes.c_int32), ("t_begin", ctypes.c_int64), ("t_cap", ctypes.c_int64),
                ("data", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("rot", ctypes.c_void_p),
                ("key_ch", ctypes.c_int32), ("group", ctypes.c_int32)]


class mkv_cache(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("segs", ctypes.POINTER(mkv_segment)), ("len", ctypes.POINTER(ctypes.c_int64)),
                ("rot", ctypes.c_void_p)]


class MkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, mkv_status_str(status), status))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmkv.so not built at %s (run __graft_entry__.build())" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.mkv_status_str.restype = ctypes.c_char_p
    L.mkv_status_str.argtypes = [ctypes.c_int]
    L.mkv_rotation_from_prefill.restype = ctypes.c_int
    L.mkv_rotation_from_prefill.argtypes = [P, I32, I64, I32, P, P]
    L.mkv_segment_bytes.restype = SZ
    L.mkv_segment_bytes.argtypes = [I32, I32, I32, I32, I32, I64, I32, I32, ctypes.POINTER(SZ)]
    L.mkv_compress_append.restype = ctypes.c_int
    L.mkv_compress_append.argtypes = [ctypes.POINTER(mkv_cache), P, P, P, I32, P]
    L.mkv_block_meta.restype = ctypes.c_int
    L.mkv_block_meta.argtypes = [ctypes.POINTER(mkv_cache), I32, P]
    L.mkv_decode_workspace_bytes.restype = SZ
    L.mkv_decode_workspace_bytes.argtypes = [ctypes.POINTER(mkv_cache)]
    L.mkv_decode_sel_cols.restype = I64
    L.mkv_decode_sel_cols.argtypes = [ctypes.POINTER(mkv_cache)]
    L.mkv_decode_attn.restype = ctypes.c_int
    L.mkv_decode_attn.argtypes = [ctypes.POINTER(mkv_cache), P, P, P, I64, P, SZ, P]
    L.mkv_append_decode.restype = ctypes.c_int
    L.mkv_append_decode.argtypes = [ctypes.POINTER(mkv_cache), P, P, P, I32, P, P, P, I64, P, SZ, P]
    L.mkv_recompress_segment.restype = ctypes.c_int
    L.mkv_recompress_segment.argtypes = [P, P, I32, I32, I32, I64, I64, I32, I32, I32, I32, P, P, P]
    L.mkv_strategy_loss_curve.restype = ctypes.c_int
    L.mkv_strategy_loss_curve.argtypes = [P, P, I32, I32, I32, I64, I64, P, P]
    L.mkv_strategy_segments.restype = ctypes.c_int
    L.mkv_strategy_segments.argtypes = [P, P, I32, I32, I32, I64, I64, P, I32, ctypes.c_double, ctypes.c_double,
                                        I32, I32, I64, I64, I64, P, P, P, P]
    L.mkv_swap_segment.restype = ctypes.c_int
    L.mkv_swap_segment.argtypes = [ctypes.POINTER(mkv_cache), I32, I32, P, P, P, P, P]
    L.mkv_decode_attn_noalloc.restype = ctypes.c_int
    L.mkv_decode_attn_noalloc.argtypes = [ctypes.POINTER(mkv_cache), P, P, P, I64, P]
    L.mkv_timing_enable.restype = ctypes.c_int
    L.mkv_timing_enable.argtypes = [I32]
    L.mkv_timing_read.restype = ctypes.c_int
    L.mkv_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), I32]
    L.mkv_stage_name.restype = ctypes.c_char_p
    L.mkv_stage_name.argtypes = [I32]
    return L


LIB = _load()


def _check(st: int, where: str):
    if st != MKV_OK:
        raise MkvError(st, where)


def mkv_status_str(st: int) -> str:
    return LIB.mkv_status_str(st).decode()


def mkv_rotation_from_prefill(x_ptr: int, dtype: int, T: int, d: int, R_out_ptr: int, sigma_out_ptr):
    _check(LIB.mkv_rotation_from_prefill(x_ptr, dtype, T, d, R_out_ptr, sigma_out_ptr),
           "mkv_rotation_from_prefill")


def mkv_segment_bytes(dtype: int, kind: int, r: int, d: int, n_kv_heads: int, t_cap: int, key_ch: int = 0,
                      group: int = 0):
    meta = ctypes.c_size_t(0)
    data = LIB.mkv_segment_bytes(dtype, kind, r, d, n_kv_heads, t_cap, key_ch, group, ctypes.byref(meta))
    return int(data), int(meta.value)


def mkv_compress_append(cache: mkv_cache, k_ptr: int, v_ptr: int, n_new_ptr: int, n_max: int, stream: int):
    _check(LIB.mkv_compress_append(ctypes.byref(cache), k_ptr, v_ptr, n_new_ptr, n_max, stream),
           "mkv_compress_append")


def mkv_block_meta(cache: mkv_cache, seg: int, stream: int):
    _check(LIB.mkv_block_meta(ctypes.byref(cache), seg, stream), "mkv_block_meta")


def mkv_decode_workspace_bytes(cache: mkv_cache) -> int:
    return int(LIB.mkv_decode_workspace_bytes(ctypes.byref(cache)))


def mkv_decode_sel_cols(cache: mkv_cache) -> int:
    return int(LIB.mkv_decode_sel_cols(ctypes.byref(cache)))


def mkv_decode_attn(cache: mkv_cache, q_ptr: int, out_ptr: int, sel_ptr, sel_cols: int, ws_ptr: int,
                    ws_bytes: int, stream: int):
    _check(LIB.mkv_decode_attn(ctypes.byref(cache), q_ptr, out_ptr, sel_ptr, sel_cols, ws_ptr, ws_bytes,
                               stream), "mkv_decode_attn")


def mkv_append_decode(cache: mkv_cache, k_ptr: int, v_ptr: int, n_new_ptr: int, n_max: int, q_ptr: int,
                      out_ptr: int, sel_ptr, sel_cols: int, ws_ptr: int, ws_bytes: int, stream: int):
    _check(LIB.mkv_append_decode(ctypes.byref(cache), k_ptr, v_ptr, n_new_ptr, n_max, q_ptr, out_ptr, sel_ptr,
                                 sel_cols, ws_ptr, ws_bytes, stream), "mkv_append_decode")


def mkv_recompress_segment(k_ptr: int, v_ptr: int, dtype: int, d: int, n_kv_heads: int, n_tokens: int, t_cap: int,
                           kind: int, r: int, data_ptr: int, meta_ptr: int, rot_ptr: int, key_ch: int = 0,
                           group: int = 0):
    _check(LIB.mkv_recompress_segment(k_ptr, v_ptr, dtype, d, n_kv_heads, n_tokens, t_cap, kind, r, key_ch, group,
                                      data_ptr, meta_ptr, rot_ptr), "mkv_recompress_segment")


def _host_stream(K, V):
    """(k, v, dtype code, d, n_kv_heads, n_tokens, row_stride) of host arrays [H][n][d]
    (float32 values, or uint16 bf16 bit patterns)."""
    import numpy as np
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    if K.shape != V.shape or K.ndim != 3 or K.dtype != V.dtype or K.dtype not in (np.float32, np.uint16):
        raise ValueError("K and V: equal shapes [H][n][d], float32 or uint16 (bf16 bits)")
    code = MKV_F32 if K.dtype == np.float32 else MKV_BF16
    H, n, d = K.shape
    return K, V, code, d, H, n, n


def mkv_strategy_loss_curve(K, V, rot):
    """Loss for r = 0 .. d of every token under rot [H][2][d][d] (float32)."""
    import numpy as np
    K, V, code, d, H, n, stride = _host_stream(K, V)
    rot = np.ascontiguousarray(rot, dtype=np.float32)
    out = np.empty(d + 1, np.float64)
    _check(LIB.mkv_strategy_loss_curve(K.ctypes.data, V.ctypes.data, code, d, H, n, stride, rot.ctypes.data,
                                       out.ctypes.data), "mkv_strategy_loss_curve")
    return out


def mkv_strategy_segments(K, V, rot0, r0: int, cut_loss: float, keep_loss: float, r_min: int, r_max: int,
                          min_len: int, max_len: int, seg_cap: int = 1024):
    """[(end, r, rot [H][2][d][d] float32)] of one request's token stream."""
    import numpy as np
    K, V, code, d, H, n, stride = _host_stream(K, V)
    rot0 = np.ascontiguousarray(rot0, dtype=np.float32)
    ends = np.zeros(seg_cap, np.int64)
    rs = np.zeros(seg_cap, np.int32)
    rots = np.zeros((seg_cap, H, 2, d, d), np.float32)
    ns = ctypes.c_int64(0)
    _check(LIB.mkv_strategy_segments(K.ctypes.data, V.ctypes.data, code, d, H, n, stride, rot0.ctypes.data, r0,
                                     float(cut_loss), float(keep_loss), r_min, r_max, min_len, max_len, seg_cap,
                                     ends.ctypes.data, rs.ctypes.data, rots.ctypes.data, ctypes.byref(ns)),
           "mkv_strategy_segments")
    return [(int(ends[i]), int(rs[i]), rots[i]) for i in range(ns.value)]


def mkv_swap_segment(cache: mkv_cache, b: int, seg: int, data_ptr: int, meta_ptr: int, rot_ptr: int, event,
                     stream: int):
    _check(LIB.mkv_swap_segment(ctypes.byref(cache), b, seg, data_ptr, meta_ptr, rot_ptr, event, stream),
           "mkv_swap_segment")


def mkv_decode_attn_noalloc(cache: mkv_cache, q_ptr: int, out_ptr: int, sel_ptr, sel_cols: int, stream: int):
    _check(LIB.mkv_decode_attn_noalloc(ctypes.byref(cache), q_ptr, out_ptr, sel_ptr, sel_cols, stream),
           "mkv_decode_attn_noalloc")


def mkv_timing_enable(on: bool):
    _check(LIB.mkv_timing_enable(1 if on else 0), "mkv_timing_enable")


def mkv_timing_read():
    ms = (ctypes.c_double * MKV_N_STAGES)()
    cnt = (ctypes.c_int64 * MKV_N_STAGES)()
    _check(LIB.mkv_timing_read(ms, cnt, MKV_N_STAGES), "mkv_timing_read")
    return {LIB.mkv_stage_name(i).decode(): (ms[i], int(cnt[i])) for i in range(MKV_N_STAGES)}


def mkv_stage_name(i: int) -> str:
    return LIB.mkv_stage_name(i).decode()
