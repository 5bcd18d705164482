"""A compressed cache whose device buffers are torch tensors.

Plumbing only: torch provides device memory and the current HIP stream, the
library (libmkv.so) does all the work. Buffers are zero-initialised.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib as L

DTYPES = {"f32": (L.MKV_F32, torch.float32, 4), "bf16": (L.MKV_BF16, torch.bfloat16, 2)}


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class Cache:
    """segs: list (per request) of lists of dicts with kind, t_begin, t_cap, r,
    keep_ppm, k_abs (see include/mkv.h)."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, dtype: str, segs, device="cuda",
                 head_dim: int = L.MKV_HEAD_DIM):
        self.batch, self.hq, self.hkv, self.d = batch, n_q_heads, n_kv_heads, head_dim
        self.dtype = dtype
        self.code, self.tdtype, self.sbytes = DTYPES[dtype]
        self.device = device
        self.nseg = len(segs[0])
        self.seg_list = [list(s) for s in segs]
        self._segs = (L.mkv_segment * (batch * self.nseg))()
        self._len = (ctypes.c_int64 * batch)()
        self.data, self.meta = [], []
        for b in range(batch):
            drow, mrow = [], []
            for j, s in enumerate(segs[b]):
                nbytes, mbytes = L.mkv_segment_bytes(self.code, s["kind"], s["r"] or 1, head_dim,
                                                      n_kv_heads, s["t_cap"], s.get("key_ch", 0), s.get("group", 0))
                if nbytes == 0:
                    raise ValueError("invalid segment %r" % (s,))
                dt = torch.zeros(nbytes, dtype=torch.uint8, device=device)
                mt = torch.zeros(mbytes, dtype=torch.uint8, device=device) if mbytes else None
                drow.append(dt)
                mrow.append(mt)
                e = self._segs[b * self.nseg + j]
                e.kind, e.r, e.keep_ppm, e.k_abs = s["kind"], s["r"], s["keep_ppm"], s["k_abs"]
                e.t_begin, e.t_cap = s["t_begin"], s["t_cap"]
                e.key_ch = s.get("key_ch", 0)
                e.group = s.get("group", 0)
                e.data = dt.data_ptr()
                e.meta = mt.data_ptr() if mt is not None else None
            self.data.append(drow)
            self.meta.append(mrow)
        self.seg_rot = [[None] * self.nseg for _ in range(batch)]  # segments' own rotations (device tensors)
        self.rot = torch.zeros((batch, n_kv_heads, 2, head_dim, head_dim), dtype=torch.float32, device=device)
        self.c = L.mkv_cache(batch, n_q_heads, n_kv_heads, head_dim, self.code, self.nseg,
                             ctypes.cast(self._segs, ctypes.POINTER(L.mkv_segment)),
                             ctypes.cast(self._len, ctypes.POINTER(ctypes.c_int64)), self.rot.data_ptr())
        self._ws = None

    # ------------------------------------------------------------------
    @property
    def lengths(self):
        return [int(self._len[b]) for b in range(self.batch)]

    def set_rotation(self, R):
        """R: [batch][n_kv][2][d][d] float32 (numpy or torch)."""
        self.rot.copy_(torch.as_tensor(np.asarray(R, np.float32)).to(self.device))

    def set_segment_rotation(self, b: int, j: int, R):
        """Give segment j of request b its own rotation before any token reaches it:
        R [n_kv][2][d][d] float32 (numpy or torch)."""
        t = torch.as_tensor(np.asarray(R, np.float32)).to(self.device).contiguous()
        self.seg_rot[b][j] = t
        self._segs[b * self.nseg + j].rot = t.data_ptr()

    def recompress_segment(self, b: int, j: int, k_host, v_host):
        """Host recompression of segment j of request b (mkv_recompress_segment) from
        its raw keys and values, numpy [n_kv][n_tokens][d] (float32, or bf16 bits as
        uint16). Returns host (data, meta, rot) in the device layouts."""
        s = self.seg_list[b][j]
        nbytes, mbytes = L.mkv_segment_bytes(self.code, s["kind"], s["r"], self.d, self.hkv, s["t_cap"],
                                             s.get("key_ch", 0), s.get("group", 0))
        data = np.zeros(nbytes, np.uint8)
        meta = np.zeros(mbytes, np.uint8)
        rot = np.zeros((self.hkv, 2, self.d, self.d), np.float32)
        k = np.ascontiguousarray(k_host)
        v = np.ascontiguousarray(v_host)
        L.mkv_recompress_segment(k.ctypes.data, v.ctypes.data, self.code, self.d, self.hkv, int(k.shape[1]),
                                 s["t_cap"], s["kind"], s["r"], data.ctypes.data, meta.ctypes.data, rot.ctypes.data,
                                 s.get("key_ch", 0), s.get("group", 0))
        return data, meta, rot

    def swap_segment(self, b: int, j: int, data, meta, rot, copy_stream=None):
        """Copy host (data, meta, rot) to new device buffers on copy_stream (a side
        stream by default) and swap them in for segment j of request b
        (mkv_swap_segment): the current stream waits for the copies, the host does
        not. Returns the previous device buffers, which must outlive the work
        enqueued before the swap."""
        copy_stream = copy_stream or torch.cuda.Stream()
        ev = torch.cuda.Event()
        with torch.cuda.stream(copy_stream):
            dt = torch.from_numpy(np.asarray(data, np.uint8)).pin_memory().to(self.device, non_blocking=True)
            mt = torch.from_numpy(np.asarray(meta, np.uint8)).pin_memory().to(self.device, non_blocking=True)
            rt = torch.from_numpy(np.asarray(rot, np.float32)).pin_memory().to(self.device, non_blocking=True)
            ev.record(copy_stream)
        old = (self.data[b][j], self.meta[b][j], self.seg_rot[b][j])
        L.mkv_swap_segment(self.c, b, j, dt.data_ptr(), mt.data_ptr(), rt.data_ptr(), ev.cuda_event, _stream())
        self.data[b][j], self.meta[b][j], self.seg_rot[b][j] = dt, mt, rt
        self._keep = (ev, copy_stream)
        return old

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, n_new):
        """k_new, v_new: device tensors [batch][n_kv][n_max][d] of the storage dtype
        (or same-size integer views of the bit patterns)."""
        assert k_new.is_contiguous() and v_new.is_contiguous()
        assert k_new.element_size() == self.sbytes and k_new.shape[:2] == (self.batch, self.hkv)
        n_max = int(k_new.shape[2])
        nn = (ctypes.c_int32 * self.batch)(*[int(x) for x in n_new])
        L.mkv_compress_append(self.c, k_new.data_ptr(), v_new.data_ptr(), ctypes.addressof(nn), n_max, _stream())

    def block_meta(self, seg: int):
        L.mkv_block_meta(self.c, seg, _stream())

    def workspace_bytes(self) -> int:
        return L.mkv_decode_workspace_bytes(self.c)

    def sel_cols(self) -> int:
        return L.mkv_decode_sel_cols(self.c)

    def workspace(self):
        need = self.workspace_bytes()
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def decode(self, q: torch.Tensor, out: torch.Tensor | None = None, want_sel: bool = False,
               sel_cols: int | None = None):
        """q: device float32 [batch][n_q][d]. Returns out (and sel_out if asked)."""
        assert q.dtype == torch.float32 and q.is_contiguous()
        if out is None:
            out = torch.empty((self.batch, self.hq, self.d), dtype=torch.float32, device=self.device)
        sel = None
        cols = 0
        if want_sel:
            cols = self.sel_cols() if sel_cols is None else sel_cols
            sel = torch.empty((self.batch, self.hq, max(cols, 1)), dtype=torch.int32, device=self.device)
        ws = self.workspace()
        L.mkv_decode_attn(self.c, q.data_ptr(), out.data_ptr(), sel.data_ptr() if sel is not None else None,
                          cols, ws.data_ptr(), ws.numel(), _stream())
        return (out, sel) if want_sel else out

    def append_decode(self, k_new: torch.Tensor, v_new: torch.Tensor, n_new, q: torch.Tensor,
                      out: torch.Tensor | None = None, want_sel: bool = False, sel_cols: int | None = None):
        """append(k_new, v_new, n_new) then decode(q) in one library call (same results)."""
        assert k_new.is_contiguous() and v_new.is_contiguous()
        assert k_new.element_size() == self.sbytes and k_new.shape[:2] == (self.batch, self.hkv)
        assert q.dtype == torch.float32 and q.is_contiguous()
        n_max = int(k_new.shape[2])
        nn = (ctypes.c_int32 * self.batch)(*[int(x) for x in n_new])
        if out is None:
            out = torch.empty((self.batch, self.hq, self.d), dtype=torch.float32, device=self.device)
        sel = None
        cols = 0
        if want_sel:
            if sel_cols is None:  # columns needed at the lengths after the append
                self._len_add(n_new)
                cols = self.sel_cols()
                self._len_add([-int(x) for x in n_new])
            else:
                cols = sel_cols
            sel = torch.empty((self.batch, self.hq, max(cols, 1)), dtype=torch.int32, device=self.device)
        ws = self.workspace()
        L.mkv_append_decode(self.c, k_new.data_ptr(), v_new.data_ptr(), ctypes.addressof(nn), n_max, q.data_ptr(),
                            out.data_ptr(), sel.data_ptr() if sel is not None else None, cols, ws.data_ptr(),
                            ws.numel(), _stream())
        return (out, sel) if want_sel else out

    def _len_add(self, n):
        for b in range(self.batch):
            self._len[b] += int(n[b])
