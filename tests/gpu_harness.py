"""Shared helpers of the GPU parity tests: build a cache from the seeded
workloads through the C ABI, run the oracle on chosen (request, KV head)
units, and compare the two sides."""
from __future__ import annotations

import ctypes
import sys
import time

import numpy as np

import mkv_synth as synth
from oracle import oracle as orc

DT_CODE = {"f32": 0, "bf16": 1}


def log(msg):
    print("[%s] %s" % (time.strftime("%H:%M:%S"), msg), flush=True)
    sys.stdout.flush()


def raw_to_f64(bits_or_vals, dtype):
    if dtype == "bf16":
        return synth.bf16_bits_to_f32(bits_or_vals).astype(np.float64)
    return np.asarray(bits_or_vals, np.float32).astype(np.float64)


def gen_raw(w, t_ends, t_begins=None):
    """Raw stored K/V for every (b, g): arrays [B][Hkv][Tmax][d] of uint16 bits (bf16)
    or float32 (f32), rows [t_begin_b, t_end_b) of each request's stream."""
    B, hkv, d, dt = w["batch"], w["n_kv_heads"], w["d"], w["dtype"]
    t_begins = t_begins if t_begins is not None else [0] * B
    n = [int(e) - int(s) for s, e in zip(t_begins, t_ends)]
    nmax = max(max(n), 1)
    npdt = np.uint16 if dt == "bf16" else np.float32
    K = np.zeros((B, hkv, nmax, d), npdt)
    V = np.zeros((B, hkv, nmax, d), npdt)
    for b in range(B):
        for g in range(hkv):
            for kind, arr in ((0, K), (1, V)):
                out = np.empty((n[b], d), npdt)
                synth.gen_kv_into(w["cfg"], b, g, kind, int(t_begins[b]), int(t_ends[b]), dt, out, d)
                arr[b, g, :n[b]] = out
    return K, V, n


def rotations(L, w, K, V, n):
    """Library rotations from each unit's prefill rows: [B][Hkv][2][d][d] float32."""
    B, hkv, d = w["batch"], w["n_kv_heads"], w["d"]
    R = np.zeros((B, hkv, 2, d, d), np.float32)
    code = DT_CODE[w["dtype"]]
    for b in range(B):
        for g in range(hkv):
            for kind, arr in ((0, K), (1, V)):
                x = np.ascontiguousarray(arr[b, g, :n[b]])
                out = np.empty((d, d), np.float32)
                L.mkv_rotation_from_prefill(x.ctypes.data, code, n[b], d, out.ctypes.data, None)
                R[b, g, kind] = out
    return R


def to_device(torch, arr, device="cuda"):
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device)
    return torch.from_numpy(arr).to(device)


def build(torch, w, lengths=None, R=None, raw=None):
    """Cache filled with every request's first `lengths[b]` tokens in one append."""
    from kv_cache_compression_mkv_amd import _lib as L
    from kv_cache_compression_mkv_amd.cache import Cache
    lengths = list(w["lengths"] if lengths is None else lengths)
    if raw is None:
        raw = gen_raw(w, lengths)
    K, V, _ = raw
    n = lengths
    if R is None:
        R = rotations(L, w, K, V, n)
    c = Cache(w["batch"], w["n_q_heads"], w["n_kv_heads"], w["dtype"], w["segs"])
    c.set_rotation(R)
    c.append(to_device(torch, K), to_device(torch, V), n)
    torch.cuda.synchronize()
    return c, (K, V, n), R


def oracle_unit(w, raw, R, b, g, length, segs=None):
    K, V, _ = raw
    dt = w["dtype"]
    segs = w["segs"][b] if segs is None else segs
    Kr = raw_to_f64(K[b, g, :length], dt)
    Vr = raw_to_f64(V[b, g, :length], dt)
    Rk = R[b, g, 0].astype(np.float64)
    Rv = R[b, g, 1].astype(np.float64)
    return orc.compress_unit(Kr, Vr, Rk, Rv, segs, length, dt), Rk, Rv


def bits_of(values_f64, dtype):
    f = np.asarray(values_f64, np.float64).astype(np.float32)
    if dtype == "bf16":
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    return f.view(np.uint32)


def _head_bytes(t, g, per_head):
    return t[g * per_head:(g + 1) * per_head].cpu().numpy()


def _first_bad(ok_rows, t0):
    bad = np.nonzero(~ok_rows)[0]
    return int(bad[0]) + t0 if bad.size else None


def compare_compress(cache, w, comp, b, g, length):
    """Bit-exact comparison of one unit's stored cache with the oracle's: dense
    rows, packed indices and values, zero padding of the tail block, block keys."""
    from kv_cache_compression_mkv_amd import layout
    dt = w["dtype"]
    sb = 2 if dt == "bf16" else 4
    d = w.get("d", 128)
    pj = 0
    for j, s in enumerate(w["segs"][b]):
        nbcap = -(-s["t_cap"] // 16)
        filled = min(max(length - s["t_begin"], 0), s["t_cap"])
        nb = -(-filled // 16)
        tb = s["t_begin"]
        if s["kind"] == synth.DENSE:
            data = _head_bytes(cache.data[b][j], g, nbcap * 2 * 16 * d * sb)
            _, bits = layout.unpack_dense(data, 1, nbcap, dt, d)
            for kind, hat in ((0, comp["Khat"]), (1, comp["Vhat"])):
                got = bits[0, :, kind].reshape(nbcap * 16, d)[:filled]
                exp = bits_of(hat[tb:tb + filled], dt)
                bad = _first_bad(np.all(got == exp, axis=1), tb)
                assert bad is None, "dense b=%d g=%d seg=%d t=%d kind=%d" % (b, g, j, bad, kind)
            if filled % 16:
                assert np.all(bits[0, nb - 1, :, filled % 16:] == 0)
            continue
        r = s["r"]
        gs = s.get("group", 0)
        rec = layout.record_bytes(s["kind"], r, dt, d, gs)
        P = layout.unpack_records(_head_bytes(cache.data[b][j], g, nbcap * rec), 1, nbcap, r, dt, s["kind"], d, gs)
        for hat, idx, gbits, gidx, name in ((comp["Khat"], comp["Kidx"], P["kbits"], P["kidx"], "K"),
                                            (comp["Vhat"], comp["Vidx"], P["vbits"], P["vidx"], "V")):
            ei = idx[tb:tb + filled, :r].astype(np.int64)
            if s["kind"] == synth.BITMAP:
                # the bitmap holds exactly the kept channels, and nothing past the last token
                ebm = np.zeros((nbcap * 16, d), bool)
                np.put_along_axis(ebm[:filled], ei, True, axis=1)
                gbm = P[name.lower() + "bm"][0].reshape(nbcap * 16, d)
                bad = _first_bad(np.all(gbm[:filled] == ebm[:filled], axis=1), tb)
                assert bad is None, "%s bitmap b=%d g=%d seg=%d t=%d" % (name, b, g, j, bad)
                assert not gbm[filled:nb * 16].any(), "%s bitmap padding b=%d g=%d seg=%d" % (name, b, g, j)
            gi = gidx[0].reshape(nbcap * 16, r)[:filled].astype(np.int64)
            bad = _first_bad(np.all(gi == ei, axis=1), tb)
            assert bad is None, "%s idx b=%d g=%d seg=%d t=%d: %s vs %s" % (
                name, b, g, j, bad, gi[bad - tb], ei[bad - tb])
            ev = bits_of(np.take_along_axis(hat[tb:tb + filled], ei, axis=1), dt)
            gv = gbits[0].reshape(nbcap * 16, r)[:filled]
            bad = _first_bad(np.all(gv == ev, axis=1), tb)
            assert bad is None, "%s val b=%d g=%d seg=%d t=%d" % (name, b, g, j, bad)
        if filled % 16:
            assert np.all(P["kbits"][0, nb - 1, filled % 16:] == 0)
            assert np.all(P["vbits"][0, nb - 1, filled % 16:] == 0)
            assert np.all(P["kidx"][0, nb - 1, filled % 16:] == 0)
            assert np.all(P["vidx"][0, nb - 1, filled % 16:] == 0)
        kch = s.get("key_ch", 0) or d
        ng = layout.meta_groups(dt, d, kch)
        ntile = -(-nbcap // 64)
        mraw = _head_bytes(cache.meta[b][j], g, ntile * ng * 64 * 16)
        _, mbits = layout.unpack_meta(mraw, 1, nbcap, dt, d, kch)
        om = comp["meta"][pj][:, :, :kch]
        assert om.shape[0] == nb
        if nb:
            ok = np.all(mbits[0, :nb] == bits_of(om, dt), axis=(1, 2))
            bad = _first_bad(ok, 0)
            assert bad is None, "meta b=%d g=%d seg=%d block=%d" % (b, g, j, bad)
        pj += 1


def split_sel(sel_row, seg_k):
    """sel_out row [Hq-slice][cols] -> list over packed segments of [G][k]."""
    out, o = [], 0
    for k in seg_k:
        out.append(sel_row[:, o:o + k])
        o += k
    return out


def check_decode_unit(w, comp, Rk, Rv, q_unit, out_gpu, sel_gpu_unit, tol, length, b, g):
    """Compare one unit's decode: selection (with the near-tie exemption) and
    outputs against the oracle forced to the GPU's selection."""
    segs = w["segs"][b]
    nk = orc.seg_blocks(segs, length)
    seg_k = [k for _, k in nk]
    gsel = split_sel(sel_gpu_unit, seg_k)
    own = orc.decode_unit(comp, q_unit, Rk, Rv)
    forced = orc.decode_unit(comp, q_unit, Rk, Rv, forced_sel=gsel)
    G = q_unit.shape[0]
    n_exempt = 0
    for pj, (gs, os_, sc) in enumerate(zip(gsel, own["sel"], own["scores"])):
        for h in range(G):
            a, e = set(gs[h].tolist()), set(os_[h].tolist())
            assert len(a) == len(gs[h]) and all(0 <= x < sc.shape[1] for x in a), "invalid GPU selection"
            assert list(gs[h]) == sorted(gs[h]), "GPU selection not ascending"
            if a != e:
                tau = own["tau"][h, pj]
                smax = np.abs(sc[h]).max()
                for blk in a ^ e:
                    s = sc[h, blk]
                    lim = 1e-4 * max(abs(s), abs(tau), 1e-6 * smax)
                    assert abs(s - tau) <= lim, \
                        "b=%d g=%d h=%d seg=%d block %d score %.9g vs threshold %.9g" % (b, g, h, pj, blk, s, tau)
                    n_exempt += 1
    for h in range(G):
        ref = forced["out"][h]
        nr = np.linalg.norm(ref)
        err = np.linalg.norm(out_gpu[h] - ref)
        if nr == 0:
            assert err == 0, "b=%d g=%d h=%d expected zeros" % (b, g, h)
        else:
            assert err / nr <= tol, "b=%d g=%d h=%d rel L2 %.3g > %.3g" % (b, g, h, err / nr, tol)
    return n_exempt


def _pidx(segs, j):
    """Index of segment j among the packed segments."""
    return sum(1 for s in segs[:j] if synth.is_packed(s["kind"]))


def compare_packed_blocks(cache, w, comp, b, g, j, blocks, length):
    """Bit-exact comparison of the given blocks of packed segment j of unit (b, g)
    with the oracle: indices and values of every valid slot, zeros in the slots
    after the last token, and the blocks' keys."""
    from kv_cache_compression_mkv_amd import layout
    dt, d = w["dtype"], w.get("d", 128)
    sb = 2 if dt == "bf16" else 4
    s = w["segs"][b][j]
    r, tb = s["r"], s["t_begin"]
    nbcap = -(-s["t_cap"] // 16)
    rec = layout.record_bytes(s["kind"], r, dt, d, s.get("group", 0))
    filled = min(max(length - tb, 0), s["t_cap"])
    data = cache.data[b][j]
    for l in blocks:
        off = (g * nbcap + l) * rec
        P = layout.unpack_records(data[off:off + rec].cpu().numpy(), 1, 1, r, dt, s["kind"], d, s.get("group", 0))
        nv = min(16, filled - 16 * l)
        for hat, idx, gb, gi, name in ((comp["Khat"], comp["Kidx"], P["kbits"], P["kidx"], "K"),
                                       (comp["Vhat"], comp["Vidx"], P["vbits"], P["vidx"], "V")):
            ei = idx[tb + 16 * l:tb + 16 * l + nv, :r].astype(np.int64)
            assert np.array_equal(gi[0, 0, :nv].astype(np.int64), ei), "%s idx b=%d g=%d seg=%d block=%d" % (
                name, b, g, j, l)
            ev = bits_of(np.take_along_axis(hat[tb + 16 * l:tb + 16 * l + nv], ei, axis=1), dt)
            assert np.array_equal(gb[0, 0, :nv], ev), "%s val b=%d g=%d seg=%d block=%d" % (name, b, g, j, l)
            assert np.all(gb[0, 0, nv:] == 0) and np.all(gi[0, 0, nv:] == 0), "padding b=%d block=%d" % (b, l)
    kch = s.get("key_ch", 0) or d
    ng = layout.meta_groups(dt, d, kch)
    ntile = -(-nbcap // 64)
    mraw = _head_bytes(cache.meta[b][j], g, ntile * ng * 64 * 16)
    _, mbits = layout.unpack_meta(mraw, 1, nbcap, dt, d, kch)
    om = comp["meta"][_pidx(w["segs"][b], j)][:, :, :kch]
    for l in blocks:
        assert np.array_equal(mbits[0, l], bits_of(om[l], dt)), "keys b=%d g=%d seg=%d block=%d" % (b, g, j, l)


class Snapshot:
    """Device copy of a cache's segment buffers, to find which blocks a step changed."""

    def __init__(self, cache):
        self.data = [[t.clone() for t in row] for row in cache.data]
        self.meta = [[t.clone() if t is not None else None for t in row] for row in cache.meta]

    @staticmethod
    def _diff(cur, prev):
        return torch_nonzero_offsets(cur, prev)

    def changed(self, cache, w, b, j):
        """Sorted (KV head, block) pairs whose stored bytes (data or keys) differ
        from the snapshot in segment j of request b; (-1, -1) marks bytes past
        the last block."""
        dt, d, hkv = w["dtype"], w.get("d", 128), w["n_kv_heads"]
        sb = 2 if dt == "bf16" else 4
        s = w["segs"][b][j]
        nbcap = -(-s["t_cap"] // 16)
        out = set()
        if synth.is_packed(s["kind"]):
            from kv_cache_compression_mkv_amd import layout
            per = layout.record_bytes(s["kind"], s["r"], dt, d, s.get("group", 0))
        else:
            per = 2 * 16 * d * sb
        for off in self._diff(cache.data[b][j], self.data[b][j]):
            g, rem = divmod(int(off), nbcap * per)
            out.add((g, rem // per) if g < hkv else (-1, -1))
        if synth.is_packed(s["kind"]):
            from kv_cache_compression_mkv_amd import layout
            ntile = -(-nbcap // 64)
            tile_bytes = layout.meta_groups(dt, d, s.get("key_ch", 0)) * 64 * 16
            for off in self._diff(cache.meta[b][j], self.meta[b][j]):
                g, rem = divmod(int(off), ntile * tile_bytes)
                tile, rem = divmod(rem, tile_bytes)
                out.add((g, tile * 64 + (rem % 1024) // 16))
        return sorted(out)


def torch_nonzero_offsets(cur, prev):
    """Byte offsets where two equally sized device byte tensors differ (host list)."""
    return (cur != prev).nonzero().flatten().cpu().tolist()
