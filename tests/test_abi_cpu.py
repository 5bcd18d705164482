"""The C-ABI library on the host: it loads, exports every declared symbol,
reports sizes, rejects invalid arguments before any device work, and its host
rotation matches the oracle's. No GPU is needed (no call here reaches a launch).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import mkv_synth as synth
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from kv_cache_compression_mkv_amd import _lib
    return _lib


def test_exports_every_declared_symbol(L):
    hdr = open(os.path.join(ROOT, "include", "mkv.h")).read()
    declared = set(re.findall(r"\b(mkv_[a-z_]+)\s*\(", hdr))
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(L.LIB, name), name
    assert declared == set(L.EXPORTS)


def test_status_strings(L):
    for s in range(7):
        assert L.mkv_status_str(s) and L.mkv_status_str(s) != "unknown status"
    assert L.mkv_status_str(99) == "unknown status"


def test_segment_bytes(L):
    # packed r=38 bf16: 3648-byte records; meta 512 B per block in 64-block tiles
    data, meta = L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_PACKED, 38, 128, 8, 63456)
    assert data == 8 * 3966 * 3648 + L.MKV_PACKED_TAIL_BYTES
    assert meta == 8 * 62 * 64 * 512
    data, meta = L.mkv_segment_bytes(L.MKV_F32, L.MKV_SEG_PACKED, 32, 128, 1, 4016)
    assert data == 251 * 5120 + L.MKV_PACKED_TAIL_BYTES and meta == 4 * 64 * 1024
    data, meta = L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_PACKED, 26, 128, 1, 16)
    assert data == 2496 + L.MKV_PACKED_TAIL_BYTES
    data, meta = L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_DENSE, 0, 128, 8, 100)
    assert data == 8 * 7 * 2 * 16 * 128 * 2 and meta == 0
    assert L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_PACKED, 0, 128, 8, 100)[0] == 0
    assert L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_PACKED, 129, 128, 8, 100)[0] == 0
    assert L.mkv_segment_bytes(7, L.MKV_SEG_DENSE, 0, 128, 8, 100)[0] == 0
    assert L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_DENSE, 0, 128, 8, 0)[0] == 0
    # bitmap records: the values, then one 16-byte position bitmap per vector
    data, meta = L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_BITMAP, 38, 128, 8, 63456)
    assert data == 8 * 3966 * (2 * 16 * 38 * 2 + 2 * 16 * 16) + L.MKV_PACKED_TAIL_BYTES
    assert meta == 8 * 62 * 64 * 512
    data, meta = L.mkv_segment_bytes(L.MKV_F32, L.MKV_SEG_BITMAP, 128, 128, 1, 17)
    assert data == 2 * (2 * 16 * 128 * 4 + 2 * 16 * 16) + L.MKV_PACKED_TAIL_BYTES and meta == 64 * 1024
    assert L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_BITMAP, 8, 64, 8, 100)[0] == 0  # 128 channels only
    assert L.mkv_segment_bytes(L.MKV_BF16, 3, 8, 128, 8, 100)[0] == 0
    # block keys over the leading key_ch channels: the meta shrinks to key_ch / d, the records do not
    for key_ch, ok in ((32, True), (96, True), (128, True), (8, True), (12, False), (136, False), (-8, False)):
        data, meta = L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_PACKED, 38, 128, 8, 63456, key_ch)
        if ok:
            assert data == 8 * 3966 * 3648 + L.MKV_PACKED_TAIL_BYTES and meta == 8 * 62 * 64 * 2 * key_ch * 2
        else:
            assert data == 0
    data, meta = L.mkv_segment_bytes(L.MKV_F32, L.MKV_SEG_BITMAP, 16, 128, 2, 100, 24)
    assert meta == 2 * 1 * 64 * 2 * 24 * 4
    assert L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_DENSE, 0, 128, 8, 100, 12)[0] > 0  # ignored for dense
    # element groups: bitmaps of one bit per group; u8 records unchanged; g must divide r
    for g, bm_bytes in ((1, 16), (2, 8), (4, 4), (8, 2)):
        data, _ = L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_BITMAP, 40, 128, 8, 63456, 0, g)
        assert data == 8 * 3966 * (2 * 16 * 40 * 2 + 2 * 16 * bm_bytes) + L.MKV_PACKED_TAIL_BYTES
        data, _ = L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_PACKED, 40, 128, 8, 63456, 0, g)
        assert data == 8 * 3966 * 16 * 40 * 2 * 3 + L.MKV_PACKED_TAIL_BYTES
    for g in (3, 16, -2):
        assert L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_BITMAP, 40, 128, 8, 100, 0, g)[0] == 0
    assert L.mkv_segment_bytes(L.MKV_BF16, L.MKV_SEG_BITMAP, 38, 128, 8, 100, 0, 4)[0] == 0  # 4 does not divide 38


class FakeCache:
    """A host-only descriptor with fake (never dereferenced) device pointers."""

    def __init__(self, L, segs, batch=1, hq=32, hkv=8, dtype=None, d=128, lengths=None):
        self.L = L
        n = len(segs)
        self.arr = (L.mkv_segment * (batch * n))()
        self.len = (ctypes.c_int64 * batch)(*(lengths or [0] * batch))
        for b in range(batch):
            for j, s in enumerate(segs):
                e = self.arr[b * n + j]
                e.kind, e.r, e.keep_ppm, e.k_abs = s["kind"], s["r"], s["keep_ppm"], s["k_abs"]
                e.t_begin, e.t_cap = s["t_begin"], s["t_cap"]
                e.key_ch = s.get("key_ch", 0)
                e.group = s.get("group", 0)
                e.data = 0x10000 * (1 + b * n + j)
                e.meta = 0x90000000 + 0x10000 * (b * n + j) if s["kind"] in (1, 2) else None
        self.c = L.mkv_cache(batch, hq, hkv, d, L.MKV_BF16 if dtype is None else dtype, n,
                             ctypes.cast(self.arr, ctypes.POINTER(L.mkv_segment)),
                             ctypes.cast(self.len, ctypes.POINTER(ctypes.c_int64)), 0x5000000)


def _segs_cfg2(scale=1):
    return synth.workload(2, scale=scale)["segs"][0]


def test_workspace_and_sel_cols(L):
    f = FakeCache(L, _segs_cfg2(), lengths=[32768])
    ws = L.mkv_decode_workspace_bytes(f.c)
    assert ws > 0 and ws % 256 == 0
    assert L.mkv_decode_sel_cols(f.c) == 198  # 10% of 1980 blocks
    f.len[0] = 64 + 17  # two blocks in the packed segment -> k = 1
    assert L.mkv_decode_sel_cols(f.c) == 1
    f.len[0] = 10
    assert L.mkv_decode_sel_cols(f.c) == 0


def test_invalid_descriptors_are_rejected(L):
    segs = _segs_cfg2()
    # wrong head dim, group size, dtype
    assert L.mkv_decode_workspace_bytes(FakeCache(L, segs, d=64).c) == 0
    assert L.mkv_decode_workspace_bytes(FakeCache(L, segs, hq=64, hkv=8).c) == 0  # G = 8 unsupported
    assert L.mkv_decode_workspace_bytes(FakeCache(L, segs, hq=30, hkv=8).c) == 0
    assert L.mkv_decode_workspace_bytes(FakeCache(L, segs, dtype=5).c) == 0
    # non-contiguous segments
    bad = [dict(s) for s in segs]
    bad[1]["t_begin"] += 1
    assert L.mkv_decode_workspace_bytes(FakeCache(L, bad).c) == 0
    bad = [dict(s) for s in segs]
    bad[1]["r"] = 0
    assert L.mkv_decode_workspace_bytes(FakeCache(L, bad).c) == 0
    bad = [dict(s) for s in segs]
    bad[1]["keep_ppm"] = 0
    assert L.mkv_decode_workspace_bytes(FakeCache(L, bad).c) == 0
    bad[1]["k_abs"] = 5  # an absolute count makes keep_ppm irrelevant
    assert L.mkv_decode_workspace_bytes(FakeCache(L, bad).c) > 0
    # length beyond capacity
    assert L.mkv_decode_workspace_bytes(FakeCache(L, segs, lengths=[10 ** 6]).c) == 0
    # too many blocks in one packed segment
    big = [synth.seg(1, 0, 16 * 65537, 32, 40000, 0)]
    assert L.mkv_decode_workspace_bytes(FakeCache(L, big).c) == 0


def test_bitmap_descriptors(L):
    """A cache may use either packed record format, but only one of them."""
    segs = _segs_cfg2()
    bm = synth.as_bitmap([segs])[0]
    assert [s["kind"] for s in bm] == [L.MKV_SEG_DENSE, L.MKV_SEG_BITMAP, L.MKV_SEG_DENSE]
    f = FakeCache(L, bm, lengths=[32768])
    assert L.mkv_decode_workspace_bytes(f.c) > 0
    assert L.mkv_decode_sel_cols(f.c) == 198  # the same blocks as the u8-index layout
    # mixed packed formats in one cache are rejected
    two = [synth.seg(synth.DENSE, 0, 64), synth.seg(synth.PACKED, 64, 1024, 32, 100000, 0),
           synth.seg(synth.BITMAP, 1088, 1024, 32, 100000, 0)]
    assert L.mkv_decode_workspace_bytes(FakeCache(L, two, lengths=[1500]).c) == 0
    two[1]["kind"] = synth.BITMAP
    assert L.mkv_decode_workspace_bytes(FakeCache(L, two, lengths=[1500]).c) > 0
    # an unknown kind
    bad = [dict(s) for s in segs]
    bad[1]["kind"] = 3
    assert L.mkv_decode_workspace_bytes(FakeCache(L, bad).c) == 0


def test_key_channel_descriptors(L):
    """key_ch: 0 or a multiple of 8 up to head_dim, the same in every request."""
    base = _segs_cfg2()
    for key_ch, ok in ((0, True), (32, True), (128, True), (20, False), (136, False), (-8, False)):
        segs = synth.with_key_channels([base], key_ch)[0]
        assert (L.mkv_decode_workspace_bytes(FakeCache(L, segs, lengths=[32768]).c) > 0) == ok, key_ch
    # per-request key_ch must agree
    f = FakeCache(L, synth.with_key_channels([base], 32)[0], batch=2, lengths=[32768, 32768])
    assert L.mkv_decode_workspace_bytes(f.c) > 0
    f.arr[1 * len(base) + 1].key_ch = 64
    assert L.mkv_decode_workspace_bytes(f.c) == 0
    f.arr[1 * len(base) + 1].key_ch = 32
    assert L.mkv_decode_workspace_bytes(f.c) > 0


def test_group_descriptors(L):
    """group: 0, 1, 2, 4 or 8, dividing r, the same in every request."""
    base = _segs_cfg2()  # r = 38
    for g, ok in ((0, True), (1, True), (2, True), (4, False), (3, False), (16, False)):
        segs = synth.with_groups([base], g)[0]
        assert (L.mkv_decode_workspace_bytes(FakeCache(L, segs, lengths=[32768]).c) > 0) == ok, g
    f = FakeCache(L, synth.with_groups([base], 2)[0], batch=2, lengths=[32768, 32768])
    assert L.mkv_decode_workspace_bytes(f.c) > 0
    f.arr[1 * len(base) + 1].group = 0
    assert L.mkv_decode_workspace_bytes(f.c) == 0


def test_calls_fail_before_any_launch(L):
    segs = _segs_cfg2()
    f = FakeCache(L, segs, lengths=[32760])
    n_new = (ctypes.c_int32 * 1)(9)
    with pytest.raises(L.MkvError) as e:  # capacity: 32760 + 9 > 32768
        L.mkv_compress_append(f.c, 0x1000, 0x2000, ctypes.addressof(n_new), 9, 0)
    assert e.value.status == L.MKV_ERR_CAPACITY
    assert f.len[0] == 32760  # unchanged
    n_new[0] = 3
    with pytest.raises(L.MkvError) as e:  # n_new > n_max
        L.mkv_compress_append(f.c, 0x1000, 0x2000, ctypes.addressof(n_new), 2, 0)
    assert e.value.status == L.MKV_ERR_ARG
    with pytest.raises(L.MkvError) as e:  # null inputs
        L.mkv_compress_append(f.c, None, None, ctypes.addressof(n_new), 3, 0)
    assert e.value.status == L.MKV_ERR_ARG
    n_new[0] = 0
    L.mkv_compress_append(f.c, None, None, ctypes.addressof(n_new), 0, 0)  # nothing to do: OK, no launch
    with pytest.raises(L.MkvError) as e:  # block meta of a dense segment
        L.mkv_block_meta(f.c, 0, 0)
    assert e.value.status == L.MKV_ERR_ARG
    with pytest.raises(L.MkvError) as e:  # workspace too small
        L.mkv_decode_attn(f.c, 0x1000, 0x2000, None, 0, 0x3000, 16, 0)
    assert e.value.status == L.MKV_ERR_WORKSPACE
    with pytest.raises(L.MkvError) as e:  # sel_out too narrow
        L.mkv_decode_attn(f.c, 0x1000, 0x2000, 0x4000, 3, 0x3000, 1 << 40, 0)
    assert e.value.status == L.MKV_ERR_ARG
    with pytest.raises(L.MkvError) as e:
        L.mkv_decode_attn(f.c, None, 0x2000, None, 0, 0x3000, 1 << 40, 0)
    assert e.value.status == L.MKV_ERR_ARG
    g = FakeCache(L, segs, hq=64, hkv=8)
    with pytest.raises(L.MkvError) as e:
        L.mkv_decode_attn(g.c, 0x1000, 0x2000, None, 0, 0x3000, 1 << 40, 0)
    assert e.value.status == L.MKV_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_host_rotation_matches_oracle(L, dtype):
    """mkv_rotation_from_prefill (Householder + implicit QR) against the oracle's
    cyclic Jacobi on the same stored inputs; both fix the sign the same way."""
    vals, bits = synth.gen_kv(3, 1, 2, 0, 0, 4096, dtype)
    x = np.ascontiguousarray(bits if dtype == "bf16" else vals)
    R = np.empty((128, 128), np.float32)
    sig = np.empty(128, np.float64)
    L.mkv_rotation_from_prefill(x.ctypes.data, L.MKV_BF16 if dtype == "bf16" else L.MKV_F32, 4096, 128,
                                R.ctypes.data, sig.ctypes.data)
    Ro, so = orc.rotation(vals.astype(np.float64))
    assert np.abs(R.astype(np.float64) - Ro).max() <= 1e-6
    assert np.abs(sig - so).max() / so.max() <= 1e-12
    assert np.abs(R.astype(np.float64) @ R.T.astype(np.float64) - np.eye(128)).max() <= 1e-6


def test_host_rotation_edge_cases(L):
    R = np.empty((4, 4), np.float32)
    sig = np.empty(4, np.float64)
    x = np.zeros((0, 4), np.float32)
    L.mkv_rotation_from_prefill(x.ctypes.data, L.MKV_F32, 0, 4, R.ctypes.data, sig.ctypes.data)
    assert np.array_equal(R, np.eye(4, dtype=np.float32)) and np.all(sig == 0)
    x = np.array([[3.0, 0, 0, 0], [0, 0, 2.0, 0]], np.float32)
    L.mkv_rotation_from_prefill(x.ctypes.data, L.MKV_F32, 2, 4, R.ctypes.data, sig.ctypes.data)
    assert sig[0] == 3.0 and sig[1] == 2.0
    assert R[0, 0] == 1.0 and R[1, 2] == 1.0
    with pytest.raises(L.MkvError):
        L.mkv_rotation_from_prefill(x.ctypes.data, L.MKV_F32, 2, 0, R.ctypes.data, None)
    with pytest.raises(L.MkvError):
        L.mkv_rotation_from_prefill(None, L.MKV_F32, 2, 4, R.ctypes.data, None)


def test_host_rotation_is_bitwise_independent_of_thread_count():
    """The Gram sums run in a fixed order, so R and sigma are the same bits at 1
    host thread and at several."""
    import hashlib
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys, hashlib, numpy as np\n"
        "sys.path.insert(0, %r)\n"
        "import mkv_synth as synth\n"
        "from kv_cache_compression_mkv_amd import _lib as L\n"
        "_, bits = synth.gen_kv(3, 0, 1, 1, 0, 20001, 'bf16')\n"
        "R = np.empty((128, 128), np.float32); s = np.empty(128, np.float64)\n"
        "L.mkv_rotation_from_prefill(bits.ctypes.data, L.MKV_BF16, 20001, 128, R.ctypes.data, s.ctypes.data)\n"
        "print(hashlib.sha256(R.tobytes() + s.tobytes()).hexdigest())\n" % root)
    digests = set()
    for n in (1, 3, 8):
        env = dict(os.environ, OMP_NUM_THREADS=str(n))
        out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
        digests.add(out.stdout.strip().splitlines()[-1])
    assert len(digests) == 1


def test_noalloc_rejects_caches_beyond_its_scratch(L):
    """mkv_decode_attn_noalloc refuses, before any device work, a cache whose
    decode needs more than MKV_SCRATCH_BYTES of scratch (64 requests of a
    million-token packed segment: 64 x 32 heads x 65536 fp32 scores alone are
    512 MiB). The device pointers are never dereferenced."""
    B, ns = 64, 1
    segs = (L.mkv_segment * (B * ns))()
    lens = (ctypes.c_int64 * B)(*([1000] * B))
    for b in range(B):
        e = segs[b]
        e.kind, e.r, e.keep_ppm, e.k_abs, e.t_begin, e.t_cap = L.MKV_SEG_PACKED, 32, 40000, 0, 0, 1 << 20
        e.data, e.meta = 4096, 8192
    c = L.mkv_cache(B, 32, 8, 128, L.MKV_BF16, ns, ctypes.cast(segs, ctypes.POINTER(L.mkv_segment)),
                    ctypes.cast(lens, ctypes.POINTER(ctypes.c_int64)), 4096)
    assert L.mkv_decode_workspace_bytes(c) > L.MKV_SCRATCH_BYTES
    with pytest.raises(L.MkvError) as e:
        L.mkv_decode_attn_noalloc(c, 4096, 4096, None, 0, None)
    assert e.value.status == L.MKV_ERR_WORKSPACE
