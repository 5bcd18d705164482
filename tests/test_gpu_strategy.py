"""Segment strategy generation driving the GPU path: a request whose key and
value statistics change twice is cut into segments by mkv_strategy_segments
(the paper summary's sections 4.3 and 5.5); each segment is packed with the
r and the own rotation the strategy gave it; after one bulk append the
stored records and block keys equal the oracle's, and a decode's selections
and outputs match the oracle with per-segment rotations."""
import numpy as np
import pytest

import mkv_synth as synth
from oracle import oracle as orc

from gpu_harness import build, check_decode_unit, compare_compress, log, raw_to_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_compression_mkv_amd import _lib  # noqa: F401


def _haar(rng, d):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))


def test_strategy_segments_drive_compression_and_decode():
    from kv_cache_compression_mkv_amd import _lib as L
    rng = np.random.default_rng(21)
    hkv, d, sink = 2, 128, 64
    regimes = [sink + 1200, 1600, 900]
    sig = np.exp(-np.arange(d) / 12.0)
    parts = []
    for n in regimes:
        Q = np.stack([_haar(rng, d) for _ in range(hkv)])
        parts.append(np.einsum("hnd,hdc->hnc", rng.standard_normal((hkv, n, d)) * sig, Q) * 4.0)
    X = np.concatenate(parts, axis=1)
    T = X.shape[1]
    Kb = synth.f32_to_bf16_bits(X.astype(np.float32)).reshape(1, hkv, T, d)
    Vb = synth.f32_to_bf16_bits((X * 0.5 + 0.25).astype(np.float32)).reshape(1, hkv, T, d)
    # the cache's rotation: from the first regime's prefill
    R = np.empty((1, hkv, 2, d, d), np.float32)
    for g in range(hkv):
        for kind, arr in ((0, Kb), (1, Vb)):
            x = np.ascontiguousarray(arr[0, g, :regimes[0]])
            L.mkv_rotation_from_prefill(x.ctypes.data, L.MKV_BF16, x.shape[0], d, R[0, g, kind].ctypes.data, None)
    seg = L.mkv_strategy_segments(np.ascontiguousarray(Kb[0, :, sink:]), np.ascontiguousarray(Vb[0, :, sink:]),
                                  R[0], 32, 0.1, 0.02, 8, 96, 256, 65536)
    log("strategy segments (end, r): %s" % [(sink + e, r) for e, r, _ in seg])
    assert 3 <= len(seg) <= 7 and seg[-1][0] == T - sink
    segs = [synth.seg(synth.DENSE, 0, sink)]
    start = sink
    for e, r, _ in seg:
        segs.append(synth.seg(synth.PACKED, start, sink + e - start, r, 100000, 0))
        start = sink + e
    w = dict(cfg=2, batch=1, n_q_heads=4 * hkv, n_kv_heads=hkv, d=d, dtype="bf16", lengths=np.array([T]),
             segs=[segs])
    from kv_cache_compression_mkv_amd.cache import Cache
    c = Cache(1, 4 * hkv, hkv, "bf16", [segs])
    c.set_rotation(R)
    for j, (_, _, rot) in enumerate(seg):
        c.set_segment_rotation(0, j + 1, rot)
    from gpu_harness import to_device
    c.append(to_device(torch, Kb), to_device(torch, Vb), [T])
    q = synth.gen_q(2, 31, 1, 4 * hkv, "bf16")
    out, sel = c.decode(torch.from_numpy(q).cuda(), want_sel=True)
    torch.cuda.synchronize()
    out, sel = out.cpu().numpy(), sel.cpu().numpy()
    for g in range(hkv):
        seg_rot = [None] + [(rot[g, 0].astype(np.float64), rot[g, 1].astype(np.float64)) for _, _, rot in seg]
        Kr, Vr = raw_to_f64(Kb[0, g], "bf16"), raw_to_f64(Vb[0, g], "bf16")
        Rk, Rv = R[0, g, 0].astype(np.float64), R[0, g, 1].astype(np.float64)
        comp = orc.compress_unit(Kr, Vr, Rk, Rv, segs, T, "bf16", seg_rot=seg_rot)
        compare_compress(c, w, comp, 0, g, T)
        check_decode_unit(w, comp, Rk, Rv, q[0, 4 * g:4 * g + 4].astype(np.float64), out[0, 4 * g:4 * g + 4],
                          sel[0, 4 * g:4 * g + 4], 5e-3, T, 0, g)
    log("strategy-driven segments: records, keys, selections and outputs match the oracle")
