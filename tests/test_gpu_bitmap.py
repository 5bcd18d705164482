"""GPU parity of the bitmap record format (MKV_SEG_BITMAP; the paper summary's
section 5.1: a position bitmap per vector instead of per-element indices).

The kept set, the values and their order, the block keys and every selection
are those of the u8-index format, so the oracle is the same: records and keys
must match it bit for bit (each bitmap holding exactly the kept channels),
mkv_block_meta must rebuild the keys from bitmap records, appends in ragged
pieces must equal one bulk append, and decodes (alone and fused with an
append) must select the oracle's blocks and match its outputs, with the same
selections as the same cache in the u8 format."""
import numpy as np
import pytest

import mkv_synth as synth

from gpu_harness import build, check_decode_unit, compare_compress, gen_raw, log, oracle_unit, rotations, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = {"f32": 1e-5, "bf16": 5e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_compression_mkv_amd import _lib  # noqa: F401


def _bitmap(w):
    w = dict(w)
    w["segs"] = synth.as_bitmap(w["segs"])
    return w


@pytest.mark.parametrize("cfg,scale,batch", [(1, 1, None), (2, 8, None), (3, 32, None), (5, 64, 3)])
def test_bitmap_records_and_decode_match_oracle(cfg, scale, batch):
    from kv_cache_compression_mkv_amd import _lib as L
    wu = synth.workload(cfg, scale=scale, batch=batch)
    w = _bitmap(wu)
    T = [int(t) for t in w["lengths"]]
    log("bitmap cfg=%d scale=%d lengths=%s" % (cfg, scale, T))
    K, V, n = gen_raw(w, T)
    R = rotations(L, w, K, V, n)
    c, raw, _ = build(torch, w, raw=(K, V, n), R=R)
    u, _, _ = build(torch, wu, raw=(K, V, n), R=R)
    for b in range(w["batch"]):
        for g in range(w["n_kv_heads"]):
            comp, _, _ = oracle_unit(w, raw, R, b, g, T[b])
            compare_compress(c, w, comp, b, g, T[b])
    G = w["n_q_heads"] // w["n_kv_heads"]
    for it in range(2):
        q = synth.gen_q(cfg, it, w["batch"], w["n_q_heads"], w["dtype"])
        out, sel = c.decode(torch.from_numpy(q).cuda(), want_sel=True)
        _, sel_u = u.decode(torch.from_numpy(q).cuda(), want_sel=True)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_u), "bitmap and u8 caches select different blocks"
        out, sel = out.cpu().numpy(), sel.cpu().numpy()
        for b in range(w["batch"]):
            for g in sorted({0, w["n_kv_heads"] - 1}):
                comp, Rk, Rv = oracle_unit(w, raw, R, b, g, T[b])
                hs = slice(g * G, (g + 1) * G)
                check_decode_unit(w, comp, Rk, Rv, q[b, hs].astype(np.float64), out[b, hs], sel[b, hs],
                                  TOL[w["dtype"]], T[b], b, g)
        log("  iteration %d: selections equal the u8 layout's and the oracle's" % it)


def test_bitmap_incremental_appends_and_block_meta():
    """Ragged appends equal one bulk append; mkv_block_meta rebuilds the keys
    from bitmap records."""
    from kv_cache_compression_mkv_amd import _lib as L
    from kv_cache_compression_mkv_amd import layout
    from kv_cache_compression_mkv_amd.cache import Cache
    w = _bitmap(synth.workload(5, scale=64, batch=3))
    T = [int(t) for t in w["lengths"]]
    K, V, n = gen_raw(w, T)
    R = rotations(L, w, K, V, n)
    bulk, _, _ = build(torch, w, raw=(K, V, n), R=R)
    inc = Cache(w["batch"], w["n_q_heads"], w["n_kv_heads"], w["dtype"], w["segs"])
    inc.set_rotation(R)
    rng = np.random.default_rng(3)
    done = [0] * w["batch"]
    while any(d < t for d, t in zip(done, T)):
        step = [int(min(t - d, rng.integers(0, 40))) for d, t in zip(done, T)]
        nmax = max(max(step), 1)
        kk = np.zeros((w["batch"], w["n_kv_heads"], nmax, 128), K.dtype)
        vv = np.zeros_like(kk)
        for b in range(w["batch"]):
            kk[b, :, :step[b]] = K[b, :, done[b]:done[b] + step[b]]
            vv[b, :, :step[b]] = V[b, :, done[b]:done[b] + step[b]]
        inc.append(to_device(torch, kk), to_device(torch, vv), step)
        done = [d + s for d, s in zip(done, step)]
    torch.cuda.synchronize()
    for b in range(w["batch"]):
        for j in range(len(w["segs"][b])):
            assert torch.equal(inc.data[b][j], bulk.data[b][j]), "records differ b=%d seg=%d" % (b, j)
            if inc.meta[b][j] is not None:
                assert torch.equal(inc.meta[b][j], bulk.meta[b][j]), "keys differ b=%d seg=%d" % (b, j)
    saved = [[m.clone() if m is not None else None for m in row] for row in bulk.meta]
    for row in bulk.meta:
        for m in row:
            if m is not None:
                m.fill_(0xAB)
    bulk.block_meta(1)
    torch.cuda.synchronize()
    for b in range(w["batch"]):
        nb = -(-(T[b] - w["segs"][b][1]["t_begin"]) // 16)
        cap = -(-w["segs"][b][1]["t_cap"] // 16)
        _, got = layout.unpack_meta(bulk.meta[b][1].cpu().numpy(), w["n_kv_heads"], cap, w["dtype"])
        _, exp = layout.unpack_meta(saved[b][1].cpu().numpy(), w["n_kv_heads"], cap, w["dtype"])
        assert np.array_equal(got[:, :nb], exp[:, :nb])
    log("bitmap records: ragged appends = bulk append; block keys rebuilt from bitmaps")


def test_bitmap_append_decode_serving_steps():
    """Serving steps through mkv_append_decode on a bitmap cache equal separate
    append and decode calls bit for bit, and match the oracle."""
    from kv_cache_compression_mkv_amd import _lib as L
    w = _bitmap(synth.workload(5, scale=64, batch=4))
    T0 = [int(t) for t in w["lengths"]]
    steps = [[1] * 4] * 3 + [[40] * 4, [1, 0, 17, 1]]
    extra = sum(max(s) for s in steps)
    K, V, _ = gen_raw(w, [t + extra for t in T0])
    R = rotations(L, w, K, V, T0)
    a, raw, _ = build(torch, w, lengths=T0, raw=(K, V, T0), R=R)
    t, _, _ = build(torch, w, lengths=T0, raw=(K, V, T0), R=R)
    G = w["n_q_heads"] // w["n_kv_heads"]
    for i, n_new in enumerate(steps):
        lens = a.lengths
        nmax = max(1, max(n_new))
        kk = np.zeros((4, w["n_kv_heads"], nmax, 128), K.dtype)
        vv = np.zeros_like(kk)
        for b in range(4):
            kk[b, :, :n_new[b]] = K[b, :, lens[b]:lens[b] + n_new[b]]
            vv[b, :, :n_new[b]] = V[b, :, lens[b]:lens[b] + n_new[b]]
        q = synth.gen_q(5, 400 + i, 4, w["n_q_heads"], w["dtype"])
        o1, s1 = a.append_decode(to_device(torch, kk), to_device(torch, vv), n_new, torch.from_numpy(q).cuda(),
                                 want_sel=True)
        t.append(to_device(torch, kk), to_device(torch, vv), n_new)
        o2, s2 = t.decode(torch.from_numpy(q).cuda(), want_sel=True)
        torch.cuda.synchronize()
        assert torch.equal(s1, s2) and torch.equal(o1.view(torch.int32), o2.view(torch.int32))
        out, sel = o1.cpu().numpy(), s1.cpu().numpy()
        for b, g in ((0, 0), (3, w["n_kv_heads"] - 1)):
            length = a.lengths[b]
            comp, Rk, Rv = oracle_unit(w, (K, V, a.lengths), R, b, g, length)
            compare_compress(a, w, comp, b, g, length)
            check_decode_unit(w, comp, Rk, Rv, q[b, G * g:G * g + G].astype(np.float64), out[b, G * g:G * g + G],
                              sel[b, G * g:G * g + G], 5e-3, length, b, g)
        log("  bitmap serving step %d n_new=%s: append_decode = separate calls = oracle" % (i, n_new))
