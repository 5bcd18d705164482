"""GPU parity of mkv_decode_attn against the oracle.

Selected block ids must equal the oracle's per (request, query head, packed
segment) except where a block's oracle score lies within 1e-4 (relative) of
the k-th largest score. Outputs are compared with the oracle run on the GPU's
selection: relative L2 per head <= 1e-5 for float32 storage, 5e-3 for bf16.
"""
import math

import numpy as np
import pytest

import mkv_synth as synth
from oracle import oracle as orc

from gpu_harness import build, check_decode_unit, gen_raw, log, oracle_unit, rotations, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = {"f32": 1e-5, "bf16": 5e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_compression_mkv_amd import _lib  # noqa: F401


def _decode_and_check(w, c, raw, R, q, units=None, it=0):
    out, sel = c.decode(torch.from_numpy(q).cuda(), want_sel=True)
    torch.cuda.synchronize()
    out, sel = out.cpu().numpy(), sel.cpu().numpy()
    G = w["n_q_heads"] // w["n_kv_heads"]
    units = units or [(b, g) for b in range(w["batch"]) for g in range(w["n_kv_heads"])]
    ex = 0
    for b, g in units:
        length = c.lengths[b]
        comp, Rk, Rv = oracle_unit(w, raw, R, b, g, length)
        hs = slice(g * G, (g + 1) * G)
        ex += check_decode_unit(w, comp, Rk, Rv, q[b, hs].astype(np.float64), out[b, hs], sel[b, hs],
                                TOL[w["dtype"]], length, b, g)
        # padding after the selected blocks
        ksum = sum(k for _, k in orc.seg_blocks(w["segs"][b], length))
        assert np.all(sel[b, hs, ksum:] == -1)
    return out, sel, ex


@pytest.mark.parametrize("cfg,scale,batch", [(1, 1, None), (2, 4, None), (3, 16, None), (4, 64, None),
                                             (5, 32, 4)])
def test_decode_matches_oracle(cfg, scale, batch):
    w = synth.workload(cfg, scale=scale, batch=batch)
    log("decode cfg=%d scale=%d lengths=%s" % (cfg, scale, list(w["lengths"])))
    c, raw, R = build(torch, w)
    for it in range(2):
        q = synth.gen_q(cfg, it, w["batch"], w["n_q_heads"], w["dtype"])
        _, _, ex = _decode_and_check(w, c, raw, R, q, it=it)
        log("  iteration %d: %d exempt near-tie blocks" % (it, ex))


def test_full_retention_equals_dense_attention():
    """r = d and every block kept (float32 storage): decode equals plain softmax
    attention on the raw keys/values (the reading notes' Eq. 1), since R is
    orthogonal -- up to float32 storage rounding."""
    T = 1000
    segs = [synth.seg(synth.DENSE, 0, 40), synth.seg(synth.PACKED, 40, 900, 128, 1000000, 0),
            synth.seg(synth.DENSE, 940, 60)]
    w = dict(cfg=1, batch=1, n_q_heads=4, n_kv_heads=1, d=128, dtype="f32", lengths=np.array([T]), segs=[segs])
    c, raw, R = build(torch, w)
    q = synth.gen_q(7, 0, 1, 4, "f32")
    out = c.decode(torch.from_numpy(q).cuda()).cpu().numpy()
    K = raw[0][0, 0, :T].astype(np.float64)
    V = raw[1][0, 0, :T].astype(np.float64)
    for h in range(4):
        z = K @ q[0, h].astype(np.float64) / math.sqrt(128)
        p = np.exp(z - z.max())
        ref = (p / p.sum()) @ V
        assert np.linalg.norm(out[0, h] - ref) / np.linalg.norm(ref) <= 1e-5


def test_edge_lengths_and_degenerate_queries():
    """Empty requests output zeros; requests that end inside the sink attend only
    dense tokens; a zero query ties every score so the lowest blocks win; a
    single-token packed segment keeps its one block."""
    base = synth.workload(2, scale=16)
    segs = base["segs"][0]
    w = dict(base)
    w["batch"] = 5
    w["segs"] = [segs] * 5
    sink = segs[0]["t_cap"]
    lengths = [0, 3, sink, sink + 1, int(base["lengths"][0])]
    w["lengths"] = np.array(lengths)
    K, V, n = gen_raw(w, [max(t, 1) for t in lengths])
    n = lengths
    from kv_cache_compression_mkv_amd import _lib as L
    R = rotations(L, w, K, V, [max(t, 1) for t in lengths])
    c, raw, R = build(torch, w, lengths=lengths, raw=(K, V, n), R=R)
    q = synth.gen_q(2, 5, 5, w["n_q_heads"], "bf16")
    q[4, :8] = 0.0  # zero queries for the first two KV heads of the last request
    out, sel, _ = _decode_and_check(w, c, raw, R, q)
    assert np.all(out[0] == 0)
    # zero query: the k lowest blocks are chosen
    k = orc.seg_blocks(segs, lengths[4])[0][1]
    assert np.array_equal(sel[4, 0, :k], np.arange(k))


def test_keep_everything_and_absolute_counts():
    """k_abs larger than the segment keeps every block; keep_ppm = 10^6 too."""
    segs = [synth.seg(synth.DENSE, 0, 16), synth.seg(synth.PACKED, 16, 200, 20, 0, 1000),
            synth.seg(synth.PACKED, 216, 300, 9, 1000000, 0), synth.seg(synth.PACKED, 516, 100, 3, 1, 0)]
    w = dict(cfg=9, batch=2, n_q_heads=2, n_kv_heads=1, d=128, dtype="bf16", lengths=np.array([600, 517]),
             segs=[segs, segs])
    c, raw, R = build(torch, w)
    q = synth.gen_q(9, 0, 2, 2, "bf16")
    out, sel, _ = _decode_and_check(w, c, raw, R, q)
    assert np.array_equal(sel[0, 0, :13], np.arange(13))


def test_decode_is_deterministic():
    w = synth.workload(3, scale=32)
    c, raw, R = build(torch, w)
    q = torch.from_numpy(synth.gen_q(3, 0, w["batch"], w["n_q_heads"], "bf16")).cuda()
    o1, s1 = c.decode(q, want_sel=True)
    o2, s2 = c.decode(q, want_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))


def test_serving_steps_append_then_decode():
    """The serving workload's step: append one token per request (rotate, top-r,
    pack, block-key update), then decode; every step checked."""
    w = synth.workload(5, scale=64, batch=4)
    T0 = [int(t) for t in w["lengths"]]
    steps = 20
    K, V, n = gen_raw(w, [t + steps for t in T0])
    from kv_cache_compression_mkv_amd import _lib as L
    R = rotations(L, w, K, V, T0)  # from each request's own prefill rows
    c, raw, R = build(torch, w, lengths=T0, raw=(K, V, n), R=R)
    for s in range(steps):
        kk = np.stack([K[b, :, T0[b] + s:T0[b] + s + 1] for b in range(w["batch"])])
        vv = np.stack([V[b, :, T0[b] + s:T0[b] + s + 1] for b in range(w["batch"])])
        c.append(to_device(torch, np.ascontiguousarray(kk)), to_device(torch, np.ascontiguousarray(vv)),
                 [1] * w["batch"])
        q = synth.gen_q(5, 100 + s, w["batch"], w["n_q_heads"], "bf16")
        units = [(b, g) for b in range(w["batch"]) for g in (0, 5)] if s % 5 else None
        _decode_and_check(w, c, raw, R, q, units=units)
    assert c.lengths == [t + steps for t in T0]


def test_all_dense_cache_pads_selection():
    """Without packed segments nothing is selected: every column of sel_out, at
    any width, is -1; the outputs still match the oracle."""
    from kv_cache_compression_mkv_amd import _lib as L
    segs = [synth.seg(synth.DENSE, 0, 64), synth.seg(synth.DENSE, 64, 200)]
    w = dict(cfg=2, batch=2, n_q_heads=8, n_kv_heads=2, d=128, dtype="bf16", lengths=np.array([150, 90]),
             segs=[segs, segs])
    c, raw, R = build(torch, w)
    assert c.sel_cols() == 0
    q = synth.gen_q(2, 7, 2, 8, "bf16")
    qd = torch.from_numpy(q).cuda()
    out = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
    sel = torch.full((2, 8, 7), 12345, dtype=torch.int32, device="cuda")
    ws = c.workspace()
    L.mkv_decode_attn(c.c, qd.data_ptr(), out.data_ptr(), sel.data_ptr(), 7, ws.data_ptr(), ws.numel(),
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(sel == -1)
    out = out.cpu().numpy()
    for b in range(2):
        for g in range(2):
            comp, Rk, Rv = oracle_unit(w, raw, R, b, g, c.lengths[b])
            ref = orc.decode_unit(comp, q[b, 4 * g:4 * g + 4].astype(np.float64), Rk, Rv)["out"]
            for h in range(4):
                err = np.linalg.norm(out[b, 4 * g + h] - ref[h]) / np.linalg.norm(ref[h])
                assert err <= TOL["bf16"]
