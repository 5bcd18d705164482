"""GPU parity across query-group sizes: the decode kernels are instantiated for
1, 2 and 4 query heads per KV head. The workloads use 4 (and 1 with a single
KV head); these cases run 8 KV heads with 1 and 2 query heads each, in bf16
and fp32 storage, through both calls (mkv_decode_attn after appends, and
mkv_append_decode against separate calls), against the oracle."""
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


def _workload(G, dtype, B=2):
    segs = [synth.seg(synth.DENSE, 0, 64), synth.seg(synth.PACKED, 64, 16 * 150, 26, 50000, 0),
            synth.seg(synth.PACKED, 64 + 16 * 150, 16 * 130, 38, 100000, 0),
            synth.seg(synth.DENSE, 64 + 16 * 280, 256), synth.seg(synth.PACKED, 64 + 16 * 296, 160, 38, 100000, 0)]
    T = [64 + 16 * 296 + 5, 64 + 16 * 280 + 100][:B]
    return dict(cfg=2, batch=B, n_q_heads=8 * G, n_kv_heads=8, d=128, dtype=dtype, lengths=np.array(T),
                segs=[segs] * B)


@pytest.mark.parametrize("G,dtype,layout", [(1, "bf16", "u8"), (2, "bf16", "u8"), (2, "f32", "u8"), (1, "f32", "u8"),
                                            (1, "bf16", "bitmap"), (2, "bf16", "bitmap_pairs"),
                                            (2, "f32", "bitmap")])
def test_group_sizes_match_oracle(G, dtype, layout):
    """Also with bitmap records (one bit per channel, or per pair of channels
    with element pairs), whose decode runs its own kernel instances."""
    from kv_cache_compression_mkv_amd import _lib as L
    w = _workload(G, dtype)
    if layout != "u8":
        w["segs"] = synth.as_bitmap(w["segs"])
    if layout == "bitmap_pairs":
        w["segs"] = synth.with_groups(w["segs"], 2)
    T0 = [int(t) for t in w["lengths"]]
    steps = [1, 1, 24]
    K, V, _ = gen_raw(w, [t + sum(steps) for t in T0])
    R = rotations(L, w, K, V, T0)
    a, _, _ = build(torch, w, lengths=T0, raw=(K, V, T0), R=R)
    t, _, _ = build(torch, w, lengths=T0, raw=(K, V, T0), R=R)
    log("groups G=%d %s %s lengths=%s" % (G, dtype, layout, T0))
    B, hq = w["batch"], w["n_q_heads"]
    for i, nn in enumerate(steps):
        lens = a.lengths
        kk = np.ascontiguousarray(np.stack([K[b, :, lens[b]:lens[b] + nn] for b in range(B)]))
        vv = np.ascontiguousarray(np.stack([V[b, :, lens[b]:lens[b] + nn] for b in range(B)]))
        q = synth.gen_q(2, 700 + i, B, hq, dtype)
        o1, s1 = a.append_decode(to_device(torch, kk), to_device(torch, vv), [nn] * B, torch.from_numpy(q).cuda(),
                                 want_sel=True)
        t.append(to_device(torch, kk), to_device(torch, vv), [nn] * B)
        o2, s2 = t.decode(torch.from_numpy(q).cuda(), want_sel=True)
        torch.cuda.synchronize()
        assert torch.equal(s1, s2) and torch.equal(o1.view(torch.int32), o2.view(torch.int32))
        out, sel = o1.cpu().numpy(), s1.cpu().numpy()
        for b in range(B):
            for g in (0, 3, 7):
                length = a.lengths[b]
                comp, Rk, Rv = oracle_unit(w, (K, V, a.lengths), R, b, g, length)
                if i == len(steps) - 1:
                    compare_compress(a, w, comp, b, g, length)
                hs = slice(g * G, (g + 1) * G)
                check_decode_unit(w, comp, Rk, Rv, q[b, hs].astype(np.float64), out[b, hs], sel[b, hs],
                                  TOL[dtype], length, b, g)
        log("  step %d (+%d): append_decode = separate calls = oracle" % (i, nn))
