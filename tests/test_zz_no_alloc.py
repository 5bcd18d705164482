"""mkv_decode_attn_noalloc, the decode entry point that allocates nothing (its
workspace is the library's own scratch array): through the C ABI its outputs
and selections equal mkv_decode_attn's with a caller workspace, bit for bit,
on two calls in a row, the second with a smaller input, and again on the
first input after that."""
import numpy as np
import pytest

import mkv_synth as synth

from gpu_harness import build, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_compression_mkv_amd import _lib  # noqa: F401


def _both(c, q):
    from kv_cache_compression_mkv_amd import _lib as L
    ref_out, ref_sel = c.decode(q, want_sel=True)
    out = torch.empty_like(ref_out)
    sel = torch.full_like(ref_sel, 777)
    L.mkv_decode_attn_noalloc(c.c, q.data_ptr(), out.data_ptr(), sel.data_ptr(), ref_sel.shape[2],
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return ref_out, ref_sel, out, sel


def test_noalloc_equals_workspace_decode():
    from kv_cache_compression_mkv_amd import _lib as L
    big = synth.with_update_segment(synth.workload(3, scale=8), cap=64)   # batch 4, T = 16384, 3 packed segments
    small = synth.workload(2, scale=4)                                     # batch 1, T = 8192, 1 packed segment
    caches = []
    for name, w in (("batch 4, T=16384", big), ("batch 1, T=8192", small)):
        c, _, _ = build(torch, w)
        assert c.workspace_bytes() <= L.MKV_SCRATCH_BYTES
        caches.append((name, w, c))
    assert caches[1][2].workspace_bytes() < caches[0][2].workspace_bytes()
    for i, (name, w, c) in enumerate(caches + caches[:1]):
        q = torch.from_numpy(synth.gen_q(w["cfg"], 40 + i, w["batch"], w["n_q_heads"], w["dtype"])).cuda()
        ref_out, ref_sel, out, sel = _both(c, q)
        assert torch.equal(sel, ref_sel), name
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), name
        assert np.all(np.isfinite(out.cpu().numpy()))
        log("noalloc call %d (%s): outputs and selections equal the workspace call's" % (i, name))


def test_noalloc_equals_workspace_decode_other_layouts():
    """The same equality for bitmap records with element pairs and 64-channel
    block keys, then the default layout again (the scratch array keeps the
    previous call's contents)."""
    from kv_cache_compression_mkv_amd import _lib as L
    w = synth.workload(3, scale=16)
    w["segs"] = synth.with_key_channels(synth.with_groups(synth.as_bitmap(w["segs"]), 2), 64)
    c, _, _ = build(torch, w)
    d, _, _ = build(torch, synth.workload(2, scale=8))
    for i, (name, ww, cc) in enumerate((("bitmap pairs, 64-channel keys", w, c), ("default", synth.workload(2, scale=8), d))):
        assert cc.workspace_bytes() <= L.MKV_SCRATCH_BYTES
        q = torch.from_numpy(synth.gen_q(ww["cfg"], 60 + i, ww["batch"], ww["n_q_heads"], ww["dtype"])).cuda()
        ref_out, ref_sel, out, sel = _both(cc, q)
        assert torch.equal(sel, ref_sel), name
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), name
        log("noalloc (%s): outputs and selections equal the workspace call's" % name)
