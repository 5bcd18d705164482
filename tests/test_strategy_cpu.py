"""Host segment strategy generation (mkv_strategy_loss_curve,
mkv_strategy_segments) against the oracle (oracle/strategy.py): loss curves
on the same rotations, the same cut positions and r on streams whose
regimes change, binary32 rotations close to the oracle's, the closed forms
at the thresholds' limits, argument checks and bitwise independence of the
host thread count. CPU only."""
import os
import subprocess
import sys

import numpy as np
import pytest

import mkv_synth as synth
from oracle import strategy as st


@pytest.fixture(scope="module")
def L():
    from kv_cache_compression_mkv_amd import _lib
    return _lib


def _haar(rng, d):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))


def _stream(rng, H, d, lengths, decay):
    """Regimes of the given lengths, each with its own basis per head; float32."""
    sig = np.exp(-np.arange(d) / decay)
    parts = []
    for n in lengths:
        Q = np.stack([_haar(rng, d) for _ in range(H)])
        parts.append(np.einsum("hnd,hdc->hnc", rng.standard_normal((H, n, d)) * sig, Q))
    K = np.concatenate(parts, axis=1).astype(np.float32)
    V = (np.concatenate(parts, axis=1) * 0.7 + 0.01).astype(np.float32)
    return K, V


def _as(dtype, X):
    """(library input, oracle fp64 values) of float32 data in the storage dtype."""
    if dtype == "f32":
        return X, X.astype(np.float64)
    bits = synth.f32_to_bf16_bits(X)
    return bits, synth.bf16_bits_to_f32(bits).reshape(X.shape).astype(np.float64)


def _rot_table(Rk, Rv):
    return np.stack([Rk, Rv], axis=1).astype(np.float32)  # [H][2][d][d]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_loss_curve_matches_oracle(L, dtype):
    rng = np.random.default_rng(1)
    H, d = 2, 64
    K, V = _stream(rng, H, d, [300], 5.0)
    Rk = np.stack([_haar(rng, d) for _ in range(H)]).astype(np.float32)
    Rv = np.stack([_haar(rng, d) for _ in range(H)]).astype(np.float32)
    kl, ko = _as(dtype, K)
    vl, vo = _as(dtype, V)
    got = L.mkv_strategy_loss_curve(kl, vl, _rot_table(Rk, Rv))
    exp = st.loss_curve(ko, vo, Rk.astype(np.float64), Rv.astype(np.float64))
    assert np.allclose(got, exp, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_segments_match_oracle(L, dtype):
    rng = np.random.default_rng(2)
    H, d = 2, 64
    K, V = _stream(rng, H, d, [400, 600, 300], 2.5)
    kl, ko = _as(dtype, K)
    vl, vo = _as(dtype, V)
    R0 = np.stack([_haar(rng, d) for _ in range(H)])
    R0 = R0.astype(np.float32).astype(np.float64)
    args = (10, 0.2, 0.02, 4, 48, 32, 4096)
    got = L.mkv_strategy_segments(kl, vl, _rot_table(R0, R0), *args)
    exp = st.segments(ko, vo, R0, R0, *args)
    assert [(e, r) for e, r, _ in got] == [(e, r) for e, r, _, _ in exp]
    assert len(got) >= 3  # the first cut is forced by the strategy in force, then each regime change
    # Rotations: the leading rows (well-separated eigenvalues) agree; trailing
    # rows span numerically degenerate eigenvalues, where any orthonormal basis
    # is an answer, so there both are checked through the loss they give.
    start = 0
    for (e, r, rot), (_, _, Rk, Rv) in zip(got, exp):
        assert np.allclose(rot[:, 0, :8], Rk[:, :8], atol=2e-5) and np.allclose(rot[:, 1, :8], Rv[:, :8], atol=2e-5)
        for R in rot.reshape(-1, d, d).astype(np.float64):
            assert np.allclose(R @ R.T, np.eye(d), atol=1e-5)
        own = st.loss_curve(ko[:, start:e], vo[:, start:e], rot[:, 0].astype(np.float64),
                            rot[:, 1].astype(np.float64))
        ref = st.loss_curve(ko[:, start:e], vo[:, start:e], Rk, Rv)
        assert np.allclose(own, ref, atol=1e-6)
        start = e


def test_segments_closed_forms(L):
    rng = np.random.default_rng(3)
    H, d = 1, 32
    n = 16 * 21 + 5
    K, V = _stream(rng, H, d, [n], 4.0)
    R0 = _rot_table(np.stack([np.eye(d)]), np.stack([np.eye(d)]))
    assert [e for e, _, _ in L.mkv_strategy_segments(K, V, R0, 4, np.inf, 0.1, 1, d, 16, 96)] == [96, 192, 288, n]
    assert [e for e, _, _ in L.mkv_strategy_segments(K, V, R0, 4, -1.0, 0.1, 1, d, 40, 4096)] == \
        [48, 96, 144, 192, 240, 288, 336, n]


def test_strategy_argument_checks(L):
    import ctypes
    rng = np.random.default_rng(4)
    K, V = _stream(rng, 1, 32, [40], 4.0)
    R0 = _rot_table(np.stack([np.eye(32)]), np.stack([np.eye(32)]))
    for bad in (dict(r_min=5, r_max=4), dict(r_max=33), dict(max_len=40), dict(max_len=0), dict(r0=-1),
                dict(cut_loss=float("nan"))):
        a = dict(r0=4, cut_loss=0.1, keep_loss=0.1, r_min=1, r_max=32, min_len=16, max_len=64)
        a.update(bad)
        with pytest.raises(RuntimeError):
            L.mkv_strategy_segments(K, V, R0, a["r0"], a["cut_loss"], a["keep_loss"], a["r_min"], a["r_max"],
                                    a["min_len"], a["max_len"])
    # more segments than the caller's table: the first ones are written, then an error
    with pytest.raises(RuntimeError):
        L.mkv_strategy_segments(K, V, R0, 4, -1.0, 0.1, 1, 32, 16, 64, seg_cap=1)
    st_ = L.LIB.mkv_strategy_segments(None, None, L.MKV_F32, 32, 1, 0, 0, R0.ctypes.data, 4, 0.1, 0.1, 1, 32, 16,
                                      64, 4, np.zeros(4, np.int64).ctypes.data, np.zeros(4, np.int32).ctypes.data,
                                      None, ctypes.byref(ctypes.c_int64(7)))
    assert st_ == 0  # an empty stream is no segment


def test_segments_are_bitwise_independent_of_thread_count():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys, hashlib, numpy as np\n"
        "sys.path.insert(0, %r)\n"
        "from kv_cache_compression_mkv_amd import _lib as L\n"
        "rng = np.random.default_rng(5)\n"
        "K = rng.standard_normal((3, 700, 48)).astype(np.float32)\n"
        "V = (rng.standard_normal((3, 700, 48)) * np.exp(-np.arange(48) / 4)).astype(np.float32)\n"
        "R0 = np.tile(np.eye(48, dtype=np.float32), (3, 2, 1, 1))\n"
        "seg = L.mkv_strategy_segments(K, V, R0, 8, 0.3, 0.05, 2, 40, 16, 256)\n"
        "h = hashlib.sha256()\n"
        "for e, r, rot in seg: h.update(np.int64(e).tobytes() + np.int32(r).tobytes() + rot.tobytes())\n"
        "h.update(L.mkv_strategy_loss_curve(K, V, R0).tobytes())\n"
        "print(len(seg), h.hexdigest())\n" % root)
    outs = set()
    for n in (1, 2, 5):
        env = dict(os.environ, OMP_NUM_THREADS=str(n))
        out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
        outs.add(out.stdout.strip().splitlines()[-1])
    assert len(outs) == 1
