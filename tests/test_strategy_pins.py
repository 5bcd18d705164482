"""Pins of the segment strategy oracle (oracle/strategy.py) to facts that do
not come from the oracle itself: closed forms of the loss curve, the energy
bound of the reading notes' Eq. 5, an exact-equality case built from
Hadamard sign patterns, and closed forms of the segment cuts in the limits
of the thresholds. CPU only."""
import numpy as np
import pytest

from oracle import oracle as orc
from oracle import strategy as st


def _haar(rng, d):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))


def _hadamard(n):
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_loss_curve_ends_and_monotone():
    rng = np.random.default_rng(1)
    H, n, d = 2, 40, 32
    K = rng.standard_normal((H, n, d))
    V = rng.standard_normal((H, n, d)) * 3.0
    Rk = np.stack([_haar(rng, d) for _ in range(H)])
    Rv = np.stack([_haar(rng, d) for _ in range(H)])
    L = st.loss_curve(K, V, Rk, Rv)
    assert L.shape == (d + 1,)
    assert L[0] == pytest.approx(1.0, abs=1e-14)
    assert L[d] == 0.0
    assert np.all(np.diff(L) <= 1e-15)


def test_one_hot_tokens_lose_nothing_at_r_one():
    """Tokens along single channels of the rotated space: top-1 keeps all."""
    rng = np.random.default_rng(2)
    d, n = 16, 50
    R = _haar(rng, d)
    Xr = np.zeros((n, d))
    Xr[np.arange(n), rng.integers(0, d, n)] = rng.standard_normal(n)
    X = Xr @ R                                         # x = R^T x'
    L = st.loss_curve(X[None], X[None], R[None], R[None])
    assert L[1] == pytest.approx(0.0, abs=1e-12)


def test_energy_bound_of_eq5():
    """With R the segment's own SVD rotation, per-token top-r keeps at least the
    energy of the first r rotated channels, so L(r) <= 1 - Energy(r) with
    Energy(r) = sum_{c<r} sigma_c^2 / sum_c sigma_c^2 (reading notes Eq. 5)."""
    rng = np.random.default_rng(3)
    d, n = 32, 300
    X = rng.standard_normal((n, d)) @ np.diag(np.exp(-np.arange(d) / 6.0)) @ _haar(rng, d).T
    R, sig = orc.rotation(X)
    L = st.loss_curve(X[None], X[None], R[None], R[None])
    e2 = sig ** 2
    energy = np.concatenate([[0.0], np.cumsum(e2)]) / e2.sum()
    assert np.all(L <= 1.0 - energy + 1e-12)
    assert np.any(L < 1.0 - energy - 1e-3)  # strictly better somewhere on generic data


def test_energy_bound_is_exact_when_every_token_is_sorted():
    """Tokens x_t = Q^T (s_t * a) with s_t the rows of a Sylvester Hadamard
    matrix and a strictly decreasing: the Gram matrix is Q^T diag(d a^2) Q, so
    the SVD rotation is Q (up to signs), every token's rotated magnitudes are a
    in order, per-token top-r keeps the first r channels, and L(r) equals
    1 - Energy(r) = sum_{c>=r} a_c^2 / sum_c a_c^2 exactly."""
    rng = np.random.default_rng(4)
    d = 32
    Q = _haar(rng, d)
    a = np.linspace(2.0, 0.1, d)
    S = _hadamard(d)
    X = (S * a) @ Q
    R, _ = orc.rotation(X)
    L = st.loss_curve(X[None], X[None], R[None], R[None])
    expect = np.concatenate([np.cumsum((a ** 2)[::-1])[::-1], [0.0]]) / (a ** 2).sum()
    assert np.allclose(L, expect, atol=1e-12)


def test_choose_r_takes_the_smallest_passing_r():
    L = np.array([1.0, 0.6, 0.4, 0.4, 0.1, 0.0])
    assert st.choose_r(L, 0.4, 1, 5) == 2
    assert st.choose_r(L, 0.4, 3, 5) == 3
    assert st.choose_r(L, 0.05, 1, 4) == 4     # none passes within range: r_max
    assert st.choose_r(L, 1.0, 0, 5) == 0


def _two_regimes(rng, H, d, n_a, n_b, decay=3.0):
    """Tokens from one low-rank regime, then from another with its own basis."""
    sig = np.exp(-np.arange(d) / decay)
    QA = np.stack([_haar(rng, d) for _ in range(H)])
    QB = np.stack([_haar(rng, d) for _ in range(H)])
    # x = Q^T z with z scaled by sig: the rotation Q (rows) maps x back to z
    K = np.concatenate([np.einsum("hnd,hdc->hnc", rng.standard_normal((H, n_a, d)) * sig, QA),
                        np.einsum("hnd,hdc->hnc", rng.standard_normal((H, n_b, d)) * sig, QB)], axis=1)
    V = K * 0.5 + 0.0
    return K, V, QA, QB


def test_segments_closed_forms_at_threshold_limits():
    rng = np.random.default_rng(5)
    H, d = 1, 16
    n = 16 * 21 + 5
    K, V, QA, _ = _two_regimes(rng, H, d, 200, n - 200)
    R0 = QA  # rows of QA: the first regime's basis
    # never exceeded: cuts only at max_len (a multiple of 16) and at the end
    seg = st.segments(K, V, R0, R0, 4, np.inf, 0.1, 1, d, 16, 96)
    assert [s[0] for s in seg] == [96, 192, 288, n]
    # always exceeded once min_len tokens are in: min_len rounded up to a block
    seg = st.segments(K, V, R0, R0, 4, -1.0, 0.1, 1, d, 40, 4096)
    assert [s[0] for s in seg] == [48, 96, 144, 192, 240, 288, 336, n]


def test_segments_cut_after_a_change_of_regime():
    """The strategy in force fits the first regime: no cut before the change;
    the second regime's loss under it is large, so a segment ends inside the
    second regime; its own strategy then fits and no further cut follows."""
    rng = np.random.default_rng(6)
    H, d = 2, 32
    n_a, n_b = 320, 480
    K, V, QA, QB = _two_regimes(rng, H, d, n_a, n_b, decay=2.0)
    r0 = 8
    fit = st.loss_curve(K[:, :n_a], V[:, :n_a], QA, QA)[r0]
    off = st.loss_curve(K[:, n_a:], V[:, n_a:], QA, QA)[r0]
    assert fit < 0.01 and off > 0.3  # the construction separates the regimes
    seg = st.segments(K, V, QA, QA, r0, 0.1, 0.01, 1, d, 16, 65536)
    ends = [s[0] for s in seg]
    # the running loss first exceeds 0.1 about n_a (0.1 - fit) / (off - 0.1) tokens
    # into the second regime (equal energy per token on average); allow twice that
    assert ends[0] > n_a and ends[0] <= n_a + 2 * n_a * (0.1 - fit) / (off - 0.1) + 32
    assert ends[0] % 16 == 0
    assert ends[-1] == n_a + n_b
    # the first segment mixes both regimes; the rest is the second regime only
    assert len(ends) == 2
    for end, r, Rk, Rv in seg:
        assert 1 <= r <= d
        for R in np.concatenate([Rk, Rv]):
            assert np.allclose(R @ R.T, np.eye(d), atol=1e-6)  # binary32 rotations


def test_segment_r_is_the_smallest_r_meeting_keep_loss():
    rng = np.random.default_rng(7)
    H, d = 1, 16
    K, V, QA, _ = _two_regimes(rng, H, d, 160, 0)
    seg = st.segments(K, V, QA, QA, 4, np.inf, 0.02, 2, 12, 16, 65536)
    (end, r, Rk, Rv), = seg
    L = st.loss_curve(K, V, Rk, Rv)
    assert L[r] <= 0.02 and (r == 2 or L[r - 1] > 0.02)


def test_running_loss_is_exact_on_sorted_tokens():
    """Every token of the Hadamard construction loses exactly
    lam = sum_{c>=r} a_c^2 / sum_c a_c^2 under R = Q, so a cut threshold just
    below lam ends the first segment at min_len and one just above it never
    cuts."""
    rng = np.random.default_rng(8)
    d, r = 32, 8
    Q = _haar(rng, d)
    a = np.linspace(2.0, 0.1, d)
    X = np.tile(_hadamard(d) * a, (3, 1)) @ Q          # 96 tokens
    K, V = X[None], X[None] * 0.25
    lam = float((a[r:] ** 2).sum() / (a ** 2).sum())
    below = st.segments(K, V, Q[None], Q[None], r, lam * (1 - 1e-9), 0.5, 1, d, 16, 65536)
    above = st.segments(K, V, Q[None], Q[None], r, lam * (1 + 1e-9), 0.5, 1, d, 16, 65536)
    assert below[0][0] == 16
    assert [s[0] for s in above] == [96]
