"""Segment strategy generation, fp64 reference -- TEST INFRASTRUCTURE ONLY.

Only the tests may import this module; the product library never does, and
it imports nothing from the product package. It follows the paper summary
("MosaicKV: Serving Long-Context LLM with Dynamic Two-D KV Cache
Compression", paperlayer.ai), sections 4.3 and 5.5, read as follows (each
reading is also listed in the design notes):

  * Compression loss of a token under a strategy (R, r): the energy of its
    rotated vector x' = R x outside its own r largest magnitudes (the
    elements that per-vector top-r drops, reading notes Eq. 9 and
    Algorithm 1), and the loss of a set of tokens is their dropped energy
    over their total rotated energy, summed over the request's KV heads and
    over keys and values (one segment table serves every head, and one r
    serves K and V).
  * A segment ends, at a 16-token block boundary, once it holds at least
    min_len tokens and its loss under the strategy in force exceeds
    cut_loss, or when it reaches max_len tokens (the paper: 64K). The last
    segment ends with the data.
  * A finished segment gets its own rotation per head and matrix, from its
    own tokens (the Gram matrix of the segment, as at prefill: reading notes
    Eq. 4, 6, 7), and the smallest r in [r_min, r_max] whose loss under that
    rotation is at most keep_loss (r_max if none is). That strategy is the
    one in force for the next segment (section 5.4: the current segment is
    compressed with the previous strategy until it is finished).
  * The token-block size stays 16 and the sequence rate is static (section
    5.5 says the sequence compression rate is static).
  * Rotations are applied as stored for compression: rounded to binary32.

The reading notes' Algorithm 2 (variance, outlier ratio and entropy mapped to
r by constants the notes leave open) is not followed: the paper summary's
loss-threshold rule is the primary description.

Parity unpinned: the loss definition (dropped-energy fraction) and the cut
rule's details (block-aligned cuts, min_len, strict "exceeds") are readings
no page value fixes.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as orc

BLOCK = 16


def rotated_energies(X: np.ndarray, R: np.ndarray) -> np.ndarray:
    """Per token, the squared rotated elements sorted descending: [n][d]."""
    Xr = np.asarray(X, np.float64) @ np.asarray(R, np.float64).T  # x'_c = sum_j R[c][j] x_j
    e = Xr * Xr
    return -np.sort(-e, axis=1)


def dropped_total(X: np.ndarray, R: np.ndarray, r: int):
    """(energy dropped by per-token top-r, total rotated energy) over the rows of X."""
    e = rotated_energies(X, R)
    return float(e[:, r:].sum()), float(e.sum())


def loss_curve(K, V, Rk, Rv) -> np.ndarray:
    """L(r) for r = 0 .. d: dropped over total energy of every head's keys and
    values (K, V: [H][n][d]; Rk, Rv: [H][d][d])."""
    d = K.shape[-1]
    dropped = np.zeros(d + 1)
    total = 0.0
    for X, Rs in ((K, Rk), (V, Rv)):
        for h in range(X.shape[0]):
            e = rotated_energies(X[h], Rs[h])
            col = e.sum(axis=0)                    # energy of the i-th largest element, summed over tokens
            tail = np.concatenate([np.cumsum(col[::-1])[::-1], [0.0]])  # tail[r] = sum_{i >= r} col[i]
            dropped += tail
            total += float(col.sum())
    return dropped / total if total > 0 else np.zeros(d + 1)


def choose_r(L: np.ndarray, keep_loss: float, r_min: int, r_max: int) -> int:
    for r in range(r_min, r_max + 1):
        if L[r] <= keep_loss:
            return r
    return r_max


def own_rotation(X: np.ndarray) -> np.ndarray:
    """A segment's rotation from its own rows, rounded to binary32 as stored."""
    R, _ = orc.rotation(np.asarray(X, np.float64))
    return R.astype(np.float32).astype(np.float64)


def segments(K, V, Rk0, Rv0, r0: int, cut_loss: float, keep_loss: float, r_min: int, r_max: int,
             min_len: int, max_len: int):
    """Segments of one request's token stream (K, V: [H][n][d] fp64 values of the
    stored inputs). Returns a list of (end, r, Rk [H][d][d], Rv [H][d][d])."""
    H, n, d = K.shape
    Rk = np.asarray(Rk0, np.float64)
    Rv = np.asarray(Rv0, np.float64)
    r = int(r0)
    out = []
    start = 0
    while start < n:
        end = n
        num = den = 0.0
        pos = start
        while pos < n:
            stop = min(pos + BLOCK, n)
            for X, Rs in ((K, Rk), (V, Rv)):
                for h in range(H):
                    dr, tt = dropped_total(X[h, pos:stop], Rs[h], r)
                    num += dr
                    den += tt
            pos = stop
            length = pos - start
            if length >= max_len or (length >= min_len and num > cut_loss * den):
                end = pos
                break
        Rk = np.stack([own_rotation(K[h, start:end]) for h in range(H)])
        Rv = np.stack([own_rotation(V[h, start:end]) for h in range(H)])
        r = choose_r(loss_curve(K[:, start:end], V[:, start:end], Rk, Rv), keep_loss, r_min, r_max)
        out.append((end, r, Rk, Rv))
        start = end
    return out
