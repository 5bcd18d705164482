"""Brute force on tiny inputs -- TEST INFRASTRUCTURE ONLY.

Independent code paths that pin the oracle:
  * top-r by enumerating every r-subset of channels and maximising the exact
    sum of magnitudes (ties: lexicographically smallest subset), the
    definition behind the reading notes' Eq. 9 / Algorithm 1;
  * group-granular top-r (one position bit per group of g adjacent channels,
    the paper's section 5.1) by enumerating every choice of r / g groups and
    maximising their exact total energy (same tie rule);
  * top-k blocks by enumerating every k-subset of blocks (same rule), the
    definition behind the paper's top-k block selection (section 4.2);
  * attention by dense reconstruction (zero-filled K^, V^), a masked softmax
    and float64 matrix products, Eq. 13 / Eq. 14 of the reading notes;
  * nearest-even rounding to bfloat16 by searching the sorted table of every
    finite bfloat16 value.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np


def topr_subsets(xr, r: int):
    xr = [Fraction(float(v)) for v in np.asarray(xr, np.float64)]
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(xr)), r):
        s = sum((abs(xr[c]) for c in sub), Fraction(0))
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    return np.array(best, dtype=np.int32)


def topr_group_subsets(xr, r: int, g: int):
    """Channels (ascending) of the best choice of r / g groups of g adjacent channels."""
    xr = [Fraction(float(v)) for v in np.asarray(xr, np.float64)]
    ng = len(xr) // g
    energy = [sum((xr[g * i + m] ** 2 for m in range(g)), Fraction(0)) for i in range(ng)]
    best, best_sum = None, None
    for sub in itertools.combinations(range(ng), r // g):
        s = sum((energy[i] for i in sub), Fraction(0))
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    return np.array([g * i + m for i in best for m in range(g)], dtype=np.int32)


def topk_subsets(scores, k: int):
    sc = [Fraction(float(v)) for v in np.asarray(scores, np.float64)]
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(sc)), k):
        s = sum((sc[i] for i in sub), Fraction(0))
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    return np.array(best, dtype=np.int32)


def attention_dense(Khat, Vhat, qrot, attend, d: int):
    """softmax(q' K^T / sqrt d) V^ over the rows where attend is True."""
    K = np.asarray(Khat, np.float64)[attend]
    V = np.asarray(Vhat, np.float64)[attend]
    z = (K @ np.asarray(qrot, np.float64)) / np.sqrt(d)
    p = np.exp(z - z.max())
    return (p / p.sum()) @ V


def _bf16_table():
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).view(np.float32).astype(np.float64)
    finite = np.isfinite(vals)
    bits, vals = bits[finite], vals[finite]
    # +0 and -0 compare equal; keep +0 once, -0 handled through the sign below
    keep = ~((vals == 0) & (bits != 0))
    bits, vals = bits[keep], vals[keep]
    order = np.argsort(vals, kind="stable")
    return vals[order], bits[order]


_TABLE = None


def nearest_bf16_bits(x):
    """bfloat16 bit pattern nearest to each float64 (ties to even, overflow to inf)."""
    global _TABLE
    if _TABLE is None:
        _TABLE = _bf16_table()
    vals, bits = _TABLE
    x = np.asarray(x, np.float64)
    out = np.empty(x.shape, np.uint32)
    maxv = vals[-1]
    ulp_top = maxv - vals[-2]
    for i, v in np.ndenumerate(x):
        a = abs(v)
        if a >= maxv + ulp_top / 2:
            b = 0x7F80
        else:
            j = np.searchsorted(vals, a)
            cands = [jj for jj in (j - 1, j) if 0 <= jj < len(vals)]
            dist = [abs(vals[jj] - a) for jj in cands]
            m = min(dist)
            tied = [cands[t] for t in range(len(cands)) if dist[t] == m]
            if len(tied) > 1:
                tied = [jj for jj in tied if (bits[jj] & 1) == 0]
            b = int(bits[tied[0]])
        if np.signbit(v):
            b |= 0x8000
        out[i] = b
    return out
