"""The strategy pins reject copies of oracle/strategy.py with one planted
mistake each (an off-by-one dropped set, cuts not on block boundaries, the
largest passing r instead of the smallest), and accept an unmodified copy.
CPU only."""
import os
import types

import pytest

import test_strategy_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "strategy.py")
PIN_TESTS = [f for n, f in sorted(vars(pins).items()) if n.startswith("test_")]

MUTANTS = [
    ("tail_off_by_one", "tail = np.concatenate([np.cumsum(col[::-1])[::-1], [0.0]])",
     "tail = np.concatenate([np.cumsum(col[::-1])[::-1][1:], [0.0, 0.0]])"),
    ("cut_inside_blocks", "stop = min(pos + BLOCK, n)", "stop = min(pos + 1, n)"),
    ("largest_passing_r", "for r in range(r_min, r_max + 1):", "for r in range(r_max, r_min - 1, -1):"),
    ("dropped_keeps_one_more", "return float(e[:, r:].sum()), float(e.sum())",
     "return float(e[:, r + 1:].sum()), float(e.sum())"),
]


def _module(text, name):
    m = types.ModuleType(name)
    exec(compile(text, SRC, "exec"), m.__dict__)
    return m


def _failures(mod, monkeypatch):
    monkeypatch.setattr(pins, "st", mod)
    bad = 0
    for f in PIN_TESTS:
        try:
            f()
        except AssertionError:
            bad += 1
    return bad


def test_unmodified_copy_passes(monkeypatch):
    assert _failures(_module(open(SRC).read(), "strategy_copy"), monkeypatch) == 0


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(name, old, new, monkeypatch):
    text = open(SRC).read()
    assert text.count(old) == 1, name
    assert _failures(_module(text.replace(old, new), "strategy_" + name), monkeypatch) > 0
