"""Pins of oracle.depth: the paper's worked example, closed forms and the
propositions' inequalities ("Depth Exploration for LLM Decoding", Section 2.3
and Appendix A.3/A.4)."""

import json
import os
import random

import pytest

from oracle.depth import (ceil_x, check_x, ead, ead_stable, resolution, speedup,
                          speedup_bounds)
from synthetic.configs import ORDER, WORKLOADS


def test_appendix_a3_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "exploration_example.json")))
    assert ceil_x(g["ead"], g["X"]) == g["ceil"]
    assert ceil_x(g["ead"], g["X"]) - g["ead"] == g["overhead"]
    assert resolution(g["X"], g["L"]) == g["delta"]


@pytest.mark.parametrize("name,delta", list(zip(ORDER, [1, 7, 3, 4, 3])))
def test_resolution_of_uniform_sets(name, delta):
    # A uniform set with spacing s starting at d_0 = s leaves l = 1 furthest
    # from its ceiling: Delta = s - 1.
    w = WORKLOADS[name]
    check_x(w.X, w.n_layers)
    assert resolution(w.X, w.n_layers) == delta == w.X[0] - 1


def test_ceiling_is_identity_on_full_set():
    L = 12
    X = list(range(1, L + 1))
    assert all(ceil_x(l, X) == l for l in range(1, L + 1))
    assert resolution(X, L) == 0


def test_final_only_set():
    L = 9
    assert all(ceil_x(l, [L]) == L for l in range(1, L + 1))
    assert resolution([L], L) == L - 1


@pytest.mark.parametrize("bad", [[], [3, 2, 8], [0, 8], [2, 4, 6], [2, 2, 8]])
def test_invalid_sets_rejected(bad):
    with pytest.raises(ValueError):
        check_x(bad, 8)


def test_ead_hand_examples():
    # Omega over depths 1..4 (the last entry is accepted by construction).
    assert ead([True, False, True, False]) == 1
    assert ead_stable([True, False, True, False]) == 3          # transient match at 1
    assert ead_stable([False, False, False, False]) == 4
    assert ead([False, False, False, False]) == 4
    assert ead_stable([True, True, True, True]) == 1
    assert ead_stable([False, True, True, True]) == 2


def test_proposition6_bound_random_sets():
    rng = random.Random(7)
    for _ in range(300):
        L = rng.randint(1, 40)
        X = sorted(set(rng.sample(range(1, L + 1), rng.randint(1, L))) | {L})
        D = resolution(X, L)
        for l in range(1, L + 1):
            assert 0 <= ceil_x(l, X) - l <= D


def test_proposition7_bounds_and_monotonicity():
    rng = random.Random(11)
    for _ in range(200):
        L = rng.randint(2, 40)
        T = rng.randint(1, 30)
        eads = [rng.randint(1, L) for _ in range(T)]
        X = sorted(set(rng.sample(range(1, L + 1), rng.randint(1, L))) | {L})
        Xf = sorted(set(X) | set(rng.sample(range(1, L + 1), rng.randint(1, L))))
        D = resolution(X, L)
        sx = speedup(L, [ceil_x(e, X) for e in eads])
        sxf = speedup(L, [ceil_x(e, Xf) for e in eads])
        lo, hi = speedup_bounds(L, eads, D)
        assert 1.0 <= lo + 1e-12 and lo <= sx + 1e-12 and sx <= hi + 1e-12
        assert sx <= sxf + 1e-12 <= hi + 2e-12
        full = list(range(1, L + 1))
        assert abs(speedup(L, [ceil_x(e, full) for e in eads]) - hi) < 1e-12
