"""Depth arithmetic of "Depth Exploration for LLM Decoding", Section 2
(test infrastructure only).

* ``ceil_x``     - depth ceiling, Definition 4 eq. (6): min{d in X : d >= l}.
* ``resolution`` - Delta(X), eq. (7): max over l in [L] of ceil_X(l) - l.
* ``ead``        - earliest available depth, Definition 1 eq. (1).
* ``ead_stable`` - stable EAD, eqs. (2)-(3): the smallest l such that the
                   candidate is accepted at every depth n >= l.
* ``speedup``    - depth-side speedup, Proposition 7 eq. (12): L T / sum W(t).
* ``speedup_bounds`` - the two outer terms of eq. (14).
"""

from typing import Iterable, Sequence


def check_x(X: Sequence[int], L: int) -> None:
    """Definition 4: d_0 < ... < d_{N-1} = L, all in [L]."""
    if len(X) == 0 or any(b <= a for a, b in zip(X, X[1:])) or X[0] < 1 or X[-1] != L:
        raise ValueError(f"invalid exploration set {X} for L={L}")


def ceil_x(l: int, X: Sequence[int]) -> int:
    return min(d for d in X if d >= l)


def resolution(X: Sequence[int], L: int) -> int:
    return max(ceil_x(l, X) - l for l in range(1, L + 1))


def ead(accept: Sequence[bool]) -> int:
    """``accept[l-1]`` is Omega(t, l) for l = 1..L; Omega(t, L) is 1 by
    construction, so the last entry is ignored and treated as accepted."""
    L = len(accept)
    for l in range(1, L):
        if accept[l - 1]:
            return l
    return L


def ead_stable(accept: Sequence[bool]) -> int:
    L = len(accept)
    best = L
    for l in range(L - 1, 0, -1):       # walk down from L-1 while accepted
        if accept[l - 1]:
            best = l
        else:
            break
    return best


def speedup(L: int, work: Iterable[float]) -> float:
    w = list(work)
    return L * len(w) / sum(w)


def speedup_bounds(L: int, eads: Sequence[int], delta: int):
    """(lower, upper) of eq. (14): LT / sum min(EAD + Delta, L), LT / sum EAD."""
    T = len(eads)
    lo = L * T / sum(min(e + delta, L) for e in eads)
    hi = L * T / sum(eads)
    return lo, hi
