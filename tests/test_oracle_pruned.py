"""Pins of the pruned-lattice oracle (the sparse lattice that "Depth Exploration
for LLM Decoding", Appendix E ("Expansion growth and overhead"), names as future work; the policy is this
repository's: only explorers j < cap spawn position children).

* Lossless: the committed stream, the selected branch, the layers and the
  anchor candidates equal plain AR decoding's, for every cap, greedy and
  shared-Gumbel sampling, DECS on and off.
* FSM: N rounds to the first commit; after a commit with branch b, b + 1
  rounds when b < cap (the branch's subtree was kept), N otherwise (fresh
  tree).
* Structure: the round at state q creates, per explorer, exactly the nodes
  whose root path (q moves, depth or position) has no run of cap or more
  depth moves before a position move; counted here by enumerating the move
  strings, independently of the oracle's parent/child construction.
* cap >= N (and cap 0) is the full lattice; cap 1 has the single-exit node set
  (one node per explorer 0..q).
"""

import itertools

import numpy as np
import pytest

from oracle.decode import ar_decode, dex_decode
from oracle.model import PlainModel, SlotEvaluator
from synthetic import get_workload
from synthetic.noise import gumbel_rows
from synthetic.prompts import prompt_ids
from synthetic.weights import generate
from tests.scripted import ScriptedEvaluator


def _rows_by_path_strings(q, N, cap):
    """Nodes of the round at state q per explorer, by enumerating the q moves
    of each node's root path (0 = depth move, 1 = position move)."""
    rows = [0] * N
    for moves in itertools.product((0, 1), repeat=q):
        run, ok = 0, True
        for m in moves:
            if m == 1:
                if cap and run >= cap:
                    ok = False
                    break
                run = 0
            else:
                run += 1
        if ok:
            rows[run] += 1     # trailing depth moves = the node's explorer
    return rows


def _expected_rounds(bs, N, cap):
    eff = cap if 0 < cap < N else N
    return [N] + [b + 1 if b < eff else N for b in bs[:-1]]


def _states(recs, N, cap):
    """FSM state of every round, from the commit records alone."""
    eff = cap if 0 < cap < N else N
    q, out = 0, []
    for r in recs:
        assert r["rounds"] == N - q
        out.extend(range(q, N))
        q = N - 1 - r["b"] if r["b"] < eff else 0
    return out


@pytest.mark.parametrize("N", [2, 3, 4, 6])
@pytest.mark.parametrize("cap", [1, 2, 3])
@pytest.mark.parametrize("decs", [True, False])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_scripted_pruned_equals_ar(N, cap, decs, mode):
    L = 12
    X = sorted(set([round(L * (k + 1) / N) for k in range(N)]))
    V = 13
    prompt = [3, 1, 4, 1, 5]
    T = 60
    G = np.random.default_rng(20 + N).gumbel(size=(T + N + 2, V)) if mode == "sample" else None
    ar = ar_decode(ScriptedEvaluator(V, L, salt=N), prompt, T, X, mode=mode, tau=0.8, gumbel=G, decs=decs)
    st = {}
    dx = dex_decode(ScriptedEvaluator(V, L, salt=N), prompt, T, X, mode=mode, tau=0.8, gumbel=G,
                    decs=decs, stats=st, branch_cap=cap)
    for key in ("token", "b", "layers", "u"):
        assert [r[key] for r in dx] == [r[key] for r in ar], key
    bs = [r["b"] for r in dx]
    if N > cap:
        assert any(b >= cap for b in bs[:-1]) and any(b < cap for b in bs[:-1]), \
            "scripted model must drive both kept and pruned branches"
    assert [r["rounds"] for r in dx] == _expected_rounds(bs, N, cap)
    states = _states(dx, N, cap)
    assert len(states) == len(st["rows_per_round"]) == st["rounds"]
    for q, rows in zip(states, st["rows_per_round"]):
        assert rows == _rows_by_path_strings(q, N, cap), (q, rows)


@pytest.mark.parametrize("N", [3, 4, 5])
def test_cap_at_least_n_is_the_full_lattice(N):
    L = 10
    X = sorted(set([round(L * (k + 1) / N) for k in range(N)]))
    V = 11
    prompt = [2, 7, 1]
    T = 40
    full_st, cap_st, zero_st = {}, {}, {}
    full = dex_decode(ScriptedEvaluator(V, L, salt=N), prompt, T, X, stats=full_st)
    capped = dex_decode(ScriptedEvaluator(V, L, salt=N), prompt, T, X, stats=cap_st, branch_cap=N)
    zero = dex_decode(ScriptedEvaluator(V, L, salt=N), prompt, T, X, stats=zero_st, branch_cap=0)
    assert capped == full and zero == full
    assert cap_st["rows_per_round"] == full_st["rows_per_round"] == zero_st["rows_per_round"]
    for q in range(N):   # the full lattice's closed form, 2^(q-1-j) nodes at explorer j < q and one at q
        assert _rows_by_path_strings(q, N, 0) == [2 ** (q - 1 - j) if j < q else int(j == q) for j in range(N)]


@pytest.mark.parametrize("N", [2, 4, 6])
def test_cap_one_has_the_single_exit_node_set(N):
    for q in range(N):
        assert _rows_by_path_strings(q, N, 1) == [1] * (q + 1) + [0] * (N - 1 - q)


@pytest.mark.parametrize("variant", [
    ("tiny_f32", dict(), 40, 2),
    ("tiny_f32", dict(mode="sample", tau=1.0, seed_g=3001), 40, 1),
    ("llama7b_x8_sample", dict(d_model=256, n_heads=2, n_kv_heads=1, d_ffn=512, vocab=4096,
                               prompt_len=24, n_layers=16, X=tuple(range(2, 17, 2))), 16, 3),
])
def test_real_model_pruned(variant):
    name, kw, T, cap = variant
    w = get_workload(name).scaled(**kw)
    m = PlainModel(w, generate(w))
    p = prompt_ids(w.prompt_dist, w.vocab, w.prompt_len, w.seed_p, 0)
    N = len(w.X)
    G = gumbel_rows(w.seed_g, 1, T + N + 1, w.vocab).numpy()[0] if w.mode == "sample" else None
    ar = ar_decode(SlotEvaluator(m), p, T, w.X, mode=w.mode, tau=w.tau, gumbel=G, brute_ead=False)
    dx = dex_decode(SlotEvaluator(m), p, T, w.X, mode=w.mode, tau=w.tau, gumbel=G, branch_cap=cap)
    for key in ("token", "b", "layers"):
        assert [r[key] for r in dx] == [r[key] for r in ar], key
    assert [r["rounds"] for r in dx] == _expected_rounds([r["b"] for r in dx], N, cap)
