"""Pins of the DEX lattice oracle ("Depth Exploration for LLM Decoding",
Algorithm 1, Sections 3.2-3.3).

* Lossless invariant (Section 3.2): the committed stream equals plain AR
  decoding, greedy and shared-Gumbel sampling, DECS on and off.
* The selected branch and layers per token equal what the anchor path's
  candidates imply at each committed position, computed independently by the
  AR driver.
* layers(t) <= ceil_X(EAD_stab(t)); with DECS off, layers(t) is the first
  explored depth whose candidate equals the committed token.
* Structure stated in Section 3.2 and Appendix E: ETK_1/ETK_2 are the depth
  and position children of ETK_0, state q holds 2^q - 1 nodes, a cycle holds at
  most 2^K - 1 nodes; X = {L} degenerates to AR with b = 0.
"""

import json
import os

import numpy as np
import pytest

from oracle.decode import ar_decode, dex_decode
from oracle.depth import ceil_x, ead_stable, resolution
from oracle.model import PlainModel, SlotEvaluator
from synthetic import get_workload
from synthetic.noise import gumbel_rows
from synthetic.prompts import prompt_ids
from synthetic.weights import generate
from tests.scripted import ScriptedEvaluator


def _same(ar, dx):
    assert [r["token"] for r in ar] == [r["token"] for r in dx]
    assert [r["b"] for r in ar] == [r["b"] for r in dx]
    assert [r["layers"] for r in ar] == [r["layers"] for r in dx]
    assert [r["u"] for r in ar] == [r["u"] for r in dx]


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("decs", [True, False])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_scripted_dex_equals_ar(N, decs, mode):
    L = 12
    X = sorted(set([round(L * (k + 1) / N) for k in range(N)]))
    V = 13
    prompt = [3, 1, 4, 1, 5]
    T = 60
    G = np.random.default_rng(N).gumbel(size=(T + N + 2, V)) if mode == "sample" else None
    ar = ar_decode(ScriptedEvaluator(V, L, salt=N), prompt, T, X, mode=mode, tau=0.8, gumbel=G, decs=decs)
    st = {}
    dx = dex_decode(ScriptedEvaluator(V, L, salt=N), prompt, T, X, mode=mode, tau=0.8, gumbel=G,
                    decs=decs, stats=st)
    _same(ar, dx)
    bs = [r["b"] for r in dx]
    if N > 1:
        assert len(set(bs)) >= min(N, 3), "scripted model must drive several collapse cases"
    # FSM arithmetic: N rounds to the first commit, then b+1 rounds per commit
    assert st["rounds"] == N + sum(b + 1 for b in bs[:-1])
    assert [r["rounds"] for r in dx] == [N] + [b + 1 for b in bs[:-1]]
    for r in ar:
        assert r["layers"] <= ceil_x(r["ead_stab"], X)
        if not decs:
            assert r["layers"] == min(d for d in X if r["cand_by_depth"][d - 1] == r["token"])
        else:
            assert len(set(r["u"][:-1])) == N - 1, "DECS keeps non-final candidates distinct"


def test_scripted_covers_every_collapse_case():
    L, N, V = 16, 8, 101
    X = list(range(2, 17, 2))
    seen = set()
    for salt in range(6):
        ar = ar_decode(ScriptedEvaluator(V, L, salt=salt), [1, 2, 3], 40, X)
        dx = dex_decode(ScriptedEvaluator(V, L, salt=salt), [1, 2, 3], 40, X)
        _same(ar, dx)
        seen |= {r["b"] for r in dx}
    assert seen == set(range(N))


def test_lattice_facts_from_the_paper(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "lattice_facts.json")))
    N = g["n_explorers"]
    st = {}
    # a model whose tokens are never ready early keeps the first cycle full
    dex_decode(ScriptedEvaluator(97, 8, salt=5), [7, 7], 1, [2, 4, 6, 8], stats=st)
    rounds = st["nodes_per_round"]
    assert rounds[0] == [(0, 0, -1, "root", 1)]
    kids = {n[3]: n[0] for n in rounds[1] if n[2] == 0}
    assert kids == {"depth": g["etk0_depth_child"], "position": g["etk0_position_child"]}
    total = 0
    for q in range(1, N + 1):
        total += len(rounds[q - 1])
        assert total == g["tokens_at_state"][str(q)] == 2 ** q - 1
    assert total <= 2 ** N - 1
    # rows per explorer in the round at state q: 2^(q-1-j) for j < q, 1 for j = q
    for q, rows in enumerate(st["rows_per_round"][:N]):
        assert rows == [2 ** (q - 1 - j) if j < q else (1 if j == q else 0) for j in range(N)]


def _real(name, **kw):
    w = get_workload(name).scaled(**kw)
    return w, PlainModel(w, generate(w))


@pytest.mark.parametrize("variant", [
    ("tiny_f32", dict(), 64),
    ("tiny_f32", dict(mode="sample", tau=1.0, seed_g=3001), 48),
    ("tiny_f32", dict(tied=False, gamma=0.8, n_layers=8), 40),
    ("llama7b_x4_greedy", dict(d_model=256, n_heads=2, n_kv_heads=2, d_ffn=512, vocab=4096,
                               prompt_len=24), 24),
    ("llama7b_x8_sample", dict(d_model=256, n_heads=2, n_kv_heads=1, d_ffn=512, vocab=4096,
                               prompt_len=24, n_layers=16, X=tuple(range(2, 17, 2))), 16),
])
def test_real_model_dex_equals_ar(variant):
    name, kw, T = variant
    w, m = _real(name, **kw)
    p = prompt_ids(w.prompt_dist, w.vocab, w.prompt_len, w.seed_p, 0)
    G = gumbel_rows(w.seed_g, 1, T + len(w.X) + 1, w.vocab).numpy()[0] if w.mode == "sample" else None
    ar = ar_decode(SlotEvaluator(m), p, T, w.X, mode=w.mode, tau=w.tau, gumbel=G)
    dx = dex_decode(SlotEvaluator(m), p, T, w.X, mode=w.mode, tau=w.tau, gumbel=G)
    _same(ar, dx)
    D = resolution(w.X, w.n_layers)
    for r in ar:
        assert r["layers"] <= ceil_x(r["ead_stab"], w.X)
        assert 0 <= ceil_x(r["ead_stab"], w.X) - r["ead_stab"] <= D


def test_final_only_set_is_plain_ar():
    w, m = _real("tiny_f32", tied=False, gamma=0.8)
    p = prompt_ids("uniform", w.vocab, 16, 9, 0)
    st = {}
    dx = dex_decode(SlotEvaluator(m), p, 20, [w.n_layers], stats=st)
    ar = ar_decode(SlotEvaluator(m), p, 20, [w.n_layers])
    _same(ar, dx)
    assert all(r["b"] == 0 and r["layers"] == w.n_layers for r in dx)
    assert st["rounds"] == 20


def test_every_layer_explored_reaches_the_ead_oracle():
    w, m = _real("tiny_f32", tied=False, gamma=0.8)
    p = prompt_ids("uniform", w.vocab, 16, 10, 0)
    X = list(range(1, w.n_layers + 1))
    ar = ar_decode(SlotEvaluator(m), p, 12, X, decs=False)
    for r in ar:
        assert ceil_x(r["ead_stab"], X) == r["ead_stab"]
        assert r["layers"] <= r["ead_stab"]
        assert r["layers"] == r["ead"]


def _single_exit_expected(ar, X):
    """Branch of the single-exit ablation, from the AR driver alone: the first
    depth when its unmasked proposal is the committed token, else the final."""
    N = len(X)
    return [0 if r["cand_by_depth"][X[0] - 1] == r["token"] else N - 1 for r in ar]


@pytest.mark.parametrize("N", [2, 3, 4, 6])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_scripted_single_exit(N, mode):
    """Single-exit ablation ("Depth Exploration for LLM Decoding", Section 4,
    Figure 4 right-top): lossless; branch 0 exactly when the first depth's
    proposal is the committed token, else the final depth; one node per
    explorer 0..q in the round at state q; b + 1 rounds per commit."""
    L = 12
    X = sorted(set([round(L * (k + 1) / N) for k in range(N)]))
    V = 13
    prompt = [2, 7, 1, 8]
    T = 60
    G = np.random.default_rng(10 + N).gumbel(size=(T + N + 2, V)) if mode == "sample" else None
    ar = ar_decode(ScriptedEvaluator(V, L, salt=N), prompt, T, X, mode=mode, tau=0.8, gumbel=G)
    st = {}
    dx = dex_decode(ScriptedEvaluator(V, L, salt=N), prompt, T, X, mode=mode, tau=0.8, gumbel=G,
                    stats=st, single_exit=True)
    assert [r["token"] for r in dx] == [r["token"] for r in ar]
    bs = [r["b"] for r in dx]
    assert bs == _single_exit_expected(ar, X)
    assert [r["layers"] for r in dx] == [X[b] for b in bs]
    assert set(bs) == ({0, N - 1} if N > 1 else {0}), "scripted model must hit and miss the first depth"
    assert [r["rounds"] for r in dx] == [N] + [b + 1 for b in bs[:-1]]
    for rows in st["rows_per_round"]:
        k = sum(rows)
        assert rows == [1] * k + [0] * (N - k)


@pytest.mark.parametrize("variant", [
    ("tiny_f32", dict(), 40),
    ("tiny_f32", dict(mode="sample", tau=1.0, seed_g=3001), 40),
])
def test_real_model_single_exit(variant):
    name, kw, T = variant
    w, m = _real(name, **kw)
    p = prompt_ids(w.prompt_dist, w.vocab, w.prompt_len, w.seed_p, 0)
    G = gumbel_rows(w.seed_g, 1, T + len(w.X) + 1, w.vocab).numpy()[0] if w.mode == "sample" else None
    ar = ar_decode(SlotEvaluator(m), p, T, w.X, mode=w.mode, tau=w.tau, gumbel=G)
    dx = dex_decode(SlotEvaluator(m), p, T, w.X, mode=w.mode, tau=w.tau, gumbel=G, single_exit=True)
    assert [r["token"] for r in dx] == [r["token"] for r in ar]
    assert [r["b"] for r in dx] == _single_exit_expected(ar, w.X)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_reprefill_resumes_the_stream(mode):
    """Recovery by re-prefill: a decode restarted from a prefill of
    prompt || the first k committed tokens continues with the same tokens,
    branches and layers (every committed quantity is a function of the
    committed prefix, Section 3.2, "Commit process"; the Gumbel row of a
    target position is the same whichever prefill reached it)."""
    w, m = _real("tiny_f32", tied=False, gamma=0.8, mode=mode, seed_g=3001)
    p = list(prompt_ids(w.prompt_dist, w.vocab, 20, w.seed_p, 0))
    T, k = 24, 9
    G = gumbel_rows(w.seed_g, 1, T + len(w.X) + 1, w.vocab).numpy()[0] if mode == "sample" else None
    full = dex_decode(SlotEvaluator(m), p, T, w.X, mode=mode, tau=w.tau, gumbel=G)
    again = dex_decode(SlotEvaluator(m), p + [r["token"] for r in full[:k]], T - k, w.X, mode=mode, tau=w.tau,
                       gumbel=None if G is None else G[k:])
    assert [(r["token"], r["b"], r["layers"], r["u"]) for r in full[k:]] == \
           [(r["token"], r["b"], r["layers"], r["u"]) for r in again]
    assert [r["position"] for r in full[k:]] == [r["position"] for r in again]
