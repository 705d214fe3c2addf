"""Pins of the inducing-adapter forward in the oracle ("Depth Exploration for
LLM Decoding", Section 3.4 and Appendix C.2).

* Shapes: the generated adapter has 4h^2 + 4h + 1 parameters at m = 2h, and
  that count reproduces the pages' totals for CodeLlama-34B and Llama-2-70B.
* RMSNorm inside: the adapter output does not change when h is scaled.
* Closed forms: W1 = 0 gives alpha (W2 SiLU(b1) + b2); W2 = 0 gives alpha b2;
  alpha = 0 gives the plain exit head.
* Losslessness: with adapters at the non-final depths, DEX still commits the
  AR stream, the final-depth logits are those of the model without adapters,
  and the intermediate proposals do change.
"""

import json
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle.decode import ar_decode, dex_decode
from oracle.model import PlainModel, SlotEvaluator
from synthetic import get_workload
from synthetic.adapters import generate_adapters
from synthetic.noise import gumbel_rows
from synthetic.prompts import prompt_ids
from synthetic.weights import generate


def _count(ad):
    return sum(int(np.prod(v.shape)) for k, v in ad.items() if k != "alpha") + 1


def test_parameter_count_matches_the_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "adapter_params.json")))
    counts = {}
    for h in (64, 96):
        w = get_workload("tiny_f32").scaled(d_model=h)
        counts[h] = _count(generate_adapters(w)[0])
    # fit P(h) = a h^2 + b h + c from the generator's shapes at three sizes
    w = get_workload("tiny_f32").scaled(d_model=32)
    counts[32] = _count(generate_adapters(w)[0])
    hs = np.array(sorted(counts), dtype=np.float64)
    a, b, c = np.linalg.solve(np.vander(hs, 3), np.array([counts[int(x)] for x in hs], dtype=np.float64))
    assert (round(a), round(b), round(c)) == (4, 4, 1)
    H = g["hidden"]
    for ex in g["examples"]:
        total = (ex["K"] - 1) * (4 * H * H + 4 * H + 1)
        assert f"{total:.{ex['rel_digits']}g}" == f"{ex['params']:.{ex['rel_digits']}g}", (ex, total)


def _model_with(w, ads, depths):
    return PlainModel(w, generate(w), adapters=dict(zip(depths, ads)))


def _ads(w, alpha, **override):
    ads = generate_adapters(w, alpha=alpha)
    for a in ads:
        for k, v in override.items():
            a[k] = v(a[k])
    return ads


def test_norm_inside_the_adapter():
    w = get_workload("tiny_f32")
    m = _model_with(w, _ads(w, 0.7), w.X[:-1])
    # RMSNorm is scale invariant up to its eps: take mean(h^2) ~ 1e6 >> eps
    h = 1e3 * np.random.default_rng(1).normal(size=w.d_model)
    for depth in w.X[:-1]:
        np.testing.assert_allclose(m.adapter_delta(3.0 * h, depth), m.adapter_delta(h, depth), rtol=1e-9)
        assert np.abs(m.adapter_delta(h, depth)).max() > 1e-3


def test_closed_forms():
    w = get_workload("tiny_f32")
    h = np.random.default_rng(2).normal(size=w.d_model)
    d0 = w.X[0]
    m = _model_with(w, _ads(w, 0.25, w1=torch.zeros_like), w.X[:-1])
    a = m.adapters[d0]
    np.testing.assert_allclose(m.adapter_delta(h, d0), 0.25 * (a["w2"] @ (a["b1"] * expit(a["b1"])) + a["b2"]),
                               rtol=1e-12)
    m = _model_with(w, _ads(w, 0.25, w2=torch.zeros_like), w.X[:-1])
    np.testing.assert_array_equal(m.adapter_delta(h, d0), 0.25 * m.adapters[d0]["b2"])
    m0 = PlainModel(w, generate(w))
    m = _model_with(w, _ads(w, 0.0), w.X[:-1])
    np.testing.assert_array_equal(m.exit_logits(h, d0), m0.logits(h))


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_adapted_dex_is_lossless(mode):
    w = get_workload("tiny_f32").scaled(tied=False, gamma=0.8, mode=mode, seed_g=3001)
    T = 32
    p = prompt_ids(w.prompt_dist, w.vocab, w.prompt_len, w.seed_p, 0)
    G = gumbel_rows(w.seed_g, 1, T + len(w.X) + 1, w.vocab).numpy()[0] if mode == "sample" else None
    plain = PlainModel(w, generate(w))
    adapted = _model_with(w, _ads(w, 0.5), w.X[:-1])
    ar0 = ar_decode(SlotEvaluator(plain), p, T, w.X, mode=mode, gumbel=G, keep_logits=True, brute_ead=False)
    ar = ar_decode(SlotEvaluator(adapted), p, T, w.X, mode=mode, gumbel=G, keep_logits=True, brute_ead=False)
    dx = dex_decode(SlotEvaluator(adapted), p, T, w.X, mode=mode, gumbel=G)
    assert [r["token"] for r in dx] == [r["token"] for r in ar] == [r["token"] for r in ar0]
    assert [r["b"] for r in dx] == [r["b"] for r in ar]
    for r, r0 in zip(ar, ar0):
        np.testing.assert_array_equal(r["final_logits"], r0["final_logits"])
    assert any(r["u"][:-1] != r0["u"][:-1] for r, r0 in zip(ar, ar0)), "adapters must change some proposal"
