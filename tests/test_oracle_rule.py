"""Pins of oracle.rule (Algorithm 2's decoding step) and of the Gumbel noise
generator it consumes: tie-breaking, masking, and the Gumbel-max law
(argmax(z / tau + g) is distributed as softmax(z / tau), the paper's [12])."""

import numpy as np
from scipy import stats

from oracle.rule import decode
from synthetic.noise import gumbel_rows


def test_greedy_ties_go_to_lowest_id_with_zero_margin():
    z = np.array([0.5, 2.0, -1.0, 2.0, 1.0])
    y, m, _ = decode(z, [], "greedy", 1.0, None)
    assert (y, m) == (1, 0.0)
    y, m, _ = decode(z, [1], "greedy", 1.0, None)
    assert (y, m) == (3, 1.0)


def test_masked_tokens_are_never_chosen():
    rng = np.random.default_rng(3)
    for _ in range(50):
        z = rng.normal(size=20)
        masked = list(rng.choice(20, size=5, replace=False))
        y, m, s = decode(z, masked, "greedy", 1.0, None)
        assert y not in masked and np.all(np.isneginf(s[masked]))
        assert y == max((v for v in range(20) if v not in masked), key=lambda v: (z[v], -v))


def test_gumbel_rows_follow_the_gumbel_cdf():
    g = gumbel_rows(123, 2, 8, 4096).numpy().ravel().astype(np.float64)
    ks = stats.kstest(g, lambda x: np.exp(-np.exp(-x)))
    assert ks.pvalue > 1e-3


def test_gumbel_max_samples_softmax():
    z = np.linspace(-1.5, 1.5, 16) + np.sin(np.arange(16))
    tau = 0.7
    n = 20000
    G = gumbel_rows(77, 1, n, 16).numpy()[0]
    counts = np.zeros(16)
    for j in range(n):
        counts[decode(z, [], "sample", tau, G[j])[0]] += 1
    p = np.exp(z / tau - np.max(z / tau))
    p /= p.sum()
    chi2 = stats.chisquare(counts, p * n)
    assert chi2.pvalue > 1e-3


def test_sampling_margin_is_gap_of_perturbed_scores():
    z = np.array([1.0, 0.0, 0.5])
    g = np.array([0.0, 1.2, 0.0])
    y, m, s = decode(z, [], "sample", 1.0, g)
    assert y == 1 and np.isclose(m, 0.2)
