"""Seeded prompt token ids.

"uniform": ids uniform over [0, V), id = floor(h * V / 2^32) for a 32-bit hash h.
"zipf1.1": rank r in [1, V] with P(r) proportional to r^-1.1 (truncated at V),
id = r - 1, drawn by inverse CDF with u = (h + 0.5) / 2^32.
Sequence b of a batch uses hash stream b.
"""

import numpy as np
import torch

from .configs import Workload
from .hashing import hash_range


def prompt_ids(dist: str, vocab: int, length: int, seed: int, stream: int) -> np.ndarray:
    h = hash_range(seed, stream, 0, length).numpy().astype(np.uint64)
    if dist == "uniform":
        ids = (h * np.uint64(vocab)) >> np.uint64(32)
        return ids.astype(np.int32)
    if dist.startswith("zipf"):
        s = float(dist[4:])
        ranks = np.arange(1, vocab + 1, dtype=np.float64)
        cdf = np.cumsum(ranks ** (-s))
        cdf /= cdf[-1]
        u = (h.astype(np.float64) + 0.5) / 4294967296.0
        r = np.searchsorted(cdf, u, side="left")
        return np.minimum(r, vocab - 1).astype(np.int32)
    raise ValueError(dist)


def batch_prompts(w: Workload, length: int = None, batch: int = None):
    """List of int32 arrays, one prompt per sequence."""
    length = w.prompt_len if length is None else length
    batch = w.batch if batch is None else batch
    return [prompt_ids(w.prompt_dist, w.vocab, length, w.seed_p, b) for b in range(batch)]
