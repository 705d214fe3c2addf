"""Gumbel(0, 1) noise rows that sampled decoding consumes.

Row (b, j) serves sequence b at target position prompt_len_b + j: every node
whose candidate predicts that position reads the same row, so all depths of a
slot chain share it and plain autoregressive decoding reads the same row for
the same position. Element v: u = (h + 0.5) / 2^32 from a 32-bit hash h of
(seed, stream = b * 2^20 + j, v); g = -log(-log(u)) in float64, rounded to
float32. Generated on the CPU and handed to both sides unchanged.
"""

import torch

from .hashing import hash_range


def gumbel_rows(seed: int, batch: int, rows: int, vocab: int) -> torch.Tensor:
    """float32 tensor [batch, rows, vocab] on the CPU."""
    out = torch.empty(batch, rows, vocab, dtype=torch.float32)
    for b in range(batch):
        for j in range(rows):
            h = hash_range(seed, b * (1 << 20) + j, 0, vocab)
            u = (h.to(torch.float64) + 0.5) / 4294967296.0
            out[b, j] = (-torch.log(-torch.log(u))).to(torch.float32)
    return out
