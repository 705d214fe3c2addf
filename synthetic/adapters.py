"""Seeded inducing adapters (inputs, no method arithmetic).

The pages train one residual adapter per non-final exploration depth by
self-distillation ("Depth Exploration for LLM Decoding", Section 3.4 and
Appendix C.2); training needs data that is not here, so the adapters are
seeded stand-ins with the pages' shapes: hidden width m = 2h, two linear
layers with biases, an RMSNorm scale and a scalar gate alpha (initialised to
1e-3 on the pages; a larger alpha makes the adapter visible in tests).

Per adapter k (explorer k < N - 1): w1 [m][h], b1 [m], w2 [h][m], b2 [h] are
N(0, 0.02) from the same quantised-normal generator as the model weights,
seed seed_w + 7919, tensor ids 6k .. 6k + 3; norm [h] is all ones.
"""

from typing import List

import torch

from .configs import Workload
from .weights import normal_tensor, torch_dtype

ADAPTER_SEED_OFFSET = 7919


def adapter_hidden(w: Workload) -> int:
    return 2 * w.d_model


def generate_adapters(w: Workload, alpha: float = 1e-3, device="cpu", dtype: torch.dtype = None) -> List[dict]:
    """One dict per non-final explorer: w1, b1, w2, b2, norm (storage dtype) and alpha (float)."""
    dt = dtype or torch_dtype(w.dtype)
    d, m = w.d_model, adapter_hidden(w)
    seed = w.seed_w + ADAPTER_SEED_OFFSET
    out = []
    for k in range(len(w.X) - 1):
        out.append(dict(
            w1=normal_tensor((m, d), seed, 6 * k, 0.02, dt, device),
            b1=normal_tensor((m,), seed, 6 * k + 1, 0.02, dt, device),
            w2=normal_tensor((d, m), seed, 6 * k + 2, 0.02, dt, device),
            b2=normal_tensor((d,), seed, 6 * k + 3, 0.02, dt, device),
            norm=torch.ones(d, dtype=dt, device=device),
            alpha=float(alpha)))
    return out
