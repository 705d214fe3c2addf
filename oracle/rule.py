"""Decoding rule with depth-coupled sampling (test infrastructure only).

"Depth Exploration for LLM Decoding", Section 3.3 and Appendix C.1,
Algorithm 2 (DECS): tokens already proposed by shallower nodes of the same
slot chain are set to -inf before a non-final node decodes; the final-depth
reference node decodes from unmasked logits. Greedy mode takes the argmax;
sampling mode takes argmax(logits / tau + g) with the Gumbel row g shared by
the slot chain (Gumbel-max trick, the paper's reference [12]).

Readings where the paper is silent: ties go to the lowest token id; the
returned margin is the gap between the largest and second-largest value of the
quantity being maximised (0 on a tie), used to decide which comparisons are
numerically meaningful.
"""

from typing import Iterable, Optional

import numpy as np


def decode(logits: np.ndarray, masked: Iterable[int], mode: str, tau: float,
           gumbel: Optional[np.ndarray]):
    """Returns (token, margin, scores)."""
    s = np.array(logits, dtype=np.float64, copy=True)
    for v in masked:
        s[v] = -np.inf
    if mode == "sample":
        s = s / tau + np.asarray(gumbel, dtype=np.float64)
    elif mode != "greedy":
        raise ValueError(mode)
    y = int(np.argmax(s))              # first maximum = lowest id on ties
    top2 = np.partition(s, -2)[-2:]
    margin = float(top2[1] - top2[0])
    return y, margin, s
