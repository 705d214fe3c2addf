"""A scripted-logit stand-in for the transformer (test helper).

Per context (committed tokens followed by the slot) it fixes a reference
token y* and a readiness depth r in [1, L]. At depth d >= r the top logit is
y*; below r the top logit is another token, y* is the runner-up (so DECS
masking the top exposes y*, a DECS-induced match), and one depth in five
proposes y* early (a transient match). This drives the DEX lattice through
every collapse case without a real model.
"""

import hashlib

import numpy as np


def _h(*parts) -> int:
    b = np.asarray(parts[0], dtype=np.int64).tobytes() + repr(parts[1:]).encode()
    return int.from_bytes(hashlib.blake2b(b, digest_size=8).digest(), "little")


class ScriptedEvaluator:
    def __init__(self, vocab: int, L: int, salt: int = 0):
        self.V, self.L, self.salt = vocab, L, salt

    def begin(self, prompt):
        self.ctx = [int(t) for t in prompt[:-1]]
        self.anchor = int(prompt[-1])
        self.C = len(self.ctx)

    def eval_slots(self, slots):
        pass

    def logits(self, slot, depth):
        c = self.ctx + list(slot)
        hc = _h(c, self.salt)
        ystar = hc % self.V
        r = (hc >> 20) % self.L + 1
        rng = np.random.default_rng(_h(c, self.salt, depth))
        z = rng.random(self.V)
        if depth >= r or (depth < r and (hc >> (depth % 40)) % 5 == 0):
            z[ystar] = 5.0
        else:
            other = (ystar + 1 + (_h(c, depth) % (self.V - 1))) % self.V
            z[other] = 5.0
            z[ystar] = 4.0
        return z

    def commit(self, y):
        self.ctx.append(self.anchor)
        self.anchor = int(y)
        self.C += 1
