"""Plain decoder-only transformer in float64 (test infrastructure only).

The model DEX wraps is an ordinary Llama-style decoder ("Depth Exploration for
LLM Decoding", Section 2.1 treats it as a stack of L layers; Section 3.4 and
Appendix C.2 state that every depth is decoded by the same final norm and LM
head). Per layer l = 1..L, for a token at absolute position p:

    a = RMSNorm(h) * g_attn,   RMSNorm(h) = h / sqrt(mean(h^2) + eps)
    Q, K, V = a Wq^T, a Wk^T, a Wv^T          (split into heads of size hd)
    Q, K rotated by RoPE at p: pairs (i, i + hd/2), angle p * base^(-2i/hd)
    per query head h (kv head h // (n_heads / n_kv_heads)):
        o_h = softmax(Q_h K^T / sqrt(hd)) V   over keys at positions <= p
    h = h + o Wo^T
    f = RMSNorm(h) * g_ffn
    h = h + (SiLU(f Wg^T) * (f Wu^T)) Wd^T

Depth-l logits: z_l = (RMSNorm(h_l) * g_final) W_head^T.

Inducing adapters (Section 3.4, Appendix C.2), optional, at non-final
exploration depths l only: the proposal at depth l is decoded from
    h~_l = h_l + alpha_l (W2_l SiLU(W1_l (RMSNorm(h_l) * g_l) + b1_l) + b2_l)
(two linear layers with biases, an RMSNorm scale g_l and a scalar gate; the
activation is the backbone's, SiLU). The residual stream itself is not
changed, and the final depth never has an adapter.

Storage-dtype weights (bf16 or fp32) are upcast exactly to float64; all
arithmetic is float64. With ``resident=False`` the layer weights stay in their
storage dtype and one layer at a time is upcast when a forward reaches it (the
same values, so the same results), which keeps full-size models in host memory.
"""

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np


def _f64(t) -> np.ndarray:
    """torch tensor (any float dtype) or array -> float64 ndarray (exact upcast)."""
    if hasattr(t, "detach"):
        import torch
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


@dataclass
class LayerW:
    attn_norm: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    ffn_norm: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray


_LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


class PlainModel:
    def __init__(self, cfg, weights, adapters=None, resident=True):
        """``cfg`` needs n_layers, d_model, n_heads, n_kv_heads, head_dim,
        d_ffn, vocab, rope_base, eps; ``weights`` is the dict produced by
        ``synthetic.weights.generate``; ``adapters`` (optional) maps a depth
        l < L to a dict w1, b1, w2, b2, norm, alpha. ``resident=False`` keeps
        the layer weights and the embedding as given and upcasts a layer (or
        the gathered embedding rows) each time it is used."""
        self.L = cfg.n_layers
        self.d = cfg.d_model
        self.nq = cfg.n_heads
        self.nkv = cfg.n_kv_heads
        self.hd = cfg.head_dim
        self.V = cfg.vocab
        self.eps = float(cfg.eps)
        self.base = float(cfg.rope_base)
        tied = weights["lm_head"] is weights["embed"]
        self.resident = bool(resident)
        if self.resident:
            self.embed = _f64(weights["embed"])
            self.layers: Optional[List[LayerW]] = [self._upcast(lw) for lw in weights["layers"]]
        else:
            self.embed = weights["embed"]
            self.layers = None
            self._raw_layers = list(weights["layers"])
        self.final_norm = _f64(weights["final_norm"])
        if tied:
            self.head = self.embed if self.resident else _f64(weights["embed"])
        else:
            self.head = _f64(weights["lm_head"])
        self.adapters = {}
        for l, a in (adapters or {}).items():
            assert 1 <= l < self.L, "adapters sit at non-final depths"
            self.adapters[int(l)] = {k: (float(v) if k == "alpha" else _f64(v)) for k, v in a.items()}

    @staticmethod
    def _upcast(lw) -> LayerW:
        return LayerW(**{k: _f64(lw[k]) for k in _LAYER_KEYS})

    def layer(self, l: int) -> LayerW:
        """Weights of layer l (0-based) in float64."""
        if self.layers is not None:
            return self.layers[l]
        return self._upcast(self._raw_layers[l])

    def embed_rows(self, tokens: Sequence[int]) -> np.ndarray:
        """E[tokens] in float64: the embedding rows of the given token ids."""
        idx = np.asarray(tokens, dtype=np.int64)
        if self.resident:
            return self.embed[idx]
        e = self.embed
        if hasattr(e, "detach"):
            import torch
            return _f64(e[torch.from_numpy(idx)])
        return _f64(np.asarray(e)[idx])

    # -- elementary pieces ------------------------------------------------
    def rmsnorm(self, x: np.ndarray, g: np.ndarray) -> np.ndarray:
        return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + self.eps) * g

    def rope(self, x: np.ndarray, pos: np.ndarray) -> np.ndarray:
        """x: [n, heads, hd]; pos: [n] absolute positions."""
        half = self.hd // 2
        inv = self.base ** (-2.0 * np.arange(half, dtype=np.float64) / self.hd)
        ang = pos.astype(np.float64)[:, None] * inv[None, :]          # [n, half]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        x1, x2 = x[..., :half], x[..., half:]
        return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)

    def attend(self, q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
        """One query row. q: [nq, hd]; K, V: [n_keys, nkv, hd] -> [nq * hd]."""
        rep = self.nq // self.nkv
        out = np.empty((self.nq, self.hd))
        for h in range(self.nq):
            kh = K[:, h // rep, :]
            vh = V[:, h // rep, :]
            s = kh @ q[h] / np.sqrt(self.hd)
            s = s - s.max()
            p = np.exp(s)
            p /= p.sum()
            out[h] = p @ vh
        return out.reshape(-1)

    def causal_attention(self, q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
        """All rows of a prompt at positions 0..n-1 at once: row i attends to
        keys 0..i. q: [n, nq, hd]; k, v: [n, nkv, hd] -> [n, nq * hd].
        Per query head, softmax(Q K^T / sqrt(hd) + M) V with M = -inf above
        the diagonal (the same softmax as ``attend``, row by row)."""
        import torch
        n = q.shape[0]
        rep = self.nq // self.nkv
        out = np.empty((n, self.nq, self.hd))
        future = torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1)
        for h in range(self.nq):
            qh = torch.from_numpy(np.ascontiguousarray(q[:, h, :]))
            kh = torch.from_numpy(np.ascontiguousarray(k[:, h // rep, :]))
            vh = torch.from_numpy(np.ascontiguousarray(v[:, h // rep, :]))
            s = (qh @ kh.T) / np.sqrt(self.hd)
            s.masked_fill_(future, -np.inf)
            p = torch.softmax(s, dim=-1)
            out[:, h, :] = (p @ vh).numpy()
            del s, p
        return out.reshape(n, -1)

    def logits(self, h: np.ndarray) -> np.ndarray:
        """Shared exit head: h [..., d] -> [..., V]."""
        return self.rmsnorm(h, self.final_norm) @ self.head.T

    def adapter_delta(self, h: np.ndarray, depth: int) -> np.ndarray:
        """Delta h of the adapter at ``depth`` (zero where there is none)."""
        a = self.adapters.get(int(depth))
        if a is None:
            return np.zeros_like(h)
        u = self.rmsnorm(h, a["norm"]) @ a["w1"].T + a["b1"]
        return a["alpha"] * ((u / (1.0 + np.exp(-u))) @ a["w2"].T + a["b2"])

    def exit_logits(self, h: np.ndarray, depth: int) -> np.ndarray:
        """Logits of a proposal made after ``depth`` layers (adapter applied)."""
        return self.logits(h + self.adapter_delta(h, depth))

    # -- forward passes ---------------------------------------------------
    def prefill(self, tokens: Sequence[int], keep_hidden: bool = True):
        """Full causal forward of ``tokens`` at positions 0..n-1.

        Returns (K, V, hiddens): K, V as lists over layers of [n, nkv, hd];
        hiddens [L+1, n, d] (hiddens[l] = residual stream after l layers), or
        None when ``keep_hidden`` is false.
        """
        n = len(tokens)
        pos = np.arange(n)
        h = self.embed_rows(tokens)
        Ks, Vs, hs = [], [], [h.copy()] if keep_hidden else None
        for l in range(self.L):
            lw = self.layer(l)
            a = self.rmsnorm(h, lw.attn_norm)
            q = self.rope((a @ lw.wq.T).reshape(n, self.nq, self.hd), pos)
            k = self.rope((a @ lw.wk.T).reshape(n, self.nkv, self.hd), pos)
            v = (a @ lw.wv.T).reshape(n, self.nkv, self.hd)
            o = self.causal_attention(q, k, v) if n else np.zeros((0, self.nq * self.hd))
            h = h + o @ lw.wo.T
            f = self.rmsnorm(h, lw.ffn_norm)
            g = f @ lw.w_gate.T
            h = h + ((g / (1.0 + np.exp(-g))) * (f @ lw.w_up.T)) @ lw.w_down.T
            Ks.append(k)
            Vs.append(v)
            if keep_hidden:
                hs.append(h.copy())
            del lw
        return Ks, Vs, (np.stack(hs) if keep_hidden else None)

    def extend(self, tokens: Sequence[int], positions: Sequence[int], past) -> tuple:
        """Forward independent single-token rows, each with its own past keys.

        ``past(i, l, k_i, v_i)`` returns (K, V) arrays [n_keys, nkv, hd] of the
        keys row i attends to at layer l: its past positions, then its own key
        and value (k_i, v_i, [nkv, hd]) last. Rows do not see each other.
        Returns (hiddens [n, L+1, d], K [n, L, nkv, hd], V [n, L, nkv, hd]).
        """
        n = len(tokens)
        pos = np.asarray(positions, dtype=np.int64)
        h = self.embed_rows(tokens)
        hs = [h.copy()]
        kn = np.empty((n, self.L, self.nkv, self.hd))
        vn = np.empty((n, self.L, self.nkv, self.hd))
        for l in range(self.L):
            lw = self.layer(l)
            a = self.rmsnorm(h, lw.attn_norm)
            q = self.rope((a @ lw.wq.T).reshape(n, self.nq, self.hd), pos)
            k = self.rope((a @ lw.wk.T).reshape(n, self.nkv, self.hd), pos)
            v = (a @ lw.wv.T).reshape(n, self.nkv, self.hd)
            kn[:, l], vn[:, l] = k, v
            o = np.empty((n, self.nq * self.hd))
            for i in range(n):
                keys, vals = past(i, l, k[i], v[i])
                o[i] = self.attend(q[i], keys, vals)
            h = h + o @ lw.wo.T
            f = self.rmsnorm(h, lw.ffn_norm)
            g = f @ lw.w_gate.T
            h = h + ((g / (1.0 + np.exp(-g))) * (f @ lw.w_up.T)) @ lw.w_down.T
            hs.append(h.copy())
        return np.stack(hs, axis=1), kn, vn


class SlotEvaluator:
    """Per-depth logits of the plain model for branch contexts.

    A *slot* is the tuple of tokens that follow the committed KV cache: its
    first element is the anchor token (at position C, the committed length)
    and element m sits at position C + m. The slot's candidate predicts
    position C + len(slot). Results are memoised per slot; every slot's proper
    prefixes must have been evaluated before it (true for both plain
    autoregressive decoding and the DEX lattice, where a position child is
    created only after its parent slot).
    """

    def __init__(self, model: PlainModel):
        self.m = model

    def begin(self, prompt: Sequence[int]):
        """Cache prompt[:-1]; the last prompt token becomes the anchor."""
        K, V, _ = self.m.prefill(list(prompt[:-1]), keep_hidden=False)
        self.C = len(prompt) - 1
        # Per layer, the committed keys and values sit in rows [0, C) of a
        # buffer; the rows after them are scratch where a row's ancestor and
        # own entries are laid out behind the committed ones before it attends.
        self.Kb = [np.empty((self.C + 64, self.m.nkv, self.m.hd)) for _ in range(self.m.L)]
        self.Vb = [np.empty((self.C + 64, self.m.nkv, self.m.hd)) for _ in range(self.m.L)]
        for l in range(self.m.L):
            self.Kb[l][:self.C] = K[l]
            self.Vb[l][:self.C] = V[l]
        self.memo = {}                # slot -> (hiddens [L+1, d], K [L,nkv,hd], V)

    @property
    def K(self):
        """Committed keys per layer, [C, nkv, hd] each."""
        return [k[:self.C] for k in self.Kb]

    @property
    def V(self):
        return [v[:self.C] for v in self.Vb]

    def _reserve(self, rows: int):
        if rows <= self.Kb[0].shape[0]:
            return
        cap = 2 * rows
        for buf in (self.Kb, self.Vb):
            for l in range(self.m.L):
                b = np.empty((cap, self.m.nkv, self.m.hd))
                b[:self.C] = buf[l][:self.C]
                buf[l] = b

    def fork(self) -> "SlotEvaluator":
        """An evaluator with a copy of this one's committed cache and an empty
        memo (the state right after a prefill or a commit)."""
        ev = SlotEvaluator(self.m)
        ev.C = self.C
        ev.Kb = [k[:self.C + 64].copy() for k in self.Kb]
        ev.Vb = [v[:self.C + 64].copy() for v in self.Vb]
        ev._reserve(self.C + 64)
        ev.memo = {}
        return ev

    def eval_slots(self, slots: Sequence[tuple]):
        todo = [s for s in dict.fromkeys(slots) if s not in self.memo]
        if not todo:
            return
        for s in todo:
            for m in range(1, len(s)):
                assert s[:m] in self.memo, "slot evaluated before its prefix"

        self._reserve(self.C + max(len(s) for s in todo))

        def past(i, l, k_self, v_self):
            # committed keys, then the slot's earlier tokens, then its own
            s = todo[i]
            C, n = self.C, len(s)
            for m in range(1, n):
                self.Kb[l][C + m - 1] = self.memo[s[:m]][1][l]
                self.Vb[l][C + m - 1] = self.memo[s[:m]][2][l]
            self.Kb[l][C + n - 1] = k_self
            self.Vb[l][C + n - 1] = v_self
            return self.Kb[l][:C + n], self.Vb[l][:C + n]

        hs, kn, vn = self.m.extend([s[-1] for s in todo],
                                   [self.C + len(s) - 1 for s in todo], past)
        for i, s in enumerate(todo):
            self.memo[s] = (hs[i], kn[i], vn[i])

    def logits(self, slot: tuple, depth: int) -> np.ndarray:
        """Logits after ``depth`` layers for the slot's last token (through the
        depth's inducing adapter when the model has one)."""
        return self.m.exit_logits(self.memo[slot][0][depth], depth)

    def commit(self, y: int):
        """The anchor token's KV joins the cache; ``y`` becomes the new anchor.

        Memo entries are kept only for slots that continue (anchor, y, ...),
        re-keyed by dropping the old anchor.
        """
        anchor = [s for s in self.memo if len(s) == 1]
        assert len(anchor) == 1
        a = anchor[0]
        _, k, v = self.memo[a]
        self._reserve(self.C + 1)
        for l in range(self.m.L):
            self.Kb[l][self.C] = k[l]
            self.Vb[l][self.C] = v[l]
        self.C += 1
        self.memo = {s[1:]: val for s, val in self.memo.items()
                     if len(s) >= 2 and s[0] == a[0] and s[1] == y}
