"""Seeded weights of a pre-RMSNorm, SwiGLU, RoPE decoder (Llama layout).

Every random tensor is N(0, 0.02) per element, realised as a 16-bit quantised
normal: a 32-bit hash h of (seed, tensor id, element index) selects the
quantile Q[h >> 16] = Phi^-1((j + 0.5) / 65536) of a float64 table. The value
Q * 0.02 * scale is formed in float64, rounded to float32 and then (for bf16
models) rounded to bfloat16, both round-to-nearest-even. This gives identical
bits on the CPU and on a GPU.

Tensor layout is row-major [out_features, in_features] for every projection.
Manifest order (tensor ids): embed; per layer l = 1..L: wq, wk, wv, wo, w_gate,
w_up, w_down; then lm_head (untied models only). Norm weights are all ones.
"""

from typing import Dict, List

import numpy as np
import torch

from .configs import Workload
from .hashing import hash_range

_QTABLE = None
CHUNK_CPU = 1 << 18   # cache-sized pieces: several times faster on the CPU
CHUNK_GPU = 1 << 26


def quantile_table() -> torch.Tensor:
    global _QTABLE
    if _QTABLE is None:
        from scipy.special import ndtri
        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _QTABLE = torch.from_numpy(ndtri(p))
    return _QTABLE


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def normal_tensor(shape, seed: int, stream: int, std: float, dtype: torch.dtype,
                  device="cpu") -> torch.Tensor:
    """N(0, std) tensor of ``shape`` from (seed, stream), bit-reproducible."""
    n = 1
    for s in shape:
        n *= int(s)
    out = torch.empty(n, dtype=dtype, device=device)
    table = quantile_table().to(device)
    chunk = CHUNK_CPU if str(device) == "cpu" else CHUNK_GPU
    for start in range(0, n, chunk):
        cnt = min(chunk, n - start)
        h = hash_range(seed, stream, start, cnt, device=device)
        v = table[h >> 16] * std
        out[start:start + cnt] = v.to(torch.float32).to(dtype)
        del h, v
    return out.view(*shape)


def layer_names() -> List[str]:
    return ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]


def shapes(w: Workload) -> Dict[str, tuple]:
    d, hd = w.d_model, w.head_dim
    return {
        "embed": (w.vocab, d),
        "wq": (w.n_heads * hd, d),
        "wk": (w.n_kv_heads * hd, d),
        "wv": (w.n_kv_heads * hd, d),
        "wo": (d, w.n_heads * hd),
        "w_gate": (w.d_ffn, d),
        "w_up": (w.d_ffn, d),
        "w_down": (d, w.d_ffn),
        "lm_head": (w.vocab, d),
    }


def generate(w: Workload, device="cpu", dtype: torch.dtype = None) -> Dict[str, object]:
    """All weights of workload ``w``.

    Returns a dict with ``embed``, ``layers`` (list of dicts with the seven
    projections plus ``attn_norm``/``ffn_norm``), ``final_norm`` and
    ``lm_head`` (the same tensor object as ``embed`` when tied).
    ``dtype`` defaults to the workload's storage dtype.
    """
    dt = dtype or torch_dtype(w.dtype)
    sh = shapes(w)
    std = 0.02
    sid = 0
    out: Dict[str, object] = {}
    out["embed"] = normal_tensor(sh["embed"], w.seed_w, sid, std, dt, device)
    sid += 1
    layers = []
    for l in range(1, w.n_layers + 1):
        lw = {}
        for name in layer_names():
            scale = std * (w.gamma ** l if name in ("wo", "w_down") else 1.0)
            lw[name] = normal_tensor(sh[name], w.seed_w, sid, scale, dt, device)
            sid += 1
        lw["attn_norm"] = torch.ones(w.d_model, dtype=dt, device=device)
        lw["ffn_norm"] = torch.ones(w.d_model, dtype=dt, device=device)
        layers.append(lw)
    out["layers"] = layers
    out["final_norm"] = torch.ones(w.d_model, dtype=dt, device=device)
    if w.tied:
        out["lm_head"] = out["embed"]
    else:
        out["lm_head"] = normal_tensor(sh["lm_head"], w.seed_w, sid, std, dt, device)
    return out
