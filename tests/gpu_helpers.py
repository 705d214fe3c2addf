"""Helpers for the GPU parity tests: build a library context for a synthetic
workload, run DEX or plain AR through the C ABI, and compare with the oracle
under the margin gate."""

import numpy as np
import torch

from lossless_depth_adaptive_amd import dex as D
from synthetic.noise import gumbel_rows
from synthetic.weights import generate


def device_weights(w):
    return generate(w, device="cuda")


def make_ctx(w, Wd, batch, T, X=None, decs=True, debug=True, max_context=None, gumbel=None, graphs=True,
             single_exit=False, adapters=None, branch_cap=0, span_attention=False):
    """``adapters``: device adapter dicts (synthetic.adapters layout) or None."""
    X = list(X or w.X)
    m = adapters[0]["w1"].shape[0] if adapters else 0
    cfg = D.model_config(w.n_layers, w.d_model, w.n_heads, w.n_kv_heads, w.head_dim, w.d_ffn,
                         w.vocab, w.rope_base, w.eps, w.tied, w.dtype, adapter_hidden=m)
    if max_context is None:
        max_context = w.prompt_len + T + len(X) + 8
    if w.mode == "sample" and gumbel is None:
        gumbel = gumbel_rows(w.seed_g, batch, T + len(X), w.vocab).cuda()
    opt = D.options(w.mode, w.tau, decs, batch, max_context, T, gumbel, debug, graphs, single_exit, branch_cap,
                    span_attention)
    ctx = D.Dex(cfg, Wd, X, opt, adapters=adapters)
    ctx._gumbel = gumbel
    ctx._adapters = adapters
    return ctx


def run(ctx, prompts, T, ar=False, logits_at=None):
    """Decode T tokens per sequence. Returns per-sequence lists of records;
    each record adds u, margins and (for commit indices in ``logits_at``, or
    all when None) the final-depth logits."""
    ctx.prefill(prompts)
    out = [[] for _ in prompts]
    steps = 0
    while any(len(o) < T for o in out):
        recs = ctx.ar_step() if ar else ctx.step()
        steps += 1
        for r in recs:
            t = len(out[r["seq"]])
            want = logits_at is None or t in logits_at
            u, m, lg = ctx.debug_anchor(r["seq"], want_logits=want)
            r["u"], r["margins"] = u, m
            if want:
                r["logits"] = lg
            out[r["seq"]].append(r)
    return out, steps


def compare_with_oracle(gpu_recs, orc_recs, gate, logit_tol, N, check_chain=True):
    """Gated comparison (GPU follows its own stream; the oracle was forced onto
    it). Returns a dict of counters; asserts every gated quantity."""
    n_tok = n_b = 0
    worst = 0.0
    for g, o in zip(gpu_recs, orc_recs):
        assert g["token"] == o["token"]            # oracle was forced onto the GPU stream
        if o["final_margin"] > gate:
            assert g["token"] == o["decoded"], (g, o["decoded"], o["final_margin"])
            n_tok += 1
        if check_chain:
            ok_prefix = True
            for j in range(N):
                ok_prefix = ok_prefix and o["margins"][j] > gate
                if ok_prefix and N > 1:
                    assert g["u"][j] == o["u"][j], (j, g["u"], o["u"], o["margins"])
            # b = min{j : u_j == y} is decided by u_0..u_b and y alone
            if o["final_margin"] > gate and all(m > gate for m in o["margins"][:o["b"] + 1]):
                assert g["branch"] == o["b"] and g["layers"] == o["layers"], (g, o["u"], o["margins"])
                n_b += 1
        if "logits" in g and g["logits"] is not None and "final_logits" in o:
            err = float(np.max(np.abs(g["logits"].astype(np.float64) - o["final_logits"])))
            worst = max(worst, err)
            assert err <= logit_tol, (err, logit_tol)
    return dict(tokens=n_tok, branches=n_b, worst_logit_err=worst)
