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


def run(ctx, prompts, T, ar=False, logits_at=None, rows_log=None, noalloc=False):
    """Decode T tokens per sequence. Returns per-sequence lists of records;
    each record adds u, margins and (for commit indices in ``logits_at``, or
    all when None) the final-depth logits. ``rows_log`` (a list) receives the
    rows each step ran per explorer."""
    ctx.prefill(prompts)
    out = [[] for _ in prompts]
    steps = 0
    while any(len(o) < T for o in out):
        recs = ctx.ar_step() if ar else (ctx.step_noalloc() if noalloc else ctx.step())
        steps += 1
        if rows_log is not None:
            rows_log.append(ctx.last_step_rows()[0])
        for r in recs:
            r["step"] = steps
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


def gated_commit(o, gate):
    """The commit's token and branch are decided with margins above the gate:
    the final-depth decision and the anchor candidates u_0..u_b."""
    return o["final_margin"] > gate and all(m > gate for m in o["margins"][:o["b"] + 1])


def check_ead(gpu_recs, orc_recs, gate, X, decs=True):
    """Layers per token against the depth ceiling of the stable EAD
    ("Depth Exploration for LLM Decoding", Definition 1 eqs. (1)-(3),
    Definition 4 eq. (6), Proposition 6): on every commit whose decisions clear
    the gate, the GPU's layers(t) <= ceil_X(EAD_stab(t)) computed by the
    oracle's brute force over every depth. A commit below the ceiling is a
    transient match (the unmasked candidate at d_b already equals y although
    a deeper layer disagrees) or, with DECS, DECS-induced (masking a shallower
    duplicate exposed y). Returns counts: checked, agree, transient, decs."""
    from oracle.depth import ceil_x
    st = dict(checked=0, agree=0, transient=0, decs=0)
    for g, o in zip(gpu_recs, orc_recs):
        if not gated_commit(o, gate):
            continue
        c = ceil_x(o["ead_stab"], X)
        assert g["layers"] <= c, (g, o["ead_stab"], c)
        st["checked"] += 1
        if g["layers"] == c:
            st["agree"] += 1
        elif o["cand_by_depth"][g["layers"] - 1] == g["token"]:
            st["transient"] += 1
        else:
            assert decs, "without DECS the committed depth is the first explored depth proposing y"
            st["decs"] += 1
        if not decs:
            first = min(d for d in X if o["cand_by_depth"][d - 1] == g["token"])
            assert g["layers"] == first, (g, first)
    return st


def compare_lattice(gpu_recs, gpu_rows, orc_recs, orc_rows, gate, N):
    """One sequence decoded alone on the GPU against the oracle's DEX lattice
    forced onto its stream ("Depth Exploration for LLM Decoding", Algorithm 1,
    Section 3.2): gated token, anchor candidates, branch and layers per
    commit; and, while every branch agrees, the rounds between commits and the
    rows each round ran per explorer (the lattice's node set). Returns the
    number of rounds compared."""
    assert len(gpu_recs) == len(orc_recs)
    agree_upto = len(gpu_recs)
    prev_step = 0
    for t, (g, o) in enumerate(zip(gpu_recs, orc_recs)):
        assert g["token"] == o["token"]
        if o["margins"][-1] > gate:
            assert g["token"] == o["decoded"]
        ok = True
        for j in range(N):
            ok = ok and o["margins"][j] > gate
            if ok:
                assert g["u"][j] == o["u"][j], (t, j, g["u"], o["u"])
        if g["branch"] != o["b"]:
            assert not all(m > gate for m in o["margins"][:max(g["branch"], o["b"]) + 1]), (t, g, o)
            agree_upto = min(agree_upto, t)
        elif t <= agree_upto:
            assert g["layers"] == o["layers"]
        if t <= agree_upto:
            assert g["step"] - prev_step == o["rounds"], (t, g["step"], prev_step, o["rounds"])
        prev_step = g["step"]
    # rounds up to (and including) the last commit whose branch history agrees
    last = gpu_recs[min(agree_upto, len(gpu_recs) - 1)]["step"]
    for r in range(min(last, len(orc_rows), len(gpu_rows))):
        assert list(gpu_rows[r]) == list(orc_rows[r]), (r, gpu_rows[r], orc_rows[r])
    return min(last, len(orc_rows), len(gpu_rows))
