"""Writes tests/golden/fullsize_<workload>.json: the CPU oracle's plain
autoregressive decoding of the first commits of some sequences of a full-size
workload (test infrastructure; calls only ``oracle/`` and ``synthetic/``).

DEX is lossless ("Depth Exploration for LLM Decoding", Section 3.2, "Commit
process"): the committed stream is the plain model's, and what a commit
records besides the token (the anchor-path candidates u_0..u_{N-1} with DECS,
the branch b = min{j : u_j = y} and the layers d_b) is a function of the
committed prefix. So ``oracle.decode.ar_decode`` gives every quantity the GPU
path reports per commit, plus the brute-force stable EAD (Definition 1,
eqs. (1)-(3)) and its depth ceiling (Definition 4, eq. (6)).

The oracle follows its own stream here (nothing is forced), so a GPU test can
compare commits up to the first one where the two streams may legitimately
part (a final-depth margin below the gate).

Usage (full-size models need their bf16 weights in host memory: about 26 GB
for the 13B shape, 16 GB for the GQA shape):

    python tests/golden/make_fullsize.py llama13b_x8_b8 --seqs 0 1 --commits 8
    python tests/golden/make_fullsize.py qwen8b_x9_b16 --seqs 0 --commits 8
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle.decode import ar_decode  # noqa: E402
from oracle.depth import ceil_x  # noqa: E402
from oracle.model import PlainModel, SlotEvaluator  # noqa: E402
from synthetic import get_workload  # noqa: E402
from synthetic.noise import gumbel_rows  # noqa: E402
from synthetic.prompts import batch_prompts  # noqa: E402
from synthetic.weights import generate  # noqa: E402

# Logit samples kept per commit: the 16 largest final-depth logits and every
# LOGIT_STRIDE-th vocabulary entry.
TOPK = 16
LOGIT_STRIDE = 997


def log(*a):
    print(time.strftime("%H:%M:%S"), *a, file=sys.stderr, flush=True)


def record(w, r):
    z = r["final_logits"]
    top = np.argsort(-z, kind="stable")[:TOPK]
    ids = np.arange(0, w.vocab, LOGIT_STRIDE)
    ceil = ceil_x(r["ead_stab"], w.X)
    return dict(token=int(r["token"]), position=int(r["position"]), final_margin=float(r["final_margin"]),
                u=[int(x) for x in r["u"]], margins=[float(x) for x in r["margins"]], b=int(r["b"]),
                layers=int(r["layers"]), ead=int(r["ead"]), ead_stab=int(r["ead_stab"]), ceil_ead_stab=int(ceil),
                cand_by_depth=[int(x) for x in r["cand_by_depth"]],
                top_ids=[int(i) for i in top], top_logits=[float(z[i]) for i in top],
                sample_ids=[int(i) for i in ids], sample_logits=[float(z[i]) for i in ids])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--seqs", type=int, nargs="+", default=[0])
    ap.add_argument("--commits", type=int, default=8)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    w = get_workload(args.workload)
    t0 = time.time()
    W = generate(w, device="cpu")
    log(f"{w.name}: weights generated in {time.time() - t0:.0f}s")
    model = PlainModel(w, W, resident=False)
    prompts = batch_prompts(w)
    T = args.commits
    gum = gumbel_rows(w.seed_g, w.batch, T + len(w.X), w.vocab) if w.mode == "sample" else None
    seqs = {}
    for s in args.seqs:
        t1 = time.time()
        g = gum[s].numpy() if gum is not None else None
        recs = ar_decode(SlotEvaluator(model), prompts[s], T, w.X, mode=w.mode, tau=w.tau, gumbel=g,
                         brute_ead=True, keep_logits=True)
        seqs[str(s)] = [record(w, r) for r in recs]
        log(f"{w.name} seq {s}: {T} commits in {time.time() - t1:.0f}s; tokens {[r['token'] for r in recs]}")
    out = dict(workload=w.name, X=list(w.X), n_layers=w.n_layers, vocab=w.vocab, mode=w.mode, tau=w.tau,
               prompt_len=w.prompt_len, seed_w=w.seed_w, seed_p=w.seed_p, seed_g=w.seed_g,
               precision="float64 arithmetic on the storage-dtype weights", topk=TOPK, logit_stride=LOGIT_STRIDE,
               script="tests/golden/make_fullsize.py", seqs=seqs)
    path = args.out or os.path.join(HERE, f"fullsize_{w.name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    log(f"wrote {path}")


if __name__ == "__main__":
    main()
