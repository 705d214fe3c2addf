"""Full-size parity on every bf16 workload, in the launch configuration
bench.py times.

7B-shaped workloads (batch 1, prompt 512 or 1024, 256 new tokens):
* DEX and plain AR on the GPU commit the same 256 tokens; the final-depth
  logits of sampled commits are bit-identical (a property that holds at any
  size: batch invariance of every kernel).
* The first 16 commits are checked against the oracle's stored plain decoding
  (below).

Batched workloads (13B-shaped, 8 sequences, prompts of 1024 Zipf ids, sampled
at temperature 0.7; GQA 32/8 heads, vocabulary 151936, 16 sequences, prompts
of 8192 ids, greedy):
* DEX and plain AR on the GPU commit the same tokens for every sequence over
  the whole generation, with bit-identical final logits at sampled commits;
* the first commits of some sequences are checked against the oracle's plain
  decoding stored in tests/golden/fullsize_<workload>.json (written by
  tests/golden/make_fullsize.py, which calls only the oracle and the input
  generators): token, anchor candidates, branch and layers under the margin
  gate, final logits at stored vocabulary ids within 3e-2, and layers per
  token against the depth ceiling of the brute-force stable EAD.
"""

import json
import os

import numpy as np
import pytest

from synthetic import get_workload
from synthetic.noise import gumbel_rows
from synthetic.prompts import batch_prompts

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# The target's margin gate and logit bound for bf16 weights, and a tighter
# second gate for the decisions compared: over three times the worst full-size
# logit error of the path with its fp16 K/V cache (measured 4.1e-3 on the 7B
# workloads, 4.0e-3 on 13B, 6.0e-3 on the GQA one; 6-7e-3 when the oracle
# itself rounds K/V to fp16 on the 7B and 13B shapes).
GATE, GATE2, TOL = 5e-2, 2e-2, 3e-2


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama7b_x4_greedy", "llama7b_x8_sample"])
def test_fullsize_7b(name):
    from tests.gpu_helpers import device_weights, make_ctx, run
    gold = json.load(open(os.path.join(GOLDEN, f"fullsize_{name}.json")))
    w = get_workload(name)
    T, N = w.gen, len(w.X)
    assert gold["X"] == list(w.X) and gold["seed_w"] == w.seed_w and gold["seed_p"] == w.seed_p
    print(f"[full] {name}: L={w.n_layers} d={w.d_model} X={w.X} prompt={w.prompt_len} T={T}", flush=True)
    Wd = device_weights(w)
    prompts = batch_prompts(w)
    gum = gumbel_rows(w.seed_g, 1, T + N, w.vocab) if w.mode == "sample" else None
    gum_d = gum.cuda() if gum is not None else None
    n_gold = len(gold["seqs"]["0"])
    sample_at = set(range(0, T, 16)) | set(range(n_gold))
    ctx = make_ctx(w, Wd, 1, T, gumbel=gum_d)
    dex_recs, steps = run(ctx, prompts, T, logits_at=sample_at)
    ctx.close()
    ctx = make_ctx(w, Wd, 1, T, gumbel=gum_d)
    ar_recs, _ = run(ctx, prompts, T, ar=True, logits_at=sample_at)
    ctx.close()
    d, a = dex_recs[0], ar_recs[0]
    assert [r["token"] for r in d] == [r["token"] for r in a]
    for i in sorted(sample_at):
        assert np.array_equal(d[i]["logits"].view(np.uint32), a[i]["logits"].view(np.uint32))
    bs = [r["branch"] for r in d]
    assert steps == N + sum(b + 1 for b in bs[:-1])
    print(f"[full] {name}: {T} tokens, {steps} rounds, branch histogram {np.bincount(bs, minlength=N).tolist()}",
          flush=True)
    n, n_dec, ead, worst = compare_golden(d, gold["seqs"]["0"], GATE, GATE2, TOL, N)
    print(f"[full] {name}: {n}/{n_gold} commits equal to the oracle's, {n_dec} anchor candidates compared; "
          f"layers vs ceil_X(EAD_stab): {ead}; worst logit err={worst:.3g}", flush=True)


def compare_golden(gpu, gold, gate, gate2, tol, N):
    """GPU commits of one sequence against the oracle's stored plain decoding.
    The oracle followed its own stream, so the comparison runs until the first
    commit where the streams part, which is only allowed where the oracle's
    final-depth margin is below the tighter gate. Returns (commits compared,
    decisions compared at gate2, layers-vs-EAD counts, worst logit error)."""
    n = n_dec = 0
    worst = 0.0
    ead = dict(agree=0, below=0)
    for g, o in zip(gpu, gold):
        if g["token"] != o["token"]:
            assert o["final_margin"] <= gate2, (g["token"], o["token"], o["final_margin"])
            break
        ok = True
        for j in range(N):
            ok = ok and o["margins"][j] > gate2
            if ok:
                assert g["u"][j] == o["u"][j], (j, g["u"], o["u"], o["margins"])
                n_dec += 1
        if o["final_margin"] > gate2 and all(m > gate2 for m in o["margins"][:o["b"] + 1]):
            assert g["branch"] == o["b"] and g["layers"] == o["layers"], (g, o["u"], o["margins"])
            assert g["layers"] <= o["ceil_ead_stab"]
            ead["agree" if g["layers"] == o["ceil_ead_stab"] else "below"] += 1
        if g.get("logits") is not None:
            z = g["logits"].astype(np.float64)
            for ids, vals in ((o["top_ids"], o["top_logits"]), (o["sample_ids"], o["sample_logits"])):
                err = float(np.max(np.abs(z[ids] - np.asarray(vals))))
                assert err <= tol, (err, tol)
                worst = max(worst, err)
        n += 1
    return n, n_dec, ead, worst


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama13b_x8_b8", "qwen8b_x9_b16"])
def test_fullsize_batched(name):
    from tests.gpu_helpers import device_weights, make_ctx, run
    gold = json.load(open(os.path.join(GOLDEN, f"fullsize_{name}.json")))
    w = get_workload(name)
    T, N = w.gen, len(w.X)
    assert gold["X"] == list(w.X) and gold["seed_w"] == w.seed_w and gold["seed_p"] == w.seed_p
    print(f"[full] {name}: L={w.n_layers} d={w.d_model} heads={w.n_heads}/{w.n_kv_heads} V={w.vocab} "
          f"X={w.X} batch={w.batch} prompt={w.prompt_len} T={T}", flush=True)
    Wd = device_weights(w)
    prompts = batch_prompts(w)
    gum = gumbel_rows(w.seed_g, w.batch, T + N, w.vocab).cuda() if w.mode == "sample" else None
    n_gold = max(len(v) for v in gold["seqs"].values())
    sample_at = set(range(0, T, 32)) | set(range(n_gold))
    ctx = make_ctx(w, Wd, w.batch, T, gumbel=gum)
    dex_recs, steps = run(ctx, prompts, T, logits_at=sample_at)
    ctx.close()
    print(f"[full] {name}: DEX done, {steps} rounds", flush=True)
    ctx = make_ctx(w, Wd, w.batch, T, gumbel=gum)
    ar_recs, _ = run(ctx, prompts, T, ar=True, logits_at=sample_at)
    ctx.close()
    for s in range(w.batch):
        assert [r["token"] for r in dex_recs[s]] == [r["token"] for r in ar_recs[s]], f"seq {s}: DEX != AR"
        for i in sorted(sample_at):
            assert np.array_equal(dex_recs[s][i]["logits"].view(np.uint32), ar_recs[s][i]["logits"].view(np.uint32))
        assert all(r["layers"] == w.X[r["branch"]] for r in dex_recs[s])
    hist = np.bincount([r["branch"] for s in range(w.batch) for r in dex_recs[s]], minlength=N).tolist()
    print(f"[full] {name}: {w.batch} x {T} tokens equal to GPU AR; branch histogram {hist}", flush=True)
    for key, grecs in gold["seqs"].items():
        n, n_dec, ead, worst = compare_golden(dex_recs[int(key)], grecs, GATE, GATE2, TOL, N)
        print(f"[full] {name} seq {key}: {n}/{len(grecs)} commits equal to the oracle's, {n_dec} anchor "
              f"candidates compared; layers vs ceil_X(EAD_stab): {ead}; worst logit err={worst:.3g}", flush=True)
