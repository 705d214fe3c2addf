"""Full-size parity on the 7B-shaped workloads, in the launch configuration
bench.py times (batch 1, prompt 512 or 1024, 256 new tokens).

* DEX and plain AR on the GPU commit the same 256 tokens; the final-depth
  logits of sampled commits are bit-identical (a property that holds at any
  size: batch invariance of every kernel).
* The CPU oracle, forced onto the GPU stream, checks the first commits one by
  one: token, anchor candidates, branch (margin-gated at 5e-2) and final
  logits within 3e-2.
"""

import numpy as np
import pytest

from oracle.decode import ar_decode
from oracle.model import PlainModel, SlotEvaluator
from synthetic import get_workload
from synthetic.noise import gumbel_rows
from synthetic.prompts import batch_prompts

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,oracle_commits", [("llama7b_x4_greedy", 4), ("llama7b_x8_sample", 3)])
def test_fullsize_7b(name, oracle_commits):
    import torch
    from tests.gpu_helpers import compare_with_oracle, device_weights, make_ctx, run
    w = get_workload(name)
    T, N = w.gen, len(w.X)
    print(f"[full] {name}: L={w.n_layers} d={w.d_model} X={w.X} prompt={w.prompt_len} T={T}", flush=True)
    Wd = device_weights(w)
    prompts = batch_prompts(w)
    gum = gumbel_rows(w.seed_g, 1, T + N, w.vocab) if w.mode == "sample" else None
    gum_d = gum.cuda() if gum is not None else None
    sample_at = set(range(0, T, 16)) | set(range(oracle_commits))
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
    # oracle on the first commits (weights copied from the generator's device tensors)
    Wc = {"embed": Wd["embed"].cpu(), "final_norm": Wd["final_norm"].cpu(),
          "layers": [{k: v.cpu() for k, v in l.items()} for l in Wd["layers"]]}
    Wc["lm_head"] = Wd["lm_head"].cpu()
    del Wd
    torch.cuda.empty_cache()
    m = PlainModel(w, Wc)
    del Wc
    g = gum[0].numpy() if gum is not None else None
    orc = ar_decode(SlotEvaluator(m), prompts[0], oracle_commits, w.X, mode=w.mode, tau=w.tau, gumbel=g,
                    forced=[r["token"] for r in d[:oracle_commits]], brute_ead=False, keep_logits=True)
    st = compare_with_oracle(d[:oracle_commits], orc, 5e-2, 3e-2, N)
    print(f"[full] {name}: oracle compared {st}", flush=True)
