"""dex_step_noalloc, the lattice-step entry point for callers that cannot
allocate device memory, against dex_step through the C ABI: the same commits
(token, position, branch, layers), the same anchor candidates and the same
final-depth logit bits, on two decodes in a row on the same contexts, the
second with a smaller input (one shorter prompt instead of four), so that the
static scratch still holds the first decode's contents; and a context whose
per-round scratch exceeds the static array is refused before any work."""

import numpy as np
import pytest

from synthetic import get_workload
from synthetic.prompts import batch_prompts

pytestmark = pytest.mark.gpu

tiny = get_workload("tiny_f32")
CASES = {
    "tiny_f32": tiny.scaled(batch=4),
    # bf16 storage: the exit head and stage-0 GEMMs take the wide kernel (16 rows
    # and more per group), whose split-range partials also live in the scratch
    "tiny_bf16_sample": tiny.scaled(dtype="bf16", tied=False, gamma=0.8, batch=4, mode="sample", seed_g=3001),
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_noalloc_matches_step(name):
    from tests.gpu_helpers import device_weights, make_ctx, run
    w = CASES[name]
    T = 24
    Wd = device_weights(w)
    big = batch_prompts(w, length=40)
    small = [batch_prompts(w, length=9)[1]]
    mc = 40 + T + len(w.X) + 8
    ref_ctx = make_ctx(w, Wd, 4, T, max_context=mc)
    na_ctx = make_ctx(w, Wd, 4, T, max_context=mc)
    for call, (prompts, t) in enumerate([(big, T), (small, 12)]):
        print(f"[case] noalloc {name} call {call}: {len(prompts)} prompts of {len(prompts[0])} tokens, {t} commits",
              flush=True)
        ref, s_ref = run(ref_ctx, prompts, t)
        got, s_got = run(na_ctx, prompts, t, noalloc=True)
        assert s_ref == s_got
        for s in range(len(prompts)):
            assert len(ref[s]) == len(got[s]) >= t
            for a, b in zip(ref[s], got[s]):
                assert (a["token"], a["position"], a["branch"], a["layers"]) == \
                       (b["token"], b["position"], b["branch"], b["layers"])
                assert a["u"] == b["u"]
                assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
        print(f"[case] noalloc {name} call {call}: {s_got} rounds equal to dex_step", flush=True)
    ref_ctx.close()
    na_ctx.close()


def test_step_noalloc_refuses_large_scratch():
    from lossless_depth_adaptive_amd import dex as D
    from tests.gpu_helpers import device_weights, make_ctx
    # a 151936-token vocabulary at batch 64: a decode round's exit-head tile
    # summaries alone need 64 x 2^(4-1) rows x 9496 tiles x 12 bytes (58 MB),
    # with the split-range GEMM partials (34 MB) beyond 64 MiB
    w = tiny.scaled(dtype="bf16", tied=False, vocab=151936)
    ctx = make_ctx(w, device_weights(w), 64, 4)
    with pytest.raises(D.DexError) as e:
        ctx.step_noalloc()
    assert e.value.code == D.DEX_ENOSPC
    assert "exceeds the static scratch" in str(e.value)
    ctx.close()
