#!/usr/bin/env python3
"""Benchmark of the DEX lattice step on one MI355X.

A step is one dex_step call: one lattice round (expand every new node through
its stage, exit head with depth-coupled sampling, commit and collapse) for
every live sequence of the workload. The timed region holds exactly --steps
rounds after --warmup untimed rounds, with the prompt already prefilled and
every input resident in HBM. Reported value: committed tokens per second over
the timed rounds.

Extra fields on the JSON line:
  roofline      - the dominant kernel (the stage-batched layer GEMMs): its
                  algorithmic bytes per launch over its mean launch time,
                  against MI355X's 8 TB/s HBM peak; traffic is filled from
                  rocprofv3 counter runs when available (else null). The
                  timed rounds replay captured HIP graphs, inside which event
                  records do not bracket kernels, so the launch time comes
                  from HIP events on the library's stream over the next
                  --steps rounds of the same decode, run eagerly right after
                  the timed region;
  cpu_baseline  - the CPU oracle's DEX decoder timed on this host's cores on a
                  bounded sample (the first few commits of the same prompt);
  dex / ar      - layers per committed token, rows per round, and plain
                  autoregressive decoding on the same kernels for context.
Only one GPU is used: --gpus above 1 is refused.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(w, Wd, prompts, commits, variant="dex", adapter_alpha=None, branch_cap=0):
    """Time the oracle's DEX decoder (oracle/decode.py, as it stands) on the
    first ``commits`` commits of sequence 0, excluding its prefill."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle.decode import dex_decode
    from oracle.model import PlainModel, SlotEvaluator
    from synthetic.noise import gumbel_rows

    t0 = time.time()
    Wc = {"embed": Wd["embed"].cpu(), "final_norm": Wd["final_norm"].cpu(),
          "layers": [{k: v.cpu() for k, v in l.items()} for l in Wd["layers"]]}
    Wc["lm_head"] = Wc["embed"] if w.tied else Wd["lm_head"].cpu()
    ads = None
    if adapter_alpha is not None:
        from synthetic.adapters import generate_adapters
        ads = dict(zip(w.X[:-1], generate_adapters(w, adapter_alpha)))
    model = PlainModel(w, Wc, adapters=ads)
    del Wc
    log(f"[cpu] weights on host in fp64 after {time.time() - t0:.1f}s")
    ev = SlotEvaluator(model)
    t1 = time.time()
    ev.begin(list(prompts[0]))
    t_prefill = time.time() - t1
    log(f"[cpu] oracle prefill of {len(prompts[0]) - 1} positions: {t_prefill:.1f}s")

    class Prefilled:
        """The evaluator with its prefill already done (decode-only timing)."""
        def __init__(self, inner):
            self.inner = inner

        def begin(self, prompt):
            pass

        def __getattr__(self, k):
            return getattr(self.inner, k)

    g = gumbel_rows(w.seed_g, 1, commits + len(w.X), w.vocab)[0].numpy() if w.mode == "sample" else None
    t2 = time.time()
    recs = dex_decode(Prefilled(ev), prompts[0], commits, w.X, mode=w.mode, tau=w.tau, gumbel=g,
                      decs=variant != "vanilla", single_exit=variant == "single_exit",
                      branch_cap=branch_cap if variant == "pruned" else 0)
    t_dec = time.time() - t2
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = blas[0]["num_threads"] if blas else 1
    log(f"[cpu] oracle DEX decode: {len(recs)} commits in {t_dec:.1f}s with {threads} BLAS threads")
    return dict(value=len(recs) / t_dec, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"oracle DEX decode (fp64 NumPy) of the first {len(recs)} committed tokens of "
                       f"sequence 0 after a {len(prompts[0]) - 1}-position prefill (prefill {t_prefill:.1f}s, "
                       f"not counted); decode {t_dec:.1f}s",
                tokens=[r["token"] for r in recs])


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b_x4_greedy")
    ap.add_argument("--cpu-commits", type=int, default=6)
    ap.add_argument("--X", default=None,
                    help="comma-separated exploration set replacing the workload's (e.g. 4,12,20,32: stages "
                         "of unequal length; the exploration-resolution study of Section 4)")
    ap.add_argument("--adapter-alpha", type=float, default=None,
                    help="attach seeded inducing adapters (m = 2 d_model) with this gate at the non-final depths "
                         "(Section 3.4, Appendix C.2); the pages initialise alpha to 1e-3")
    ap.add_argument("--variant", choices=["dex", "single_exit", "vanilla", "pruned"], default="dex",
                    help="dex: full depth exploration with DECS; single_exit: only the first and final "
                         "explorers propose (ablation of Section 4, Figure 4 right-top); vanilla: DECS off "
                         "(Figure 4 right-bottom); pruned: only explorers below --branch-cap spawn "
                         "position children (the sparse lattice of Section 6)")
    ap.add_argument("--branch-cap", type=int, default=2,
                    help="pruned variant: position children only from explorers j < this cap")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ar", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic_gemm_llama7b_x4_greedy.json"),
                    help="counter-derived HBM bytes per GEMM launch (from rocprofv3 --pmc runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device-to-device copy before the timed rounds (a known-size "
                         "reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the DEX lattice step runs every explorer on a single device "
              "(no collectives or sharding); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lossless_depth_adaptive_amd import dex as D
    from synthetic import get_workload
    from synthetic.noise import gumbel_rows
    from synthetic.prompts import batch_prompts
    from synthetic.weights import generate

    torch.cuda.set_device(0)
    w = get_workload(args.workload)
    if args.X:
        w = w.scaled(X=tuple(int(x) for x in args.X.split(",")))
    N = len(w.X)
    T = max(w.gen, args.warmup + 2 * args.steps)
    t0 = time.time()
    Wd = generate(w, device="cuda")
    torch.cuda.synchronize()
    log(f"[gpu] {w.name}: weights generated on device in {time.time() - t0:.1f}s")
    prompts = batch_prompts(w)
    gum = gumbel_rows(w.seed_g, w.batch, T + N, w.vocab).cuda() if w.mode == "sample" else None
    ads = None
    if args.adapter_alpha is not None:
        from synthetic.adapters import adapter_hidden, generate_adapters
        ads = generate_adapters(w, args.adapter_alpha, device="cuda")
    cfg = D.model_config(w.n_layers, w.d_model, w.n_heads, w.n_kv_heads, w.head_dim, w.d_ffn, w.vocab,
                         w.rope_base, w.eps, w.tied, w.dtype, adapter_hidden=adapter_hidden(w) if ads else 0)
    max_ctx = w.prompt_len + T + N + 8
    branch_cap = args.branch_cap if args.variant == "pruned" else 0
    opt = D.options(w.mode, w.tau, args.variant != "vanilla", w.batch, max_ctx, T, gum, False,
                    single_exit=args.variant == "single_exit", branch_cap=branch_cap)
    ctx = D.Dex(cfg, Wd, w.X, opt, adapters=ads)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ctx.prefill(prompts)
    t_prefill = time.perf_counter() - t0
    log(f"[gpu] prefill of {w.batch} x {w.prompt_len} tokens: {t_prefill * 1e3:.1f} ms")
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[gpu] copy calibration: 1 GiB read + 1 GiB written")
    for _ in range(args.warmup):
        ctx.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    commits, rows = [], []
    for _ in range(args.steps):
        commits += ctx.step()
        rows.append(ctx.last_step_rows()[1])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    value = len(commits) / dt
    log(f"[gpu] {args.steps} rounds in {dt * 1e3:.1f} ms: {len(commits)} commits, {value:.1f} tokens/s")
    ctx.profile(True)
    t0 = time.perf_counter()
    n_prof = 0
    for _ in range(args.steps):
        n_prof += len(ctx.step())
    torch.cuda.synchronize()
    dt_prof = time.perf_counter() - t0
    prof = ctx.profile(False)
    ctx.close()
    log(f"[gpu] {args.steps} eager profiled rounds in {dt_prof * 1e3:.1f} ms: {n_prof} commits")

    g = prof["gemm"]
    achieved = g["bytes"] / (g["ms"] * 1e-3) / 1e9 if g["ms"] > 0 else 0.0
    traffic = None
    if os.path.exists(args.traffic):
        tr = json.load(open(args.traffic))
        if tr.get("workload") == w.name and g["launches"]:
            traffic = tr.get("bytes_per_launch")
    per_launch_bytes = g["bytes"] / max(1, g["launches"])
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel="gemm_kernel (stage-batched layer GEMMs)",
                    algorithmic_bytes_per_launch=per_launch_bytes,
                    mean_launch_us=g["ms"] * 1e3 / max(1, g["launches"]), launches=g["launches"])
    classes = {k: dict(ms=round(v["ms"], 3), launches=v["launches"],
                       gb_per_s=round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1) if v["ms"] else None,
                       tflops=round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2) if v["ms"] else None)
               for k, v in prof.items()}
    step_bytes = sum(v["bytes"] for v in prof.values()) / args.steps
    roofline["timing"] = (f"HIP events around each launch over {args.steps} eager rounds that follow the timed "
                          f"rounds ({n_prof / dt_prof:.1f} tokens/s without graph replay)")

    ar = None
    if not args.no_ar:
        ctx = D.Dex(cfg, Wd, w.X, opt, adapters=ads)
        ctx.prefill(prompts)
        k_ar = min(64, T)
        for _ in range(4):
            ctx.ar_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n_ar = 0
        for _ in range(k_ar - 4):
            n_ar += len(ctx.ar_step())
        torch.cuda.synchronize()
        ar = dict(tokens_per_s=round(n_ar / (time.perf_counter() - t0), 2), steps=k_ar - 4)
        ctx.close()
        log(f"[gpu] plain AR on the same kernels: {ar['tokens_per_s']} tokens/s")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, Wd, prompts, args.cpu_commits, args.variant, args.adapter_alpha, branch_cap)

    layers = [c["layers"] for c in commits]
    out = {
        "metric": "committed tokens/sec at 1 GPU; layers/token vs ceil_X(EAD); HBM GB/s % of peak",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded random-init weights and prompts)",
        "config": {"workload": w.name, "layers": w.n_layers, "d_model": w.d_model, "X": list(w.X),
                   "batch": w.batch, "prompt_len": w.prompt_len, "max_new_tokens": T, "mode": w.mode,
                   "variant": args.variant, "adapter_alpha": args.adapter_alpha,
                   "branch_cap": branch_cap or None},
        "roofline": roofline,
        "cpu_baseline": None if cpu is None else {k: v for k, v in cpu.items() if k != "tokens"},
        "dex": {"commits": len(commits), "mean_layers_per_token": round(float(np.mean(layers)), 3) if layers else None,
                "branch_hist": np.bincount([c["branch"] for c in commits], minlength=N).tolist(),
                "mean_rows_per_round": round(float(np.mean(rows)), 2),
                "algorithmic_bytes_per_round": step_bytes, "prefill_ms": round(t_prefill * 1e3, 2),
                "kernel_classes": classes},
        "ar": ar,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
