#!/usr/bin/env python3
"""Benchmark of the DEX lattice step on one MI355X.

A step is one dex_step call: one lattice round (expand every new node through
its stage, exit head with depth-coupled sampling, commit and collapse) for
every live sequence of the workload. The default workload is the largest
model that fits one GPU at its batch: the 13B-shaped decoder with eight
exploration depths, 8 sequences with 1024-token Zipf prompts, sampled at
temperature 0.7.

Timing protocol: --runs independent runs (default 3) on one context; each
prefills the prompts, runs --warmup untimed rounds and times exactly --steps
rounds, with every input resident in HBM. Reported value: committed tokens per
second of the median run (each run's rounds are the same rounds of the same
decode, since DEX is deterministic; the spread is in `runs`).

Extra fields on the JSON line:
  roofline      - the dominant kernel class (the stage-batched layer GEMMs):
                  algorithmic bytes per launch over the mean launch time,
                  against MI355X's 8 TB/s HBM peak. Timed rounds replay
                  captured HIP graphs, inside which event records do not
                  bracket kernels, so the launch time comes from HIP events on
                  the library's stream over --steps further rounds of the same
                  decode run eagerly right after the last timed run; traffic
                  comes from rocprofv3 counter runs of this workload
                  (profiles/traffic_gemm_<workload>.json) when present and
                  taken with the library this run loads (same digest; else
                  null);
  e2e           - end-to-end committed tokens per second of one whole
                  generation (prefill included; the pages' throughput
                  definition, Appendix D) next to the decode-only value;
  ead           - mean layers per committed token against the mean depth
                  ceiling of the stable EAD, brute-forced by the oracle on a
                  sample of sequence 0's GPU commits (Definition 1, eqs.
                  (1)-(3); Definition 4, eq. (6)), with the agreement rate and
                  every miss labelled transient or DECS-induced;
  cpu_baseline  - the CPU oracle's DEX decoder (as it stands) timed on this
                  host's cores on a bounded sample (the first commits of
                  sequence 0), its tokens checked against the GPU's;
  dex / ar      - layers per committed token, branch histogram, rows per
                  round, per-class kernel times, and plain autoregressive
                  decoding on the same kernels for context.
Only one GPU is used: --gpus above 1 is refused.
"""

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from lossless_depth_adaptive_amd.build import library_digest  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# Oracle commits timed by default (about 10-30 s of host work on 16 cores).
CPU_COMMITS = {"tiny_f32": 32, "llama7b_x4_greedy": 6, "llama7b_x8_sample": 3, "llama13b_x8_b8": 2,
               "qwen8b_x9_b16": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def counted_traffic(path: str, workload: str, lib_path: str):
    """HBM bytes per layer-GEMM launch from a counter summary
    (profiles/traffic_gemm_<workload>.json), or None when there is none for
    this workload or it was counted with another build of the library."""
    if not os.path.exists(path):
        return None
    tr = json.load(open(path))
    if tr.get("workload") != workload:
        return None
    if tr.get("library") != library_digest(lib_path):
        log(f"[gpu] {path} was measured with another build of the library: traffic left null")
        return None
    return tr.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class _Prefilled:
    """An oracle evaluator whose prefill is already done: begin() is a no-op."""

    def __init__(self, inner):
        self.inner = inner

    def begin(self, prompt):
        pass

    def __getattr__(self, k):
        return getattr(self.inner, k)


def cpu_baseline(w, Wd, prompts, gpu_seq0, commits, gate, variant="dex", adapter_alpha=None, branch_cap=0):
    """Time the oracle's DEX decoder (oracle/decode.py, as it stands) on the
    first ``commits`` commits of sequence 0 after its prefill (not counted);
    check its tokens against the GPU's; then brute-force the stable EAD of the
    GPU's first commits with the oracle's plain decoder forced onto them."""
    import numpy as np
    import psutil
    import torch
    from threadpoolctl import threadpool_info

    from oracle.decode import ar_decode, dex_decode
    from oracle.depth import ceil_x
    from oracle.model import PlainModel, SlotEvaluator
    from synthetic.noise import gumbel_rows

    t0 = time.time()
    Wc = {"embed": Wd["embed"].cpu(), "final_norm": Wd["final_norm"].cpu(),
          "layers": [{k: v.cpu() for k, v in l.items()} for l in Wd["layers"]]}
    Wc["lm_head"] = Wc["embed"] if w.tied else Wd["lm_head"].cpu()
    n_par = sum(t.numel() for l in Wc["layers"] for t in l.values()) + Wc["embed"].numel()
    resident = psutil.virtual_memory().available > 1.5 * 8 * n_par
    ads = None
    if adapter_alpha is not None:
        from synthetic.adapters import generate_adapters
        ads = dict(zip(w.X[:-1], generate_adapters(w, adapter_alpha)))
    model = PlainModel(w, Wc, adapters=ads, resident=resident)
    del Wc
    log(f"[cpu] weights on host after {time.time() - t0:.1f}s ({'fp64 resident' if resident else 'streamed per layer'})")
    ev = SlotEvaluator(model)
    t1 = time.time()
    ev.begin(list(prompts[0]))
    t_prefill = time.time() - t1
    log(f"[cpu] oracle prefill of {len(prompts[0]) - 1} positions: {t_prefill:.1f}s")
    ev_ead = ev.fork()
    g = gumbel_rows(w.seed_g, 1, commits + len(w.X), w.vocab)[0].numpy() if w.mode == "sample" else None
    t2 = time.time()
    recs = dex_decode(_Prefilled(ev), prompts[0], commits, w.X, mode=w.mode, tau=w.tau, gumbel=g,
                      decs=variant != "vanilla", single_exit=variant == "single_exit",
                      branch_cap=branch_cap if variant == "pruned" else 0,
                      on_commit=lambda r: log(f"[cpu] oracle DEX commit at position {r['position']}: token "
                                              f"{r['token']}, branch {r['b']} ({time.time() - t2:.1f}s)"))
    t_dec = time.time() - t2
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = blas[0]["num_threads"] if blas else 1
    log(f"[cpu] oracle DEX decode: {len(recs)} commits in {t_dec:.1f}s with {threads} BLAS threads")
    # the oracle's stream against the GPU's: equal until the first commit whose
    # final-depth margin is below the gate (after that the streams may part)
    agree = 0
    for o, gr in zip(recs, gpu_seq0):
        if o["token"] != gr["token"]:
            if o["margins"][-1] > gate:
                raise RuntimeError(f"CPU oracle and GPU disagree at commit {agree} of sequence 0: "
                                   f"{o['token']} vs {gr['token']} with margin {o['margins'][-1]:.3g}")
            break
        agree += 1
    # stable EAD of the GPU's commits (oracle plain decoding forced onto them)
    n_ead = min(len(gpu_seq0), commits)
    t3 = time.time()
    orc = ar_decode(_Prefilled(ev_ead), prompts[0], n_ead, w.X, mode=w.mode, tau=w.tau, gumbel=g,
                    decs=variant != "vanilla", forced=[r["token"] for r in gpu_seq0[:n_ead]], brute_ead=True,
                    on_commit=lambda r: log(f"[cpu] EAD_stab at position {r['position']}: {r['ead_stab']}"))
    log(f"[cpu] brute-force EAD of {n_ead} GPU commits: {time.time() - t3:.1f}s")
    ead = dict(sample=f"the first {n_ead} commits of sequence 0", commits=n_ead, agree=0, transient=0,
               decs_induced=0, gated=0, layers=[], ceil_ead_stab=[], ead_stab=[])
    for gr, o in zip(gpu_seq0[:n_ead], orc):
        c = ceil_x(o["ead_stab"], w.X)
        ead["layers"].append(gr["layers"])
        ead["ceil_ead_stab"].append(c)
        ead["ead_stab"].append(o["ead_stab"])
        if gr["layers"] == c:
            ead["agree"] += 1
        elif o["cand_by_depth"][gr["layers"] - 1] == gr["token"]:
            ead["transient"] += 1
        else:
            ead["decs_induced"] += 1
        if o["final_margin"] > gate and all(m > gate for m in o["margins"][:o["b"] + 1]):
            ead["gated"] += 1
            if gr["layers"] > c:
                raise RuntimeError(f"GPU layers {gr['layers']} above ceil_X(EAD_stab) {c}")
    ead["mean_layers_per_token"] = float(np.mean(ead["layers"])) if n_ead else None
    ead["mean_ceil_ead_stab"] = float(np.mean(ead["ceil_ead_stab"])) if n_ead else None
    ead["agreement_rate"] = ead["agree"] / n_ead if n_ead else None
    cpu = dict(value=len(recs) / t_dec, unit="tokens/s", cores=int(threads), kind="oracle",
               sample=f"oracle DEX decode ({'fp64 NumPy' if resident else 'fp64 NumPy, layers upcast on use'}) of "
                      f"the first {len(recs)} committed tokens of sequence 0 after a {len(prompts[0]) - 1}-position "
                      f"prefill (prefill {t_prefill:.1f}s, not counted); decode {t_dec:.1f}s; "
                      f"{agree}/{len(recs)} tokens equal to the GPU's; host CPU {cpu_model()}, "
                      f"{len(os.sched_getaffinity(0))} cores in the affinity mask, {threads} BLAS threads, "
                      f"{torch.get_num_threads()} torch threads")
    return cpu, ead


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--runs", type=int, default=3, help="timed runs; the median is reported")
    ap.add_argument("--workload", default="llama13b_x8_b8")
    ap.add_argument("--cpu-commits", type=int, default=None)
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
                         "position children (the sparse lattice of Appendix E, 'Expansion growth and overhead')")
    ap.add_argument("--branch-cap", type=int, default=2,
                    help="pruned variant: position children only from explorers j < this cap")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ar", action="store_true")
    ap.add_argument("--no-e2e", action="store_true")
    ap.add_argument("--traffic", default=None,
                    help="counter-derived HBM bytes per GEMM launch (from rocprofv3 --pmc runs); default "
                         "profiles/traffic_gemm_<workload>.json")
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
    from synthetic.adapters import adapter_hidden
    if args.adapter_alpha is not None:
        from synthetic.adapters import generate_adapters
        ads = generate_adapters(w, args.adapter_alpha, device="cuda")
    cfg = D.model_config(w.n_layers, w.d_model, w.n_heads, w.n_kv_heads, w.head_dim, w.d_ffn, w.vocab,
                         w.rope_base, w.eps, w.tied, w.dtype, adapter_hidden=adapter_hidden(w) if ads else 0)
    branch_cap = args.branch_cap if args.variant == "pruned" else 0

    def make(max_new):
        opt = D.options(w.mode, w.tau, args.variant != "vanilla", w.batch, w.prompt_len + max_new + N + 8, max_new,
                        gum, False, single_exit=args.variant == "single_exit", branch_cap=branch_cap)
        return D.Dex(cfg, Wd, w.X, opt, adapters=ads)

    ctx = make(T)
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[gpu] copy calibration: 1 GiB read + 1 GiB written")
    runs, seq0 = [], []
    for run in range(args.runs):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ctx.prefill(prompts)
        t_prefill = time.perf_counter() - t0
        for _ in range(args.warmup):
            recs = ctx.step()
            if run == 0:
                seq0 += [r for r in recs if r["seq"] == 0]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        commits, rows = [], []
        for _ in range(args.steps):
            recs = ctx.step()
            commits += recs
            rows.append(ctx.last_step_rows()[1])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if run == 0:
            seq0 += [r for r in commits if r["seq"] == 0]
        runs.append(dict(tokens_per_s=len(commits) / dt, seconds=dt, commits=commits, rows=rows,
                         prefill_ms=t_prefill * 1e3))
        log(f"[gpu] run {run}: prefill {t_prefill * 1e3:.1f} ms; {args.steps} rounds in {dt * 1e3:.1f} ms: "
            f"{len(commits)} commits, {len(commits) / dt:.1f} tokens/s")
    med = sorted(runs, key=lambda r: r["tokens_per_s"])[len(runs) // 2]
    value, dt, commits, rows = med["tokens_per_s"], med["seconds"], med["commits"], med["rows"]
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
    tpath = args.traffic or os.path.join(ROOT, "profiles", f"traffic_gemm_{w.name}.json")
    if not args.X and args.variant == "dex" and args.adapter_alpha is None and g["launches"]:
        traffic = counted_traffic(tpath, w.name, D.LIB_PATH)
    per_launch_bytes = g["bytes"] / max(1, g["launches"])
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel="stage-batched layer GEMMs (gemm_wide_kernel, gemm_kernel, gemm_split_reduce_kernel)",
                    algorithmic_bytes_per_launch=per_launch_bytes,
                    mean_launch_us=g["ms"] * 1e3 / max(1, g["launches"]), launches=g["launches"],
                    mfma_frac=round(g["flops"] / (g["ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4) if g["ms"] else None)
    classes = {k: dict(ms=round(v["ms"], 3), launches=v["launches"],
                       gb_per_s=round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1) if v["ms"] else None,
                       tflops=round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2) if v["ms"] else None)
               for k, v in prof.items()}
    if prof["attention"]["ms"] and w.dtype == "f32":
        # an fp32 model's cache holds each K/V value as a bf16 (hi, lo) pair, 4
        # bytes; at 2 bytes per value the K/V stream (all but the per-row query
        # and output vectors, under 1% of it) is half as many bytes
        classes["attention"]["gb_per_s_kv_2_bytes"] = round(classes["attention"]["gb_per_s"] / 2, 1)
    step_bytes = sum(v["bytes"] for v in prof.values()) / args.steps
    roofline["timing"] = (f"HIP events around each launch over {args.steps} eager rounds that follow the timed "
                          f"runs ({n_prof / dt_prof:.1f} tokens/s without graph replay)")

    e2e = None
    if not args.no_e2e:
        ctx = make(w.gen)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ctx.prefill(prompts)
        t_pre = time.perf_counter() - t0
        n_e2e = steps_e2e = 0
        while n_e2e < w.gen * w.batch:
            n_e2e += len(ctx.step())
            steps_e2e += 1
        torch.cuda.synchronize()
        t_all = time.perf_counter() - t0
        ctx.close()
        e2e = dict(tokens_per_s=round(n_e2e / t_all, 2), tokens=n_e2e, seconds=round(t_all, 4),
                   prefill_s=round(t_pre, 4), rounds=steps_e2e,
                   decode_only_tokens_per_s=round(n_e2e / (t_all - t_pre), 2),
                   note=f"one whole generation: {w.batch} x {w.prompt_len}-token prompts prefilled, then "
                        f"{w.gen} tokens per sequence; includes the first rounds, which the timed runs skip")
        log(f"[gpu] end to end: {n_e2e} tokens in {t_all:.3f}s ({e2e['tokens_per_s']} tokens/s)")

    ar = None
    if not args.no_ar:
        ctx = make(T)
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

    cpu = ead = None
    if not args.no_cpu_baseline:
        n_cpu = args.cpu_commits or CPU_COMMITS.get(w.name, 4)
        gate = 1e-3 if w.dtype == "f32" else 5e-2
        torch.cuda.empty_cache()
        cpu, ead = cpu_baseline(w, Wd, prompts, seq0, n_cpu, gate, args.variant, args.adapter_alpha, branch_cap)

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
        "window": {"runs": args.runs, "rounds": [args.warmup + 1, args.warmup + args.steps],
                   "note": "each run prefills, then times rounds warmup+1 .. warmup+steps after the prefill; "
                           "value is the median run",
                   "tokens_per_s": [round(r["tokens_per_s"], 2) for r in runs]},
        "library": {"path": os.path.relpath(D.LIB_PATH, ROOT), "digest": library_digest(D.LIB_PATH)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ead": ead,
        "e2e": e2e,
        "dex": {"commits": len(commits), "mean_layers_per_token": round(float(np.mean(layers)), 3) if layers else None,
                "branch_hist": np.bincount([c["branch"] for c in commits], minlength=N).tolist(),
                "mean_rows_per_round": round(float(np.mean(rows)), 2),
                "algorithmic_bytes_per_round": step_bytes, "prefill_ms": round(med["prefill_ms"], 2),
                "kernel_classes": classes},
        "ar": ar,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
