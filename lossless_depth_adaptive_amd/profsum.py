"""Summaries of rocprofv3 result databases (rocpd SQLite) for the lattice step.

  python -m lossless_depth_adaptive_amd.profsum trace RESULTS.db [--bench-json B --command C]
      Per-kernel statistics of the decode window (from the first schedule or
      autoregressive-row kernel to the end of the trace): calls, mean and
      total duration, share, plus the mean over every layer-GEMM dispatch;
      with --bench-json, a header naming the workload, the command and what
      the traced bench.py run printed.

  python -m lossless_depth_adaptive_amd.profsum pmc RESULTS.db
      Per-kernel means of every counter of a --pmc run over the decode window.

  python -m lossless_depth_adaptive_amd.profsum traffic --fetch F.db --write W.db \
        --bench-json BENCH.json --out traffic.json
      HBM bytes of the layer GEMMs from the FETCH_SIZE and WRITE_SIZE counter
      runs (KiB per dispatch), each scaled by what the same counter reads for a
      1 GiB device-to-device copy in the same process (bench.py
      --copy-calibration), summed over the layer-GEMM dispatches of the rounds
      bench.py timed with HIP events (the last roofline.launches of the decode
      window; run bench.py with --no-ar) and divided by their count; compared
      with the algorithmic bytes per launch the library reported for the same
      rounds. The summary names the library the counted run loaded (its
      digest, from the bench line); bench.py uses it only with that library.
"""

import argparse
import json
import sqlite3
import sys


GIB = 1 << 30


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "").strip()


def _dispatches(db):
    cur = sqlite3.connect(db).cursor()
    return cur.execute("select name, start, end, duration from kernels order by start").fetchall()


def gemm_epilogue(name: str):
    """Epilogue id of a GEMM dispatch (0 QKV, 1 residual, 2 SwiGLU, 3 exit head,
    4/5 adapters), or None for other kernels. gemm_kernel<T, MB, NB, EPI>,
    gemm_wide_kernel<EPI, SPLIT, WT, NWV>, gemm_split_reduce_kernel<EPI>."""
    k = _short(name)
    if "<" not in k:
        return None
    args = [a.strip() for a in k[k.index("<") + 1:k.rindex(">")].split(",")]
    if k.startswith("dex::gemm_kernel"):
        return int(args[3])
    if k.startswith("dex::gemm_wide_kernel") or k.startswith("dex::gemm_split_reduce_kernel"):
        return int(args[0])
    return None


def is_layer_gemm(name: str) -> bool:
    """A stage-batched layer GEMM dispatch: QKV, O, gate/up or down (exit head
    and adapters excluded)."""
    return gemm_epilogue(name) in (0, 1, 2)


def decode_window(rows):
    for i, r in enumerate(rows):
        if "sched_kernel" in r[0] or "ar_rows_kernel" in r[0]:
            return rows[i:]
    return []


def trace_header(bench_json: str, command: str) -> str:
    """Header lines of a trace summary: the workload, the command that made
    the database, and what the traced bench.py run printed."""
    d = json.loads(open(bench_json).read().strip().splitlines()[-1])
    c, rl = d["config"], d["roofline"]
    out = [f"# Kernel trace: lattice step, workload {c['workload']} ({c.get('layers')} layers, d {c.get('d_model')}, "
           f"X={c.get('X')}, batch {c.get('batch')}, prompts {c.get('prompt_len')}, {c.get('mode')})",
           f"# library {d.get('library', {}).get('digest')}",
           "#",
           "# Commands (repository root, MI355X, ROCm 7.2):",
           "#   export TMPDIR=/tmp",
           f"#   rocprofv3 --kernel-trace --stats -d D -o bench -- {command}",
           "#   python3 -m lossless_depth_adaptive_amd.profsum trace D/bench_results.db --bench-json B.json "
           "--command '...'   (B.json: what the traced command printed)",
           "#",
           f"# Window: {d['warmup']} warmup + {d['steps']} timed rounds (replayed HIP graphs) + {d['steps']} eagerly "
           "profiled rounds, after prefill.",
           f"# bench.py in this traced command: {d['value']} tokens/s; layer-GEMM class by HIP events over the eager "
           f"rounds: {rl['mean_launch_us']:.1f} us per launch, {rl['algorithmic_bytes_per_launch'] / 1e6:.1f} MB "
           f"algorithmic per launch, {rl['achieved']:.0f} GB/s ({rl['frac']:.3f} of 8 TB/s); the events also span "
           "launch gaps."]
    return "\n".join(out) + "\n"


def trace_summary(db: str, bench_json: str = None) -> str:
    rows = [r for r in decode_window(_dispatches(db)) if "dex::" in r[0]]
    if not rows:
        return "no decode-window dispatches found\n"
    stats = {}
    for name, s, e, d in rows:
        stats.setdefault(_short(name), []).append(d)
    total = sum(sum(v) for v in stats.values())
    span = rows[-1][2] - rows[0][1]
    out = [f"decode window: {len(rows)} dispatches, {total / 1e6:.2f} ms in kernels, {span / 1e6:.2f} ms wall",
           f"{'kernel':<52} {'calls':>7} {'mean_us':>10} {'total_ms':>10} {'share':>7}"]
    for k, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{k:<52} {len(v):>7} {sum(v) / len(v) / 1e3:>10.2f} {sum(v) / 1e6:>10.2f} "
                   f"{100.0 * sum(v) / total:>6.1f}%")
    lg = [d for k, v in stats.items() if is_layer_gemm(k) for d in v]
    out.append(f"layer GEMM dispatches (QKV, O, gate/up, down: gemm_kernel, gemm_wide_kernel and "
               f"gemm_split_reduce_kernel): {len(lg)}, mean {sum(lg) / max(1, len(lg)) / 1e3:.2f} us, "
               f"total {sum(lg) / 1e6:.2f} ms")
    hg = [d for k, v in stats.items() if gemm_epilogue(k) == 3 or "head_reduce" in k for d in v]
    out.append(f"exit-head dispatches: {len(hg)}, total {sum(hg) / 1e6:.2f} ms")
    if bench_json:
        # the rounds bench.py timed with HIP events: the last roofline.launches
        # layer-GEMM dispatches of the window
        rl = json.loads(open(bench_json).read().strip().splitlines()[-1])["roofline"]
        n = rl["launches"]
        last = [d for name, _, _, d in rows if is_layer_gemm(name)][-n:]
        if last:
            mean = sum(last) / len(last)
            gbs = rl["algorithmic_bytes_per_launch"] / (mean * 1e-9) / 1e9
            out.append(f"the {len(last)} layer-GEMM dispatches of the event-timed rounds: mean {mean / 1e3:.2f} us "
                       f"(events: {rl['mean_launch_us']:.2f} us), {gbs:.0f} GB/s algorithmic, {gbs / 8000.0:.3f} "
                       "of 8 TB/s")
    return "\n".join(out) + "\n"


def _counters(db, counter):
    cur = sqlite3.connect(db).cursor()
    return cur.execute("select dispatch_id, kernel_name, value from counters_collection where counter_name = ? "
                       "order by dispatch_id", (counter,)).fetchall()


def _calibration(rows):
    """Counter reading of the 1 GiB copy: the dispatch right after the fill."""
    for i, (_, name, _) in enumerate(rows):
        if "FillFunctor<float>" in name and i + 1 < len(rows):
            return rows[i + 1][2]
    raise SystemExit("calibration copy not found (run bench.py with --copy-calibration)")


def _gemm_window(rows):
    start = next(i for i, r in enumerate(rows) if "sched_kernel" in r[1] or "ar_rows_kernel" in r[1])
    return [r for r in rows[start:] if is_layer_gemm(r[1])]


def traffic(fetch_db, write_db, bench_json, workload=None):
    f, w = _counters(fetch_db, "FETCH_SIZE"), _counters(write_db, "WRITE_SIZE")
    f_scale = GIB / (_calibration(f) * 1024.0)
    w_scale = GIB / (_calibration(w) * 1024.0)
    bench = json.loads(open(bench_json).read().strip().splitlines()[-1])
    rl = bench["roofline"]
    n = rl["launches"]
    fg, wg = _gemm_window(f)[-n:], _gemm_window(w)[-n:]
    fetch = sum(v for _, _, v in fg) * 1024.0 * f_scale
    write = sum(v for _, _, v in wg) * 1024.0 * w_scale
    fpl, wpl = fetch / max(1, len(fg)), write / max(1, len(wg))
    return dict(workload=workload or bench["config"]["workload"], launches=n,
                fetch_bytes_per_launch=fpl, write_bytes_per_launch=wpl, bytes_per_launch=fpl + wpl,
                algorithmic_bytes_per_launch=rl["algorithmic_bytes_per_launch"],
                fetch_scale=f_scale, write_scale=w_scale, library=bench.get("library", {}).get("digest"),
                note="layer GEMM launches (exit head excluded) of the HIP-event-timed rounds; counters in KiB "
                     "per dispatch scaled by a 1 GiB copy read/write in the same process")


def pmc_summary(db: str, top: int = 12) -> str:
    """Per-kernel means of every counter in a --pmc database over the decode
    window (the kernels with the most dispatches first)."""
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection "
                       "order by dispatch_id").fetchall()
    start = next((d for d, k, _, _ in rows if "sched_kernel" in k or "ar_rows_kernel" in k), None)
    if start is None:
        return "no decode-window dispatches found\n"
    acc, disp = {}, {}
    for d, k, c, v in rows:
        if d < start or "dex::" not in k:
            continue
        k = _short(k)
        acc.setdefault(k, {}).setdefault(c, 0.0)
        acc[k][c] += v
        disp.setdefault(k, set()).add(d)
    counters = sorted({c for v in acc.values() for c in v})
    out = [f"{'kernel':<44} {'calls':>6} " + " ".join(f"{c[:18]:>18}" for c in counters)]
    for k in sorted(acc, key=lambda k: -len(disp[k]))[:top]:
        n = len(disp[k])
        out.append(f"{k:<44} {n:>6} " + " ".join(f"{acc[k].get(c, 0.0) / n:>18.4g}" for c in counters))
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--bench-json", help="what the traced bench.py command printed (adds a header)")
    t.add_argument("--command", default="python3 bench.py ...", help="the traced command, for the header")
    c = sub.add_parser("pmc")
    c.add_argument("db")
    r = sub.add_parser("traffic")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--bench-json", required=True)
    r.add_argument("--workload")
    r.add_argument("--out")
    a = ap.parse_args(argv)
    if a.cmd == "pmc":
        sys.stdout.write(pmc_summary(a.db))
    elif a.cmd == "trace":
        if a.bench_json:
            sys.stdout.write(trace_header(a.bench_json, a.command))
        sys.stdout.write(trace_summary(a.db, a.bench_json))
    else:
        res = traffic(a.fetch, a.write, a.bench_json, a.workload)
        txt = json.dumps(res, indent=2)
        if a.out:
            open(a.out, "w").write(txt + "\n")
        print(txt)


if __name__ == "__main__":
    main()
