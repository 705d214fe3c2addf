"""The profile summariser (lossless_depth_adaptive_amd/profsum.py) on small
synthetic rocprofv3 databases: which dispatches count as layer GEMMs, where
the decode window starts, the mean over the event-timed rounds, and the
counter scaling by the 1 GiB copy."""

import json
import sqlite3

import pytest

from lossless_depth_adaptive_amd import profsum

GEMM_QKV = "void dex::gemm_wide_kernel<0, false, 4, 8>(dex::GemmArgs)"
GEMM_DOWN = "void dex::gemm_kernel<unsigned short, 1, 1, 1>(dex::GemmArgs)"
GEMM_RED = "void dex::gemm_split_reduce_kernel<2>(dex::GemmArgs)"
HEAD = "void dex::gemm_wide_kernel<3, false, 2, 4>(dex::GemmArgs)"
ATTN = "void dex::attn_kernel<128>(dex::AttnItem const*)"
SCHED = "dex::sched_kernel(dex::SeqPlan const*)"


def test_gemm_epilogue_names():
    assert profsum.gemm_epilogue(GEMM_QKV) == 0
    assert profsum.gemm_epilogue(GEMM_DOWN) == 1
    assert profsum.gemm_epilogue(GEMM_RED) == 2
    assert profsum.gemm_epilogue(HEAD) == 3
    assert profsum.gemm_epilogue(ATTN) is None
    assert [profsum.is_layer_gemm(k) for k in (GEMM_QKV, GEMM_DOWN, GEMM_RED, HEAD, ATTN)] == \
        [True, True, True, False, False]


def _bench_json(path, launches, bytes_per_launch, us):
    path.write_text(json.dumps({"value": 1.0, "steps": 2, "warmup": 1, "config": {"workload": "w"},
                                "library": {"digest": "abc"},
                                "roofline": {"launches": launches, "algorithmic_bytes_per_launch": bytes_per_launch,
                                             "mean_launch_us": us, "achieved": 0.0, "frac": 0.0}}))


def test_trace_window_and_event_rounds(tmp_path):
    db = tmp_path / "t.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start int, end int, duration int)")
    rows = [(GEMM_QKV, 0, 5000, 5000)]          # prefill: before the first schedule kernel
    t = 10000
    for d in (100, 200, 300, 400):              # four layer GEMMs of the decode window (ns)
        rows += [(SCHED, t, t + 10, 10), (GEMM_QKV, t + 20, t + 20 + d, d), (HEAD, t + 500, t + 600, 100)]
        t += 1000
    con.executemany("insert into kernels values (?, ?, ?, ?)", rows)
    con.commit()
    bench = tmp_path / "b.json"
    _bench_json(bench, 2, 7.0e3, 0.4)           # the last two GEMM dispatches were event-timed
    out = profsum.trace_summary(str(db), str(bench))
    assert "decode window: 12 dispatches" in out
    assert "layer GEMM dispatches" in out and ": 4, mean 0.25 us" in out
    assert "exit-head dispatches: 4" in out
    # the last two: (300 + 400) / 2 ns = 0.35 us; 7e3 bytes / 0.35 us = 20 GB/s
    assert "the 2 layer-GEMM dispatches of the event-timed rounds: mean 0.35 us" in out
    assert "20 GB/s algorithmic" in out


def test_traffic_scales_by_the_copy(tmp_path):
    def counters(name, counter, calib_kib, gemm_kib):
        db = tmp_path / name
        con = sqlite3.connect(db)
        con.execute("create table counters_collection (dispatch_id int, kernel_name text, counter_name text, "
                    "value real)")
        rows = [(1, "void at::native::FillFunctor<float>(float)", counter, 0.0),
                (2, "copy_kernel", counter, calib_kib),
                (3, SCHED, counter, 1.0)]
        rows += [(4 + i, GEMM_QKV, counter, v) for i, v in enumerate(gemm_kib)]
        con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
        con.commit()
        return str(db)
    # the copy reads 1 GiB; FETCH_SIZE reports half of it, WRITE_SIZE all of it
    f = counters("f.db", "FETCH_SIZE", (1 << 20) / 2, [100.0, 200.0, 300.0])
    w = counters("w.db", "WRITE_SIZE", float(1 << 20), [10.0, 20.0, 30.0])
    bench = tmp_path / "b.json"
    _bench_json(bench, 2, 1.0e6, 1.0)
    r = profsum.traffic(f, w, str(bench))
    assert r["fetch_scale"] == pytest.approx(2.0) and r["write_scale"] == pytest.approx(1.0)
    # the last two GEMM dispatches: fetch (200 + 300) / 2 KiB x 2, write (20 + 30) / 2 KiB
    assert r["fetch_bytes_per_launch"] == pytest.approx(500.0 * 1024)
    assert r["write_bytes_per_launch"] == pytest.approx(25.0 * 1024)
    assert r["library"] == "abc" and r["launches"] == 2
