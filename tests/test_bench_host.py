"""Host-side pieces of bench.py that need no GPU: the counter summary is used
only for its own workload and only with the library build it was counted on."""

import json

import bench
from lossless_depth_adaptive_amd.build import library_digest


def test_counted_traffic_needs_the_same_library(tmp_path):
    lib = tmp_path / "libdex.so"
    lib.write_bytes(b"one build")
    other = tmp_path / "other.so"
    other.write_bytes(b"another build")
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({"workload": "w", "library": library_digest(str(lib)), "bytes_per_launch": 123.0}))
    assert bench.counted_traffic(str(path), "w", str(lib)) == 123.0
    assert bench.counted_traffic(str(path), "w", str(other)) is None   # counted with another build
    assert bench.counted_traffic(str(path), "v", str(lib)) is None     # another workload
    assert bench.counted_traffic(str(tmp_path / "missing.json"), "w", str(lib)) is None


def test_library_digest_is_content_only(tmp_path):
    a, b = tmp_path / "a.so", tmp_path / "b.so"
    a.write_bytes(b"same bytes")
    b.write_bytes(b"same bytes")
    assert library_digest(str(a)) == library_digest(str(b))
    b.write_bytes(b"same bytes!")
    assert library_digest(str(a)) != library_digest(str(b))
