"""Host-side pieces of bench.py (no GPU): the code hash that ties the recorded
HBM traffic counters to the kernel they were taken on."""
from __future__ import annotations

import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_hash_ignores_comments_but_not_code(tmp_path):
    b = _bench()
    base = "int f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n"
    p = tmp_path / "a.hip"
    p.write_text(base)
    h0 = b.kernel_code_sha256(str(p))
    p.write_text(base.replace("// one", "// another comment").replace("block", "other"))
    assert b.kernel_code_sha256(str(p)) == h0
    p.write_text(base.replace("  return", "\n\n    return"))  # whitespace only
    assert b.kernel_code_sha256(str(p)) == h0
    p.write_text(base.replace("x + 1", "x + 2"))
    assert b.kernel_code_sha256(str(p)) != h0


def test_recorded_traffic_is_consistent():
    rec = json.load(open(os.path.join(ROOT, "profiles", "k_partial32_long_t262144_traffic.txt")))
    assert len(rec["kernel_code_sha256"]) == 64
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    # calibrated = raw KiB x 1024 x (copy bytes / copy counter)
    for raw, fac, cal in (("fetch_kib_raw", "fetch_factor", "fetch_bytes"),
                          ("write_kib_raw", "write_factor", "write_bytes")):
        assert abs(rec[raw] * 1024 * rec[fac] - rec[cal]) <= 1e-3 * rec[cal]
