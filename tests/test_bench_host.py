"""Host-side pieces of bench.py (no GPU): the code hash that ties the recorded
HBM traffic counters to the kernel they were taken on, and the parsing of the
power sampler's output and its windows."""
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


SAMPLE_TEXT = """SAMPLE 100.25
GPU: 0
    POWER:
        SOCKET_POWER: 1390 W
    CLOCK:
        GFX_0:
            CLK: 1900 MHz
            MIN_CLK: 500 MHz
        GFX_1:
            CLK: 2000 MHz
        MEM_0:
            CLK: 2000 MHz
SAMPLE 101.50
amd-smi: some error text
SAMPLE 102.75
GPU: 0
    POWER:
        SOCKET_POWER: 1100 W
    CLOCK:
        GFX_0:
            CLK: 2400 MHz
"""


def test_power_samples_and_windows():
    b = _bench()
    s = b.parse_power_samples(SAMPLE_TEXT)
    # the block without a power reading is dropped; MIN_CLK and MEM clocks are not GFX clocks
    assert s == [(100.25, 1390.0, 1950.0), (102.75, 1100.0, 2400.0)]
    w = b.power_window(s, 100.0, 101.0)
    assert w["samples"] == 1 and w["socket_w_median"] == 1390.0 and w["gfx_mhz_mean"] == 1950.0
    assert b.power_window(s, 0.0, 1.0) == {"samples": 0}
    both = b.power_window(s, 100.0, 103.0)
    assert both["samples"] == 2 and both["socket_w_max"] == 1390.0
