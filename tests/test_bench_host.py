"""Host-side checks of bench.py's bookkeeping (no GPU needed).

The roofline line attaches counter traffic by looking the timed kernel up in
the committed FETCH_SIZE / WRITE_SIZE summary; a kernel whose symbol changed
(a new template argument, a renamed kernel) would silently report no traffic.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mla_latent_kv_08_amd import synth  # noqa: E402

MEASURED = ["dense_b1_h128_t4096", "ragged_b32_h128_t16384", "topk2048_b8_h128_t65536",
            "fp8_b16_h128_t32768"]


@pytest.mark.parametrize("workload", MEASURED)
@pytest.mark.parametrize("kernel", ["absorb", "attention", "combine", "uproj"])
def test_profile_rows_resolve(workload, kernel):
    w = synth.WORKLOADS[workload]
    t = bench.counter_traffic(workload, bench.kernel_symbol(kernel, w), check_sources=False)
    assert t is not None and t > 0, (workload, kernel, bench.kernel_symbol(kernel, w))


def test_attention_symbol_is_unique_per_workload():
    text = open(os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")).read()
    for workload in MEASURED:
        pre = bench.kernel_symbol("attention", synth.WORKLOADS[workload])
        rows = [l for l in text.splitlines() if l.startswith("| %s | `%s" % (workload, pre))]
        assert len(rows) == 1, (workload, rows)
