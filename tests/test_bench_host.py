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


# Algorithmic bytes and GFLOP per step of the fixed-length workloads, as the
# hot-path survey's measurement table derives them from its per-call formulas
# (q, wkv_b once, the rows read, lengths, indices and output; absorb,
# scores, reduction and up-projection), rounded as printed there.
SURVEY_TOTALS = {
    "tiny_b1_h16_t256": (4.50e6, 0.013e9),
    "dense_b1_h128_t4096": (38.36e6, 1.174e9),
    "fp8_b16_h128_t32768": (378.8e6, 146.6e9),
    "topk2048_b8_h128_t65536": (53.15e6, 4.83e9),
}


@pytest.mark.parametrize("workload", sorted(SURVEY_TOTALS))
def test_roofline_arithmetic_matches_survey(workload):
    w = synth.WORKLOADS[workload]
    _, total_bytes, total_flops, _, _ = bench.workload_bytes_flops(w, [w.max_seq_len] * w.batch, w.topk)
    want_bytes, want_flops = SURVEY_TOTALS[workload]
    assert abs(total_bytes / want_bytes - 1) < 2e-3, (total_bytes, want_bytes)
    # the tiny workload's GFLOP is printed with two significant digits
    assert abs(total_flops / want_flops - 1) < (1e-2 if workload.startswith("tiny") else 2e-3), (total_flops, want_flops)


def test_per_kernel_bytes_add_up():
    """The per-launch figures the roofline divides by partition the step's
    counted bytes and FLOPs: the absorb holds W_UK and q_nope, the attention
    the rows, q_pe, lengths and indices, the up-projection W_UV and the
    output; the fused absorb also carries the new rows it stores, which the
    step total leaves out."""
    for name in ["dense_b1_h128_t4096", "fp8_b16_h128_t32768", "topk2048_b8_h128_t65536"]:
        w = synth.WORKLOADS[name]
        out, total_bytes, total_flops, _, row_bytes = bench.workload_bytes_flops(
            w, [w.max_seq_len] * w.batch, w.topk)
        assert out["combine"] == (0, 0)
        assert sum(f for _, f in out.values()) == total_flops, name
        stores = w.batch * 2 * 576 + w.batch * row_bytes + 4 * w.batch if bench.FUSED else 0
        assert sum(b for b, _ in out.values()) - stores == total_bytes, name


def test_extra_workload_specs():
    w, s = bench.extra_workload("dense_b1_h128_t4096", synth, 1)
    assert (w.name, w.heads, s) == ("dense_b1_h128_t4096", 128, 1)
    w, s = bench.extra_workload("ragged_b32_h128_t16384:16:2", synth, 1)
    assert (w.name, w.heads, w.batch, s) == ("ragged_b32_h128_t16384_h16", 16, 32, 2)
    w, s = bench.extra_workload("fp8_b16_h128_t32768:32", synth, 3)
    assert (w.name, w.heads, w.fp8, s) == ("fp8_b16_h128_t32768_h32", 32, True, 3)
    # the default run's packed line has its counter rows in the committed summary
    for kernel in ["absorb", "attention", "combine", "uproj"]:
        w, s = bench.extra_workload(bench.EXTRA[-1], synth, 1)
        assert bench.counter_traffic(f"{w.name}_s{s}", bench.kernel_symbol(kernel, w),
                                     check_sources=False), kernel


def test_more_than_one_gpu_is_refused():
    """The benchmark measures one GPU; asking for more exits with a message
    (before touching torch or a device)."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r
    assert "one GPU" in r.stderr
    assert r.stdout == ""
