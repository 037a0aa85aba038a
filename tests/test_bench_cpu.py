"""bench.py's host-side contract, without a GPU: the one-GPU exit, the
algorithmic work model, the per-kernel roofline arithmetic and the guard that
ties recorded counter data to the kernel sources it was taken from."""
from __future__ import annotations

import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_algorithmic_work_closed_forms():
    d, r, T = 8192, 384, 4096
    w = bench.algorithmic_work(d, d, r, T)
    # the two large contractions of the step: [x | xs] [W0 | B]^T and [gz | ts] [W0 ; A]
    assert w["fused_fwd_gemm"] == ("flop", 2 * T * d * (d + r))
    assert w["dx_gemm"] == ("flop", 2 * T * d * (d + r))
    assert w["fused_fwd_gemm"][1] == 575_525_617_664
    # the rank-r products: one multiply-add per (row, column, k)
    for k in ("down_proj_xs", "t_proj", "dB_gemm", "dA_gemm"):
        assert w[k] == ("flop", 2 * T * d * r), k
    # the compose backward reads gy and y, writes gz, and the per-64-token partials
    kind, nbytes = w["compose_bwd"]
    assert kind == "byte"
    assert nbytes == 3 * T * d * 2 + d * (2 + 4) + (T // 64) * d * 4
    # every entry is a positive amount of a known kind
    assert all(kind in ("flop", "byte") and amount > 0 for kind, amount in w.values())


def test_kernel_table_arithmetic():
    work = bench.algorithmic_work(8192, 8192, 384, 4096)
    # two launches of dx totalling 1 ms over 2 steps: 500 us each
    timing = {"dx_gemm": (2, 1.0), "compose_bwd": (2, 0.07)}
    table = bench.kernel_table(timing, 2, work, {}, peaks={"mfma_bf16_TFs": 2400.0,
                                                          "hbm_stream_GBs": 5600.0})
    dx = table["dx_gemm"]
    assert dx["launches_per_step"] == 1.0 and dx["avg_us"] == 500.0
    tf = work["dx_gemm"][1] / 500e-6 / 1e12
    assert abs(dx["tflops"] - tf) < 0.01
    assert abs(dx["frac_mfma_peak"] - tf / bench.BF16_PEAK_TFS) < 1e-4
    assert abs(dx["frac_measured_mfma"] - tf / 2400.0) < 1e-4
    cb = table["compose_bwd"]
    gbs = work["compose_bwd"][1] / 35e-6 / 1e9
    assert abs(cb["gbps"] - gbs) < 0.1
    assert abs(cb["frac_hbm_peak"] - gbs / bench.HBM_PEAK_GBS) < 1e-4


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    assert bench.kernel_source_hash() == h


def test_code_tokens_drop_comments_only():
    """The source hash sees code, not comments: comments and whitespace runs go,
    string and character literals (even ones holding comment markers) stay."""
    src = "int a = 1; // note\n/* block\n comment */ const char* s = \"x // y /* z */\";\nchar c = '/';"
    assert bench.code_tokens(src) == "int a = 1; const char* s = \"x // y /* z */\"; char c = '/';"
    assert bench.code_tokens("a  +\n\tb") == bench.code_tokens("a + b")
    assert bench.code_tokens("a + b") != bench.code_tokens("a - b")


def test_recorded_traffic_belongs_to_these_sources():
    """Counter data recorded for other sources is never reported: the traffic
    table is either empty or carries bytes for the step's kernels."""
    traffic = bench.recorded_traffic()
    if not traffic:
        return
    assert "dx_gemm" in traffic and "fused_fwd_gemm" in traffic
    # dx reads at least its operands once (W0, A, gz, ts) and writes dx
    d, r, T = 8192, 384, 4096
    floor = (d * d + r * d + T * (d + r) + T * d) * 2
    assert traffic["dx_gemm"]["total_bytes"] >= floor


def test_norm_summary_arithmetic():
    d, r = 8192, 384
    nbytes, flops = bench.norm_work(d, d, r)
    assert nbytes == (d * d + r * d + d * r) * 2 + d * 4
    assert flops == 2 * d * r * d + 2 * r * r * d + 2 * d * r * r
    # two kernels of the chain, 40 us per step in total over 2 steps
    timing = {"gram_AAt": (2, 0.01), "cross_gram_proj": (2, 0.07), "dx_gemm": (2, 1.0)}
    n = bench.norm_summary(timing, 2, d, d, r)
    assert n["us"] == 40.0 and n["launches_per_step"] == 2.0
    assert n["kernels"] == ["cross_gram_proj", "gram_AAt"]
    assert abs(n["gbps"] - nbytes / 40e-6 / 1e9) < 0.1
    bound = max(nbytes / 8e12, flops / 2.5e15) * 1e6
    assert abs(n["bound_us"] - bound) < 0.01 and abs(n["frac_of_bound"] - bound / 40.0) < 1e-4
    assert bench.norm_summary({"dx_gemm": (1, 1.0)}, 1, d, d, r) is None


def test_step_stats_from_one_series():
    per = [1.2, 1.1, 1.3, 1.15]
    st = bench.step_stats(per)
    assert st["n"] == 4 and st["min_us"] == 1100.0 and st["max_us"] == 1300.0
    assert st["min_us"] <= st["mean_us"] <= st["max_us"]


def test_cpu_baseline_protocol_on_a_tiny_layer():
    import synth
    shape = synth.LayerShape(16, 24, 8, 5, 2.0, "bf16")
    layer = synth.make_layer(shape, 3, grad=True)
    cb = bench.cpu_baseline(layer, shape, True, reps=3)
    for k in ("value", "unit", "cores", "kind", "sample", "norm_us", "forward_us", "backward_us",
              "factored_norm_us", "host_cpus", "blas_threads", "cpu_model"):
        assert k in cb, k
    assert cb["kind"] == "oracle" and cb["unit"] == "us"
    assert abs(cb["value"] - (cb["forward_us"] + cb["backward_us"])) < 0.2
    assert cb["cores"] >= 1 and cb["host_cpus"] >= 1
