"""DoRA layer forward + backward on one MI355X: time per step, per-kernel roofline.

One step = dora_forward (factored norm, down-projection, fused base + low-rank
GEMM with the near-unity compose epilogue) + dora_backward (compose backward,
dx, dA, dB, dm) of one bf16 layer with d_out = d_in = 8192, r = 384, s = 2 and
4096 tokens, the headline shape of the Scaling DoRA paper (d_in = 8192,
r = 384, bf16).  Inputs are synthetic (seeded, see synth), resident in HBM
before the timed region; every output and workspace buffer is allocated
before it too.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]
                    [--config NAME] [--cold] [--graph] [--separate-compose] [--no-peaks]

Prints one JSON line.  ``value`` is microseconds per step (lower is better),
from events between consecutive back-to-back steps (``step_spread`` summarises
the same series).  ``roofline`` covers the dominant kernel (largest share of
the step), timed with HIP events on the library's launch stream in a separate
pass; ``kernels`` lists every kernel of the step the same way.  ``norm`` is the
whole factored-norm chain timed as back-to-back dora_norm calls (µs,
algorithmic GB/s against 8 TB/s, fraction of its max(HBM, MFMA) bound;
``norm_kernels`` sums the chain's kernels from the per-kernel pass, whose
events add a few µs to every short kernel); ``compose_fwd`` times the standalone one-pass
compose kernel in the same process (the default path runs the compose as the
forward GEMM's epilogue) and ``compose_bwd`` the backward's.  ``configs``
gives the forward of the other synthetic layers (a tiny float32 layer, the
2048 x 6144 crossover, the 8192 x 8192 headline and the 27648 x 5120 MLP).
``cpu_baseline`` times the float64 oracle (dense W0 + sBA) on the host: norm,
forward and backward separately, each the median of three after a warm-up.
``measured_peaks`` gives the achievable HBM copy rate and sustained MFMA rate
measured in the same process; fractions of them sit beside the fractions of
the published peaks.  ``--config`` times another synthetic layer's forward;
``--cold`` evicts the MALL before every step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DoRA layer fwd+bwd µs & norm/compose GB/s (% HBM peak), d=8192 r=384 bf16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFS = 2500.0         # MI355X dense bf16 MFMA, TFLOP/s
FP32_PEAK_TFS = 157.3          # MI355X fp32 vector / matrix, TFLOP/s (the fp32 layers' GEMMs run on fp32 MFMA)
DEFAULT_CONFIG = "highrank_bwd_bf16"


KERNEL_SOURCES = ["include/dora.h"] + [
    f"parameter_efficient_fine_dora_amd/csrc/{f}"
    for f in ("api.hip", "gemm.hip", "gram.hip", "rowwise.hip", "small.hip", "noalloc.hip",
              "common.h", "kernels.h", "entry.h")]
WORKLOAD_TAG = "highrank_d8192_r384_t4096"


def code_tokens(text: str) -> str:
    """C/C++/HIP source with its comments removed and whitespace runs collapsed
    (string and character literals kept as written), so that an edit to the
    comments alone leaves it unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                           # literal: copy through its closing quote
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """sha256 over the library sources' code (comments and whitespace aside):
    recorded counter data applies only to the code it was taken from."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(rel.encode() + b"\0" + code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic():
    """Per-kernel HBM bytes from the committed PMC summary, if it matches these sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{WORKLOAD_TAG}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return {}
    return rec.get("traffic", {})


def algorithmic_work(d_out, d_in, r, T, e=2):
    """Per-launch algorithmic work of each kernel: ("flop", n) or ("byte", n).

    Flops count 2 per multiply-add of the contraction the method needs; bytes
    count one read of every input and one write of every output (e = element
    bytes of the layer dtype).
    """
    return {
        "gram_AAt": ("flop", 2 * r * r * d_in),
        "cross_gram_proj": ("flop", 2 * d_out * r * d_in + 2 * d_out * r * r),
        "row_norm": ("byte", d_out * d_in * e + d_out * r * e + d_out * r * 4 + d_out * 4),
        "down_proj_xs": ("flop", 2 * T * r * d_in),
        "fused_fwd_gemm": ("flop", 2 * T * d_out * (d_in + r)),
        "base_gemm": ("flop", 2 * T * d_out * d_in),
        "up_proj_lora": ("flop", 2 * T * d_out * r),
        "compose_fwd": ("byte", 3 * T * d_out * e + d_out * (e + 4)),
        "compose_bwd": ("byte", 3 * T * d_out * e + d_out * (e + 4) + ((T + 63) // 64) * d_out * 4),
        "dm_finalize": ("byte", ((T + 63) // 64) * d_out * 4 + d_out * (e + 4)),
        "t_proj": ("flop", 2 * T * d_out * r),
        "dx_gemm": ("flop", 2 * T * d_in * (d_out + r)),
        "dB_gemm": ("flop", 2 * d_out * r * T),
        "dA_gemm": ("flop", 2 * r * d_in * T),
        "gram_finalize": ("byte", r * r * 4 * 2 + r * r * 4),
        # a small float32 layer's forward: one pass over K (x W0^T, x A^T, W0 A^T,
        # A A^T and ||W0_i||^2), then the split sums, the norm and the compose
        "small_partials": ("flop", 2 * T * d_out * d_in + 2 * T * r * d_in + 2 * d_out * r * d_in
                           + 2 * r * r * d_in + 2 * d_out * d_in),
        "small_finish": ("flop", 2 * T * d_out * r + 2 * d_out * r * r + 4 * d_out * r),
    }


def kernel_table(timing, steps, work, traffic, peaks=None, flop_peak=None):
    peaks = peaks or {}
    flop_peak = flop_peak or BF16_PEAK_TFS
    out = {}
    for name, (count, total_ms) in sorted(timing.items(), key=lambda kv: -kv[1][1]):
        per = count / steps if steps else 0
        avg_us = 1e3 * total_ms / count
        row = {"launches_per_step": per, "avg_us": round(avg_us, 3),
               "share": None}
        if name in work:
            kind, amount = work[name]
            if kind == "flop":
                tf = amount / (avg_us * 1e-6) / 1e12
                row.update(tflops=round(tf, 2), frac_mfma_peak=round(tf / flop_peak, 4))
                if peaks.get("mfma_bf16_TFs") and flop_peak == BF16_PEAK_TFS:
                    row["frac_measured_mfma"] = round(tf / peaks["mfma_bf16_TFs"], 4)
            else:
                gbs = amount / (avg_us * 1e-6) / 1e9
                row.update(gbps=round(gbs, 1), frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
                if peaks.get("hbm_stream_GBs"):
                    row["frac_measured_hbm"] = round(gbs / peaks["hbm_stream_GBs"], 4)
        if name in traffic:
            row["hbm_traffic_bytes"] = traffic[name]["total_bytes"]
        out[name] = row
    tot = sum(v[1] for v in timing.values())
    for name, row in out.items():
        row["share"] = round(timing[name][1] / tot, 4) if tot else None
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads") or 1) for i in threadpool_info()
                   if i.get("user_api") == "blas")
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def cpu_baseline(layer_np, shape, backward=True, reps=3):
    """The float64 oracle, as it stands, on the host cores: its dense norm, forward
    and (detached) backward of the same layer, each the median of ``reps`` runs
    after one warm-up (input decoding excluded).  A float64 factored norm (the
    oracle's base + cross + Gram terms, the GPU path's algorithm) is timed too."""
    import numpy as np
    import oracle
    import synth
    L = synth.layer_f64(layer_np, shape.dtype)

    def med(fn):
        fn()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)) * 1e6

    def factored():
        base, cross, gram = oracle.norm_terms(L["W0"], L["A"], L["B"], shape.s)
        return np.sqrt(np.maximum(base + cross + gram, 0.0))

    t_norm = med(lambda: oracle.dora_norm(L["W0"], L["A"], L["B"], shape.s))
    t_fact = med(factored)
    t_fwd = med(lambda: oracle.dora_forward(L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s))
    t_bwd = med(lambda: oracle.dora_backward(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"],
                                             shape.s)) if backward else 0.0
    what = "forward + detached backward" if backward else "forward"
    return {"value": round(t_fwd + t_bwd, 1), "unit": "us", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"one full step ({what}) of the same d_out={shape.d_out} d_in={shape.d_in} "
                      f"r={shape.r} T={shape.tokens} layer in float64 (dense W0 + sBA), inputs "
                      f"decoded from the same {shape.dtype} bits; each part the median of "
                      f"{reps} runs after one warm-up",
            "norm_us": round(t_norm, 1), "forward_us": round(t_fwd, 1),
            "backward_us": round(t_bwd, 1), "factored_norm_us": round(t_fact, 1),
            "host_cpus": os.cpu_count(), "blas_threads": _blas_threads(),
            "cpu_model": _cpu_model()}


def measure_peaks(torch, ops, dev):
    """The HBM rate of a 1 GiB device-to-device copy and the sustained MFMA rate of
    the library's register-only probe, each the best of a few launches."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(6):
        ev0.record()
        dst.copy_(src)
        ev1.record()
        torch.cuda.synchronize()
        best = min(best, ev0.elapsed_time(ev1) * 1e-3)
    hbm = 2.0 * src.numel() / best / 1e9
    del src, dst
    n = (512 << 20) // 4
    a, b, c = (torch.empty(n, dtype=torch.float32, device=dev) for _ in range(3))
    best = float("inf")
    for _ in range(6):
        ev0.record()
        ops.probe_stream(a, b, c)
        ev1.record()
        torch.cuda.synchronize()
        best = min(best, ev0.elapsed_time(ev1) * 1e-3)
    stream = 3.0 * n * 4 / best / 1e9
    del a, b, c
    blocks, iters = 4096, 4096
    out, flops = ops.probe_mfma(iters, blocks)
    best = float("inf")
    for _ in range(4):
        ev0.record()
        ops.probe_mfma(iters, blocks, out=out)
        ev1.record()
        torch.cuda.synchronize()
        best = min(best, ev0.elapsed_time(ev1) * 1e-3)
    return {"hbm_copy_GBs": round(hbm, 1), "hbm_stream_GBs": round(stream, 1),
            "mfma_bf16_TFs": round(flops / best / 1e12, 1),
            "how": "1 GiB device-to-device copy (read + write); the library's c = a + b probe "
                   "over 512 MiB per stream (2 reads + 1 write); register-only "
                   "v_mfma_f32_32x32x16_bf16 chains, 4096 workgroups of 4 waves"}


# Kernels of the factored norm (dora_norm's chain inside dora_forward).
NORM_LABELS = ("gram_AAt", "gram_finalize", "cross_gram_proj", "row_norm")
# Forward-only workloads reported beside the headline step (synth.CONFIGS names).
FORWARD_CONFIGS = ("tiny_f32", "crossover_bf16", "highrank_bf16", "widemlp_bf16")


def norm_work(d_out, d_in, r, e=2):
    """Algorithmic work of the whole factored norm: bytes = W0, A, B read once and
    the norms written; flops = U = W0 A^T, G = A A^T and B G (2 per multiply-add)."""
    nbytes = (d_out * d_in + r * d_in + d_out * r) * e + d_out * 4
    flops = 2 * d_out * r * d_in + 2 * r * r * d_in + 2 * d_out * r * r
    return nbytes, flops


def norm_summary(timing, steps, d_out, d_in, r, e=2):
    """The norm chain per step: µs, algorithmic GB/s against 8 TB/s, and the
    fraction of its max(HBM, MFMA) bound."""
    parts = {k: timing[k] for k in NORM_LABELS if k in timing}
    if not parts or not steps:
        return None
    us = sum(tot for _, tot in parts.values()) / steps * 1e3
    nbytes, flops = norm_work(d_out, d_in, r, e)
    bound_us = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFS * 1e12)) * 1e6
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "launches_per_step": round(sum(c for c, _ in parts.values()) / steps, 2),
            "kernels": sorted(parts), "bytes": nbytes, "gbps": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "flops": flops,
            "bound_us": round(bound_us, 2), "frac_of_bound": round(bound_us / us, 4),
            "bound": "max(bytes at 8 TB/s, flops at 2.5 PFLOP/s)"}


def norm_call_summary(ms, per_ms, d_out, d_in, r, e=2):
    """dora_norm timed as one call (events between back-to-back calls): the norm
    chain without the per-kernel events of the kernel table."""
    nbytes, flops = norm_work(d_out, d_in, r, e)
    us = ms * 1e3
    bound_us = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFS * 1e12)) * 1e6
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "per_call": step_stats(per_ms), "gbps": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bound_us": round(bound_us, 2),
            "frac_of_bound": round(bound_us / us, 4)}


def step_stats(per_ms):
    import numpy as np
    return {"median_us": round(float(np.median(per_ms)) * 1e3, 2),
            "mean_us": round(float(np.mean(per_ms)) * 1e3, 2),
            "min_us": round(float(np.min(per_ms)) * 1e3, 2),
            "max_us": round(float(np.max(per_ms)) * 1e3, 2), "n": len(per_ms)}


def timed_series(torch, run, steps):
    """K back-to-back steps with an event between consecutive steps: the total
    (first to last event) and every step's own duration come from one series."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    host = [0.0] * (steps + 1)
    torch.cuda.synchronize()
    host[0] = time.perf_counter()
    evs[0].record()
    for k in range(steps):
        run()
        evs[k + 1].record()
        host[k + 1] = time.perf_counter()
    torch.cuda.synchronize()
    per = [evs[k].elapsed_time(evs[k + 1]) for k in range(steps)]
    timed_series.host_ms = [(host[k + 1] - host[k]) * 1e3 for k in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / steps, per


def _upload(torch, np, a, is_bf, dev):
    a = np.ascontiguousarray(a)
    if is_bf:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def forward_config(torch, np, ops, synth, name, dev, steps, warmup, tensors=None):
    """Forward (factored norm + fused compose) of one synthetic layer: µs per
    forward from events between consecutive back-to-back forwards, and the
    per-kernel table of a separate pass."""
    shape = synth.CONFIGS[name]
    is_bf = shape.dtype == "bf16"
    tdt = torch.bfloat16 if is_bf else torch.float32
    e = 2 if is_bf else 4
    d_out, d_in, r, T, s = shape.d_out, shape.d_in, shape.r, shape.tokens, shape.s
    if tensors is None:
        layer = synth.make_layer(shape, synth.CONFIG_SEED[name])
        tensors = {k: _upload(torch, np, v, is_bf, dev) for k, v in layer.items()}
    d = tensors
    y = torch.empty(T, d_out, dtype=tdt, device=dev)
    norm = torch.empty(d_out, dtype=torch.float32, device=dev)
    xs = torch.empty(T, r, dtype=tdt, device=dev)
    ws = torch.empty(max(1, ops.workspace_bytes(d_out, d_in, r, T, tdt, 1)), dtype=torch.uint8,
                     device=dev)

    def fwd():
        ops.dora_forward(d["x"], d["W0"], d["A"], d["B"], d["m"], s, y=y, norm_out=norm,
                         xs_out=xs, workspace=ws)

    for _ in range(warmup):
        fwd()
    ms, per = timed_series(torch, fwd, steps)
    # the factored norm alone, as one call (no per-kernel events between its launches)
    ws_n = torch.empty(max(1, ops.workspace_bytes(d_out, d_in, r, T, tdt, 0)), dtype=torch.uint8,
                       device=dev)

    def nrm():
        ops.dora_norm(d["W0"], d["A"], d["B"], s, out=norm, workspace=ws_n)

    for _ in range(warmup):
        nrm()
    norm_ms, norm_per = timed_series(torch, nrm, steps)
    ops.timing_enable(True)
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    ops.timing_enable(False)
    timing = ops.timing_collect()
    work = algorithmic_work(d_out, d_in, r, T, e)
    flop_peak = BF16_PEAK_TFS if is_bf else FP32_PEAK_TFS
    fwd_flops = 2 * T * d_out * (d_in + r) + 2 * T * r * d_in
    nb, nf = norm_work(d_out, d_in, r, e)
    return {"d_out": d_out, "d_in": d_in, "r": r, "tokens": T, "dtype": shape.dtype,
            "fwd_us": round(ms * 1e3, 2), "per_forward": step_stats(per),
            "launches_per_forward": round(sum(c for c, _ in timing.values()) / steps, 2),
            "algorithmic_flops": fwd_flops + nf,
            "tflops": round((fwd_flops + nf) / (ms * 1e-3) / 1e12, 2),
            "norm": norm_summary(timing, steps, d_out, d_in, r, e),
            "norm_call": norm_call_summary(norm_ms, norm_per, d_out, d_in, r, e),
            "kernels": kernel_table(timing, steps, work, {}, None, flop_peak)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the forward-only timings of the other synthetic layers")
    ap.add_argument("--separate-compose", action="store_true",
                    help="run the standalone compose kernels instead of the GEMM-fused ones")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--config", default=DEFAULT_CONFIG,
                    help="synthetic layer (synth.CONFIGS); the backward runs only for the "
                         "backward config, the others time the forward (norm + compose)")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB buffer between steps (evicts the 256 MB MALL) and "
                         "time each step alone")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the achievable HBM and MFMA rates")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step as a HIP graph and time its replays")
    ap.add_argument("--serial", action="store_true",
                    help="keep every kernel on one stream (the library's timing hook on for "
                         "all steps), so that profiles see one launch order")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the DoRA layer's "
              "multi-GPU sharding is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from parameter_efficient_fine_dora_amd import ops

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    if args.config not in synth.CONFIGS:
        print(f"unknown --config {args.config}; one of {sorted(synth.CONFIGS)}", file=sys.stderr)
        sys.exit(2)
    shape = synth.CONFIGS[args.config]
    backward = args.config == DEFAULT_CONFIG
    d_out, d_in, r, T, s = shape.d_out, shape.d_in, shape.r, shape.tokens, shape.s
    is_bf = shape.dtype == "bf16"
    tdt = torch.bfloat16 if is_bf else torch.float32
    e = 2 if is_bf else 4
    flags = ops.FLAG_SEPARATE_COMPOSE if args.separate_compose else 0
    print(f"# generating inputs {args.config}: d_out={d_out} d_in={d_in} r={r} T={T}",
          file=sys.stderr, flush=True)
    layer = synth.make_layer(shape, synth.CONFIG_SEED[shape.name], grad=backward)
    d = {k: _upload(torch, np, v, is_bf, dev) for k, v in layer.items()}
    y = torch.empty(T, d_out, dtype=tdt, device=dev)
    norm = torch.empty(d_out, dtype=torch.float32, device=dev)
    xs = torch.empty(T, r, dtype=tdt, device=dev)
    gx = torch.empty(T, d_in, dtype=tdt, device=dev)
    gA = torch.empty(r, d_in, dtype=tdt, device=dev)
    gB = torch.empty(d_out, r, dtype=tdt, device=dev)
    gm = torch.empty(d_out, dtype=torch.float32, device=dev)
    ws_f = torch.empty(max(1, ops.workspace_bytes(d_out, d_in, r, T, tdt, 1, flags)),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, ops.workspace_bytes(d_out, d_in, r, T, tdt, 2, flags)),
                       dtype=torch.uint8, device=dev) if backward else None

    def step():
        ops.dora_forward(d["x"], d["W0"], d["A"], d["B"], d["m"], s, y=y, norm_out=norm,
                         xs_out=xs, workspace=ws_f, flags=flags)
        if backward:
            ops.dora_backward(d["gy"], d["x"], d["W0"], d["A"], d["B"], d["m"], norm, xs, y, s,
                              grad_x=gx, grad_A=gA, grad_B=gB, grad_m=gm, workspace=ws_b,
                              flags=flags)

    evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.serial:
        ops.timing_enable(True)
    print("# warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.serial:
        ops.timing_collect()   # drop the warm-up records

    run = step
    if args.graph:
        # capture one step (the library's side stream joins the capture through
        # its fork/join events); every buffer is already allocated
        print("# capturing one step as a graph", file=sys.stderr, flush=True)
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step()
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        run = graph.replay
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
    print(f"# timing {args.steps} steps{' (cold)' if args.cold else ''}"
          f"{' (graph replays)' if args.graph else ''}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.cold:
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        per = []
        for _ in range(args.steps):
            evict.fill_(1)
            ev0.record()
            run()
            ev1.record()
            torch.cuda.synchronize()
            per.append(ev0.elapsed_time(ev1))
        ms_per_step = float(np.median(per))
    else:
        ms_per_step, per = timed_series(torch, run, args.steps)
    wall = time.perf_counter() - t0
    spread = step_stats(per)
    spread["first_steps_us"] = [round(v * 1e3, 1) for v in per[:5]]
    if not args.cold:
        # host time to enqueue each step (the library's launches and events); a
        # step whose enqueue takes longer than the GPU's work leaves the GPU waiting
        hms = timed_series.host_ms
        spread["host_enqueue_us"] = {"median": round(float(np.median(hms)) * 1e3, 1),
                                     "first_steps": [round(v * 1e3, 1) for v in hms[:5]]}

    # per-kernel times: the same steps again, each launch bracketed by HIP events
    print("# per-kernel timing", file=sys.stderr, flush=True)
    ops.timing_enable(True)
    for _ in range(args.steps):
        if args.cold:
            evict.fill_(1)
        step()
    torch.cuda.synchronize()
    ops.timing_enable(False)
    timing = ops.timing_collect()
    if args.serial:   # the timed steps' records, then the per-kernel pass's (same kernels)
        timing = {k: (v[0] / 2, v[1] / 2) for k, v in timing.items()}

    # the standalone one-pass compose (the default path folds it into the forward
    # GEMM's epilogue): a few separate-compose forwards in the same process
    compose_fwd = None
    if not args.cold:
        sep = ops.FLAG_SEPARATE_COMPOSE
        ws_sep = torch.empty(max(1, ops.workspace_bytes(d_out, d_in, r, T, tdt, 1, sep)),
                             dtype=torch.uint8, device=dev)
        y_sep = torch.empty_like(y)
        for _ in range(3):
            ops.dora_forward(d["x"], d["W0"], d["A"], d["B"], d["m"], s, y=y_sep, norm_out=norm,
                             xs_out=xs, workspace=ws_sep, flags=sep)
        torch.cuda.synchronize()
        ops.timing_enable(True)
        n_sep = max(5, min(args.steps, 20))
        for _ in range(n_sep):
            ops.dora_forward(d["x"], d["W0"], d["A"], d["B"], d["m"], s, y=y_sep, norm_out=norm,
                             xs_out=xs, workspace=ws_sep, flags=sep)
        torch.cuda.synchronize()
        ops.timing_enable(False)
        tsep = ops.timing_collect()
        del ws_sep, y_sep
        if "compose_fwd" in tsep:
            cnt, tot = tsep["compose_fwd"]
            us = tot / cnt * 1e3
            nbytes = algorithmic_work(d_out, d_in, r, T, e)["compose_fwd"][1]
            gbs = nbytes / (us * 1e-6) / 1e9
            compose_fwd = {
                "avg_us": round(us, 3), "bytes": nbytes, "gbps": round(gbs, 1),
                "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "how": "the standalone one-pass compose kernel (DORA_FLAG_SEPARATE_COMPOSE: "
                       "read base and s*lora, write y), timed in the same process; the "
                       "default path applies the same formula in the forward GEMM's "
                       "epilogue, which adds only the m and n reads "
                       f"({d_out * (e + 4)} bytes) to that GEMM"}

    peaks = None
    if not args.no_peaks:
        print("# achievable peaks (copy, MFMA probe)", file=sys.stderr, flush=True)
        peaks = measure_peaks(torch, ops, dev)
    flop_peak = BF16_PEAK_TFS if is_bf else FP32_PEAK_TFS
    work = algorithmic_work(d_out, d_in, r, T, e)
    headline = args.config == DEFAULT_CONFIG and not flags and not args.cold
    traffic = recorded_traffic() if headline else {}
    kernels = kernel_table(timing, args.steps, work, traffic, peaks, flop_peak)
    if peaks and compose_fwd:
        compose_fwd["frac_measured_hbm"] = round(compose_fwd["gbps"] / peaks["hbm_stream_GBs"], 4)
    # the dominant kernel among those with a work model (split-K reductions have none)
    dominant = max((k for k in timing if k in work), key=lambda k: timing[k][1], default=None)
    kind, amount = work[dominant] if dominant else (None, 0)
    avg_s = timing[dominant][1] / timing[dominant][0] * 1e-3 if dominant else 0.0
    if dominant is None:
        roof = None
    elif kind == "flop":
        achieved = amount / avg_s / 1e12
        # every GEMM runs on the matrix cores (bf16, or fp32 MFMA for float32 layers);
        # the two-kernel small float32 forward runs on the vector ALUs
        on_alu = dominant.startswith("small_")
        roof = {"bound": "alu" if on_alu else "mfma", "achieved": round(achieved, 2),
                "peak": flop_peak,
                "unit": "TFLOP/s", "frac": round(achieved / flop_peak, 4),
                "traffic": traffic.get(dominant, {}).get("total_bytes"),
                "kernel": dominant, "per_launch": f"{amount / 1e9:.3g} GFLOP",
                "avg_us": round(avg_s * 1e6, 2)}
        if peaks and is_bf:
            roof["frac_of_measured"] = round(achieved / peaks["mfma_bf16_TFs"], 4)
    else:
        achieved = amount / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic.get(dominant, {}).get("total_bytes"),
                "kernel": dominant, "per_launch": f"{amount / 1e6:.1f} MB",
                "avg_us": round(avg_s * 1e6, 2)}
        if peaks:
            roof["frac_of_measured"] = round(achieved / peaks["hbm_stream_GBs"], 4)

    norm_call = None
    if not args.cold and not args.graph:
        ws_n = torch.empty(max(1, ops.workspace_bytes(d_out, d_in, r, T, tdt, 0)),
                           dtype=torch.uint8, device=dev)
        nrm_out = torch.empty(d_out, dtype=torch.float32, device=dev)

        def nrm():
            ops.dora_norm(d["W0"], d["A"], d["B"], s, out=nrm_out, workspace=ws_n)

        for _ in range(max(3, args.warmup)):
            nrm()
        n_ms, n_per = timed_series(torch, nrm, max(10, args.steps))
        norm_call = norm_call_summary(n_ms, n_per, d_out, d_in, r, e)
        del ws_n

    configs = None
    if backward and not args.no_configs and not args.cold and not args.graph and not flags:
        configs = {}
        for name in FORWARD_CONFIGS:
            print(f"# forward of {name}", file=sys.stderr, flush=True)
            reuse = None
            if name == "highrank_bf16":   # the step's own layer: same shape and distributions
                reuse = {k: d[k] for k in ("x", "W0", "A", "B", "m")}
            configs[name] = forward_config(torch, np, ops, synth, name, dev,
                                           max(10, min(args.steps, 50)), max(3, args.warmup),
                                           reuse)
            if reuse is not None:
                configs[name]["inputs"] = "the backward layer's (same shape and distributions)"
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (float64 oracle: norm, forward, backward)", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(layer, shape, backward)

    if args.config == DEFAULT_CONFIG:
        metric = METRIC
        workload = "DoRA linear fwd (factored norm + fused compose) + bwd"
    else:
        metric = f"DoRA layer fwd µs, d_out={d_out} d_in={d_in} r={r} T={T} {shape.dtype}"
        workload = "DoRA linear fwd (factored norm + fused compose)"
    rec = {
        "metric": metric, "value": round(ms_per_step * 1e3, 2), "unit": "us",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "step_spread": spread,
        "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": shape.dtype, "data": "synthetic",
        "config": {"workload": f"{workload}, {shape.dtype}", "name": args.config,
                   "d_out": d_out, "d_in": d_in, "r": r, "tokens": T, "s": s,
                   "compose": "separate" if flags else "gemm-fused",
                   "cache": "cold (MALL evicted before each step)" if args.cold else "warm",
                   "launch": "HIP graph replay" if args.graph else "eager",
                   "parallelism": "dp1"},
        "roofline": roof,
        "norm": norm_call,
        "norm_kernels": norm_summary(timing, args.steps, d_out, d_in, r, e),
        "compose_fwd": compose_fwd,
        "compose_bwd": kernels.get("compose_bwd"),
        "cpu_baseline": cpu,
        "measured_peaks": peaks,
        "kernels": kernels,
        "configs": configs,
        "kernel_source_hash": kernel_source_hash(),
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
