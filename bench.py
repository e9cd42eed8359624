"""Benchmark of the fused shifted-window attention on one MI355X.

One step = one wattn_forward call over one batch of the workload (gather + shift + RoPE +
bias channels + QK^T + mask + online softmax + PV + normalise + scatter, all in one kernel
launch).  Inputs are resident in HBM before timing starts; several input sets are used in
rotation so that consecutive steps do not find their inputs in the last-level cache.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--out-dtype fp32|bf16] [--pass fwd|bwd|gated]

Prints one JSON line.  The default workload is the dense patch-2 grid at M = 32
(16 images x 128 x 128 tokens, 3 heads x 32, shift 16), the configuration the headline
metric is quoted on.  With --pass bwd a step is one wattn_backward call (dq, dk, dv and
dtheta of the same workload, given the forward pass's output, its row log-sum-exp and an
output gradient, all resident), timed the same way.  With --pass gated a step is the gated
local path of hybrid linear/softmax attention on the dense grid with 8 x 8 (or 16 x 16)
blocks: one wattn_gated_local call (the ~30% of blocks whose gate exceeds tau get
out += O_local - O_lin-local, in place); the list form (wattn_select_blocks followed by
wattn_local_residual) is timed beside it.  With --pass stack a step runs six window-attention
layers over the SR-style grid (8 x 192 x 192 tokens, 6 heads x 32) whose windows cycle 16, 32,
64 (shifted on every second layer), each with a rank-16 bias and the convolutional gate: per
layer wattn_cla_logits on the layer input, then wattn_forward_gated.  With --pass model a step
is the FlashSwin-T forward pass of a batch of 256 px images (overlapping stem, 2-2-6-2 blocks,
patch merging, head), every step in the library's kernels.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "window-attn tokens/s + TFLOP/s (% bf16 MFMA peak), M=32 p=2 grid"
METRIC_BWD = "window-attn backward tokens/s + TFLOP/s (% bf16 MFMA peak), M=32 p=2 grid"
METRIC_STACK = "window-attn stack tokens/s (cyclic windows 16/32/64, rank-16 bias, convolutional gate), SR grid"
METRIC_MODEL = "FlashSwin-T forward img/s (stem, 12 blocks, merging, head)"
METRIC_GATED = "gated local path tokens/s (routing + local softmax residual), % of HBM peak, p=2 grid"
WARMUP_MIN_S = 0.5          # untimed back-to-back launches before timing (clock ramp)
WARMUP_MAX_STEPS = 20000
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CSRC = os.path.join(ROOT, "vision_transformer_windowed_window_amd", "csrc")
# the sources each profiled kernel is compiled from (their hash tags the traffic records)
KERNEL_SRCS = {
    "attention": [os.path.join(CSRC, f) for f in ("wattn_kernels.hip", "wattn_device.h", "wattn_plan.h")],
    "gated": [os.path.join(CSRC, f) for f in ("wattn_gated.hip", "wattn_device.h", "wattn_aux_plan.h")],
}
PIPE_RATES = os.path.join(ROOT, "vision_transformer_windowed_window_amd", "pipe_rates")
MFMA_FLOPS = 16 * 16 * 32 * 2  # one v_mfma_f32_16x16x32_bf16 / _f16
COPY_BYTES = 256 << 20      # the calibration copy of --pass copy


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dense_p2_m32")
    ap.add_argument("--out-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--input-sets", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="time only the named workload (by default the forward pass also times the other "
                         "bf16 workloads for a few seconds each, reported under 'configs')")
    ap.add_argument("--sweep-steps", type=int, default=30, help="timed steps of each swept workload")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd", "gated", "stack", "model", "copy"],
                    help="fwd: wattn_forward (the headline); bwd: wattn_backward; gated: the gated local path; "
                         "stack: six layers with cyclic windows and the convolutional gate; "
                         "model: the FlashSwin-T forward pass (--workload flashswin_t_p4_m32 or _p2_m32); "
                         "copy: a plain 256 MiB device copy, the scale for the HBM byte counters")
    return ap.parse_args()


def kernel_sha(which: str = "attention") -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS[which]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, out_dtype: str, which: str = "attention"):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they were taken on
    the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{out_dtype}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != kernel_sha(which):
        return None
    return rec.get("hbm_bytes_per_launch")


def pipe_bound(exps: float, mfma_flops: float, kernel_s: float):
    """Least time the workload's exponentials and matrix products take on this GPU.

    Runs the pipe_rates program (built with the library) as a child process; it times the
    v_exp_f32 and 16x16x32 MFMA rates per SIMD.  Every executed (query, key) pair costs one
    exponential; the products cost mfma_flops.  Returns None if the program is missing or fails.
    """
    import subprocess

    if not os.path.exists(PIPE_RATES):
        return None
    try:
        res = subprocess.run([PIPE_RATES], capture_output=True, text=True, timeout=120)
        rates = json.loads(res.stdout.strip().splitlines()[-1]) if res.returncode == 0 else None
    except Exception:
        rates = None
    if not rates:
        return None
    ns = rates["ns_per_instruction"]
    simds = rates["simds"]
    t_exp = exps / 64.0 * ns["exp_f32"] / simds * 1e-3          # us, 64 lanes per instruction
    t_mfma = mfma_flops / MFMA_FLOPS * ns["mfma_f32_16x16x32_bf16"] / simds * 1e-3
    # the attention kernel's steady state: one 32 x 32 step per 1024 executed pairs, on every SIMD
    step_ns = rates.get("softmax_step_ns")
    t_steps = exps / 1024.0 / simds * step_ns * 1e-3 if step_ns else None
    return {
        "source": "vision_transformer_windowed_window_amd/pipe_rates",
        "ns_per_instruction": ns,
        "exp_us": t_exp,
        "mfma_us": t_mfma,
        "kernel_us": kernel_s * 1e6,
        "kernel_vs_exp_plus_mfma": (t_exp + t_mfma) / (kernel_s * 1e6),
        "mfma_fma_split_vs_serial": rates["split_mfma_fma_ns_per_iteration"] / rates["serial_mfma_fma_ns_per_iteration"],
        "mfma_exp_interleaved_vs_serial": rates["interleaved_4mfma_16exp_ns"] / rates["serial_4mfma_16exp_ns"],
        "exp_fma_same_wave_vs_serial": (rates["expfma_same_wave_ns_per_iteration"] / rates["serial_exp_fma_ns_per_iteration"]
                                        if "expfma_same_wave_ns_per_iteration" in rates else None),
        "softmax_step_ns": step_ns,
        "softmax_step_pipelined_ns": rates.get("softmax_step_pipelined_ns"),
        "steady_state_step_floor_us": t_steps,
        "kernel_vs_step_floor": (t_steps / (kernel_s * 1e6)) if t_steps else None,
        "shader_clock_ghz_mfma_load": rates.get("shader_clock_ghz_mfma_load"),
    }


def cpu_baseline_bwd(cfg, budget_s: float):
    """Time the float64 oracle's backward pass on whole images of the same workload."""
    import numpy as np

    import oracle
    from inputs import make_inputs

    inp = make_inputs(cfg, batch=1)
    dout = np.random.default_rng(0).normal(size=inp["q"].shape)
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.window_attention_backward(inp["q"], inp["k"], inp["v"], dout, cfg.M, cfg.shift, inp["theta"],
                                         inp["bias_u"], inp["bias_v"])
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {
        "value": done * cfg.Hg * cfg.Wg / el,
        "unit": "tokens/s",
        "cores": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{done} image(s) of {cfg.Hg}x{cfg.Wg} tokens x {cfg.H} heads, backward of every window, "
                  f"{el:.1f} s, numpy float64 with materialised scores",
    }


def cpu_baseline(cfg, budget_s: float):
    """Time the float64 oracle on a random sample of window-heads of the same workload."""
    import numpy as np

    import oracle
    from inputs import make_inputs

    threads = None
    try:
        from threadpoolctl import threadpool_info

        info = threadpool_info()
        threads = max((d.get("num_threads") or 1) for d in info) if info else None
    except Exception:
        pass
    inp = make_inputs(cfg, batch=1)
    rng = np.random.default_rng(0)
    nwy, nwx = cfg.Hg // cfg.M, cfg.Wg // cfg.M
    done = 0
    t0 = time.perf_counter()
    while True:
        wy, wx, h = int(rng.integers(nwy)), int(rng.integers(nwx)), int(rng.integers(cfg.H))
        oracle.window_head_output(inp["q"], inp["k"], inp["v"], cfg.M, cfg.shift, 0, wy, wx, h, inp["theta"],
                                  inp["bias_u"], inp["bias_v"])
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    token_equiv = done * cfg.N / cfg.H  # one token needs all H heads
    return {
        "value": token_equiv / el,
        "unit": "tokens/s",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "sample": f"{done} random window-heads of one image ({done * cfg.N} query rows x 1 head, "
                  f"{el:.1f} s, numpy float64 with materialised scores), scaled to tokens of all {cfg.H} heads",
    }


def cpu_baseline_gated(cfg, budget_s: float):
    """Time the float64 oracle's residual on random selected blocks of the gated workload."""
    import numpy as np

    import oracle
    from inputs import make_gated_inputs

    inp = make_gated_inputs(cfg, batch=1)
    sel = oracle.select_blocks(inp["gate"], cfg.tau)
    frac = sel.size / (inp["gate"].size)
    rng = np.random.default_rng(0)
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.local_residual_window(inp["q"], inp["k"], inp["v"], int(rng.choice(sel)), cfg.w, cfg.eps)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    # one selected block per (w*w / frac) layer tokens
    return {
        "value": done * cfg.w * cfg.w / frac / el,
        "unit": "tokens/s",
        "cores": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{done} random selected {cfg.w}x{cfg.w} blocks of one image (all {cfg.H} heads, {el:.1f} s, "
                  f"numpy float64 with materialised weights), scaled by the selected fraction {frac:.3f} to "
                  "tokens of the layer",
    }


def main_gated(args):
    """--pass gated: routing + residual correction of the gated local path."""
    import numpy as np
    import torch

    import vision_transformer_windowed_window_amd as wattn
    from inputs import GATED_CONFIGS, make_gated_inputs

    name = args.workload if args.workload in GATED_CONFIGS else "gated_p2_w8"
    cfg = GATED_CONFIGS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    odt = torch.float32 if args.out_dtype == "fp32" else torch.bfloat16
    base = make_gated_inputs(cfg)
    nsel = int(np.count_nonzero(base["gate"] > cfg.tau))
    sets = []
    for i in range(args.input_sets):
        g = torch.Generator(device="cpu").manual_seed(i)
        perm = torch.randperm(cfg.B, generator=g) if i else torch.arange(cfg.B)
        t = {key: torch.from_numpy(np.ascontiguousarray(base[key])).to(torch.bfloat16)[perm].contiguous().to(dev)
             for key in ("q", "k", "v")}
        t["out"] = torch.from_numpy(base["base"])[perm].contiguous().to(odt).to(dev)
        t["gate"] = torch.from_numpy(base["gate"])[perm].contiguous().to(dev)
        t["blocks"] = torch.empty(cfg.blocks, dtype=torch.int32, device=dev)
        t["count"] = torch.empty(1, dtype=torch.int32, device=dev)
        sets.append(t)
    del base

    def step(i):  # routing and residual in one launch
        t = sets[i % len(sets)]
        wattn.gated_local_path(t["q"], t["k"], t["v"], t["out"], t["gate"], cfg.tau, w=cfg.w, eps=cfg.eps)

    def step_list(i):  # the list form: wattn_select_blocks, then wattn_local_residual
        t = sets[i % len(sets)]
        wattn.select_blocks(t["gate"], cfg.tau, blocks=t["blocks"], count=t["count"])
        wattn.local_residual(t["q"], t["k"], t["v"], t["out"], t["blocks"], t["count"], w=cfg.w, eps=cfg.eps)

    t_w = time.perf_counter()
    i = 0
    while i < args.warmup or (time.perf_counter() - t_w < WARMUP_MIN_S and i < WARMUP_MAX_STEPS):
        step(i)
        step_list(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    avg_s = ev[0].elapsed_time(ev[1]) / args.steps / 1e3
    ev[2].record(stream)
    for i in range(args.steps):
        step_list(i)
    ev[3].record(stream)
    torch.cuda.synchronize()
    list_s = ev[2].elapsed_time(ev[3]) / args.steps / 1e3
    osz = 4 if args.out_dtype == "fp32" else 2
    T = cfg.w * cfg.w
    kp = (T + 31) // 32 * 32
    unit_heads = nsel * cfg.H
    # q, k, v read and out read + written on the selected tokens, every block's gate read
    alg_bytes = unit_heads * T * (3 * cfg.d * 2 + 2 * cfg.d * osz) + cfg.blocks * 4
    # matrix-core flops per (block, head): scores and PV over the padded keys, relu(K)^T V and
    # the key sums, the linear apply (high + low parts)
    flops = unit_heads * (4.0 * T * kp * cfg.d + 2.0 * kp * cfg.d * (cfg.d + 32) + 4.0 * T * cfg.d * cfg.d)
    achieved = alg_bytes / avg_s / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic_from_profiles(cfg.name, args.out_dtype, "gated")}
    rec = {
        "metric": METRIC_GATED,
        "value": cfg.tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v rounded to bf16; i.i.d. uniform block gates; N(0,1) base output)",
        "config": {"workload": cfg.name, "B": cfg.B, "Hgrid": cfg.Hg, "Wgrid": cfg.Wg, "H": cfg.H, "d": cfg.d,
                   "w": cfg.w, "tau": cfg.tau, "eps": cfg.eps, "blocks": cfg.blocks, "selected_blocks": nsel,
                   "out_dtype": args.out_dtype, "global_batch": cfg.B, "tokens_per_step": cfg.tokens,
                   "input_sets": args.input_sets,
                   "pass": "gated local path (routing + residual in one launch, wattn_gated_local)"},
        "kernel_ms_avg": avg_s * 1e3,
        "list_form_ms_avg": list_s * 1e3,
        "algorithmic_gbs_kernel": achieved,
        "tflops_executed_kernel": flops / avg_s / 1e12,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_gated(cfg, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def cpu_baseline_stack(cfg, budget_s: float):
    """Time the float64 oracle on random window-heads of every layer of the stack (gate logits
    of the window's tokens included), scaled to tokens through the whole stack."""
    import numpy as np

    import oracle
    from inputs import make_stack_layer

    rng = np.random.default_rng(0)
    per_layer = budget_s / len(cfg.layers)
    s_per_token = 0.0
    parts = []
    for l, (M, shift) in enumerate(cfg.layers):
        inp = make_stack_layer(cfg, l, batch=1)
        z = oracle.cla_gate_logits(inp["x"], inp["w_dw"], inp["b_dw"], inp["w_pw"], inp["b_pw"]).reshape(
            inp["q"].shape)
        done = 0
        t0 = time.perf_counter()
        while True:
            wy, wx, h = int(rng.integers(cfg.Hg // M)), int(rng.integers(cfg.Wg // M)), int(rng.integers(cfg.H))
            o, ys, xs = oracle.window_head_output(inp["q"], inp["k"], inp["v"], M, shift, 0, wy, wx, h, None,
                                                  inp["bias_u"], inp["bias_v"])
            _ = o * oracle.sigmoid(z[0, ys, xs, h])
            done += 1
            el = time.perf_counter() - t0
            if el >= per_layer:
                break
        t_conv = time.perf_counter()
        oracle.cla_gate_logits(inp["x"][:, :16], inp["w_dw"], inp["b_dw"], inp["w_pw"], inp["b_pw"])
        conv_per_token = (time.perf_counter() - t_conv) / (16 * cfg.Wg)
        s_per_token += el / (done * M * M / cfg.H) + conv_per_token
        parts.append(f"M={M}: {done} window-heads")
    return {
        "value": 1.0 / s_per_token,
        "unit": "tokens/s",
        "cores": os.cpu_count(),
        "kind": "oracle",
        "sample": "random window-heads of each layer (" + ", ".join(parts) + f", {budget_s:.0f} s in all) and "
                  "the gate logits of a 16-row strip per layer, numpy float64 with materialised scores, "
                  "scaled to tokens through all six layers",
    }


def main_stack(args):
    """--pass stack: the cyclic-window stack with the convolutional gate."""
    import numpy as np
    import torch

    import vision_transformer_windowed_window_amd as wattn
    from inputs import STACK_CONFIGS, make_stack_layer

    cfg = STACK_CONFIGS["sst_cycle_sr"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf, f32 = torch.bfloat16, torch.float32
    layers = []
    for l in range(len(cfg.layers)):
        inp = make_stack_layer(cfg, l)
        t = {key: torch.from_numpy(inp[key]).to(bf).to(dev) for key in ("q", "k", "v", "x", "bias_u", "bias_v")}
        t.update({key: torch.from_numpy(inp[key]).to(dev) for key in ("w_dw", "b_dw", "w_pw", "b_pw")})
        t["z"] = torch.empty_like(t["x"])
        t["out"] = torch.empty_like(t["q"])
        layers.append(t)
        del inp

    def conv(l):
        t = layers[l]
        wattn.cla_logits(t["x"], t["w_dw"], t["w_pw"], t["b_dw"], t["b_pw"], out=t["z"])

    def attn(l):
        t = layers[l]
        M, shift = cfg.layers[l]
        wattn.forward(t["q"], t["k"], t["v"], M=M, shift=shift, bias_u=t["bias_u"], bias_v=t["bias_v"],
                      out=t["out"], gate_z=t["z"].view(t["q"].shape))

    def step(i):
        for l in range(len(layers)):
            conv(l)
            attn(l)

    t_w = time.perf_counter()
    i = 0
    while i < args.warmup or (time.perf_counter() - t_w < WARMUP_MIN_S and i < WARMUP_MAX_STEPS):
        step(i)
        i += 1
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    step_s = ev0.elapsed_time(ev1) / args.steps / 1e3

    # per-kernel averages, each kernel launched back to back on its own
    def timed(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps / 1e3

    reps = max(3, args.steps // 5)
    per_layer = []
    dense_total = 0.0
    for l, (M, shift) in enumerate(cfg.layers):
        t_conv = timed(lambda: conv(l), reps)
        t_attn = timed(lambda: attn(l), reps)
        dense = 4.0 * cfg.tokens * M * M * cfg.d * cfg.H
        pairs = wattn.pair_count(cfg.B, cfg.H, cfg.Hg, cfg.Wg, M, shift)
        executed = 2.0 * pairs * (cfg.d + cfg.r + cfg.d)
        dense_total += dense
        per_layer.append({"M": M, "shift": shift, "cla_logits_ms": t_conv * 1e3, "attention_ms": t_attn * 1e3,
                          "attention_tflops_dense": dense / t_attn / 1e12,
                          "attention_tflops_executed": executed / t_attn / 1e12,
                          "cla_logits_gbs": 4.0 * cfg.tokens * cfg.C / t_conv / 1e9})
    # the dominant kernel: the gated attention of the slowest layer
    dom = max(range(len(per_layer)), key=lambda l: per_layer[l]["attention_ms"])
    achieved = per_layer[dom]["attention_tflops_dense"]
    roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
            "kernel": f"wattn_forward_gated, layer {dom} (M={cfg.layers[dom][0]}, shift={cfg.layers[dom][1]})"}
    rec = {
        "metric": METRIC_STACK,
        "value": cfg.tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v and layer inputs rounded to bf16; seeded RIB-MLP bias factors "
                "and gate convolution weights per layer)",
        "config": {"workload": cfg.name, "B": cfg.B, "Hgrid": cfg.Hg, "Wgrid": cfg.Wg, "H": cfg.H, "d": cfg.d,
                   "r": cfg.r, "layers": [list(x) for x in cfg.layers], "out_dtype": "bf16",
                   "global_batch": cfg.B, "tokens_per_step": cfg.tokens,
                   "pass": "per layer: wattn_cla_logits + wattn_forward_gated"},
        "kernel_ms_avg": step_s * 1e3,
        "tflops_dense_stack": dense_total / step_s / 1e12,
        "per_layer": per_layer,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_stack(cfg, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def cpu_baseline_model(cfg, budget_s: float):
    """Time the float64 oracle's forward pass on one image of the workload."""
    import oracle
    from inputs import images, model_params

    P = model_params(cfg, "bf16")
    img = images(1, cfg.img, cfg.seed + 1, "bf16")
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.flashswin_forward(img, P, cfg.p, cfg.M)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": done / el, "unit": "img/s", "cores": os.cpu_count(), "kind": "oracle",
            "sample": f"{done} forward pass(es) of one {cfg.img} px image, {el:.1f} s, numpy float64 with "
                      "materialised window scores"}


def main_model(args):
    """--pass model: the FlashSwin-T forward pass."""
    import torch

    import vision_transformer_windowed_window_amd as wattn
    from inputs import MODEL_CONFIGS, images, model_params
    from vision_transformer_windowed_window_amd.model import FlashSwinT, stage_window

    name = args.workload if args.workload in MODEL_CONFIGS else "flashswin_t_p4_m32"
    cfg = MODEL_CONFIGS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    net = FlashSwinT(model_params(cfg, "bf16"), p=cfg.p, M=cfg.M)
    imgs = [torch.from_numpy(images(cfg.B, cfg.img, cfg.seed + 10 + i, "bf16")).to(torch.bfloat16).to(dev)
            for i in range(2)]

    def step(i):
        return net(imgs[i % 2])

    t_w = time.perf_counter()
    i = 0
    while i < args.warmup or (time.perf_counter() - t_w < WARMUP_MIN_S and i < WARMUP_MAX_STEPS):
        step(i)
        i += 1
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    step_s = ev0.elapsed_time(ev1) / args.steps / 1e3

    # the window-attention kernels of the pass, timed alone on inputs of their shapes
    att_s, att_flops, parts = 0.0, 0.0, []
    grid, C = cfg.img // cfg.p, cfg.C
    for s_idx, (depth, heads) in enumerate(zip(cfg.depths, cfg.heads)):
        g = torch.Generator(device="cpu").manual_seed(s_idx)
        q, k, v = (torch.randn((cfg.B, grid, grid, heads, 32), generator=g).to(torch.bfloat16).to(dev)
                   for _ in range(3))
        th = net.stages[s_idx]["theta"]
        for i in range(depth):
            Mw, sh = stage_window(grid, cfg.M, 0 if i % 2 == 0 else cfg.M // 2)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            a.record(stream)
            for _ in range(reps):
                wattn.forward(q, k, v, M=Mw, shift=sh, theta=th)
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / reps / 1e3
            att_s += t
            att_flops += 4.0 * cfg.B * grid * grid * Mw * Mw * 32 * heads
            parts.append({"stage": s_idx, "grid": grid, "M": Mw, "shift": sh, "ms": t * 1e3})
        grid //= 2
        C *= 2
    achieved = att_flops / att_s / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
            "kernel": "wattn_fwd_bf16_kernel over the pass's 12 attention calls (dense flops / their summed time)"}
    rec = {
        "metric": METRIC_MODEL,
        "value": cfg.B / (ms_per_step / 1e3),
        "unit": "img/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) NHWC images rounded to bf16; seeded random weights)",
        "config": {"workload": cfg.name, "B": cfg.B, "img": cfg.img, "p": cfg.p, "M": cfg.M, "C": cfg.C,
                   "depths": list(cfg.depths), "heads": list(cfg.heads), "global_batch": cfg.B,
                   "tokens_stage1": cfg.tokens, "pass": "forward (inference), batch resident in HBM"},
        "kernel_ms_avg": step_s * 1e3,
        "attention_ms_in_pass": att_s * 1e3,
        "attention_share": att_s / step_s,
        "attention_calls": parts,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_model(cfg, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def make_fwd_sets(cfg, args, torch, dev):
    """Resident input sets of a forward workload (the batch permuted per set) and its parameters."""
    import numpy as np

    from inputs import make_inputs

    tdt = torch.bfloat16
    odt = torch.float32 if args.out_dtype == "fp32" else torch.bfloat16
    base = make_inputs(cfg)
    sets = []
    for i in range(args.input_sets):
        g = torch.Generator(device="cpu").manual_seed(i)
        perm = torch.randperm(cfg.B, generator=g) if i else torch.arange(cfg.B)
        t = {key: torch.from_numpy(np.ascontiguousarray(base[key])).to(tdt)[perm].contiguous().to(dev)
             for key in ("q", "k", "v")}
        t["out"] = torch.empty(t["q"].shape, dtype=odt, device=dev)
        sets.append(t)
    params = {
        "theta": None if base["theta"] is None else torch.from_numpy(base["theta"]).to(dev),
        "bias_u": None if base["bias_u"] is None else torch.from_numpy(base["bias_u"]).to(tdt).to(dev),
        "bias_v": None if base["bias_v"] is None else torch.from_numpy(base["bias_v"]).to(tdt).to(dev),
    }
    return sets, params


def main_copy(args):
    """A plain device copy of known size, the scale for the HBM counters.

    One step reads COPY_BYTES and writes COPY_BYTES (an element-wise negation of fp32 data, one
    kernel).  Under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, the counters' reading for this
    kernel divided by COPY_BYTES gives the factor that turns the same counters into bytes for
    the attention kernels."""
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = COPY_BYTES // 4
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)

    def step(i):
        torch.neg(src, out=dst)

    wall_s, avg_kern_s, _ = time_steps(step, args.steps, args.warmup, torch)
    print(json.dumps({
        "metric": "device copy GB/s (read + write)", "value": 2 * COPY_BYTES / avg_kern_s / 1e9, "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "copy", "bytes_read_per_step": COPY_BYTES, "bytes_written_per_step": COPY_BYTES},
        "kernel_ms_avg": avg_kern_s * 1e3}), flush=True)


def time_steps(step, steps: int, warmup: int, torch, warmup_min_s: float = WARMUP_MIN_S):
    """Untimed warm-up, then `steps` back-to-back steps bracketed by events on the stream the
    kernels run on.  Returns (wall seconds per step, kernel seconds per step, peak extra bytes)."""
    # The GPU's clocks only reach their sustained level after tens of milliseconds of load, so
    # the warm-up runs at least warmup_min_s seconds of back-to-back launches.
    t_w = time.perf_counter()
    i = 0
    while i < warmup or (time.perf_counter() - t_w < warmup_min_s and i < WARMUP_MAX_STEPS):
        step(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    # The host enqueues faster than the kernel runs, so the stream never idles between the
    # launches and the event interval over K is the kernel's average duration.
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    peak_extra = torch.cuda.max_memory_allocated() - mem0
    return elapsed / steps, ev0.elapsed_time(ev1) / steps / 1e3, int(peak_extra)


def fwd_figures(cfg, wattn, out_dtype: str, which: str, kernel_s: float):
    """Flop and byte counts of one step and the roofline record of the dominant kernel."""
    dense = cfg.dense_flops() * (2.5 if which == "bwd" else 1.0)  # backward: 5 products vs 2
    pairs = wattn.pair_count(cfg.B, cfg.H, cfg.Hg, cfg.Wg, cfg.M, cfg.shift)
    executed = 2.0 * pairs * (cfg.d + cfg.r + cfg.d)
    osz = 4 if out_dtype == "fp32" else 2
    el = cfg.tokens * cfg.H * cfg.d
    if which == "fwd":
        alg_bytes = 3 * el * 2 + el * osz  # q, k, v read once, out written once
    else:
        executed *= 2.5
        # q, k, v, out, dout and lse read once; dq, dk, dv and the row scratch written once
        alg_bytes = 3 * el * 2 + 2 * el * osz + cfg.tokens * cfg.H * 4 + 3 * el * 4 + cfg.tokens * cfg.H * 4
    compute_bound = cfg.N / 2 >= PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3  # AI vs ridge (FLOP/B)
    if compute_bound:
        achieved = dense / kernel_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    else:
        achieved = alg_bytes / kernel_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    return dense, pairs, executed, alg_bytes, roof


def sweep_record(cfg, args, wattn, torch, dev):
    """Time one more forward workload briefly (a few seconds) with the headline's protocol."""
    sets, prm = make_fwd_sets(cfg, args, torch, dev)

    def step(i):
        t = sets[i % len(sets)]
        wattn.forward(t["q"], t["k"], t["v"], M=cfg.M, shift=cfg.shift, theta=prm["theta"], bias_u=prm["bias_u"],
                      bias_v=prm["bias_v"], out=t["out"])

    steps = max(5, min(args.steps, args.sweep_steps))
    wall_s, kern_s, peak_extra = time_steps(step, steps, 3, torch, warmup_min_s=0.2)
    dense, pairs, executed, alg_bytes, roof = fwd_figures(cfg, wattn, args.out_dtype, "fwd", kern_s)
    roof["traffic"] = traffic_from_profiles(cfg.name, args.out_dtype)
    del sets
    torch.cuda.empty_cache()
    return {
        "shape": {"B": cfg.B, "Hgrid": cfg.Hg, "Wgrid": cfg.Wg, "M": cfg.M, "shift": cfg.shift, "H": cfg.H,
                  "d": cfg.d, "r": cfg.r, "rope": cfg.rope},
        "steps": steps,
        "kernel_ms": kern_s * 1e3,
        "ms_per_step": wall_s * 1e3,
        "tokens_per_s": cfg.tokens / kern_s,
        "tflops_dense_kernel": dense / kern_s / 1e12,
        "tflops_executed_kernel": executed / kern_s / 1e12,
        "pct_bf16_peak_dense": 100.0 * dense / kern_s / 1e12 / PEAK_BF16_TFLOPS,
        "algorithmic_gbs_kernel": alg_bytes / kern_s / 1e9,
        "pct_hbm_peak": 100.0 * alg_bytes / kern_s / 1e9 / PEAK_HBM_GBS,
        "peak_extra_device_bytes": peak_extra,
        "materialised_scores_bytes": int(cfg.tokens * cfg.H * cfg.N * 4),
        "roofline": roof,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator needs no collective: batch and window sharding are communication-free)",
              file=sys.stderr)
        sys.exit(2)
    if args.which == "gated":
        main_gated(args)
        return
    if args.which == "stack":
        main_stack(args)
        return
    if args.which == "model":
        main_model(args)
        return
    if args.which == "copy":
        main_copy(args)
        return

    import torch

    import vision_transformer_windowed_window_amd as wattn
    from inputs import CONFIGS

    cfg = CONFIGS[args.workload]
    assert cfg.dtype == "bf16", "the benchmark covers the bf16 workloads"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    odt = torch.float32 if args.out_dtype == "fp32" else torch.bfloat16

    # ---- inputs resident in HBM (several sets, rotated)
    sets, prm = make_fwd_sets(cfg, args, torch, dev)
    theta, bu, bv = prm["theta"], prm["bias_u"], prm["bias_v"]

    def step(i):
        t = sets[i % len(sets)]
        wattn.forward(t["q"], t["k"], t["v"], M=cfg.M, shift=cfg.shift, theta=theta, bias_u=bu, bias_v=bv,
                      out=t["out"])

    if args.which == "bwd":
        # forward output, row statistic and a seeded output gradient per set, computed untimed
        for i, t in enumerate(sets):
            t["out"], t["lse"] = wattn.forward(t["q"], t["k"], t["v"], M=cfg.M, shift=cfg.shift, theta=theta,
                                               bias_u=bu, bias_v=bv, out_dtype=odt, return_lse=True)
            g = torch.Generator(device="cpu").manual_seed(100 + i)
            t["dout"] = torch.randn(t["q"].shape, generator=g).to(odt).to(dev)

        def step(i):  # noqa: F811 -- the backward pass replaces the forward step
            t = sets[i % len(sets)]
            wattn.backward(t["q"], t["k"], t["v"], t["out"], t["dout"], t["lse"], M=cfg.M, shift=cfg.shift,
                           theta=theta, bias_u=bu, bias_v=bv)

    wall_s, avg_kern_s, peak_extra = time_steps(step, args.steps, args.warmup, torch)
    ms_per_step = wall_s * 1e3
    tokens = cfg.tokens
    value = tokens / wall_s
    dense, pairs, executed, alg_bytes, roof = fwd_figures(cfg, wattn, args.out_dtype, args.which, avg_kern_s)
    roof["traffic"] = traffic_from_profiles(args.workload if args.which == "fwd" else args.workload + "_bwd",
                                            args.out_dtype)

    rec = {
        "metric": METRIC if args.which == "fwd" else METRIC_BWD,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v rounded to bf16; learned-theta RoPE table"
                + ("; seeded RIB-MLP bias factors" if cfg.r else "") + ")",
        "config": {
            "workload": cfg.name, "B": cfg.B, "Hgrid": cfg.Hg, "Wgrid": cfg.Wg, "M": cfg.M, "shift": cfg.shift,
            "H": cfg.H, "d": cfg.d, "r": cfg.r, "rope": cfg.rope, "out_dtype": args.out_dtype,
            "global_batch": cfg.B, "tokens_per_step": tokens, "input_sets": args.input_sets,
        },
        "tflops_dense": dense / wall_s / 1e12,
        "pct_bf16_peak_dense": 100.0 * dense / wall_s / 1e12 / PEAK_BF16_TFLOPS,
        "kernel_ms_avg": avg_kern_s * 1e3,
        "tflops_dense_kernel": dense / avg_kern_s / 1e12,
        "tflops_executed_kernel": executed / avg_kern_s / 1e12,
        "mfma_frac_executed": executed / avg_kern_s / 1e12 / PEAK_BF16_TFLOPS,
        "algorithmic_gbs_kernel": alg_bytes / avg_kern_s / 1e9,
        "peak_extra_device_bytes": peak_extra,
        "roofline": roof,
    }
    if args.which == "fwd":
        rec["pipe_bound"] = pipe_bound(float(pairs), executed, avg_kern_s)
        if rec["pipe_bound"] is not None:
            rec["shader_clock_ghz"] = rec["pipe_bound"].get("shader_clock_ghz_mfma_load")
        if not args.no_sweep:
            # the other workloads of the forward pass, each timed for a few seconds after the
            # headline (the tiny fp32 case is a parity case only)
            del sets
            torch.cuda.empty_cache()
            rec["configs"] = {}
            for name in ("swin_t_m8", "large_m32", "dense_p2_m16", "dense_p2_m8", "sr_m96_rib"):
                if name != cfg.name:
                    rec["configs"][name] = sweep_record(CONFIGS[name], args, wattn, torch, dev)
    else:
        rec["config"]["pass"] = "backward (dq, dk, dv, dtheta" + (", dbias_u, dbias_v" if cfg.r else "") + ")"
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = (cpu_baseline(cfg, args.cpu_seconds) if args.which == "fwd"
                               else cpu_baseline_bwd(cfg, args.cpu_seconds))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
