"""Benchmark of the NVFP4 dense MLP on one MI355X.

A step is one whole MLP forward (quantize -> fused gate_up + SwiGLU + NVFP4
re-quant -> down_proj) over one batch of synthetic input, with inputs and
packed weights resident in HBM. The weights are rotated over several copies
(>= 1 GB in total) so the 256 MB Infinity Cache cannot serve them, as the
distinct weights of successive layers would not be cached either.

Prints one JSON line. `value` is algorithmic bytes (decode workloads, GB/s)
or algorithmic flops (prefill, TFLOP/s) per second of wall clock over the
timed steps (no events inside them: an event record between kernels costs a
few microseconds of idle GPU); `roofline` reports the dominant kernel (the
single-launch decode kernel, i.e. the whole forward, at one token in W4A4
and W4A16; otherwise the fused gate_up kernel; for the grouped and SiLU-quantize
workloads the one call they time), measured with one HIP event pair around a
back-to-back run of it on the stream it runs on; `cpu_baseline` is the CPU
oracle timed on a bounded sample of the same workload; `step_us` is the
median, p10 and p90 of per-step GPU time from an event pair around each
step, in a second pass after the timed one. Other workloads:
`--workload silu_quant`, `grouped_w4a4`, `grouped_w4a16`.

With no --workload, --M or --sweep the line is the one-token decode (hidden
5120, intermediate 17408) and carries the metric's other halves as extra
keys, each a whole result of its own (value, roofline, cpu_baseline):
`decode_m16`, the fused small-batch MLP at 16 tokens (hidden 7168,
intermediate 18432), and `prefill`, the 8192-token W4A4 prefill on the same
weights.
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import nvfp4_quantized_dense_amd as nv  # noqa: E402
import nvfp4_synth as synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 MFMA
NVFP4_BYTES = 0.5625           # per element: 4-bit code + 1/16 of a scale byte

WORKLOADS = {
    # name: (M, H, I, mode, outliers, n_seeds, default steps, default warmup)
    "decode_w4a4": (1, 5120, 17408, "w4a4", True, 1000, 1000, 50),
    "smallbatch_w4a4": (16, 7168, 18432, "w4a4", False, 64, 500, 50),
    "prefill_w4a4": (8192, 7168, 18432, "w4a4", False, 2, 20, 3),
    "w4a16": (16, 5120, 17408, "w4a16", False, 64, 500, 50),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_tensor(bits: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def algorithmic(M, H, I, mode, out_bytes):
    """Compulsory bytes and real flops of one forward, per kernel."""
    w_gu = 2 * I * H * NVFP4_BYTES
    w_d = H * I * NVFP4_BYTES
    if mode == "w4a4":
        quant = M * H * 2 + M * H * NVFP4_BYTES
        fused = w_gu + M * H * NVFP4_BYTES + M * I * NVFP4_BYTES
        down = w_d + M * I * NVFP4_BYTES + M * H * out_bytes
    else:
        quant = 0.0
        fused = w_gu + M * H * 2 + M * I * 2
        down = w_d + M * I * 2 + M * H * out_bytes
    flops_fused = 2.0 * M * (2 * I) * H
    flops_down = 2.0 * M * H * I
    return dict(quant=quant, fused=fused, down=down, total=quant + fused + down,
                flops_fused=flops_fused, flops=flops_fused + flops_down)


def kernel_source_hash() -> str:
    """sha256[:16] over the kernel sources, as recorded in profiles/*.md."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "nvfp4_quantized_dense_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, M: int):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if the kernels are unchanged
    since those counters were taken; else None."""
    src = kernel_source_hash()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                if not line.startswith("bench-traffic:"):
                    continue
                kv = dict(t.split("=", 1) for t in line.split()[1:] if "=" in t)
                if kv.get("workload") == workload and kv.get("M") == str(M) and kv.get("src") == src:
                    return float(kv["bytes_per_launch"])
    return None


def prepare_weights(H, I, dev, copies):
    """fp32 synthetic weights -> GPU calibrate + quantize + repack (the library's
    own one-time weight preparation), replicated `copies` times."""
    out = []
    gs = []
    for tid, R, C, kind in [(synth.TENSOR_W_GATE_UP, 2 * I, H, nv.REPACK_SWIGLU),
                            (synth.TENSOR_W_DOWN, H, I, nv.REPACK_PLAIN)]:
        w = torch.from_numpy(synth.weights(0, R, C, tid)).to(dev)
        g, g_inv = nv.nvfp4_calibrate(w)
        c, s = nv.nvfp4_quantize(w, g_inv)
        del w
        p = nv.nvfp4_repack_weight(kind, c, s)
        del c, s
        out.append([p] + [p.clone() for _ in range(copies - 1)])
        gs.append(g)
    torch.cuda.synchronize()
    return out[0], out[1], gs[0], gs[1]


def step_percentiles(step, n, stream):
    """Per-step GPU time in us (median, p10, p90): one HIP event pair around
    each of n steps on the launch stream, run after the timed region."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
            "p90": float(np.percentile(t, 90)), "n": n}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_ORACLE_WEIGHTS = {}


def oracle_weights(H, I):
    """The seed-0 weights quantized by the oracle (cached per shape)."""
    import oracle
    if (H, I) not in _ORACLE_WEIGHTS:
        _ORACLE_WEIGHTS.clear()
        wgu = synth.weights(0, 2 * I, H, synth.TENSOR_W_GATE_UP)
        g_gu, gi_gu = oracle.global_scale(wgu)
        c_gu, s_gu = oracle.quantize(wgu, gi_gu)
        del wgu
        wd = synth.weights(0, H, I, synth.TENSOR_W_DOWN)
        g_d, gi_d = oracle.global_scale(wd)
        c_d, s_d = oracle.quantize(wd, gi_d)
        _ORACLE_WEIGHTS[(H, I)] = (g_gu, c_gu, s_gu, g_d, c_d, s_d)
    return _ORACLE_WEIGHTS[(H, I)]


def cpu_baseline(M, H, I, mode, outliers, per_step_bytes, per_step_flops, budget_s, use_flops, dyn=False,
                 awq=False):
    """The CPU oracle on a bounded sample of the workload's steps."""
    import oracle
    g_gu, c_gu, s_gu, g_d, c_d, s_d = oracle_weights(H, I)
    rows = min(M, 8)
    x0 = synth.activations(0, M, H, outliers=outliers)[:rows]
    if awq:
        rs = np.random.default_rng(7)
        sc_gu = synth.f32_to_bf16_bits(np.exp(0.6 * rs.standard_normal(H)).astype(np.float32))
        sc_d = synth.f32_to_bf16_bits(np.exp(0.6 * rs.standard_normal(I)).astype(np.float32))
    if mode == "w4a4":
        g1, g1_inv = oracle.global_scale(x0)
        a_gu = oracle.alpha(g1, g_gu)
        h = oracle.swiglu(oracle.gemm_w4a4(*oracle.quantize(x0, g1_inv), c_gu, s_gu, a_gu))
        g2, g2_inv = oracle.global_scale(h)
        a_d = oracle.alpha(g2, g_d)
    n = 0
    t0 = time.perf_counter()
    while True:
        x = synth.activations(n, M, H, outliers=outliers)[:rows]
        if dyn:
            oracle.mlp_w4a4_per_token(x, c_gu, s_gu, g_gu, c_d, s_d, a_d, g2_inv)
        elif mode == "w4a4":
            oracle.mlp_w4a4(x, c_gu, s_gu, a_gu, c_d, s_d, a_d, g1_inv, g2_inv)
        elif awq:
            oracle.mlp_w4a16_awq(x, c_gu, s_gu, g_gu, sc_gu, c_d, s_d, g_d, sc_d)
        else:
            oracle.mlp_w4a16(x, c_gu, s_gu, g_gu, c_d, s_d, g_d)
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    frac = rows / M  # the oracle ran `rows` of the M tokens per step
    step_s = dt / n / frac
    if use_flops:
        value, unit = per_step_flops / step_s / 1e12, "TFLOP/s"
    else:
        value, unit = per_step_bytes / step_s / 1e9, "GB/s"
    return {"value": value, "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} steps of {rows} of {M} token rows each, full MLP forward, "
                      f"{dt:.1f} s, scaled to whole steps", "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None,
                    choices=list(WORKLOADS) + ["silu_quant", "grouped_w4a4", "grouped_w4a16"],
                    help="default: decode_w4a4, with the decode_m16 and prefill legs in the same line")
    ap.add_argument("--experts", type=int, default=8, help="experts of the grouped workloads")
    ap.add_argument("--M", type=int, default=None, help="override the token count")
    ap.add_argument("--copies", type=int, default=None, help="weight copies rotated (default >= 1 GB)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", type=int, default=0, help="kernel class override (0 = auto)")
    ap.add_argument("--awq", action="store_true",
                    help="W4A16 with AWQ pre-quant scales on both GEMM inputs")
    ap.add_argument("--per-token", action="store_true",
                    help="W4A4 with per-token dynamic activation scales for x")
    ap.add_argument("--sweep", default=None,
                    help="comma-separated token counts: one JSON line per M on the same weights")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 device-to-device copies of BYTES bytes (a plain copy kernel of "
                         "known size, to scale the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path; its figure is one GPU's throughput)")
        sys.exit(2)

    default_line = args.workload is None and args.M is None and args.sweep is None
    if args.workload is None:
        args.workload = "decode_w4a4"
    nv.set_path(args.path)
    if args.workload == "silu_quant":
        print(json.dumps(run_silu_quant(args)), flush=True)
        return
    if args.workload.startswith("grouped"):
        print(json.dumps(run_grouped(args)), flush=True)
        return
    dev = torch.device("cuda:0")
    if not default_line:
        M0 = WORKLOADS[args.workload][0]
        Ms = [int(v) for v in args.sweep.split(",")] if args.sweep else [args.M if args.M is not None else M0]
        for res in run_workload(args, dev, args.workload, Ms):
            print(json.dumps(res), flush=True)
        return
    # The metric's three figures in one line: one-token decode (the headline
    # fields), then 16 tokens and 8192 tokens of the hidden-7168 MLP on one
    # set of weights.
    res = run_workload(args, dev, "decode_w4a4", [1])[0]
    res["decode_m16"], res["prefill"] = run_workload(args, dev, "smallbatch_w4a4", [16, 8192],
                                                     names=["smallbatch_w4a4", "prefill_w4a4"])
    print(json.dumps(res), flush=True)


def run_workload(args, dev, workload, Ms, names=None):
    """Results of the workload's MLP at each token count in Ms, on one set of
    packed weights (names: the workload name each M is reported under)."""
    _, H, I, mode, outliers, _, _, _ = WORKLOADS[workload]
    weight_bytes = 3 * H * I * NVFP4_BYTES
    copies = args.copies or max(1, int(np.ceil(1.0e9 / weight_bytes)))
    t = time.perf_counter()
    p_gu, p_d, g_gu, g_d = prepare_weights(H, I, dev, copies)
    log(f"[bench] weights ready in {time.perf_counter() - t:.1f}s ({copies} copies)")
    out = []
    for k, M in enumerate(Ms):
        name = names[k] if names else workload
        M0, _, _, _, outliers, n_seeds0, d_steps, d_warm = WORKLOADS[name]
        n_seeds = n_seeds0 if M == M0 else max(2, min(n_seeds0, (1 << 22) // max(1, M * H)))
        steps = args.steps if args.steps is not None else (d_steps if M == M0 else max(10, min(500, int(2e5 / M))))
        warmup = args.warmup if args.warmup is not None else min(d_warm, steps)
        out.append(run_one(args, name, dev, M, H, I, mode, outliers, n_seeds, steps, warmup, copies,
                           p_gu, p_d, g_gu, g_d))
    del p_gu, p_d
    torch.cuda.empty_cache()
    return out


def compute_dtype(mode, M, path):
    """The arithmetic the dominant kernel computes in: the one-token (and
    two-token) W4A4 decode GEMVs multiply E2M1 codes on the FP4 matrix core
    (exact products, E4M3 scales and sums in f32); the other W4A4 kernels
    run f16 MFMA on dequantized operands, W4A16 bf16 MFMA (or, at one token,
    bf16 dot products on the vector ALU)."""
    if mode == "w4a4":
        if (path == 0 and M <= 2) or path == 1:
            return "fp4", "E2M1 x E2M1 on the FP4 MFMA (unit E8M0 scales); E4M3 block scales and sums in f32"
        return "f16", "f16 MFMA on dequantized q*s (exact in f16), f32 accumulation"
    if (path == 0 and M <= 1) or path == 1:
        return "bf16", "bf16 dot products on the vector ALU against q*s, f32 accumulation"
    return "bf16", "bf16 MFMA on dequantized q*s (exact in bf16), f32 accumulation"


def run_one(args, workload, dev, M, H, I, mode, outliers, n_seeds, steps, warmup, copies, p_gu, p_d, g_gu, g_d):
    out_dtype = torch.bfloat16
    alg = algorithmic(M, H, I, mode, 2)
    prefill = M >= 256
    log(f"[bench] workload {workload} M={M} H={H} I={I} mode={mode} copies={copies} "
        f"steps={steps} warmup={warmup}")
    xs = [bf16_tensor(synth.activations(s, M, H, outliers=outliers), dev) for s in range(n_seeds)]

    # Static activation scales, calibrated on the seed-0 input: g1 from x,
    # g2 from the fused kernel's own fp32 h for that x.
    dyn = mode == "w4a4" and args.per_token
    awq = mode == "w4a16" and args.awq
    qmode = nv.MODE_W4A4_DYN if dyn else (nv.MODE_W4A4 if mode == "w4a4" else
                                          (nv.MODE_W4A16_AWQ if awq else nv.MODE_W4A16))
    ws = torch.zeros(max(1, nv.mlp_workspace_bytes(qmode, M, H, I)), dtype=torch.uint8, device=dev)
    out = torch.empty((M, H), dtype=out_dtype, device=dev)
    if mode == "w4a4":
        g1, g1_inv = nv.nvfp4_calibrate(xs[0])
        a_gu = torch.tensor([np.float32(g1.item()) * np.float32(g_gu.item())], device=dev)
        xq, xsc = nv.nvfp4_quantize(xs[0], g1_inv)
        h = nv.gemm_swiglu(0, xq, xsc, p_gu[0], I, H, a_gu, h_dtype=torch.float32)
        g2, g2_inv = nv.nvfp4_calibrate(h)
        a_d = torch.tensor([np.float32(g2.item()) * np.float32(g_d.item())], device=dev)
        del h
        xq = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
        xsc = torch.empty((M, H // 16), dtype=torch.uint8, device=dev)
        hq = torch.empty((M, I // 2), dtype=torch.uint8, device=dev)
        hsc = torch.empty((M, I // 16), dtype=torch.uint8, device=dev)
        if dyn:
            # x scaled per token: gate_up takes the weight's g alone (h keeps
            # the static g2 calibrated above) and the fused leg the token g's
            xq, xsc, row_g = nv.nvfp4_quantize_per_token(xs[0])
    else:
        a_gu, a_d = g_gu, g_d
        hb = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
        if awq:
            # synthetic per-channel pre-quant scales, AWQ's typical spread
            rs = np.random.default_rng(7)
            s_gu = bf16_tensor(synth.f32_to_bf16_bits(np.exp(0.6 * rs.standard_normal(H)).astype(np.float32)), dev)
            s_d = bf16_tensor(synth.f32_to_bf16_bits(np.exp(0.6 * rs.standard_normal(I)).astype(np.float32)), dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def fused(i):
        r = i % copies
        if dyn:
            nv.gemm_swiglu_nvfp4_quant_rowscale(xq, xsc, row_g, p_gu[r], I, H, g_gu, g2_inv, hq, hsc,
                                                stream=stream)
        elif mode == "w4a4":
            nv.gemm_swiglu_nvfp4_quant(xq, xsc, p_gu[r], I, H, a_gu, g2_inv, hq, hsc, stream=stream)
        else:
            nv.gemm_swiglu(1, xs[i % n_seeds], None, p_gu[r], I, H, a_gu, h=hb, stream=stream)

    # One step: the whole forward in one library call (quantize x, fused
    # gate_up + SwiGLU + NVFP4 re-quant, down_proj), on the rotating weight
    # copies and seeds.
    def step(i):
        x = xs[i % n_seeds]
        r = i % copies
        if dyn:
            nv.mlp_forward(nv.MODE_W4A4_DYN, x, p_gu[r], g_gu, p_d[r], a_d, I, g2_inv=g2_inv,
                           ws=ws, out=out, stream=stream)
        elif mode == "w4a4":
            nv.mlp_forward(0, x, p_gu[r], a_gu, p_d[r], a_d, I, g1_inv=g1_inv, g2_inv=g2_inv,
                           ws=ws, out=out, stream=stream)
        elif awq:
            nv.mlp_forward_w4a16_awq(x, p_gu[r], a_gu, s_gu, p_d[r], a_d, s_d, I, ws=ws, out=out, stream=stream)
        else:
            nv.mlp_forward(1, x, p_gu[r], a_gu, p_d[r], a_d, I, ws=ws, out=out, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    log("[bench] warmup done")
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"[bench] timed {steps} steps in {dt:.3f}s")

    # Dominant kernel, back to back on the same stream (rotating weight
    # copies), bracketed by one HIP event pair: at M = 1 under the automatic
    # path the whole forward is one launch (the single-launch decode kernel
    # of W4A4 or W4A16), so that launch, with the whole forward's bytes;
    # otherwise the fused gate_up launch alone.
    single = not dyn and not awq and M == 1 and args.path == 0
    leg = step if single else fused
    leg_bytes = alg["total"] if single else alg["fused"]
    leg_flops = alg["flops"] if single else alg["flops_fused"]
    n_k = max(steps, 20)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    leg(0)
    e0.record(stream)
    for i in range(n_k):
        leg(i)
    e1.record(stream)
    torch.cuda.synchronize()
    fused_ms = e0.elapsed_time(e1) / n_k
    ms_per_step = dt * 1e3 / steps
    if prefill:
        value = alg["flops"] / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = leg_flops / (fused_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": None}
    else:
        value = alg["total"] / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = leg_bytes / (fused_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    roof["traffic"] = recorded_traffic(workload + ("_per_token" if dyn else "") + ("_awq" if awq else ""), M)
    if single:
        roof["kernel"] = ("mlp_forward single-launch decode (k_decode_mlp)" if mode == "w4a4" else
                          "mlp_forward single-launch decode (k_decode_mlp16)")
    else:
        roof["kernel"] = ("gemm_swiglu_nvfp4_quant_rowscale" if dyn else
                          "gemm_swiglu_nvfp4_quant" if mode == "w4a4" else "gemm_swiglu(w4a16, bf16 h)")
    roof["kernel_us"] = fused_ms * 1e3
    roof["launches_timed"] = n_k
    roof["algorithmic_bytes"] = leg_bytes
    roof["algorithmic_flops"] = leg_flops
    step_us = step_percentiles(step, steps, stream)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(M, H, I, mode, outliers, alg["total"], alg["flops"], args.cpu_budget, prefill,
                           dyn, awq)

    res = {
        "metric": "NVFP4 MLP TFLOPS + GB/s (% roofline), decode M=1..16 and prefill M=8192",
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(mode, M, args.path)[0],
        "compute": compute_dtype(mode, M, args.path)[1],
        "data": "synthetic",
        "config": {"workload": f"{workload}{' per-token' if dyn else ''}{' awq' if awq else ''} M={M} H={H} I={I}",
                   "M": M, "hidden": H, "intermediate": I,
                   "mode": "w4a4_per_token" if dyn else ("w4a16_awq" if awq else mode), "seeds": n_seeds, "weight_copies": copies,
                   "out_dtype": "bf16", "tflops": alg["flops"] / (ms_per_step * 1e-3) / 1e12,
                   "gbs": alg["total"] / (ms_per_step * 1e-3) / 1e9},
        "roofline": roof,
        "forward": {"us": ms_per_step * 1e3,
                    "frac": (alg["total"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS if not prefill else
                             alg["flops"] / (ms_per_step * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS),
                    "of": "the whole forward's algorithmic " + ("flops" if prefill else "bytes") +
                          " per wall-clock step against the same peak"},
        "step_us": step_us,
        "cpu_baseline": cpu,
    }
    return res


def run_silu_quant(args):
    """The standalone SiLU(gate) * up + NVFP4 quantize of a bf16 gate_up (one
    expert, all rows valid): M tokens (default 8192) of intermediate 18432,
    the prefill MLP's h. HBM-bound: 4 bytes read and 0.5625 written per
    output element. A step is one call; inputs rotate over copies of >= 1 GB
    so the last-level cache cannot serve them."""
    dev = torch.device("cuda:0")
    M = args.M if args.M is not None else 8192
    I = 18432
    per_bytes = M * I * (4 + NVFP4_BYTES)
    copies = max(2, int(np.ceil(1.0e9 / (M * I * 4))))
    steps = args.steps if args.steps is not None else 200
    warmup = args.warmup if args.warmup is not None else 10
    log(f"[bench] workload silu_quant M={M} I={I} copies={copies} steps={steps} warmup={warmup}")
    x = synth.activations(0, M, 2 * I)
    gus = [bf16_tensor(x, dev).reshape(1, M, 2 * I)]
    for _ in range(copies - 1):
        gus.append(gus[0].clone())
    g_inv = torch.tensor([np.float32(0.05)], device=dev)
    mm = torch.tensor([M], dtype=torch.int32, device=dev)
    codes = torch.empty((1, M, I // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((1, M, I // 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        nv.silu_mul_nvfp4_quant(gus[i % copies], g_inv, mm, codes=codes, scales=scales, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    k_us = e0.elapsed_time(e1) * 1e3 / steps
    ms_per_step = dt * 1e3 / steps
    achieved = per_bytes / (k_us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = 8
        sub = x[:rows].reshape(1, rows, 2 * I)
        n, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_budget:
            oracle.silu_mul_quant_experts(sub, np.array([rows], np.int32), np.array([0.05], np.float32))
            n += 1
        cdt = time.perf_counter() - t1
        cpu = {"value": per_bytes * rows / M * n / cdt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} calls on {rows} of {M} rows, {cdt:.1f} s, scaled to algorithmic bytes"}
    return {
        "metric": "NVFP4 MLP TFLOPS + GB/s (% roofline), decode M=1..16 and prefill M=8192",
        "value": per_bytes / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"silu_quant E=1 M={M} I={I}", "M": M, "intermediate": I, "experts": 1,
                   "input_copies": copies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic("silu_quant", M),
                     "kernel": "k_silu_mul_quant",
                     "kernel_us": k_us, "launches_timed": steps, "algorithmic_bytes": per_bytes},
        "cpu_baseline": cpu,
    }


def run_grouped(args):
    """The grouped (expert) GEMM with masked_m: E experts' GEMMs of hidden
    7168 -> 4096 (the gate_up of a 2048-wide expert), a capacity of M tokens
    per expert (default 64) of which masked_m[e], drawn once from a seeded
    generator in [1, M], are valid; W4A4 (NVFP4 activations) or W4A16 (bf16).
    A step is one nvfp4_grouped_gemm call on bf16 output. The experts'
    weights rotate over copies of >= 1 GB in all; algorithmic bytes are the
    weights plus the valid rows' activations and outputs."""
    dev = torch.device("cuda:0")
    mode = 0 if args.workload == "grouped_w4a4" else 1
    E, N, K = args.experts, 4096, 7168
    M = args.M if args.M is not None else 64
    steps = args.steps if args.steps is not None else 300
    warmup = args.warmup if args.warmup is not None else 20
    mm_h = np.random.default_rng(11).integers(1, M + 1, E).astype(np.int32)
    packed, g_w = [], []
    for e in range(E):
        w = torch.from_numpy(synth.weights(e, N, K, synth.TENSOR_W_GATE_UP)).to(dev)
        g, gi = nv.nvfp4_calibrate(w)
        c, sc = nv.nvfp4_quantize(w, gi)
        packed.append(nv.nvfp4_repack_weight(nv.REPACK_PLAIN, c, sc).reshape(-1))
        g_w.append(g)
        del w, c, sc
    w0 = torch.cat(packed)
    del packed
    copies = args.copies or max(2, int(np.ceil(1.0e9 / w0.numel())))
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    x = np.stack([synth.activations(100 + e, M, K) for e in range(E)])  # bf16 bits [E, M, K]
    xd = bf16_tensor(x.reshape(E * M, K), dev)
    gw = torch.cat(g_w)
    if mode == 0:
        g_a, gi_a = nv.nvfp4_calibrate(xd)
        ac, asc = nv.nvfp4_quantize(xd, gi_a)
        a, a_s = ac.reshape(E, M, K // 2), asc.reshape(E, M, K // 16)
        alpha = (gw * g_a).contiguous()  # fp32 product per expert
        a_row = K * NVFP4_BYTES
    else:
        a, a_s = xd.reshape(E, M, K), None
        alpha = gw.contiguous()
        a_row = K * 2
    mm = torch.from_numpy(mm_h).to(dev)
    out = torch.empty((E, M, N), dtype=torch.bfloat16, device=dev)
    rows = int(mm_h.sum())
    per_bytes = E * N * K * NVFP4_BYTES + rows * (a_row + N * 2)
    per_flops = 2.0 * rows * N * K
    stream = torch.cuda.current_stream()
    log(f"[bench] workload {args.workload} E={E} M={M} N={N} K={K} valid rows {rows} copies={copies} "
        f"steps={steps} warmup={warmup}")

    def step(i):
        nv.nvfp4_grouped_gemm(mode, a, a_s, ws[i % copies], N, K, alpha, masked_m=mm, out=out, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    k_us = e0.elapsed_time(e1) * 1e3 / steps
    ms_per_step = dt * 1e3 / steps
    # From 256 tokens per expert the tiled MFMA kernel runs it: MFMA-bound.
    if M >= 256:
        achieved = per_flops / (k_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_F16_PEAK_TFLOPS}
    else:
        achieved = per_bytes / (k_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    roof.update({"traffic": recorded_traffic(f"{args.workload}_E{E}", M),
                 "kernel": f"nvfp4_grouped_gemm (one launch over {E} experts)", "kernel_us": k_us,
                 "launches_timed": steps, "algorithmic_bytes": per_bytes, "algorithmic_flops": per_flops})
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n_e = 2  # the oracle on the first two experts, scaled by their share of the bytes
        wc, wsc = [], []
        for e in range(n_e):
            wf = synth.weights(e, N, K, synth.TENSOR_W_GATE_UP)
            _, gi = oracle.global_scale(wf)
            c, sc = oracle.quantize(wf, gi)
            wc.append(c)
            wsc.append(sc)
        wc, wsc = np.stack(wc), np.stack(wsc)
        if mode == 0:
            _, gia = oracle.global_scale(x.reshape(E * M, K))
            c, sc = oracle.quantize(x[:n_e].reshape(n_e * M, K), gia)
            oa, oas = c.reshape(n_e, M, K // 2), sc.reshape(n_e, M, K // 16)
        else:
            oa, oas = x[:n_e], None
        al = np.ones(n_e, np.float32)
        sub_bytes = n_e * N * K * NVFP4_BYTES + int(mm_h[:n_e].sum()) * (a_row + N * 2)
        n, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_budget:
            oracle.grouped_gemm(mode, oa, oas, wc, wsc, mm_h[:n_e], al)
            n += 1
        cdt = time.perf_counter() - t1
        sub_flops = 2.0 * int(mm_h[:n_e].sum()) * N * K
        cpu = {"value": (sub_flops * n / cdt / 1e12 if M >= 256 else sub_bytes * n / cdt / 1e9),
               "unit": "TFLOP/s" if M >= 256 else "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{n} calls on {n_e} of {E} experts ({int(mm_h[:n_e].sum())} valid rows), {cdt:.1f} s, "
                         f"algorithmic {'flops' if M >= 256 else 'bytes'} of those experts"}
    return {
        "metric": "NVFP4 MLP TFLOPS + GB/s (% roofline), decode M=1..16 and prefill M=8192",
        "value": (per_flops / (ms_per_step * 1e-3) / 1e12 if M >= 256 else
                  per_bytes / (ms_per_step * 1e-3) / 1e9),
        "unit": "TFLOP/s" if M >= 256 else "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16" if mode == 0 else "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload} E={E} M={M} N={N} K={K}", "experts": E, "M": M, "N": N, "K": K,
                   "masked_m": mm_h.tolist(), "weight_copies": copies,
                   "tflops": per_flops / (ms_per_step * 1e-3) / 1e12},
        "roofline": roof,
        "cpu_baseline": cpu,
    }


if __name__ == "__main__":
    main()
