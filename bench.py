"""Benchmark of the FP8 dynamic-quant linear path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch: per-token FP8 quantization of the bf16
activations (dq_quantize_fp8) followed by the FP8 GEMM with its fused epilogue (dq_linear_fp8).
Weights are quantized once, off the timed path. Inputs are seeded synthetic tensors of the
workload's shapes, resident in HBM before timing starts; several buffer sets rotate so that the
256 MB last-level cache does not hold a step's inputs. The default warm-up (300 untimed steps)
brings the chip to the steady clock it holds under this load before the timed steps.

Prints one JSON line: whole-step throughput (TFLOP/s), the GEMM kernel against the FP8 matrix
peak, the quantize kernel and the fused LayerNorm + modulation + quantize kernel against HBM
bandwidth, the attention input projection with its fused query/key norm + rotary epilogue, the
linears of a full FLUX-dev denoising step
(ms), and the CPU oracle timed on the host as a baseline.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 matrix peak
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E bandwidth
METRIC = "FP8-DQ linear TFLOP/s & % FP8 MFMA peak; quantizer GB/s; DiT-step linears ms"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "gemm": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "gemm_fp8.hip"),
    "quantize": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "quantize.hip"),
    "ln_modulate": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "quantize.hip"),
    "qkv": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "gemm_fp8.hip"),
    "attention": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "attention.hip"),
    "mx_linear": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "gemm_mx.hip"),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(kind, workload_name):
    """HBM bytes per launch measured with rocprofv3 counters, if the kernel source is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
        rec = data[workload_name][kind]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kind]):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------------------------

def to_dev_bf16(torch, u16, dev):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(dev)


def bench_linear(shape, seed, steps, warmup, n_sets):
    """Time `steps` steps of quantize + linear. Returns a dict of timings."""
    import torch
    import fp8_dynamic_quant_amd as dq
    from workloads import make_linear_inputs

    dev = torch.device("cuda:0")
    inp = make_linear_inputs(shape, seed)
    M, K, N = shape.M, shape.K, shape.N
    gated = shape.epilogue == "gated_residual"
    sets = []
    for _ in range(n_sets):
        x = to_dev_bf16(torch, inp.x, dev)
        w = to_dev_bf16(torch, inp.w, dev)
        qw, sw = dq.dq_quantize_weight_fp8(w)
        del w
        st = {
            "x": x, "qw": qw, "sw": sw,
            "q": torch.empty((M, K), dtype=torch.uint8, device=dev),
            "sa": torch.empty((M,), dtype=torch.float32, device=dev),
            "bias": to_dev_bf16(torch, inp.bias, dev),
            "out": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
            "gate": to_dev_bf16(torch, inp.gate, dev) if gated else None,
            "res": to_dev_bf16(torch, inp.residual, dev) if gated else None,
        }
        sets.append(st)
    torch.cuda.synchronize()

    def step(st):
        dq.dq_quantize_fp8(st["x"], st["q"], st["sa"])
        e_mid = torch.cuda.Event(enable_timing=True)
        e_mid.record()
        if gated:   # in place on the residual stream, as in the model
            dq.dq_linear_fp8(st["q"], st["sa"], st["qw"], st["sw"], st["bias"], shape.epilogue,
                             st["gate"], st["res"], out=st["res"])
        else:
            dq.dq_linear_fp8(st["q"], st["sa"], st["qw"], st["sw"], st["bias"], shape.epilogue,
                             out=st["out"])
        return e_mid

    for i in range(warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()
    starts, mids, ends = [], [], []
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record()
    for i in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record()
        em = step(sets[i % n_sets])
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        starts.append(e0)
        mids.append(em)
        ends.append(e1)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_begin.elapsed_time(t_end)
    q_ms = np.array([a.elapsed_time(b) for a, b in zip(starts, mids)])
    g_ms = np.array([a.elapsed_time(b) for a, b in zip(mids, ends)])
    # the quantizer alone, back to back (its launches are short, so per-launch events would
    # mostly time the events themselves)
    reps = 4 * steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        st = sets[i % n_sets]
        dq.dq_quantize_fp8(st["x"], st["q"], st["sa"])
    e1.record()
    torch.cuda.synchronize()
    q_loop_ms = e0.elapsed_time(e1) / reps
    return {"total_ms": total_ms, "wall_s": wall, "quant_ms": q_ms, "gemm_ms": g_ms,
            "quant_loop_ms": q_loop_ms}


def bench_modulate(M, K, steps, n_sets, seed=11):
    """The fused LayerNorm + modulation + quantization over M x K hidden states, back to back over
    rotating inputs: without storing y (what a block feeding only the next linear runs), with y,
    and, for context, the unfused sequence (torch LayerNorm and modulation in bf16, then
    dq_quantize_fp8). Returns microseconds per call."""
    import torch
    import torch.nn.functional as F
    import fp8_dynamic_quant_amd as dq
    from workloads import make_modulation, make_rows

    dev = torch.device("cuda:0")
    x16 = make_rows(M, K, seed)
    s16, t16 = make_modulation(K, seed)
    ms, mt = to_dev_bf16(torch, s16, dev), to_dev_bf16(torch, t16, dev)
    sets = [{"x": to_dev_bf16(torch, x16, dev),
             "q": torch.empty((M, K), dtype=torch.uint8, device=dev),
             "s": torch.empty((M,), dtype=torch.float32, device=dev),
             "y": torch.empty((M, K), dtype=torch.bfloat16, device=dev)} for _ in range(n_sets)]
    torch.cuda.synchronize()

    def fused(st, store_y):
        dq.dq_layernorm_modulate_quantize_fp8(st["x"], ms, mt, store_y=store_y, q=st["q"],
                                              scale=st["s"], y=st["y"] if store_y else None)

    def unfused(st):
        h = F.layer_norm(st["x"], (K,), eps=1e-6) * (1 + ms) + mt
        dq.dq_quantize_fp8(h, st["q"], st["s"])

    def timed(fn, reps):
        for i in range(max(reps // 4, n_sets)):
            fn(sets[i % n_sets])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(sets[i % n_sets])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    reps = 4 * steps
    return {"no_y_us": timed(lambda st: fused(st, False), reps),
            "y_us": timed(lambda st: fused(st, True), reps),
            "unfused_us": timed(unfused, max(reps // 4, 1))}


def bench_qkv(steps, warmup, n_sets, M=4096, K=3072, heads=24, seed=3200):
    """The attention input projection of the image stream at 1024^2 (4096 tokens, 3072 -> 3 x 24
    heads x 128) with the fused query/key RMS norm + rotary epilogue, against the same GEMM with
    the plain bias epilogue and, for context, that GEMM followed by the torch ops the fusion
    replaces. Event pairs around each call; returns microseconds per call."""
    import torch
    import torch.nn.functional as F
    import fp8_dynamic_quant_amd as dq
    from workloads import LinearShape, make_linear_inputs, make_qk_norm, make_rope

    dev = torch.device("cuda:0")
    N = 3 * heads * 128
    shape = LinearShape("image.qkv", M, K, N, "bias", 31, 30.0)
    inp = make_linear_inputs(shape, seed)
    cos, sin = make_rope(M, n_text=0)
    tcos = torch.from_numpy(cos).to(dev)
    tsin = torch.from_numpy(sin).to(dev)
    nqk = to_dev_bf16(torch, make_qk_norm(seed), dev)
    sets = []
    for _ in range(n_sets):
        q, sa = dq.dq_quantize_fp8(to_dev_bf16(torch, inp.x, dev))
        qw, sw = dq.dq_quantize_weight_fp8(to_dev_bf16(torch, inp.w, dev))
        sets.append({"q": q, "sa": sa, "qw": qw, "sw": sw, "b": to_dev_bf16(torch, inp.bias, dev),
                     "o": tuple(torch.empty((heads, M, 128), dtype=torch.bfloat16, device=dev)
                                for _ in range(3)),
                     "plain": torch.empty((M, N), dtype=torch.bfloat16, device=dev)})
    torch.cuda.synchronize()
    c2 = tcos[:, None, :]
    s2 = tsin[:, None, :]

    def fused(st):
        dq.dq_linear_qkv_fp8(st["q"], st["sa"], st["qw"], st["sw"], heads, st["b"], nqk, tcos,
                             tsin, out=st["o"])

    def plain(st):
        dq.dq_linear_fp8(st["q"], st["sa"], st["qw"], st["sw"], st["b"], "bias", out=st["plain"])

    def unfused(st):
        plain(st)
        t = st["plain"].view(M, 3, heads, 128)
        outs = []
        for r in range(2):
            h = F.rms_norm(t[:, r].float(), (128,), nqk[r].float(), eps=1e-6)
            a, b = h[..., 0::2], h[..., 1::2]
            rot = torch.stack((c2 * a - s2 * b, s2 * a + c2 * b), dim=-1).flatten(-2)
            outs.append(rot.to(torch.bfloat16).transpose(0, 1).contiguous())
        outs.append(t[:, 2].transpose(0, 1).contiguous())
        return outs

    def timed(fn, n):
        for i in range(warmup):
            fn(sets[i % n_sets])
        torch.cuda.synchronize()
        evs = []
        for i in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(sets[i % n_sets])
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3

    return {"fused_us": timed(fused, steps), "plain_us": timed(plain, steps),
            "unfused_us": timed(unfused, max(steps // 4, 5)), "flops": 2 * M * N * K,
            "shape": [M, K, N], "heads": heads}


def bench_attention(steps, warmup, n_sets, H=24, S=4608, seed=11):
    """Joint text + image attention of a FLUX block at 1024^2 (24 heads, 4608 tokens): the FP8
    attention kernel (codes already quantized), the quantization of q, k and v, and, for
    context, torch's bf16 scaled_dot_product_attention on the same bf16 inputs."""
    import torch
    import torch.nn.functional as F
    import fp8_dynamic_quant_amd as dq

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    sets = []
    for _ in range(n_sets):
        q, k, v = (torch.randn((H, S, 128), generator=gen, device=dev).to(torch.bfloat16)
                   for _ in range(3))
        sets.append({"bf": (q, k, v), "fp8": dq.quantize_qkv_heads_fp8(q, k, v),
                     "out": torch.empty((S, H, 128), dtype=torch.bfloat16, device=dev)})
    torch.cuda.synchronize()

    def timed(fn, n):
        for i in range(warmup):
            fn(sets[i % n_sets])
        torch.cuda.synchronize()
        evs = []
        for i in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(sets[i % n_sets])
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3

    attn = timed(lambda st: dq.dq_attention_fp8(*st["fp8"], out=st["out"]), steps)
    quant = timed(lambda st: dq.quantize_qkv_heads_fp8(*st["bf"]), steps)
    sdpa = timed(lambda st: F.scaled_dot_product_attention(*(t[None] for t in st["bf"])), steps)
    return {"attn_us": attn, "quant_us": quant, "sdpa_us": sdpa, "flops": 4 * H * S * S * 128,
            "H": H, "S": S}


def bench_mx(shape, seed, steps, warmup, n_sets):
    """The block-scaled (MX) FP8 path on the benchmark linear's shape: per-32 block quantization
    of the activations, then the GEMM on the scaled FP8 matrix instruction, weights quantized
    once; the per-row FP8 GEMM on the same inputs is timed beside it. Event pairs around each
    call; returns microseconds per call."""
    import torch
    import fp8_dynamic_quant_amd as dq
    from workloads import make_linear_inputs

    dev = torch.device("cuda:0")
    M, K, N = shape.M, shape.K, shape.N
    inp = make_linear_inputs(shape, seed)
    epi = "gelu_tanh" if shape.epilogue == "gelu_tanh" else "bias"
    wb = to_dev_bf16(torch, inp.w, dev)
    qw, sw = dq.dq_quantize_mx_fp8(wb)
    rq, rs = dq.dq_quantize_weight_fp8(wb)
    bias = to_dev_bf16(torch, inp.bias, dev)
    xb = to_dev_bf16(torch, inp.x, dev)
    sets = []
    for i in range(n_sets):
        x = xb if i == 0 else (xb * (1.0 + 0.01 * i)).to(torch.bfloat16)
        qa, sa = dq.dq_quantize_mx_fp8(x)
        q8, s8 = dq.dq_quantize_fp8(x)
        sets.append({"x": x, "qa": qa, "sa": sa, "q8": q8, "s8": s8,
                     "out": torch.empty((M, N), dtype=torch.bfloat16, device=dev)})
    torch.cuda.synchronize()

    def timed(fn, n):
        for i in range(warmup):
            fn(sets[i % n_sets])
        torch.cuda.synchronize()
        evs = []
        for i in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(sets[i % n_sets])
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3

    gemm = timed(lambda st: dq.dq_linear_mx_fp8(st["qa"], st["sa"], qw, sw, bias, epi,
                                                out=st["out"]), steps)
    # the quantizer (a few microseconds) as back-to-back launches, one event pair around the loop
    n_q = 4 * steps
    for i in range(warmup):
        dq.dq_quantize_mx_fp8(sets[i % n_sets]["x"], sets[i % n_sets]["qa"], sets[i % n_sets]["sa"])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_q):
        dq.dq_quantize_mx_fp8(sets[i % n_sets]["x"], sets[i % n_sets]["qa"], sets[i % n_sets]["sa"])
    e1.record()
    torch.cuda.synchronize()
    quant = e0.elapsed_time(e1) * 1e3 / n_q
    rowwise = timed(lambda st: dq.dq_linear_fp8(st["q8"], st["s8"], rq, rs, bias, epi,
                                                out=st["out"]), steps)
    return {"gemm_us": gemm, "quant_us": quant, "rowwise_us": rowwise,
            "flops": 2 * M * N * K, "shape": [M, K, N], "epilogue": epi,
            "quant_bytes": M * K * 2 + M * K + M * K // 32}


def bench_dit_step(steps, warmup):
    """All linears of one 1024^2 FLUX-dev denoising step (228 quantize + GEMM pairs), distinct
    weights per block, timed end to end as one sequence on one stream."""
    import torch
    import fp8_dynamic_quant_amd as dq
    from workloads import dit_step_device_inputs, workload

    w = workload("flux-dit-step-1024")
    dev = torch.device("cuda:0")
    plan, acts, residuals = dit_step_device_inputs(w, dev, dq.dq_quantize_weight_fp8)
    outs = {}
    qbuf = {}
    for lin in plan:
        M, K, N = lin["M"], lin["K"], lin["N"]
        if (M, K) not in qbuf:
            qbuf[(M, K)] = (torch.empty((M, K), dtype=torch.uint8, device=dev),
                            torch.empty((M,), dtype=torch.float32, device=dev))
        if lin["epilogue"] != "gated_residual" and (M, N) not in outs:
            outs[(M, N)] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def run():
        for lin in plan:
            M, K, N = lin["M"], lin["K"], lin["N"]
            q, sa = qbuf[(M, K)]
            dq.dq_quantize_fp8(acts[lin["act"]], q, sa)
            if lin["epilogue"] == "gated_residual":
                r = residuals[lin["residual"]]
                dq.dq_linear_fp8(q, sa, lin["qw"], lin["sw"], lin["bias"], "gated_residual",
                                 lin["gate"], r, out=r)
            else:
                dq.dq_linear_fp8(q, sa, lin["qw"], lin["sw"], lin["bias"], lin["epilogue"],
                                 out=outs[(M, N)])

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = w.flops_per_step
    wbytes = sum(l["N"] * l["K"] for l in plan)
    return {"ms": ms, "tflops": flops / ms / 1e9, "linears": len(plan), "weight_bytes": wbytes}


# ---------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host
# ---------------------------------------------------------------------------------------------

def cpu_baseline(shape, seed, reps=2):
    from threadpoolctl import threadpool_info
    from oracle import linear_ref, quantize_rows
    from workloads import bf16_bits_to_f32, make_linear_inputs

    inp = make_linear_inputs(shape, seed)
    qw, sw = quantize_rows(bf16_bits_to_f32(inp.w))       # weight prep, not timed
    x = bf16_bits_to_f32(inp.x)
    bias = bf16_bits_to_f32(inp.bias)
    gate = None if inp.gate is None else bf16_bits_to_f32(inp.gate)
    res = None if inp.residual is None else bf16_bits_to_f32(inp.residual)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        q, sa = quantize_rows(x)
        y = linear_ref(q, sa, qw, sw, bias, shape.epilogue, gate, res)
        times.append(time.perf_counter() - t0)
        del y
    t = float(np.mean(times))
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    return {
        "value": round(shape.flops / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"the whole {shape.M}x{shape.K}x{shape.N} {shape.epilogue} step (quantize "
                   f"x + exact float64 contraction + epilogue), mean of {reps} runs; "
                   f"elementwise NumPy single-threaded, BLAS with {threads} threads"),
        "seconds_per_step": round(t, 3),
        "host_cpus_visible": os.cpu_count(),
    }


# ---------------------------------------------------------------------------------------------

def calibrate_copy(nbytes=1 << 30):
    """One plain device-to-device copy of known size (a reference for HBM byte counters)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"calibration copy of {nbytes} bytes done")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The chip's clock settles over the first tens of milliseconds of dense FP8 work: 300
    # untimed steps (about 60 ms) reach the steady state that the timed steps then measure.
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="flux-mlp-up-1024")
    ap.add_argument("--linear", type=int, default=0, help="index of the linear in the workload")
    ap.add_argument("--sets", type=int, default=6, help="rotating input/output buffer sets")
    ap.add_argument("--dit-steps", type=int, default=5)
    ap.add_argument("--no-dit", action="store_true")
    ap.add_argument("--no-modulate", action="store_true")
    ap.add_argument("--no-qkv", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-mx", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB plain copy first (reference for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X and has no "
              "multi-GPU mode (--gpus must be 1).", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    from workloads import workload
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import fp8_dynamic_quant_amd as dq

    if args.calibrate_copy:
        calibrate_copy()

    w = workload(args.workload)
    shape = w.linears[args.linear]
    log(f"workload {w.name}[{args.linear}] M={shape.M} K={shape.K} N={shape.N} "
        f"epilogue={shape.epilogue}; warmup {args.warmup}, steps {args.steps}")
    r = bench_linear(shape, w.seed, args.steps, args.warmup, args.sets)
    ms_per_step = r["total_ms"] / args.steps
    value = shape.flops / ms_per_step / 1e9          # TFLOP/s
    gemm_ms = float(np.mean(r["gemm_ms"]))
    quant_ms = float(r["quant_loop_ms"])
    quant_in_step_ms = float(np.mean(r["quant_ms"]))
    gemm_tflops = shape.flops / gemm_ms / 1e9
    qbytes = 3 * shape.M * shape.K + 4 * shape.M
    quant_gbps = qbytes / quant_ms / 1e6
    log(f"step {ms_per_step * 1e3:.1f} us: quantize {quant_ms * 1e3:.1f} us "
        f"({quant_gbps:.0f} GB/s; {quant_in_step_ms * 1e3:.1f} us between events inside steps), "
        f"GEMM {gemm_ms * 1e3:.1f} us ({gemm_tflops:.0f} TFLOP/s)")

    traffic = stored_traffic("gemm", w.name)
    qtraffic = stored_traffic("quantize", w.name)
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 in/out)",
        "data": "synthetic",
        "config": {"workload": w.name, "linear": shape.name, "M": shape.M, "K": shape.K,
                   "N": shape.N, "epilogue": shape.epilogue, "rotating_sets": args.sets,
                   "parallelism": "none (1 GPU)"},
        "roofline": {
            "kernel": f"gemm_fp8_pp<{shape.epilogue}>",
            "timing": ("HIP events around each dq_linear_fp8 call on its stream; a call is one "
                       "launch, or two when the tiles left after the full rounds run as "
                       "256 x 128 halves (the second, narrow launch follows on the stream)"),
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(gemm_ms * 1e3, 2),
            "algorithmic_flop_per_launch": shape.flops,
        },
        "quantizer": {
            "kernel": "quant_rows_reg",
            "timing": "back-to-back launches over rotating inputs, HIP events around the loop",
            "bound": "hbm",
            "achieved": round(quant_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(quant_gbps / PEAK_HBM_GBPS, 4),
            "traffic": qtraffic,
            "avg_launch_us": round(quant_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": qbytes,
        },
    }
    if not args.no_modulate:
        Mm, Km = shape.M, shape.K
        mo = bench_modulate(Mm, Km, args.steps, args.sets)
        b_no_y = 3 * Mm * Km + 4 * Mm + 4 * Km       # read x, write codes and scales, read mod
        b_y = b_no_y + 2 * Mm * Km                   # plus the bf16 y
        gb_no_y = b_no_y / mo["no_y_us"] / 1e3
        gb_y = b_y / mo["y_us"] / 1e3
        log(f"LN+modulate+quantize {Mm}x{Km}: {mo['no_y_us']:.1f} us ({gb_no_y:.0f} GB/s), "
            f"with y {mo['y_us']:.1f} us ({gb_y:.0f} GB/s); unfused {mo['unfused_us']:.1f} us")
        res["ln_modulate_quantizer"] = {
            "kernel": "ln_mod_quant_rows",
            "timing": "back-to-back launches over rotating inputs, HIP events around the loop",
            "shape": [Mm, Km],
            "bound": "hbm",
            "achieved": round(gb_no_y, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(gb_no_y / PEAK_HBM_GBPS, 4),
            "traffic": stored_traffic("ln_modulate", w.name),
            "avg_launch_us": round(mo["no_y_us"], 2),
            "algorithmic_bytes_per_launch": b_no_y,
            "with_y": {"avg_launch_us": round(mo["y_us"], 2), "achieved": round(gb_y, 1),
                       "frac": round(gb_y / PEAK_HBM_GBPS, 4),
                       "algorithmic_bytes_per_launch": b_y},
            "unfused_torch_then_quantize_us": round(mo["unfused_us"], 2),
        }
    if not args.no_qkv:
        qk = bench_qkv(args.steps, min(args.warmup, 100), min(args.sets, 4))
        tf = qk["flops"] / qk["fused_us"] / 1e6
        log(f"QKV + norm + rotary {qk['shape']}: {qk['fused_us']:.1f} us ({tf:.0f} TFLOP/s); "
            f"bias epilogue {qk['plain_us']:.1f} us; unfused {qk['unfused_us']:.1f} us")
        res["qkv_linear"] = {
            "kernel": "gemm_fp8_pp<qkv>",
            "timing": "HIP events around each call, rotating inputs (1 or 2 launches per call)",
            "shape": qk["shape"], "heads": qk["heads"],
            "bound": "mfma",
            "achieved": round(tf, 1),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / PEAK_FP8_TFLOPS, 4),
            "traffic": stored_traffic("qkv", w.name),
            "avg_launch_us": round(qk["fused_us"], 2),
            "algorithmic_flop_per_launch": qk["flops"],
            "bias_epilogue_us": round(qk["plain_us"], 2),
            "unfused_torch_us": round(qk["unfused_us"], 2),
        }
    if not args.no_attention:
        at = bench_attention(args.steps, min(args.warmup, 50), 3)
        tf = at["flops"] / at["attn_us"] / 1e6
        # half the work on the FP8 matrix units (5.0 PF), half on bf16 (2.5 PF)
        mixed_peak = 4.0 / (2.0 / PEAK_FP8_TFLOPS + 2.0 / (PEAK_FP8_TFLOPS / 2))
        log(f"FP8 attention H={at['H']} S={at['S']}: {at['attn_us']:.1f} us ({tf:.0f} TFLOP/s); "
            f"q/k/v quantization {at['quant_us']:.1f} us; torch bf16 SDPA {at['sdpa_us']:.1f} us")
        res["attention"] = {
            "kernel": "attn_fp8",
            "timing": "HIP events around each call, rotating inputs",
            "shape": {"heads": at["H"], "tokens": at["S"], "head_dim": 128},
            "bound": "mfma",
            "achieved": round(tf, 1),
            "peak": round(mixed_peak, 1),
            "peak_note": "q k^T on FP8 (5.0 PF), p v on bf16 (2.5 PF): 4 / (2/5.0 + 2/2.5) PF",
            "unit": "TFLOP/s",
            "frac": round(tf / mixed_peak, 4),
            "traffic": stored_traffic("attention", w.name),
            "avg_launch_us": round(at["attn_us"], 2),
            "algorithmic_flop_per_launch": at["flops"],
            "qkv_quantization_us": round(at["quant_us"], 2),
            "torch_bf16_sdpa_us": round(at["sdpa_us"], 2),
        }
    if not args.no_mx:
        mx = bench_mx(shape, w.seed, args.steps, min(args.warmup, 100), min(args.sets, 4))
        tf = mx["flops"] / mx["gemm_us"] / 1e6
        gbq = mx["quant_bytes"] / mx["quant_us"] / 1e3
        log(f"MX (block-scaled) FP8 {mx['shape']} {mx['epilogue']}: GEMM {mx['gemm_us']:.1f} us "
            f"({tf:.0f} TFLOP/s), quantizer {mx['quant_us']:.1f} us ({gbq:.0f} GB/s); per-row FP8 "
            f"GEMM {mx['rowwise_us']:.1f} us")
        res["mx_linear"] = {
            "kernel": "gemm_mx<%s>" % mx["epilogue"],
            "timing": "HIP events around each call, rotating inputs",
            "shape": mx["shape"], "epilogue": mx["epilogue"],
            "bound": "mfma",
            "achieved": round(tf, 1),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / PEAK_FP8_TFLOPS, 4),
            "traffic": stored_traffic("mx_linear", w.name),
            "avg_launch_us": round(mx["gemm_us"], 2),
            "algorithmic_flop_per_launch": mx["flops"],
            "quantizer_us": round(mx["quant_us"], 2),
            "quantizer_gbps": round(gbq, 1),
            "rowwise_fp8_gemm_us": round(mx["rowwise_us"], 2),
        }
    if not args.no_dit:
        log("DiT step: generating 228 distinct FP8 weights on the device")
        d = bench_dit_step(args.dit_steps, 2)
        floor_ms = 13.74
        res["dit_step"] = {"workload": "flux-dit-step-1024", "linears": d["linears"],
                           "ms": round(d["ms"], 3), "tflops": round(d["tflops"], 1),
                           "roofline_floor_ms": floor_ms,
                           "frac": round(floor_ms / d["ms"], 4), "steps": args.dit_steps}
        log(f"DiT step linears: {d['ms']:.2f} ms ({d['tflops']:.0f} TFLOP/s)")
    if not args.no_cpu_baseline:
        log("CPU baseline: timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(shape, w.seed)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
