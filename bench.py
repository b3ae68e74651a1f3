"""Benchmark of the FP8 dynamic-quant linear path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default workload is the whole linear sequence of one 1024^2 FLUX-dev denoising step: 228
dynamically quantized linears (19 double-stream blocks with an image and a text stream, 38
single-stream blocks), each a per-token FP8 quantization of its bf16 activations
(dq_quantize_fp8) followed by the FP8 GEMM with its fused epilogue (dq_linear_fp8), with distinct
weights per block (8.6 GB of FP8 codes, quantized once off the timed path). A step is one pass
over that sequence; W untimed steps, then K timed steps between two HIP events on the stream.
`value` is the step's TFLOP/s; `roofline` is the step's dominant kernel, the GEMM of the
single-stream blocks' first linear (4608 x 3072 -> 21504), timed by an event pair around one of
its calls in each timed step.

After the headline, one leg per further configuration (the tiny linear, the MLP up-projection at
1024^2 and at 2048^2, the single-stream block pair), each quantize + GEMM over rotating buffer
sets; then the fused kernels (LayerNorm + modulation + quantize, the QKV projection with its
norm + rotary epilogue, FP8 attention, the block-scaled FP8 GEMM); then the CPU oracle timed on
the host on a bounded sample of the step, and on the four single configurations whole. Every
leg is timed as back-to-back calls with one event pair around the loop.
Every input is a seeded synthetic tensor resident in HBM before timing starts.

Prints one JSON line.
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
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense FP4 (and FP6) matrix peak
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E bandwidth
METRIC = "FP8-DQ linear TFLOP/s & % FP8 MFMA peak; quantizer GB/s; DiT-step linears ms"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "gemm": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "gemm_fp8.hip"),
    "quantize": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "quantize.hip"),
    "ln_modulate": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "quantize.hip"),
    "ln_modulate_y": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "quantize.hip"),
    "mx_quantize": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "gemm_mx.hip"),
    "qkv": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "gemm_fp8.hip"),
    "attention": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "attention.hip"),
    "mx_linear": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "gemm_fp8.hip"),
    "mxfp4_linear": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "gemm_fp8.hip"),
    "mxfp4_quantize": os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", "gemm_mx.hip"),
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


def loop_us(fn, sets, reps, warmup):
    """Microseconds per call of `fn` over `reps` back-to-back calls on the rotating `sets`, with one
    HIP event pair around the loop on the current stream (after `warmup` untimed calls and a
    synchronization). An event between two launches keeps the second from starting under the
    first one's tail and adds about 10 us of idle time, so calls are not bracketed one by one."""
    import torch
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(sets[i % len(sets)])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def bench_linear(shape, seed, steps, warmup, n_sets):
    """Time `steps` steps of quantize + linear. Returns a dict of timings."""
    import torch
    import fp8_dynamic_quant_amd as dq

    dev = torch.device("cuda:0")
    inp = linear_inputs(shape, seed)
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

    def quantize(st):
        dq.dq_quantize_fp8(st["x"], st["q"], st["sa"])

    def linear(st):
        if gated:   # in place on the residual stream, as in the model
            dq.dq_linear_fp8(st["q"], st["sa"], st["qw"], st["sw"], st["bias"], shape.epilogue,
                             st["gate"], st["res"], out=st["res"])
        else:
            dq.dq_linear_fp8(st["q"], st["sa"], st["qw"], st["sw"], st["bias"], shape.epilogue,
                             out=st["out"])

    def step(st):
        quantize(st)
        linear(st)

    wall0 = time.perf_counter()
    step_us = loop_us(step, sets, steps, warmup)
    wall = time.perf_counter() - wall0
    gemm_us = loop_us(linear, sets, steps, n_sets)
    # the quantizer's launches are short: four times as many
    quant_us = loop_us(quantize, sets, 4 * steps, n_sets)
    return {"step_us": step_us, "wall_s": wall, "gemm_us": gemm_us, "quant_us": quant_us}


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
        return loop_us(fn, sets, reps, max(reps // 4, n_sets))

    reps = 4 * steps
    return {"no_y_us": timed(lambda st: fused(st, False), reps),
            "y_us": timed(lambda st: fused(st, True), reps),
            "unfused_us": timed(unfused, max(reps // 4, 1))}


def bench_qkv(steps, warmup, n_sets, M=4096, K=3072, heads=24, seed=3200):
    """The attention input projection of the image stream at 1024^2 (4096 tokens, 3072 -> 3 x 24
    heads x 128) with the fused query/key RMS norm + rotary epilogue, against the same GEMM with
    the plain bias epilogue and, for context, that GEMM followed by the torch ops the fusion
    replaces; then the variant whose outputs leave as FP8 codes for the attention kernel, against
    the bf16 variant followed by the three quantizations it replaces.
    Back-to-back calls, one event pair around each loop; returns microseconds per call."""
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
                     "o8": (torch.empty((heads, M, 128), dtype=torch.uint8, device=dev),
                            torch.empty((heads, M), dtype=torch.float32, device=dev),
                            torch.empty((heads, M, 128), dtype=torch.uint8, device=dev),
                            torch.empty((heads, M), dtype=torch.float32, device=dev),
                            torch.empty((heads, 128, M), dtype=torch.uint8, device=dev),
                            torch.empty((heads, M), dtype=torch.float32, device=dev)),
                     "plain": torch.empty((M, N), dtype=torch.bfloat16, device=dev)})
    torch.cuda.synchronize()
    c2 = tcos[:, None, :]
    s2 = tsin[:, None, :]

    def fused(st):
        dq.dq_linear_qkv_fp8(st["q"], st["sa"], st["qw"], st["sw"], heads, st["b"], nqk, tcos,
                             tsin, out=st["o"])

    def plain(st):
        dq.dq_linear_fp8(st["q"], st["sa"], st["qw"], st["sw"], st["b"], "bias", out=st["plain"])

    def fused8(st):
        dq.dq_linear_qkv_fp8_attn(st["q"], st["sa"], st["qw"], st["sw"], heads, st["b"], nqk, tcos,
                                  tsin, out=st["o8"])

    def fused_then_quantize(st):
        fused(st)
        o8 = st["o8"]
        dq.dq_quantize_fp8(st["o"][0].view(heads * M, 128), q=o8[0].view(heads * M, 128),
                           scale=o8[1].view(heads * M))
        dq.dq_quantize_fp8(st["o"][1].view(heads * M, 128), q=o8[2].view(heads * M, 128),
                           scale=o8[3].view(heads * M))
        dq.dq_quantize_v_fp8(st["o"][2], vt=o8[4], v_scale=o8[5])

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
        return loop_us(fn, sets, n, warmup)

    return {"fused_us": timed(fused, steps), "plain_us": timed(plain, steps),
            "unfused_us": timed(unfused, max(steps // 4, 5)), "fp8_qk_us": timed(fused8, steps),
            "bf16_then_quantize_us": timed(fused_then_quantize, steps), "flops": 2 * M * N * K,
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
        return loop_us(fn, sets, n, warmup)

    attn = timed(lambda st: dq.dq_attention_fp8(*st["fp8"], out=st["out"]), steps)
    quant = timed(lambda st: dq.quantize_qkv_heads_fp8(*st["bf"]), steps)
    sdpa = timed(lambda st: F.scaled_dot_product_attention(*(t[None] for t in st["bf"])), steps)
    return {"attn_us": attn, "quant_us": quant, "sdpa_us": sdpa, "flops": 4 * H * S * S * 128,
            "H": H, "S": S}


def bench_mx(shape, seed, steps, warmup, n_sets):
    """The block-scaled (MX) paths on the benchmark linear's shape: per-32 block quantization of
    the activations, then the GEMM on the scaled matrix instruction with FP8 (E4M3) and with FP4
    (E2M1) elements, weights quantized once; the per-row FP8 GEMM on the same inputs is timed
    beside them. Back-to-back calls, one event pair around each loop; returns microseconds per
    call."""
    import torch
    import fp8_dynamic_quant_amd as dq

    dev = torch.device("cuda:0")
    M, K, N = shape.M, shape.K, shape.N
    inp = linear_inputs(shape, seed)
    epi = "gelu_tanh" if shape.epilogue == "gelu_tanh" else "bias"
    wb = to_dev_bf16(torch, inp.w, dev)
    qw, sw = dq.dq_quantize_mx_fp8(wb)
    qw4, sw4 = dq.dq_quantize_mxfp4(wb)
    rq, rs = dq.dq_quantize_weight_fp8(wb)
    bias = to_dev_bf16(torch, inp.bias, dev)
    xb = to_dev_bf16(torch, inp.x, dev)
    sets = []
    for i in range(n_sets):
        x = xb if i == 0 else (xb * (1.0 + 0.01 * i)).to(torch.bfloat16)
        qa, sa = dq.dq_quantize_mx_fp8(x)
        q4, s4 = dq.dq_quantize_mxfp4(x)
        q8, s8 = dq.dq_quantize_fp8(x)
        sets.append({"x": x, "qa": qa, "sa": sa, "q4": q4, "s4": s4, "q8": q8, "s8": s8,
                     "out": torch.empty((M, N), dtype=torch.bfloat16, device=dev)})
    torch.cuda.synchronize()

    def timed(fn, n):
        return loop_us(fn, sets, n, warmup)

    gemm = timed(lambda st: dq.dq_linear_mx_fp8(st["qa"], st["sa"], qw, sw, bias, epi,
                                                out=st["out"]), steps)
    # the quantizer's launches are short: four times as many
    quant = loop_us(lambda st: dq.dq_quantize_mx_fp8(st["x"], st["qa"], st["sa"]), sets,
                    4 * steps, warmup)
    rowwise = timed(lambda st: dq.dq_linear_fp8(st["q8"], st["s8"], rq, rs, bias, epi,
                                                out=st["out"]), steps)
    gemm4 = timed(lambda st: dq.dq_linear_mxfp4(st["q4"], st["s4"], qw4, sw4, bias, epi,
                                                out=st["out"]), steps)
    quant4 = loop_us(lambda st: dq.dq_quantize_mxfp4(st["x"], st["q4"], st["s4"]), sets,
                     4 * steps, warmup)
    return {"gemm_us": gemm, "quant_us": quant, "rowwise_us": rowwise,
            "fp4_gemm_us": gemm4, "fp4_quant_us": quant4,
            "flops": 2 * M * N * K, "shape": [M, K, N], "epilogue": epi,
            "quant_bytes": M * K * 2 + M * K + M * K // 32,
            "fp4_quant_bytes": M * K * 2 + M * K // 2 + M * K // 32}


def bench_text_stream(steps, n_sets=4, seed=21):
    """The double-stream linears at 1024^2 three ways, quantized inputs already in place: the
    image stream's linear alone (4096 rows), the text stream's alone (512 rows), and both in one
    segmented call over the joint 4608 rows. Weights rotate over n_sets sets (cold, as in the
    step). Back-to-back calls, one event pair around each loop; returns microseconds per call."""
    import torch
    import fp8_dynamic_quant_amd as dq
    from workloads import workload

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    w = workload("flux-dit-step-1024")
    res = {}
    for part in ("qkv", "proj", "fc1", "fc2"):
        img = next(l for l in w.linears if l.name == f"double.img.{part}")
        txt = next(l for l in w.linears if l.name == f"double.txt.{part}")
        K, N, epi = img.K, img.N, img.epilogue
        gated = epi == "gated_residual"
        x = torch.randn((4608, K), generator=gen, device=dev).to(torch.bfloat16)
        q, sa = dq.dq_quantize_fp8(x)
        del x
        sets = []
        for _ in range(n_sets):
            ws = []
            for _ in range(2):
                wt = (torch.randn((N, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
                qw, sw = dq.dq_quantize_weight_fp8(wt)
                del wt
                b = (torch.randn(N, generator=gen, device=dev) * 0.01).to(torch.bfloat16)
                g = (1 + 0.1 * torch.randn(N, generator=gen, device=dev)).to(torch.bfloat16)
                ws.append((qw, sw, b, g))
            sets.append(ws)
        out = torch.randn((4608, N), generator=gen, device=dev).to(torch.bfloat16)
        qt, st_, qi, si = q[:512], sa[:512], q[512:], sa[512:]
        ot, oi = out[:512], out[512:]

        def one(qq, ss, wsb, o):
            qw, sw, b, g = wsb
            dq.dq_linear_fp8(qq, ss, qw, sw, b, epi, g if gated else None, o if gated else None,
                             out=o)

        def joint(st):
            dq.dq_linear_fp8_segmented(q, sa, [512, 4096], [st[0][0], st[1][0]],
                                       [st[0][1], st[1][1]], [st[0][2], st[1][2]], epi,
                                       [st[0][3], st[1][3]] if gated else None,
                                       out if gated else None, out=out)

        def timed(fn):
            return loop_us(fn, sets, steps, 10)

        qt, st_, qi, si = qt.contiguous(), st_.contiguous(), qi.contiguous(), si.contiguous()
        ot, oi = ot.contiguous(), oi.contiguous()
        r = {"image_us": timed(lambda st: one(qi, si, st[1], oi)),
             "text_us": timed(lambda st: one(qt, st_, st[0], ot)),
             "joint_us": timed(joint)}
        r["text_marginal_us"] = r["joint_us"] - r["image_us"]
        r["separate_us"] = r["image_us"] + r["text_us"]
        r["flops_joint"] = img.flops + txt.flops
        res[part] = {k: (round(v, 2) if isinstance(v, float) else v) for k, v in r.items()}
        del sets, q, sa, out
        torch.cuda.empty_cache()
    return res


def linear_bytes(M, K, N, epilogue):
    """Compulsory HBM bytes of one FP8 GEMM + epilogue: both code matrices, the bf16 output, the
    scales, bias (and gate + residual when gated)."""
    b = M * K + N * K + 2 * M * N + 4 * M + 4 * N + 2 * N
    if epilogue == "gated_residual":
        b += 2 * M * N + 2 * N
    return b


def quantizer_bytes(M, K):
    """Algorithmic bytes of one per-row quantization: read bf16, write codes and fp32 scales."""
    return 3 * M * K + 4 * M


def linear_bytes_mxfp4(M, K, N, epilogue):
    """Compulsory HBM bytes of one MXFP4 GEMM + epilogue: both packed code matrices (K / 2 bytes
    a row), their scale bytes (K / 32 a row), the bf16 output, bias (and gate + residual)."""
    b = (M + N) * (K // 2 + K // 32) + 2 * M * N + 2 * N
    if epilogue == "gated_residual":
        b += 2 * M * N + 2 * N
    return b


def quantizer_bytes_mxfp4(M, K):
    """Algorithmic bytes of one MXFP4 quantization: read bf16, write packed codes and scale
    bytes."""
    return 2 * M * K + M * K // 2 + M * K // 32


FORMATS = {
    # weight quantizer, peak of the GEMM, its bytes, the activation quantizer's bytes
    "fp8": ("dq_quantize_weight_fp8", PEAK_FP8_TFLOPS, linear_bytes, quantizer_bytes),
    "mxfp4": ("dq_quantize_mxfp4", PEAK_FP4_TFLOPS, linear_bytes_mxfp4, quantizer_bytes_mxfp4),
}


def dit_floor_ms(w, fmt="fp8"):
    """Roofline floor of one step: per linear max(FLOP / matrix peak, bytes / HBM), plus every
    quantizer's bytes at HBM bandwidth."""
    _, peak, lbytes, qbytes = FORMATS[fmt]
    t = 0.0
    for l, r in zip(w.linears, w.repeat):
        t += r * max(l.flops / (peak * 1e12),
                     lbytes(l.M, l.K, l.N, l.epilogue) / (PEAK_HBM_GBPS * 1e9))
        t += r * qbytes(l.M, l.K) / (PEAK_HBM_GBPS * 1e9)
    return t * 1e3


def bench_dit_step(steps, warmup, breakdown_steps=2, focus="single.linear1", fmt="fp8"):
    """All linears of one 1024^2 FLUX-dev denoising step, distinct weights per block, timed end
    to end as one sequence on one stream: per double-stream block four calls over the joint
    sequence (512 text + 4096 image rows, one quantization and one segmented linear each, the
    text and image weights as two row segments), per single-stream block two (228 weights in
    152 quantize + linear pairs). fmt "fp8": per-row FP8 codes (dq_quantize_fp8,
    dq_linear_fp8[_segmented]); "mxfp4": block-scaled E2M1 (dq_quantize_mxfp4,
    dq_linear_mxfp4[_segmented]) on the same inputs.

    Each timed step carries one HIP event pair, around one call of `focus` (the step's dominant
    kernel; step k times its k-th call, cycling), on the stream the kernels run on. After them,
    `breakdown_steps` further steps carry event pairs around every call, for the per-call
    table."""
    import torch
    import fp8_dynamic_quant_amd as dq
    from workloads import dit_step_device_inputs, workload

    w = workload("flux-dit-step-1024")
    dev = torch.device("cuda:0")
    wq_name, peak, _, qbytes = FORMATS[fmt]
    fp4 = fmt == "mxfp4"
    calls, acts, residuals = dit_step_device_inputs(w, dev, getattr(dq, wq_name))
    quantize = dq.dq_quantize_mxfp4 if fp4 else dq.dq_quantize_fp8
    one_linear = dq.dq_linear_mxfp4 if fp4 else dq.dq_linear_fp8
    seg_linear = dq.dq_linear_mxfp4_segmented if fp4 else dq.dq_linear_fp8_segmented
    outs = {}
    qbuf = {}
    for c in calls:
        M, K, N = c["M"], c["K"], c["N"]
        if (M, K) not in qbuf:
            qbuf[(M, K)] = ((torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                             torch.empty((M, K // 32), dtype=torch.uint8, device=dev)) if fp4
                            else (torch.empty((M, K), dtype=torch.uint8, device=dev),
                                  torch.empty((M,), dtype=torch.float32, device=dev)))
        if c["epilogue"] != "gated_residual" and (M, N) not in outs:
            outs[(M, N)] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def linear(c, q, sa):
        segs = c["segments"]
        gated = c["epilogue"] == "gated_residual"
        out = residuals[c["residual"]] if gated else outs[(c["M"], c["N"])]
        if len(segs) == 1:
            s0 = segs[0]
            one_linear(q, sa, s0["qw"], s0["sw"], s0["bias"], c["epilogue"],
                       s0["gate"], out if gated else None, out=out)
        else:
            seg_linear(q, sa, [g["rows"] for g in segs], [g["qw"] for g in segs],
                       [g["sw"] for g in segs], [g["bias"] for g in segs], c["epilogue"],
                       [g["gate"] for g in segs] if gated else None,
                       out if gated else None, out=out)

    focus_at = [i for i, c in enumerate(calls) if c["name"] == focus]

    def run(marks=None, all_calls=False, pick=-1, pool=None):
        # events come from `pool`, created before the step is enqueued
        for i, c in enumerate(calls):
            q, sa = qbuf[(c["M"], c["K"])]
            timed_call = marks is not None and (all_calls or i == pick)
            e0 = None
            if timed_call and all_calls:
                e0 = pool.pop()
                e0.record()
            quantize(acts[c["act"]], q, sa)
            if timed_call:
                e1 = pool.pop()
                e1.record()
            linear(c, q, sa)
            if timed_call:
                e2 = pool.pop()
                e2.record()
                marks.append((c["name"], e0, e1, e2))

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    focus_marks = []
    pool = [ev() for _ in range(2 * steps)]
    t0, t1 = ev(), ev()
    t0.record()
    for k in range(steps):
        # one event pair per step, on a different call of the focus linear each step: an event
        # between two launches keeps the second from starting under the first one's tail, so a
        # pair around every call would itself lengthen the step (about 12 us per pair)
        run(focus_marks, pick=focus_at[k % len(focus_at)], pool=pool)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    focus_us = float(np.mean([a.elapsed_time(b) for _, _, a, b in focus_marks])) * 1e3

    marks = []
    pool = [ev() for _ in range(3 * len(calls) * breakdown_steps)]
    torch.cuda.synchronize()
    for _ in range(breakdown_steps):
        run(marks, all_calls=True, pool=pool)
    torch.cuda.synchronize()
    by = {}
    for name, e0, e1, e2 in marks:
        d = by.setdefault(name, {"quant": [], "gemm": []})
        d["quant"].append(e0.elapsed_time(e1) * 1e3)
        d["gemm"].append(e1.elapsed_time(e2) * 1e3)
    table = {}
    for c in calls:
        if c["name"] in table:
            table[c["name"]]["per_step"] += 1
            continue
        d = by[c["name"]]
        g_us, q_us = float(np.mean(d["gemm"])), float(np.mean(d["quant"]))
        tf = c["flops"] / g_us / 1e6
        qgb = qbytes(c["M"], c["K"]) / q_us / 1e3
        table[c["name"]] = {
            "shape": [c["M"], c["K"], c["N"]], "epilogue": c["epilogue"],
            "segments": [g["rows"] for g in c["segments"]], "per_step": 1,
            "gemm_us": round(g_us, 2), "gemm_tflops": round(tf, 1),
            "gemm_frac": round(tf / peak, 4),
            "quant_us": round(q_us, 2), "quant_gbps": round(qgb, 1),
            "quant_frac": round(qgb / PEAK_HBM_GBPS, 4),
        }
        if not fp4:
            table[c["name"]]["gemm_traffic"] = stored_traffic(
                "gemm", f"flux-dit-step-1024/{c['name']}")
            table[c["name"]]["quant_traffic"] = stored_traffic(
                "quantize", f"flux-dit-step-1024/{c['name']}")
    for row in table.values():
        row["ms_per_step"] = round(row["per_step"] * (row["gemm_us"] + row["quant_us"]) / 1e3, 3)
    return {"ms": ms, "tflops": w.flops_per_step / ms / 1e9, "calls": len(calls),
            "linears": sum(len(c["segments"]) for c in calls),
            "weight_bytes": sum(g["qw"].numel() for c in calls for g in c["segments"]),
            "flops": w.flops_per_step, "floor_ms": dit_floor_ms(w, fmt), "focus": focus,
            "focus_gemm_us": focus_us, "focus_calls": len(focus_marks), "breakdown": table}


_INPUTS = {}


def linear_inputs(shape, seed):
    """Seeded host inputs of one linear, drawn once per (shape, seed) and shared by the GPU legs
    and the CPU baseline."""
    from workloads import make_linear_inputs
    key = (shape, seed)
    if key not in _INPUTS:
        _INPUTS[key] = make_linear_inputs(shape, seed)
    return _INPUTS[key]


def blas_threads():
    from threadpoolctl import threadpool_info
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    return int(max([i.get("num_threads", 1) for i in blas] or [1]))


def cpu_oracle_linear(shape, seed):
    """Time the oracle on one linear as it stands: quantize x per token, then the exact float64
    contraction and the epilogue (weights quantized beforehand, untimed). Returns seconds for the
    quantization and for the linear."""
    from oracle import linear_ref, quantize_rows
    from workloads import bf16_bits_to_f32

    inp = linear_inputs(shape, seed)
    qw, sw = quantize_rows(bf16_bits_to_f32(inp.w))
    x = bf16_bits_to_f32(inp.x)
    bias = bf16_bits_to_f32(inp.bias)
    gate = None if inp.gate is None else bf16_bits_to_f32(inp.gate)
    res = None if inp.residual is None else bf16_bits_to_f32(inp.residual)
    t0 = time.perf_counter()
    q, sa = quantize_rows(x)
    t1 = time.perf_counter()
    y = linear_ref(q, sa, qw, sw, bias, shape.epilogue, gate, res)
    t2 = time.perf_counter()
    del y
    return t1 - t0, t2 - t1


def cpu_baseline_dit():
    """The oracle on a bounded sample of the DiT step: each of its 10 linear shapes once, whole
    (one block's worth: the four double-stream linears of the image and of the text stream, the
    two single-stream linears), drawn from the same distributions, each time multiplied by the
    shape's multiplicity per step (19 or 38)."""
    from workloads import workload
    w = workload("flux-dit-step-1024")
    total, work = 0.0, 0.0
    for i, (l, rep) in enumerate(zip(w.linears, w.repeat)):
        tq, tl = cpu_oracle_linear(l, 100 + i)
        work += tq + tl
        total += rep * (tq + tl)
    threads = blas_threads()
    return {
        "value": round(w.flops_per_step / total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"each of the step's 10 linear shapes once, whole: quantize x + exact float64 "
                   f"contraction + epilogue, times its multiplicity (19 or 38) to one "
                   f"228-linear step; elementwise NumPy single-threaded, BLAS with {threads} "
                   f"threads; {work:.1f} s of CPU work"),
        "seconds_per_step": round(total, 2),
        "host_cpus_visible": os.cpu_count(),
    }


def cpu_oracle_configs(configs):
    """The oracle timed on whole configurations (every linear of each), as it stands."""
    res = {}
    for name, w in configs:
        t = 0.0
        parts = {}
        for l in w.linears:
            tq, tl = cpu_oracle_linear(l, w.seed)
            parts[l.name] = {"quant_s": round(tq, 3), "linear_s": round(tl, 3)}
            t += tq + tl
        flops = sum(l.flops for l in w.linears)
        res[name] = {"seconds": round(t, 3), "tflops": round(flops / t / 1e12, 6), "parts": parts}
        log(f"CPU oracle {name}: {t:.2f} s ({flops / t / 1e12:.4f} TFLOP/s)")
    return res


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


def linear_leg(shape, seed, steps, warmup, n_sets, traffic_key=None):
    """Quantize + GEMM of one linear (bench_linear) as a JSON object: the quantizer against HBM
    bandwidth, the GEMM against the FP8 matrix peak."""
    r = bench_linear(shape, seed, steps, warmup, n_sets)
    step_ms = r["step_us"] / 1e3
    gemm_ms = r["gemm_us"] / 1e3
    quant_ms = r["quant_us"] / 1e3
    qbytes = quantizer_bytes(shape.M, shape.K)
    tf = shape.flops / gemm_ms / 1e9
    gb = qbytes / quant_ms / 1e6
    log(f"{shape.name} {shape.M}x{shape.K}->{shape.N} {shape.epilogue}: "
        f"step {step_ms * 1e3:.1f} us; quantize {quant_ms * 1e3:.2f} us ({gb:.0f} GB/s), "
        f"GEMM {gemm_ms * 1e3:.1f} us ({tf:.0f} TFLOP/s)")
    return {
        "shape": [shape.M, shape.K, shape.N], "epilogue": shape.epilogue,
        "step_us": round(step_ms * 1e3, 2),
        "gemm": {"kernel": f"gemm_fp8_pp<{shape.epilogue}>", "bound": "mfma",
                 "avg_launch_us": round(gemm_ms * 1e3, 2), "achieved": round(tf, 1),
                 "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                 "algorithmic_flop_per_launch": shape.flops,
                 "traffic": stored_traffic("gemm", traffic_key) if traffic_key else None},
        "quantizer": {"kernel": "quant_rows", "bound": "hbm",
                      "avg_launch_us": round(quant_ms * 1e3, 2), "achieved": round(gb, 1),
                      "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gb / PEAK_HBM_GBPS, 4),
                      "algorithmic_bytes_per_launch": qbytes,
                      "traffic": stored_traffic("quantize", traffic_key) if traffic_key else None},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="flux-dit-step-1024",
                    help="flux-dit-step-1024 (the whole step) or a single-linear workload")
    ap.add_argument("--linear", type=int, default=0, help="index of the linear in the workload")
    ap.add_argument("--sets", type=int, default=6, help="rotating input/output buffer sets")
    ap.add_argument("--leg-steps", type=int, default=30, help="timed calls per leg")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-text-stream", action="store_true")
    ap.add_argument("--no-modulate", action="store_true")
    ap.add_argument("--no-qkv", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-mx", action="store_true")
    ap.add_argument("--no-dit-mxfp4", action="store_true",
                    help="skip the step's MXFP4 variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cpu-configs", action="store_true")
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
    import fp8_dynamic_quant_amd as dq  # noqa: F401  (fails loudly when libdq.so is missing)

    if args.calibrate_copy:
        calibrate_copy()

    w = workload(args.workload)
    res = {"metric": METRIC}
    ls = args.leg_steps
    if w.name == "flux-dit-step-1024":
        log(f"DiT step: drawing 228 distinct weights on the device; warmup {args.warmup}, "
            f"steps {args.steps}")
        d = bench_dit_step(args.steps, args.warmup)
        focus = next(l for l in w.linears if l.name == d["focus"])
        ftf = focus.flops / d["focus_gemm_us"] / 1e6
        log(f"DiT step linears: {d['ms']:.3f} ms ({d['tflops']:.0f} TFLOP/s; floor "
            f"{d['floor_ms']:.2f} ms); {d['focus']} GEMM {d['focus_gemm_us']:.1f} us "
            f"({ftf:.0f} TFLOP/s)")
        for name, row in d["breakdown"].items():
            log(f"  {name:16s} x{row['per_step']} {row['segments']}: GEMM {row['gemm_us']:7.1f} us "
                f"({row['gemm_tflops']:6.0f} TFLOP/s)  quantize {row['quant_us']:6.1f} us "
                f"({row['quant_gbps']:5.0f} GB/s)  -> {row['ms_per_step']:.2f} ms/step")
        res.update({
            "value": round(d["tflops"], 3), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(d["ms"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8_e4m3 (fp32 accumulate, bf16 in/out)", "data": "synthetic",
            "config": {"workload": w.name, "linears_per_step": d["linears"],
                       "launch_pairs_per_step": d["calls"],
                       "flop_per_step": d["flops"], "weight_bytes_fp8": d["weight_bytes"],
                       "parallelism": "none (1 GPU)"},
            "roofline": {
                "kernel": f"gemm_fp8_pp<bias> on {d['focus']} {list(focus_shape(focus))}",
                "timing": (f"HIP event pair around one {d['focus']} dq_linear_fp8 call in each "
                           f"timed step (a different block's call each step, "
                           f"{d['focus_calls']} calls), on the stream the kernels run on"),
                "bound": "mfma", "achieved": round(ftf, 2), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ftf / PEAK_FP8_TFLOPS, 4),
                "traffic": stored_traffic("gemm", f"flux-dit-step-1024/{d['focus']}"),
                "avg_launch_us": round(d["focus_gemm_us"], 2),
                "algorithmic_flop_per_launch": focus.flops,
            },
            "dit_step": {"ms": round(d["ms"], 4), "tflops": round(d["tflops"], 1),
                         "roofline_floor_ms": round(d["floor_ms"], 3),
                         "frac": round(d["floor_ms"] / d["ms"], 4),
                         "breakdown_timing": ("event pairs around every call of 2 further "
                                              "steps; a double-block call covers the text and "
                                              "the image stream (two row segments)"),
                         "breakdown": d["breakdown"]},
        })
    else:
        shape = w.linears[args.linear]
        log(f"workload {w.name}[{args.linear}] M={shape.M} K={shape.K} N={shape.N} "
            f"epilogue={shape.epilogue}; warmup {args.warmup}, steps {args.steps}")
        leg = linear_leg(shape, w.seed, args.steps, args.warmup, args.sets,
                         f"{w.name}/{shape.name}")
        ms_per_step = leg["step_us"] / 1e3
        res.update({
            "value": round(shape.flops / ms_per_step / 1e9, 3), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate, bf16 in/out)",
            "data": "synthetic",
            "config": {"workload": w.name, "linear": shape.name, "M": shape.M, "K": shape.K,
                       "N": shape.N, "epilogue": shape.epilogue, "rotating_sets": args.sets,
                       "parallelism": "none (1 GPU)"},
            "roofline": dict(leg["gemm"], timing=(
                "back-to-back dq_linear_fp8 calls over rotating inputs (one launch each, or two "
                "when the left-over tiles run as 256 x 128 halves), one HIP event pair around "
                "the loop on the stream the kernels run on")),
            "quantizer": leg["quantizer"],
        })
    if not args.no_dit_mxfp4 and w.name == "flux-dit-step-1024":
        torch.cuda.empty_cache()
        log("DiT step, MXFP4 variant: the same weights and activations in block-scaled E2M1")
        d4 = bench_dit_step(args.steps, args.warmup, fmt="mxfp4")
        ftf4 = focus.flops / d4["focus_gemm_us"] / 1e6
        log(f"DiT step linears, MXFP4: {d4['ms']:.3f} ms ({d4['tflops']:.0f} TFLOP/s; floor "
            f"{d4['floor_ms']:.2f} ms); {d4['focus']} GEMM {d4['focus_gemm_us']:.1f} us "
            f"({ftf4:.0f} TFLOP/s); {d['ms'] / d4['ms']:.2f}x the FP8 step")
        for name, row in d4["breakdown"].items():
            log(f"  {name:16s} x{row['per_step']} {row['segments']}: GEMM {row['gemm_us']:7.1f} us "
                f"({row['gemm_tflops']:6.0f} TFLOP/s)  quantize {row['quant_us']:6.1f} us "
                f"({row['quant_gbps']:5.0f} GB/s)  -> {row['ms_per_step']:.2f} ms/step")
        res["dit_step_mxfp4"] = {
            "ms": round(d4["ms"], 4), "tflops": round(d4["tflops"], 1),
            "speedup_vs_fp8_step": round(d["ms"] / d4["ms"], 3),
            "roofline_floor_ms": round(d4["floor_ms"], 3),
            "frac": round(d4["floor_ms"] / d4["ms"], 4),
            "weight_bytes_codes": d4["weight_bytes"],
            "focus": {"linear": d4["focus"], "avg_launch_us": round(d4["focus_gemm_us"], 2),
                      "achieved": round(ftf4, 1), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(ftf4 / PEAK_FP4_TFLOPS, 4)},
            "timing": ("as the FP8 step: one HIP event pair around one focus call per timed "
                       "step, event pairs around every call of 2 further steps"),
            "breakdown": d4["breakdown"],
        }
        del d4
        torch.cuda.empty_cache()
    if not args.no_text_stream and w.name == "flux-dit-step-1024":
        ts = bench_text_stream(ls)
        for part, r in ts.items():
            log(f"double.{part}: image {r['image_us']:.1f} us, text {r['text_us']:.1f} us, "
                f"separate {r['separate_us']:.1f} us; joint segmented {r['joint_us']:.1f} us "
                f"(text adds {r['text_marginal_us']:.1f} us)")
        res["text_stream"] = {"timing": "back-to-back calls, weights rotating over 4 sets, codes "
                                        "already quantized, one HIP event pair around the loop",
                              "linears": ts}
    cfg_names = ["tiny-64x256x512", "flux-mlp-up-1024", "flux-single-block-1024",
                 "flux-mlp-up-2048"]
    if not args.no_configs and w.name == "flux-dit-step-1024":
        res["configs"] = {}
        for name in cfg_names:
            cw = workload(name)
            res["configs"][name] = {l.name: linear_leg(l, cw.seed, ls, 20, args.sets,
                                                       f"{name}/{l.name}")
                                    for l in cw.linears}
    shape = workload("flux-mlp-up-1024").linears[0]
    seed = workload("flux-mlp-up-1024").seed
    if not args.no_modulate:
        Mm, Km = shape.M, shape.K
        mo = bench_modulate(Mm, Km, ls, args.sets)
        b_no_y = 3 * Mm * Km + 4 * Mm + 4 * Km       # read x, write codes and scales, read mod
        b_y = b_no_y + 2 * Mm * Km                   # plus the bf16 y
        gb_no_y = b_no_y / mo["no_y_us"] / 1e3
        gb_y = b_y / mo["y_us"] / 1e3
        log(f"LN+modulate+quantize {Mm}x{Km}: {mo['no_y_us']:.1f} us ({gb_no_y:.0f} GB/s), "
            f"with y {mo['y_us']:.1f} us ({gb_y:.0f} GB/s); unfused {mo['unfused_us']:.1f} us")
        res["ln_modulate_quantizer"] = {
            "kernel": "ln_mod_quant_rows",
            "timing": "back-to-back launches over rotating inputs, HIP events around the loop",
            "shape": [Mm, Km], "bound": "hbm", "achieved": round(gb_no_y, 1),
            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gb_no_y / PEAK_HBM_GBPS, 4),
            "traffic": stored_traffic("ln_modulate", "fused-1024"),
            "avg_launch_us": round(mo["no_y_us"], 2), "algorithmic_bytes_per_launch": b_no_y,
            "with_y": {"avg_launch_us": round(mo["y_us"], 2), "achieved": round(gb_y, 1),
                       "frac": round(gb_y / PEAK_HBM_GBPS, 4),
                       "algorithmic_bytes_per_launch": b_y,
                       "traffic": stored_traffic("ln_modulate_y", "fused-1024")},
            "unfused_torch_then_quantize_us": round(mo["unfused_us"], 2),
        }
    if not args.no_qkv:
        qk = bench_qkv(ls, 20, min(args.sets, 4))
        tf = qk["flops"] / qk["fused_us"] / 1e6
        log(f"QKV + norm + rotary {qk['shape']}: {qk['fused_us']:.1f} us ({tf:.0f} TFLOP/s); "
            f"bias epilogue {qk['plain_us']:.1f} us; unfused {qk['unfused_us']:.1f} us; "
            f"outputs as FP8 codes {qk['fp8_qk_us']:.1f} us (bf16 outputs then quantized: "
            f"{qk['bf16_then_quantize_us']:.1f} us)")
        res["qkv_linear"] = {
            "kernel": "gemm_fp8_pp<qkv>",
            "timing": ("back-to-back calls over rotating inputs (1 or 2 launches per call), one "
                       "HIP event pair around the loop"),
            "shape": qk["shape"], "heads": qk["heads"], "bound": "mfma",
            "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_FP8_TFLOPS, 4),
            "traffic": stored_traffic("qkv", "fused-1024"),
            "avg_launch_us": round(qk["fused_us"], 2),
            "algorithmic_flop_per_launch": qk["flops"],
            "bias_epilogue_us": round(qk["plain_us"], 2),
            "unfused_torch_us": round(qk["unfused_us"], 2),
            "fp8_outputs_us": round(qk["fp8_qk_us"], 2),
            "bf16_then_quantize_us": round(qk["bf16_then_quantize_us"], 2),
        }
    if not args.no_attention:
        at = bench_attention(ls, 20, 3)
        tf = at["flops"] / at["attn_us"] / 1e6
        # half the work on the FP8 matrix units (5.0 PF), half on bf16 (2.5 PF)
        mixed_peak = 4.0 / (2.0 / PEAK_FP8_TFLOPS + 2.0 / (PEAK_FP8_TFLOPS / 2))
        log(f"FP8 attention H={at['H']} S={at['S']}: {at['attn_us']:.1f} us ({tf:.0f} TFLOP/s); "
            f"q/k/v quantization {at['quant_us']:.1f} us; torch bf16 SDPA {at['sdpa_us']:.1f} us")
        res["attention"] = {
            "kernel": "attn_fp8",
            "timing": "back-to-back calls over rotating inputs, one HIP event pair around the loop",
            "shape": {"heads": at["H"], "tokens": at["S"], "head_dim": 128},
            "bound": "mfma", "achieved": round(tf, 1), "peak": round(mixed_peak, 1),
            "peak_note": "q k^T on FP8 (5.0 PF), p v on bf16 (2.5 PF): 4 / (2/5.0 + 2/2.5) PF",
            "unit": "TFLOP/s", "frac": round(tf / mixed_peak, 4),
            "traffic": stored_traffic("attention", "fused-1024"),
            "avg_launch_us": round(at["attn_us"], 2),
            "algorithmic_flop_per_launch": at["flops"],
            "qkv_quantization_us": round(at["quant_us"], 2),
            "torch_bf16_sdpa_us": round(at["sdpa_us"], 2),
        }
    if not args.no_mx:
        mx = bench_mx(shape, seed, ls, 20, min(args.sets, 4))
        tf = mx["flops"] / mx["gemm_us"] / 1e6
        gbq = mx["quant_bytes"] / mx["quant_us"] / 1e3
        log(f"MX (block-scaled) FP8 {mx['shape']} {mx['epilogue']}: GEMM {mx['gemm_us']:.1f} us "
            f"({tf:.0f} TFLOP/s), quantizer {mx['quant_us']:.1f} us ({gbq:.0f} GB/s); per-row FP8 "
            f"GEMM {mx['rowwise_us']:.1f} us")
        res["mx_linear"] = {
            "kernel": "gemm_fp8_pp<mx_%s>" % mx["epilogue"],
            "timing": "back-to-back calls over rotating inputs, one HIP event pair around the loop",
            "shape": mx["shape"], "epilogue": mx["epilogue"], "bound": "mfma",
            "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_FP8_TFLOPS, 4),
            "traffic": stored_traffic("mx_linear", "fused-1024"),
            "avg_launch_us": round(mx["gemm_us"], 2),
            "algorithmic_flop_per_launch": mx["flops"],
            "quantizer_us": round(mx["quant_us"], 2),
            "quantizer_gbps": round(gbq, 1),
            "quantizer_traffic": stored_traffic("mx_quantize", "fused-1024"),
            "rowwise_fp8_gemm_us": round(mx["rowwise_us"], 2),
        }
        tf4 = mx["flops"] / mx["fp4_gemm_us"] / 1e6
        gb4 = mx["fp4_quant_bytes"] / mx["fp4_quant_us"] / 1e3
        log(f"MXFP4 (block-scaled E2M1) {mx['shape']} {mx['epilogue']}: GEMM "
            f"{mx['fp4_gemm_us']:.1f} us ({tf4:.0f} TFLOP/s), quantizer {mx['fp4_quant_us']:.1f} us "
            f"({gb4:.0f} GB/s)")
        res["mxfp4_linear"] = {
            "kernel": "gemm_fp8_pp<mx4_%s>" % mx["epilogue"],
            "timing": ("back-to-back calls over rotating inputs, one HIP event pair around the "
                       "loop"),
            "shape": mx["shape"], "epilogue": mx["epilogue"], "bound": "mfma",
            "achieved": round(tf4, 1), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf4 / PEAK_FP4_TFLOPS, 4),
            "traffic": stored_traffic("mxfp4_linear", "fused-1024"),
            "avg_launch_us": round(mx["fp4_gemm_us"], 2),
            "algorithmic_flop_per_launch": mx["flops"],
            "quantizer_us": round(mx["fp4_quant_us"], 2),
            "quantizer_gbps": round(gb4, 1),
            "quantizer_algorithmic_bytes": mx["fp4_quant_bytes"],
            "quantizer_traffic": stored_traffic("mxfp4_quantize", "fused-1024"),
        }
    if not args.no_cpu_baseline:
        log("CPU baseline: timing the oracle on the host")
        if w.name == "flux-dit-step-1024":
            res["cpu_baseline"] = cpu_baseline_dit()
        else:
            t = sum(cpu_oracle_linear(w.linears[args.linear], w.seed))
            fl = w.linears[args.linear].flops
            res["cpu_baseline"] = {"value": round(fl / t / 1e12, 6), "unit": "TFLOP/s",
                                   "cores": blas_threads(), "kind": "oracle",
                                   "sample": "the whole linear once (quantize x + exact float64 "
                                             "contraction + epilogue)",
                                   "seconds_per_step": round(t, 3),
                                   "host_cpus_visible": os.cpu_count()}
        log(f"CPU oracle: {res['cpu_baseline']['value']} TFLOP/s "
            f"({res['cpu_baseline']['seconds_per_step']} s per step)")
        if not args.no_cpu_configs:
            res["cpu_oracle_configs"] = cpu_oracle_configs(
                [(n, workload(n)) for n in cfg_names])
    print(json.dumps(res), flush=True)


def focus_shape(l):
    return (l.M, l.K, l.N)


if __name__ == "__main__":
    main()
