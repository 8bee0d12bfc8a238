"""Benchmark of the FP8 MoE prefill hot path on one MI355X.

A step is one MoE prefill layer -- activation quantisation, top-k routing and grouping,
the grouped gate|up GEMM with fused SwiGLU + requantisation, the grouped down GEMM, and
the weighted combine -- over the 4096-token workload (hidden 2048, 64 experts, top-8,
intermediate 768, packed-int4 experts with group-128 scales). Inputs are synthetic and
already resident in HBM; three copies of the weight bank and of the inputs are rotated so
the 151 MB bank cannot stay in the 256 MB Infinity Cache between steps.

Prints one JSON line: MoE prefill tokens/s for the whole layer (K steps timed with nothing
between the launches), plus the roofline of the dominant kernel (the grouped gate|up GEMM,
FP8 MFMA bound) from HIP events around each stage on the launch stream over a second pass
of the same K steps, and the CPU oracle timed on a bounded sample.

Also on the line: the layer against the sum of its stages' rooflines; the layer replayed
from HIP graphs (launch overhead removed; checked bit for bit against the eager layer);
the W8A8 dense projections at 2048 x 4096 x {6144, 4096} (per-tensor, row-wise and
block-128 scales); the layer with MXFP4 activations; the decode regime (16 tokens, M <= 16
projections; replayed from HIP graphs, with the eager host-issued times beside them); the skewed large layer (16384 tokens, hidden 4096, 128 Zipf-routed experts,
I = 1536) with its stage times and roofline fraction; the shader clock and the GEMM's HBM
bytes from the committed rocprofv3 counter runs (null once the kernel source differs);
the host CPU; and the depth stack (T=2048, L=8 by default, --stack 12 or 0): prefill
tokens/s of the whole forward (L layers of W8A8 q/k/v/o, causal GQA attention, router and
FP8 MoE, then the bf16 LM head), with its time against the sum of its parts' MFMA
rooflines (FP8 parts at the FP8 peak, bf16 parts at the bf16 peak).

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline] [--no-dense]
                    [--no-skewed] [--no-mxfp4] [--no-decode] [--stack {0,8,12}]
                    [--stack-only] [--layer-only] [--decode-only]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "grouped FP8 expert GEMM TFLOP/s (% FP8 MFMA peak); MoE prefill tokens/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_gemm_gate_up_moe_prefill_traffic.json")
CLOCK_FILE = os.path.join(ROOT, "profiles", "grouped_gemm_moe_prefill_counters.json")
GEMM_SOURCES = [os.path.join(ROOT, "fp8_moe_prefill_amd", "csrc", n)
                for n in ("grouped_gemm.hip", "lds_dma.h", "common.h")]


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dense", action="store_true",
                    help="(default) time the W8A8 dense projections (2048 x 4096 x {6144, 4096})")
    ap.add_argument("--no-dense", action="store_true", help="skip the W8A8 dense projections")
    ap.add_argument("--no-skewed", action="store_true",
                    help="skip the skewed large layer (16384 tokens, hidden 4096, 128 experts)")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--stack", type=int, default=8, choices=[0, 8, 12],
                    help="also time the depth stack of this many layers (0: skip)")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the layer with MXFP4 activations")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-regime timings (16-token layer, M <= 16 projections)")
    ap.add_argument("--stack-only", action="store_true",
                    help="time only the depth stack (for profiling it alone)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode regime (16-token layer, M <= 16 projections): "
                         "for profiling it alone")
    ap.add_argument("--layer-only", action="store_true",
                    help="time only the 4096-token layer (no graph replay, clock sampling, "
                         "dense, MXFP4, decode, stack, skewed or CPU legs): for counter runs")
    args = ap.parse_args()
    if args.layer_only:
        args.no_dense = args.no_mxfp4 = args.no_decode = args.no_skewed = True
        args.no_cpu_baseline = True
        args.stack = 0
    return args


def source_hash(paths) -> str:
    """First 16 hex digits of the SHA-256 of the concatenated sources."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_per_launch():
    """HBM bytes per gate|up launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs, or None when the kernel source changed after they were taken."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != source_hash(GEMM_SOURCES):
        return None
    return d.get("hbm_bytes_per_launch")


def committed_clock():
    """Shader clock under the grouped GEMMs from the committed rocprofv3 counter run
    (SQ_BUSY_CYCLES per shader engine over the same dispatches' durations), or None when
    the kernel source changed after it was taken."""
    try:
        d = json.load(open(CLOCK_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != source_hash(GEMM_SOURCES):
        return None
    return {"mhz": d.get("sclk_mhz"), "method": d.get("method"), "source": d.get("source")}


def cpu_baseline(n_tokens: int, min_seconds: float = 10.0, max_reps: int = 5):
    """The NumPy oracle on the first n_tokens tokens of the same layer (same weights),
    repeated until about min_seconds of CPU work (bounded by max_reps)."""
    import numpy as np  # noqa: F401

    from oracle.moe import moe_layer
    from synth import CONFIGS, moe_inputs

    c = CONFIGS["moe_prefill"]
    inp = moe_inputs(c, T=n_tokens)
    reps, total = 0, 0.0
    while reps < max_reps and (reps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        moe_layer(inp["x"], inp["logits"], inp["w_gu"], inp["s_gu"], inp["w_dn"], inp["s_dn"], c.k)
        total += time.perf_counter() - t0
        reps += 1
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = len(os.sched_getaffinity(0))
    return {"value": reps * n_tokens / total, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"the NumPy fp64 oracle MoE layer on the first {n_tokens} of the 4096 "
                      f"tokens (all 64 experts), {reps} runs, {total:.1f} s"}


def layer_roofline_us(c) -> dict:
    """Per-stage rooflines of one MoE layer, max(FLOP / FP8 peak, bytes / HBM), in us:
    quant (bf16 in, e4m3 + scales + code sums out), routing (logits in, ids/weights and
    grouping out), gate|up (bank + gathered rows + scales in, codes + scales + sums out),
    down (bank + codes in, bf16 rows out), combine (rows + weights in, bf16 out)."""
    T, H, E, k, I = c.T, c.H, c.E, c.k, c.I
    R = T * k
    G = 128

    def us(flop, nbytes):
        return max(flop / (PEAK_FP8_TFLOPS * 1e6), nbytes / (PEAK_HBM_GBS * 1e3))

    bank_gu = E * 2 * I * H / 2 + E * 2 * I * (H / G) * 4
    bank_dn = E * H * I / 2 + E * H * (I / G) * 4
    st = {
        "quant": us(0, T * H * 2 + T * H + 2 * T * (H / G) * 4),
        "route": us(0, T * E * 4 + T * k * 8 + 2 * R * 4 + (E + 1) * 4),
        "gate_up": us(4.0 * R * H * I, bank_gu + R * H + 2 * R * (H / G) * 4 + R * I
                      + 2 * R * (I / G) * 4),
        "down": us(2.0 * R * I * H, bank_dn + R * I + 2 * R * (I / G) * 4 + R * H * 2),
        "combine": us(0, R * H * 2 + T * k * 8 + T * H * 2),
    }
    st["layer"] = sum(st.values())
    return st


def stack_flops(c):
    """Algorithmic FLOP of one stack forward, split by MFMA dtype: FP8 (q/k/v/o, experts)
    and bf16 (causal attention, router, LM head)."""
    T, H, d = c.T, c.H, c.head_dim
    nqkv = (c.n_q + 2 * c.n_kv) * d
    fp8 = 2.0 * T * H * nqkv + 2.0 * T * c.n_q * d * H + 6.0 * T * c.k * H * c.I
    attn = 4.0 * d * (T * (T + 1) / 2) * c.n_q  # q.k and p.v over the causal pairs
    bf16 = attn + 2.0 * T * H * c.E
    head = 2.0 * T * H * c.V
    return c.L * fp8, c.L * bf16 + head


# FreeToken PR #389, "Why": per-rank decode projections (N x K) at M = 1, 8, 16
DECODE_SHAPES = [(6656, 2560), (2560, 3072), (8192, 2560)]
ROT_DECODE = 16


def bench_decode(steps: int = 20):
    """W8A8 at decode sizes: the weight-streaming path, HBM-bound. Sixteen copies of the
    weight (272-336 MB, more than the 256 MB Infinity Cache) are rotated so every launch
    streams its weight from HBM; achieved GB/s counts weights + activations + output once."""
    import torch

    import fp8_moe_prefill_amd as f

    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(0)
    res = {}
    for (N, K) in DECODE_SHAPES:
        w = (torch.randn((N, K), generator=g) * 0.02).to(torch.bfloat16).to(dev)
        wq, sw = f.quantize_weight(w)
        ws = [(wq.clone(), sw.clone()) for _ in range(ROT_DECODE)]
        for M in (1, 8, 16):
            x = torch.randn((M, K), generator=g).to(torch.bfloat16).to(dev)
            xq, blk = f.fp8_quant_act(x, 0)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            for i in range(3):
                f.fp8_dense_gemm(xq, blk, ws[i % ROT_DECODE][0], ws[i % ROT_DECODE][1], out=y)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for i in range(steps):
                f.fp8_dense_gemm(xq, blk, ws[i % ROT_DECODE][0], ws[i % ROT_DECODE][1], out=y)
            b.record()
            torch.cuda.synchronize()
            us_eager = a.elapsed_time(b) / steps * 1e3
            # the same calls captured once in a HIP graph and replayed: the kernels' own time
            # (issued one by one from Python, a call this small is bound by the host)
            ref = y.clone()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for i in range(steps):
                    f.fp8_dense_gemm(xq, blk, ws[i % ROT_DECODE][0], ws[i % ROT_DECODE][1],
                                     out=y)
            gr.replay()
            torch.cuda.synchronize()
            if not torch.equal(y, ref):
                raise RuntimeError("decode W8A8 graph replay differs from the eager call")
            reps = 5
            a.record()
            for _ in range(reps):
                gr.replay()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / (reps * steps) * 1e3
            nbytes = N * K + M * K + 2 * M * N
            res[f"M{M}_N{N}_K{K}"] = {"us": us, "GBps": nbytes / (us * 1e-6) / 1e9,
                                      "frac_hbm": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                      "us_eager": us_eager}
    return res


def bench_stack(L: int, warmup: int, steps: int):
    """The depth stack forward (T=2048): prefill tokens/s, per-layer and LM-head times."""
    import numpy as np
    import torch

    import fp8_moe_prefill_amd as f
    from synth import CONFIGS, stack_inputs

    c = CONFIGS[f"stack_L{L}"]
    dev = torch.device("cuda:0")
    inp = stack_inputs(c)
    stack = f.DepthStack.from_host(inp, c.n_q, c.n_kv, c.head_dim, c.k, dev)
    x0 = torch.from_numpy(inp["x0"].view(np.int16)).to(dev).view(torch.bfloat16)
    del inp
    runner = f.StackRunner(stack, c.T, dev)
    for _ in range(max(warmup, 1)):
        runner.run(x0)
    torch.cuda.synchronize()

    def evp():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    t0, t1 = evp()
    t0.record()
    for _ in range(steps):
        runner.run(x0)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    # one more forward with per-part events (not part of the timed loop above)
    ev = {"layer": ([torch.cuda.Event(enable_timing=True) for _ in range(L)],
                    [torch.cuda.Event(enable_timing=True) for _ in range(L)]),
          "lm_head": evp()}
    runner.run(x0, events=ev)
    torch.cuda.synchronize()
    layer_us = [ev["layer"][0][i].elapsed_time(ev["layer"][1][i]) * 1e3 for i in range(L)]
    head_us = ev["lm_head"][0].elapsed_time(ev["lm_head"][1]) * 1e3
    f8, b16 = stack_flops(c)
    roof_us = (f8 / PEAK_FP8_TFLOPS + b16 / PEAK_BF16_TFLOPS) / 1e6
    return {"workload": f"stack_L{L}: {L} layers, T={c.T}, hidden {c.H}, {c.n_q}/{c.n_kv} heads "
                        f"of {c.head_dim}, W8A8 q/k/v/o, causal GQA attention, FP8 MoE "
                        f"(E={c.E}, top-{c.k}, I={c.I}), bf16 LM head V={c.V}",
            "prefill_tokens_per_s": c.T / (ms * 1e-3), "ms_per_forward": ms, "steps": steps,
            "layer_us_mean": float(np.mean(layer_us)), "lm_head_us": head_us,
            "tflops": (f8 + b16) / (ms * 1e-3) / 1e12,
            "roofline_us": roof_us, "frac_roofline": roof_us / (ms * 1e3)}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (--gpus {args.gpus} requested); "
              "the multi-GPU expert-parallel path is not built", file=sys.stderr)
        sys.exit(2)

    if args.stack_only:
        st = bench_stack(args.stack or 8, args.warmup, args.steps)
        print(json.dumps({"metric": "depth stack prefill tokens/s", "value":
                          st["prefill_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                          "steps": st["steps"], "warmup": args.warmup,
                          "ms_per_step": st["ms_per_forward"], "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
                          "data": "synthetic", "config": {"workload": st["workload"]},
                          "stack": st}))
        return

    import numpy as np
    import torch

    import fp8_moe_prefill_amd as f
    from synth import CONFIGS, dense_inputs, moe_inputs

    dev = torch.device("cuda:0")
    c = CONFIGS["moe_prefill"]
    ROT = 3
    xs, lgs, banks = [], [], []
    for r in range(ROT):
        inp = moe_inputs(c, seed=r)
        xs.append(torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16))
        lgs.append(torch.from_numpy(inp["logits"]).to(dev))
        banks.append(f.ExpertBank.from_host(inp, dev))
    runner = f.MoELayerRunner(c.T, c.H, c.E, c.k, c.I, dev)
    R = c.T * c.k

    if args.decode_only:
        d = bench_decode_regime(c, xs, lgs, banks, dev)
        print(json.dumps({"metric": "decode MoE layer us (16 tokens)",
                          "value": d["decode_moe"]["us_per_layer"], "unit": "us",
                          "n_gpus": 1, "steps": 30, "warmup": 3,
                          "ms_per_step": d["decode_moe"]["us_per_layer"] * 1e-3,
                          "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
                          "dtype": "e4m3", "data": "synthetic",
                          "config": {"workload": "decode_moe: the 64-expert layer (hidden "
                                                 "2048, top-8, intermediate 768) at 16 tokens"},
                          **d}))
        return

    for i in range(args.warmup):
        runner.run(xs[i % ROT], lgs[i % ROT], banks[i % ROT])
    torch.cuda.synchronize()

    ms_step, per = time_layer(runner, xs, lgs, banks, args.steps)

    flop_gu = 4.0 * R * c.H * c.I
    flop_dn = 2.0 * R * c.I * c.H
    gu_tflops = flop_gu / (per["gate_up"] * 1e-3) / 1e12
    gemm_tflops = (flop_gu + flop_dn) / ((per["gate_up"] + per["down"]) * 1e-3) / 1e12
    traffic = traffic_per_launch()

    out = {
        "metric": METRIC,
        "value": c.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": "moe_prefill: one MoE prefill layer, T=4096 tokens, hidden 2048, "
                               "64 experts, top-8, intermediate 768 (SwiGLU), packed int4 "
                               "experts with group-128 fp32 scales, e4m3 activations with "
                               "per-(token,128) scales",
                   "tokens": c.T, "hidden": c.H, "experts": c.E, "top_k": c.k,
                   "intermediate": c.I, "weight_banks_rotated": ROT},
        "grouped_gemm": {"tflops": gemm_tflops, "frac_fp8_peak": gemm_tflops / PEAK_FP8_TFLOPS,
                         "gate_up_us": per["gate_up"] * 1e3, "down_us": per["down"] * 1e3},
        "stages_us": {s: v * 1e3 for s, v in per.items()},
        "roofline": {"kernel": "grouped_gemm gate|up (+SwiGLU+requant)", "bound": "mfma",
                     "achieved": gu_tflops, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": gu_tflops / PEAK_FP8_TFLOPS, "traffic": traffic,
                     "algorithmic_flop_per_launch": flop_gu},
    }
    out["host_launch_us_per_step"] = getattr(runner, "host_us_per_step", None)
    roof = layer_roofline_us(c)
    out["layer_roofline"] = {"us": roof["layer"], "frac": roof["layer"] / (ms_step * 1e3),
                             "stages_us": {s: v for s, v in roof.items() if s != "layer"}}
    if args.layer_only:
        print(json.dumps(out))
        return
    try:
        out["graph_replay"] = {"ms_per_step": time_graph_replay(runner, xs, lgs, banks,
                                                                args.steps)}
        out["graph_replay"]["tokens_per_s"] = c.T / (out["graph_replay"]["ms_per_step"] * 1e-3)
    except RuntimeError as e:  # reported, never silently replaced by the eager number
        out["graph_replay"] = {"error": str(e)}
    out["sclk"] = committed_clock()
    out["host"] = host_info()

    if not args.no_dense:
        d = dense_inputs(CONFIGS["dense_w8a8"])
        x = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        res = {}
        for wn in ("w_qkv", "w_o"):
            w = torch.from_numpy(d[wn].view(np.int16)).to(dev).view(torch.bfloat16)
            wq, sw = f.quantize_weight(w)
            xq, blk = f.fp8_quant_act(x, 0)
            y = f.fp8_dense_gemm(xq, blk, wq, sw)
            for _ in range(3):
                f.fp8_dense_gemm(xq, blk, wq, sw, out=y)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(20):
                f.fp8_dense_gemm(xq, blk, wq, sw, out=y)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / 20 * 1e3
            fl = 2.0 * x.shape[0] * w.shape[0] * x.shape[1]
            res[wn] = {"us": us, "tflops": fl / (us * 1e-6) / 1e12,
                       "frac_fp8_peak": fl / (us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS}
            # row-wise activation scales (one per token) on the same projection
            xr, sr = f.fp8_quant_act(x, f.QUANT_ROW)
            yr = f.fp8_dense_gemm_rowwise(xr, sr, wq, sw)
            for _ in range(3):
                f.fp8_dense_gemm_rowwise(xr, sr, wq, sw, out=yr)
            a.record()
            for _ in range(20):
                f.fp8_dense_gemm_rowwise(xr, sr, wq, sw, out=yr)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / 20 * 1e3
            res[wn + "_rowwise"] = {"us": us, "tflops": fl / (us * 1e-6) / 1e12}
            # block-128 e4m3 weights with per-(token, 128) activation scales
            wb, wbs = f.fp8_quant_weight_block128(w)
            xg, xgs = f.fp8_quant_act(x, 128)
            yb = f.fp8_block_gemm(xg, xgs, wb, wbs)
            for _ in range(3):
                f.fp8_block_gemm(xg, xgs, wb, wbs, out=yb)
            a.record()
            for _ in range(20):
                f.fp8_block_gemm(xg, xgs, wb, wbs, out=yb)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / 20 * 1e3
            res[wn + "_block128"] = {"us": us, "tflops": fl / (us * 1e-6) / 1e12}
        out["dense_w8a8"] = res

    if not args.no_mxfp4:
        out["mxfp4_act"] = bench_mxfp4_layer(c, xs, lgs, args.warmup, min(args.steps, 30), dev)
    if not args.no_decode:
        out.update(bench_decode_regime(c, xs, lgs, banks, dev))
    if args.stack:
        out["stack"] = bench_stack(args.stack, args.warmup, min(args.steps, 20))

    if not args.no_skewed:
        del banks, runner
        torch.cuda.empty_cache()
        out["moe_skewed"] = bench_skewed(args.warmup, min(args.steps, 20), dev)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_tokens)
    print(json.dumps(out))


def time_graph_replay(runner, xs, lgs, banks, steps):
    """ms per layer step with each rotation's step captured once in a HIP graph and the
    graphs replayed (launch overhead gone); the graphs are checked bit for bit against an
    eager step on the same inputs."""
    import torch

    n = len(xs)
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n):  # warm the allocator on the capture stream
            runner.run(xs[i], lgs[i], banks[i])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            runner.run(xs[i], lgs[i], banks[i])
        graphs.append(g)
    torch.cuda.synchronize()
    graphs[0].replay()
    torch.cuda.synchronize()
    got = runner.out.clone()
    runner.run(xs[0], lgs[0], banks[0])
    torch.cuda.synchronize()
    if not torch.equal(got, runner.out):
        raise RuntimeError("graph replay differs from the eager layer")
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        graphs[i % n].replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def host_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_threads": len(os.sched_getaffinity(0))}


def bench_skewed(warmup: int, steps: int, dev) -> dict:
    """The skewed large layer (16384 tokens, hidden 4096, 128 experts with Zipf(1.2)
    routing and empty experts, top-8, I = 1536): layer time and per-stage times, the
    grouped GEMMs' rate against the FP8 peak and the layer against its roofline. Its
    1.2 GB bank does not fit the 256 MB Infinity Cache, so one bank is used."""
    import numpy as np
    import torch

    import fp8_moe_prefill_amd as f
    from synth import CONFIGS, moe_inputs

    c = CONFIGS["moe_skewed"]
    inp = moe_inputs(c)
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    lg = torch.from_numpy(inp["logits"]).to(dev)
    bank = f.ExpertBank.from_host(inp, dev)
    del inp
    runner = f.MoELayerRunner(c.T, c.H, c.E, c.k, c.I, dev)
    for _ in range(max(warmup, 1)):
        runner.run(x, lg, bank)
    torch.cuda.synchronize()
    ms, per = time_layer(runner, [x], [lg], [bank], steps)
    R = c.T * c.k
    fl_gu, fl_dn = 4.0 * R * c.H * c.I, 2.0 * R * c.I * c.H
    roof = layer_roofline_us(c)
    gu_tf = fl_gu / (per["gate_up"] * 1e-3) / 1e12
    dn_tf = fl_dn / (per["down"] * 1e-3) / 1e12
    tf = (fl_gu + fl_dn) / ((per["gate_up"] + per["down"]) * 1e-3) / 1e12
    return {"workload": "moe_skewed: T=16384 tokens, hidden 4096, 128 experts (Zipf 1.2 "
                        "router bias, some experts empty), top-8, intermediate 1536",
            "tokens_per_s": c.T / (ms * 1e-3), "ms_per_step": ms,
            "stages_us": {s: v * 1e3 for s, v in per.items()},
            "grouped_gemm": {"tflops": tf, "frac_fp8_peak": tf / PEAK_FP8_TFLOPS,
                             "gate_up_tflops": gu_tf, "down_tflops": dn_tf},
            "layer_roofline_us": roof["layer"],
            "frac_layer_roofline": roof["layer"] / (ms * 1e3)}


def time_layer(runner, xs, lgs, banks, steps):
    """(ms per layer step, {stage: ms}). The steps are timed twice: first with nothing
    between the launches but the launches themselves (the step time; a HIP event recorded
    between kernels costs several microseconds of GPU time here), then again with a pair of
    events around each stage on the launch stream (the per-stage and per-kernel times)."""
    import numpy as np
    import torch

    n = len(xs)
    stages = runner.STAGES
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    h0 = time.perf_counter()
    for i in range(steps):
        runner.run(xs[i % n], lgs[i % n], banks[i % n])
    host_us = (time.perf_counter() - h0) / steps * 1e6  # launch cost on the host per step
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    runner.host_us_per_step = host_us
    ev = [{s: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for s in stages} for _ in range(steps)]
    for i in range(steps):
        runner.run(xs[i % n], lgs[i % n], banks[i % n], events=ev[i])
    torch.cuda.synchronize()
    per = {s: float(np.mean([e[s][0].elapsed_time(e[s][1]) for e in ev])) for s in stages}
    return ms_step, per


def bench_mxfp4_layer(c, xs, lgs, warmup, steps, dev) -> dict:
    """The same layer with MXFP4 activations into gate|up (E2M1 codes, one E8M0 scale per
    32, applied by the MFMA): per-stage times and the gate|up rate."""
    import numpy as np
    import torch

    import fp8_moe_prefill_amd as f
    from synth import moe_inputs

    banks = [f.ExpertBank.from_host(moe_inputs(c, seed=r), dev, act="mxfp4")
             for r in range(len(xs))]
    runner = f.MoELayerRunner(c.T, c.H, c.E, c.k, c.I, dev, act="mxfp4")
    n = len(xs)
    for i in range(warmup):
        runner.run(xs[i % n], lgs[i % n], banks[i % n])
    ms, per = time_layer(runner, xs, lgs, banks, steps)
    per = {s: v * 1e3 for s, v in per.items()}
    flop_gu = 4.0 * c.T * c.k * c.H * c.I
    tf = flop_gu / (per["gate_up"] * 1e-6) / 1e12
    return {"tokens_per_s": c.T / (ms * 1e-3), "ms_per_step": ms, "stages_us": per,
            "gate_up_tflops": tf, "gate_up_frac_fp8_peak": tf / PEAK_FP8_TFLOPS}


def bench_decode_regime(c, xs, lgs, banks, dev) -> dict:
    """Decode regime of the same layer: 16 tokens (128 routed rows, one or two per expert)
    against the same rotated banks, the whole bank read once per layer; plus the M <= 16
    W8A8 projections."""
    import torch

    import fp8_moe_prefill_amd as f

    out = {}
    Td = 16
    rd = f.MoELayerRunner(Td, c.H, c.E, c.k, c.I, dev)
    for i in range(3):
        rd.run(xs[i % len(banks)][:Td], lgs[i % len(banks)][:Td], banks[i % len(banks)])
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(30):
        rd.run(xs[i % len(banks)][:Td], lgs[i % len(banks)][:Td], banks[i % len(banks)])
    b.record()
    torch.cuda.synchronize()
    us_eager = a.elapsed_time(b) / 30 * 1e3
    # replayed from HIP graphs (checked bit for bit against the eager layer): the GPU's own
    # time; issued call by call from Python the 16-token layer is close to host-bound
    xd = [x[:Td] for x in xs[:len(banks)]]
    ld = [lg[:Td] for lg in lgs[:len(banks)]]
    us = time_graph_replay(rd, xd, ld, list(banks), 30) * 1e3
    bank_bytes = 3 * c.E * c.H * c.I // 2 + 3 * c.E * c.H * c.I * 4 // 128
    out["decode_moe"] = {"tokens": Td, "us_per_layer": us, "us_per_layer_eager": us_eager,
                         "bank_GBps": bank_bytes / (us * 1e-6) / 1e9,
                         "frac_hbm": bank_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    out["decode_w8a8"] = bench_decode()
    return out


if __name__ == "__main__":
    main()
