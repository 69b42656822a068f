#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 expert path on one MI355X.

Workload (default): the long-sequence learner batch through one Qwen3-30B-A3B-shaped
mixture-of-experts layer -- 65536 tokens (8 sequences x 8192), hidden 2048, 128
experts, top-8, expert intermediate 768, SwiGLU, skewed routing (13 experts
empty, the 4 hottest holding a quarter of the assignments), seeded synthetic
BF16 inputs and upstream gradients.

A step is the whole expert path, forward and backward, with every input resident
in HBM: quantise X (amax + quantise), route + permute, grouped GEMM gate/up +
SwiGLU (+ amax), quantise the SwiGLU output, grouped GEMM down, combine; then
quantise each upstream gradient along its rows and, in the same pass, along its
tokens per expert segment; the two data-gradient grouped GEMMs; the
token-direction quantisations of the SwiGLU output and of X (gathered into
expert order); the two weight-gradient grouped GEMMs.  Expert-weight quantisation (the
weights and their per-expert transposes) happens once per optimizer step and is
timed and reported separately.  `--forward-only` times the forward alone.

Prints one JSON line: throughput (algorithmic FLOPs of the expert GEMMs / wall
time, and tokens/s), per-kernel times from HIP events recorded on the launch
stream, the roofline of the dominant kernel, and the CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2] [--config learner_64k]
                    [--forward-only] [--token-scale] [--recipe nvfp4|nvfp4-sr|dequantized|bf16-backward|bf16]
                    [--no-compare] [--no-cpu-baseline] [--no-graph]

Besides the timed recipe (default: NVFP4 forward and backward), the same step is
timed for the other recipes of the pages for comparison ("compare"): the BF16
(unquantised) layer, the NVFP4 forward with the dequantized or the BF16
backward, and the NVFP4 backward with stochastically rounded gradients.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 MoE layer TFLOP/s + tokens/s (Qwen3-30B-A3B-shaped, 1 GPU)"
PEAK_F16_MFMA_TFLOPS = 2516.6   # MI355X dense FP16/BF16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E

# Grouped GEMMs: (stage name, FLOPs as a multiple of R*H*I, description)
GEMMS = {
    "gemm1_swiglu": (4.0, "k_gemm gate/up grouped GEMM + SwiGLU epilogue (GROUP_M)"),
    "gemm2": (2.0, "k_gemm down grouped GEMM (GROUP_M)"),
    "dgrad_hact": (2.0, "k_gemm dY2 . W2 data gradient (GROUP_M)"),
    "dgrad_x": (4.0, "k_gemm dY13 . W13 data gradient (GROUP_M)"),
    "wgrad_w2": (2.0, "k_gemm dY2^T . Hact weight gradient (GROUP_K)"),
    "wgrad_w13": (4.0, "k_gemm dY13^T . X weight gradient (GROUP_K)"),
}


def hbm_bytes(cfg, recipe: str = "nvfp4", hact_cols: bool = False) -> dict:
    """Algorithmic HBM bytes of the memory-bound kernels (NVFP4: 0.5 B per code and
    1/16 B per scale; BF16 2 B, FP32 4 B).  hact_cols: the forward's SwiGLU-output
    quantisation also writes the column form."""
    T, H, I, k, R, E = cfg.T, cfg.H, cfg.I, cfg.k, cfg.R, cfg.E
    q1 = 2 + 0.5 + 1 / 16           # one-pass quantiser, per element
    kc = ((R + 15 * E + 63) // 64) * 64
    cols = lambda C: R * C * 2 + C * kc * (0.5 + 1 / 16)
    # upstream gradients: amax pass + one pass writing the row and the column operands
    dual = lambda C: R * C * (2 + 2 + 0.5 + 1 / 16) + C * kc * (0.5 + 1 / 16)
    return {
        "quantize_x": T * H * (2 + q1),                      # amax pass + one pass
        "quantize_hact": R * I * q1 + (I * kc * (0.5 + 1 / 16) if hact_cols else 0),
        "combine": T * (k * H * 4 + k * 8 + H * 2),
        "quantize_dy2": dual(H),
        "quantize_dy13": dual(2 * I),
        "quantize_cols_dy2": cols(H),
        "quantize_cols_hact": cols(I),
        "quantize_cols_dy13": cols(2 * I),
        "quantize_cols_x": cols(H),
        # BF16 column operands (read the source, write BF16 [C, kc]); an NVFP4 source
        # (the dequantized backward) reads codes and scales instead of BF16
        "cols_dy2_hact": R * H * 2 + H * kc * 2 + R * I * (0.5 + 1 / 16 if recipe == "dequantized" else 2)
                         + I * kc * 2,
        "cols_dy13_x": R * 2 * I * 2 + 2 * I * kc * 2 + R * H * (0.5 + 1 / 16 if recipe == "dequantized" else 2)
                       + H * kc * 2,
    }


def measured_traffic(stage: str, workload: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by the same counters of a plain copy), or None
    when there is none or the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in vals.get("sources", "").split():
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if not vals.get("sources") or h.hexdigest() != vals.get("sources_sha256"):
        return None
    return float(vals["hbm_bytes_per_launch"])


def cpu_baseline(d, cfg, backward: bool, token_sample: int = 4096, expert_stride: int = 16,
                 max_experts: int = 3, max_rows: int = 8192) -> dict:
    """The oracle on a bounded sample of the same workload, scaled to one step.

    Sample: the per-token stages (quantise X, route, permute, combine) on the first
    `token_sample` tokens, scaled by T / token_sample; the expert stages (forward:
    gate/up GEMM + SwiGLU, BF16 rounding, quantise, down GEMM; backward: row and
    column quantisation of the expert's dY rows, SwiGLU output and X rows, both
    data-gradient and both weight-gradient GEMMs) for the first `max_experts` of
    every `expert_stride`-th expert that hold 1..`max_rows` routed rows, at their
    real rows, scaled by R / sampled rows.  Set-up, untimed:
    the full routing (to find each expert's rows), the tensor amaxes, and the
    oracle's quantisation of the sampled experts' weights and transposes."""
    import numpy as np
    from oracle import formats as F
    from oracle import moe
    from oracle import nvfp4 as Q
    from oracle import pipeline
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        limiter = threadpoolctl.threadpool_limits(limits=cores, user_api="blas")
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpoolctl.threadpool_info()
                                if i["user_api"] == "blas"}))
    except Exception:
        limiter, blas = None, "unknown"
    E, H, I, k = cfg.E, cfg.H, cfg.I, cfg.k
    X, lg = d["X"], d["logits"]
    # set-up
    ids, _ = moe.route_topk(lg, k)
    perm = moe.permute(ids, E)
    off, rtok = perm["offsets"], perm["row_token"]
    experts = [e for e in range(0, E, expert_stride) if 0 < off[e + 1] - off[e] <= max_rows][:max_experts]
    amax_x = np.abs(X).max()
    # one scale per expert and projection (gate, up, down), as the forward uses
    wq = {e: pipeline.quantize_expert_weights(d["W13"][e:e + 1], d["W2"][e:e + 1]) for e in experts}
    w13 = {e: wq[e][0].dequant() for e in experts}
    w2 = {e: wq[e][1].dequant() for e in experts}
    if backward:
        wtq = {e: pipeline.quantize_expert_weights_t(d["W13"][e:e + 1], d["W2"][e:e + 1]) for e in experts}
        w2t = {e: wtq[e][0].dequant() for e in experts}     # [I, H]
        w13t = {e: wtq[e][1].dequant() for e in experts}    # [H, 2I]
        amax_dy2, amax_dy13 = np.abs(d["dY2"]).max(), np.abs(d["dY13"]).max()
    Ts = min(token_sample, cfg.T)
    # per-token stages on the token sample
    t0 = time.perf_counter()
    Q.quantize_rows(X[:Ts], amax=amax_x)
    ids_s, w_s = moe.route_topk(lg[:Ts], k)
    p_s = moe.permute(ids_s, E)
    moe.combine(np.zeros((Ts * k, H), np.float32), p_s["token_row"], w_s)
    t1 = time.perf_counter()
    # expert stages
    rows = 0
    for e in experts:
        a, b = off[e], off[e + 1]
        rows += b - a
        xe = Q.quantize_rows(X[rtok[a:b]], amax=amax_x).dequant()
        h = moe.swiglu(xe @ w13[e].T)
        h16 = F.bf16_bits_to_f32(F.f32_to_bf16_bits(F.f32(h)))
        F.f32(Q.quantize_rows(h16, amax=np.abs(h16).max()).dequant() @ w2[e].T)
        if backward:
            seg = np.array([0, b - a])
            dy2, dy13 = d["dY2"][a:b], d["dY13"][a:b]
            Q.quantize_rows(dy2, amax=amax_dy2).dequant() @ w2t[e].T
            Q.quantize_rows(dy13, amax=amax_dy13).dequant() @ w13t[e].T
            dy2c = Q.quantize_cols(dy2, seg, amax=amax_dy2)[0].dequant()
            hc = Q.quantize_cols(h16, seg)[0].dequant()
            dy2c @ hc.T
            dy13c = Q.quantize_cols(dy13, seg, amax=amax_dy13)[0].dequant()
            xc = Q.quantize_cols(X[rtok[a:b]], seg, amax=amax_x)[0].dequant()
            dy13c @ xc.T
    t2 = time.perf_counter()
    if limiter is not None:
        limiter.restore_original_limits()
    per_token = (t1 - t0) * cfg.T / Ts
    expert = (t2 - t1) * cfg.R / max(rows, 1)
    step = per_token + expert
    flops = cfg.R * cfg.H * cfg.I * (18.0 if backward else 6.0)
    return {"value": round(flops / step / 1e12, 4), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cores_source": "len(os.sched_getaffinity(0)); BLAS threads limited to it", "blas": blas,
            "os_cpu_count": os.cpu_count(),
            "tokens_per_s": round(cfg.T / step, 1), "step_s_extrapolated": round(step, 2),
            "sample": (f"per-token stages on {Ts} of {cfg.T} tokens ({t1 - t0:.2f} s, scaled to {per_token:.2f} s); "
                       f"{'forward and backward' if backward else 'forward'} expert stages for {len(experts)} of {E} "
                       f"experts ({rows} of {cfg.R} routed rows, {t2 - t1:.2f} s, scaled by routed rows to "
                       f"{expert:.2f} s); FP64 numpy ({blas}), {cores} BLAS threads; the quantisers, routing and "
                       f"combine are single-threaded numpy")}


def timed_events(torch, fn, reps: int, stream, flush=None) -> list:
    """Milliseconds of `reps` calls of fn(), each bracketed by HIP events on `stream`
    (the stream the kernels are launched on); with `flush`, a call of flush() before
    every rep (outside the events) evicts the caches."""
    out = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        out.append(a.elapsed_time(b))
    return out


def stats(ms: list) -> dict:
    import numpy as np
    a = np.asarray(ms, np.float64)
    return {"median_ms": round(float(np.median(a)), 5), "min_ms": round(float(a.min()), 5),
            "max_ms": round(float(a.max()), 5), "reps": len(ms)}


def measure_ceilings(nv4, torch, reps: int = 20) -> dict:
    """What plain kernels reach on this device (include/nv4moe_bench.h): a 16-byte
    non-temporal stream copy of 1 GiB (2 GiB of traffic), a read-only stream of 2 GiB,
    a write-only stream of 2 GiB, a 4:1 read:write stream, 16-byte LDS reads on every
    CU, and a loop of FP16 32x32x16 MFMAs with one and two waves per SIMD.  Median, min
    and max over `reps` event-timed calls; the rate is reported at the median."""
    st = torch.cuda.current_stream()
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    big = torch.ones(2 * n // 4, dtype=torch.float32, device="cuda")
    res = {}
    for _ in range(3):
        nv4.nv4_bench_copy(src, dst)
        nv4.nv4_bench_read(big, sink)
    c = stats(timed_events(torch, lambda: nv4.nv4_bench_copy(src, dst), reps, st))
    c["gbs"] = round(2 * n / (c["median_ms"] * 1e-3) / 1e9, 1)
    c["kernel"] = "k_stream_copy"
    res["copy"] = c
    r = stats(timed_events(torch, lambda: nv4.nv4_bench_read(big, sink), reps, st))
    r["gbs"] = round(2 * n / (r["median_ms"] * 1e-3) / 1e9, 1)
    r["kernel"] = "k_stream_read"
    res["read"] = r
    nv4.nv4_bench_write(big)
    w = stats(timed_events(torch, lambda: nv4.nv4_bench_write(big), reps, st))
    w["gbs"] = round(2 * n / (w["median_ms"] * 1e-3) / 1e9, 1)
    w["kernel"] = "k_stream_write"
    res["write"] = w
    quarter = torch.empty(2 * n // 16, dtype=torch.float32, device="cuda")
    nv4.nv4_bench_mix(big, quarter)
    m = stats(timed_events(torch, lambda: nv4.nv4_bench_mix(big, quarter), reps, st))
    m["gbs"] = round(2.5 * n / (m["median_ms"] * 1e-3) / 1e9, 1)
    m["kernel"] = "k_stream_mix (4 B read : 1 B written)"
    res["mix_4_1"] = m
    del quarter
    del src, dst, big
    lo, nb = nv4.nv4_bench_lds(None, 4096)
    m = stats(timed_events(torch, lambda: nv4.nv4_bench_lds(lo, 4096), max(5, reps // 4), st))
    m["bytes_per_ns_per_cu"] = round(nb / (m["median_ms"] * 1e6) / torch.cuda.get_device_properties(0).multi_processor_count, 1)
    m["kernel"] = "k_lds_read (16-byte reads, two 4-wave workgroups per CU)"
    res["lds_read"] = m
    out = None
    for w in (1, 2):
        out, fl = nv4.nv4_bench_mfma(out, 4096, w)
        m = stats(timed_events(torch, lambda: nv4.nv4_bench_mfma(out, 4096, w), max(5, reps // 4), st))
        m["tflops"] = round(fl / (m["median_ms"] * 1e-3) / 1e12, 1)
        m["kernel"] = f"k_mfma_loop<{w}>"
        res[f"mfma_f16_{w}wave"] = m
    torch.cuda.synchronize()
    return res


RECIPES = {
    "nvfp4": "NVFP4 forward and NVFP4 backward (every backward operand re-quantised along its new "
             "contraction dimension)",
    "nvfp4-sr": "NVFP4 forward and NVFP4 backward with the upstream gradients rounded stochastically "
                "(Philox4x64-10, fixed seed)",
    "dequantized": "NVFP4 forward, dequantized backward (BF16 GEMMs on the BF16 values of the forward's "
                   "NVFP4 weights and activations, BF16 upstream gradients)",
    "bf16-backward": "NVFP4 forward, BF16 backward on the unquantised weights and activations",
    "bf16": "BF16 (unquantised) forward and backward",
}
DTYPES = {
    "nvfp4": "nvfp4 (e2m1 + e4m3 block scales, fp32 tensor scales) decoded exactly to f16, f16 MFMA, f32 accumulate",
    "nvfp4-sr": "nvfp4 (stochastic rounding of the gradient elements) decoded exactly to f16, f16 MFMA, "
                "f32 accumulate",
    "dequantized": "forward nvfp4 decoded exactly to f16 (f16 MFMA); backward bf16 MFMA; f32 accumulate",
    "bf16-backward": "forward nvfp4 decoded exactly to f16 (f16 MFMA); backward bf16 MFMA; f32 accumulate",
    "bf16": "bf16 MFMA, f32 accumulate",
}


SR_SEED = 0x5EED   # the stochastic-rounding seed of the timed steps (a training loop would vary it)
FLUSH_BYTES = 512 << 20   # written before every timed rep: more than the 256 MB Infinity Cache and the L2s


class Flusher:
    """Evicts the caches by writing FLUSH_BYTES on the current stream (a fill kernel)."""

    def __init__(self, torch):
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(float(self.n & 0xFF))


def stage_stats(ev) -> dict:
    """Per-stage event times of several steps -> {stage: stats}."""
    per = {}
    for name, a, b in ev:
        per.setdefault(name, []).append(a.elapsed_time(b))
    return {k: stats(v) for k, v in per.items()}


def time_recipe(nv4, torch, np, cfg, inp, recipe, part, args, stages: bool, flush) -> dict:
    """One recipe on one configuration.  `part` is "fwd", "bwd" (the forward runs once,
    untimed, to produce the backward's inputs) or "fwd+bwd".  Weights are prepared once
    (timed separately); warm-up; one step captured into a HIP graph.  Timed:
      wall     exactly `steps` replays back to back between two synchronisations;
      flushed  `reps` replays, each after a cache eviction, bracketed by HIP events;
      stages   (with `stages`) `reps` eager steps with HIP events on the launch stream
               around every call and a cache eviction before every stage."""
    x, lg, W13, W2, dY2, dY13 = (inp[n] for n in ("x", "lg", "W13", "W2", "dY2", "dY13"))
    nvfp4_fwd = recipe != "bf16"
    backward = part != "fwd"

    f16 = args.weights_f16  # keep the decoded FP16 weights next to the NVFP4 ones

    def prep():
        w = nv4.quantize_expert_weights(W13, W2, f16=f16 and recipe != "dequantized") if nvfp4_fwd else None
        wt = None
        if backward:
            if recipe in ("nvfp4", "nvfp4-sr"):
                wt = nv4.quantize_expert_weights_t(W13, W2, f16=f16)
            elif recipe == "dequantized":
                wt = nv4.dequantize_expert_weights_t(w)
            else:
                wt = nv4.bf16_expert_weights_t(W13, W2)
        return w, wt

    wq_ms = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        w, wt = prep()
        e1.record()
        torch.cuda.synchronize()
        wq_ms.append(e0.elapsed_time(e1))

    if nvfp4_fwd:
        # a full step quantises the SwiGLU output once for its rows and columns (the
        # column form is the NVFP4 backward's); a timed backward alone does its own
        hact_cols = part == "fwd+bwd" and recipe in ("nvfp4", "nvfp4-sr") and not args.token_scale
        fb = nv4.alloc_forward(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, token_scale=args.token_scale, hact_cols=hact_cols)
    else:
        fb = nv4.alloc_forward_bf16(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I)
    bb = None
    if backward:
        bb = (nv4.alloc_backward(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I) if recipe in ("nvfp4", "nvfp4-sr")
              else nv4.alloc_backward_bf16(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I))

    def fwd(ev=None):
        if nvfp4_fwd:
            nv4.moe_forward(x, lg, w, cfg.k, fb, stage_events=ev)
        else:
            nv4.moe_forward_bf16(x, lg, W13, W2, cfg.k, fb, stage_events=ev)

    def bwd(ev=None):
        if recipe == "nvfp4":
            nv4.moe_backward(x, fb, wt, dY2, dY13, bb, stage_events=ev)
        elif recipe == "nvfp4-sr":
            nv4.moe_backward(x, fb, wt, dY2, dY13, bb, stage_events=ev, sr_seed=SR_SEED)
        elif recipe == "dequantized":
            nv4.moe_backward_bf16(fb.xq, fb.hq, wt, dY2, dY13, fb.routing, bb, stage_events=ev)
        else:
            nv4.moe_backward_bf16(x, fb.hact, wt, dY2, dY13, fb.routing, bb, stage_events=ev)

    def step(ev=None):
        if part != "bwd":
            fwd(ev)
        if backward:
            bwd(ev)

    label = f"{cfg.name} {recipe} {part}"
    print(f"[bench] {label}: warm-up {args.warmup} steps", file=sys.stderr, flush=True)
    if part == "bwd":
        fwd()                      # the backward's inputs, once
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the step's launches captured once into a HIP graph (the library allocates
    # nothing and clears buffers with kernels, so the step is capturable)
    run = step
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        run = graph.replay

    # wall: exactly `steps` steps, synchronised on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    st = torch.cuda.current_stream()
    flushed = stats(timed_events(torch, run, args.reps, st, flush))
    print(f"[bench] {label}: {args.steps} steps {ms_step:.3f} ms/step; flushed median {flushed['median_ms']:.3f} ms",
          file=sys.stderr, flush=True)

    stage_st = {}
    if stages:
        ev = nv4.StageEvents(before=flush)
        for _ in range(args.reps):
            step(ev)
        torch.cuda.synchronize()
        stage_st = stage_stats(ev)
    counts = np.diff(fb.routing.offsets.cpu().numpy())
    out = {"ms_per_step": ms_step, "flushed": flushed, "stages": stage_st, "counts": counts,
           "weight_ms": float(np.median(wq_ms))}
    del run, fb, bb, w, wt, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def vendor_bf16_rates(torch, cfg, reps: int = 5) -> dict:
    """The ROCm BLAS library's dense BF16 GEMM (torch.matmul, hipBLASLt) on the shapes of
    the six expert GEMMs with all routed rows in one dense product (no grouping, gather
    or epilogue): the best dense BF16 rate this device reaches on those shapes."""
    R, H, I = cfg.R, cfg.H, cfg.I
    shapes = {"gemm1_swiglu": (R, H, 2 * I), "gemm2": (R, I, H), "dgrad_hact": (R, H, I), "dgrad_x": (R, 2 * I, H),
              "wgrad_w2": (H, R, I), "wgrad_w13": (2 * I, R, H)}
    out = {}
    st = torch.cuda.current_stream()
    for name, (m, k, n) in shapes.items():
        a = torch.randn(m, k, dtype=torch.bfloat16, device="cuda")
        b = torch.randn(k, n, dtype=torch.bfloat16, device="cuda")
        c = torch.matmul(a, b)
        ms = stats(timed_events(torch, lambda: torch.matmul(a, b, out=c), reps, st))["median_ms"]
        out[name] = {"ms": ms, "tflops": round(2.0 * m * k * n / (ms * 1e-3) / 1e12, 1)}
        del a, b, c
    torch.cuda.empty_cache()
    return out


def dense_gemm(nv4, torch, np, synth, args, flush) -> dict:
    """The single dense NVFP4 W4A4 GEMM: M = 8192 tokens, K = 2048, N = 768, FP32 out,
    as a one-expert grouped GEMM; timed alone (operands quantised beforehand) and
    with the quantisation of A (amax pass + quantisation) in front of it."""
    cfg = synth.CONFIGS["dense_gemm"]
    M, K, N = cfg.T, cfg.H, cfg.I
    A, B = synth.dense_gemm_inputs(cfg)
    a = torch.from_numpy(A).to(torch.bfloat16).cuda()
    b = torch.from_numpy(B).to(torch.bfloat16).cuda()
    bq = nv4.nvfp4_quantize(b)
    aq = nv4.NVFP4.empty(M, K)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    off = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    quant = lambda: nv4.nvfp4_quantize(a, out=aq, amax_out=amax)
    gemm = lambda: nv4.nvfp4_grouped_gemm(aq, bq, off, 1, N, M_cap=M, C=C)
    both = lambda: (quant(), gemm())
    for _ in range(3):
        both()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    g = stats(timed_events(torch, gemm, args.reps, st, flush))
    q = stats(timed_events(torch, quant, args.reps, st, flush))
    w = stats(timed_events(torch, both, args.reps, st, flush))
    flops = 2.0 * M * N * K
    tf = flops / (g["median_ms"] * 1e-3) / 1e12
    qbytes = M * K * (2 + 2 + 0.5 + 1 / 16)
    return {"workload": "dense NVFP4 W4A4 GEMM M=8192 K=2048 N=768, FP32 out (one-expert grouped GEMM)",
            "gemm": dict(g, tflops=round(tf, 1)),
            "quantize_a": dict(q, gbs=round(qbytes / (q["median_ms"] * 1e-3) / 1e9, 1),
                               bytes_note="amax pass 2 B + one pass 2.5625 B per element"),
            "quantize_a_then_gemm": dict(w, tflops=round(flops / (w["median_ms"] * 1e-3) / 1e12, 1)),
            "roofline": {"bound": "mfma", "kernel": "k_gemm (GROUP_M, one expert)", "achieved": round(tf, 2),
                         "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_F16_MFMA_TFLOPS, 4)},
            "flops": flops}


def layer_inputs_dev(torch, np, synth, cfg, backward):
    d = synth.layer_inputs(cfg, with_grads=backward)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    inp = dict(x=dev(d["X"], torch.bfloat16), lg=dev(d["logits"], torch.float32),
               W13=dev(d["W13"], torch.bfloat16), W2=dev(d["W2"], torch.bfloat16),
               dY2=dev(d["dY2"], torch.bfloat16) if backward else None,
               dY13=dev(d["dY13"], torch.bfloat16) if backward else None)
    torch.cuda.synchronize()
    return d, inp


def summarize(cfg, res, part, recipe, ceil) -> dict:
    """Throughput, per-stage rates and the dominant kernel's roofline of one timed part."""
    rhi = float(cfg.R) * cfg.H * cfg.I
    mult = {"fwd": 6.0, "bwd": 12.0, "fwd+bwd": 18.0}[part]
    flops = rhi * mult
    med = {k: v["median_ms"] for k, v in res["stages"].items()}
    gemm = {n: (m * rhi / (med[n] * 1e-3) / 1e12, desc) for n, (m, desc) in GEMMS.items() if n in med}
    dom = max(gemm, key=lambda n: med[n]) if gemm else None
    # the forward made the SwiGLU output's column form when the step's backward did not
    hact_cols = part == "fwd+bwd" and recipe in ("nvfp4", "nvfp4-sr") and "quantize_cols_hact" not in med
    nbytes = hbm_bytes(cfg, recipe, hact_cols)
    mfma_ceil = ceil.get("mfma_f16_2wave", {}).get("tflops") if ceil else None
    read_ceil = ceil.get("read", {}).get("gbs") if ceil else None
    copy_ceil = ceil.get("copy", {}).get("gbs") if ceil else None
    mix_ceil = ceil.get("mix_4_1", {}).get("gbs") if ceil else None
    other = {}
    for n, (tf, desc) in gemm.items():
        e = {"achieved_tflops": round(tf, 2), "frac": round(tf / PEAK_F16_MFMA_TFLOPS, 4),
             "ms": round(med[n], 4), "min_ms": res["stages"][n]["min_ms"], "max_ms": res["stages"][n]["max_ms"]}
        if mfma_ceil:
            e["frac_of_measured_mfma_loop"] = round(tf / mfma_ceil, 4)
        other[n] = e
    for n, b in nbytes.items():
        if n in med:
            gbs = b / (med[n] * 1e-3) / 1e9
            e = {"achieved_gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "ms": round(med[n], 4),
                 "min_ms": res["stages"][n]["min_ms"], "max_ms": res["stages"][n]["max_ms"]}
            if read_ceil:
                e["frac_of_measured_read_stream"] = round(gbs / read_ceil, 4)
                e["frac_of_measured_copy_stream"] = round(gbs / copy_ceil, 4)
                e["frac_of_measured_4to1_stream"] = round(gbs / mix_ceil, 4)
            other[n] = e
    t_med = res["flushed"]["median_ms"]
    out = {"ms_per_step": round(res["ms_per_step"], 4), "flushed": res["flushed"],
           "tflops": round(flops / (res["ms_per_step"] * 1e-3) / 1e12, 2),
           "tflops_flushed_median": round(flops / (t_med * 1e-3) / 1e12, 2),
           "tokens_per_s": round(cfg.T / (res["ms_per_step"] * 1e-3), 1),
           "flops_per_step": flops, "stages": other}
    if dom:
        bf16_stage = recipe == "bf16" or (recipe in ("dequantized", "bf16-backward") and dom not in
                                          ("gemm1_swiglu", "gemm2"))
        kernel = gemm[dom][1].replace("k_gemm", "k_gemm (BF16 operands)") if bf16_stage else gemm[dom][1]
        out["roofline"] = {"bound": "mfma", "kernel": kernel, "stage": dom, "achieved": round(gemm[dom][0], 2),
                           "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(gemm[dom][0] / PEAK_F16_MFMA_TFLOPS, 4),
                           "traffic": measured_traffic(dom, cfg.name) if recipe in ("nvfp4", "nvfp4-sr") else None}
        if mfma_ceil:
            out["roofline"]["frac_of_measured_mfma_loop"] = round(gemm[dom][0] / mfma_ceil, 4)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--reps", type=int, default=20, help="cache-flushed reps for median/min/max (and per-stage times)")
    ap.add_argument("--config", default="learner_64k", choices=["learner_64k", "qwen3_fwd", "qwen3_bwd", "dense_gemm"],
                    help="the workload of the JSON line: the learner batch forward + backward (default), the "
                         "16384-token forward, the same layer's backward, or the dense 8192x2048x768 GEMM")
    ap.add_argument("--forward-only", action="store_true")
    ap.add_argument("--weights-f16", action="store_true",
                    help="keep each NVFP4 weight tensor's exact decoded FP16 values (made with the weight "
                         "quantisation, once per optimizer step), which the grouped GEMMs read instead of "
                         "decoding the weights")
    ap.add_argument("--token-scale", action="store_true",
                    help="per-token FP32 scales for X and the SwiGLU output instead of one per tensor")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--recipe", default="nvfp4", choices=sorted(RECIPES),
                    help="the step timed for the JSON line (default: NVFP4 forward and backward)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip timing the other recipes (BF16 layer, dequantized and BF16 backward) for comparison")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (dense GEMM, 16384-token forward and backward) in the JSON line")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every kernel from Python each step instead of replaying a captured HIP graph")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the device's achievable stream-copy, stream-read and FP16 MFMA rates")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (three times): the known-size kernel whose "
                         "FETCH_SIZE / WRITE_SIZE counters scale the GEMM's traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the expert path is built and timed on a single MI355X "
              f"(--gpus {args.gpus} is not supported; multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))
        return

    import nvfp4_w4a4_moe_amd as nv4
    import synth

    nv4.load()
    if args.ceilings:
        print(json.dumps({"ceilings": measure_ceilings(nv4, torch), "peak_hbm_gbs": PEAK_HBM_GBS,
                          "peak_f16_mfma_tflops": PEAK_F16_MFMA_TFLOPS}))
        return
    print("[bench] measuring the device's stream and MFMA ceilings", file=sys.stderr, flush=True)
    ceil = measure_ceilings(nv4, torch)
    flush = Flusher(torch)

    if args.config == "dense_gemm":
        r = dense_gemm(nv4, torch, np, synth, args, flush)
        tf = r["gemm"]["tflops"]
        rec = {"metric": METRIC, "value": tf, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.reps, "warmup": 3,
               "ms_per_step": r["gemm"]["median_ms"], "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": DTYPES["nvfp4"],
               "data": "synthetic (seeded; A N(0,1), B N(0,0.02))",
               "config": {"workload": r["workload"], "M": 8192, "K": 2048, "N": 768},
               "timing": "cache-flushed reps, HIP events; value at the median", "dense_gemm": r,
               "roofline": dict(r["roofline"], traffic=None), "ceilings": ceil}
        print(json.dumps(rec))
        return

    cfg = synth.CONFIGS["qwen3_fwd" if args.config == "qwen3_bwd" else args.config]
    part = "bwd" if args.config == "qwen3_bwd" else ("fwd" if (args.forward_only or args.config == "qwen3_fwd")
                                                     else "fwd+bwd")
    backward = part != "fwd"
    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    d, inputs = layer_inputs_dev(torch, np, synth, cfg, backward)

    res = time_recipe(nv4, torch, np, cfg, inputs, args.recipe, part, args, stages=True, flush=flush)
    summ = summarize(cfg, res, part, args.recipe, ceil)
    counts = res["counts"]
    compare = {}
    if not args.no_compare and part == "fwd+bwd":
        others = ["bf16", "dequantized", "bf16-backward", "nvfp4-sr"]
        for rcp in others:
            if rcp == args.recipe:
                continue
            print(f"[bench] comparison recipe {rcp}", file=sys.stderr, flush=True)
            r = time_recipe(nv4, torch, np, cfg, inputs, rcp, part, args, stages=rcp == "bf16", flush=flush)
            compare[rcp] = {"recipe": RECIPES[rcp], "ms_per_step": round(r["ms_per_step"], 4),
                            "flushed": r["flushed"],
                            "tokens_per_s": round(cfg.T / (r["ms_per_step"] * 1e-3), 1),
                            "weight_prep_ms": round(r["weight_ms"], 4),
                            "time_vs_this_recipe": round(r["ms_per_step"] / res["ms_per_step"], 4)}
            if rcp == "bf16":
                # the BF16 layer with its six GEMMs at the vendor library's dense BF16 rate on the same
                # shapes (no grouping): what a BF16 layer could reach, against this recipe
                vr = vendor_bf16_rates(torch, cfg)
                st_ms = {k: v["median_ms"] for k, v in r["stages"].items()}
                non_gemm = sum(v for k, v in st_ms.items() if k not in GEMMS)
                lib_ms = non_gemm + sum(v["ms"] for v in vr.values())
                compare[rcp]["stages_ms"] = {k: round(v, 4) for k, v in st_ms.items()}
                compare[rcp]["vendor_dense_bf16_gemm"] = vr
                compare[rcp]["layer_at_vendor_gemm_rate_ms"] = round(lib_ms, 4)
                compare[rcp]["this_recipe_flushed_vs_bf16_at_vendor_rate"] = round(
                    lib_ms / res["flushed"]["median_ms"], 4)
                compare[rcp]["note"] = ("layer_at_vendor_gemm_rate_ms: this build's BF16 non-GEMM stages (cold) plus "
                                        "the six GEMMs at the vendor library's dense BF16 rate on all routed rows at "
                                        "once; ratios above 1 mean the NVFP4 step is faster")
    if not args.token_scale and part == "fwd+bwd" and not args.no_compare and args.recipe == "nvfp4":
        print("[bench] comparison: per-token activation scales", file=sys.stderr, flush=True)
        args.token_scale = True
        r = time_recipe(nv4, torch, np, cfg, inputs, "nvfp4", part, args, stages=True, flush=flush)
        args.token_scale = False
        compare["nvfp4-token-scale"] = {
            "recipe": "NVFP4 forward and backward with per-token FP32 scales for X and the SwiGLU output",
            "ms_per_step": round(r["ms_per_step"], 4), "flushed": r["flushed"],
            "tokens_per_s": round(cfg.T / (r["ms_per_step"] * 1e-3), 1),
            "time_vs_this_recipe": round(r["ms_per_step"] / res["ms_per_step"], 4),
            "stages_ms": {k: v["median_ms"] for k, v in r["stages"].items()}}

    by_config = {}
    if not args.no_configs and args.config == "learner_64k" and part == "fwd+bwd":
        del inputs
        torch.cuda.empty_cache()
        print("[bench] dense GEMM 8192x2048x768", file=sys.stderr, flush=True)
        by_config["dense_gemm_8192x2048x768"] = dense_gemm(nv4, torch, np, synth, args, flush)
        qcfg = synth.CONFIGS["qwen3_fwd"]
        print("[bench] qwen3_fwd: generating inputs", file=sys.stderr, flush=True)
        _, qin = layer_inputs_dev(torch, np, synth, qcfg, True)
        for qpart, key in (("fwd", "qwen3_fwd_16k"), ("bwd", "qwen3_bwd_16k")):
            r = time_recipe(nv4, torch, np, qcfg, qin, "nvfp4", qpart, args, stages=True, flush=flush)
            sm = summarize(qcfg, r, qpart, "nvfp4", ceil)
            qc = r["counts"]
            sm["workload"] = (f"qwen3_fwd: 16384 tokens through the Qwen3-30B-A3B-shaped layer, "
                              f"{'forward' if qpart == 'fwd' else 'backward (dgrad + wgrad grouped GEMMs)'}, "
                              f"Zipf(1.1) routing (max expert {int(qc.max())} rows, min {int(qc.min())})")
            by_config[key] = sm
        del qin
        torch.cuda.empty_cache()

    rec = {
        "metric": METRIC,
        "value": summ["tflops"],
        "unit": "TFLOP/s",
        "tokens_per_s": summ["tokens_per_s"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": summ["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPES[args.recipe],
        "data": "synthetic (seeded; random-init expert weights N(0,0.02), activations N(0,1) with 0.1% x20 outliers, "
                "upstream gradients N(0,1e-3))",
        "config": {"workload": f"{cfg.name}: Qwen3-30B-A3B-shaped MoE expert layer "
                               f"{ {'fwd': 'forward', 'bwd': 'backward', 'fwd+bwd': 'forward + backward'}[part] }"
                               f"{', per-token activation scales' if args.token_scale else ''}"
                               f"{'' if args.recipe == 'nvfp4' else ', ' + RECIPES[args.recipe]}",
                   "tokens": cfg.T, "hidden": cfg.H, "experts": cfg.E, "top_k": cfg.k, "intermediate": cfg.I,
                   "routing": cfg.routing, "expert_load_max": int(counts.max()),
                   "expert_load_min": int(counts.min()), "empty_experts": int((counts == 0).sum()),
                   "top4_share": round(float(np.sort(counts)[-4:].sum() / counts.sum()), 4),
                   "flops_per_step": summ["flops_per_step"]},
        "launch": "eager" if args.no_graph else "hip_graph",
        "timing": ("value and ms_per_step: wall clock of `steps` HIP-graph replays back to back; flushed: "
                   f"{args.reps} replays each after a {FLUSH_BYTES >> 20} MiB cache-evicting write, HIP events; "
                   "per-stage times: eager steps with a cache eviction before every stage, HIP events on the "
                   "launch stream; rates at the median"),
        "flushed": summ["flushed"],
        "tflops_flushed_median": summ["tflops_flushed_median"],
        "stages_ms": {k: v["median_ms"] for k, v in res["stages"].items()},
        "weight_quantize_ms": round(res["weight_ms"], 4),
        "roofline": summ.get("roofline"),
        "other_kernels": {k: v for k, v in summ["stages"].items()
                          if not summ.get("roofline") or k != summ["roofline"]["stage"]},
        "ceilings": ceil,
    }
    if compare:
        rec["compare"] = compare
    if by_config:
        rec["by_config"] = by_config
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(d, cfg, backward)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
