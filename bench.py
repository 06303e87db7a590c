#!/usr/bin/env python3
"""Benchmark: GPTQ quantization of one linear layer on one MI355X.

Workload (one step = the whole layer path over one calibration set):
  Llama-7B-shaped attention projection, W 4096 x 4096 bf16 ~ N(0, 0.02^2),
  calibration X = 128 sequences x 2048 tokens x 4096 bf16 ~ N(0, 1) with 0.5 %
  outlier channels x30, 4-bit asymmetric, group 128, block 128, damp 0.01.
  Inputs are synthetic, seeded, and resident in HBM before timing starts.

  step = S := 0; S += X^T X (all 262144 tokens); prepare (damp, Cholesky,
         inverse, upper factor); quantize (blocked column loop + lazy trailing
         update); pack to 4-bit words; plus the group min-max RTN baseline.

Prints ONE JSON line.  The metric is weights quantized per second
(m * n / step time).  ``roofline`` reports the dominant kernel (the bf16 MFMA
Hessian) against the MI355X dense bf16 MFMA peak, timed with HIP events on the
stream it runs on.  ``cpu_baseline`` times the fp64 oracle on a bounded sample
of the same workload on the host cores and scales it to the same unit.
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

WORKLOAD = "llama7b_attn"
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
FP64_PEAK_TFLOPS = 78.6
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_hessian_llama7b_attn.json")
HESSIAN_SRC = os.path.join(ROOT, "post_weight_quantization_22_amd", "csrc", "hessian.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-awq", action="store_true",
                    help="skip the AWQ-lite / awq_clip measurement")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the layer-sequential MLP-stack measurement")
    ap.add_argument("--cpu-sample-rows", type=int, default=4096)
    ap.add_argument("--cpu-sample-chunks", type=int, default=64)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run one Hessian accumulate of the workload and one 2 GiB device copy, "
                         "for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs, then exit")
    ap.add_argument("--dequant-probe", action="store_true",
                    help="run the quantized layer's product 10 times at 2048 and at 16 tokens "
                         "(4096 x 4096, random 4-bit codes, group 128), for rocprofv3 counter "
                         "runs, then exit")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter files of two --traffic-probe runs into "
                         "profiles/traffic_hessian_llama7b_attn.json, then exit")
    return ap.parse_args()


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per Hessian launch from committed rocprofv3 counter runs, if current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != source_hash(HESSIAN_SRC):
        return None  # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 31  # the calibration copy of --traffic-probe
HESS_KERNELS = ("syrk_bf16_dma_kernel", "reduce_full_partials_kernel")


def traffic_record(fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes of one Hessian launch from two counter runs of --traffic-probe.

    Each counter (KiB per dispatch, summed over the L2 channels) is scaled by
    the ratio of the known bytes of the 2 GiB device copy to what the same
    counter reads for that copy; the launch is the last pair of Hessian
    dispatches (interior SYRK + split reduction) in each file.
    """
    import csv
    from collections import defaultdict

    def per_dispatch(path, counter):
        val = defaultdict(float)
        name = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            val[d] += float(r["Counter_Value"])
            name[d] = r["Kernel_Name"]
        return val, name

    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        val, name = per_dispatch(path, counter)
        copies = [d for d in val if "copyBuffer" in name[d]]
        if not copies:
            raise SystemExit(f"{path}: no copy dispatch")
        copy_kib = val[max(copies)]
        hess = 0.0
        for k in HESS_KERNELS:
            ds = [d for d in val if k in name[d]]
            if not ds:
                raise SystemExit(f"{path}: no {k} dispatch")
            hess += val[max(ds)]
        factor = COPY_BYTES / (copy_kib * 1024.0)
        out[counter] = {"hessian_kib": hess, "copy_kib": copy_kib, "scale": factor,
                        "bytes": hess * 1024.0 * factor}
    return out


def cpu_baseline(wl, rows: int, chunks: int):
    """Time the fp64 oracle on a bounded sample and scale to weights/s for the full layer."""
    import numpy as np

    import oracle
    import synth

    ls = wl.layer()
    xs = wl.xs[ls.x]
    q = wl.quant
    # Hessian on `chunks` calibration sequences: cost is linear in tokens
    Xs = synth.x_all(wl, ls.x, chunks=list(range(chunks)))
    t0 = time.perf_counter()
    S = oracle.hessian_S([Xs])
    t_h = time.perf_counter() - t0
    t_h_full = t_h * xs.chunks / chunks
    # prepare at full size (the sample's S stands in for the full one)
    t0 = time.perf_counter()
    P = oracle.prepare(S, q.perc_damp, q.desc_act)
    t_p = time.perf_counter() - t0
    # column loop on a row sample: rows are independent given U, cost linear in rows
    W = synth.weight(wl, ls.name, rows=slice(0, rows))
    t0 = time.perf_counter()
    oracle.gptq_quantize(W, P.U, q.bits, q.group_size, q.block_size, P.perm, P.dead)
    t_q = time.perf_counter() - t0
    t_q_full = t_q * ls.m / rows
    total = t_h_full + t_p + t_q_full
    try:
        from threadpoolctl import threadpool_info

        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    return {
        "value": ls.m * ls.n / total,
        "unit": "weights/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 numpy/scipy oracle: Hessian over {chunks} of {xs.chunks} sequences "
                   f"({t_h:.2f} s, scaled x{xs.chunks / chunks:g}), prepare at full n={ls.n} "
                   f"({t_p:.2f} s), column loop on {rows} of {ls.m} rows ({t_q:.2f} s, scaled "
                   f"x{ls.m / rows:g}); estimated full-layer time {total:.1f} s"),
    }


def dequant_gemm_measure(gq, buf, X, m, n, q, stream):
    """The quantized layer used: Y = X W_q^T from its packed codes (gptq_dequant_gemm).

    prefill: one 2048-token calibration sequence, bound by bf16 MFMA (2 tokens m n
    flop); decode: 16 tokens, bound by HBM (codes b/8 B, scale and zero 8 B per
    group, X and Y once per weight).  The decode launches are replayed from a
    HIP graph so that the host's launch cost is not timed."""
    import torch

    out = {}
    ng = buf.scales.shape[1]
    for name, tokens, reps in (("prefill_2048", 2048, 20), ("decode_16", 16, 200)):
        Xt = X[:tokens]
        Y = torch.empty((tokens, m), dtype=torch.float32, device=X.device)
        nws = gq.gptq_dequant_gemm_workspace_size(tokens, m, n, False)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=X.device)

        def call():
            gq.gptq_dequant_gemm(Xt, buf.packed, q.bits, q.group_size, buf.scales, buf.zeros,
                                 Y, ws=ws, stream=torch.cuda.current_stream())

        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        graph = None
        if tokens <= 32:
            try:
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.stream(side):
                    with torch.cuda.graph(graph, stream=side):
                        for _ in range(reps):
                            call()
                torch.cuda.current_stream().wait_stream(side)
                graph.replay()
                torch.cuda.synchronize()
            except Exception as exc:  # capture refused: time plain launches instead
                graph = None
                out[name + "_graph_error"] = str(exc)[:200]
        e0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for _ in range(reps):
                call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        flop = 2.0 * tokens * m * n
        byts = m * n * q.bits / 8 + m * ng * 8 + tokens * n * 2 + tokens * m * 4
        rec = {"tokens": tokens, "us": round(us, 3), "tflops": round(flop / us / 1e6, 2),
               "gbs": round(byts / us / 1e3, 1), "timed": "hip graph replay" if graph else
               "stream launches"}
        if tokens > 32:
            rec["roofline"] = {"bound": "mfma", "achieved": rec["tflops"], "peak": BF16_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(rec["tflops"] / BF16_PEAK_TFLOPS, 4)}
        else:
            rec["roofline"] = {"bound": "hbm", "achieved": rec["gbs"], "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(rec["gbs"] / HBM_PEAK_GBS, 4),
                               "algorithmic_bytes": int(byts)}
        out[name] = rec
    return out


def awq_measure(gq, W, X, S, m, n, q, stream):
    """AWQ-lite then awq_clip on the same layer and calibration set (S = X^T X from
    the Hessian step): the activation statistic (one pass over X, bound by HBM),
    the alpha search (11 candidates, each one fp32 MFMA product D S of 2 m n^2
    flop) and the clip search (11 candidates per row and group, each a quadratic
    form d S'_gg d^T of 2 G^2 flop on the vector units).  Events on the stream;
    one warm-up call each, then the mean of ``reps`` calls."""
    import torch

    N = X.shape[0]
    G = q.group_size
    ng = -(-n // G)
    absum = torch.zeros(n, dtype=torch.float32, device=X.device)
    ws_abs = torch.empty(gq.awq_absum_workspace_size(n, N), dtype=torch.uint8, device=X.device)
    s = torch.empty(n, dtype=torch.float32, device=X.device)
    alpha = torch.empty(1, dtype=torch.float32, device=X.device)
    losses = torch.empty(11, dtype=torch.float32, device=X.device)
    ws_lite = torch.empty(gq.awq_lite_workspace_size(m, n), dtype=torch.uint8, device=X.device)
    codes = torch.empty((m, n), dtype=torch.uint8, device=X.device)
    scales = torch.empty((m, ng), dtype=torch.float32, device=X.device)
    zeros = torch.empty((m, ng), dtype=torch.float32, device=X.device)
    cidx = torch.empty((m, ng), dtype=torch.uint8, device=X.device)

    def absum_call():
        absum.zero_()
        gq.awq_activation_absum(X, absum, ws=ws_abs, stream=stream)

    def lite_call():
        gq.awq_lite(W, S, absum, N, q.bits, G, s, alpha, losses, ws=ws_lite, stream=stream)

    def clip_call():
        gq.awq_clip_quantize(W, S, s, q.bits, G, codes, scales, zeros, cidx, stream=stream)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_abs = timed(absum_call, 5)
    t_lite = timed(lite_call, 3)
    t_clip = timed(clip_call, 5)
    abs_bytes = N * n * 2
    lite_flop = 11 * 2.0 * m * n * n
    clip_flop = 11 * 2.0 * m * ng * G * G
    a = float(alpha.cpu()[0])
    return {
        "alpha": round(a, 2),
        "activation_absum": {"ms": round(t_abs, 4), "gbs": round(abs_bytes / t_abs / 1e6, 1),
                             "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                          "frac": round(abs_bytes / t_abs / 1e6 / HBM_PEAK_GBS, 4),
                                          "algorithmic_bytes": abs_bytes}},
        "awq_lite": {"ms": round(t_lite, 4),
                     "tflops": round(lite_flop / t_lite / 1e9, 2),
                     "roofline": {"bound": "mfma", "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(lite_flop / t_lite / 1e9 / FP32_PEAK_TFLOPS, 4),
                                  "algorithmic_work": f"11 x 2 m n^2 = {lite_flop:.4e} flop"}},
        "awq_clip": {"ms": round(t_clip, 4), "tflops": round(clip_flop / t_clip / 1e9, 2),
                     "roofline": {"bound": "alu", "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(clip_flop / t_clip / 1e9 / FP32_PEAK_TFLOPS, 4),
                                  "algorithmic_work": f"11 x 2 m ngroups G^2 = {clip_flop:.4e} flop"}},
    }


def dequant_probe(gq, dev):
    """Ten products at 2048 tokens, then ten at 16, on a 4096 x 4096 4-bit g128
    layer of random codes packed in processing order (identity order)."""
    import numpy as np
    import torch

    m = n = 4096
    bits, G = 4, 128
    rng = np.random.default_rng(0)
    codes = torch.from_numpy(rng.integers(0, 16, size=(m, n), dtype=np.uint8)).to(dev)
    packed = torch.empty((m, n * bits // 32), dtype=torch.int32, device=dev)
    gq.gptq_pack_ordered(codes, bits, None, packed)
    scales = torch.from_numpy(rng.uniform(1e-3, 1e-2, size=(m, n // G)).astype(np.float32)).to(dev)
    zeros = torch.from_numpy(rng.integers(0, 16, size=(m, n // G)).astype(np.float32)).to(dev)
    X = torch.from_numpy(rng.standard_normal((2048, n)).astype(np.float32)).to(dev).to(torch.bfloat16)
    for tokens in (2048, 16):
        Y = torch.empty((tokens, m), dtype=torch.float32, device=dev)
        nws = gq.gptq_dequant_gemm_workspace_size(tokens, m, n, False)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        for _ in range(10):
            gq.gptq_dequant_gemm(X[:tokens], packed, bits, G, scales, zeros, Y, ws=ws)
        torch.cuda.synchronize()
    print("dequant probe: 10 products at 2048 and 10 at 16 tokens done", flush=True)


def stack_measure(gq, dev):
    """Layer-sequential GPTQ of a two-block Llama-7B MLP stack (d 4096, f 11008,
    128 x 2048 calibration tokens, 4-bit g128 desc_act): each layer quantized on
    the activations the already-quantized layers produce, gate and up on one
    Hessian.  One warm-up run (allocations), then one timed run with events at
    the phase boundaries on the stream."""
    import numpy as np
    import torch

    import synth
    from post_weight_quantization_22_amd import stack

    wl = synth.get_workload("llama7b_mlp_stack")
    xs = wl.xs["x0"]
    q = wl.quant
    t0 = time.time()
    x0 = torch.empty((xs.tokens, xs.n), dtype=torch.bfloat16, device=dev)
    for c0 in range(0, xs.chunks, 16):
        idx = list(range(c0, min(xs.chunks, c0 + 16)))
        x0[c0 * xs.chunk_len:(c0 + len(idx)) * xs.chunk_len].copy_(
            torch.from_numpy(synth.x_all(wl, "x0", chunks=idx)).to(torch.bfloat16))
    blocks = len(wl.layers) // 3
    W = [tuple(torch.from_numpy(synth.weight(wl, f"{nm}_{k}")).to(dev).to(torch.bfloat16)
               for nm in ("gate", "up", "down")) for k in range(blocks)]
    t_gen = time.time() - t0
    cfg = gq.make_config(q.bits, q.group_size, q.block_size, q.perc_damp, q.desc_act, q.sym)
    stack.quantize_stack(x0, W, cfg)
    torch.cuda.synchronize()
    marks = []
    stack.quantize_stack(x0, W, cfg, marks=marks)
    torch.cuda.synchronize()
    phases = {}
    for (_, e0), (nm, e1) in zip(marks[:-1], marks[1:]):
        phases[nm] = phases.get(nm, 0.0) + e0.elapsed_time(e1)
    total = marks[0][1].elapsed_time(marks[-1][1])
    weights = sum(l.m * l.n for l in wl.layers)
    return {
        "workload": f"{blocks} Llama-7B MLP blocks (gate/up 11008x4096, down 4096x11008), "
                    f"{xs.tokens} calibration tokens, {q.bits}-bit g{q.group_size}, desc_act",
        "ms": round(total, 2),
        "weights_per_s": round(weights / (total * 1e-3), 1),
        "phase_ms": {k: round(v, 2) for k, v in phases.items()},
        "input_setup_s": round(t_gen, 1),
    }


def main():
    args = parse()
    if args.traffic_record:
        t = traffic_record(*args.traffic_record)
        rec = {
            "kernel": "gptq_hessian_accumulate: " + " + ".join(HESS_KERNELS),
            "workload": WORKLOAD,
            "bytes_per_launch": round(t["FETCH_SIZE"]["bytes"] + t["WRITE_SIZE"]["bytes"]),
            "fetch": t["FETCH_SIZE"],
            "write": t["WRITE_SIZE"],
            "calibration": f"device copy of {COPY_BYTES} bytes (read {COPY_BYTES}, write "
                           f"{COPY_BYTES})",
            "commands": [
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format "
                "csv -d $REPO/gpurun_out/pmc_fetch -o run -- python3 $REPO/bench.py "
                "--traffic-probe",
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format "
                "csv -d $REPO/gpurun_out/pmc_write -o run -- python3 $REPO/bench.py "
                "--traffic-probe",
                "python3 bench.py --traffic-record gpurun_out/pmc_fetch/run_counter_collection.csv "
                "gpurun_out/pmc_write/run_counter_collection.csv",
            ],
            "kernel_source_sha256": source_hash(HESSIAN_SRC),
        }
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU split of the path is described, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import post_weight_quantization_22_amd as gq
    from post_weight_quantization_22_amd import pipeline

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.dequant_probe:
        dequant_probe(gq, dev)
        return

    wl = synth.get_workload(WORKLOAD)
    ls = wl.layer()
    xs = wl.xs[ls.x]
    q = wl.quant
    m, n, N = ls.m, ls.n, xs.tokens

    # ---- inputs, resident in HBM before any timing -------------------------------
    t0 = time.time()
    W = torch.from_numpy(synth.weight(wl, ls.name)).to(dev).to(torch.bfloat16)
    X = torch.empty((N, n), dtype=torch.bfloat16, device=dev)
    per = 16
    for c0 in range(0, xs.chunks, per):
        idx = list(range(c0, min(xs.chunks, c0 + per)))
        host = synth.x_all(wl, ls.x, chunks=idx)
        X[c0 * xs.chunk_len:(c0 + len(idx)) * xs.chunk_len].copy_(
            torch.from_numpy(host).to(torch.bfloat16))
    torch.cuda.synchronize()
    t_gen = time.time() - t0

    cfg = gq.make_config(q.bits, q.group_size, q.block_size, q.perc_damp, q.desc_act, q.sym)
    buf = pipeline.allocate(m, n, cfg, N)
    if args.traffic_probe:
        stream = torch.cuda.current_stream()
        for _ in range(2):
            buf.S.zero_()
            gq.gptq_hessian_accumulate(buf.S, X, ws=buf.ws_hess, stream=stream)
        torch.cuda.synchronize()
        del X
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("traffic probe: 2 Hessian accumulates and one device copy of "
              f"{COPY_BYTES} bytes done", flush=True)
        return
    ng = pipeline.ngroups(n, q.group_size)
    rtn_codes = torch.empty((m, n), dtype=torch.uint8, device=dev)
    rtn_scales = torch.empty((m, ng), dtype=torch.float32, device=dev)
    rtn_zeros = torch.empty((m, ng), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        buf.S.zero_()
        gq.gptq_hessian_accumulate(buf.S, X, ws=buf.ws_hess, stream=stream)
        if ev:
            ev[1].record(stream)
        pipeline.prepare(buf, N, stream)
        if ev:
            ev[2].record(stream)
        pipeline.quantize(buf, W, stream)
        if ev:
            ev[3].record(stream)
        pipeline.pack(buf, stream)
        if ev:
            ev[4].record(stream)
        gq.rtn_minmax(W, q.bits, q.group_size, rtn_codes, rtn_scales, rtn_zeros, stream=stream)
        if ev:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pipeline.check_info(buf)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(args.steps):
        step(events[k])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    pipeline.check_info(buf)

    names = ["hessian", "prepare", "quantize", "pack", "rtn"]
    stage_ms = {nm: float(np.mean([events[k][i].elapsed_time(events[k][i + 1])
                                   for k in range(args.steps)])) for i, nm in enumerate(names)}
    hess_flops = n * (n + 1) * N
    prep_flops = 2 * n ** 3 / 3
    upd_flops = m * n * (n - q.block_size)
    hess_tf = hess_flops / (stage_ms["hessian"] * 1e-3) / 1e12
    value = m * n / (ms_per_step * 1e-3)

    roofline = {
        "bound": "mfma",
        "kernel": "hessian: gptq_hessian_accumulate (syrk_bf16_dma_kernel + reduce_full_partials_kernel)",
        "achieved": round(hess_tf, 2),
        "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(hess_tf / BF16_PEAK_TFLOPS, 4),
        "traffic": measured_traffic(),
        "algorithmic_work": f"n(n+1)N = {hess_flops:.4e} flop per launch",
        "launch_ms": round(stage_ms["hessian"], 4),
    }
    stages = {
        nm: {"ms": round(v, 4)} for nm, v in stage_ms.items()
    }
    stages["hessian"]["tflops"] = round(hess_tf, 2)
    stages["prepare"]["tflops_f64"] = round(prep_flops / (stage_ms["prepare"] * 1e-3) / 1e12, 3)
    stages["quantize"]["update_tflops_incl_block_loop"] = round(
        upd_flops / (stage_ms["quantize"] * 1e-3) / 1e12, 2)
    # the layer's roofline time: each stage at its own peak
    roof_ms = (hess_flops / (BF16_PEAK_TFLOPS * 1e12) + prep_flops / (FP64_PEAK_TFLOPS * 1e12)
               + upd_flops / (FP32_PEAK_TFLOPS * 1e12)
               + (m * n * (2 + 4 + 4 + 1) + m * n * (1 + q.bits / 8)) / (HBM_PEAK_GBS * 1e9)) * 1e3

    out = {
        "metric": "GPTQ layer weights quantized/sec; Hessian+update TFLOP/s as % MFMA peak",
        "value": round(value, 1),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->f32 MFMA (Hessian), f64 (prepare), f32 (column loop)",
        "data": "synthetic, seeded (normal activations, 0.5% outlier channels x30)",
        "config": {
            "workload": "Llama-7B-shaped attention projection 4096x4096, 128x2048 calibration "
                        "tokens, 4-bit asymmetric, group 128, block 128, damp 0.01, desc_act off",
            "m": m, "n": n, "tokens": N, "bits": q.bits, "group_size": q.group_size,
            "block_size": q.block_size, "perc_damp": q.perc_damp, "desc_act": q.desc_act,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "stages": stages,
        "layer_roofline_ms": round(roof_ms, 4),
        "layer_roofline_frac": round(roof_ms / ms_per_step, 4),
        "input_setup_s": round(t_gen, 1),
    }
    out["dequant_gemm"] = dequant_gemm_measure(gq, buf, X, m, n, q, stream)
    if not args.no_awq:
        out["awq"] = awq_measure(gq, W, X, buf.S, m, n, q, stream)
    if not args.no_stack:
        del X
        torch.cuda.empty_cache()
        out["layer_sequential"] = stack_measure(gq, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_rows, args.cpu_sample_chunks)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
