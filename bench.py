#!/usr/bin/env python3
"""Benchmark: GPTQ quantization of one linear layer on one MI355X.

Headline workload (one step = the whole layer path over one calibration set):
  70B-shaped down projection, W 8192 x 28672 bf16 ~ N(0, 0.01^2), calibration
  X = 256 sequences x 2048 tokens x 28672 bf16 ~ Laplace(0, 1), 4-bit
  asymmetric, group 64, block 128, damp 0.01, desc_act on (columns by
  descending Hessian diagonal).  The largest of the five workloads; the other
  four (256^2 fp32; Llama-7B attention 4096^2; Llama-7B MLP gate/up 11008 x
  4096 sharing one Hessian plus down 4096 x 11008; 70B square 8192^2 3-bit)
  are measured the same way and reported under ``configs``.  Inputs are
  synthetic, seeded, and resident in HBM before timing starts.

  step = S := 0; S += X^T X (all tokens); prepare (damp, order, Cholesky,
         inverse, upper factor); quantize (blocked column loop + lazy trailing
         update) of every layer sharing the Hessian; pack; plus the group
         min-max RTN baseline of each layer.

Prints ONE JSON line.  The metric is weights quantized per second
(m * n / step time).  ``roofline`` reports the dominant kernel (the bf16 MFMA
Hessian) against the MI355X dense bf16 MFMA peak, timed with HIP events on the
stream it runs on.  ``breakdown`` sums the durations of every kernel of one
extra step by kernel (from the profiler's activity trace), which separates the
column loop's block chain from its trailing-update products.  ``cpu_baseline``
times the fp64 oracle on a bounded sample of the headline workload on the host
cores and scales it to the same unit.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "llama70b_down"
EXTRA = ("layer256", "llama7b_attn", "llama7b_mlp", "llama70b_square")
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
FP64_PEAK_TFLOPS = 78.6
HBM_PEAK_GBS = 8000.0
HESSIAN_SRC = os.path.join(ROOT, "post_weight_quantization_22_amd", "csrc", "hessian.hip")
EXTRA_STEPS = {"layer256": (20, 3), "llama7b_attn": (10, 2), "llama7b_mlp": (5, 1),
               "llama70b_square": (5, 1)}


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_hessian_{workload}.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=HEADLINE,
                    help="headline workload (default: the 70B down projection)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other four workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-kernel breakdown of one extra step")
    ap.add_argument("--no-awq", action="store_true",
                    help="skip the AWQ-lite / awq_clip measurement")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the layer-sequential MLP-stack measurement")
    ap.add_argument("--no-dequant", action="store_true",
                    help="skip the dequantized-weight product measurement")
    ap.add_argument("--no-library-gemm", action="store_true",
                    help="skip the library bf16 product on the headline's tokens (context for "
                         "the Hessian's rate)")
    ap.add_argument("--library-gemm-probe", action="store_true",
                    help="run only the library bf16 product X^T X on the workload's first "
                         "65536 tokens, 1 + 8 times, for rocprofv3 counter runs, then exit")
    ap.add_argument("--cpu-sample-rows", type=int, default=512)
    ap.add_argument("--cpu-sample-chunks", type=int, default=2)
    ap.add_argument("--cpu-prepare-n", type=int, default=8192)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run one Hessian accumulate of the workload, one whole layer step "
                         "and one 2 GiB device copy, for rocprofv3 --pmc runs, then exit")
    ap.add_argument("--dequant-probe", action="store_true",
                    help="run the quantized layer's product 10 times at 2048 and at 16 tokens "
                         "(4096 x 4096, random 4-bit codes, group 128), for rocprofv3 counter "
                         "runs, then exit")
    ap.add_argument("--dequant-probe-layer", action="store_true",
                    help="as --dequant-probe, on the weight shape, width and group size of "
                         "--workload's layer (random codes, identity order), then exit")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter files of two --traffic-probe runs of --workload into "
                         "profiles/traffic_hessian_<workload>.json, then exit")
    return ap.parse_args()


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per Hessian kernel launch from committed rocprofv3 counter
    runs (the probe's one accumulate call over its launches), if current."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != source_hash(HESSIAN_SRC):
        return None  # the kernel changed since the counters were taken
    if "bytes_per_call" not in rec:
        return None
    return round(rec["bytes_per_call"] / max(1, rec.get("launches_per_call", 1)))


COPY_BYTES = 1 << 31  # the calibration copy of --traffic-probe
HESS_KERNELS = ("syrk_bf16_dma_kernel", "reduce_full_partials_kernel")
HESS_LAUNCH_TOKENS = 65536  # tokens per launch of an unsplit Hessian product


def short_kernel_name(name: str) -> str:
    """A kernel's name without return type, namespaces and argument list."""
    if name.startswith("void "):
        name = name[5:]
    name = name.replace("(anonymous namespace)::", "").split("(")[0]
    return name[len("gptq::"):] if name.startswith("gptq::") else name


def traffic_record(fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes of one Hessian launch from two counter runs of --traffic-probe.

    Each counter (KiB per dispatch, summed over the L2 channels) is scaled by
    the ratio of the known bytes of the 2 GiB device copy to what the same
    counter reads for that copy; the call is every dispatch of the Hessian
    kernels in the file (the probe's lone accumulate; the product kernel may
    run as several launches, counted in ``launches``).  Every other kernel of
    the probe's layer step is summed by name as well (``per_kernel``), for the
    quantize, pack and RTN bandwidths.
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
        factor = COPY_BYTES / (copy_kib * 1024.0)
        hess = 0.0
        ds = [d for d in val if HESS_KERNELS[0] in name[d]]
        if not ds:
            raise SystemExit(f"{path}: no Hessian dispatch")
        launches = len(ds)
        for k in HESS_KERNELS:
            hess += sum(val[d] for d in val if k in name[d])
        per_kernel = defaultdict(float)
        for d, v in val.items():
            if "copyBuffer" in name[d]:
                continue
            per_kernel[short_kernel_name(name[d])] += v * 1024.0 * factor
        out[counter] = {"hessian_kib": hess, "copy_kib": copy_kib, "scale": factor,
                        "bytes": hess * 1024.0 * factor, "launches": launches,
                        "per_kernel_bytes": dict(per_kernel)}
    return out


def upload_x(wl, xname, dev):
    """The calibration stream X [tokens, n] on the device (bf16 or fp32).

    Chunks are drawn on host threads (synth's generators), reduced to their
    storage bits there (the values are already bf16-exact), and copied in
    order while later chunks are still being drawn."""
    import numpy as np
    import torch

    import synth

    xs = wl.xs[xname]
    bf16 = xs.dtype == "bf16"
    X = torch.empty((xs.tokens, xs.n), dtype=torch.bfloat16 if bf16 else torch.float32,
                    device=dev)
    outl = synth.outlier_channels(wl, xname)

    def draw(c):
        a = synth.x_chunk(wl, xname, c, outl)
        if bf16:
            a = (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        return a

    threads = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(threads) as ex:
        futs = {}
        nxt = 0
        for c in range(xs.chunks):
            while nxt < xs.chunks and nxt < c + 2 * threads:
                futs[nxt] = ex.submit(draw, nxt)
                nxt += 1
            a = futs.pop(c).result()
            t = torch.from_numpy(a)
            if bf16:
                t = t.view(torch.bfloat16)
            X[c * xs.chunk_len:(c + 1) * xs.chunk_len].copy_(t)
    torch.cuda.synchronize()
    return X


def layer_groups(wl):
    """Layers that share a calibration stream share one Hessian and prepare."""
    groups = {}
    for l in wl.layers:
        groups.setdefault(l.x, []).append(l)
    return list(groups.items())


def stage_roof_ms(m, n, N, q, prep_peak=FP32_PEAK_TFLOPS, with_hessian=True):
    """A layer's time at roofline: Hessian n(n+1)N flop at the bf16 MFMA peak,
    prepare 2n^3/3 at ``prep_peak``, trailing update m n (n - 128) at the fp32
    MFMA peak, quantize + pack (9 + 8/G + 1 + b/8 bytes per weight) at HBM."""
    G = q.group_size if q.group_size > 0 else n
    t = 0.0
    if with_hessian:
        t += n * (n + 1) * N / (BF16_PEAK_TFLOPS * 1e12)
        t += 2 * n ** 3 / 3 / (prep_peak * 1e12)
    t += m * n * max(n - q.block_size, 0) / (FP32_PEAK_TFLOPS * 1e12)
    t += m * n * (9 + 8 / G + 1 + q.bits / 8) / (HBM_PEAK_GBS * 1e9)
    return t * 1e3


KERNEL_STAGE = (
    ("hessian", ("syrk_", "reduce_full_partials", "reduce_partials")),
    ("prepare", ("diag_damp", "rank_", "chunk_sort", "iota_kernel", "build_a", "sym_kernel",
                 "gather_a", "node_kernel", "gemm_f64",
                 "gemm_splitk", "gemm_tall128", "write_u")),
    ("quantize", ("prep_weights", "prep_rows", "block_quant", "update_gemm", "unpermute",
                  "static_params",
                  "row_params", "invert_perm", "fill_i32", "zero_f32")),
    ("pack", ("pack_",)),
    ("rtn", ("rtn_",)),
)


def kernel_breakdown(run_once):
    """Per-kernel duration sums of one call of ``run_once`` from torch's
    profiler (its activity trace records every kernel the process dispatches,
    the library's included).  Returns None when the trace holds no kernels."""
    import torch
    from torch.profiler import ProfilerActivity, profile

    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        run_once()
        torch.cuda.synchronize()
    per = {}
    for ev in prof.key_averages():
        dt = getattr(ev, "device_time_total", None)
        if dt is None:
            dt = getattr(ev, "cuda_time_total", 0.0)
        if not dt:
            continue
        name = short_kernel_name(ev.key)
        rec = per.setdefault(name, [0.0, 0])
        rec[0] += dt / 1e3
        rec[1] += ev.count
    if not per:
        return None
    return {k: {"ms": round(v[0], 4), "calls": v[1]} for k, v in
            sorted(per.items(), key=lambda kv: -kv[1][0])}


def stage_of(kernel: str):
    for st, prefixes in KERNEL_STAGE:
        if any(kernel.startswith(p) for p in prefixes):
            return st
    return None


def run_workload(gq, wl, dev, steps, warmup, breakdown=False, keep=False):
    """Time the whole path of a workload: per calibration stream one Hessian and
    one prepare, then quantize + pack + RTN of every layer that reads it.
    Returns (record, resident state of the last stream if ``keep``)."""
    import numpy as np
    import torch

    import synth
    from post_weight_quantization_22_amd import pipeline

    q = wl.quant
    cfg = gq.make_config(q.bits, q.group_size, q.block_size, q.perc_damp, q.desc_act, q.sym)
    stream = torch.cuda.current_stream()
    groups_out = []
    total_ms = 0.0
    total_weights = 0
    roof_ms = 0.0
    roof64_ms = 0.0
    t_setup = 0.0
    state = None
    for xname, layers in layer_groups(wl):
        xs = wl.xs[xname]
        n, N = xs.n, xs.tokens
        t0 = time.time()
        X = upload_x(wl, xname, dev)
        Ws = []
        for l in layers:
            Wh = synth.weight(wl, l.name)
            dt = torch.bfloat16 if l.w_dtype == "bf16" else torch.float32
            if l.w_dtype == "bf16":
                Ws.append(torch.from_numpy((Wh.view(np.uint32) >> np.uint32(16))
                                           .astype(np.uint16)).view(dt).to(dev))
            else:
                Ws.append(torch.from_numpy(Wh).to(dev))
            del Wh
        torch.cuda.synchronize()
        t_setup += time.time() - t0
        bufs = [pipeline.allocate(layers[0].m, n, cfg, N, device=dev)]
        for l in layers[1:]:
            b = pipeline.allocate(l.m, n, cfg, 0, device=dev)
            b.S, b.U, b.perm, b.dead = bufs[0].S, bufs[0].U, bufs[0].perm, bufs[0].dead
            bufs.append(b)
        rtn = []
        for l in layers:
            ng = pipeline.ngroups(n, q.group_size)
            rtn.append((torch.empty((l.m, n), dtype=torch.uint8, device=dev),
                        torch.empty((l.m, ng), dtype=torch.float32, device=dev),
                        torch.empty((l.m, ng), dtype=torch.float32, device=dev)))
        b0 = bufs[0]

        def step(ev=None):
            if ev:
                ev[0].record(stream)
            b0.S.zero_()
            gq.gptq_hessian_accumulate(b0.S, X, ws=b0.ws_hess, stream=stream)
            if ev:
                ev[1].record(stream)
            pipeline.prepare(b0, N, stream)
            if ev:
                ev[2].record(stream)
            for b, W in zip(bufs, Ws):
                pipeline.quantize(b, W, stream)
            if ev:
                ev[3].record(stream)
            for b in bufs:
                pipeline.pack(b, stream)
            if ev:
                ev[4].record(stream)
            for (c, s_, z), W in zip(rtn, Ws):
                gq.rtn_minmax(W, q.bits, q.group_size, c, s_, z, stream=stream)
            if ev:
                ev[5].record(stream)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        for b in bufs:
            pipeline.check_info(b)
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(steps):
            step(events[k])
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        for b in bufs:
            pipeline.check_info(b)
        names = ["hessian", "prepare", "quantize", "pack", "rtn"]
        stage_ms = {nm: float(np.mean([events[k][i].elapsed_time(events[k][i + 1])
                                       for k in range(steps)])) for i, nm in enumerate(names)}
        weights = sum(l.m for l in layers) * n
        hess_flops = n * (n + 1) * N
        prep_flops = 2 * n ** 3 / 3
        upd_flops = sum(l.m for l in layers) * n * max(n - q.block_size, 0)
        g_roof = stage_roof_ms(layers[0].m, n, N, q)
        g_roof64 = stage_roof_ms(layers[0].m, n, N, q, prep_peak=FP64_PEAK_TFLOPS)
        for l in layers[1:]:
            g_roof += stage_roof_ms(l.m, n, N, q, with_hessian=False)
            g_roof64 += stage_roof_ms(l.m, n, N, q, with_hessian=False)
        rec = {
            "layers": [f"{l.name} {l.m}x{l.n}" for l in layers],
            "tokens": N,
            "ms_per_step": round(ms, 4),
            "weights_per_s": round(weights / (ms * 1e-3), 1),
            "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
            "hessian_tflops": round(hess_flops / (stage_ms["hessian"] * 1e-3) / 1e12, 2),
            "hessian_frac_bf16_peak": round(hess_flops / (stage_ms["hessian"] * 1e-3) / 1e12
                                            / BF16_PEAK_TFLOPS, 4),
            "prepare_tflops_f64": round(prep_flops / (stage_ms["prepare"] * 1e-3) / 1e12, 3),
            "quantize_update_tflops_incl_block_loop": round(
                upd_flops / (stage_ms["quantize"] * 1e-3) / 1e12, 2),
            "layer_roofline_ms": round(g_roof, 4),
            "layer_roofline_frac": round(g_roof / ms, 4),
            "layer_roofline_ms_f64_prepare": round(g_roof64, 4),
            "layer_roofline_frac_f64_prepare": round(g_roof64 / ms, 4),
        }
        if breakdown:
            try:
                per = kernel_breakdown(step)
            except Exception as exc:  # the trace is optional evidence
                per = None
                rec["breakdown_error"] = str(exc)[:200]
            if per:
                rec["breakdown"] = per
                upd = sum(v["ms"] for k, v in per.items() if k.startswith("update_gemm"))
                chain = sum(v["ms"] for k, v in per.items() if k.startswith("block_quant"))
                rec["quantize_split"] = {
                    "block_chain_ms": round(chain, 4),
                    "update_gemm_ms": round(upd, 4),
                    "update_gemm_tflops": round(upd_flops / (upd * 1e-3) / 1e12, 2)
                    if upd else None,
                    "update_gemm_frac_fp32_peak": round(upd_flops / (upd * 1e-3) / 1e12
                                                        / FP32_PEAK_TFLOPS, 4) if upd else None,
                    "other_quantize_kernels_ms": round(sum(
                        v["ms"] for k, v in per.items() if stage_of(k) == "quantize") - upd
                        - chain, 4),
                }
                prep_gemm = sum(v["ms"] for k, v in per.items() if k.startswith("gemm_"))
                if prep_gemm:
                    rec["prepare_products_tflops_f64"] = round(
                        prep_flops / (prep_gemm * 1e-3) / 1e12, 2)
        groups_out.append(rec)
        total_ms += ms
        total_weights += weights
        roof_ms += g_roof
        roof64_ms += g_roof64
        if keep:
            state = dict(X=X, W=Ws[0], buf=b0, stream=stream, hess_flops=hess_flops, N=N, n=n,
                         m=layers[0].m, q=q)
        else:
            del X, Ws, bufs, rtn, b0
            torch.cuda.empty_cache()
    out = {
        "workload": wl.description,
        "ms_per_step": round(total_ms, 4),
        "weights_per_s": round(total_weights / (total_ms * 1e-3), 1),
        "layer_roofline_ms": round(roof_ms, 4),
        "layer_roofline_frac": round(roof_ms / total_ms, 4),
        "layer_roofline_ms_f64_prepare": round(roof64_ms, 4),
        "layer_roofline_frac_f64_prepare": round(roof64_ms / total_ms, 4),
        "steps": steps,
        "warmup": warmup,
        "input_setup_s": round(t_setup, 1),
        "streams": groups_out,
    }
    return out, state


def cpu_baseline(wl, rows: int, chunks: int, prep_n: int):
    """Time the fp64 oracle on a bounded sample and scale to weights/s for the
    whole workload: the Hessian over ``chunks`` calibration sequences (cost
    linear in tokens), prepare at n' = min(n, prep_n) on that sample's leading
    n' x n' block (cost ~ n^3), and the column loop on ``rows`` rows (rows are
    independent given U; the loop's work does not depend on U's values, so a
    unit upper factor stands in where n' < n)."""
    import numpy as np

    import oracle
    import synth

    q = wl.quant
    total = 0.0
    parts = []
    for xname, layers in layer_groups(wl):
        xs = wl.xs[xname]
        n = xs.n
        c = min(chunks, xs.chunks)
        Xs = synth.x_all(wl, xname, chunks=list(range(c)))
        t0 = time.perf_counter()
        S = oracle.hessian_S([Xs])
        t_h = time.perf_counter() - t0
        del Xs
        t_h_full = t_h * xs.chunks / c
        npr = min(n, prep_n)
        t0 = time.perf_counter()
        P = oracle.prepare(np.ascontiguousarray(S[:npr, :npr]), q.perc_damp, q.desc_act)
        t_p = time.perf_counter() - t0
        t_p_full = t_p * (n / npr) ** 3
        del S
        if npr == n:
            U, perm, dead = P.U, P.perm, P.dead
        else:
            U, perm, dead = np.eye(n), np.arange(n), None
        t_q_full = 0.0
        for l in layers:
            r = min(rows, l.m)
            W = synth.weight(wl, l.name, rows=slice(0, r))
            t0 = time.perf_counter()
            oracle.gptq_quantize(W, U, q.bits, q.group_size, q.block_size, perm, dead, q.sym)
            t_q = time.perf_counter() - t0
            t_q_full += t_q * l.m / r
        del U
        total += t_h_full + t_p_full + t_q_full
        parts.append(f"{xname}: Hessian over {c} of {xs.chunks} sequences ({t_h:.2f} s, scaled "
                     f"x{xs.chunks / c:g}), prepare at n={npr} ({t_p:.2f} s, scaled "
                     f"x{(n / npr) ** 3:.4g}), column loop on {min(rows, layers[0].m)} rows of "
                     f"each of {len(layers)} layer(s) (scaled to all rows"
                     + ("" if npr == n else "; unit upper factor") + ")")
    weights = sum(l.m * l.n for l in wl.layers)
    try:
        from threadpoolctl import threadpool_info

        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    return {
        "value": weights / total,
        "unit": "weights/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": "fp64 numpy/scipy oracle; " + "; ".join(parts)
                  + f"; estimated whole-workload time {total:.1f} s",
    }


def dequant_gemm_measure(gq, buf, X, m, n, q, stream, desc_act=False):
    """The quantized layer used: Y = X W_q^T from its packed codes (gptq_dequant_gemm).

    prefill: one 2048-token calibration sequence, bound by bf16 MFMA (2 tokens m n
    flop); decode: 16 tokens, bound by HBM (codes b/8 B, scale and zero 8 B per
    group, X and Y once per weight).  The decode launches are replayed from a
    HIP graph so that the host's launch cost is not timed.  With desc_act the
    codes are packed in processing order (gptq_pack_ordered) and the product
    gathers the activations into that order (timed with it)."""
    import torch

    out = {}
    ng = buf.scales.shape[1]
    packed, perm = buf.packed, None
    if desc_act:
        packed = torch.empty_like(buf.packed)
        gq.gptq_pack_ordered(buf.codes, q.bits, buf.perm, packed, stream=stream)
        perm = buf.perm
    for name, tokens, reps in (("prefill_2048", 2048, 20), ("decode_16", 16, 200)):
        Xt = X[:tokens]
        Y = torch.empty((tokens, m), dtype=torch.float32, device=X.device)
        nws = gq.gptq_dequant_gemm_workspace_size(tokens, m, n, perm is not None)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=X.device)

        def call():
            gq.gptq_dequant_gemm(Xt, packed, q.bits, q.group_size, buf.scales, buf.zeros,
                                 Y, perm=perm, ws=ws, stream=torch.cuda.current_stream())

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


def layer_error_measure(gq, W, buf, m, n, q, stream):
    """The layer objective ||W X - W_q X||^2 over the calibration tokens, from S, on the
    device (gptq_layer_error), for the step's GPTQ codes and for RTN's on the same
    layer; timed with HIP events (one call, after a warm-up), against the fp32 MFMA
    peak (2 m n^2 flop: the product of the differences with S)."""
    import torch

    err = torch.empty(m, dtype=torch.float64, device=W.device)
    ws = torch.empty(gq.gptq_layer_error_workspace_size(m, n), dtype=torch.uint8,
                     device=W.device)

    def call(codes, scales, zeros, g_idx):
        gq.gptq_layer_error(W, codes, scales, zeros, g_idx, buf.S, err, ws=ws, stream=stream)

    call(buf.codes, buf.scales, buf.zeros, buf.g_idx)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    call(buf.codes, buf.scales, buf.zeros, buf.g_idx)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    gptq = float(err.sum().item())
    rc, rs, rz = torch.empty_like(buf.codes), torch.empty_like(buf.scales), torch.empty_like(
        buf.zeros)
    gq.rtn_minmax(W, q.bits, q.group_size, rc, rs, rz, sym=bool(q.sym), stream=stream)
    G = q.group_size if q.group_size > 0 else n
    rg = (torch.arange(n, device=W.device, dtype=torch.int32) // G).contiguous()
    call(rc, rs, rz, rg)
    torch.cuda.synchronize()
    rtn = float(err.sum().item())
    tf = 2.0 * m * n * n / (ms * 1e-3) / 1e12
    return {"gptq": gptq, "rtn": rtn, "gptq_over_rtn": round(gptq / rtn, 4),
            "ms": round(ms, 3), "tflops": round(tf, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / FP32_PEAK_TFLOPS, 4)},
            "what": "sum over rows of delta_r S delta_r^T (gptq_layer_error), the step's GPTQ "
                    "codes and RTN (group min-max) on the same layer"}


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


def dequant_probe(gq, dev, m=4096, n=4096, bits=4, G=128):
    """Ten products at 2048 tokens, then ten at 16, on an m x n layer (default
    4096 x 4096, 4-bit g128) of random codes packed in processing order
    (identity order)."""
    import numpy as np
    import torch

    rng = np.random.default_rng(0)
    codes = torch.from_numpy(rng.integers(0, 2 ** bits, size=(m, n), dtype=np.uint8)).to(dev)
    packed = torch.empty((m, -(-n * bits // 32)), dtype=torch.int32, device=dev)
    gq.gptq_pack_ordered(codes, bits, None, packed)
    ng = -(-n // G) if G > 0 else 1
    scales = torch.from_numpy(rng.uniform(1e-3, 1e-2, size=(m, ng)).astype(np.float32)).to(dev)
    zeros = torch.from_numpy(rng.integers(0, 2 ** bits, size=(m, ng)).astype(np.float32)).to(dev)
    X = torch.from_numpy(rng.standard_normal((2048, n)).astype(np.float32)).to(dev).to(torch.bfloat16)
    for tokens in (2048, 16):
        Y = torch.empty((tokens, m), dtype=torch.float32, device=dev)
        nws = gq.gptq_dequant_gemm_workspace_size(tokens, m, n, False)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        for _ in range(10):
            gq.gptq_dequant_gemm(X[:tokens], packed, bits, G, scales, zeros, Y, ws=ws)
        torch.cuda.synchronize()
    print(f"dequant probe ({m} x {n}, {bits}-bit, group {G}): 10 products at 2048 and 10 at 16 "
          "tokens done", flush=True)


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
            "workload": args.workload,
            "bytes_per_call": round(t["FETCH_SIZE"]["bytes"] + t["WRITE_SIZE"]["bytes"]),
            "launches_per_call": t["FETCH_SIZE"]["launches"],
            "fetch": {k: v for k, v in t["FETCH_SIZE"].items()
                      if k not in ("per_kernel_bytes", "launches")},
            "write": {k: v for k, v in t["WRITE_SIZE"].items()
                      if k not in ("per_kernel_bytes", "launches")},
            "per_kernel_step_bytes": {
                k: {"fetch": round(t["FETCH_SIZE"]["per_kernel_bytes"].get(k, 0.0)),
                    "write": round(t["WRITE_SIZE"]["per_kernel_bytes"].get(k, 0.0))}
                for k in sorted(set(t["FETCH_SIZE"]["per_kernel_bytes"])
                                | set(t["WRITE_SIZE"]["per_kernel_bytes"]))},
            "calibration": f"device copy of {COPY_BYTES} bytes (read {COPY_BYTES}, write "
                           f"{COPY_BYTES})",
            "commands": [
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format "
                f"csv -d $OUT/pmc_fetch -o run -- python3 $REPO/bench.py "
                f"--traffic-probe --workload {args.workload}",
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format "
                f"csv -d $OUT/pmc_write -o run -- python3 $REPO/bench.py "
                f"--traffic-probe --workload {args.workload}",
                "python3 bench.py --traffic-record $OUT/pmc_fetch/run_counter_collection.csv "
                f"$OUT/pmc_write/run_counter_collection.csv --workload {args.workload}",
            ],
            "kernel_source_sha256": source_hash(HESSIAN_SRC),
        }
        with open(traffic_file(args.workload), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU split of the path is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import post_weight_quantization_22_amd as gq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.dequant_probe:
        dequant_probe(gq, dev)
        return
    if args.dequant_probe_layer:
        ls = synth.get_workload(args.workload).layer()
        q = synth.get_workload(args.workload).quant
        dequant_probe(gq, dev, ls.m, ls.n, q.bits, q.group_size)
        return

    wl = synth.get_workload(args.workload)
    if args.traffic_probe:
        traffic_probe(gq, wl, dev)
        return
    if args.library_gemm_probe:
        ls = wl.layer()
        X = upload_x(wl, ls.x, dev)
        rec = library_gemm_measure(X)
        print(f"library gemm probe ({wl.name}): {json.dumps(rec)}", flush=True)
        return

    print(f"bench: headline {args.workload}", file=sys.stderr, flush=True)
    head, hstate = run_workload(gq, wl, dev, args.steps, args.warmup,
                                breakdown=not args.no_breakdown, keep=not args.no_dequant)
    g0 = head["streams"][0]
    ls = wl.layer()
    xs = wl.xs[ls.x]
    n, N, q = xs.n, xs.tokens, wl.quant
    hess_flops = n * (n + 1) * N
    hess_ms = g0["stages_ms"]["hessian"]
    hess_tf = hess_flops / (hess_ms * 1e-3) / 1e12
    split = gq.gptq_hessian_workspace_size(n, N) > 0
    # launches of the product kernel per accumulate call: counted in the
    # profiled step, else the library's rule (an unsplit product runs one
    # launch per HESS_LAUNCH_TOKENS tokens)
    launches = g0.get("breakdown", {}).get(HESS_KERNELS[0], {}).get("calls")
    if not launches:
        launches = 1 if split else -(-N // HESS_LAUNCH_TOKENS)
    roofline = {
        "bound": "mfma",
        "kernel": "hessian: gptq_hessian_accumulate (syrk_bf16_dma_kernel"
                  + (" + reduce_full_partials_kernel" if split else "") + ")",
        "achieved": round(hess_tf, 2),
        "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(hess_tf / BF16_PEAK_TFLOPS, 4),
        "traffic": measured_traffic(args.workload),
        "algorithmic_work": f"n(n+1)N/launches = {hess_flops / launches:.4e} flop per launch "
                            f"({launches} launches per accumulate call, {N} tokens)",
        "launches_per_call": launches,
        "launch_ms": round(hess_ms / launches, 4),
        "call_ms": round(hess_ms, 4),
    }
    weights = sum(l.m * l.n for l in wl.layers)
    out = {
        "metric": "GPTQ layer weights quantized/sec; Hessian+update TFLOP/s as % MFMA peak",
        "value": round(weights / (head["ms_per_step"] * 1e-3), 1),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->f32 MFMA (Hessian), f64 (prepare), f32 (column loop)",
        "data": "synthetic, seeded (" + {
            "normal": "normal activations", "laplace": "Laplace(0, 1) activations",
            "student_t4": "Student-t (nu = 4) activations"}[xs.dist] + ")",
        "config": {
            "workload": WORKLOAD_LABEL.get(args.workload, wl.description),
            "m": ls.m, "n": n, "tokens": N, "bits": q.bits, "group_size": q.group_size,
            "block_size": q.block_size, "perc_damp": q.perc_damp, "desc_act": q.desc_act,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "stages": g0["stages_ms"],
        "layer_roofline_ms": head["layer_roofline_ms"],
        "layer_roofline_frac": head["layer_roofline_frac"],
        "layer_roofline_ms_f64_prepare": head["layer_roofline_ms_f64_prepare"],
        "layer_roofline_frac_f64_prepare": head["layer_roofline_frac_f64_prepare"],
        "input_setup_s": head["input_setup_s"],
        "detail": g0,
    }
    if hstate is not None and not args.no_library_gemm:
        print("bench: library bf16 product on the headline's tokens", file=sys.stderr, flush=True)
        lib = library_gemm_measure(hstate["X"])
        if lib is not None:
            lib["hessian_launch_over_library"] = round(hess_tf / lib["tflops"], 4)
        out["library_gemm"] = lib
    if hstate is not None:
        out["layer_error"] = layer_error_measure(gq, hstate["W"], hstate["buf"], hstate["m"],
                                                 hstate["n"], hstate["q"], hstate["stream"])
    if hstate is not None:
        # the headline layer's own product: its codes, its shape, its activation order
        print("bench: dequantized-weight product of the headline layer", file=sys.stderr,
              flush=True)
        out.setdefault("dequant_gemm", {})[args.workload] = dequant_gemm_measure(
            gq, hstate["buf"], hstate["X"], hstate["m"], hstate["n"], hstate["q"],
            hstate["stream"], desc_act=bool(hstate["q"].desc_act))
    del hstate
    torch.cuda.empty_cache()
    if not args.no_extra:
        configs = {}
        for name in EXTRA:
            if name == args.workload:
                continue
            print(f"bench: workload {name}", file=sys.stderr, flush=True)
            st, wu = EXTRA_STEPS[name]
            keep = name == "llama7b_attn" and not (args.no_awq and args.no_dequant)
            rec, state = run_workload(gq, synth.get_workload(name), dev, st, wu,
                                      breakdown=not args.no_breakdown, keep=keep)
            configs[name] = rec
            if state is not None:
                if not args.no_dequant:
                    out.setdefault("dequant_gemm", {})[name] = dequant_gemm_measure(
                        gq, state["buf"], state["X"], state["m"], state["n"], state["q"],
                        state["stream"], desc_act=bool(state["q"].desc_act))
                if not args.no_awq:
                    out["awq"] = awq_measure(gq, state["W"], state["X"], state["buf"].S,
                                             state["m"], state["n"], state["q"], state["stream"])
                del state
            torch.cuda.empty_cache()
        out["configs"] = configs
    if not args.no_stack:
        print("bench: layer-sequential stack", file=sys.stderr, flush=True)
        out["layer_sequential"] = stack_measure(gq, dev)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("bench: oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_rows, args.cpu_sample_chunks,
                                           args.cpu_prepare_n)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


WORKLOAD_LABEL = {
    "llama70b_down": "70B-shaped down projection 8192x28672 (28672^2 Hessian), 256x2048 "
                     "Laplace(0,1) bf16 calibration tokens, 4-bit asymmetric, group 64, block "
                     "128, damp 0.01, desc_act on",
    "llama7b_attn": "Llama-7B-shaped attention projection 4096x4096, 128x2048 calibration "
                    "tokens, 4-bit asymmetric, group 128, block 128, damp 0.01, desc_act off",
}


def library_gemm_measure(X, tokens: int = HESS_LAUNCH_TOKENS, calls: int = 8):
    """Context for the Hessian's rate, not a step of the path: the ROCm library's
    bf16 product (torch.mm, hipBLASLt) C = X^T X over the first ``tokens``
    calibration tokens, the whole n x n square (2 n^2 tokens flop), bf16 out,
    ``calls`` back to back after one warm-up, on the same values the Hessian
    reads.  Its sustained rate is what the chip delivers on these values under
    its power limit."""
    import torch

    if X.dtype != torch.bfloat16 or X.shape[0] < tokens:
        return None
    Xs = X[:tokens].contiguous()
    XT = Xs.t().contiguous()  # a plain row-major left operand
    n = Xs.shape[1]
    C = torch.mm(XT, Xs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        torch.mm(XT, Xs, out=C)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    flop = 2.0 * n * n * tokens
    del C, XT, Xs
    torch.cuda.empty_cache()
    return {
        "what": f"torch.mm bf16 X^T X over {tokens} of the same tokens, full {n} x {n} square, "
                f"bf16 out, {calls} calls after one warm-up (the library's sustained MFMA rate "
                "on these values; context, not a step of the path)",
        "ms_per_call": round(ms, 4),
        "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
        "frac_bf16_peak": round(flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
    }


def traffic_probe(gq, wl, dev):
    """One Hessian accumulate, one whole layer step (prepare, quantize, pack,
    RTN of the first layer) and a 2 GiB device copy, for counter runs."""
    import torch

    import synth
    from post_weight_quantization_22_amd import pipeline

    ls = wl.layer()
    xs = wl.xs[ls.x]
    q = wl.quant
    n, N = xs.n, xs.tokens
    X = upload_x(wl, ls.x, dev)
    W = torch.from_numpy(synth.weight(wl, ls.name)).to(dev)
    if ls.w_dtype == "bf16":
        W = W.to(torch.bfloat16)
    cfg = gq.make_config(q.bits, q.group_size, q.block_size, q.perc_damp, q.desc_act, q.sym)
    buf = pipeline.allocate(ls.m, n, cfg, N, device=dev)
    stream = torch.cuda.current_stream()
    buf.S.zero_()
    gq.gptq_hessian_accumulate(buf.S, X, ws=buf.ws_hess, stream=stream)
    torch.cuda.synchronize()
    del X
    torch.cuda.empty_cache()
    pipeline.prepare(buf, N, stream)
    pipeline.quantize(buf, W, stream)
    pipeline.pack(buf, stream)
    ng = pipeline.ngroups(n, q.group_size)
    gq.rtn_minmax(W, q.bits, q.group_size, torch.empty((ls.m, n), dtype=torch.uint8, device=dev),
                  torch.empty((ls.m, ng), dtype=torch.float32, device=dev),
                  torch.empty((ls.m, ng), dtype=torch.float32, device=dev), stream=stream)
    torch.cuda.synchronize()
    pipeline.check_info(buf)
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"traffic probe ({wl.name}): one Hessian accumulate, one layer step and one device "
          f"copy of {COPY_BYTES} bytes done", flush=True)


if __name__ == "__main__":
    main()
