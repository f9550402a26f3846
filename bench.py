#!/usr/bin/env python3
"""Decode-step benchmark of the weight-only quantised linear stack on one MI355X.

Default workload: the 70B-shaped outlier-INT4 decode stack (hidden 8192,
intermediate 28672, 80 layers, 64 q / 8 kv heads of 128), batch 1, every
weight resident in HBM.  One step = one decode pass through every linear of
every layer (q|k|v, o, gate|up, down per layer, each with its input
permutation), each product launched after the previous one has finished.
``--config 2`` runs the 3B-shaped stack, ``--config 3`` the 9B-shaped INT8
stack, ``--config 5`` the 9B INT8 stack streamed from pinned host memory and
``--config 1`` the single INT8 4096 x 4096 linear.

Prints one JSON line.  ``value`` is the achieved algorithmic bandwidth of the
whole step (bytes the method must move per step / step time); ``decode_tok_s``
is batch / step time.  ``roofline`` covers the dominant kernel (the product
kernel, every launch of the step), timed with HIP events on the stream it is
launched on.  ``cpu_baseline`` times the CPU oracle on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dequant-GEMV achieved HBM GB/s (% of peak) and decode tok/s, batch 1, 1 GPU"
HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(fmt: str, N: int, K: int, b: int) -> int:
    """Bytes the method must move for one linear call: codes (unpadded), scales,
    FP16 outlier columns, fp16 activations in and out."""
    if fmt == "int8":
        return N * K + 4 + 2 * b * (K + N)
    n_out = (K + 99) // 100
    K_bg = K - n_out
    G = -(-K_bg // 128)
    return (N * K_bg) // 2 + 2 * N * G + 2 * N * n_out + 2 * b * (K + N)


TRAFFIC_PROFILES = {
    # (config, batch) -> committed counter summary of that workload
    (4, 1): "profiles/qgemv_int4o_tile__70b_int4o_stack_b1__traffic.md",
    (2, 1): "profiles/qgemv_int4o_tile__3b_int4o_stack_b1__traffic.md",
    (3, 1): "profiles/qgemv_int8_valu__9b_int8_stack_b1__kernel_stats_traffic.md",
}


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("weight_only_quantized_quantize_amd/csrc/woq_gemv.h",
              "weight_only_quantized_quantize_amd/csrc/woq_device.hip"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg: int, b: int):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if there is none for this workload or the kernel sources
    changed since the counters were taken."""
    path = TRAFFIC_PROFILES.get((cfg, b))
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    fields = {}
    with open(os.path.join(ROOT, path)) as fh:
        for ln in fh:
            if ":" in ln and ln.split(":")[0] in ("traffic_bytes_per_launch", "kernel_source_sha256_16"):
                k, v = ln.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_baseline(spec, b: int, timed_s: float = 10.0, max_rows: int = 1024):
    """The oracle, untuned, on a bounded sample of the workload: the first
    ``max_rows`` output rows (all of them where a linear has fewer) of every
    linear of layer 0.

    prep   - the oracle's encoding of the sample.  INT4O: per input space the
             column sums of the sampled rows of every linear reading it, the
             scores against the space's profile, the top-1% selection and the
             permutation; per linear the group scales, codes, FP16 outlier
             columns and the 2:1 packing.  INT8: the per-tensor scale and codes
             of the sampled rows (the scale taken over the sample).
    decode - the sample's products at batch b, the activations' permutation
             and split included, repeated for about ``timed_s`` seconds.

    ``value`` is the decode rate in algorithmic bytes per second (the metric's
    unit), which a whole step would see; ``decode_tok_s`` is batch / the step
    time at that rate.  The prep rate is in fp32 weight bytes encoded per
    second.  Both run on all BLAS threads (elementwise NumPy is one thread);
    ``value_one_core`` repeats one decode pass with BLAS limited to one thread.
    """
    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    groups = ((("q", "k", "v"), 0), (("o",), 1), (("gate", "up"), 2), (("down",), 3))
    Ws, rows = {}, {}
    for lin in spec.linears():
        R = min(lin.N, max_rows)
        Ws[lin.name] = np.ascontiguousarray(synth.weight(spec, 0, lin)[:R])
        rows[lin.name] = R
    fp32_bytes = sum(W.nbytes for W in Ws.values())

    # prep
    t0 = time.perf_counter()
    enc, perms = {}, {}
    if spec.fmt == "int4o":
        for space in sorted({lin.space for lin in spec.linears()}):
            K = spec.space_width(space)
            colabs = O.space_column_abs_sum(Ws[lin.name] for lin in spec.linears() if lin.space == space)
            scores = O.outlier_scores(colabs, synth.profile(spec, space))
            perms[space] = O.global_perm(K, O.select_outliers(scores, O.n_outliers(K)))
        for lin in spec.linears():
            c, sc, wo = O.quantize_int4o(Ws[lin.name], perms[lin.space], O.n_outliers(lin.K))
            O.pack_int4(c)
            enc[lin.name] = (c, sc, wo)
    else:
        for lin in spec.linears():
            enc[lin.name] = O.quantize_int8(Ws[lin.name])
    prep_s = time.perf_counter() - t0
    del Ws

    xs = {inp: synth.decode_input(spec, 0, inp, b) for _, inp in groups}

    def one_pass():
        for names, inp in groups:
            x = xs[inp]
            if spec.fmt == "int4o":
                lin0 = spec.linear(names[0])
                x_bg, x_out = O.permute_split(x, perms[lin0.space], O.n_outliers(lin0.K))
                for n in names:
                    O.linear_int4o(*enc[n], x_bg, x_out)
            else:
                for n in names:
                    O.linear_int8(*enc[n], x)

    sample_bytes = sum(algorithmic_bytes(spec.fmt, rows[lin.name], lin.K, b) for lin in spec.linears())
    step_bytes = spec.layers * sum(algorithmic_bytes(spec.fmt, lin.N, lin.K, b) for lin in spec.linears())
    one_pass()                                       # untimed (page faults, thread-pool start)
    t_dec, passes = 0.0, 0
    while t_dec < timed_s:
        t0 = time.perf_counter()
        one_pass()
        t_dec += time.perf_counter() - t0
        passes += 1
    rate = sample_bytes * passes / t_dec
    one_core = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            one_pass()
            one_core = round(sample_bytes / (time.perf_counter() - t0) / 1e9, 4)
    except ImportError:
        pass
    covered = sample_bytes / (step_bytes / spec.layers)
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "value_one_core": one_core,
            "decode_tok_s": round(b / (step_bytes / rate), 5),
            "prep_s": round(prep_s, 3), "prep_fp32_gbs": round(fp32_bytes / prep_s / 1e9, 4),
            "decode_s": round(t_dec, 2), "decode_passes": passes,
            "sample": f"float64 NumPy oracle on the first {max_rows} output rows (all rows of shorter linears) of "
                      f"each of the 7 linears of layer 0 ({covered:.1%} of one layer's algorithmic bytes, "
                      f"{1 / spec.layers:.2%} of the layers): prep (encoding, {fp32_bytes / 1e6:.0f} MB of fp32 "
                      f"weights) timed once, {prep_s:.1f} s; decode products at batch {b} in {passes} timed passes, "
                      f"{t_dec:.1f} s; the decode rate is scaled to a whole step; host os.cpu_count()="
                      f"{os.cpu_count()}, BLAS threads={blas_threads}"}


def stream_read_ceiling(stream, reps: int = 10) -> float:
    """GB/s of the library's plain streaming-read kernel over 1 GiB (larger than
    the 256 MB last-level cache), timed with events on `stream`."""
    import torch
    from weight_only_quantized_quantize_amd import woq
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for _ in range(2):
            woq.woq_stream_read(buf, stream)
        e0.record(stream)
        for _ in range(reps):
            woq.woq_stream_read(buf, stream)
        e1.record(stream)
    e1.synchronize()
    del buf
    return (1 << 30) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def bench_single(args):
    """One INT8 linear, 4096 x 4096, batch 1: the product alone, launched back
    to back over 32 copies of the weights (537 MB, more than the last-level
    cache), timed with events over the steps."""
    import torch
    import synth
    from weight_only_quantized_quantize_amd import woq
    W, x = synth.config1_inputs()
    q, sc = woq.woq_quantize_int8(W)
    copies = 32
    devs = [woq.DeviceInt8([(q, sc)]) for _ in range(copies)]
    del W
    xd = torch.from_numpy(x.copy()).cuda()
    y = torch.empty(1, 4096, dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(max(args.warmup, copies)):
        woq.woq_qgemv_int8(devs[i % copies].desc, xd, y, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        woq.woq_qgemv_int8(devs[i % copies].desc, xd, y, stream)
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = algorithmic_bytes("int8", 4096, 4096, 1)
    value = nbytes / (ms * 1e-3) / 1e9
    ceiling = stream_read_ceiling(stream)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16xf16->f32 on int8 codes", "data": "synthetic",
        "config": {"workload": "single INT8 linear 4096x4096, batch 1, weights rotated over 32 copies",
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "kernel": "qgemv_int8_valu", "achieved": round(value, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
                     "stream_read_ceiling_gbs": round(ceiling, 1), "frac_of_stream_ceiling": round(value / ceiling, 4)},
    }
    print(json.dumps(result), flush=True)


def copy_calibration():
    """Three device-to-device copies of 1 GiB: each reads and writes exactly
    2**30 bytes, which fixes the scale of the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    x = torch.empty(2 ** 30, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copied_bytes": 3 * 2 ** 30, "copies": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="4 (default): 70B INT4O, 2: 3B INT4O, 3: 9B INT8 (resident stacks); "
                         "5: 9B INT8 streamed from pinned host memory; 1: one INT8 4096x4096 linear")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None, help="resident layers (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pool-roundtrip", action="store_true",
                    help="stacks 2-4: encode every layer, save the pool file under $TMPDIR, load it back, run a "
                         "pass (checked against the in-memory stack) and report the times")
    ap.add_argument("--prep", action="store_true",
                    help="stacks 2-4: time the encoders (device and host) on the linears of one layer")
    ap.add_argument("--hbm-budget", type=float, default=None,
                    help="stacks 2-4: device-memory budget in GB for the weights; the first layers stay resident, "
                         "the rest stream from pinned host memory (tiered pass)")
    ap.add_argument("--no-vocab", action="store_true",
                    help="outlier-INT4 stacks: skip the INT8 token lookup and tied lm_head timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB on the device three times (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on exactly one GPU (the decode linears are measured on one "
              "device's share); --gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from weight_only_quantized_quantize_amd import woq
    from weight_only_quantized_quantize_amd.stack import GROUPS, ResidentStack

    woq.require_gpu()
    if args.config == 1:
        return bench_single(args)
    spec = synth.stack_spec(args.config)
    b = args.batch or spec.batches[0]
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731
    if args.config == 5:
        return bench_streamed(args, spec, b, log)
    if args.prep:
        return bench_prep(args, spec, log)
    if args.pool_roundtrip:
        return bench_pool(args, spec, b, log)
    if args.hbm_budget is not None:
        return bench_tiered(args, spec, b, log)
    t0 = time.perf_counter()
    rs = ResidentStack(spec, lambda layer, lin, out: synth.weight(spec, layer, lin, out=out),
                       lambda space: synth.profile(spec, space), layers=args.layers, log=log)
    L = rs.n_layers
    log(f"prepared {L} layers in {time.perf_counter() - t0:.1f} s; {rs.device_bytes() / 1e9:.3f} GB resident")

    inputs, outputs = [], []
    for layer in range(L):
        for names, inp in GROUPS:
            x = synth.decode_input(spec, layer, inp, b)
            inputs.append(torch.from_numpy(x).cuda())
            N = sum(spec.linear(n).N for n in names)
            outputs.append(torch.empty(b, N, dtype=torch.float16, device="cuda"))
    runner = rs.make_runner(max(b, 1))
    runner.bind(inputs, outputs)
    stream = torch.cuda.current_stream()

    shapes = rs.group_shapes()
    step_bytes = sum(algorithmic_bytes(spec.fmt, N, K, b) for N, K, _ in shapes)
    for _ in range(args.warmup):
        runner.run(b, stream)
    torch.cuda.synchronize()

    # timed region: K passes without instrumentation
    t_start = time.perf_counter()
    for _ in range(args.steps):
        runner.run(b, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    # the same K passes with HIP events at every step's own dispatch
    # boundaries (from the start of its first launch to the end of its last)
    step_ms, pass_ms = runner.time(b, args.steps, stream)
    launches = runner.launches(b)
    kern_ms = sum(step_ms)
    if spec.fmt == "int4o":
        if b <= 2:
            kname = "qgemv_int4o_tile (vector kernel; permutation folded in)"
        elif launches > 2 * len(shapes):
            kname = "woq_permute_x + qgemm_int4o_mfma + split-K reduction"
        elif launches == 2 * len(shapes):
            kname = "woq_permute_x + qgemm_int4o_mfma"
        else:
            kname = "qgemm_int4o_mfma (permutation folded in where the permuted row fits on chip)"
    else:
        kname = "qgemv_int8_valu" if b < 4 else "qgemv_int8_valu + qgemm_int8_mfma"
    # Dispatch-boundary spans of consecutive launches overlap by part of the
    # dispatch, so their sum can exceed the pass.  The per-launch figure is
    # used only when it fits inside the measured step; otherwise the step
    # itself is the kernel time (an upper bound on it).
    if kern_ms <= ms_per_step:
        basis, kernel_ms = "launch", kern_ms
    else:
        basis, kernel_ms = "step", ms_per_step
    achieved = step_bytes / (kernel_ms * 1e-3) / 1e9
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # per product of a layer: mean span over the layers and its rate
    per_product = []
    for gi, (names, _) in enumerate(GROUPS):
        idx = range(gi, len(shapes), len(GROUPS))
        N, K, _ = shapes[gi]
        by = algorithmic_bytes(spec.fmt, N, K, b)
        us = 1e3 * sum(step_ms[i] for i in idx) / len(idx)
        per_product.append({"product": "|".join(names), "N": N, "K": K, "algorithmic_bytes": by,
                            "mean_us": round(us, 3), "gbs": round(by / (us * 1e-6) / 1e9, 1),
                            "frac": round(by / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32 on int4 codes" if spec.fmt == "int4o" else "f16xf16->f32 on int8 codes",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}, batch {b}" + (f", {L} layers resident" if L != spec.layers else
                                                            ", every layer resident in HBM"),
                   "format": spec.fmt, "layers": L, "hidden": spec.hidden, "intermediate": spec.inter,
                   "q_heads": spec.q_heads, "kv_heads": spec.kv_heads, "head_dim": spec.head_dim,
                   "batch": b, "launches_per_step": launches, "products_per_step": len(shapes),
                   "algorithmic_bytes_per_step": step_bytes},
        "decode_tok_s": round(b / (ms_per_step * 1e-3), 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.config, b),
                     "basis": basis,
                     "launches_per_step": launches,
                     "sum_of_step_spans_ms": round(kern_ms, 5), "events_pass_ms": round(pass_ms, 5),
                     "mean_launch_us": round(1e3 * kernel_ms / launches, 3),
                     "mean_algorithmic_bytes_per_launch": step_bytes // launches,
                     "per_product": per_product},
    }
    if spec.fmt == "int4o" and not args.no_vocab:
        result["vocab"] = bench_vocab(args, spec, rs, b, runner.run, stream, log)
    ceiling = stream_read_ceiling(stream)
    result["roofline"]["stream_read_ceiling_gbs"] = round(ceiling, 1)
    result["roofline"]["frac_of_stream_ceiling"] = round(achieved / ceiling, 4)
    # What a dependent launch costs before its own work, measured on an empty
    # kernel of one 256-thread workgroup per compute unit: the mean interval of
    # such launches back to back (no per-launch events).  The latency model of
    # a step is one interval per launch plus the step's bytes at the
    # streaming-read rate; the step reaches frac_of_interval_plus_stream of it.
    span_us, interval_us = woq.woq_dispatch_floor(256, 256, 200, stream)
    model_ms = launches * interval_us * 1e-3 + step_bytes / (ceiling * 1e9) * 1e3
    result["roofline"]["empty_launch_span_us"] = round(span_us, 3)
    result["roofline"]["empty_launch_interval_us"] = round(interval_us, 3)
    result["roofline"]["interval_plus_stream_ms"] = round(model_ms, 5)
    result["roofline"]["frac_of_interval_plus_stream"] = round(model_ms / ms_per_step, 4)
    runner.close()
    del rs
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(spec, b)
    print(json.dumps(result), flush=True)


def bench_vocab(args, spec, rs, b, run, stream, log):
    """The steps on either side of the stack: INT8 token lookup before it and
    the tied outlier-INT4 lm_head after it, timed alone (HIP events) and as
    part of a whole decode step (lookup, stack pass, lm_head)."""
    import numpy as np
    import torch
    import synth
    from weight_only_quantized_quantize_amd.stack import TiedVocab

    t0 = time.perf_counter()
    E = synth.embedding(spec)
    tv = TiedVocab(E, rs.perm_host["h"], max_b=b)
    del E
    V, H = tv.V, tv.H
    log(f"tied vocabulary {V}x{H} prepared in {time.perf_counter() - t0:.1f} s; "
        f"{tv.device_bytes() / 1e9:.3f} GB resident")
    ids = torch.from_numpy(synth.token_ids(spec, b)).cuda()
    emb = torch.empty(b, H, dtype=torch.float16, device="cuda")
    h = torch.from_numpy(synth.decode_input(spec, spec.layers, 0, b)).cuda()   # the hidden state after the stack
    logits = torch.empty(b, V, dtype=torch.float16, device="cuda")

    def timed(fn, n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(3):
            fn()
        ev[0].record(stream)
        for _ in range(n):
            fn()
        ev[1].record(stream)
        ev[1].synchronize()
        return ev[0].elapsed_time(ev[1]) / n

    n = max(args.steps, 20)
    embed_ms = timed(lambda: tv.embed(ids, emb, stream), n)
    head_ms = timed(lambda: tv.logits(h, logits, stream), n)

    def step():
        tv.embed(ids, emb, stream)
        run(b, stream)
        tv.logits(h, logits, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    full_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    head_bytes = algorithmic_bytes("int4o", V, H, b)
    embed_bytes = b * H * 3 + 4 * b + 4
    return {"vocab": V, "hidden": H, "table_bytes": int(tv.table.nbytes),
            "embed_us": round(embed_ms * 1e3, 3), "embed_algorithmic_bytes": embed_bytes,
            "lm_head_us": round(head_ms * 1e3, 3), "lm_head_algorithmic_bytes": head_bytes,
            "lm_head_gbs": round(head_bytes / (head_ms * 1e-3) / 1e9, 1),
            "lm_head_launches": 2,
            "ms_per_step_with_vocab": round(full_ms, 5),
            "decode_tok_s_with_vocab": round(b / (full_ms * 1e-3), 2)}


def bench_pool(args, spec, b, log):
    """Persisted pool: encode (host, all threads) into a pinned pool, save the
    file, load it into a fresh stack (every layer read into pinned memory, or
    through it into device memory for the layers a budget keeps resident) and
    run one pass; the loaded stack's outputs must equal the original's bit for
    bit.  The file is deleted afterwards."""
    import tempfile

    import torch
    import synth
    from weight_only_quantized_quantize_amd.stack import GROUPS, PooledStack, TieredStack

    L = args.layers or spec.layers
    t0 = time.perf_counter()
    ts = TieredStack(spec, lambda layer, lin, out: synth.weight(spec, layer, lin, out=out),
                     lambda space: synth.profile(spec, space), 0, layers=L, resident=[0] * L, log=log)
    encode_s = time.perf_counter() - t0
    fd, path = tempfile.mkstemp(suffix=".woqpool")
    os.close(fd)
    try:
        t0 = time.perf_counter()
        ts.save_pool(path)
        save_s = time.perf_counter() - t0
        file_bytes = os.path.getsize(path)
        inputs, outs_a, outs_b = [], [], []
        for layer in range(L):
            for names, inp in GROUPS:
                inputs.append(torch.from_numpy(synth.decode_input(spec, layer, inp, b)).cuda())
                N = sum(spec.linear(n).N for n in names)
                outs_a.append(torch.empty(b, N, dtype=torch.float16, device="cuda"))
                outs_b.append(torch.empty(b, N, dtype=torch.float16, device="cuda"))
        compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
        pa = ts.make_pager(b)
        pa.bind(inputs, outs_a)
        pa.run(b, compute, copy)
        torch.cuda.synchronize()
        pa.close()
        del ts, pa
        budget = int(args.hbm_budget * 1e9) if args.hbm_budget is not None else None
        t0 = time.perf_counter()
        ps = PooledStack(path, budget_bytes=budget, resident=None if budget is not None else [1] * L)
        load_s = time.perf_counter() - t0
        pb = ps.make_pager(b)
        pb.bind(inputs, outs_b)
        pb.run(b, compute, copy)
        torch.cuda.synchronize()
        pb.close()
        same = all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(outs_a, outs_b))
    finally:
        os.remove(path)
    print(json.dumps({
        "workload": f"{spec.name}" + (f", {L} layers" if L != spec.layers else "") + ": persisted pool round trip",
        "format": spec.fmt, "layers": L, "file_bytes": file_bytes, "encode_s": round(encode_s, 2),
        "save_s": round(save_s, 2), "save_gbs": round(file_bytes / save_s / 1e9, 2),
        "load_s": round(load_s, 2), "load_gbs": round(file_bytes / load_s / 1e9, 2),
        "loaded_resident_layers": ps.n_resident, "outputs_equal_after_load": bool(same),
        "note": "load right after save reads from the page cache"}), flush=True)


def bench_prep(args, spec, log):
    """Encoders on the seven linears of layer 0: the device encoder (fp32
    weights already in device memory, HIP events around the encoder launches)
    against the host encoder plus the host layout transform (wall clock, all
    host threads).  Both give the same bytes (checked here)."""
    import numpy as np
    import torch
    import synth
    from weight_only_quantized_quantize_amd import woq

    lins = spec.linears()
    Ws = [synth.weight(spec, 0, lin) for lin in lins]
    perms = {}
    if spec.fmt == "int4o":
        # the selector over this layer's linears (the stack selects over all layers)
        for sp in sorted({lin.space for lin in lins}):
            perms[sp] = woq.woq_outlier_perm([W for lin, W in zip(lins, Ws) if lin.space == sp],
                                             synth.profile(spec, sp))
    stream = torch.cuda.current_stream()
    dev_out, host_out = [], []
    Wd = [torch.from_numpy(W).cuda() for W in Ws]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run_device():
        outs = []
        for lin, W in zip(lins, Wd):
            if spec.fmt == "int4o":
                g = woq.woq_int4o_geometry(lin.K)
                cb, sb, wb = woq.woq_int4o_dev_sizes(lin.N, g)
                c = torch.empty(cb, dtype=torch.uint8, device="cuda")
                sc = torch.empty(sb // 2, dtype=torch.int16, device="cuda")
                wo = torch.empty(wb // 2, dtype=torch.int16, device="cuda")
                pd = torch.from_numpy(perms[lin.space]).cuda()
                outs.append((c, sc, wo, pd))
            else:
                outs.append((torch.empty(woq.lib().woq_int8_dev_bytes(lin.N, lin.K), dtype=torch.uint8,
                                         device="cuda"), torch.empty(1, dtype=torch.float32, device="cuda")))
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for lin, W, o in zip(lins, Wd, outs):
            if spec.fmt == "int4o":
                woq.woq_quantize_int4o_dev(W, o[3], woq.woq_int4o_geometry(lin.K), o[0], o[1], o[2], status, stream)
            else:
                woq.woq_quantize_int8_dev(W, o[0], o[1], status, stream)
        ev[1].record(stream)
        ev[1].synchronize()
        return ev[0].elapsed_time(ev[1]), outs

    run_device()                                   # warm-up
    dev_ms, dev_out = min((run_device() for _ in range(3)), key=lambda t: t[0])
    t0 = time.perf_counter()
    for lin, W in zip(lins, Ws):
        if spec.fmt == "int4o":
            g = woq.woq_int4o_geometry(lin.K)
            host_out.append(woq.woq_layout_int4o(*woq.woq_quantize_int4o(W, perms[lin.space]), g))
        else:
            q, sc = woq.woq_quantize_int8(W)
            host_out.append((woq.woq_layout_int8(q), sc))
    host_ms = (time.perf_counter() - t0) * 1e3
    same = True
    for d, h in zip(dev_out, host_out):
        if spec.fmt == "int4o":
            same &= np.array_equal(d[0].cpu().numpy(), h[0]) and np.array_equal(d[1].cpu().numpy().view(np.uint16), h[1])
            same &= np.array_equal(d[2].cpu().numpy().view(np.uint16), h[2])
        else:
            same &= np.array_equal(d[0].cpu().numpy(), h[0]) and float(d[1].cpu()[0]) == float(h[1])
    fp32_bytes = sum(W.nbytes for W in Ws)
    print(json.dumps({
        "workload": f"{spec.name}: encoders on the {len(lins)} linears of one layer",
        "format": spec.fmt, "fp32_weight_bytes": fp32_bytes,
        "device_ms": round(dev_ms, 3), "device_gbs_fp32_in": round(fp32_bytes / (dev_ms * 1e-3) / 1e9, 1),
        "host_ms": round(host_ms, 1), "host_gbs_fp32_in": round(fp32_bytes / (host_ms * 1e-3) / 1e9, 2),
        "host_threads": os.cpu_count(), "device_equals_host": bool(same),
        "status": int(status.cpu()[0])}), flush=True)


def bench_tiered(args, spec, b, log):
    """Tiered decode under a device-memory budget: the planner keeps the first
    layers resident and streams the rest from one pinned host pool through two
    device slots.  ``value`` is the algorithmic bandwidth of the whole step;
    the overlap efficiency compares the step with the serial copy time of the
    streamed blocks at the measured host-to-device bandwidth."""
    import statistics

    import torch
    import synth
    from weight_only_quantized_quantize_amd.stack import GROUPS, TieredStack

    budget = int(args.hbm_budget * 1e9)
    t0 = time.perf_counter()
    ts = TieredStack(spec, lambda layer, lin, out: synth.weight(spec, layer, lin, out=out),
                     lambda space: synth.profile(spec, space), budget, layers=args.layers, log=log)
    L, nA = ts.n_layers, ts.n_resident
    streamed_bytes = ts.streamed_bytes()
    log(f"prepared {L} layers in {time.perf_counter() - t0:.1f} s: {nA} resident, {L - nA} streamed "
        f"({streamed_bytes / 1e9:.2f} GB pinned, {ts.block_bytes / 1e6:.1f} MB per layer)")
    inputs, outputs = [], []
    for layer in range(L):
        for names, inp in GROUPS:
            inputs.append(torch.from_numpy(synth.decode_input(spec, layer, inp, b)).cuda())
            outputs.append(torch.empty(b, sum(spec.linear(n).N for n in names), dtype=torch.float16, device="cuda"))
    pager = ts.make_pager(b)
    pager.bind(inputs, outputs)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    step_bytes = L * sum(algorithmic_bytes(spec.fmt, sum(spec.linear(n).N for n in names), spec.linear(names[0]).K, b)
                         for names, _ in GROUPS)

    bw_h2d = None
    copy_pass_ms = None
    if streamed_bytes:
        slot = torch.empty(ts.block_bytes, dtype=torch.uint8, device="cuda")
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        copy_ms = []
        nB = L - nA
        with torch.cuda.stream(copy):
            for i in range(12):
                j = i % nB
                blk = ts.pool[j * ts.block_bytes:(j + 1) * ts.block_bytes]
                ev0.record(copy)
                slot.copy_(blk, non_blocking=True)
                ev1.record(copy)
                ev1.synchronize()
                if i >= 2:
                    copy_ms.append(ev0.elapsed_time(ev1))
        bw_h2d = ts.block_bytes / (statistics.median(copy_ms) * 1e-3) / 1e9
        log(f"host-to-device: {bw_h2d:.2f} GB/s (median of {len(copy_ms)} copies of {ts.block_bytes / 1e6:.1f} MB)")
        # the pass's copies alone: every streamed block once, back to back into
        # two alternating slots (the link's sustained rate), median of three
        slots = [slot, torch.empty(ts.block_bytes, dtype=torch.uint8, device="cuda")]
        pass_ms = []
        for _ in range(3):
            with torch.cuda.stream(copy):
                ev0.record(copy)
                for j in range(nB):
                    slots[j % 2].copy_(ts.pool[j * ts.block_bytes:(j + 1) * ts.block_bytes], non_blocking=True)
                ev1.record(copy)
            ev1.synchronize()
            pass_ms.append(ev0.elapsed_time(ev1))
        copy_pass_ms = statistics.median(pass_ms)
        del slot, slots
        log(f"copies of the {nB} streamed blocks alone: {copy_pass_ms:.1f} ms")

    for _ in range(args.warmup):
        pager.run(b, compute, copy)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        pager.run(b, compute, copy)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    pager.close()
    copy_serial_ms = streamed_bytes / (bw_h2d * 1e9) * 1e3 if bw_h2d else 0.0
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32 on int4 codes" if spec.fmt == "int4o" else "f16xf16->f32 on int8 codes",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}, batch {b}, {args.hbm_budget:g} GB device budget: "
                               f"{nA} layers resident, {L - nA} streamed from pinned host memory",
                   "format": spec.fmt, "layers": L, "hidden": spec.hidden, "intermediate": spec.inter,
                   "q_heads": spec.q_heads, "kv_heads": spec.kv_heads, "head_dim": spec.head_dim, "batch": b,
                   "runner": "tiered", "hbm_budget_bytes": budget, "resident_layers": nA,
                   "streamed_layers": L - nA, "layer_block_bytes": ts.block_bytes,
                   "algorithmic_bytes_per_step": step_bytes},
        "decode_tok_s": round(b / (ms_per_step * 1e-3), 3),
        "tiered": {"planned_device_bytes": int(ts.planned_device_bytes), "streamed_bytes_per_step": streamed_bytes,
                   "h2d_gbs_measured": round(bw_h2d, 3) if bw_h2d else None,
                   "copy_serial_ms": round(copy_serial_ms, 3),
                   "copy_pass_ms": round(copy_pass_ms, 3) if copy_pass_ms else None,
                   "overlap_efficiency": round(copy_serial_ms / ms_per_step, 4) if bw_h2d else None,
                   "overlap_efficiency_vs_copy_pass": round(copy_pass_ms / ms_per_step, 4) if copy_pass_ms else None},
    }
    print(json.dumps(result), flush=True)


def bench_streamed(args, spec, b, log):
    """Streamed INT8 decode: every layer lives in one pinned host pool and is
    copied into one of two device slots on a side stream while the previous
    layer computes.  ``value`` is the algorithmic bandwidth of the whole step;
    the overlap efficiency compares the step with the serial copy time at the
    measured host-to-device bandwidth."""
    import statistics

    import torch
    import synth
    from weight_only_quantized_quantize_amd import woq
    from weight_only_quantized_quantize_amd.stack import GROUPS, StreamedInt8Stack

    t0 = time.perf_counter()
    ss = StreamedInt8Stack(spec, lambda layer, lin, out: synth.weight(spec, layer, lin, out=out), layers=args.layers,
                           log=log)
    L = ss.n_layers
    pool_bytes = L * ss.block_bytes
    log(f"prepared {L} layers in {time.perf_counter() - t0:.1f} s; pinned pool {pool_bytes / 1e9:.3f} GB")
    inputs, outputs = [], []
    for layer in range(L):
        for names, inp in GROUPS:
            inputs.append(torch.from_numpy(synth.decode_input(spec, layer, inp, b)).cuda())
            outputs.append(torch.empty(b, sum(spec.linear(n).N for n in names), dtype=torch.float16, device="cuda"))
    pager = ss.make_pager(b)
    pager.bind(inputs, outputs)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    step_bytes = sum(algorithmic_bytes("int8", st.w.N, st.w.K, b) for st in ss.steps)

    # host-to-device bandwidth: median of 20 pinned copies of one layer block
    slot = torch.empty(ss.block_bytes, dtype=torch.uint8, device="cuda")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    copy_ms = []
    with torch.cuda.stream(copy):
        for i in range(22):
            blk = ss.pool[(i % L) * ss.block_bytes:(i % L + 1) * ss.block_bytes]
            ev0.record(copy)
            slot.copy_(blk, non_blocking=True)
            ev1.record(copy)
            ev1.synchronize()
            if i >= 2:
                copy_ms.append(ev0.elapsed_time(ev1))
    bw_h2d = ss.block_bytes / (statistics.median(copy_ms) * 1e-3) / 1e9
    log(f"host-to-device: {bw_h2d:.2f} GB/s (median of {len(copy_ms)} copies of {ss.block_bytes / 1e6:.1f} MB)")
    # the pass's copies alone: every block once, back to back into two
    # alternating slots on the copy stream (the link's sustained rate over the
    # whole pool), median of three passes
    slots = [slot, torch.empty(ss.block_bytes, dtype=torch.uint8, device="cuda")]
    pass_ms = []
    for _ in range(3):
        with torch.cuda.stream(copy):
            ev0.record(copy)
            for layer in range(L):
                slots[layer % 2].copy_(ss.pool[layer * ss.block_bytes:(layer + 1) * ss.block_bytes], non_blocking=True)
            ev1.record(copy)
        ev1.synchronize()
        pass_ms.append(ev0.elapsed_time(ev1))
    copy_pass_ms = statistics.median(pass_ms)
    del slot, slots
    log(f"copies of all {L} blocks alone: {copy_pass_ms:.1f} ms ({pool_bytes / (copy_pass_ms * 1e-3) / 1e9:.2f} GB/s)")

    for _ in range(args.warmup):
        pager.run(b, compute, copy)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        pager.run(b, compute, copy)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    streamed_out = [t.cpu() for t in outputs]
    # per-copy timeline of a few more passes: HIP events on the copy stream
    # around every block copy (no tracer, nothing dropped)
    copy_passes = []
    for _ in range(3):
        waits, starts, ends, pass_ms = pager.time(b, compute, copy)
        dur = [e - s for s, e in zip(starts, ends)]
        gaps = [starts[j + 1] - ends[j] for j in range(len(ends) - 1)]
        slot_waits = [s - w for w, s in zip(waits, starts)]
        copy_passes.append({"pass_ms": round(pass_ms, 3), "first_copy_start_ms": round(starts[0], 3),
                            "last_copy_end_ms": round(ends[-1], 3),
                            "copy_busy_ms": round(sum(dur), 3),
                            "copy_gbs": round(L * ss.block_bytes / (sum(dur) * 1e-3) / 1e9, 2),
                            "gaps_between_copies_ms": round(sum(gaps), 3),
                            "max_gap_ms": round(max(gaps) if gaps else 0.0, 3),
                            "waits_for_a_free_slot_ms": round(sum(slot_waits), 3),
                            "min_copy_ms": round(min(dur), 3), "max_copy_ms": round(max(dur), 3)})

    # compute alone: the same products over a device-resident copy of the pool
    dev_pool = ss.pool.to("cuda")
    steps = []
    for layer in range(L):
        for gi in range(len(GROUPS)):
            i = layer * len(GROUPS) + gi
            st = woq.StackStep()
            st.fmt, st.in_slot, st.out_slot = woq.FMT_INT8, i, i
            st.w8 = ss.steps[i].w
            st.w8.codes = dev_pool.data_ptr() + ss.layer_off[layer] + ss.steps[i].code_offset
            steps.append(st)
    runner = woq.Stack(steps, b)
    runner.bind(inputs, outputs)
    for _ in range(args.warmup):
        runner.run(b, compute)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        runner.run(b, compute)
    torch.cuda.synchronize()
    compute_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    same = all(torch.equal(a.view(torch.int16), o.cpu().view(torch.int16)) for a, o in zip(streamed_out, outputs))
    step_ms, _ = runner.time(b, args.steps, compute)
    kern_ms = sum(step_ms)
    runner.close()
    pager.close()

    copy_serial_ms = pool_bytes / (bw_h2d * 1e9) * 1e3
    eta = copy_serial_ms / ms_per_step
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32 on int8 codes",
        "data": "synthetic",
        "config": {"workload": f"{spec.name} streamed from pinned host memory, batch {b}"
                               + (f", {L} layers" if L != spec.layers else ""),
                   "format": "int8", "layers": L, "hidden": spec.hidden, "intermediate": spec.inter,
                   "q_heads": spec.q_heads, "kv_heads": spec.kv_heads, "head_dim": spec.head_dim, "batch": b,
                   "runner": "pager", "layer_block_bytes": ss.block_bytes, "algorithmic_bytes_per_step": step_bytes},
        "decode_tok_s": round(b / (ms_per_step * 1e-3), 3),
        "streamed": {"h2d_gbs_measured": round(bw_h2d, 3), "copy_serial_ms": round(copy_serial_ms, 3),
                     "copy_pass_ms": round(copy_pass_ms, 3),
                     "copy_pass_gbs": round(pool_bytes / (copy_pass_ms * 1e-3) / 1e9, 3),
                     "overlap_efficiency_vs_copy_pass": round(copy_pass_ms / ms_per_step, 4),
                     "compute_only_ms": round(compute_ms, 4), "overlap_efficiency": round(eta, 4),
                     "step_minus_copy_per_block_ms": round((ms_per_step - copy_serial_ms) / L, 4),
                     "bit_identical_to_resident": bool(same),
                     "copy_timeline": copy_passes},
        "roofline": {"bound": "hbm", "kernel": "qgemv_int8_valu", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "launches_per_step": len(steps),
                     "mean_launch_us": round(1e3 * kern_ms / len(steps), 3),
                     "mean_algorithmic_bytes_per_launch": step_bytes // len(steps)},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(spec, b)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
