#!/usr/bin/env python3
"""Benchmark of the fused dequant-GEMV (batch 1) and the MFMA GEMM (batch 64).

Headline (one JSON line on stdout): packed-code HBM GB/s of the fused GEMV
on the 4096x4096 computed-code layer set -- 1MAD and 3INST, k = 2, 3, 4,
V = 1, RHT 4096 with random signs, x ~ N(0,1) fp16, batch 1.  One step runs
one fused GEMV per layer of the set (six launches); consecutive steps use
different, equally random code buffers from a pool larger than the 256 MiB
Infinity Cache, so every step reads its codes from HBM.  Inputs are resident
in HBM before the timed region.  The line also carries:
  roofline      the dominant kernel's achieved algorithmic bytes per launch
                over its average launch duration (HIP events on its stream),
                against the 8 TB/s HBM peak
  cpu_baseline  the CPU oracle (decode, O(B^2) Hadamard, fp64 matvec) on a
                bounded sample of the same workload, on the host cores
  detail        per-variant kernel times, the Llama-3-8B-shaped decoder layer
                (microseconds per layer at batch 1 and 8) and the batch-64
                GEMM on the 28672x8192 up-projection (TFLOP/s vs fp16 MFMA peak)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
POOL_MIB = 1152
POOL_BYTES = 1 << 30
METRIC = "fused dequant-GEMV HBM GB/s + µs/layer (b=1); GEMM TFLOP/s (b=64)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pool-mib", type=int, default=POOL_MIB)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--only", default="", help="restrict the step to one variant, e.g. 3INST_k4")
    ap.add_argument("--eager", action="store_true",
                    help="(the default) launch every GEMV of a step directly")
    ap.add_argument("--graphs", action="store_true",
                    help="replay the step's other GEMVs from HIP graphs instead of launching them directly")
    ap.add_argument("--event-every", type=int, default=8,
                    help="bracket the dominant call with HIP events on every N-th timed step")
    ap.add_argument("--layer", default="",
                    help="only run 8 direct calls of one layer, CODE:M:N:K:B (e.g. HYB:28672:8192:2:1; "
                         "B > 8 takes qdec_gemm), for counter collection; prints no JSON line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, copy this many MiB device-to-device 5 times "
                         "(a plain copy of known size to scale HBM counters by)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Launch:
    """One pre-marshalled C call: avoids per-call Python work in timed loops.
    It holds the layer and the tensors whose device pointers it passes, so
    their memory cannot be freed (and, by torch.cuda.empty_cache, which every
    graph capture calls, unmapped) while the call can still run."""

    def __init__(self, q, fn, layer, x, y, b, ws, stream):
        import ctypes
        self.fn = getattr(q._lib, fn)
        self.keep = (layer, x, y, ws)
        self.args = (ctypes.byref(layer.desc()), x.data_ptr(), y.data_ptr(), b, ws.data_ptr(),
                     ws.numel(), stream)

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("launch failed with status %d" % st)


class LazyLaunch(Launch):
    """A Launch that picks up the current stream at call time (so it can be
    captured into a graph on torch's capture stream)."""

    def __init__(self, q, fn, layer, x, y, b, ws):
        super().__init__(q, fn, layer, x, y, b, ws, None)

    def __call__(self):
        import torch
        args = self.args[:-1] + (torch.cuda.current_stream().cuda_stream,)
        st = self.fn(*args)
        if st != 0:
            raise RuntimeError("launch failed with status %d" % st)


def algorithmic_bytes(m, n, k, b, lut_bytes=0, gscale_bytes=0):
    """Minimal HBM bytes of one call: packed codes, fp16 x and y, the two sign
    vectors, and the code tables."""
    return m * n * k // 8 + 2 * b * n + 2 * b * m + (m + n) // 8 + lut_bytes + gscale_bytes


def make_pool_layers(q, torch, dev, code, m, n, k, count, tag, **kw):
    """`count` layers sharing signs/LUT but with distinct random codes (extra
    keyword arguments go to synth.make_layer, e.g. V and Q)."""
    import synth
    g = torch.Generator(device=dev)
    g.manual_seed(int.from_bytes(tag.encode()[:8].ljust(8, b"\0"), "little") & 0x7FFFFFFF)
    words = synth.code_words(code, m, n, k, kw.get("V"), kw.get("kv", 0), kw.get("kv_b", 0),
                             kw.get("m_a", 0))
    pool = torch.randint(-(1 << 31), (1 << 31) - 1, (count, words), dtype=torch.int32, device=dev,
                         generator=g)
    host = synth.make_layer(code, m, n, k, tag=tag, codes=np.zeros(words, dtype=np.uint32), **kw)
    base = q.upload_layer(host, dev)
    layers = []
    for i in range(count):
        layers.append(q.Layer(code=base.code, L=base.L, k=base.k, V=base.V, Q=base.Q, m=m, n=n,
                              codes=pool[i], lut=base.lut, group_scale=base.group_scale,
                              group=base.group, layer_scale=base.layer_scale,
                              sign_in=base.sign_in, sign_out=base.sign_out, had_in=base.had_in,
                              had_out=base.had_out, kv=base.kv, kv_b=base.kv_b, m_a=base.m_a))
    return layers, pool, base


def run_one_layer(q, torch, dev, stream, spec):
    """8 direct calls of one layer (4 distinct code sets), for counters."""
    import synth
    name, m, n, k, b = spec.split(":")
    code = {v: c for c, v in synth.CODE_NAMES.items()}[name]
    m, n, k, b = int(m), int(n), int(k), int(b)
    kw = dict(had_in=8192, had_out=4096) if (m, n) == (28672, 8192) and b > 8 else {}
    layers, pool, base = make_pool_layers(q, torch, dev, code, m, n, k, 4, "bench/layer", **kw)
    x = torch.from_numpy(synth.activations("bench/layer/x", b, n).view(np.int16)).to(dev)
    y = torch.empty((b, m), dtype=torch.float16, device=dev)
    op, fn = (q.QDEC_OP_GEMV, "qdec_gemv") if b <= 8 else (q.QDEC_OP_GEMM, "qdec_gemm")
    ws = q.workspace(base, b, op, dev)
    calls = [Launch(q, fn, L, x, y, b, ws, stream) for L in layers]
    for i in range(8):
        calls[i % 4]()
    torch.cuda.synchronize()
    log("layer %s: 8 calls done" % spec)


def time_events(torch, fn, reps):
    """Average device time of fn() over reps launches, one event pair each."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3  # us


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU; the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import dequant_matmul_packed_amd as q
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream().cuda_stream
    if args.layer:
        run_one_layer(q, torch, dev, stream, args.layer)
        return

    # ---- the headline workload: 4096x4096 computed codes, b = 1 -----------
    wl = synth.WORKLOADS["computed4096"]
    specs = [s for s in wl.layers if not args.only or s.name == args.only]
    step_bytes = sum(s.m * s.n * s.k // 8 for s in specs)
    P = max(2, int(args.pool_mib * 2 ** 20 // step_bytes))
    log("workload %s: %d layers per step, %.1f MiB codes per step, pool of %d steps"
        % (wl.name, len(specs), step_bytes / 2 ** 20, P))
    x16 = synth.activations(wl.name + "/x", 1, 4096)
    x = torch.from_numpy(x16.view(np.int16)).to(dev)
    variants = []
    keep = []
    for s in specs:
        layers, pool, base = make_pool_layers(q, torch, dev, s.code, s.m, s.n, s.k, P, wl.name + "/" + s.name)
        keep.append(pool)
        ws = q.workspace(base, 1, q.QDEC_OP_GEMV, dev)
        y = torch.empty((1, s.m), dtype=torch.float16, device=dev)
        launches = [LazyLaunch(q, "qdec_gemv", L, x, y, 1, ws) for L in layers]
        variants.append(dict(spec=s, launches=launches, layers=layers, y=y, ws=ws,
                             bytes=algorithmic_bytes(s.m, s.n, s.k, 1)))
    torch.cuda.synchronize()

    # One step = the six fused GEMVs on one pool slot, launched directly
    # (replaying the step from HIP graphs measured slower on this stack:
    # 74 against 70 us per step).  On every N-th timed step the dominant
    # variant's call is bracketed by two HIP events (created before the timed
    # region) on the stream it runs on; an event pair costs the GPU about 9 us
    # per step (it waits for the queue to drain), so it is sampled, not taken
    # on every step.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g


    for v in variants:          # warm the launch paths once, eagerly
        v["launches"][0]()
    torch.cuda.synchronize()
    per_variant = {}
    for v in variants:          # per-variant GEMV time, graph of 20 calls
        g = capture(lambda v=v: [v["launches"][j % P]() for j in range(20)])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        per_variant[v["spec"].name] = e0.elapsed_time(e1) * 1e3 / 100
        del g
    # the dominant variant: the longest call; variants within 2 % of it are
    # the same time within noise, and among them the one moving most bytes
    longest = max(per_variant.values())
    dom = max((v for v in variants if per_variant[v["spec"].name] >= 0.98 * longest),
              key=lambda v: v["bytes"])
    log("per-variant us per GEMV (graph replay):", {k: round(t, 2) for k, t in per_variant.items()})
    others = [v for v in variants if v is not dom]
    if not args.graphs:
        graphs = None
        direct = [[Launch(q, "qdec_gemv", L, x, v["y"], 1, v["ws"], stream) for L in v["layers"]]
                  for v in others]

        def eager_others(i):
            for d in direct:
                d[i % P]()
    else:
        graphs = [capture(lambda i=i: [v["launches"][i]() for v in others]) for i in range(P)] if others else None
    dom_launch = [Launch(q, "qdec_gemv", L, x, dom["y"], 1, dom["ws"], stream)
                  for L in dom["layers"]]
    dom_call = dom_launch

    def step(i, ev=None):
        if graphs is not None:
            graphs[i % P].replay()
        else:
            eager_others(i)
        if ev is not None:
            ev[0].record()
            dom_call[i % P]()
            ev[1].record()
        else:
            dom_call[i % P]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps ---------------------------------
    every = max(1, args.event_every)
    dom_events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for i in range(0, args.steps, every)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i + args.warmup, dom_events[i // every] if i % every == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed / args.steps * 1e3
    gbs = step_bytes * args.steps / elapsed / 1e9
    dom_us = sum(a.elapsed_time(b) for a, b in dom_events) / len(dom_events) * 1e3
    dom_gbs = dom["bytes"] / (dom_us * 1e-6) / 1e9
    log("timed %d steps in %.4f s: %.1f GB/s packed, %.2f us/layer; dominant %s %.2f us"
        % (args.steps, elapsed, gbs, ms_per_step * 1e3 / len(variants), dom["spec"].name, dom_us))

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for r in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 5 device-to-device copies of %d MiB" % args.copy_calibration_mib)
        del src, dst

    # sanity: outputs are finite
    for v in variants:
        if not torch.isfinite(v["y"].float()).all():
            raise RuntimeError("non-finite output in %s" % v["spec"].name)

    detail = {"per_variant_kernel_us": {k: round(t, 3) for k, t in per_variant.items()},
              "us_per_layer": round(ms_per_step * 1e3 / len(variants), 3),
              "pool_steps": P}
    if not args.no_detail and not args.only:
        detail.update(bench_llama_layer(q, torch, dev, stream))
        detail.update(bench_llama_layer(q, torch, dev, stream, "llama3_8b_layer_fused"))
        detail.update(bench_gemm(q, torch, dev, stream))
        detail.update(bench_configs(q, torch, dev, stream))
        detail.update(bench_code_variants(q, torch, dev, stream))
        detail.update(bench_fractional(q, torch, dev, stream))
        detail.update(bench_encoder(q, torch, dev, cpu=not args.no_cpu_baseline))
        detail.update(bench_rht(q, torch, dev, stream))

    if not args.no_detail and not args.only:
        detail["pages_context"] = pages_context()
        ceil = measured_ceilings(torch, dev)
        detail["measured_ceilings"] = ceil
        g = detail.get("gemm_b64_up70b")
        if g:
            g["frac_of_measured_fp16_matmul"] = round(g["TFLOPs"] / ceil["fp16_matmul_8192_TFLOPs"], 4)
        detail["headline_frac_of_measured_copy"] = round(dom_gbs / ceil["copy_GBps_read_plus_write"], 4)
        detail["headline_frac_of_measured_read"] = round(dom_gbs / ceil["read_GBps_colsum_1GiB"], 4)
        for v in detail["configs_b1"].values():
            v["frac_of_measured_read"] = round(v["algorithmic_GBps"] / ceil["read_GBps_colsum_1GiB"], 4)
    cpu = None
    if not args.no_cpu_baseline:
        cpu, cpu_detail = cpu_baseline(specs, x16)
        if not args.no_detail and not args.only:
            cpu_detail["per_config"] = cpu_per_config()
        detail["cpu_oracle"] = cpu_detail

    # HBM bytes per call of the dominant variant from the committed counter
    # summary (None once the kernel sources differ from the profiled ones)
    traffic = measured_traffic(dom["spec"], dom_us)
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 (codes k=2,3,4 bit; fp32 accumulate)",
        "data": "synthetic: seeded random code words, N(0,1) fp16 activations, random signs",
        "config": {"workload": "4096x4096 linear, 1MAD and 3INST computed codes, k=2,3,4, V=1, "
                               "RHT 4096/4096, batch 1 (six fused GEMVs per step)",
                   "global_batch": 1, "layers_per_step": len(variants),
                   "packed_bytes_per_step": step_bytes, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "qdec_gemv %s k=%d b=1 (gemv_kernel + gemv_finish_kernel)"
                     % (synth.CODE_NAMES[dom["spec"].code], dom["spec"].k),
                     "achieved": round(dom_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic["bytes_per_call"] if traffic else None,
                     "traffic_detail": traffic,
                     "bytes_per_launch": dom["bytes"], "avg_launch_us": round(dom_us, 3)},
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


def measured_traffic(spec, us):
    """HBM bytes per call of this variant from the committed counter summary
    (profiles/gemv_hbm_traffic.json), as GB/s over the measured call time;
    None when the kernels changed since the counters were taken."""
    import synth
    path = os.path.join(ROOT, "profiles", "gemv_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    import profile_traffic
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != profile_traffic.kernel_source_hash():
        return None
    v = rec["variants"].get("%s_k%d" % (synth.CODE_NAMES[spec.code], spec.k))
    if v is None:
        return None
    return {"bytes_per_call": int(v["bytes_per_call"]), "GBps": round(v["bytes_per_call"] / (us * 1e-6) / 1e9, 2),
            "over_algorithmic": round(v["bytes_per_call"] / v["algorithmic"], 3),
            "source": "profiles/gemv_hbm_traffic.md (FETCH_SIZE, WRITE_SIZE scaled by a 256 MiB copy)"}


def bench_llama_layer(q, torch, dev, stream, name="llama3_8b_layer"):
    """Llama-3-8B-shaped decoder layer (one fused GEMV per projection: 7, or
    4 with QKV and gate+up fused), microseconds per layer at batch 1 and 8,
    rotating through distinct layer instances; the layers launched directly
    and replayed from HIP graphs, the faster of the two reported."""
    import synth
    wl = synth.WORKLOADS[name]
    layer_bytes = wl.code_bytes
    P = max(2, int(1200 * 2 ** 20 // layer_bytes))
    out = {}
    pools = []
    for b in wl.batches:
        x = {}
        calls = []
        direct = []
        for s in wl.layers:
            layers, pool, base = make_pool_layers(q, torch, dev, s.code, s.m, s.n, s.k, P,
                                                  "bench/llama/" + s.name)
            pools.append(pool)
            if s.n not in x:
                x[s.n] = torch.from_numpy(synth.activations("bench/llama/x", b, s.n).view(np.int16)).to(dev)
            ws = q.workspace(base, b, q.QDEC_OP_GEMV, dev)
            y = torch.empty((b, s.m), dtype=torch.float16, device=dev)
            calls.append([LazyLaunch(q, "qdec_gemv", L, x[s.n], y, b, ws) for L in layers])
            direct.append([Launch(q, "qdec_gemv", L, x[s.n], y, b, ws, stream) for L in layers])
        for c in calls:
            c[0]()
        torch.cuda.synchronize()
        graphs = []
        for i in range(P):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in calls:
                    c[i]()
            graphs.append(g)
        for i in range(P):
            graphs[i].replay()
        torch.cuda.synchronize()
        reps = 60
        t0 = time.perf_counter()
        for i in range(reps):
            graphs[i % P].replay()
        torch.cuda.synchronize()
        us_graph = (time.perf_counter() - t0) / reps * 1e6
        del graphs
        for i in range(P):
            for c in direct:
                c[i]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(reps):
            for c in direct:
                c[i % P]()
        torch.cuda.synchronize()
        us_direct = (time.perf_counter() - t0) / reps * 1e6
        us = min(us_graph, us_direct)
        out["%s_b%d" % (name, b)] = {"us_per_layer": round(us, 2),
                                     "packed_GBps": round(layer_bytes / (us * 1e-6) / 1e9, 1),
                                     "gemv_calls": len(wl.layers),
                                     "direct_us": round(us_direct, 2), "graph_us": round(us_graph, 2)}
        log("%s b=%d: %.2f us/layer (direct %.2f, graph %.2f)" % (name, b, us, us_direct, us_graph))
        del calls, direct
        pools.clear()
        torch.cuda.empty_cache()
    return out


def time_layer(q, torch, dev, stream, code, m, n, k, b, tag, **kw):
    """Device microseconds per call of one layer shape at batch b (qdec_gemv
    up to 8, qdec_gemm above): distinct random code sets in rotation from a
    pool of at least 1 GiB, four times the 256 MiB Infinity Cache, so no call
    finds its codes there; 20 warm-up calls, then 5 repeats of 200
    back-to-back direct launches, each bracketed by one event pair on the
    launch stream; the median repeat.  Returns (us, the layer's descriptor)."""
    import synth
    words = synth.code_words(code, m, n, k, kw.get("V"), kw.get("kv", 0), kw.get("kv_b", 0),
                             kw.get("m_a", 0))
    P = int(min(512, max(4, -(-POOL_BYTES // (4 * words)))))
    layers, pool, base = make_pool_layers(q, torch, dev, code, m, n, k, P, tag, **kw)
    x = torch.from_numpy(synth.activations(tag + "/x", b, n).view(np.int16)).to(dev)
    y = torch.empty((b, m), dtype=torch.float16, device=dev)
    op, fn = (q.QDEC_OP_GEMV, "qdec_gemv") if b <= 8 else (q.QDEC_OP_GEMM, "qdec_gemm")
    ws = q.workspace(base, b, op, dev)
    calls = [Launch(q, fn, L, x, y, b, ws, stream) for L in layers]
    for i in range(20):
        calls[i % P]()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    reps = []
    j = 0
    for r in range(5):
        e0.record()
        for i in range(200):
            calls[j % P]()
            j += 1
        e1.record()
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) * 1e3 / 200)
    if not torch.isfinite(y.float()).all():
        raise RuntimeError("non-finite output in %s" % tag)
    del calls, layers, pool, ws, x, y
    torch.cuda.empty_cache()
    return float(np.median(reps)), base


def tensor_bytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def time_4096_variants(q, torch, dev, stream, variants, tagbase):
    """Time per call of 4096x4096 layers at b=1 (qdec_gemv) and b=64
    (qdec_gemm) for each (name, code, k, make_layer keywords) variant."""
    out = {}
    for name, code, k, kw in variants:
        res = {}
        for b in (1, 64):
            us, base = time_layer(q, torch, dev, stream, code, 4096, 4096, k, b, tagbase + name, **kw)
            res["b%d_us" % b] = round(us, 2)
            if b == 1:
                res["b1_packed_GBps"] = round(base.code_bytes / (us * 1e-6) / 1e9, 1)
            else:
                res["b64_TFLOPs"] = round(2 * 4096 * 4096 * 64 / (us * 1e-6) / 1e12, 1)
        out[name] = res
    return out


def bench_configs(q, torch, dev, stream):
    """The single-layer configurations at batch 1, timed as in time_layer:
    the 4096x4096 HYB k=2 layer (V=2, Q=9, 512-pair table), and the
    4096x14336 down-projection shape with the 3-bit non-uniform scalar
    quantizer (fp16 scale per 128 weights) and with the 2-D vector quantizer
    (8-bit index per weight pair).  GB/s on the packed codes, and on the
    algorithmic bytes (codes, x, y, signs, tables and group scales) as a
    fraction of the 8 TB/s HBM peak."""
    import synth
    out = {}
    for wname in ("hyb4096", "down_nuq", "down_vq"):
        s = synth.WORKLOADS[wname].layers[0]
        kw = dict(scale=s.scale)
        us, base = time_layer(q, torch, dev, stream, s.code, s.m, s.n, s.k, 1, "bench/cfg/" + wname, **kw)
        alg = (base.code_bytes + 2 * s.n + 2 * s.m + (s.m + s.n) // 8 + tensor_bytes(base.lut)
               + tensor_bytes(base.group_scale))
        out[wname] = {"layer": synth.WORKLOADS[wname].description, "us_per_call": round(us, 2),
                      "packed_bytes": base.code_bytes, "algorithmic_bytes": alg,
                      "packed_GBps": round(base.code_bytes / (us * 1e-6) / 1e9, 1),
                      "algorithmic_GBps": round(alg / (us * 1e-6) / 1e9, 1),
                      "frac_of_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    log("single-layer configs b=1:", {k: (v["us_per_call"], v["algorithmic_GBps"]) for k, v in out.items()})
    return {"configs_b1": out}


def bench_code_variants(q, torch, dev, stream):
    """The table-size knob of the trellis codes on one 4096x4096 k=2 layer at
    b=1 and b=64: HYB with 2^9 pairs (V=2), HYB with a 2^6-value codebook
    (V=1) and the pure lookup of 2^16 values (a 128 KiB table in LDS)."""
    import synth
    out = time_4096_variants(q, torch, dev, stream, (
        ("HYB_V2_Q9", synth.HYB, 2, dict(V=2, Q=9)), ("HYB_V1_Q6", synth.HYB, 2, dict(V=1, Q=6)),
        ("LUT_L16", synth.LUT, 2, {})), "bench/var/")
    log("code variants (4096x4096 k=2):", out)
    return {"code_variants_4096_k2": out}


def bench_encoder(q, torch, dev, cpu=True):
    """The tail-biting trellis encoder on a 4096x4096 HYB layer at 2 bits
    (65536 tiles) of i.i.d. N(0,1) x 0.02 targets: tiles/s on the GPU, the
    MSE per weight relative to the target variance, and (cpu) the oracle's
    one-thread time on a few tiles of the same layer."""
    import synth
    m = n = 4096
    host = synth.make_layer(synth.HYB, m, n, 2, tag="bench/enc", codes=np.zeros(m * n * 2 // 32, np.uint32))
    lay = q.upload_layer(host, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    W = torch.randn((m, n), generator=g, device=dev, dtype=torch.float32) * 0.02
    ws = q.workspace(lay, 1, q.QDEC_OP_ENCODE, dev)
    codes = torch.empty(m * n * 2 // 32, dtype=torch.int32, device=dev)
    q.encode(lay, W, codes, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    q.encode(lay, W, codes, ws)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3
    ntiles = (m // 16) * (n // 16)
    # error of the decoded layer, tiles in storage order
    lay2 = q.Layer(code=lay.code, L=lay.L, k=lay.k, V=lay.V, Q=lay.Q, m=m, n=n, codes=codes, lut=lay.lut,
                   layer_scale=lay.layer_scale, had_in=lay.had_in, had_out=lay.had_out)
    dec = torch.empty((ntiles, 256), dtype=torch.float16, device=dev)
    q.qdec_decode_tile(lay2, 0, ntiles, dec)
    Wt = W.view(m // 128, 8, 16, n // 16, 16).permute(0, 3, 1, 2, 4).reshape(ntiles, 256)
    mse = ((Wt - dec.float() * np.float32(host.scale)) ** 2).mean().item() / 0.02 ** 2
    out = {"layer": "4096x4096 HYB k=2 V=2 Q=9", "tiles": ntiles, "seconds": round(sec, 4),
           "tiles_per_s": round(ntiles / sec), "mse_rel": round(mse, 5)}
    if cpu:
        import oracle
        threads = oracle.omp_threads()
        oracle.set_threads(1)
        Wh = W[:16, :64].cpu().numpy()
        vals = oracle.state_values_all(synth.HYB, 16, host.Q, host.lut, 2).view(np.float16).astype(np.float32)
        t0 = time.time()
        for c in range(4):
            oracle.encode_stream(16, 4, 2, vals, Wh[:, 16 * c:16 * c + 16].reshape(-1), host.scale)
        cpu_tile = (time.time() - t0) / 4
        oracle.set_threads(threads)
        out["oracle_one_thread_s_per_tile"] = round(cpu_tile, 4)
        out["gpu_vs_oracle_one_thread"] = round(ntiles / sec * cpu_tile, 1)
    log("encoder:", out)
    return {"encoder_4096_hyb_k2": out}


def bench_fractional(q, torch, dev, stream):
    """Bit widths of one 4096x4096 HYB layer (V=2, Q=9) at b=1 and b=64:
    2 to 4 bits per weight in half-bit steps (kV = 4 .. 8 bits per trellis
    step), and half-TCQ with the rows cut in two halves at 2.5 and 3 bits
    (2.75 on average)."""
    import synth
    H = synth.HYB
    out = time_4096_variants(q, torch, dev, stream, (
        ("k2.0", H, 2, {}), ("k2.5", H, 0, dict(kv=5)), ("k3.0", H, 3, {}), ("k3.5", H, 0, dict(kv=7)),
        ("k4.0", H, 4, {}), ("half_k2.5_k3.0", H, 0, dict(kv=5, kv_b=6, m_a=2048))), "bench/frac/")
    log("bit widths (4096x4096 HYB):", out)
    return {"bit_widths_4096_hyb": out}


def bench_gemm(q, torch, dev, stream):
    """28672x8192 HYB k=3 up-projection with X of 64x8192: time per call and
    TFLOP/s of the three-launch batched path, with the per-layer protocol
    (time_layer: code sets rotating through a pool of at least 1 GiB, 20
    warm-up calls, 5 repeats of 200 back-to-back calls, the median)."""
    import synth
    wl = synth.WORKLOADS["up70b_prefill"]
    s = wl.layers[0]
    b = wl.batches[0]
    us, _ = time_layer(q, torch, dev, stream, s.code, s.m, s.n, s.k, b, "bench/up70b",
                       had_in=s.had_in, had_out=s.had_out)
    flops = 2.0 * s.m * s.n * b
    tf = flops / (us * 1e-6) / 1e12
    log("gemm b=64: %.1f us, %.1f TFLOP/s" % (us, tf))
    return {"gemm_b64_up70b": {"us_per_call": round(us, 2), "TFLOPs": round(tf, 1),
                               "frac_of_fp16_mfma_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                               "launches": "rht_in + gemm + rht_out", "protocol": "time_layer"}}


def cpu_baseline(specs, x16):
    """The oracle as it stands, on the host cores: one full forward per layer
    of the step (decode of every tile, O(B^2) Hadamards, fp64 matvec) with
    all threads; then, for the detail, decode-only on all threads and both
    on one thread over the first layer.  It is a correctness reference, not
    a tuned CPU competitor."""
    import oracle
    import synth
    threads = oracle.omp_threads()
    hosts = [s.build("cpu_baseline") for s in specs]
    nbytes = [s.m * s.n * s.k // 8 for s in specs]
    nweights = [s.m * s.n for s in specs]

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0
    t_fwd = sum(timed(lambda h=h: oracle.forward(h, x16)) for h in hosts)
    t_dec = sum(timed(lambda h=h: oracle.decode_tiles_storage(h, 0, h.n_tiles)) for h in hosts)
    oracle.set_threads(1)
    t_fwd1 = timed(lambda: oracle.forward(hosts[0], x16))
    t_dec1 = timed(lambda: oracle.decode_tiles_storage(hosts[0], 0, hosts[0].n_tiles))
    oracle.set_threads(threads)
    gbs = sum(nbytes) / t_fwd / 1e9
    log("cpu oracle: forward %.2f s for %d layers (%.4f GB/s, %d threads); one thread, one layer: "
        "forward %.2f s, decode %.2f s" % (t_fwd, len(specs), gbs, threads, t_fwd1, t_dec1))
    base = {"value": round(gbs, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "one full forward of each of the %d layers of one step (%.1f MiB of codes), "
                      "%.2f s" % (len(specs), sum(nbytes) / 2 ** 20, t_fwd)}
    detail = {"affinity_cores": len(os.sched_getaffinity(0)), "threads": threads,
              "forward_GBps": round(gbs, 5),
              "decode_Mweights_per_s": round(sum(nweights) / t_dec / 1e6, 2),
              "one_thread_forward_GBps": round(nbytes[0] / t_fwd1 / 1e9, 5),
              "one_thread_decode_Mweights_per_s": round(nweights[0] / t_dec1 / 1e6, 2),
              "sample": "all threads: forward and decode-only of the %d layers; one thread: the first "
                        "layer (%s)" % (len(specs), specs[0].name)}
    return base, detail


def cpu_per_config():
    """The oracle on each of the other configurations, all threads: decode
    only (every tile of every layer, bit-serial walk and code lookup) and one
    full forward (decode, O(B^2) Hadamards on both sides, fp64 matvec) per
    batch size.  The 28672x8192 batch-64 forward is timed on 8 of its 64
    batch columns: its decode and weight work are whole, the per-column work
    is an eighth.  Rates are weights/s and packed code bytes/s."""
    import oracle
    import synth
    threads = oracle.omp_threads()
    out = {}
    for wname, cols in (("hyb4096", None), ("llama3_8b_layer", None), ("down_nuq", None),
                        ("down_vq", None), ("up70b_prefill", 8)):
        wl = synth.WORKLOADS[wname]
        hosts = [s.build("cpu_per_config") for s in wl.layers]
        weights = sum(h.m * h.n for h in hosts)
        nbytes = sum(h.code_bytes for h in hosts)
        t0 = time.perf_counter()
        for h in hosts:
            oracle.decode_tiles_storage(h, 0, h.n_tiles)
        t_dec = time.perf_counter() - t0
        rec = {"layers": len(hosts), "weights": weights, "packed_bytes": nbytes,
               "decode_s": round(t_dec, 3), "decode_Mweights_per_s": round(weights / t_dec / 1e6, 2),
               "decode_packed_GBps": round(nbytes / t_dec / 1e9, 5)}
        for b in wl.batches:
            bb = min(b, cols) if cols else b
            t0 = time.perf_counter()
            for h in hosts:
                oracle.forward(h, synth.activations("cpu_per_config/x", bb, h.n))
            t_fwd = time.perf_counter() - t0
            rec["forward_b%d" % b] = {"columns_timed": bb, "s": round(t_fwd, 3),
                                      "Mweights_per_s": round(weights / t_fwd / 1e6, 2),
                                      "packed_GBps": round(nbytes / t_fwd / 1e9, 5)}
        out[wname] = rec
        log("cpu oracle %s: decode %.2f s, forward %s" % (
            wname, t_dec, ", ".join("b=%s %.2f s" % (k[9:], v["s"]) for k, v in rec.items()
                                    if k.startswith("forward_b"))))
    return {"threads": threads, "configs": out,
            "note": "the oracle is a plain correctness reference (bit-serial walk, O(B^2) Hadamard), "
                    "not a tuned CPU implementation"}


def pages_context():
    """The pages' own decode-cost figures, beside the VALU lane-instructions
    per weight measured on this chip (read from the committed SQ-counter
    summaries; a GEMV counts decode plus one v_dot2 per weight pair, a GEMM
    the decode alone)."""
    out = {"pages": {"hyb_int32_ops_per_weight": "~2 (LUT decompress 0.5 + trellis unpack and index ~1.5)",
                     "e8p_int32_ops_per_weight": "~3 (QuIP# E8P, the pages' comparator)",
                     "hardware": "NVIDIA GPUs, as stated on the pages",
                     "source": "QTIP OpenReview discussion, untitled ALU-op comment"},
           "measured_valu_per_weight": {}}
    for name, path in (("gemv_hyb_k2_b1_28672x8192", "sq_counters_gemv_hyb_28672x8192_b1.md"),
                       ("gemm_hyb_k3_b64_28672x8192", "sq_counters_gemm_hyb_28672x8192_b64.md")):
        f = os.path.join(ROOT, "profiles", path)
        if not os.path.exists(f):
            continue
        with open(f) as fh:
            for line in fh:
                cells = [c.strip() for c in line.split("|")]
                if len(cells) > 11 and cells[1].startswith("`qdec::gem") and cells[10]:
                    out["measured_valu_per_weight"][name] = float(cells[10])
                    break
    out["measured_source"] = "profiles/sq_counters_*.md (SQ_INSTS_VALU x 64 / weights)"
    return out


def bench_rht(q, torch, dev, stream):
    """qdec_rht on its own, at the shapes the batched path runs it on and on a
    large input: the time per call (200 back-to-back launches between one
    event pair, inputs rotating through a pool of at least 1 GiB so that no
    call finds its input in the caches; the median of 5 repeats) and its
    rate against HBM: bytes = input + output + the sign bits."""
    import ctypes
    cases = [  # name, rows, n, block, input dtype (0 fp16, 1 fp32), output dtype, mode
        ("input_64x8192_B8192_f16", 64, 8192, 8192, 0, 0, 0),
        ("output_64x28672_B4096_f32_to_f16", 64, 28672, 4096, 1, 0, 1),
        ("output_8x14336_B2048_f32_to_f16", 8, 14336, 2048, 1, 0, 1),
        ("input_4096x4096_B4096_f16", 4096, 4096, 4096, 0, 0, 0),
    ]
    fn = q._lib.qdec_rht
    out = {}
    for name, rows, n, block, idt, odt, mode in cases:
        ib, ob = (4 if idt else 2), (4 if odt else 2)
        in_bytes = rows * n * ib
        P = int(min(512, max(4, -(-POOL_BYTES // in_bytes))))
        g = torch.Generator(device=dev)
        g.manual_seed(rows * 7919 + n)
        dt = torch.float32 if idt else torch.float16
        pool = torch.randn((P, rows, n), generator=g, device=dev).to(dt)
        signs = torch.randint(-(1 << 31), (1 << 31) - 1, ((n + 31) // 32,), dtype=torch.int32, device=dev,
                              generator=g)
        y = torch.empty((rows, n), dtype=torch.float32 if odt else torch.float16, device=dev)
        scale = ctypes.c_float(1.0)

        def call(i):
            st = fn(pool[i % P].data_ptr(), idt, y.data_ptr(), odt, rows, n, block, signs.data_ptr(), mode,
                    scale, stream)
            if st != 0:
                raise RuntimeError("qdec_rht failed: %d" % st)
        for i in range(20):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps, j = [], 0
        for r in range(5):
            e0.record()
            for i in range(200):
                call(j)
                j += 1
            e1.record()
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) * 1e3 / 200)
        us = sorted(reps)[2]
        nbytes = in_bytes + rows * n * ob + (n + 7) // 8
        gbs = nbytes / us / 1e3
        out[name] = {"us": round(us, 2), "bytes": nbytes, "GBps": round(gbs, 1),
                     "frac_of_8TBps": round(gbs / 8000.0, 4)}
        del pool
        torch.cuda.empty_cache()
    log("qdec_rht alone:", {k: (v["us"], v["GBps"]) for k, v in out.items()})
    return {"rht_alone": out}


def measured_ceilings(torch, dev):
    """What plain library kernels reach on this GPU: a device-to-device copy
    (HBM read + write), a reduction that only reads, and a large fp16 matmul
    (hipBLASLt, MFMA)."""
    nbytes = 512 << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for r in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    # pure read: column sums of 1 GiB of fp32 seen as 262144 x 1024 (torch's
    # reduction over the outer dimension, each thread summing one column:
    # coalesced reads, 4 KiB written); a full reduction to one scalar
    # measured slower (3.9 TB/s against 5.7)
    rd = torch.zeros(POOL_BYTES // 4, dtype=torch.float32, device=dev).view(-1, 1024)
    for r in range(3):
        s = rd.sum(0)
    torch.cuda.synchronize()
    e0.record()
    for r in range(10):
        s = rd.sum(0)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = POOL_BYTES * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # the same read on the headline layer's scale: 4 MiB column sums, each
    # call on the next 4 MiB of the pool (as the GEMV's code slices rotate),
    # 200 back-to-back calls; and the floor of a two-kernel call: two
    # one-workgroup fills of a 4 KiB tensor per iteration
    small = POOL_BYTES // (4 << 20)
    views = [rd[i * 1024:(i + 1) * 1024] for i in range(small)]
    for r in range(20):
        s = views[r % small].sum(0)
    torch.cuda.synchronize()
    e0.record()
    for r in range(200):
        s = views[r % small].sum(0)
    e1.record()
    torch.cuda.synchronize()
    small_us = e0.elapsed_time(e1) * 1e3 / 200
    tiny = torch.empty(1024, dtype=torch.float32, device=dev)
    for r in range(20):
        tiny.fill_(1.0)
    torch.cuda.synchronize()
    e0.record()
    for r in range(200):
        tiny.fill_(1.0)
        tiny.fill_(2.0)
    e1.record()
    torch.cuda.synchronize()
    pair_us = e0.elapsed_time(e1) * 1e3 / 200
    del rd, s, views, tiny
    n = 8192
    a = torch.randn(n, n, dtype=torch.float16, device=dev)
    b = torch.randn(n, n, dtype=torch.float16, device=dev)
    for r in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for r in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    mm_tf = 2 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    log("measured ceilings: copy %.0f GB/s (read + write), read %.0f GB/s, 4 MiB read %.2f us (%.0f GB/s), "
        "two empty kernels %.2f us, fp16 matmul %d^3 %.0f TFLOP/s"
        % (copy_gbs, read_gbs, small_us, (4 << 20) / (small_us * 1e-6) / 1e9, pair_us, n, mm_tf))
    return {"copy_GBps_read_plus_write": round(copy_gbs, 1), "read_GBps_colsum_1GiB": round(read_gbs, 1),
            "read_4MiB_colsum_us": round(small_us, 2),
            "read_4MiB_colsum_GBps": round((4 << 20) / (small_us * 1e-6) / 1e9, 1),
            "two_tiny_kernels_us": round(pair_us, 2),
            "fp16_matmul_8192_TFLOPs": round(mm_tf, 1)}


if __name__ == "__main__":
    main()
