#!/usr/bin/env python3
"""Benchmark of the fused dequant-GEMV (batch 1) and the MFMA GEMM (batch 64).

Headline (one JSON line on stdout): packed-code HBM GB/s, and microseconds
per layer, of the seven linear layers of a Llama-3-8B-shaped decoder layer
(q, o 4096x4096; k, v 1024x4096; gate, up 14336x4096; down 4096x14336), HYB
trellis codes at 2 bits per weight (L = 16, V = 2, Q = 9), RHT on both sides,
batch 1.  One step is one pass through a stack of 64 such layers, each with
codes of its own (3.49 GB per step, 13.6 times the 256 MiB Infinity Cache,
so every layer reads its codes from HBM), in the order a decoder layer runs
them: q, k and v in one grouped call (they read the same activations), o,
gate and up in one grouped call, down.  Inputs are resident in HBM before the
timed region.  The line also carries:
  roofline      the dominant call of a layer -- the grouped gate+up call
                (its MFMA GEMV kernel and its finisher) -- as algorithmic
                bytes per call over its event-timed duration, against the
                8 TB/s HBM peak
  roofline_b64  the batch-64 GEMM on the 28672x8192 up-projection (HYB k=3):
                TFLOP/s per call against the 2.5 PFLOP/s fp16 MFMA peak
  cpu_baseline  the CPU oracle (decode, O(B^2) Hadamard, fp64 matvec) on a
                bounded sample of the same workload, on the host cores
  detail        per-projection times, the layer at batch 8 and with fused
                projections, the single-layer configurations, the measured
                ceilings of this GPU and the pages' decode-cost figures
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2516.6          # 256 CUs x 2.4 GHz x 4096 fp16 flop per clock, dense
POOL_BYTES = 1 << 30
STACK_LAYERS = 64
METRIC = "fused dequant-GEMV HBM GB/s + µs/layer (b=1); GEMM TFLOP/s (b=64)"
GEMM_LAYER = "HYB:28672:8192:3:64"     # the b=64 GEMM of the headline, as a --layer spec
CSRC = os.path.join(ROOT, "dequant_matmul_packed_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=STACK_LAYERS,
                    help="distinct Llama-3-8B-shaped layers per step (codes of their own each)")
    ap.add_argument("--launch", choices=("auto", "graph", "direct"), default="auto",
                    help="replay each step from one HIP graph, launch its calls directly, or time "
                         "both before the timed region and take the faster")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--full-detail", action="store_true",
                    help="add the encoder, bit-width and code-variant tables (several minutes)")
    ap.add_argument("--layer", default="",
                    help="only run 8 direct calls of one layer, CODE:M:N:K:B (e.g. HYB:28672:8192:2:1; "
                         "B > 8 takes qdec_gemm), for counter collection; prints no JSON line")
    ap.add_argument("--call", default="", choices=("", "qkv", "o", "gate_up", "down", "gemm"),
                    help="only run 8 direct calls of one call of the headline (a call of the Llama layer "
                         "stack, or the b=64 GEMM), then the copy calibration if asked, for counter "
                         "collection; prints no JSON line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, copy this many MiB device-to-device 5 times "
                         "(a plain copy of known size to scale HBM counters by)")
    return ap.parse_args()


def code_only(text: str) -> str:
    """The source without comments, trailing spaces and blank lines: what the
    compiler sees (a comment edit does not change the profiled kernels)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def kernel_source_hash(csrc: str = CSRC) -> str:
    """Hash of the kernel sources (code only), stored with counter summaries
    so that the bench reports HBM traffic only while the kernels are the
    ones that were profiled."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


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

    def __call__(self, stream=None):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("launch failed with status %d" % st)


class LazyLaunch(Launch):
    """A Launch that picks up the current stream at call time (so it can be
    captured into a graph on torch's capture stream), or takes the stream
    handle from its caller (a timed loop looks it up once: the lookup costs
    about as much host time as the library's launch itself)."""

    def __init__(self, q, fn, layer, x, y, b, ws):
        super().__init__(q, fn, layer, x, y, b, ws, None)

    def __call__(self, stream=None):
        import torch
        args = self.args[:-1] + (stream if stream is not None else torch.cuda.current_stream().cuda_stream,)
        st = self.fn(*args)
        if st != 0:
            raise RuntimeError("launch failed with status %d" % st)


def algorithmic_bytes(m, n, k, b, lut_bytes=0, gscale_bytes=0):
    """Minimal HBM bytes of one call: packed codes, fp16 x and y, the two sign
    vectors, and the code tables."""
    return m * n * k // 8 + 2 * b * n + 2 * b * m + (m + n) // 8 + lut_bytes + gscale_bytes


def sha256_tensor(torch, t, chunk=1 << 26):
    """SHA-256 of a tensor's bytes (copied to the host 64 MiB at a time)."""
    h = hashlib.sha256()
    flat = t.reshape(-1).view(torch.uint8)
    for i in range(0, flat.numel(), chunk):
        h.update(flat[i:i + chunk].cpu().numpy().tobytes())
    return h.hexdigest()


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



class GroupLaunch:
    """One pre-marshalled qdec_gemv_group call (its pointer arrays built
    once).  It holds the layers and tensors it passes by pointer, so their
    memory stays mapped while the call can run; it takes torch's current
    stream at call time, so it can be captured into a graph."""

    def __init__(self, q, layers, xs, ys, ws):
        self.fn = q._lib.qdec_gemv_group
        self.call = q.GroupCall(layers, xs, ys)
        self.keep = (list(layers), list(xs), list(ys), ws)
        self.ws, self.nbytes = ws.data_ptr(), ws.numel()

    def __call__(self, stream=None):
        import torch
        st = self.fn(self.call.lp, self.call.count, self.call.xp, self.call.yp, self.ws, self.nbytes,
                     stream if stream is not None else torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError("qdec_gemv_group failed with status %d" % st)


def call_bytes(layers, b=1):
    """Algorithmic HBM bytes of one call over these layers at batch b: packed
    codes, fp16 x and y, both sign vectors and the code tables."""
    return sum(L.code_bytes + 2 * b * (L.n + L.m) + (L.m + L.n) // 8 + tensor_bytes(L.lut)
               + tensor_bytes(L.group_scale) for L in layers)


def time_calls(torch, calls, reps=5, ncalls=200):
    """Median over reps of the event-timed average of ncalls back-to-back
    calls (rotating through `calls`), on the current stream, in us."""
    s = torch.cuda.current_stream().cuda_stream
    for i in range(20):
        calls[i % len(calls)](s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out, j = [], 0
    for r in range(reps):
        e0.record()
        for i in range(ncalls):
            calls[j % len(calls)](s)
            j += 1
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / ncalls)
    return float(np.median(out))


def copy_calibration(torch, dev, mib):
    """5 device-to-device copies of mib MiB: a plain copy of known size that
    HBM counters (FETCH_SIZE, WRITE_SIZE) are scaled by."""
    if mib <= 0:
        return
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for r in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 5 device-to-device copies of %d MiB" % mib)


def llama_stack(q, torch, dev, args):
    """The headline: a stack of Llama-3-8B-shaped layers at batch 1, each layer
    with codes of its own.  Returns the JSON fields."""
    import synth
    wl = synth.WORKLOADS["llama3_8b_layer"]
    specs = {s.name: s for s in wl.layers}
    L = args.layers
    pools, lay = [], {}
    for name, s in specs.items():
        layers, pool, base = make_pool_layers(q, torch, dev, s.code, s.m, s.n, s.k, L, "bench/stack/" + name)
        pools.append(pool)
        lay[name] = layers
    layer_bytes = sum(lay[nm][0].code_bytes for nm in specs)
    step_bytes = layer_bytes * L
    # each group reads its own activations (in a model: the normed residual,
    # the attention output, the normed residual, the gated product)
    xt = {g: torch.from_numpy(synth.activations("bench/stack/x_" + g, 1, n).view(np.int16)).to(dev)
          for g, n in (("qkv", 4096), ("o", 4096), ("gate_up", 4096), ("down", 14336))}
    ys = {nm: torch.empty((1, s.m), dtype=torch.float16, device=dev) for nm, s in specs.items()}
    # the generated buffers, by SHA-256 (each projection's code pool, table
    # and sign vectors; the activations): the inputs are fixed by the seeds
    inputs = {"generator": "codes: torch.randint on the device (uniform int32 words), seeded by the tag; "
                           "tables, signs and activations: synth (SHA-256-seeded numpy generators)",
              "sha256": {}}
    for nm in (specs if not args.call else ()):     # not in counter runs (no extra copies)
        b0 = lay[nm][0]
        inputs["sha256"]["codes/" + nm] = sha256_tensor(torch, pools[list(specs).index(nm)])
        for part in ("lut", "sign_in", "sign_out"):
            if getattr(b0, part) is not None:
                inputs["sha256"]["%s/%s" % (part, nm)] = sha256_tensor(torch, getattr(b0, part))
    for g, t in (xt.items() if not args.call else ()):
        inputs["sha256"]["x/" + g] = sha256_tensor(torch, t)
    ws_qkv = torch.empty(q.qdec_gemv_group_workspace_bytes([lay[n][0] for n in ("q", "k", "v")]),
                         dtype=torch.uint8, device=dev)
    ws_gu = torch.empty(q.qdec_gemv_group_workspace_bytes([lay[n][0] for n in ("gate", "up")]),
                        dtype=torch.uint8, device=dev)
    ws_o = q.workspace(lay["o"][0], 1, q.QDEC_OP_GEMV, dev)
    ws_d = q.workspace(lay["down"][0], 1, q.QDEC_OP_GEMV, dev)
    calls = {"qkv": [], "o": [], "gate_up": [], "down": []}
    for l in range(L):
        calls["qkv"].append(GroupLaunch(q, [lay[n][l] for n in ("q", "k", "v")], [xt["qkv"]] * 3,
                                        [ys["q"], ys["k"], ys["v"]], ws_qkv))
        calls["o"].append(LazyLaunch(q, "qdec_gemv", lay["o"][l], xt["o"], ys["o"], 1, ws_o))
        calls["gate_up"].append(GroupLaunch(q, [lay[n][l] for n in ("gate", "up")], [xt["gate_up"]] * 2,
                                            [ys["gate"], ys["up"]], ws_gu))
        calls["down"].append(LazyLaunch(q, "qdec_gemv", lay["down"][l], xt["down"], ys["down"], 1, ws_d))

    def step(stream=None):
        for l in range(L):
            calls["qkv"][l](stream)
            calls["o"][l](stream)
            calls["gate_up"][l](stream)
            calls["down"][l](stream)

    def run_direct():
        step(torch.cuda.current_stream().cuda_stream)

    if args.call:                            # counter collection: one call only
        for i in range(8):
            calls[args.call][i % L]()
        torch.cuda.synchronize()
        log("call %s: 8 calls done" % args.call)
        copy_calibration(torch, dev, args.copy_calibration_mib)
        return None

    step()                                   # eager first (sets kernel attributes)
    torch.cuda.synchronize()
    graph = None
    if args.launch in ("auto", "graph"):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()

    def run_graph():
        graph.replay()

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    mode = args.launch
    probe = {}
    if mode == "auto":
        probe["graph_ms_per_step"] = round(timed(run_graph, 2) * 1e3, 3)
        probe["direct_ms_per_step"] = round(timed(run_direct, 2) * 1e3, 3)
        mode = "graph" if probe["graph_ms_per_step"] <= probe["direct_ms_per_step"] else "direct"
    run = run_graph if mode == "graph" else run_direct
    for i in range(args.warmup):
        run()
    torch.cuda.synchronize()
    # ---- timed region: exactly `steps` steps --------------------------------
    t0 = time.perf_counter()
    for i in range(args.steps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for nm, y in ys.items():
        if not torch.isfinite(y.float()).all():
            raise RuntimeError("non-finite output in %s" % nm)
    ms_per_step = elapsed / args.steps * 1e3
    gbs = step_bytes * args.steps / elapsed / 1e9
    us_layer = elapsed / (args.steps * L) * 1e6
    log("stack of %d layers: %d steps in %.4f s (%s): %.1f GB/s packed, %.2f us/layer"
        % (L, args.steps, elapsed, mode, gbs, us_layer))
    copy_calibration(torch, dev, args.copy_calibration_mib)
    del graph
    # ---- the calls of a layer, each alone: event-timed, rotating layers ----
    per_call = {}
    for g, cs in calls.items():
        us = time_calls(torch, cs)
        nb = call_bytes(cs[0].keep[0] if isinstance(cs[0], GroupLaunch) else [cs[0].keep[0]])
        per_call[g] = {"us": round(us, 2), "algorithmic_bytes": nb, "GBps": round(nb / us / 1e3, 1)}
    dom_name = max(per_call, key=lambda g: per_call[g]["us"])
    dom = per_call[dom_name]
    log("calls of a layer (us):", {g: v["us"] for g, v in per_call.items()})
    return {"gbs": gbs, "elapsed": elapsed, "ms_per_step": ms_per_step, "us_per_layer": us_layer,
            "step_bytes": step_bytes, "layer_bytes": layer_bytes, "mode": mode, "probe": probe,
            "per_call": per_call, "dominant": dom_name, "dom": dom, "inputs": inputs}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: every GPU box here has one, and the library's calls run on one "
              "device (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import dequant_matmul_packed_amd as q

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream().cuda_stream
    if args.layer:
        run_one_layer(q, torch, dev, stream, args.layer)
        return
    if args.call == "gemm":
        run_one_layer(q, torch, dev, stream, GEMM_LAYER)
        copy_calibration(torch, dev, args.copy_calibration_mib)
        return
    if args.call:
        args.layers = min(args.layers, 8)
        llama_stack(q, torch, dev, args)
        return
    H = llama_stack(q, torch, dev, args)
    torch.cuda.empty_cache()
    G = bench_gemm(q, torch, dev, stream)
    dom = H["dom"]
    kernels = {"gate_up": "qdec_gemv_group over gate and up (gemv_mma2_kernel + gemv_finish_lanes_kernel)",
               "qkv": "qdec_gemv_group over q, k, v (gemv_mma3_kernel + gemv_finish_lanes_kernel)",
               "down": "qdec_gemv 4096x14336 (gemv_mma1r_kernel + gemv_finish_lanes1_kernel)",
               "o": "qdec_gemv 4096x4096 (gemv_mma1_kernel + gemv_finish_lanes1_kernel)"}
    traffic = measured_traffic(H["dominant"], dom["algorithmic_bytes"])
    traffic_b64 = measured_traffic("gemm", G["algorithmic_bytes"])
    detail = {"per_call_of_a_layer": H["per_call"], "launch_probe": H["probe"],
              "gemm_b64_up70b": G}
    if not args.no_detail:
        detail.update(bench_projections(q, torch, dev, stream))
        detail.update(bench_llama_layer(q, torch, dev, stream))
        detail.update(bench_llama_layer(q, torch, dev, stream, "llama3_8b_layer_fused"))
        detail.update(bench_configs(q, torch, dev, stream))
        detail.update(bench_rht(q, torch, dev, stream))
        detail["pages_context"] = pages_context()
        ceil = measured_ceilings(torch, dev)
        detail["measured_ceilings"] = ceil
        G["frac_of_measured_fp16_matmul"] = round(G["TFLOPs"] / ceil["fp16_matmul_8192_TFLOPs"], 4)
        detail["dominant_frac_of_measured_read"] = round(dom["GBps"] / ceil["read_GBps_colsum_1GiB"], 4)
    if args.full_detail:
        detail.update(bench_code_variants(q, torch, dev, stream))
        detail.update(bench_fractional(q, torch, dev, stream))
        detail.update(bench_encoder(q, torch, dev, cpu=not args.no_cpu_baseline))
    cpu = None
    if not args.no_cpu_baseline:
        cpu, cpu_detail = cpu_baseline()
        if not args.no_detail:
            cpu_detail["per_config"] = cpu_per_config()
        detail["cpu_oracle"] = cpu_detail
    line = {
        "metric": METRIC,
        "value": round(H["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(H["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in/out, fp32 accumulate; 2-bit HYB codes",
        "data": "synthetic: seeded random code words (every word stream is a valid trellis walk), "
                "N(0,1) fp16 activations, random signs; no trained weights",
        "us_per_layer": round(H["us_per_layer"], 2),
        "config": {"workload": "Llama-3-8B-shaped decoder layers (q, o 4096x4096; k, v 1024x4096; gate, up "
                               "14336x4096; down 4096x14336), HYB k=2 V=2 Q=9, RHT both sides, batch 1; "
                               "one step = %d distinct layers, each as qkv group, o, gate+up group, down"
                               % args.layers,
                   "global_batch": 1, "layers_per_step": args.layers,
                   "packed_bytes_per_layer": H["layer_bytes"], "packed_bytes_per_step": H["step_bytes"],
                   "launch": H["mode"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kernels.get(H["dominant"], H["dominant"]),
                     "achieved": dom["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom["GBps"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic["bytes_per_call"] if traffic else None,
                     "traffic_detail": traffic,
                     "bytes_per_launch": dom["algorithmic_bytes"], "avg_launch_us": dom["us"],
                     "timing": "HIP events around 200 back-to-back calls on the launch stream (codes "
                               "rotating over the stack's layers), median of 5; a call is two kernels"},
        "roofline_b64": {"bound": "mfma", "kernel": "qdec_gemm 28672x8192 HYB k=3, X 64x8192 "
                                                    "(rht_split_kernel + gemm_kernel + rht_lanes_kernel)",
                         "achieved": G["TFLOPs"], "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(G["TFLOPs"] / MFMA_F16_PEAK_TFLOPS, 4),
                         "traffic": traffic_b64["bytes_per_call"] if traffic_b64 else None,
                         "traffic_detail": traffic_b64, "algorithmic_bytes": G["algorithmic_bytes"],
                         "flops_per_launch": G["flops"], "avg_launch_us": G["us_per_call"],
                         "timing": G["protocol"]},
        "cpu_baseline": cpu,
        "inputs": H["inputs"],
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


def measured_traffic(call, algorithmic):
    """HBM bytes per call of `call` from the committed counter summary
    (profiles/traffic.json), or None when there is none for it or the kernel
    sources differ from the profiled ones."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    v = rec.get("calls", {}).get(call)
    if v is None:
        return None
    return {"bytes_per_call": int(v["bytes_per_call"]), "read_bytes": int(v["read_bytes"]),
            "write_bytes": int(v["write_bytes"]),
            "over_algorithmic": round(v["bytes_per_call"] / algorithmic, 3),
            "source": "profiles/traffic.md (FETCH_SIZE, WRITE_SIZE scaled by a 256 MiB copy)"}


def bench_projections(q, torch, dev, stream):
    """Each projection shape of the Llama-3-8B layer alone at batch 1, timed
    as in time_layer (codes rotating through a pool of at least 1 GiB)."""
    import synth
    out = {}
    seen = set()
    for s in synth.WORKLOADS["llama3_8b_layer"].layers:
        if (s.m, s.n) in seen:
            continue
        seen.add((s.m, s.n))
        us, base = time_layer(q, torch, dev, stream, s.code, s.m, s.n, s.k, 1, "bench/proj/%dx%d" % (s.m, s.n))
        out["%dx%d" % (s.m, s.n)] = {"us_per_call": round(us, 2),
                                     "packed_GBps": round(base.code_bytes / (us * 1e-6) / 1e9, 1)}
    log("projections b=1:", {k: v["us_per_call"] for k, v in out.items()})
    return {"projections_b1": out}


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
    the 4096x4096 HYB k=2 layer (V=2, Q=9, 512-pair table), the same shape
    with the computed codes (1MAD, 3INST at k = 2, 3, 4), and the
    4096x14336 down-projection shape with the 3-bit non-uniform scalar
    quantizer (fp16 scale per 128 weights) and with the 2-D vector quantizer
    (8-bit index per weight pair).  GB/s on the packed codes, and on the
    algorithmic bytes (codes, x, y, signs, tables and group scales) as a
    fraction of the 8 TB/s HBM peak."""
    import synth
    out = {}
    cases = [("hyb4096", synth.WORKLOADS["hyb4096"].layers[0])]
    cases += [("computed4096/" + s.name, s) for s in synth.WORKLOADS["computed4096"].layers]
    cases += [("down_nuq", synth.WORKLOADS["down_nuq"].layers[0]), ("down_vq", synth.WORKLOADS["down_vq"].layers[0])]
    for wname, s in cases:
        kw = dict(scale=s.scale)
        us, base = time_layer(q, torch, dev, stream, s.code, s.m, s.n, s.k, 1, "bench/cfg/" + wname, **kw)
        alg = (base.code_bytes + 2 * s.n + 2 * s.m + (s.m + s.n) // 8 + tensor_bytes(base.lut)
               + tensor_bytes(base.group_scale))
        out[wname] = {"layer": synth.WORKLOADS[wname.split("/")[0]].description, "us_per_call": round(us, 2),
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
    # codes, X and Y in fp16, both sign vectors, the 2^Q-entry table
    nbytes = s.m * s.n * s.k // 8 + 2 * b * (s.n + s.m) + (s.m + s.n) // 8 + 4 * 512
    return {"us_per_call": round(us, 2), "TFLOPs": round(tf, 1), "flops": int(flops),
            "algorithmic_bytes": int(nbytes),
            "frac_of_fp16_mfma_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "launches": "rht_in + gemm + rht_out",
            "protocol": "HIP events around 200 back-to-back calls on the launch stream (codes rotating "
                        "through a 1 GiB pool), median of 5; a call is three kernels"}


def cpu_baseline(min_seconds=10.0, max_reps=8):
    """The oracle as it stands, on the host cores: full forwards (decode of
    every tile, O(B^2) Hadamards, fp64 matvec) of the seven projections of one
    Llama-3-8B-shaped layer at batch 1, repeated until about 10 s of CPU work;
    then, for the detail, decode-only on all threads and both on one thread
    over the q projection.  It is a correctness reference, not a tuned CPU
    competitor."""
    import oracle
    import synth
    threads = oracle.omp_threads()
    wl = synth.WORKLOADS["llama3_8b_layer"]
    hosts = [s.build("cpu_baseline") for s in wl.layers]
    xs = {n: synth.activations("cpu_baseline/x%d" % n, 1, n) for n in {h.n for h in hosts}}
    nbytes = sum(h.code_bytes for h in hosts)
    nweights = sum(h.m * h.n for h in hosts)
    reps, t_fwd = 0, 0.0
    while reps < max_reps and (reps == 0 or t_fwd < min_seconds):
        t0 = time.perf_counter()
        for h in hosts:
            oracle.forward(h, xs[h.n])
        t_fwd += time.perf_counter() - t0
        reps += 1
    t0 = time.perf_counter()
    for h in hosts:
        oracle.decode_tiles_storage(h, 0, h.n_tiles)
    t_dec = time.perf_counter() - t0
    oracle.set_threads(1)
    t0 = time.perf_counter()
    oracle.forward(hosts[0], xs[hosts[0].n])
    t_fwd1 = time.perf_counter() - t0
    oracle.set_threads(threads)
    gbs = nbytes * reps / t_fwd / 1e9
    log("cpu oracle: %d forwards of the 7 projections in %.2f s (%.4f GB/s, %d threads)"
        % (reps, t_fwd, gbs, threads))
    base = {"value": round(gbs, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d full forwards (batch 1) of the 7 projections of one Llama-3-8B-shaped layer "
                      "(%.1f MiB of codes each), %.1f s" % (reps, nbytes / 2 ** 20, t_fwd),
            "us_per_layer": round(t_fwd / reps * 1e6, 1)}
    detail = {"affinity_cores": len(os.sched_getaffinity(0)), "threads": threads,
              "forward_GBps": round(gbs, 5),
              "decode_Mweights_per_s": round(nweights / t_dec / 1e6, 2),
              "one_thread_forward_q_GBps": round(hosts[0].code_bytes / t_fwd1 / 1e9, 5)}
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
