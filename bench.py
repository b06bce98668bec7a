"""Benchmark of the routed MoE FFN layer on one MI355X.

A step is one pass of the whole layer (router, top-k, permutation, expert
SwiGLU with in-register dequant, shared expert, combine) for one decode token
through a 512-expert top-10 + 1 shared layer (H 2048, I 768, 4-bit group-32
weights, bf16 activations), with the inputs resident in HBM.  Consecutive
steps rotate over 16 distinct copies of the layer's weights (21.8 GB) so the
experts stream from HBM and not from the 256 MB last-level cache.  The K timed
steps are replayed from captured HIP graphs (up to 256 steps per graph); the
same steps launched directly are reported beside them.

Prints one JSON line (rank 0, N = 1):
  value        decode tokens/s (whole job)
  roofline     HBM roofline of the decode step: algorithmic bytes per step
               (router, the selected and shared experts, x and y) / time per step
  cpu_baseline the CPU oracle on a bounded sample of the same workload (all
               host cores and one thread)
plus extra fields: expert-weight GB/s, the directly launched steps (and the
median of 5 more repetitions), the HBM rates a plain device copy and sum reach
on this GPU, prefill tokens/s and MFMA fraction, the 5-token
verify batch, a batch sweep T = 8 .. 256 in each weight format, and one decode
step through the 48-layer 2-bit stack at batch 1 and 8 (expert planes filled
on the device), each with its distinct experts, algorithmic bytes and fraction
of 8 TB/s.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-prefill] [--no-graph] [--no-stack]
                    [--no-sweep]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_HBM_GBS = 8000.0

# HBM bytes of one decode step (the sum over its three kernels, one token, 10
# experts + shared) from two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE)
# over this script, each scaled by what the counter reads for a device copy of
# known size run in the same pass (--copy-calib-mib).  Valid for the kernel
# sources whose fingerprint is stored; reported as null once they change.
TRAFFIC_SOURCES = ("router.hip", "expert_gemv.hip", "gemv_one.h", "gemv_tile.h", "moe_device.h", "topk.h",
                   "moe_internal.h", "moe_abi.cpp")
MEASURED_TRAFFIC = {"bytes_per_step": 33959230,
                    "sources_sha256": "f43213300e6928850b0ca41a2a3349407331d2d3f4f2c3e8991c7a89db7852f4"}


def kernel_sources_sha256() -> str:
    import hashlib
    d = hashlib.sha256()
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_moe_router_amd", "csrc")
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(root, name), "rb") as f:
            d.update(f.read())
    return d.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--copies", type=int, default=16)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 4096-token prefill figure")
    ap.add_argument("--prefill-steps", type=int, default=16)
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the verify batch (5 tokens, 2-bit) and the 48-layer 2-bit stack figures")
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--no-sweep", action="store_true", help="skip the batch sweep T = 1 .. 256")
    ap.add_argument("--no-locality", action="store_true",
                    help="skip the hot-expert cache-locality figures of the 48-layer stack")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra timing of the same steps replayed from captured HIP graphs")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run 4 device-to-device copies of this many MiB (a counter calibration "
                         "kernel of known size for rocprofv3 --pmc runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from sparse_moe_router_amd import api, workload
    from synth import torch_io

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    api.lib()

    spec = synth.SPECS["decode"]
    E, K, H, I = spec.n_experts, spec.top_k, spec.hidden, spec.inter
    t0 = time.time()
    ld0 = synth.gen_layer(spec, seed=0, layer=0)
    log(f"generated the 512-expert layer in {time.time() - t0:.1f}s")
    kw0 = torch_io.layer_kwargs(ld0, dev)

    # copies 1..C-1: the same expert bytes at other addresses (experts rotated),
    # each with its own router and Zipf bias ranking
    layers = [api.Layer(**kw0)]
    for c in range(1, args.copies):
        w, b = synth.gen_router(spec, seed=0, layer=c)
        routed = {k: tuple(None if t is None else torch.roll(t, shifts=37 * c, dims=0).contiguous() for t in v)
                  for k, v in kw0["routed"].items()}
        shared = {k: tuple(None if t is None else t.clone() for t in v) for k, v in kw0["shared"].items()}
        kw = dict(kw0, router_w=torch.from_numpy(w).to(dev), router_b=torch.from_numpy(b).to(dev),
                  routed=routed, shared=shared)
        layers.append(api.Layer(**kw))
    torch.cuda.synchronize()
    log(f"{args.copies} weight copies resident ({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")

    n_tok = 256
    xs = torch_io.x_tensor(synth.gen_x(spec, seed=0, tokens=n_tok).storage, spec.act, dev)
    ws = api.workspace(layers[0], 4096, dev)
    y = torch.empty((4096, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, st):
        api.moe_layer_forward(layers[i % args.copies], xs[i % n_tok:i % n_tok + 1], 1, y, ws=ws, stream=st)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # directly launched steps: one moe_layer_forward call (three kernel
    # launches) per step from the host.  The (copy, token) pairs repeat with a
    # period of lcm(copies, n_tok) steps; their arguments are checked and
    # marshalled once, so the loop measures the GPU and not the Python
    # binding's per-call checks.
    period = n_tok * args.copies // math.gcd(n_tok, args.copies)
    bound_steps = [api.bind_layer_forward(layers[i % args.copies], xs[i % n_tok:i % n_tok + 1], 1, y, ws=ws,
                                          stream=stream) for i in range(period)]
    start.record(stream)
    for i in range(args.steps):
        bound_steps[(args.warmup + i) % period]()
    end.record(stream)
    torch.cuda.synchronize()
    direct_us = start.elapsed_time(end) * 1e3 / args.steps
    log(f"decode, direct launches: {direct_us:.2f} us/step")

    # the timed steps replayed from captured HIP graphs (a serving loop's way of
    # launching a step): graphs of up to 256 consecutive steps (one graph for
    # K <= 256), the K timed steps covered exactly, the same (copy, token)
    # sequence as above
    graph_us = None
    decode_launch = "direct"
    ms_per_step = direct_us * 1e-3
    if not args.no_graph:
        cap = torch.cuda.Stream()
        g_len = 256

        def capture(first, n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for i in range(n):
                    step(first + i, torch.cuda.current_stream())
            return g

        graphs = [capture(args.warmup + i, min(g_len, args.steps - i)) for i in range(0, args.steps, g_len)]
        for g in graphs:  # warm replays
            g.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for g in graphs:
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        graph_us = start.elapsed_time(end) * 1e3 / args.steps
        log(f"decode, HIP graph replay: {graph_us:.2f} us/step")
        decode_launch = f"HIP graph replay ({len(graphs)} graph{'s' if len(graphs) > 1 else ''} of up to {g_len} steps)"
        ms_per_step = graph_us * 1e-3
    tok_s = 1e3 / ms_per_step
    log(f"decode: {ms_per_step * 1e3:.2f} us/step, {tok_s:.0f} tok/s ({decode_launch})")

    # routing of each copy for its first timed token: distinct experts per step
    wts = torch.empty((1, K), dtype=torch.float32, device=dev)
    ids1 = torch.empty((1, K), dtype=torch.int32, device=dev)
    distinct = []
    for c in range(args.copies):
        api.moe_router_topk(layers[c], xs[c:c + 1], 1, ids1, wts, ws=ws)
        distinct.append(len(set(ids1.cpu().numpy().reshape(-1).tolist())))
    u_mean = float(np.mean(distinct))

    # median of 5 more repetitions of the timed loop (directly launched steps)
    reps5 = []
    for r in range(5):
        start.record(stream)
        for i in range(max(args.steps, 200)):
            bound_steps[(r * 997 + i) % period]()
        end.record(stream)
        torch.cuda.synchronize()
        reps5.append(start.elapsed_time(end) * 1e3 / max(args.steps, 200))
    log(f"decode, 5 more repetitions of {max(args.steps, 200)} steps: " + ", ".join(f"{v:.2f}" for v in reps5) + " us")

    exp_bytes = workload.expert_weight_bytes(spec.qfmt, H, I, int(round(u_mean)), spec.n_shared)
    layer_bytes = workload.spec_layer_bytes(spec, int(round(u_mean)), tokens=1)
    achieved = layer_bytes / (ms_per_step * 1e-3) / 1e9
    extra = {
        "expert_weight_GBps": exp_bytes / (ms_per_step * 1e-3) / 1e9,
        "expert_weight_frac_of_8TBps": exp_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "layer_algorithmic_GBps": achieved,
        "layer_algorithmic_bytes": layer_bytes,
        "decode_launch": decode_launch,
        "decode_direct_launch_us_per_step": direct_us,
        "decode_graph_replay_us_per_step": graph_us,
        "decode_direct_us_per_step_median5": float(np.median(reps5)),
        "decode_direct_us_per_step_reps5": reps5,
        "distinct_experts_per_token": u_mean,
        "weight_copies": args.copies,
    }

    if not args.no_prefill:
        ps = synth.SPECS["prefill"]
        xp = torch_io.x_tensor(synth.gen_x(ps, seed=0).storage, ps.act, dev)
        for i in range(2):
            api.moe_layer_forward(layers[i % args.copies], xp, ps.tokens, y, ws=ws, stream=stream)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.prefill_steps):
            api.moe_layer_forward(layers[i % args.copies], xp, ps.tokens, y, ws=ws, stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        pms = start.elapsed_time(end) / args.prefill_steps
        flops = workload.layer_flops(H, I, E, K, ps.tokens, ps.n_shared)
        extra["prefill_tok_s"] = ps.tokens / (pms * 1e-3)
        extra["prefill_ms_per_layer"] = pms
        extra["prefill_TFLOPs"] = flops / (pms * 1e-3) / 1e12
        extra["prefill_frac_of_bf16_mfma"] = flops / (pms * 1e-3) / 2.5e15
        log(f"prefill: {pms:.3f} ms/layer, {extra['prefill_tok_s']:.0f} tok/s")

    probe = hbm_probe(dev)
    extra["hbm_probe"] = probe
    extra["decode_frac_of_copy_probe"] = achieved / probe["copy_GBps"]

    if not args.no_stack:
        extra.update(verify_and_stack(args, dev, q4_layers=layers))
    if not args.no_locality:
        extra["hot_expert_locality"] = hot_expert_locality(args, dev)

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 4 copies of {args.copy_calib_mib} MiB")

    traffic = (MEASURED_TRAFFIC["bytes_per_step"]
               if MEASURED_TRAFFIC["sources_sha256"] == kernel_sources_sha256() else None)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(spec, ld0)

    out = {
        "metric": "MoE-layer decode tok/s + expert-weight HBM GB/s (% peak); prefill tok/s",
        "value": tok_s,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # fp32 arithmetic on bf16 activations and 4-bit codes
        "data": "synthetic",
        "config": {
            "workload": "decode: 1 token/step through one routed MoE FFN layer, hidden 2048, 512 experts, "
                        "top-10 + 1 shared, intermediate 768, 4-bit sym group-32 fp16-scale weights, bf16 activations, "
                        "fp32 router with Zipf(1.1) bias; 16 rotating weight copies; steps launched as "
                        + decode_launch,
            "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "the whole decode layer step (k_router_logits, k_fused_gateup1, k_fused_down1): "
                      "algorithmic bytes per step / time per step",
            "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic, "us_per_launch": ms_per_step * 1e3, "algorithmic_bytes_per_launch": layer_bytes,
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def _distinct(layer, x, T, ws, dev):
    """Distinct experts selected by the T tokens of one step (routing on the device)."""
    import torch

    from sparse_moe_router_amd import api
    ids = torch.empty((T, layer.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, layer.top_k), dtype=torch.float32, device=dev)
    api.moe_router_topk(layer, x, T, ids, w, ws=ws)
    return len(np.unique(ids.cpu().numpy()))


def _time_steps(fn, n, stream):
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / n


def batch_figures(spec, layers, T, xpool, ws, y, stream, dev, n_steps, prefix):
    """T tokens per step through rotating layer copies: us/step, tokens/s, the mean
    distinct experts U, the algorithmic bytes per step and their fraction of 8 TB/s."""
    from sparse_moe_router_amd import api, workload
    n_win = xpool.shape[0] // T
    copies = len(layers)
    u = [_distinct(layers[i % copies], xpool[(i % n_win) * T:(i % n_win + 1) * T], T, ws, dev)
         for i in range(min(copies * n_win, 32))]
    bound = [api.bind_layer_forward(layers[i % copies], xpool[(i % n_win) * T:(i % n_win + 1) * T], T, y, ws=ws,
                                    stream=stream) for i in range(min(copies * n_win, 64))]
    for i in range(min(len(bound), 20)):
        bound[i]()
    us = _time_steps(lambda i: bound[i % len(bound)](), n_steps, stream)
    u_mean = float(np.mean(u))
    b = float(np.mean([workload.spec_layer_bytes(spec, v, tokens=T) for v in u]))
    return {f"{prefix}_us_per_step": us, f"{prefix}_tok_s": T / (us * 1e-6), f"{prefix}_distinct_experts": u_mean,
            f"{prefix}_algorithmic_bytes": b, f"{prefix}_frac_of_8TBps": b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}


def verify_and_stack(args, dev, q4_layers=None):
    """Extra figures with expert planes filled on the device (2-bit format unless
    stated): the speculative-verify batch (5 tokens through one layer, 16 layer
    copies rotating), the batch sweep T = 1 .. 256 in each format (4-bit on the
    decode copies, 3-bit and 2-bit filled on the device), and one decode step
    through the 48-layer stack at batch 1 and 8, each with its distinct experts,
    algorithmic bytes and fraction of 8 TB/s."""
    import torch

    import synth
    from sparse_moe_router_amd import api, workload
    from synth import torch_io
    out = {}
    stream = torch.cuda.current_stream()

    vs = synth.SPECS["verify"]
    vlayers = [api.Layer(**torch_io.device_filled_kwargs(vs, c, dev)) for c in range(args.copies)]
    xv = torch_io.x_tensor(synth.gen_x(vs, seed=0, tokens=4096).storage, vs.act, dev)
    ws = api.workspace(vlayers[0], 256, dev)
    yv = torch.empty((256, vs.hidden), dtype=torch.float32, device=dev)
    f = batch_figures(vs, vlayers, vs.tokens, xv, ws, yv, stream, dev, max(200, args.steps // 4), "verify_T5_q2")
    out.update(f)
    log(f"verify (T=5, 2-bit): {f['verify_T5_q2_us_per_step']:.2f} us/step, U = "
        f"{f['verify_T5_q2_distinct_experts']:.1f}, {100 * f['verify_T5_q2_frac_of_8TBps']:.1f} % of 8 TB/s")
    if not args.no_sweep:
        sweep = {}
        q3s = synth.SPECS["decode_q3"]
        q3_layers = [api.Layer(**torch_io.device_filled_kwargs(q3s, c, dev)) for c in range(args.copies)]
        for fmt, ls, sp in (("q4", q4_layers, synth.SPECS["decode"]), ("q3", q3_layers, q3s), ("q2", vlayers, vs)):
            if ls is None:
                continue
            xq = xv if fmt == "q2" else torch_io.x_tensor(synth.gen_x(sp, seed=1, tokens=4096).storage, sp.act, dev)
            for T in (1, 5, 8, 16, 32, 64, 128, 256):
                g = batch_figures(sp, ls, T, xq, ws, yv, stream, dev, max(20, 1600 // T), f"T{T}")
                sweep[f"{fmt}_T{T}"] = {k.split("_", 1)[1]: v for k, v in g.items()}
                log(f"batch sweep {fmt} T={T}: {g[f'T{T}_us_per_step']:.1f} us/step, "
                    f"{g[f'T{T}_tok_s']:.0f} tok/s, U = {g[f'T{T}_distinct_experts']:.1f}, "
                    f"{100 * g[f'T{T}_frac_of_8TBps']:.1f} % of 8 TB/s")
        out["batch_sweep"] = sweep
        del q3_layers
    del vlayers, ws
    torch.cuda.empty_cache()

    ss = synth.SPECS["stack_t1"]
    t0 = time.time()
    stack = [api.Layer(**torch_io.device_filled_kwargs(ss, l, dev)) for l in range(ss.n_layers)]
    torch.cuda.synchronize()
    log(f"48-layer 2-bit stack filled on the device in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    for T in (1, 8):
        spec = synth.SPECS["stack_t1" if T == 1 else "stack_t8"]
        ws = api.workspace(stack[0], T, dev)
        base = torch_io.x_tensor(synth.gen_x(spec, seed=0, tokens=T).storage, spec.act, dev)
        # the distinct experts of every layer on this input (the residual stream
        # through the layers, as the stack computes it)
        cur = base.clone()
        u = []
        for L in stack:
            u.append(_distinct(L, cur, T, ws, dev))
            api.moe_layer_forward(L, cur, T, torch.empty((T, spec.hidden), dtype=torch.float32, device=dev),
                                  x_next=cur, ws=ws, stream=stream)
        torch.cuda.synchronize()
        xs = [base.clone() for _ in range(args.stack_steps + 2)]  # each step starts from the same x
        for k in range(2):
            api.moe_stack_forward(stack, xs[k], T, ws=ws, stream=stream)
        torch.cuda.synchronize()
        us = _time_steps(lambda k: api.moe_stack_forward(stack, xs[2 + k], T, ws=ws, stream=stream),
                         args.stack_steps, stream)
        b = float(sum(workload.spec_layer_bytes(ss, v, tokens=T) for v in u))
        out[f"stack48_q2_T{T}_us_per_step"] = us
        out[f"stack48_q2_T{T}_tok_s"] = T / (us * 1e-6)
        out[f"stack48_q2_T{T}_distinct_experts_per_layer"] = float(np.mean(u))
        out[f"stack48_q2_T{T}_algorithmic_bytes"] = b
        out[f"stack48_q2_T{T}_frac_of_8TBps"] = b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS
        log(f"48-layer stack, T={T}: {us:.1f} us/step ({T / (us * 1e-6):.0f} tok/s), U per layer "
            f"{np.mean(u):.1f}, {100 * out[f'stack48_q2_T{T}_frac_of_8TBps']:.1f} % of 8 TB/s")
        del ws, xs
    return out


def hot_expert_locality(args, dev):
    """Hot experts kept in the last-level cache (the 256 MB memory-side cache)
    across decode steps of the 48-layer 2-bit stack: experts numbered by
    popularity (the Zipf rank of the router bias), the layers' hot_experts set
    to 0 (every expert streams past the caches), 2, 8 or 512 (every expert
    cache-allocating), at Zipf exponents 0 (no skew), 1.1 and 2.0; one decode
    step per timing unit, batch 1 and 8, each step starting from a new token."""
    import dataclasses

    import torch

    import synth
    from sparse_moe_router_amd import api, workload
    from synth import torch_io
    out = {}
    stream = torch.cuda.current_stream()
    for s in (0.0, 1.1, 2.0):
        base = synth.SPECS["stack_t1"]
        spec = dataclasses.replace(base, zipf_s=s if s > 0 else None, ordered=True, name=f"stack_zipf{s}")
        kws = [torch_io.device_filled_kwargs(spec, l, dev) for l in range(spec.n_layers)]
        for T in (1, 8):
            xs = torch_io.x_tensor(synth.gen_x(dataclasses.replace(spec, tokens=T), seed=5, tokens=64 * T).storage,
                                   spec.act, dev)
            ws = api.workspace(api.Layer(**kws[0]), T, dev)
            for hot in (0, 2, 8, 512):
                stack = [api.Layer(**k, hot_experts=hot) for k in kws]
                bufs = [xs[(i % 64) * T:(i % 64 + 1) * T].clone() for i in range(args.stack_steps + 4)]
                for k in range(4):
                    api.moe_stack_forward(stack, bufs[k], T, ws=ws, stream=stream)
                torch.cuda.synchronize()
                us = _time_steps(lambda k: api.moe_stack_forward(stack, bufs[4 + k], T, ws=ws, stream=stream),
                                 args.stack_steps, stream)
                out[f"zipf{s}_T{T}_hot{hot}_us_per_step"] = us
                log(f"hot-expert locality: Zipf {s}, T={T}, hot_experts={hot}: {us:.1f} us/step "
                    f"({T / (us * 1e-6):.0f} tok/s)")
            del ws
        del kws
        torch.cuda.empty_cache()
    return out


def hbm_probe(dev):
    """Achievable HBM rates on this GPU with plain library kernels, as context
    for the 8 TB/s spec: a device-to-device copy of 2 GiB (bytes read plus
    bytes written over the time) and a sum of 4 GiB of fp32 (bytes read over
    the time), the median of 5 timed runs of each after two warm runs."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(fn, nbytes):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        r = []
        for _ in range(5):
            start.record()
            fn()
            end.record()
            torch.cuda.synchronize()
            r.append(nbytes / (start.elapsed_time(end) * 1e-3) / 1e9)
        return float(np.median(r))

    a = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    copy = rate(lambda: b.copy_(a), 2 * a.numel() * 4)
    del a, b
    big = torch.ones(1 << 30, dtype=torch.float32, device=dev)
    read = rate(lambda: big.sum(), big.numel() * 4)
    del big
    torch.cuda.empty_cache()
    log(f"HBM probe: copy {copy:.0f} GB/s (read + write), sum {read:.0f} GB/s (read)")
    return {"copy_GBps": copy, "sum_read_GBps": read,
            "how": "torch device copy of 2 GiB (read + written bytes) and torch sum of 4 GiB fp32 (read bytes), "
                   "median of 5"}


def _host_cpu():
    model = None
    try:
        import subprocess
        for line in subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    return model


def cpu_baseline(spec, ld):
    """The oracle (float64 NumPy) on decode tokens of the same layer: with the BLAS
    threads at their default (all host cores) and at 1 thread, each the median
    of 3 runs of about 4 s (at most 96 tokens each)."""
    import synth
    from oracle import moe_oracle as mo
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    x = synth.gen_x(spec, seed=0, tokens=96).values

    def run():
        t0 = time.time()
        n = 0
        while n < 96 and (time.time() - t0 < 4.0 or n < 2):
            mo.layer_forward(ld, x[n:n + 1], keep_expert_out=False)
            n += 1
        return n / (time.time() - t0), n

    all_cores = [run() for _ in range(3)]
    with threadpool_limits(limits=1):
        one = [run() for _ in range(3)]
    v_all = float(np.median([r for r, _ in all_cores]))
    v_one = float(np.median([r for r, _ in one]))
    log(f"cpu oracle: {v_all:.2f} tok/s on {threads} BLAS threads, {v_one:.2f} tok/s on 1 thread")
    return {"value": v_all, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": "decode tokens (T=1 each) through the same 512-expert 4-bit layer, float64 NumPy; median of 3 "
                      f"runs of about 4 s ({', '.join(str(n) for _, n in all_cores)} tokens)",
            "single_thread_value": v_one, "os_cpu_count": os.cpu_count(), "host_cpu": _host_cpu()}


if __name__ == "__main__":
    main()
