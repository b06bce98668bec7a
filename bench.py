"""Benchmark of the routed MoE FFN layer on one MI355X.

A step is one pass of the whole layer (router, top-k, permutation, expert
SwiGLU with in-register dequant, shared expert, combine) for one decode token
through a 512-expert top-10 + 1 shared layer (H 2048, I 768, 4-bit group-32
weights, bf16 activations), with the inputs resident in HBM.  Consecutive
steps rotate over 16 distinct copies of the layer's weights (21.8 GB) so the
experts stream from HBM and not from the 256 MB last-level cache.

Prints one JSON line (rank 0, N = 1):
  value        decode tokens/s (whole job)
  roofline     HBM roofline of the dominant kernel (expert gate/up + SwiGLU),
               algorithmic bytes per launch / HIP-event time per launch
  cpu_baseline the CPU oracle on a bounded sample of the same workload
plus extra fields: expert-weight GB/s of the whole layer, the same decode steps
and gate/up launches replayed from captured HIP graphs, prefill tokens/s, the
5-token verify batch and one decode step through the 48-layer 2-bit stack at
batch 1 and 8 (expert planes filled on the device).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-prefill] [--no-graph] [--no-stack]
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

# HBM bytes per launch of the roofline kernel (k_gateup1, one token, 10 experts +
# shared) from two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) over this
# script, each scaled by what the counter reads for a 256 MiB device copy
# (FETCH_SIZE x 1.99981, WRITE_SIZE x 1.0).  Valid for the kernel sources whose
# fingerprint is stored; reported as null once they change.
TRAFFIC_SOURCES = ("expert_gemv.hip", "gemv_one.h", "gemv_tile.h", "moe_device.h", "topk.h", "moe_internal.h")
MEASURED_TRAFFIC = {"bytes_per_launch": 19604844,
                    "sources_sha256": "2a1801e1b42238b9c43c6588bae4d8f5b90d526225c6d301b0c8c754ac4e5bcf"}


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
    ap.add_argument("--kernel-reps", type=int, default=2000)
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the verify batch (5 tokens, 2-bit) and the 48-layer 2-bit stack figures")
    ap.add_argument("--stack-steps", type=int, default=20)
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
    ms_per_step = start.elapsed_time(end) / args.steps
    tok_s = 1e3 / ms_per_step
    log(f"decode: {ms_per_step * 1e3:.2f} us/step, {tok_s:.0f} tok/s")

    # extra: the same steps replayed from captured HIP graphs (a serving loop's
    # way of launching a step), args.copies steps per graph, 8 graphs over
    # different tokens, cycled
    graph_us = None
    if not args.no_graph:
        g_steps, n_graphs = args.copies, 8
        cap = torch.cuda.Stream()

        def capture(first):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for i in range(g_steps):
                    step(first + i, torch.cuda.current_stream())
            return g

        graphs = [capture(j * g_steps) for j in range(n_graphs)]
        for g in graphs:  # warm replays
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // g_steps)
        start.record(stream)
        for r in range(reps):
            graphs[r % n_graphs].replay()
        end.record(stream)
        torch.cuda.synchronize()
        graph_us = start.elapsed_time(end) * 1e3 / (reps * g_steps)
        log(f"decode, HIP graph replay: {graph_us:.2f} us/step")

    # routing of each copy for its first timed token: distinct experts per step
    wts = torch.empty((1, K), dtype=torch.float32, device=dev)
    idss = [torch.empty((1, K), dtype=torch.int32, device=dev) for _ in range(args.copies)]
    offs = [torch.empty(E + 1, dtype=torch.int32, device=dev) for _ in range(args.copies)]
    sps = [torch.empty(K, dtype=torch.int32, device=dev) for _ in range(args.copies)]
    pp = torch.empty(K, dtype=torch.int32, device=dev)
    distinct = []
    for c in range(args.copies):
        api.moe_router_topk(layers[c], xs[c:c + 1], 1, idss[c], wts, ws=ws)
        api.moe_permute(layers[c], idss[c], 1, offs[c], sps[c], pp, ws)
        distinct.append(len(set(idss[c].cpu().numpy().reshape(-1).tolist())))
    u_mean = float(np.mean(distinct))

    # dominant kernel: expert gate/up + SwiGLU (one kernel per call), timed
    # with HIP events on the stream it runs on, launches back to back (bound
    # calls, as for the steps above)
    h = torch.empty((K, I), dtype=torch.bfloat16, device=dev)
    hs = torch.empty((1, I), dtype=torch.bfloat16, device=dev)
    for r in range(50):
        c = r % args.copies
        api.moe_expert_gate_up_q(layers[c], xs[c:c + 1], 1, idss[c], offs[c], sps[c], h, hs, stream=stream)
    torch.cuda.synchronize()
    bound_gu = [api.bind_expert_gate_up_q(layers[c], xs[c:c + 1], 1, idss[c], offs[c], sps[c], h, hs, stream=stream)
                for c in range(args.copies)]
    start.record(stream)
    for r in range(args.kernel_reps):
        bound_gu[r % args.copies]()
    end.record(stream)
    torch.cuda.synchronize()
    k_us = start.elapsed_time(end) * 1e3 / args.kernel_reps
    # the same launches replayed from a captured graph
    k_graph_us = None
    gg = torch.cuda.CUDAGraph() if not args.no_graph else None
    if gg is not None:
        with torch.cuda.graph(gg, stream=torch.cuda.Stream()):
            for c in range(args.copies):
                api.moe_expert_gate_up_q(layers[c], xs[c:c + 1], 1, idss[c], offs[c], sps[c], h, hs)
        gg.replay()
        torch.cuda.synchronize()
        reps = max(1, args.kernel_reps // args.copies)
        start.record(stream)
        for r in range(reps):
            gg.replay()
        end.record(stream)
        torch.cuda.synchronize()
        k_graph_us = start.elapsed_time(end) * 1e3 / (reps * args.copies)
    gu_bytes_unit = 2 * workload.matrix_bytes(spec.qfmt, I, H)       # gate + up of one expert
    gu_bytes = (u_mean + 1) * gu_bytes_unit + (u_mean + 1) * H * 2 + (K + 1) * I * 2  # + x reads, h writes
    achieved = gu_bytes / (k_us * 1e-6) / 1e9
    log(f"gate/up kernel: {k_us:.2f} us/launch, {achieved:.0f} GB/s")

    exp_bytes = workload.expert_weight_bytes(spec.qfmt, H, I, int(round(u_mean)), spec.n_shared)
    layer_bytes = workload.spec_layer_bytes(spec, int(round(u_mean)), tokens=1)
    extra = {
        "expert_weight_GBps": exp_bytes / (ms_per_step * 1e-3) / 1e9,
        "expert_weight_frac_of_8TBps": exp_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "layer_algorithmic_GBps": layer_bytes / (ms_per_step * 1e-3) / 1e9,
        "layer_algorithmic_bytes": layer_bytes,
        "decode_graph_replay_us_per_step": graph_us,
        "gateup_graph_replay_us_per_launch": k_graph_us,
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

    if not args.no_stack:
        extra.update(verify_and_stack(args, dev))

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 4 copies of {args.copy_calib_mib} MiB")

    traffic = (MEASURED_TRAFFIC["bytes_per_launch"]
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
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode: 1 token/step through one routed MoE FFN layer, hidden 2048, 512 experts, "
                        "top-10 + 1 shared, intermediate 768, 4-bit sym group-32 fp16-scale weights, bf16 activations, "
                        "fp32 router with Zipf(1.1) bias; 16 rotating weight copies",
            "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm", "kernel": "expert gate/up + SwiGLU, one token (k_gateup1)",
            "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic, "us_per_launch": k_us, "algorithmic_bytes_per_launch": gu_bytes,
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def verify_and_stack(args, dev):
    """Extra figures on the 2-bit format, with expert planes filled on the device:
    the speculative-verify batch (5 tokens through one layer, 16 layer copies
    rotating) and one decode step through the 48-layer stack at batch 1 and 8."""
    import torch

    import synth
    from sparse_moe_router_amd import api, workload
    from synth import torch_io
    out = {}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()

    vs = synth.SPECS["verify"]
    vlayers = [api.Layer(**torch_io.device_filled_kwargs(vs, c, dev)) for c in range(args.copies)]
    xv = torch_io.x_tensor(synth.gen_x(vs, seed=0, tokens=64 * vs.tokens).storage, vs.act, dev)
    ws = api.workspace(vlayers[0], vs.tokens, dev)
    yv = torch.empty((vs.tokens, vs.hidden), dtype=torch.float32, device=dev)

    def vstep(i):
        t0 = (i % 64) * vs.tokens
        api.moe_layer_forward(vlayers[i % args.copies], xv[t0:t0 + vs.tokens], vs.tokens, yv, ws=ws, stream=stream)

    for i in range(50):
        vstep(i)
    torch.cuda.synchronize()
    n = max(200, args.steps // 4)
    start.record(stream)
    for i in range(n):
        vstep(i)
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / n
    out["verify_T5_q2_us_per_step"] = us
    out["verify_T5_q2_tok_s"] = vs.tokens / (us * 1e-6)
    log(f"verify (T=5, 2-bit): {us:.2f} us/step")
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
        xs = [base.clone() for _ in range(args.stack_steps + 2)]  # each step starts from the same x
        for k in range(2):
            api.moe_stack_forward(stack, xs[k], T, ws=ws, stream=stream)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(args.stack_steps):
            api.moe_stack_forward(stack, xs[2 + k], T, ws=ws, stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        us = start.elapsed_time(end) * 1e3 / args.stack_steps
        out[f"stack48_q2_T{T}_us_per_step"] = us
        out[f"stack48_q2_T{T}_tok_s"] = T / (us * 1e-6)
        if T == 1:
            b = ss.n_layers * workload.spec_layer_bytes(ss, ss.top_k, tokens=1)
            out["stack48_q2_T1_algorithmic_GBps"] = b / (us * 1e-6) / 1e9
        log(f"48-layer stack, T={T}: {us:.1f} us/step ({T / (us * 1e-6):.0f} tok/s)")
        del ws, xs
    return out


def cpu_baseline(spec, ld):
    """The oracle (float64 NumPy) on decode tokens of the same layer, for about 12 s (at most 256 tokens)."""
    import synth
    from oracle import moe_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    x = synth.gen_x(spec, seed=0, tokens=256).values
    t0 = time.time()
    n = 0
    while n < 256 and (time.time() - t0 < 12.0 or n < 2):
        mo.layer_forward(ld, x[n:n + 1], keep_expert_out=False)
        n += 1
    dt = time.time() - t0
    log(f"cpu oracle: {n} tokens in {dt:.1f}s")
    return {"value": n / dt, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} decode tokens (T=1 each) through the same 512-expert 4-bit layer, float64 NumPy"}


if __name__ == "__main__":
    main()
