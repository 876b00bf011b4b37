"""Benchmark of the MXFP4 MoE decode layer on one MI355X.

Metric: MoE decode us/call and achieved HBM GB/s on the bytes of the touched
experts, at T = 1..32 tokens per call.  Default workload: the
gpt-oss-120b-shaped layer (K = I = 2880, 128 experts, top-4 softmax with
logits N(0, 2), biases, clamped SwiGLU), one call at each of T = 1, 4, 8, 16,
32; a "step" is one replay of the call chain of every T.  The other
workloads (gpt-oss-20b-shaped, the GLM-5.x slice, the wide-K slice) are
measured the same way and reported under `other_configs`.

Method (the pages' per-call method, "MXFP4 MoE decode kernels", Measured
results: a chain of calls in a graph, median of the replays), made robust to
the 256 MB Infinity Cache: each T gets a HIP graph of L >= 8 back-to-back
layer calls that rotate over L distinct weight replicas and input sets (L
chosen so that one rotation moves more than 512 MB); after `--warmup` untimed
replays, `--steps` replays are timed one by one with HIP events on the
launch stream and us/call = median replay time / L.  The same chains of the
three steps alone (plan, gate_up, down) give the per-kernel times; the
gate/up kernel is the dominant one and feeds `roofline`.

Weights are stored in the library's tiled layout (MOE_LAYOUT_TILE16), made in
place once at load before any timing; `--layout rows` measures the served row
layout instead.

Algorithmic bytes of one call: for every touched local expert its packed
weights and scales (3*I*K*17/32 bytes) plus biases, plus x (2TK), the router
logits (4*T*E_global) and the output (2TK).  Touched experts and local routes
are read back from the plan the library writes, so they are the realised ones.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HEADLINE = "gptoss120b"
OTHER_CONFIGS = ("gptoss20b", "glm5_ep", "widek")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30, help="timed replays of every T's call chain (median taken)")
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default=HEADLINE)
    p.add_argument("--tokens", default=None, help="comma-separated T values (default: the layer's decode sweep)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-other-configs", action="store_true",
                   help="measure the headline workload only (the other workloads are reported by default)")
    p.add_argument("--rotate-mb", type=float, default=512.0, help="bytes one replica rotation must exceed")
    p.add_argument("--copy-probe", type=float, default=0.0,
                   help="only copy this many MiB device to device a few times and exit (counter calibration)")
    p.add_argument("--encode", action="store_true",
                   help="measure the MXFP4 encoder instead (bf16 weights of the layer's w13 -> packed + scales)")
    p.add_argument("--layout", default="tile16", choices=("rows", "tile16"),
                   help="packed weight storage order (tile16: tiled in place once, before any timing)")
    p.add_argument("--w13-order", default="gate_up", choices=("gate_up", "interleaved"),
                   help="row order of w13 (interleaved: gate and up rows alternate)")
    p.add_argument("--prefill", action="store_true",
                   help="time the prefill path (unpack the touched experts to bf16, then bf16 MFMA GEMMs) "
                        "against the decode path on the same calls (default: the wide-K slice at T=256, 2048)")
    p.add_argument("--down-pairing", default="auto", choices=("auto", "on", "off"),
                   help="row pairing of the down projection (a performance control; same results)")
    p.add_argument("--mma", default="bf16", choices=("bf16", "scaled_fp4"),
                   help="matrix instructions for experts with many routes (the MFMA list path): bf16 after an "
                        "in-register FP4 decode, or scaled-FP4 MFMA on hi + lo E4M3 activations")
    p.add_argument("--per-route", action="store_true",
                   help="per-route output: fp32 [T*top_k, K] rows instead of the bf16 token sums")
    return p.parse_args()


class Replica:
    def __init__(self, torch, cfg, idx, w_np=None):
        dev = "cuda"
        K, I, E = cfg.K, cfg.I, cfg.E_local
        if w_np is not None:
            def u8(a):
                return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            self.w13p, self.w13s = u8(w_np.w13_packed), u8(w_np.w13_scales)
            self.w2p, self.w2s = u8(w_np.w2_packed), u8(w_np.w2_scales)
            self.b13 = self.b2 = None
            if w_np.b13 is not None:
                self.b13 = torch.from_numpy(w_np.b13.view(np.int16)).to(dev).view(torch.bfloat16)
                self.b2 = torch.from_numpy(w_np.b2.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(1000 * cfg.index + idx)
            self.w13p = torch.randint(0, 256, (E, 2 * I, K // 2), dtype=torch.uint8, device=dev, generator=g)
            self.w13s = torch.randint(cfg.scale_lo, cfg.scale_hi + 1, (E, 2 * I, K // 32), dtype=torch.uint8,
                                      device=dev, generator=g)
            self.w2p = torch.randint(0, 256, (E, K, I // 2), dtype=torch.uint8, device=dev, generator=g)
            self.w2s = torch.randint(cfg.scale_lo, cfg.scale_hi + 1, (E, K, I // 32), dtype=torch.uint8,
                                     device=dev, generator=g)
            self.b13 = self.b2 = None
            if cfg.bias:
                self.b13 = torch.randn((E, 2 * I), device=dev, generator=g).to(torch.bfloat16)
                self.b2 = torch.randn((E, K), device=dev, generator=g).to(torch.bfloat16)


def replica_count(cfg, tokens, rotate_mb):
    """Distinct replicas: one rotation moves > rotate_mb of expert bytes at the smallest T; at least 8."""
    t_min = min(tokens)
    exp_touched = cfg.E_local * (1 - (1 - cfg.top_k / cfg.E_global) ** t_min)
    return max(8, math.ceil(rotate_mb * 1e6 / max(1.0, exp_touched * cfg.bytes_per_expert())))


def make_replicas(torch, moe, cfg, L, layout, w0=None):
    reps = [Replica(torch, cfg, 0, w0)] + [Replica(torch, cfg, i) for i in range(1, L)]
    if layout == "tile16":   # one-time, at weight load
        for r in reps:
            moe.moe_mxfp4_tile_weights(r.w13p)
            moe.moe_mxfp4_tile_weights(r.w2p)
    torch.cuda.synchronize()
    return reps


def time_graph(torch, g, stream, replays, warmup):
    """Median, min and max of `replays` timed replays (HIP events on `stream`
    around each replay), in us.  The replays are enqueued back to back and
    read after one synchronisation, so no replay waits for the host."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    with torch.cuda.stream(stream):
        for e0, e1 in ev:
            e0.record(stream)
            g.replay()
            e1.record(stream)
    torch.cuda.synchronize()
    times = [e0.elapsed_time(e1) * 1000.0 for e0, e1 in ev]
    return statistics.median(times), min(times), max(times)


def measure_config(torch, moe, cfg, tokens, args, reps, breakdown=True):
    """Per T: us/call (median of args.steps replays of an L-call chain), bytes and
    GB/s; with `breakdown`, the plan / gate_up / down chains timed the same way."""
    from workloads import make_inputs
    L = len(reps)
    K, I = cfg.K, cfg.I
    per_expert = cfg.bytes_per_expert()
    w13_per_expert = 2 * I * (K // 2) + 2 * I * (K // 32) + (4 * I if cfg.bias else 0)
    stream = torch.cuda.Stream()
    results = {}
    for T in tokens:
        d = moe.make_desc(T=T, K=K, I=I, E_global=cfg.E_global, E_local=cfg.E_local, top_k=cfg.top_k,
                          expert_offset=cfg.expert_offset, scoring=cfg.scoring, activation=cfg.activation,
                          swiglu_alpha=cfg.swiglu_alpha, swiglu_limit=cfg.swiglu_limit, weight_layout=args.layout,
                          w13_order=args.w13_order, down_pairing=args.down_pairing, mma=args.mma)
        ws_bytes = moe.moe_mxfp4_workspace_bytes(d)
        inputs = [make_inputs(cfg, T, call=i) for i in range(L)]
        xs = [torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16) for inp in inputs]
        lg = [torch.from_numpy(inp.logits).cuda() for inp in inputs]
        wss = [torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") for _ in range(L)]
        if args.per_route:
            outs = [torch.empty((T * cfg.top_k, K), dtype=torch.float32, device="cuda") for _ in range(L)]
        else:
            outs = [torch.empty((T, K), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
        out_bytes = outs[0].numel() * outs[0].element_size()
        decode_fn = moe.moe_mxfp4_decode_routes if args.per_route else moe.moe_mxfp4_decode
        down_fn = moe.moe_mxfp4_down_routes if args.per_route else moe.moe_mxfp4_down

        def call_decode(i, s):
            r = reps[i]
            decode_fn(d, xs[i], r.w13p, r.w13s, r.w2p, r.w2s, outs[i], router_logits=lg[i],
                      w13_bias=r.b13, w2_bias=r.b2, workspace=wss[i], stream=s)

        def call_plan(i, s):
            moe.moe_mxfp4_plan(d, router_logits=lg[i], workspace=wss[i], stream=s)

        def call_gate_up(i, s):
            r = reps[i]
            moe.moe_mxfp4_gate_up(d, xs[i], r.w13p, r.w13s, wss[i], w13_bias=r.b13, stream=s)

        def call_down(i, s):
            r = reps[i]
            down_fn(d, r.w2p, r.w2s, outs[i], wss[i], w2_bias=r.b2, stream=s)

        with torch.cuda.stream(stream):
            for i in range(L):
                call_decode(i, stream)
        stream.synchronize()
        plan_hdr = [wss[i][:8].view(torch.int32).cpu().tolist() for i in range(L)]
        touched = [h[0] for h in plan_hdr]
        routes = [h[1] for h in plan_hdr]

        def chain(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(L):
                    fn(i, stream)
            return g

        names = (("decode", call_decode), ("plan", call_plan), ("gate_up", call_gate_up), ("down", call_down))
        timing = {}
        for name, fn in (names if breakdown else names[:1]):
            g = chain(fn)
            med, lo, hi = time_graph(torch, g, stream, args.steps, args.warmup)
            timing[name] = (med / L, lo / L, hi / L)
            del g
        bytes_call = float(np.mean([touched[c] * per_expert + 2 * T * K + out_bytes + 4 * T * cfg.E_global
                                    for c in range(L)]))
        w13_bytes = float(np.mean([touched[c] * w13_per_expert + 2 * T * K + 2 * routes[c] * I for c in range(L)]))
        us = timing["decode"][0]
        res = dict(us_per_call=round(us, 2), us_min=round(timing["decode"][1], 2), us_max=round(timing["decode"][2], 2),
                   calls_per_s=round(1e6 / us, 1),
                   touched_experts=round(float(np.mean(touched)), 2), local_routes=round(float(np.mean(routes)), 2),
                   bytes_per_call=int(bytes_call), gbs=round(bytes_call / us / 1e3, 1),
                   pct_peak=round(100 * bytes_call / us / 1e3 / HBM_PEAK_GBS, 1))
        if breakdown:
            res.update(us_plan=round(timing["plan"][0], 2), us_gate_up=round(timing["gate_up"][0], 2),
                       us_down=round(timing["down"][0], 2), w13_bytes=int(w13_bytes),
                       w13_gbs=round(w13_bytes / timing["gate_up"][0] / 1e3, 1))
        results[T] = res
        log(f"{cfg.name} T={T}: {json.dumps(res)}")
        del wss, outs, xs, lg
        torch.cuda.synchronize()
    return results


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this layer slice runs on a single MI355X "
              f"(--gpus {args.gpus} is not supported: a G-GPU job runs this call on each GPU's slice of "
              f"E_global / G experts and sums the partial outputs with one all-reduce)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe > 0:
        # a plain copy of known size: the FETCH_SIZE / WRITE_SIZE counters of
        # its kernel calibrate the same counters of the layer kernels
        n = int(args.copy_probe * (1 << 20))
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 4}), flush=True)
        return

    import mxfp4_mixture_experts_router_amd as moe
    from workloads import get_config, make_weights

    if args.encode:
        print(json.dumps(encode_bench(torch, moe, get_config(args.config), args)), flush=True)
        return
    if args.prefill:
        print(json.dumps(prefill_bench(torch, moe, args)), flush=True)
        return

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    tokens = [int(t) for t in args.tokens.split(",")] if args.tokens else [t for t in cfg.tokens if t <= 32] or list(cfg.tokens)
    K, I = cfg.K, cfg.I
    L = replica_count(cfg, tokens, args.rotate_mb)
    log(f"config {cfg.name}: tokens {tokens}, chain of {L} calls over {L} replicas, "
        f"{args.steps} timed replays, warmup {args.warmup}")

    t0 = time.time()
    w0 = make_weights(cfg, replica=0)
    reps = make_replicas(torch, moe, cfg, L, args.layout, w0)
    log(f"weights ready ({L} x {cfg.E_local} experts) in {time.time() - t0:.1f}s")

    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    results = measure_config(torch, moe, cfg, tokens, args, reps)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall

    step_us = sum(r["us_per_call"] for r in results.values())
    step_bytes = sum(r["bytes_per_call"] for r in results.values())
    value = step_bytes / step_us / 1e3
    # dominant step: the gate/up projection, timed alone over the same chains;
    # one launch of the stream kernel per call at every T of the decode sweep
    w13_avg_us = float(np.mean([r["us_gate_up"] for r in results.values()]))
    w13_avg_bytes = float(np.mean([r["w13_bytes"] for r in results.values()]))
    achieved = w13_avg_bytes / w13_avg_us / 1e3
    line = {
        "metric": "MoE decode us/call and achieved HBM GB/s (% peak) at T=1..32 tokens",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us * L / 1000.0, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 MFMA on MXFP4 weights decoded in registers, fp32 accumulate",
        "data": "synthetic (seeded random E2M1 codes, E8M0 scales, Gaussian x and logits)",
        "config": {"workload": f"{cfg.description}; one call at each T in {tokens} per call chain",
                   "K": K, "I": I, "E_global": cfg.E_global, "E_local": cfg.E_local, "top_k": cfg.top_k,
                   "tokens": tokens, "chain_calls": L, "replicas": L, "timing": f"median of {args.steps} replays",
                   "weight_layout": args.layout, "w13_order": args.w13_order, "down_pairing": args.down_pairing,
                   "output": "per-route fp32 rows" if args.per_route else "token sums bf16",
                   "parallelism": "single GPU"},
        "pct_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "us_per_call_sum": round(step_us, 2),
        "timed_wall_s": round(wall_s, 2),
        "per_T": {str(k): v for k, v in results.items()},
        "roofline": {"kernel": "gate/up projection: moe::stream_kernel<true,*> (one launch per call)",
                     "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg, tokens, args.layout, args.w13_order),
                     "avg_launch_us": round(w13_avg_us, 2),
                     "algorithmic_bytes_per_launch": int(w13_avg_bytes)},
        "device": torch.cuda.get_device_name(0),
    }
    del reps
    torch.cuda.empty_cache()
    if not args.no_other_configs and args.config == HEADLINE and not args.tokens:
        other = {}
        for name in OTHER_CONFIGS:
            c = get_config(name)
            toks = list(c.tokens)
            Lc = replica_count(c, toks, args.rotate_mb)
            rc = make_replicas(torch, moe, c, Lc, args.layout)
            rr = measure_config(torch, moe, c, toks, args, rc, breakdown=False)
            sus = sum(r["us_per_call"] for r in rr.values())
            sb = sum(r["bytes_per_call"] for r in rr.values())
            other[name] = {"workload": c.description, "chain_calls": Lc, "gbs_sweep": round(sb / sus / 1e3, 1),
                           "pct_peak_sweep": round(100 * sb / sus / 1e3 / HBM_PEAK_GBS, 1),
                           "per_T": {str(k): {kk: v[kk] for kk in ("us_per_call", "touched_experts", "local_routes",
                                                                  "bytes_per_call", "gbs", "pct_peak")}
                                     for k, v in rr.items()}}
            del rc
            torch.cuda.empty_cache()
        line["other_configs"] = other
    if not args.no_cpu_baseline and not args.per_route and args.w13_order == "gate_up":
        line["cpu_baseline"] = cpu_baseline(cfg, w0, torch, moe, args.layout)
    print(json.dumps(line), flush=True)


def encode_bench(torch, moe, cfg, args):
    """MXFP4 encoder throughput: the layer's w13 as bf16 [E, 2I, K] -> packed +
    scales, Quark rule; bytes = bf16 in + packed + scales out."""
    E, K, I = cfg.E_local, cfg.K, cfg.I
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 * cfg.index + 7)
    x = (torch.randn((E, 2 * I, K), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    packed = torch.empty((E, 2 * I, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, 2 * I, K // 32), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            moe.moe_mxfp4_encode(x, packed, scales, stream=stream)
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            moe.moe_mxfp4_encode(x, packed, scales, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / args.steps
    nbytes = x.numel() * 2 + packed.numel() + scales.numel()
    gbs = nbytes / us / 1e3
    return {"metric": "MXFP4 encode GB/s (bf16 in + packed/scales out)", "value": round(gbs, 1), "unit": "GB/s",
            "us_per_call": round(us, 2), "bytes_per_call": int(nbytes), "steps": args.steps,
            "config": {"workload": f"w13 of the {cfg.name} layer as bf16 [{E}, {2 * I}, {K}], Quark rule"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def prefill_bench(torch, moe, args):
    """The prefill path against the decode path: the same calls (replica-rotating
    chains, HIP events on the launch stream), the same algorithmic bytes (packed
    weights, scales and biases of the touched experts, x, logits, out)."""
    from workloads import get_config, make_inputs
    cfg = get_config("widek" if args.config == "gptoss20b" else args.config)
    tokens = [int(t) for t in args.tokens.split(",")] if args.tokens else [t for t in cfg.tokens if t > 64] or [256]
    K, I = cfg.K, cfg.I
    per_expert = cfg.bytes_per_expert()
    t_min = min(tokens)
    exp_touched = cfg.E_local * (1 - (1 - cfg.top_k / cfg.E_global) ** t_min)
    L = min(max(2, math.ceil(args.rotate_mb * 1e6 / max(1.0, exp_touched * per_expert))), args.steps)
    reps = [Replica(torch, cfg, i) for i in range(L)]
    if args.layout == "tile16":
        for r in reps:
            moe.moe_mxfp4_tile_weights(r.w13p)
            moe.moe_mxfp4_tile_weights(r.w2p)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    per_t = {}
    for T in tokens:
        d = moe.make_desc(T=T, K=K, I=I, E_global=cfg.E_global, E_local=cfg.E_local, top_k=cfg.top_k,
                          expert_offset=cfg.expert_offset, scoring=cfg.scoring, activation=cfg.activation,
                          swiglu_alpha=cfg.swiglu_alpha, swiglu_limit=cfg.swiglu_limit, weight_layout=args.layout)
        inputs = [make_inputs(cfg, T, call=i) for i in range(L)]
        xs = [torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16) for inp in inputs]
        lg = [torch.from_numpy(inp.logits).cuda() for inp in inputs]
        nb = moe.moe_mxfp4_prefill_workspace_bytes(d)
        wss = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(L)]
        outs = [torch.empty((T, K), dtype=torch.bfloat16, device="cuda") for _ in range(L)]

        def call(fn):
            def f(i, s):
                r = reps[i % L]
                fn(d, xs[i % L], r.w13p, r.w13s, r.w2p, r.w2s, outs[i % L], router_logits=lg[i % L],
                   w13_bias=r.b13, w2_bias=r.b2, workspace=wss[i % L], stream=s)
            return f

        timing = {}
        for name, fn in (("decode", moe.moe_mxfp4_decode), ("prefill", moe.moe_mxfp4_prefill)):
            f = call(fn)
            with torch.cuda.stream(stream):
                for i in range(L):
                    f(i, stream)
            stream.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(args.steps):
                    f(i, stream)
            with torch.cuda.stream(stream):
                for _ in range(args.warmup):
                    g.replay()
                stream.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            timing[name] = e0.elapsed_time(e1) * 1000.0 / args.steps
            del g
        touched = [int(wss[i][:4].view(torch.int32).item()) for i in range(L)]
        calls = [i % L for i in range(args.steps)]
        bytes_call = float(np.mean([touched[c] * per_expert + 4 * T * K + 4 * T * cfg.E_global for c in calls]))
        unpacked = float(np.mean([touched[c] * 3 * I * K * 2 for c in calls]))
        per_t[str(T)] = dict(touched_experts=round(float(np.mean([touched[c] for c in calls])), 2),
                             bytes_per_call=int(bytes_call), unpacked_bf16_bytes=int(unpacked),
                             us_decode=round(timing["decode"], 2), us_prefill=round(timing["prefill"], 2),
                             gbs_decode=round(bytes_call / timing["decode"] / 1e3, 1),
                             gbs_prefill=round(bytes_call / timing["prefill"] / 1e3, 1))
        log(f"T={T}: {json.dumps(per_t[str(T)])}")
        del wss, outs
        torch.cuda.synchronize()
    us_p = sum(v["us_prefill"] for v in per_t.values())
    us_d = sum(v["us_decode"] for v in per_t.values())
    nbytes = sum(v["bytes_per_call"] for v in per_t.values())
    return {"metric": "MoE prefill-path us/call and GB/s of touched-expert packed bytes (vs the decode path)",
            "value": round(nbytes / us_p / 1e3, 1), "unit": "GB/s", "decode_path_gbs": round(nbytes / us_d / 1e3, 1),
            "steps": args.steps, "warmup": args.warmup,
            "config": {"workload": f"{cfg.description}; one call at each T in {tokens}", "replicas": L,
                       "weight_layout": args.layout},
            "per_T": per_t}


# sources of the gate/up stream kernel: counters taken with other sources are stale
TRAFFIC_SOURCES = ("mxfp4_mixture_experts_router_amd/csrc/stream_kernel.hip",
                   "mxfp4_mixture_experts_router_amd/csrc/kernels.h",
                   "mxfp4_mixture_experts_router_amd/csrc/device_common.h")


def source_hashes():
    out = {}
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            out[os.path.basename(rel)] = hashlib.sha256(f.read()).hexdigest()
    return out


def measured_traffic(cfg, tokens, layout, w13_order="gate_up"):
    """HBM bytes per gate/up launch (mean over T) from the committed counter runs
    (profiles/roofline_traffic.json), or None when they do not cover this
    workload or the kernel's sources have changed since they were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "roofline_traffic.json")) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return None
    if prof.get("sources_sha256") != source_hashes():
        return None
    per_t = prof.get("traffic_bytes_per_launch", {})
    if (prof.get("workload") != cfg.name or layout != "tile16" or w13_order != "gate_up"
            or any(str(t) not in per_t for t in tokens)):
        return None
    return int(np.mean([per_t[str(t)] for t in tokens]))


def cpu_baseline(cfg, w0, torch, moe, layout, tokens=(1, 4, 8)):
    """The CPU oracle, as it stands, on a bounded sample of the headline
    workload: one call at each T in `tokens` (replica 0's weights), timed with
    BLAS on 1 thread and on every core of the process's affinity set.  The
    split into dequantisation (numpy, one thread either way) and the rest
    (matmuls, activation, combine) comes from timing the oracle's dequantise
    of the sample's touched experts on their own."""
    import oracle
    from workloads import make_inputs
    from threadpoolctl import threadpool_limits

    n_all = len(os.sched_getaffinity(0))
    calls = [make_inputs(cfg, T, call=0) for T in tokens]
    runs, refs = {}, {}
    for n in (1, n_all):
        total_s = 0.0
        with threadpool_limits(limits=n):
            for T, inp in zip(tokens, calls):
                t0 = time.perf_counter()
                refs[T] = oracle.moe_forward_cfg(cfg, w0, inp)
                total_s += time.perf_counter() - t0
        runs[n] = total_s
    touched = {T: [int(e) for e in np.flatnonzero(refs[T]["counts"] > 0)] for T in tokens}
    n_touched = sum(len(v) for v in touched.values())
    total_bytes = sum(len(touched[T]) * cfg.bytes_per_expert() + 4 * T * cfg.K + 4 * T * cfg.E_global
                      for T in tokens)
    # dequantisation of the sample's touched experts, timed alone
    t0 = time.perf_counter()
    for T in tokens:
        for e in touched[T]:
            oracle.dequantize(w0.w13_packed[e], w0.w13_scales[e])
            oracle.dequantize(w0.w2_packed[e], w0.w2_scales[e])
    deq_s = time.perf_counter() - t0
    checks = {}
    for T, inp in zip(tokens, calls):
        # the same call on the device (the benchmark's layout), compared with the oracle
        g = Replica(torch, cfg, 0, w0)
        if layout == "tile16":
            moe.moe_mxfp4_tile_weights(g.w13p)
            moe.moe_mxfp4_tile_weights(g.w2p)
        d = moe.make_desc(T=T, K=cfg.K, I=cfg.I, E_global=cfg.E_global, E_local=cfg.E_local, top_k=cfg.top_k,
                          expert_offset=cfg.expert_offset, scoring=cfg.scoring, activation=cfg.activation,
                          swiglu_alpha=cfg.swiglu_alpha, swiglu_limit=cfg.swiglu_limit, weight_layout=layout)
        out = torch.empty((T, cfg.K), dtype=torch.bfloat16, device="cuda")
        moe.moe_mxfp4_decode(d, torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16), g.w13p,
                             g.w13s, g.w2p, g.w2s, out, router_logits=torch.from_numpy(inp.logits).cuda(),
                             w13_bias=g.b13, w2_bias=g.b2)
        torch.cuda.synchronize()
        y = (out.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        checks[str(T)] = {"rel_l2": float(f"{oracle.rel_l2(y, refs[T]['y']):.3e}"),
                          "cosine": float(f"{oracle.cosine(y, refs[T]['y']):.7f}")}
        del g

    def leg(n):
        return {"gbs": round(total_bytes / runs[n] / 1e9, 4), "us_per_call": round(runs[n] / len(tokens) * 1e6, 1),
                "seconds": round(runs[n], 2), "threads": n,
                "dequantise_s": round(deq_s, 2), "matmul_and_rest_s": round(max(0.0, runs[n] - deq_s), 2)}

    return {"value": round(total_bytes / runs[n_all] / 1e9, 4), "unit": "GB/s", "cores": n_all, "kind": "oracle",
            "us_per_call": round(runs[n_all] / len(tokens) * 1e6, 1),
            "sample": f"numpy oracle (fp32: full dequantise of the touched experts, then BLAS matmuls), one call "
                      f"at each T in {list(tokens)} of the {cfg.name} workload (replica 0), {n_touched} touched "
                      f"experts; timed with BLAS on {n_all} threads (value) and on 1 thread",
            "all_cores": leg(n_all), "single_thread": leg(1),
            "parity_vs_gpu": checks}


if __name__ == "__main__":
    main()
