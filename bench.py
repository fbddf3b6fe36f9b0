"""Benchmark of the decode-time MoE layer on one MI355X.

One step = one forward of the whole layer (router + top-k + bucketing, routed
gate/up + SiLU*up, shared expert, down projection + combine + residual) for
one batch of synthetic tokens.  Inputs are resident in HBM before any timed
region.

Headline: the TP8-shard layer (H 7168, E 384, top-8 sigmoid, I = Is = 256)
at batch 1.  Beside it, one line per workload the layer is specified on:

* ``tp8_b{2,4,8,16,64}``  the same shape, uniform routing (router N(0, 0.02));
* ``unit_b{8,16}``        the same shape, router N(0, 1/sqrt(H)): logits ~N(0, 1);
* ``zipf_b64``            the same shape, Zipf(1.1)-skewed routing (a per-expert
                          logit bias);
* ``spec_b{8,64}``        speculative-decoding verify batches: requests of 8
                          tokens whose activations correlate;
* ``tiny_b1``             the tiny layer (H 256, E 8, top-2 softmax, I = Is =
                          128): launch-bound, latency only;
* ``full_b{1,16,32,64}``  the unsharded layer (I = Is = 2048, 34 GB of expert
                          weights), one layer, a 1 GiB cache flush before every
                          timed step.

TP8-shape protocol: each step uses the next of 16 independently drawn layers
(and the next of 16 activation batches), as consecutive layers of a decode
step do, so weights come from HBM rather than the 256 MB Infinity Cache.
``--steps`` consecutive layer steps are recorded into one captured HIP graph
(the way a serving engine captures a decode step); the graph is replayed
``--replays`` times, each replay bracketed by synchronisation and timed with
HIP events on the stream it runs on; median, p10 and p90 of the per-step time
over the replays are reported.  The per-call rate (one library call, i.e. one
replay of the library's own per-forward graph, per step) is reported beside.

Bytes: the unique routed-expert + shared-expert weight bytes of each step's
own routing (2 * 3 * H * (I * |U| + Is)); the router's 2 * E * H bytes are
reported separately and not counted.

The CPU leg (skipped with --no-cpu) times the fp64 oracle on the host cores on
a bounded sample of the headline workload, and checks a few tokens of each
line's first step against it (per-line parity fields).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE decode layer µs & tokens/s at batch 1/16/64; achieved HBM GB/s vs peak"

# HBM traffic of the batch-1 launches (rocprofv3 FETCH_SIZE x 2.0 and
# WRITE_SIZE x 1.0 KiB per dispatch, the scales a 2 GiB device copy gives
# those counters), taken on the kernel sources with these SHA-1s and reported
# only while the sources are unchanged (profiles/layer_tp8shard_b1_hbm_traffic.md).
B1_TRAFFIC = {"kernels": {"front": (6360.7, 32.0), "experts": (45048.4, 112.2)},
              "fetch_scale": 2.0, "write_scale": 1.0,
              "sources": {"moe_fused.hip": "63cc114628b5cd87c0444d2f05fc0923af09f53c",
                          "moe_kernels.hip": "2df34530ae8683fc4340f7e22dd489f802067ade",
                          "moe_device.h": "523d680edb4b8081205135604419b051734b918e",
                          "moe_args.h": "7395a498098c31441908d3175290314c83579203"}}

DEFAULT_LINES = ("tp8_b1_prefetch,tp8_b2,tp8_b4,tp8_b8,tp8_b16,tp8_b64,unit_b8,unit_b16,zipf_b64,spec_b8,spec_b64,"
                 "tiny_b1,full_b1,full_b16,full_b32,full_b64")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="layer steps per timed replay")
    ap.add_argument("--warmup", type=int, default=16, help="untimed layer steps before timing")
    ap.add_argument("--replays", type=int, default=7, help="timed replays per line (>= 5)")
    ap.add_argument("--layers", type=int, default=16, help="independent TP8-shape layers rotated per step")
    ap.add_argument("--batches", type=int, default=16, help="activation batches rotated per step")
    ap.add_argument("--lines", type=str, default=DEFAULT_LINES, help="lines beside the headline ('' = none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU leg (oracle baseline, parity fields)")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="target CPU time of the oracle baseline sample (the measured sample runs about 10-20 s)")
    ap.add_argument("--copy-only", action="store_true",
                    help="only the device copy of a 2 GiB buffer (calibrates HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def weight_bytes(wl, n_unique: int) -> int:
    """Unique routed-expert + shared-expert weight bytes of one step."""
    return 2 * 3 * wl.hidden * (wl.inter * n_unique + wl.shared_inter)


def pct(vals, q):
    import numpy as np
    return float(np.percentile(np.asarray(vals, dtype=np.float64), q))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


class Line:
    """One workload line: a plan, its layers and activation batches."""

    def __init__(self, name, wl, batch, layers, xs, bias=None, flush=False, latency_only=False, prefetch=False):
        self.name, self.wl, self.batch = name, wl, batch
        self.layers, self.xs, self.bias = layers, xs, bias
        self.flush, self.latency_only, self.prefetch = flush, latency_only, prefetch


def run_line(moe, torch, ln: Line, steps, warmup, replays, flush_buf=None) -> dict:
    wl, B = ln.wl, ln.batch
    cfg = moe.make_config(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, B,
                          wl.score_fn, 1, 1.0, 1, ln.bias)
    plan = moe.Plan(cfg)
    info = plan.info()
    L, X = len(ln.layers), len(ln.xs)
    outs = [torch.empty_like(x) for x in ln.xs]
    nu = torch.zeros(steps, dtype=torch.int32, device="cuda")

    def step(i, record=None):
        ly = ln.layers[i % L]
        if ln.prefetch:  # the next step's layer: its router and shared weights are prefetched
            nx = ln.layers[(i + 1) % L]
            plan.forward_prefetch(ln.xs[i % X], ly["router_w"], ly["expert_w"], ly["shared_w"], outs[i % X],
                                  nx["router_w"], nx["shared_w"])
        else:
            plan.forward(ln.xs[i % X], ly["router_w"], ly["expert_w"], ly["shared_w"], outs[i % X])
        if record is not None:
            plan.routing(None, None, nu[record:record + 1], None)

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # one library call (one replay of its per-forward graph) per step
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    per_call_us = (time.perf_counter() - t0) / steps * 1e6

    per_step_us = []
    if ln.flush:
        # one step per measurement, a cache flush (1 GiB written) before each
        for r in range(replays):
            for i in range(steps):
                flush_buf.fill_(float(i & 7))
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                step(i)
                b.record(stream)
                b.synchronize()
                per_step_us.append(a.elapsed_time(b) * 1e3)
        timing = "one forward per measurement, 1 GiB cache flush before each (HIP events)"
        timed_steps = replays * steps
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        for r in range(replays):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            per_step_us.append(a.elapsed_time(b) * 1e3 / steps)
        del g
        timing = "%d layer steps per captured graph, %d timed replays (HIP events)" % (steps, replays)
        timed_steps = replays * steps

    # unique experts of each step of the same sequence
    for i in range(steps):
        step(i, record=i)
    torch.cuda.synchronize()
    n_unique = nu.cpu().numpy()

    # per-kernel durations: the same steps, eager launches bracketed by HIP events
    plan.set_profiling(True)
    for i in range(min(steps, 1024)):
        if ln.flush:
            flush_buf.fill_(0.0)
        step(i)
    prof = plan.profile_read()
    plan.set_profiling(False)

    # the first step's inputs and results, for the CPU leg's parity check
    step(0)
    idx = torch.empty((B, wl.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((B, wl.top_k), dtype=torch.float32, device="cuda")
    plan.routing(idx, w, None, None)
    torch.cuda.synchronize()
    first = {"x": ln.xs[0].clone(), "out": outs[0].clone(), "idx": idx.cpu().numpy(), "w": w.cpu().numpy(),
             "layer": ln.layers[0]}
    plan.destroy()

    med = pct(per_step_us, 50)
    bytes_mean = float(sum(weight_bytes(wl, int(u)) for u in n_unique)) / len(n_unique)
    kernel_us = {k: (v[0] * 1e3 / v[1]) for k, v in prof.items() if v[1]}
    res = {
        "workload": ln.name,
        "prefetch_next_layer": ln.prefetch,
        "shape": {"hidden": wl.hidden, "n_experts": wl.n_experts, "top_k": wl.top_k, "inter": wl.inter,
                  "shared_inter": wl.shared_inter, "score": "softmax" if wl.score_fn == 0 else "sigmoid",
                  "router_std": wl.router_std, "zipf_s": wl.zipf_s if ln.bias is not None else None},
        "batch": B,
        "variant": moe.VARIANT_NAMES[info.variant],
        "n_kernels": info.n_kernels,
        "timing": timing,
        "timed_steps": timed_steps,
        "layer_us": med,
        "layer_us_p10": pct(per_step_us, 10),
        "layer_us_p90": pct(per_step_us, 90),
        "layer_us_per_call": per_call_us,
        "tokens_per_s": B / (med * 1e-6),
        "unique_experts_mean": float(n_unique.mean()),
        "unique_experts_range": [int(n_unique.min()), int(n_unique.max())],
        "weight_bytes_mean": bytes_mean,
        "router_bytes": 2 * wl.n_experts * wl.hidden,
        "activation_bytes": 2 * 2 * B * wl.hidden,
        "kernel_us": kernel_us,
        "_first": first,
        "_prof": prof,
        "_n_unique": n_unique,
        "_shared_gateup_in": info.shared_gateup_in,
    }
    if not ln.latency_only:
        res["hbm_GBps"] = bytes_mean / (med * 1e-6) / 1e9
        res["hbm_frac"] = res["hbm_GBps"] / HBM_PEAK_GBPS
    return res


def copy_gbps(torch) -> float:
    """Device-to-device copy rate of a 2 GiB buffer (read + write bytes)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 10
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del a, b
    return 2 * 2 * n / dt / 1e9


def b1_traffic_bytes(names):
    """Counter-measured HBM bytes per batch-1 step (summed over the layer's
    launches) and per launch of `names`, or None when the kernel sources
    changed since the counters were taken."""
    if B1_TRAFFIC is None:
        return None
    import hashlib
    csrc = os.path.join(ROOT, "mixture_experts_layer_29_amd", "csrc")
    for name, digest in B1_TRAFFIC["sources"].items():
        with open(os.path.join(csrc, name), "rb") as fh:
            if hashlib.sha1(fh.read()).hexdigest() != digest:
                return None
    per = {k: 1024.0 * (v[0] * B1_TRAFFIC["fetch_scale"] + v[1] * B1_TRAFFIC["write_scale"])
           for k, v in B1_TRAFFIC["kernels"].items()}
    return {"layer": sum(per.values()), "kernels": per}


# ------------------------------------------------------------------ CPU leg

def _host_layer_access(synthetic, wl, layer):
    """Host bf16 bits of what the oracle needs, copied from the device layer."""
    E, H, I, Is = wl.n_experts, wl.hidden, wl.inter, wl.shared_inter
    ew = layer["expert_w"]
    n13 = 2 * I * H
    wr = synthetic.torch_bf16_to_bits(layer["router_w"])
    if Is:
        s13 = synthetic.torch_bf16_to_bits(layer["shared_w"][:2 * Is * H]).reshape(2 * Is, H)
        s2 = synthetic.torch_bf16_to_bits(layer["shared_w"][2 * Is * H:]).reshape(H, Is)
    else:
        s13 = s2 = None

    def experts(ids):
        w13 = [None] * E
        w2 = [None] * E
        for e in ids:
            e = int(e)
            w13[e] = synthetic.torch_bf16_to_bits(ew[e * n13:(e + 1) * n13]).reshape(2 * I, H)
            w2[e] = synthetic.torch_bf16_to_bits(ew[E * n13 + e * H * I:E * n13 + (e + 1) * H * I]).reshape(H, I)
        return w13, w2
    return wr, s13, s2, experts


def cpu_leg(torch, synthetic, head_wl, head_layer, lines, budget_s):
    """The fp64 oracle: (1) timed on the host cores on a bounded sample of the
    headline workload (touched experts staged in host RAM before the timer);
    (2) the first step of every line checked on a few tokens."""
    import numpy as np

    import oracle
    from oracle import gap as gapmod

    def shape_of(wl):
        return oracle.LayerShape(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, wl.score_fn)

    threads = oracle.max_threads()
    shape = shape_of(head_wl)
    wr, s13, s2, experts = _host_layer_access(synthetic, head_wl, head_layer)

    def sample(ntok, seed):
        x = np.stack([synthetic.token_x(head_wl, 10000 + seed * 1000 + t) for t in range(ntok)])
        z = oracle.router_logits(shape, x, wr)
        idx, _ = oracle.select(shape, z)
        w13, w2 = experts(np.unique(idx))
        t0 = time.perf_counter()
        oracle.forward(shape, x, wr, w13, w2, s13, s2)
        return time.perf_counter() - t0

    ntok = max(threads, 8)
    dt = sample(ntok, 0)
    ntok2 = int(max(ntok, min(16384, ntok * budget_s / max(dt, 1e-3) * 0.8)))
    ntok2 = (ntok2 + threads - 1) // threads * threads
    dt2 = sample(ntok2, 1)
    base = {"value": ntok2 / dt2, "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle", "us_per_token": dt2 / ntok2 * 1e6,
            "sample": "%d independent tokens of one TP8-shard layer (fp64 oracle, OpenMP over tokens, "
                      "touched experts staged in host RAM before timing), %.1f s" % (ntok2, dt2)}

    # per-line parity on the first step's tokens
    parity = {}
    for name, r in lines.items():
        f = r["_first"]
        wl = r["wl"]
        sh = shape_of(wl)
        B = r["batch"]
        ntk = min(B, 8 if wl.inter <= 256 else 2)
        rows = np.unique(np.linspace(0, B - 1, ntk).round().astype(int))
        lw = f["layer"]
        wr_l, s13_l, s2_l, experts_l = _host_layer_access(synthetic, wl, lw)
        bias = None if r["_bias"] is None else r["_bias"].cpu().numpy()
        x = synthetic.torch_bf16_to_bits(f["x"])[rows]
        z = oracle.router_logits(sh, x, wr_l, bias)
        gaps = gapmod.kth_gaps(z, sh.top_k)
        idx_o, _ = oracle.select(sh, z)
        w13, w2 = experts_l(np.unique(idx_o))
        out64, idx_o, w_o = oracle.forward(sh, x, wr_l, w13, w2, s13_l, s2_l, bias)
        og = f["out"].float().cpu().double().numpy()[rows]
        ref = torch.from_numpy(out64).to(torch.bfloat16).to(torch.float64).numpy()
        err = np.abs(og - ref)
        rms = float(np.sqrt(np.mean(out64 ** 2)))
        idx_g = f["idx"][rows]
        w_g = f["w"][rows]
        exact = all(sorted(idx_g[t].tolist()) == sorted(idx_o[t].tolist()) for t in range(len(rows)))
        wdiff = 0.0
        if exact:
            for t in range(len(rows)):
                wg = dict(zip(idx_g[t].tolist(), w_g[t].tolist()))
                wdiff = max(wdiff, max(abs(wg[e] - wv) for e, wv in zip(idx_o[t].tolist(), w_o[t].tolist())))
        parity[name] = {"tokens": int(len(rows)), "idx_exact": bool(exact), "w_maxdiff": wdiff,
                        "mae": float(err.mean()),
                        "maxrel": float(np.max(err / np.maximum(np.abs(out64), 1e-2 * rms))),
                        "raw_mae": float(np.mean(np.abs(og - out64))), "min_kth_gap": float(gaps.min())}
    return base, parity


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the layer would shard by tensor parallelism over the intermediate dimension; "
              "see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.replays < 1 or args.steps < 1:
        print("--steps and --replays must be >= 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_layer_29_amd as moe
    import synthetic

    torch.cuda.set_device(0)
    if args.copy_only:
        print(json.dumps({"copy_GBps": copy_gbps(torch), "bytes_read_per_copy": 2 << 30,
                          "bytes_written_per_copy": 2 << 30}))
        return
    want = [s.strip() for s in args.lines.split(",") if s.strip()]
    wl = synthetic.TP8
    log("drawing %d TP8-shard layers on the device" % args.layers)
    layers = [synthetic.device_layer(wl, "cuda", layer=i) for i in range(args.layers)]
    torch.cuda.synchronize()
    log("copy ceiling")
    cg = copy_gbps(torch)
    log("copy %.0f GB/s (read + write bytes)" % cg)

    def xs_for(w, batch, spec=False):
        if spec:
            return [synthetic.bits_to_torch_bf16(synthetic.spec_batch_x(w, batch, offset=4096 + i * batch), "cuda")
                    for i in range(args.batches)]
        gen = torch.Generator(device="cuda")
        gen.manual_seed(1234 + batch)
        return [torch.randn(batch, w.hidden, generator=gen, device="cuda").to(torch.bfloat16)
                for _ in range(args.batches)]

    results = {}

    def run(ln, flush_buf=None):
        r = run_line(moe, torch, ln, args.steps, args.warmup, args.replays, flush_buf)
        r["wl"] = ln.wl
        r["_bias"] = ln.bias
        results[ln.name] = r
        log("%s: %.2f us/layer (p10 %.2f, p90 %.2f; %.2f per call), |U| %.1f, %s, kernels %s" % (
            ln.name, r["layer_us"], r["layer_us_p10"], r["layer_us_p90"], r["layer_us_per_call"],
            r["unique_experts_mean"],
            ("%.0f GB/s (%.1f %%)" % (r["hbm_GBps"], 100 * r["hbm_frac"])) if "hbm_GBps" in r else "latency only",
            {k: round(v, 2) for k, v in r["kernel_us"].items()}))
        return r

    # headline: batch 1 (plain forward)
    head = run(Line("tp8_b1", wl, 1, layers, xs_for(wl, 1)))
    for name in want:
        kind, b = name.rsplit("_b", 1)
        b, _, variant = b.partition("_")
        b = int(b)
        if kind == "tp8":
            # the *_prefetch line also prefetches the next step's router and
            # shared weights (moe_decode_forward_prefetch)
            run(Line(name, wl, b, layers, xs_for(wl, b), prefetch=variant == "prefetch"))
        elif kind == "spec":
            run(Line(name, wl, b, layers, xs_for(wl, b, spec=True)))
        elif kind == "zipf":
            zb = torch.from_numpy(synthetic.zipf_bias(synthetic.TP8_ZIPF)).cuda()
            run(Line(name, synthetic.TP8_ZIPF, b, layers, xs_for(wl, b), bias=zb))
    ulayers = None
    if any(n.startswith("unit_") for n in want):
        uw = synthetic.TP8_UNIT
        ulayers = [dict(ly, router_w=synthetic.device_router(uw, "cuda", layer=i)) for i, ly in enumerate(layers)]
        for name in want:
            if name.startswith("unit_"):
                b = int(name.rsplit("_b", 1)[1])
                run(Line(name, uw, b, ulayers, xs_for(uw, b)))
    if any(n.startswith("tiny_") for n in want):
        tw = synthetic.TINY
        pk = synthetic.pack_host_layer(synthetic.host_layer(tw))
        tl = {"router_w": synthetic.bits_to_torch_bf16(pk["router_w"], "cuda"),
              "expert_w": synthetic.bits_to_torch_bf16(pk["expert_w"], "cuda"),
              "shared_w": synthetic.bits_to_torch_bf16(pk["shared_w"], "cuda")}
        for name in want:
            if name.startswith("tiny_"):
                b = int(name.rsplit("_b", 1)[1])
                run(Line(name, tw, b, [tl], xs_for(tw, b), latency_only=True))
    full_names = [n for n in want if n.startswith("full_")]
    if full_names:
        # the TP8-shape layers are released first (the lines keep only their
        # first layer, for the CPU leg): one unsharded layer holds 34 GB of
        # expert weights
        layers = ulayers = None
        torch.cuda.empty_cache()
        fw = synthetic.FULL
        log("drawing one unsharded layer on the device")
        fl = synthetic.device_layer(fw, "cuda", layer=0)
        flush_buf = torch.empty(1 << 29, dtype=torch.float16, device="cuda")  # 1 GiB
        fsteps = max(4, min(args.steps, 16))
        for name in full_names:
            b = int(name.rsplit("_b", 1)[1])
            r = run_line(moe, torch, Line(name, fw, b, [fl], xs_for(fw, b), flush=True), fsteps,
                         max(2, min(args.warmup, 4)), 1, flush_buf)
            r["wl"] = fw
            r["_bias"] = None
            results[name] = r
            log("%s: %.1f us/layer (p10 %.1f, p90 %.1f), |U| %.1f, %.0f GB/s (%.1f %%), kernels %s" % (
                name, r["layer_us"], r["layer_us_p10"], r["layer_us_p90"], r["unique_experts_mean"],
                r["hbm_GBps"], 100 * r["hbm_frac"], {k: round(v, 1) for k, v in r["kernel_us"].items()}))
        del flush_buf

    cpu, parity = None, {}
    if not args.no_cpu:
        log("cpu leg: oracle baseline and per-line parity")
        head_layer = results["tp8_b1"]["_first"]["layer"]
        cpu, parity = cpu_leg(torch, synthetic, wl, head_layer, results, args.cpu_seconds)

    # dominant kernel of the headline: the launch with the most weight bytes
    prof = head["_prof"]
    nu1 = head["_n_unique"]
    kus = head["kernel_us"]
    dom = max(kus, key=kus.get)
    sh_gu = 2 * 2 * wl.hidden * wl.shared_inter
    dom_bytes = {  # algorithmic weight bytes per launch, by slot, at batch 1
        "gateup_routed": float(sum(2 * 2 * wl.hidden * wl.inter * int(u) for u in nu1)) / len(nu1)
        + (sh_gu if head["_shared_gateup_in"] == 2 else 0),
        "down_combine": float(sum(2 * wl.hidden * wl.inter * int(u) for u in nu1)) / len(nu1)
        + 2 * wl.hidden * wl.shared_inter,
        # batch 1, one launch after the router launch: routed gate/up and down
        # rows and the shared expert's down rows
        "experts": float(sum(2 * 3 * wl.hidden * wl.inter * int(u) for u in nu1)) / len(nu1)
        + 2 * wl.hidden * wl.shared_inter,
        "layer": head["weight_bytes_mean"],
    }.get(dom)
    traffic = b1_traffic_bytes(list(kus))
    dominant = {"kernel": dom, "avg_us": kus[dom], "launches": prof[dom][1], "bytes_per_launch": dom_bytes}
    if dom_bytes:
        dominant["achieved"] = dom_bytes / (kus[dom] * 1e-6) / 1e9
        dominant["frac"] = dominant["achieved"] / HBM_PEAK_GBPS
        dominant["traffic"] = None if traffic is None else traffic["kernels"].get(dom)

    sweep = {}
    for name, r in results.items():
        if name == "tp8_b1":
            continue
        sweep[name] = {k: v for k, v in r.items() if not k.startswith("_") and k != "wl"}
        if "hbm_GBps" in r and cg:
            sweep[name]["hbm_frac_of_copy"] = r["hbm_GBps"] / cg
        if name in parity:
            sweep[name]["parity"] = parity[name]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "replays": args.replays,
        "timed_steps_total": head["timed_steps"],
        "ms_per_step": head["layer_us"] / 1e3,
        "ms_per_step_p10": head["layer_us_p10"] / 1e3,
        "ms_per_step_p90": head["layer_us_p90"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "TP8-shard MoE decode layer, batch 1", "timing": head["timing"],
                   "hidden": wl.hidden, "n_experts": wl.n_experts, "top_k": wl.top_k, "inter": wl.inter,
                   "shared_inter": wl.shared_inter, "batch": 1, "score": "sigmoid, renormalised",
                   "layers_rotated": args.layers, "activation_batches_rotated": args.batches,
                   "seed": wl.seed},
        "layer_us": head["layer_us"],
        "layer_us_per_call": head["layer_us_per_call"],
        "hbm_GBps": head["hbm_GBps"],
        "hbm_frac": head["hbm_frac"],
        "weight_bytes_per_step": head["weight_bytes_mean"],
        "n_kernels": head["n_kernels"],
        "kernel_us": head["kernel_us"],
        "copy_GBps": cg,
        # the layer's unique-weight rate against the device copy's rate (read +
        # write bytes per second of a 2 GiB copy), a measured ceiling beside 8 TB/s
        "hbm_frac_of_copy": head["hbm_GBps"] / cg if cg else None,
        "roofline": {"scope": "whole layer: unique routed + shared expert weight bytes per step / step time",
                     "bound": "hbm", "achieved": head["hbm_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": head["hbm_frac"], "traffic": None if traffic is None else traffic["layer"],
                     "bytes_per_step": head["weight_bytes_mean"], "dominant_kernel": dominant},
        "cpu_baseline": cpu,
        "parity": parity.get("tp8_b1"),
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
