"""Benchmark of the decode-time MoE layer on one MI355X.

One step = one forward of the whole layer (router + top-k + bucketing, routed
gate/up + SiLU*up, shared expert, down projection + combine + residual) for
one batch of synthetic tokens.  The timed forwards are recorded into one
captured HIP graph of consecutive layer steps (the way a serving engine
captures a decode step) and replayed; the per-call rate of the library's own
per-forward graph is reported beside it.  Inputs are resident in HBM before
the timed region.

Workload (headline): the TP8-shard layer (H 7168, E 384, top-8 sigmoid,
I = Is = 256) at batch 1.  A sweep at batch 16 and 64 is reported beside it,
speculative-decoding verify batches (requests of 8 tokens whose activations
correlate, so they share experts) at 8 and 64 tokens, and a batch of 64 with
Zipf(1.1)-skewed routing (a per-expert logit bias on the same layers).
Each step uses the next of L independently drawn layers (and the next of R
activation batches), as consecutive layers of a decode step do, so weights
stream from HBM instead of the 256 MB Infinity Cache.

Reported: tokens/s (B / step time), layer us, achieved HBM GB/s on the unique
weight bytes the step touches vs the 8 TB/s peak, a roofline entry for the
dominant kernel (routed gate/up) measured with HIP events around each launch
in a pass of eager launches over the same steps,
and the fp64 CPU oracle timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0

# HBM traffic of the gate/up launch at batch 1 (routed gate/up + the shared
# expert's gate/up rows) from rocprofv3 counters (FETCH_SIZE x 2.0 and
# WRITE_SIZE x 1.0, the scales a 2 GiB device copy gives those counters); taken
# on the kernel sources with these SHA-1s and reported only while the sources
# are unchanged (profiles/gateup_select_tp8shard_b1_hbm_traffic.md).
GATEUP_TRAFFIC = {"fetch_kib": 32422.2, "write_kib": 72.3, "fetch_scale": 2.0, "write_scale": 1.0,
                  "sources": {"moe_device.h": "a68d097bde31ec7214ddf8816a5abe073a9e7b21",
                              "moe_kernels.hip": "ff46f62c0612b5eb8ccfc2cf7ca06981c81a258c"}}


def gateup_traffic_bytes():
    """Counter-measured HBM bytes per launch of the routed gate/up kernel, or
    None when its sources changed since the counters were taken."""
    import hashlib
    csrc = os.path.join(ROOT, "mixture_experts_layer_29_amd", "csrc")
    for name, digest in GATEUP_TRAFFIC["sources"].items():
        with open(os.path.join(csrc, name), "rb") as fh:
            if hashlib.sha1(fh.read()).hexdigest() != digest:
                return None
    t = GATEUP_TRAFFIC
    return 1024.0 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])
METRIC = "MoE decode layer µs & tokens/s at batch 1/16/64; achieved HBM GB/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--layers", type=int, default=16, help="independent layers rotated per step")
    ap.add_argument("--batches", type=int, default=16, help="activation batches rotated per step")
    ap.add_argument("--capture", type=int, default=64, help="layer steps per captured graph")
    ap.add_argument("--sweep", type=str, default="16,64", help="extra batch sizes ('' = none)")
    ap.add_argument("--spec", type=str, default="8,64",
                    help="speculative-verify batch sizes, requests of 8 correlated tokens ('' = none)")
    ap.add_argument("--zipf", type=str, default="64",
                    help="batch sizes with Zipf(1.1)-skewed routing (a per-expert logit bias) ('' = none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-only", action="store_true",
                    help="only the device copy of a 2 GiB buffer (calibrates HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def weight_bytes(wl, n_unique: int) -> int:
    """Unique routed-expert + shared-expert weight bytes of one step."""
    return 2 * 3 * wl.hidden * (wl.inter * n_unique + wl.shared_inter)


def run_batch(moe, torch, synthetic, wl, layers, batch, steps, warmup, n_x, capture_len, spec=False, bias=None):
    """Times `steps` layer forwards at `batch` tokens.

    Headline: forwards recorded into one captured graph of `capture_len`
    consecutive layer steps (as a serving engine captures a decode step) and
    replayed.  Also reported: one library call per forward (its own graph).
    Then a pass reading back each step's |U|, and a pass with per-kernel HIP
    events (eager launches)."""
    cfg = moe.make_config(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, batch,
                          wl.score_fn, 1, 1.0, 1, bias)
    plan = moe.Plan(cfg)
    info = plan.info()
    if spec:  # speculative-decoding verify batches: requests of 8 correlated tokens
        xs = [synthetic.bits_to_torch_bf16(synthetic.spec_batch_x(wl, batch, offset=4096 + i * batch), "cuda")
              for i in range(n_x)]
    else:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(1234 + batch)
        xs = [torch.randn(batch, wl.hidden, generator=gen, device="cuda").to(torch.bfloat16)
              for _ in range(n_x)]
    outs = [torch.empty_like(xs[0]) for _ in range(n_x)]
    nu = torch.zeros(max(steps, capture_len), dtype=torch.int32, device="cuda")
    L = len(layers)

    def step(i, record=None):
        ly = layers[i % L]
        plan.forward(xs[i % n_x], ly["router_w"], ly["expert_w"], ly["shared_w"], outs[i % n_x])
        if record is not None:
            plan.routing(None, None, nu[record:record + 1], None)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # one library call (one graph launch) per forward
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    per_call_s = (time.perf_counter() - t0) / steps

    # captured: capture_len forwards in one graph, replayed
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(capture_len):
            step(i)
    reps = max(1, steps // capture_len)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    captured_s = (time.perf_counter() - t0) / (reps * capture_len)
    del g

    # unique experts of each step of the same sequence
    for i in range(capture_len):
        step(i, record=i)
    torch.cuda.synchronize()
    n_unique = nu[:capture_len].cpu().numpy()

    # per-kernel durations: the same steps, eager launches bracketed by HIP events
    plan.set_profiling(True)
    for i in range(min(steps, 1024)):
        step(i)
    prof = plan.profile_read()
    plan.set_profiling(False)
    plan.destroy()

    layer_s = captured_s
    bytes_mean = float(sum(weight_bytes(wl, int(u)) for u in n_unique)) / len(n_unique)
    gu_ms, gu_n = prof["gateup_routed"]
    # the routed gate/up launch also streams the shared expert's gate/up rows
    # when the plan places them there (batch <= 4)
    sh_gu = 2 * 2 * wl.hidden * wl.shared_inter if info.shared_gateup_in == 2 else 0
    gu_bytes_mean = float(sum(2 * 2 * wl.hidden * wl.inter * int(u) + sh_gu for u in n_unique)) / len(n_unique)
    gu_avg_s = gu_ms * 1e-3 / gu_n
    return {
        "batch": batch,
        "variant": moe.VARIANT_NAMES[info.variant],
        "n_kernels": info.n_kernels,
        "layer_us": layer_s * 1e6,
        "layer_us_per_call": per_call_s * 1e6,
        "tokens_per_s": batch / layer_s,
        "unique_experts_mean": float(n_unique.mean()),
        "weight_bytes_mean": bytes_mean,
        "router_bytes": 2 * wl.n_experts * wl.hidden,
        "hbm_GBps": bytes_mean / layer_s / 1e9,
        "hbm_frac": bytes_mean / layer_s / 1e9 / HBM_PEAK_GBPS,
        "kernel_us": {k: (v[0] * 1e3 / v[1] if v[1] else 0.0) for k, v in prof.items()},
        "gateup_routed": {"avg_us": gu_avg_s * 1e6, "GBps": gu_bytes_mean / gu_avg_s / 1e9,
                          "bytes_per_launch": gu_bytes_mean, "with_shared_gateup": bool(sh_gu)},
    }


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


def cpu_baseline(torch, synthetic, wl, layer, budget_s: float) -> dict:
    """The fp64 oracle on the host cores, on a bounded sample of tokens of the
    same layer (the oracle parallelises over tokens, so a batch of independent
    tokens uses every core)."""
    import numpy as np

    import oracle

    shape = oracle.LayerShape(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, wl.score_fn)
    wr = synthetic.torch_bf16_to_bits(layer["router_w"])
    ew = layer["expert_w"]
    E, H, I = wl.n_experts, wl.hidden, wl.inter
    n13 = 2 * I * H
    s13 = synthetic.torch_bf16_to_bits(layer["shared_w"][:2 * wl.shared_inter * H]).reshape(-1, H)
    s2 = synthetic.torch_bf16_to_bits(layer["shared_w"][2 * wl.shared_inter * H:]).reshape(H, -1)
    threads = oracle.max_threads()

    def sample(ntok, seed):
        x = np.stack([synthetic.token_x(wl, 10000 + seed * 1000 + t) for t in range(ntok)])
        z = oracle.router_logits(shape, x, wr)
        idx, _ = oracle.select(shape, z)
        w13 = [None] * E
        w2 = [None] * E
        for e in np.unique(idx):          # stage the touched experts in host memory first
            e = int(e)
            w13[e] = synthetic.torch_bf16_to_bits(ew[e * n13:(e + 1) * n13]).reshape(2 * I, H)
            w2[e] = synthetic.torch_bf16_to_bits(ew[E * n13 + e * H * I:E * n13 + (e + 1) * H * I]).reshape(H, I)
        t0 = time.perf_counter()
        oracle.forward(shape, x, wr, w13, w2, s13, s2)
        return time.perf_counter() - t0

    ntok = max(threads, 8)
    dt = sample(ntok, 0)
    ntok2 = int(max(ntok, min(16384, ntok * budget_s / max(dt, 1e-3) * 0.8)))
    ntok2 = (ntok2 + threads - 1) // threads * threads
    dt2 = sample(ntok2, 1)
    return {"value": ntok2 / dt2, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d independent tokens of one TP8-shard layer (fp64 oracle, OpenMP over tokens, "
                      "touched experts staged in host RAM before timing), %.1f s" % (ntok2, dt2)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the layer would shard by tensor parallelism over the intermediate dimension; "
              "see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_layer_29_amd as moe
    import synthetic

    torch.cuda.set_device(0)
    if args.copy_only:
        print(json.dumps({"copy_GBps": copy_gbps(torch), "bytes_read_per_copy": 2 << 30,
                          "bytes_written_per_copy": 2 << 30}))
        return
    wl = synthetic.TP8
    log("drawing %d TP8-shard layers on the device" % args.layers)
    layers = [synthetic.device_layer(wl, "cuda", layer=i) for i in range(args.layers)]
    torch.cuda.synchronize()
    log("copy ceiling")
    cg = copy_gbps(torch)
    log("copy %.0f GB/s; timing batch 1" % cg)
    head = run_batch(moe, torch, synthetic, wl, layers, 1, args.steps, args.warmup, args.batches, args.capture)
    log("batch 1: %.2f us/layer captured (%.2f per call), %.0f GB/s, kernels %s" % (
        head["layer_us"], head["layer_us_per_call"], head["hbm_GBps"],
        {k: round(v, 2) for k, v in head["kernel_us"].items()}))
    sweep = {}
    for b in [int(s) for s in args.sweep.split(",") if s.strip()]:
        r = run_batch(moe, torch, synthetic, wl, layers, b, args.steps, args.warmup, args.batches, args.capture)
        log("batch %d: %.2f us/layer captured (%.2f per call), %.0f GB/s, kernels %s" % (
            b, r["layer_us"], r["layer_us_per_call"], r["hbm_GBps"],
            {k: round(v, 2) for k, v in r["kernel_us"].items()}))
        sweep[str(b)] = {k: r[k] for k in ("layer_us", "layer_us_per_call", "tokens_per_s", "hbm_GBps",
                                            "hbm_frac", "unique_experts_mean", "weight_bytes_mean",
                                            "variant", "n_kernels", "kernel_us")}
    for b in [int(s) for s in args.spec.split(",") if s.strip()]:
        r = run_batch(moe, torch, synthetic, wl, layers, b, args.steps, args.warmup, args.batches, args.capture,
                      spec=True)
        log("spec-verify batch %d (%d requests x 8): %.2f us/layer captured, |U| %.1f, %.0f GB/s" % (
            b, b // 8, r["layer_us"], r["unique_experts_mean"], r["hbm_GBps"]))
        sweep["spec%d" % b] = {k: r[k] for k in ("layer_us", "layer_us_per_call", "tokens_per_s", "hbm_GBps",
                                                 "hbm_frac", "unique_experts_mean", "weight_bytes_mean",
                                                 "variant", "n_kernels", "kernel_us")}
    zb = synthetic.zipf_bias(synthetic.TP8_ZIPF)
    zbias = torch.from_numpy(zb).cuda()
    for b in [int(s) for s in args.zipf.split(",") if s.strip()]:
        r = run_batch(moe, torch, synthetic, wl, layers, b, args.steps, args.warmup, args.batches, args.capture,
                      bias=zbias)
        log("zipf-skewed batch %d: %.2f us/layer captured, |U| %.1f, %.0f GB/s" % (
            b, r["layer_us"], r["unique_experts_mean"], r["hbm_GBps"]))
        sweep["zipf%d" % b] = {k: r[k] for k in ("layer_us", "layer_us_per_call", "tokens_per_s", "hbm_GBps",
                                                 "hbm_frac", "unique_experts_mean", "weight_bytes_mean",
                                                 "variant", "n_kernels", "kernel_us")}
    cpu = None
    if not args.no_cpu:
        log("cpu oracle baseline")
        cpu = cpu_baseline(torch, synthetic, wl, layers[0], args.cpu_seconds)
    gu = head["gateup_routed"]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["layer_us"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "TP8-shard MoE decode layer, batch 1", "timing": "%d layer steps per "
                   "captured graph, replayed" % args.capture, "hidden": wl.hidden,
                   "n_experts": wl.n_experts, "top_k": wl.top_k, "inter": wl.inter,
                   "shared_inter": wl.shared_inter, "batch": 1, "score": "sigmoid, renormalised",
                   "layers_rotated": args.layers, "activation_batches_rotated": args.batches},
        "layer_us": head["layer_us"],
        "layer_us_per_call": head["layer_us_per_call"],
        "hbm_GBps": head["hbm_GBps"],
        "hbm_frac": head["hbm_frac"],
        "weight_bytes_per_step": head["weight_bytes_mean"],
        "n_kernels": head["n_kernels"],
        "kernel_us": head["kernel_us"],
        "copy_GBps": cg,
        "roofline": {"kernel": "gateup_routed" + (" + shared gate/up" if gu["with_shared_gateup"] else ""),
                     "bound": "hbm", "achieved": gu["GBps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gu["GBps"] / HBM_PEAK_GBPS,
                     "traffic": gateup_traffic_bytes(), "avg_us": gu["avg_us"], "bytes_per_launch": gu["bytes_per_launch"]},
        "cpu_baseline": cpu,
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
