"""Checks that tie the CPU oracle to things other than itself.

Each ``check_*`` takes an ``oracle.Oracle`` (the default build, or a
deliberately mutated copy) and raises AssertionError on a mismatch.  The
references used here are: hand-computed closed forms (tests/golden), an
exhaustive k-subset search, a dense all-experts NumPy formulation
(oracle.brute), torch's float64 SwiGLU FFN, NumPy's float64 matmul, and
invariants of the layer (weights sum to one, expert permutation, identical
experts, token independence, zero experts, linearity in the output
projections).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import brute
from synthetic import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def bits(a) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def rnd_layer(rng, H, E, k, I, Is, B, std=0.3, with_bias=False):
    d = {
        "x": bits(rng.standard_normal((B, H))),
        "wr": bits(rng.standard_normal((E, H)) * std),
        "w13": bits(rng.standard_normal((E, 2 * I, H)) * std),
        "w2": bits(rng.standard_normal((E, H, I)) * std),
        "s13": bits(rng.standard_normal((2 * Is, H)) * std) if Is else None,
        "s2": bits(rng.standard_normal((H, Is)) * std) if Is else None,
        "bias": (rng.standard_normal(E) * 0.5).astype(np.float32) if with_bias else None,
    }
    return d


def run(orc, shape, d):
    return orc.forward(shape, d["x"], d["wr"], d["w13"], d["w2"], d["s13"], d["s2"], d["bias"])


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------------ checks

def check_hand_examples(orc):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        shape = oracle.LayerShape(c["hidden"], c["n_experts"], c["top_k"], c["inter"],
                                  c["shared_inter"], c["score_fn"], c["renormalize"], 1.0,
                                  c["add_residual"])
        d = {"x": bits(c["x"]), "wr": bits(c["wr"]), "w13": bits(c["w13"]), "w2": bits(c["w2"]),
             "s13": bits(c["s13"]) if "s13" in c else None,
             "s2": bits(c["s2"]) if "s2" in c else None, "bias": None}
        out, idx, w = run(orc, shape, d)
        assert idx.tolist() == c["expect_idx"], (c["name"], idx)
        assert np.allclose(w, c["expect_w"], rtol=1e-14, atol=1e-15), (c["name"], w)
        assert np.allclose(out, c["expect_out"], rtol=1e-14, atol=1e-15), (c["name"], out)


def check_router_logits(orc):
    rng = np.random.default_rng(11)
    for (B, E, H, bias) in [(3, 5, 16, False), (2, 7, 24, True), (1, 384, 64, True)]:
        x = bits(rng.standard_normal((B, H)))
        wr = bits(rng.standard_normal((E, H)))
        b = (rng.standard_normal(E)).astype(np.float32) if bias else None
        shape = oracle.LayerShape(H, E, 1, 8, 0)
        z = orc.router_logits(shape, x, wr, b)
        ref = brute.bf16_bits_to_f64(x) @ brute.bf16_bits_to_f64(wr).T
        if b is not None:
            ref = ref + b.astype(np.float64)[None, :]
        assert rel_err(z, ref) < 1e-13, "router logits"


def check_selection_brute(orc):
    rng = np.random.default_rng(12)
    for trial in range(300):
        E = int(rng.integers(2, 11))
        k = int(rng.integers(1, min(E, 4) + 1))
        if trial % 3 == 0:                       # exact ties at every rank
            z = rng.integers(-3, 4, size=(1, E)).astype(np.float64)
        else:
            z = rng.standard_normal((1, E))
        shape = oracle.LayerShape(8, E, k, 8, 0, score_fn=int(trial % 2))
        idx, _ = orc.select(shape, z)
        sub = brute.best_subset(z[0], k)
        assert sorted(idx[0].tolist()) == list(sub), ("subset", z, idx, sub)
        # rank order: logits descending, equal logits by ascending index
        keys = [(-z[0, e], e) for e in idx[0]]
        assert keys == sorted(keys), ("order", z, idx)


def check_weights(orc):
    rng = np.random.default_rng(13)
    for trial in range(200):
        E = int(rng.integers(2, 12))
        k = int(rng.integers(1, E + 1))
        z = rng.standard_normal((1, E)) * 3
        for score in (0, 1):
            shape = oracle.LayerShape(8, E, k, 8, 0, score_fn=score, renormalize=1)
            idx, w = orc.select(shape, z)
            assert abs(w.sum() - 1.0) < 1e-14 and np.all(w > 0) and np.all(w <= 1.0), "sum to one"
            # the selected order is by logit, and both scores are monotone
            assert np.all(np.diff(w[0]) <= 1e-15), "weights follow the rank order"
            D = brute.dense_weights(z, k, score, 1)
            assert np.allclose(w[0], D[0, idx[0]], rtol=1e-13, atol=0), "dense weights"
            shape0 = oracle.LayerShape(8, E, k, 8, 0, score_fn=score, renormalize=0,
                                       routed_scale=0.75)
            _, w0 = orc.select(shape0, z)
            D0 = brute.dense_weights(z, k, score, 0, 0.75)
            assert np.allclose(w0[0], D0[0, idx[0]], rtol=1e-13, atol=0), "unnormalised weights"
    # closed forms
    shape = oracle.LayerShape(8, 3, 2, 8, 0, score_fn=0)
    _, w = orc.select(shape, np.array([[0.3, -1.0, 1.1]]))
    d = 1.1 - 0.3
    assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(-d))) < 1e-15, "softmax of two"
    shape = oracle.LayerShape(8, 3, 2, 8, 0, score_fn=1)
    _, w = orc.select(shape, np.array([[0.0, -1.0, math.log(3.0)]]))
    # sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2 -> weights 0.6, 0.4
    assert np.allclose(w[0], [0.6, 0.4], rtol=0, atol=1e-15), "sigmoid ratio"


def check_dense_swiglu(orc):
    """E = 1, k = 1, no shared expert, no residual: the layer is one SwiGLU FFN."""
    rng = np.random.default_rng(14)
    for (H, I, B) in [(16, 8, 3), (40, 24, 2), (64, 128, 1)]:
        d = rnd_layer(rng, H, 1, 1, I, 0, B)
        shape = oracle.LayerShape(H, 1, 1, I, 0, score_fn=1, add_residual=0)
        out, idx, w = run(orc, shape, d)
        X = torch.from_numpy(brute.bf16_bits_to_f64(d["x"]))
        W13 = torch.from_numpy(brute.bf16_bits_to_f64(d["w13"][0]))
        W2 = torch.from_numpy(brute.bf16_bits_to_f64(d["w2"][0]))
        ffn = (torch.nn.functional.silu(X @ W13[:I].T) * (X @ W13[I:].T)) @ W2.T
        assert np.all(idx == 0) and np.allclose(w, 1.0), "single expert routing"
        assert rel_err(out, ffn.numpy()) < 1e-12, "dense SwiGLU"
        y = orc.swiglu(d["w13"][0], d["w2"][0], d["x"])
        assert rel_err(y, ffn.numpy()) < 1e-12, "oracle_swiglu"


def check_brute_dense(orc):
    rng = np.random.default_rng(15)
    cases = [
        # H, E, k, I, Is, B, score, renorm, scale, resid, bias
        (16, 4, 1, 8, 0, 3, 1, 1, 1.0, 0, False),
        (16, 6, 2, 8, 8, 2, 0, 1, 1.0, 1, False),
        (24, 8, 2, 16, 16, 4, 0, 1, 1.0, 1, True),
        (32, 10, 3, 8, 16, 3, 1, 1, 1.0, 1, True),
        (16, 7, 3, 8, 8, 2, 1, 0, 2.5, 1, False),
        (16, 5, 2, 24, 0, 2, 0, 0, 0.5, 0, True),
    ]
    for (H, E, k, I, Is, B, score, ren, scale, res, bias) in cases:
        d = rnd_layer(rng, H, E, k, I, Is, B, with_bias=bias)
        shape = oracle.LayerShape(H, E, k, I, Is, score, ren, scale, res)
        out, idx, w = run(orc, shape, d)
        ref, D, _ = brute.layer(d["x"], d["wr"], d["w13"], d["w2"], d["s13"], d["s2"], d["bias"],
                                k=k, score_fn=score, renormalize=ren, routed_scale=scale,
                                add_residual=res)
        assert rel_err(out, ref) < 1e-12, ("dense formulation", (H, E, k, I, Is, B))
        for t in range(B):
            assert sorted(idx[t].tolist()) == sorted(np.nonzero(D[t])[0].tolist()), "selected set"


def check_tiny_workload(orc):
    """The tiny specified shape (H 256, E 8, top-2 softmax, I = Is = 128) against
    the dense formulation, for a few tokens."""
    import synthetic
    wl = synthetic.TINY
    d = synthetic.host_layer(wl)
    x = synthetic.batch_x(wl, 4)
    shape = oracle.LayerShape(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter,
                              wl.score_fn)
    out, idx, w = orc.forward(shape, x, d["wr"], d["w13"], d["w2"], d["s13"], d["s2"], None)
    ref, D, _ = brute.layer(x, d["wr"], d["w13"], d["w2"], d["s13"], d["s2"], None,
                            k=wl.top_k, score_fn=wl.score_fn)
    assert rel_err(out, ref) < 1e-12, "tiny workload vs dense formulation"


def check_permutation(orc):
    rng = np.random.default_rng(16)
    H, E, k, I, Is, B = 24, 9, 3, 8, 8, 4
    d = rnd_layer(rng, H, E, k, I, Is, B, with_bias=True)
    shape = oracle.LayerShape(H, E, k, I, Is, 1)
    out, idx, w = run(orc, shape, d)
    perm = rng.permutation(E)                    # new expert i is old expert perm[i]
    dp = dict(d, wr=d["wr"][perm], w13=d["w13"][perm], w2=d["w2"][perm], bias=d["bias"][perm])
    outp, idxp, wp = run(orc, shape, dp)
    assert rel_err(outp, out) < 1e-13, "permutation changes the output"
    for t in range(B):
        assert sorted(perm[idxp[t]].tolist()) == sorted(idx[t].tolist()), "selection maps"


def check_identical_experts(orc):
    rng = np.random.default_rng(17)
    H, E, k, I, B = 16, 6, 3, 8, 3
    d = rnd_layer(rng, H, E, k, I, 0, B)
    d["w13"] = np.repeat(d["w13"][:1], E, axis=0)
    d["w2"] = np.repeat(d["w2"][:1], E, axis=0)
    for score in (0, 1):
        shape = oracle.LayerShape(H, E, k, I, 0, score, 1, 1.0, 0)
        out, _, _ = run(orc, shape, d)
        y = orc.swiglu(d["w13"][0], d["w2"][0], d["x"])
        X = torch.from_numpy(brute.bf16_bits_to_f64(d["x"]))
        W13 = torch.from_numpy(brute.bf16_bits_to_f64(d["w13"][0]))
        W2 = torch.from_numpy(brute.bf16_bits_to_f64(d["w2"][0]))
        ffn = ((torch.nn.functional.silu(X @ W13[:I].T) * (X @ W13[I:].T)) @ W2.T).numpy()
        assert rel_err(out, ffn) < 1e-13 and rel_err(y, ffn) < 1e-12, "identical experts"


def check_token_independence(orc):
    rng = np.random.default_rng(18)
    H, E, k, I, Is, B = 16, 7, 2, 8, 8, 5
    d = rnd_layer(rng, H, E, k, I, Is, B, with_bias=True)
    shape = oracle.LayerShape(H, E, k, I, Is, 1)
    out, idx, w = run(orc, shape, d)
    for t in range(B):
        o1, i1, w1 = run(orc, shape, dict(d, x=d["x"][t:t + 1]))
        assert np.array_equal(o1[0], out[t]) and np.array_equal(i1[0], idx[t]), "token independence"


def check_zero_experts(orc):
    rng = np.random.default_rng(19)
    H, E, k, I, Is, B = 16, 5, 2, 8, 8, 3
    d = rnd_layer(rng, H, E, k, I, Is, B)
    d["w2"] = np.zeros_like(d["w2"])
    shape = oracle.LayerShape(H, E, k, I, Is, 0)
    out, _, _ = run(orc, shape, d)
    X = brute.bf16_bits_to_f64(d["x"])
    S13 = torch.from_numpy(brute.bf16_bits_to_f64(d["s13"]))
    S2 = torch.from_numpy(brute.bf16_bits_to_f64(d["s2"]))
    Xt = torch.from_numpy(X)
    sh = ((torch.nn.functional.silu(Xt @ S13[:Is].T) * (Xt @ S13[Is:].T)) @ S2.T).numpy()
    assert rel_err(out, X + sh) < 1e-13, "zero routed experts leave x + shared"


def check_linearity(orc):
    rng = np.random.default_rng(20)
    H, E, k, I, Is, B = 16, 6, 2, 8, 8, 3
    d = rnd_layer(rng, H, E, k, I, Is, B)
    shape = oracle.LayerShape(H, E, k, I, Is, 1)
    out, _, _ = run(orc, shape, d)
    two = lambda a: bits(brute.bf16_bits_to_f64(a) * 2.0)   # exact in bf16
    out2, _, _ = run(orc, shape, dict(d, w2=two(d["w2"]), s2=two(d["s2"])))
    X = brute.bf16_bits_to_f64(d["x"])
    assert rel_err(out2 - X, 2.0 * (out - X)) < 1e-13, "linearity in the output projections"


ALL_CHECKS = [check_hand_examples, check_router_logits, check_selection_brute, check_weights,
              check_dense_swiglu, check_brute_dense, check_tiny_workload, check_permutation,
              check_identical_experts, check_token_independence, check_zero_experts,
              check_linearity]
