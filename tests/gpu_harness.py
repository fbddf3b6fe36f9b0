"""Shared helpers for the GPU parity tests: run the HIP layer through the
C-ABI binding and the CPU oracle on the same seeded inputs, and compare.

Comparison rules (the layer's output is bf16; the oracle's is fp64):
* selected expert index SETS must be identical per token (inputs are drawn
  with an fp64 logit gap >= 1e-3 at rank k, far above fp32 rounding, so the
  selection does not depend on precision; the order inside the top-k is not
  compared because only the k-th gap is guaranteed);
* routing weights, matched by expert id: |w_gpu - w_oracle| <= 1e-4;
* out vs ref = bf16_rne(out64):  MAE = mean|out - ref| <= 1e-3 and
  max_i |out_i - ref_i| / max(|out64_i|, 1e-2 * rms(out64)) <= 2e-2.
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_layer_29_amd as moe
import oracle
import synthetic
from oracle import gap as gapmod

W_TOL = 1e-4
MAE_TOL = 1e-3
REL_TOL = 2e-2


def shape_of(wl: synthetic.Workload, **over) -> oracle.LayerShape:
    s = oracle.LayerShape(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, wl.score_fn)
    for k, v in over.items():
        setattr(s, k, v)
    return s


class DeviceLayer:
    """A layer's weights on the GPU plus host access to what the oracle needs."""

    def __init__(self, wl: synthetic.Workload, host: bool | None = None, layer: int = 0):
        self.wl = wl
        E, H, I, Is = wl.n_experts, wl.hidden, wl.inter, wl.shared_inter
        small = E * 3 * I * H <= (64 << 20) if host is None else host
        if small:
            hd = synthetic.host_layer(wl)
            pk = synthetic.pack_host_layer(hd)
            self.router_w = synthetic.bits_to_torch_bf16(pk["router_w"], "cuda")
            self.expert_w = synthetic.bits_to_torch_bf16(pk["expert_w"], "cuda")
            self.shared_w = synthetic.bits_to_torch_bf16(pk["shared_w"], "cuda")
            self.bias = None if pk["bias"] is None else torch.from_numpy(pk["bias"]).cuda()
        else:
            d = synthetic.device_layer(wl, "cuda", layer)
            self.router_w, self.expert_w, self.shared_w, self.bias = (
                d["router_w"], d["expert_w"], d["shared_w"], d["bias"])
        self.wr_bits = synthetic.torch_bf16_to_bits(self.router_w)
        self.bias_np = None if self.bias is None else self.bias.cpu().numpy()
        self._cache13, self._cache2 = {}, {}
        self._s = None

    def clear_cache(self):
        """Drops the host copies of expert weights (bounds host memory when a
        test walks many experts of a large layer)."""
        self._cache13.clear()
        self._cache2.clear()

    def expert_bits(self, e: int):
        wl = self.wl
        E, H, I = wl.n_experts, wl.hidden, wl.inter
        if e not in self._cache13:
            n13 = 2 * I * H
            self._cache13[e] = synthetic.torch_bf16_to_bits(
                self.expert_w[e * n13:(e + 1) * n13]).reshape(2 * I, H)
            off2 = E * n13
            self._cache2[e] = synthetic.torch_bf16_to_bits(
                self.expert_w[off2 + e * H * I: off2 + (e + 1) * H * I]).reshape(H, I)
        return self._cache13[e], self._cache2[e]

    def shared_bits(self):
        wl = self.wl
        H, Is = wl.hidden, wl.shared_inter
        if Is == 0:
            return None, None
        if self._s is None:
            sb = synthetic.torch_bf16_to_bits(self.shared_w)
            self._s = (sb[:2 * Is * H].reshape(2 * Is, H), sb[2 * Is * H:].reshape(H, Is))
        return self._s


def gap_x(layer: DeviceLayer, shape: oracle.LayerShape, batch: int, offset: int = 0):
    """Seeded activations for `batch` tokens with the top-k gap enforced."""
    wl = layer.wl
    x = synthetic.batch_x(wl, batch, offset)
    x, n = gapmod.enforce_gap(shape, x, layer.wr_bits, layer.bias_np,
                              lambda t, r: synthetic.token_x(wl, offset + t, r))
    return x, n


def gap_spec_x(layer: DeviceLayer, shape: oracle.LayerShape, batch: int, offset: int = 0):
    """Seeded speculative-verify activations (correlated within a request) for
    `batch` tokens, the top-k gap enforced by redrawing a token's own part."""
    wl = layer.wl
    x = synthetic.spec_batch_x(wl, batch, offset)
    x, n = gapmod.enforce_gap(shape, x, layer.wr_bits, layer.bias_np,
                              lambda t, r: synthetic.spec_token_x(wl, offset + t, r))
    return x, n


def run_oracle(layer: DeviceLayer, shape: oracle.LayerShape, x_bits: np.ndarray):
    z = oracle.router_logits(shape, x_bits, layer.wr_bits, layer.bias_np)
    idx, _ = oracle.select(shape, z)
    E = shape.n_experts
    w13 = [None] * E
    w2 = [None] * E
    for e in np.unique(idx):
        w13[e], w2[e] = layer.expert_bits(int(e))
    s13, s2 = layer.shared_bits()
    return oracle.forward(shape, x_bits, layer.wr_bits, w13, w2, s13, s2, layer.bias_np)


def make_plan(layer: DeviceLayer, shape: oracle.LayerShape, batch: int, **kw) -> moe.Plan:
    cfg = moe.make_config(shape.hidden, shape.n_experts, shape.top_k, shape.inter, shape.shared_inter,
                          batch, shape.score_fn, shape.renormalize, shape.routed_scale,
                          shape.add_residual, layer.bias, **kw)
    return moe.Plan(cfg)


def run_gpu(plan: moe.Plan, layer: DeviceLayer, x_bits: np.ndarray, shape):
    B = x_bits.shape[0]
    x = synthetic.bits_to_torch_bf16(x_bits, "cuda")
    out = torch.empty_like(x)
    plan.forward(x, layer.router_w, layer.expert_w, layer.shared_w, out)
    idx = torch.empty((B, shape.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((B, shape.top_k), dtype=torch.float32, device="cuda")
    nu = torch.empty(1, dtype=torch.int32, device="cuda")
    plan.routing(idx, w, nu)
    torch.cuda.synchronize()
    return out, idx.cpu().numpy(), w.cpu().numpy(), int(nu.item())


def bf16_round(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()


def compare_out(out_gpu: torch.Tensor, out64, label=""):
    """The output rule alone (for replays where the routing accessor only
    holds the last forward's routing)."""
    og = out_gpu.float().cpu().double().numpy()
    ref = bf16_round(out64)
    err = np.abs(og - ref)
    mae = float(err.mean())
    rms = float(np.sqrt(np.mean(out64 ** 2)))
    rel = float(np.max(err / np.maximum(np.abs(out64), 1e-2 * rms)))
    assert np.all(np.isfinite(og)), label + ": non-finite output"
    assert mae <= MAE_TOL, "%s: MAE %.3g > %g" % (label, mae, MAE_TOL)
    assert rel <= REL_TOL, "%s: max rel %.3g > %g" % (label, rel, REL_TOL)
    return {"mae": mae, "maxrel": rel}


def compare(out_gpu: torch.Tensor, idx_g, w_g, out64, idx_o, w_o, label=""):
    B = out64.shape[0]
    for t in range(B):
        assert sorted(idx_g[t].tolist()) == sorted(idx_o[t].tolist()), \
            "%s token %d: expert sets differ gpu=%s oracle=%s" % (label, t, idx_g[t], idx_o[t])
        wg = dict(zip(idx_g[t].tolist(), w_g[t].tolist()))
        for e, wv in zip(idx_o[t].tolist(), w_o[t].tolist()):
            assert abs(wg[e] - wv) <= W_TOL, "%s token %d expert %d: w %g vs %g" % (label, t, e, wg[e], wv)
    og = out_gpu.float().cpu().double().numpy()
    ref = bf16_round(out64)
    err = np.abs(og - ref)
    mae = float(err.mean())
    rms = float(np.sqrt(np.mean(out64 ** 2)))
    rel = float(np.max(err / np.maximum(np.abs(out64), 1e-2 * rms)))
    assert np.all(np.isfinite(og)), label + ": non-finite output"
    assert mae <= MAE_TOL, "%s: MAE %.3g > %g" % (label, mae, MAE_TOL)
    assert rel <= REL_TOL, "%s: max rel %.3g > %g" % (label, rel, REL_TOL)
    return {"mae": mae, "maxrel": rel, "raw_mae": float(np.mean(np.abs(og - out64)))}
