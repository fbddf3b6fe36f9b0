"""The allocation-free forward (moe_decode_forward_noalloc) against the
ordinary forward, through the C-ABI: same routing, outputs within the parity
bar, on consecutive calls of different sizes that share the device's scratch
array; and its refusals."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_layer_29_amd as moe
import synthetic
from gpu_harness import DeviceLayer, compare, compare_out, gap_x, make_plan, run_oracle, shape_of

pytestmark = pytest.mark.gpu


def routing_of(plan, B, k):
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    w = torch.empty((B, k), dtype=torch.float32, device="cuda")
    nu = torch.empty(1, dtype=torch.int32, device="cuda")
    plan.routing(idx, w, nu)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), int(nu.item())


def both_forwards(layer, shape, batch, offset):
    """Ordinary forward, then the allocation-free one, on the same inputs."""
    x_bits, _ = gap_x(layer, shape, batch, offset)
    x = synthetic.bits_to_torch_bf16(x_bits, "cuda")
    plan = make_plan(layer, shape, batch)
    ref = torch.empty_like(x)
    plan.forward(x, layer.router_w, layer.expert_w, layer.shared_w, ref)
    idx_r, w_r, nu_r = routing_of(plan, batch, shape.top_k)
    out = torch.full_like(x, float("nan"))
    plan.forward_noalloc(x, layer.router_w, layer.expert_w, layer.shared_w, out)
    idx_n, w_n, nu_n = routing_of(plan, batch, shape.top_k)
    st = plan.stats()
    plan.destroy()
    return x_bits, ref, out, (idx_r, w_r, nu_r), (idx_n, w_n, nu_n), st


@pytest.fixture(scope="module")
def tp8():
    return DeviceLayer(synthetic.TP8)


@pytest.fixture(scope="module")
def tiny():
    return DeviceLayer(synthetic.TINY)


def test_noalloc_matches_forward_on_consecutive_sizes(tp8, tiny):
    # sizes falling, then rising again; batch 1 runs as one launch
    cases = [(tp8, 16, 0), (tp8, 2, 40), (tp8, 1, 60), (tiny, 8, 0), (tiny, 1, 20), (tp8, 16, 80), (tp8, 1, 90)]
    for layer, batch, offset in cases:
        shape = shape_of(layer.wl)
        label = "%s B=%d" % (layer.wl.name, batch)
        x_bits, ref, out, r_ref, r_na, st = both_forwards(layer, shape, batch, offset)
        assert st.error_flags == 0, label
        assert r_na[2] == r_ref[2] == st.n_unique, label
        for t in range(batch):
            assert sorted(r_na[0][t].tolist()) == sorted(r_ref[0][t].tolist()), "%s token %d" % (label, t)
            wr = dict(zip(r_ref[0][t].tolist(), r_ref[1][t].tolist()))
            for e, wv in zip(r_na[0][t].tolist(), r_na[1][t].tolist()):
                assert abs(wr[e] - wv) <= 1e-6, "%s token %d expert %d" % (label, t, e)
        # the ordinary forward's output as the reference, at the parity bar
        compare_out(out, ref.double().cpu().numpy(), label + " vs forward")
        # and both against the oracle
        out64, idx_o, w_o = run_oracle(layer, shape, x_bits)
        compare(out, r_na[0], r_na[1], out64, idx_o, w_o, label + " vs oracle")


def test_noalloc_refusals(tp8):
    shape = shape_of(synthetic.TP8)
    x = torch.zeros((4, shape.hidden), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    for kw in (dict(shared_stream=1), dict(single_launch=moe.SINGLE_REQUIRED)):
        plan = make_plan(tp8, shape, 4, **kw)
        with pytest.raises(moe.MoeError) as ei:
            plan.forward_noalloc(x, tp8.router_w, tp8.expert_w, tp8.shared_w, out)
        assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
        plan.destroy()
    # a plan whose workspace exceeds the scratch array (no weights are touched:
    # the call is refused before any launch)
    cfg = moe.make_config(16384, 1024, 16, 64, 64, 64)
    plan = moe.Plan(cfg)
    assert plan.info().workspace_bytes > 48 << 20
    st = moe.lib().moe_decode_forward_noalloc(plan.handle, 256, 256, 256, 256, 1 << 24, None)
    assert st == moe.MOE_ERR_UNSUPPORTED and "scratch" in moe.last_error()
    plan.destroy()
