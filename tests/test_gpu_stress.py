"""Hand-offs between workgroups under perturbed timing.

The layer hands data between workgroups of one launch (router logits to the
selection, split-K partials to SiLU*up, and at batch 1 everything from the
router to the down projection) through device-coherent stores and counters.
A mistake there -- data read before its counter says it is complete, or a
load the compiler moved above a wait -- can pass tests whose launches always
run with the same timing (the Kimi K3 decode article, Part 2 section 3,
reports such a compiler-hoisted load).  Here forwards run while another
stream (default priority) keeps HBM and the compute units busy with copies of
varying size, and the launches are delayed by spin kernels of varying length,
so the producers and consumers of every hand-off meet in changing orders.
Each output is checked against the oracle at the parity bar and, where the
path is deterministic, against an undisturbed forward bit for bit.  The test
stops at the first mismatch.
"""
import numpy as np
import pytest
import torch

import synthetic
from gpu_harness import DeviceLayer, compare_out, gap_x, make_plan, run_oracle, shape_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp8():
    return DeviceLayer(synthetic.TP8)


@pytest.mark.parametrize("B,deterministic", [(1, True), (2, True), (3, True), (8, False), (16, False), (64, False)])
def test_forwards_next_to_a_bandwidth_hog(tp8, B, deterministic):
    shape = shape_of(synthetic.TP8)
    plan = make_plan(tp8, shape, B)
    xs = [synthetic.bits_to_torch_bf16(gap_x(tp8, shape, B, offset=2000 + 100 * i)[0], "cuda") for i in range(3)]
    refs64 = [run_oracle(tp8, shape, synthetic.torch_bf16_to_bits(x))[0] for x in xs]
    quiet = []
    for x in xs:  # undisturbed outputs
        o = torch.empty_like(x)
        plan.forward(x, tp8.router_w, tp8.expert_w, tp8.shared_w, o)
        quiet.append(o)
    torch.cuda.synchronize()
    hog = torch.cuda.Stream()  # default priority
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    rng = np.random.default_rng(B)
    main = torch.cuda.current_stream()
    for it in range(30):
        i = it % len(xs)
        n = int(rng.choice([1 << 20, 16 << 20, 64 << 20, 256 << 20]))
        with torch.cuda.stream(hog):
            for _ in range(int(rng.integers(1, 4))):
                dst[:n].copy_(src[:n])
        spin = int(rng.choice([0, 1000, 20000, 200000]))
        if spin:
            torch.cuda._sleep(spin)
        out = torch.empty_like(xs[i])
        plan.forward(xs[i], tp8.router_w, tp8.expert_w, tp8.shared_w, out, stream=main)
        torch.cuda.synchronize()
        label = "B=%d iteration %d (copy %d B, spin %d)" % (B, it, n, spin)
        if deterministic:
            assert torch.equal(out.view(torch.int16), quiet[i].view(torch.int16)), label + ": differs from quiet run"
        compare_out(out, refs64[i], label)
    st = plan.stats()
    assert st.error_flags == 0, "device-side error flags %d" % st.error_flags
    plan.destroy()
