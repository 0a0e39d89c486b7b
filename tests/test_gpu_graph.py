"""Capture of library calls in a HIP graph (torch.cuda.CUDAGraph).

A captured fused step or NS call must replay exactly what the eager call
does: the library enqueues only kernels on the caller's stream (no memset
nodes, no allocation or synchronisation once the workspace exists).  Each
replay is compared bitwise with the eager run of the same step, with eager
work and synchronisations of the program between replays.
"""

import numpy as np
import pytest

import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()


@pytest.mark.parametrize("shapes", [
    [(512, 1024), (1024, 512), (256, 768), (384, 384)],
    # small wide members: the fused one-launch kernel plus the momentum pass
    [(128, 512), (128, 512), (64, 256), (100, 300)],
])
def test_captured_step_replays_the_eager_step(shapes):
    import torch
    rng = np.random.default_rng(701)
    W = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    B = [rng.standard_normal(s, dtype=np.float32) * np.float32(0.01) for s in shapes]
    kw = dict(lr=0.02, weight_decay=0.1, mu=0.95)
    eager = [[to_dev(w, "bf16") for w in W], [to_dev(g, "bf16") for g in G], [to_dev(b, "f32") for b in B]]
    graph = [[to_dev(w, "bf16") for w in W], [to_dev(g, "bf16") for g in G], [to_dev(b, "f32") for b in B]]
    with dm.Plan(shapes) as plan:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):      # warm-up outside the capture
            plan.step(*eager, **kw)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        # the graph copy starts one step behind: catch it up eagerly
        plan.step(*graph, **kw)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.step(*graph, **kw)
        torch.cuda.synchronize()
        # capture did not run the step: both copies are still equal
        for a, b in zip(eager[0] + eager[2], graph[0] + graph[2]):
            assert torch.equal(a, b)
        for it in range(4):
            gen = torch.Generator(device="cuda").manual_seed(17 + it)
            for ge, gg in zip(eager[1], graph[1]):      # new gradients, same in both
                noise = torch.randn(ge.shape, device="cuda", generator=gen).to(torch.bfloat16) * 0.01
                ge.copy_(noise)
                gg.copy_(noise)
            torch.cuda.synchronize()
            plan.step(*eager, **kw)
            g.replay()
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(zip(eager[0], graph[0])):
                assert torch.equal(a, b), (it, i)
            for i, (a, b) in enumerate(zip(eager[2], graph[2])):
                assert torch.equal(a, b), (it, i)


@pytest.mark.parametrize("shape", [(768, 1280), (128, 512)])
def test_captured_ns_batched_replays_the_eager_call(shape):
    import torch
    rng = np.random.default_rng(709)
    inputs = [[synth.gaussian(rng, shape, 0.02, "bf16") for _ in range(3)] for _ in range(3)]
    work = [to_dev(x, "bf16") for x in inputs[0]]
    dm.ns_batched([w.clone() for w in work])           # grows the cached workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dm.ns_batched(work)
    torch.cuda.synchronize()
    for it in range(3):
        for w, x in zip(work, inputs[it]):
            w.copy_(to_dev(x, "bf16"))
        ref = [w.clone() for w in work]
        dm.ns_batched(ref)                              # eager, between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, work)):
            assert torch.equal(a, b), (it, i)
