"""dmuon_ns_batched_noalloc: the plan-free NS call in the library's static
device scratch, for callers that cannot allocate device memory.

It runs the same launch sequence as dmuon_ns_batched on the same host plan,
only in another workspace, so its results must equal that call's bitwise
(and hence meet the oracle's bf16 MFMA tolerance, checked here as well: the
Gram-space iteration of the gist.science technical summary, section 2.2).
Two calls in a row, the second on a smaller input, share the scratch.
"""

import numpy as np
import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import TOL_BF16_MFMA, rel, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()


def test_noalloc_equals_ns_batched_on_two_calls():
    import torch
    rng = np.random.default_rng(7301)
    for shape, count in [((384, 700), 3), ((200, 130), 2)]:   # second call smaller, and transposed
        mats = [synth.gaussian(rng, shape, 0.02, "bf16") for _ in range(count)]
        ref = [to_dev(m, "bf16") for m in mats]
        got = [to_dev(m, "bf16") for m in mats]
        dm.ns_batched(ref)
        dm.ns_batched_noalloc(got)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), (shape, i)
            e = rel(to_host(b), oracle.ns_gram(mats[i]))
            assert e <= TOL_BF16_MFMA, (shape, i, e)


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    import torch
    t = [torch.zeros((4096, 4096), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    t[0][0, 0] = 1.0
    before = t[0].clone()
    with pytest.raises(dm.DmuonError) as ei:
        dm.ns_batched_noalloc(t)
    assert ei.value.code == dm.ENOMEM and "allocation-free scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.equal(t[0], before)  # nothing enqueued
