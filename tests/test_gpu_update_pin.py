"""The bf16 parameter update of dmuon_step, pinned element by element.

Muon's update with decoupled weight decay (gist.science technical summary,
sections 1 and 5: DMuon keeps the update rule; reading: W <- W (1 - lr wd) -
lr s(rows, cols) O) is applied inside the kernels that produce O: the update
epilogue of the final product (grouped buckets, exact and ragged tiles, 16-bit
and fp32 MFMA operands), the fused small-matrix kernel, and the elementwise
output kernel of standard-form buckets and of zero-step calls.  A tolerance on
the whole matrix cannot see the decay term of a bf16 parameter: the rounding
of W to bf16 is as large as lr wd W at the usual hyper-parameters.

So O is taken from the GPU itself.  A first step with W = 0, lr = 1 and no
decay stores bf16(-s O) (the fused arithmetic is then c1 O alone); a second
step from the same momentum and gradient, hence the same O, applies the real
update.  On the host, W (1 - lr wd) - lr O16 (O16 = s O as stored by the
first step) must match every element of the second step's parameter within
one bf16 ulp of the result, plus lr times half an ulp of O16 (the first
step's own rounding of O).

Magnitudes: W ~ N(0, 1), lr = 0.5, wd = 0.2.  The decay term lr wd W = 0.1 W
is 13 to 26 ulps of W (a bf16 ulp is 2^-8 .. 2^-7 of |W|), and the update
term lr s O (|O| about 0.03 .. 0.1 at these shapes) is several ulps as well:
a kernel that drops or alters either term fails on almost every element.
"""

import numpy as np
import pytest

import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

LR, WD, MU = 0.5, 0.2, 0.95


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()


def ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def pinned_update(shapes, plan_kw, steps=5):
    import torch
    rng = np.random.default_rng(9001 + len(shapes) + steps)
    W = [synth.gaussian(rng, s, 1.0, "bf16") for s in shapes]
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    B = [rng.standard_normal(s, dtype=np.float32) * np.float32(0.01) for s in shapes]
    tg = [to_dev(g, "bf16") for g in G]
    with dm.Plan(shapes, **plan_kw) as plan:
        # O from the GPU: W = 0, lr = 1, no decay
        t0 = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
        plan.step(t0, tg, [to_dev(b, "f32") for b in B], lr=1.0, weight_decay=0.0, mu=MU, steps=steps)
        # the real update from the same momentum and gradient
        tw = [to_dev(w, "bf16") for w in W]
        plan.step(tw, tg, [to_dev(b, "f32") for b in B], lr=LR, weight_decay=WD, mu=MU, steps=steps)
        desc = plan.describe()
    torch.cuda.synchronize()
    worst = 0.0
    for i, s in enumerate(shapes):
        O16 = -to_host(t0[i])
        got = to_host(tw[i])
        want = W[i].astype(np.float64) * (1.0 - LR * WD) - LR * O16
        tol = ulp_bf16(want) + LR * 0.5 * ulp_bf16(O16)
        err = np.abs(got - want)
        bad = int(np.count_nonzero(err > tol))
        worst = max(worst, float(np.max(err / tol)))
        assert bad == 0, (s, bad, float(np.max(err / tol)))
        # the update term itself is visible: several ulps on average (with
        # zero steps O is the normalised momentum, whose entries are tiny)
        if steps > 0:
            assert np.mean(LR * np.abs(O16) / ulp_bf16(W[i])) > 2.0, s
    print(f"{plan_kw or 'default'} steps={steps}: worst error {worst:.2f} of the bound; "
          f"buckets {[(b['m'], b['fp32'], b['form'], b['fused']) for b in desc['recurrence']]}", flush=True)
    return desc


def test_grouped_fused_and_fp32_buckets():
    # wide and tall exact tiles (update epilogue, lower storage), ragged tiles
    # (element-wise update path), wide small members (fused kernel) and small
    # near-square members (fp32 MFMA operands, bf16 parameters)
    shapes = [(256, 768), (768, 256), (300, 700), (700, 300), (128, 512), (100, 300), (96, 96), (64, 120)]
    desc = pinned_update(shapes, {})
    rec = {b["m"]: b for b in desc["recurrence"]}
    assert rec[128]["fused"] and rec[100]["fused"]
    assert rec[96]["fp32"] and rec[64]["fp32"]
    assert rec[256]["storage"] == "lower"


def test_standard_form_bucket():
    # the standard form writes the update with the elementwise output kernel
    desc = pinned_update([(256, 256), (300, 500), (500, 300)], {"form": "standard"})
    assert all(b["form"] == "standard" for b in desc["recurrence"])


def test_zero_steps():
    # T = 0: the update of the normalised momentum, elementwise output kernel
    pinned_update([(256, 768), (300, 200)], {}, steps=0)
