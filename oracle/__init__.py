"""fp64 CPU oracle for batched Gram Newton-Schulz and the fused Muon step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers or constant tables).

Every function here is written in plain NumPy float64, following the steps in
the order the source pages give them, without blocking, fusion or reordering.
The source pages are three web summaries of one paper, "DMuon: Efficient
Distributed Muon Training with Near-Adam Overhead":

* gist.science/pt  -- Portuguese summary; its "Resumo Tecnico" (technical
  summary) has sections 1 Problem, 2 Method (2.1 owner-centric execution,
  2.2 Gram Newton-Schulz iteration, 2.3 load balancing, 2.4 autotuning),
  3 Contributions, 4 Results, 5 Significance.
* gist.science/fr  -- French translation of the same technical summary.
* shd-paper.top    -- Chinese summary page that also carries the authors'
  original English abstract.

Citations below name the page and the section.

Parity status of each function (pins live in ``tests/test_oracle.py``):

* ``ns_standard``   pinned (SVD closed form, diagonal closed form, cubic
                    polar limit via scipy, identity coefficients).
* ``ns_gram``       pinned (same pins, plus agreement with ``ns_standard``).
* ``muon_step``     pinned (diagonal closed forms for momentum, Nesterov,
                    weight decay and the shape scale; zero-gradient case).
* ``plan_buckets``  pinned (hand-derived bucket counts for the workloads).
* ``adamw_step``    pinned (first-step and constant-gradient closed forms,
                    zero gradient, agreement with torch.optim.AdamW in
                    float64 on the CPU).
* ``owners``        pinned (two independent exact solvers agree -- exhaustive
                    enumeration and the integer program via scipy's MILP --
                    plus hand-solved instances and the cost-curve definition).
"""

from .ns import (  # noqa: F401
    DEFAULT_EPS,
    QUINTIC,
    frobenius_normalise,
    orient,
    gram_recurrence,
    ns_gram,
    ns_standard,
    standard_recurrence,
    muon_step,
    shape_scale,
    plan_buckets,
)

from .adamw import adamw_step  # noqa: F401,E402
from . import owners  # noqa: F401,E402
