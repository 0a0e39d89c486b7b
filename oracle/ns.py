"""Plain fp64 NumPy oracle: Newton-Schulz orthogonalisation and the Muon step.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obviously
correct on purpose: one library matmul per algebraic product, no blocking, no
fusion, no symmetric shortcuts.

Readings taken where the source pages are silent (each is also listed in the
design notes of the repository):

* coefficients (a, b, c) and step count T are caller inputs; the quintic
  (3.4445, -4.7750, 2.0315) with T = 5 is the default workload;
* the input is normalised by its Frobenius norm plus eps = 1e-7 before the
  iteration;
* a matrix with more rows than columns is transposed first, so the Gram
  space is the smaller side, and transposed back at the end;
* the Gram recurrence starts from Q = I and multiplies Q by P on every step;
* the momentum is classic Nesterov with an undamped buffer; the update uses
  decoupled weight decay and the shape factor sqrt(max(1, rows / cols)).
"""

from __future__ import annotations

import math
from collections import OrderedDict

import numpy as np

DEFAULT_EPS = 1e-7
QUINTIC = (3.4445, -4.7750, 2.0315)


def _f64(M) -> np.ndarray:
    return np.array(M, dtype=np.float64, copy=True)


def orient(M):
    """Return (X, transposed) with X of shape (m, n), m <= n.

    The Gram iteration runs in the space of the smaller side (DMuon,
    gist.science/pt, technical summary section 2.2, bullet on the Gram-space
    recurrence: the cost falls from O(m^2 n) to O(m^3) when m < n).  A square
    matrix is not transposed.
    """
    X = _f64(M)
    if X.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    if X.shape[0] > X.shape[1]:
        return X.T.copy(), True
    return X, False


def frobenius_normalise(X, eps: float = DEFAULT_EPS):
    """X / (||X||_F + eps) and ||X||_F.

    The pages do not state the normalisation; dividing by the Frobenius norm
    bounds every singular value by 1, which the iteration needs to converge.
    """
    X = _f64(X)
    s = math.sqrt(float(np.sum(X * X)))
    return X / (s + eps), s


def standard_recurrence(X0, steps: int, a: float, b: float, c: float):
    """The plain Newton-Schulz map in the m x n space.

    Each step forms A = X X^T and replaces X by a X + (b A + c A^2) X.  This is
    the iteration the pages attribute to Muon (gist.science/pt, technical
    summary section 1: Newton-Schulz iterations applied to momentum-aggregated
    gradients, needing products such as X X^T on the whole matrix).
    """
    X = _f64(X0)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def gram_recurrence(X0, steps: int, a: float, b: float, c: float):
    """The same map carried out in the m x m Gram space.

    DMuon, gist.science/pt (and gist.science/fr), technical summary section 2.2:
    the iteration is run on G = X X^T instead of on X.  Written out:

        A <- X0 X0^T,  Q <- I
        repeat T times:   P <- a I + b A + c A^2
                          A <- P A P
                          Q <- P Q
        result = Q X0

    Every X_k equals Q_k X0 and every A_k equals X_k X_k^T, so this equals the
    standard map exactly in exact arithmetic.
    """
    X0 = _f64(X0)
    m = X0.shape[0]
    I = np.eye(m)
    A = X0 @ X0.T
    Q = I.copy()
    for _ in range(steps):
        P = a * I + b * A + c * (A @ A)
        A = P @ A @ P
        Q = P @ Q
    return Q @ X0


def _ns(M, steps, coeffs, eps, recurrence):
    if steps < 0:
        raise ValueError("steps must be >= 0")
    a, b, c = coeffs
    X, transposed = orient(M)
    if X.size == 0:
        raise ValueError("empty matrix")
    X0, _ = frobenius_normalise(X, eps)
    out = recurrence(X0, steps, a, b, c)
    return out.T.copy() if transposed else out


def ns_standard(M, steps: int = 5, coeffs=QUINTIC, eps: float = DEFAULT_EPS):
    """Orient, normalise, run the standard map, orient back."""
    return _ns(M, steps, coeffs, eps, standard_recurrence)


def ns_gram(M, steps: int = 5, coeffs=QUINTIC, eps: float = DEFAULT_EPS):
    """Orient, normalise, run the Gram-space map, orient back."""
    return _ns(M, steps, coeffs, eps, gram_recurrence)


def shape_scale(rows: int, cols: int, mode: str = "sqrt_ratio") -> float:
    """Per-matrix factor applied to the orthogonalised update.

    The pages leave it open; the reading used here is sqrt(max(1, rows/cols))
    on the caller's (rows, cols), with a "none" mode that returns 1.
    """
    if mode == "none":
        return 1.0
    if mode != "sqrt_ratio":
        raise ValueError(mode)
    return math.sqrt(max(1.0, rows / cols))


def muon_step(W, G, buf, *, lr: float, weight_decay: float, mu: float,
              nesterov: bool = True, steps: int = 5, coeffs=QUINTIC,
              eps: float = DEFAULT_EPS, scale_mode: str = "sqrt_ratio"):
    """One Muon update of one weight matrix; returns (W_new, buf_new, O).

    The pages say Muon applies Newton-Schulz to momentum-aggregated gradients
    and that DMuon leaves the update rule unchanged (gist.science/pt, technical
    summary sections 1 and 5).  The form taken here:

        buf <- mu buf + G
        U   <- G + mu buf      (Nesterov)   or   U <- buf
        O   <- NS_T(U)         (Gram form, Frobenius-normalised)
        W   <- W (1 - lr wd) - lr s(rows, cols) O
    """
    W = _f64(W)
    G = _f64(G)
    buf = _f64(buf)
    if W.shape != G.shape or W.shape != buf.shape:
        raise ValueError("W, G and buf must have the same shape")
    buf_new = mu * buf + G
    U = G + mu * buf_new if nesterov else buf_new
    O = ns_gram(U, steps=steps, coeffs=coeffs, eps=eps)
    s = shape_scale(W.shape[0], W.shape[1], scale_mode)
    W_new = W * (1.0 - lr * weight_decay) - lr * s * O
    return W_new, buf_new, O


def plan_buckets(shapes):
    """Group matrices by shape the way the planner must.

    DMuon, gist.science/pt, technical summary section 2.2 (batching bullet):
    matrices of like shape are run through the Gram recurrence together.
    Reading: the Gram product and the final product are grouped by the
    caller's exact (rows, cols) -- a matrix with more rows than columns is
    processed transposed, which changes how its operand is read and its shape
    factor, so it cannot share those launches with its transpose -- while the
    m x m recurrence is grouped by the short side m alone.  Buckets keep
    first-appearance order and list member indices in input order.

    Returns {"gemm": [((rows, cols), [idx...]), ...],
             "recurrence": [(m, [idx...]), ...]}.
    """
    gemm: "OrderedDict[tuple, list]" = OrderedDict()
    rec: "OrderedDict[int, list]" = OrderedDict()
    for i, (r, c) in enumerate(shapes):
        r, c = int(r), int(c)
        if r <= 0 or c <= 0:
            raise ValueError("shapes must be positive")
        gemm.setdefault((r, c), []).append(i)
        rec.setdefault(min(r, c), []).append(i)
    return {"gemm": list(gemm.items()), "recurrence": list(rec.items())}
