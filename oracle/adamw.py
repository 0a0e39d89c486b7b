"""Plain fp64 NumPy oracle of one AdamW step (the comparison optimizer).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages measure DMuon's cost against AdamW (gist.science/pt, technical
summary section 4: the per-step overhead over AdamW is about 2%), without
restating AdamW itself.  The plain reading is Adam with decoupled weight
decay, with bias-corrected moment estimates, element by element:

    m   <- beta1 m + (1 - beta1) g
    v   <- beta2 v + (1 - beta2) g^2
    m^  =  m / (1 - beta1^t)
    v^  =  v / (1 - beta2^t)
    W   <- W (1 - lr wd) - lr m^ / (sqrt(v^) + eps)

with t the 1-based step count.  The decay is applied to the weight as it
was before this step's update.  Parity status: pinned (closed forms for the
first step and for a constant gradient, the zero-gradient case, and
agreement with torch.optim.AdamW run in float64 on the CPU).
"""

from __future__ import annotations

import numpy as np


def adamw_step(W, G, m, v, *, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
               eps: float = 1e-8, weight_decay: float = 0.0):
    """One AdamW step of one tensor; returns (W_new, m_new, v_new) in fp64."""
    if step < 1:
        raise ValueError("step counts from 1")
    W = np.array(W, dtype=np.float64, copy=True)
    G = np.array(G, dtype=np.float64, copy=True)
    m = np.array(m, dtype=np.float64, copy=True)
    v = np.array(v, dtype=np.float64, copy=True)
    if not (W.shape == G.shape == m.shape == v.shape):
        raise ValueError("W, G, m and v must have the same shape")
    m_new = beta1 * m + (1.0 - beta1) * G
    v_new = beta2 * v + (1.0 - beta2) * G * G
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    W_new = W * (1.0 - lr * weight_decay) - lr * m_hat / (np.sqrt(v_hat) + eps)
    return W_new, m_new, v_new
