"""Helpers shared by the GPU parity tests (not a test module)."""

import numpy as np

import oracle

TOL_BF16_MFMA = 2e-2   # relative Frobenius error, 16-bit MFMA operands
TOL_F32 = 1e-4         # relative Frobenius error, fp32 MFMA


def rel(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def to_dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def block_expect(M, rp, cp, rs, cs, steps=5, coeffs=oracle.QUINTIC, eps=oracle.DEFAULT_EPS):
    """Oracle result for a permuted block-diagonal input, block by block.

    NS acts on each block separately once the whole matrix is normalised, and
    commutes with row and column permutations, so the result is the permuted
    block-diagonal matrix of per-block recurrences with the global norm.
    Returns (expected, mask) in the permuted layout.
    """
    M = np.asarray(M, np.float64)
    nrm = float(np.sqrt(np.sum(M * M)))
    D = np.empty_like(M)
    D[rp[:, None], cp[None, :]] = M
    out = np.zeros_like(M)
    mask = np.zeros(M.shape, dtype=bool)
    for r, c in zip(rs, cs):
        B = D[r, c] / (nrm + eps)
        if B.shape[0] > B.shape[1]:
            out[r, c] = oracle.gram_recurrence(B.T, steps, *coeffs).T
        else:
            out[r, c] = oracle.gram_recurrence(B, steps, *coeffs)
        mask[r, c] = True
    return out[rp][:, cp], mask[rp][:, cp]
