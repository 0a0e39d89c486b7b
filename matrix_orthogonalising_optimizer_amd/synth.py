"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds input generation only (random draws, bf16 rounding of the
draws, structured test matrices and the workload shape lists); none of the
orthogonalisation arithmetic lives here.

The source pages evaluate on trained production models (DMuon, gist.science/pt,
technical summary section 4: Wall-OSS-0.5, Pi0, Wall-WM, Qwen2.5-7B) whose
weights and data are not available, so Gaussian matrices in the same weight
shapes stand in for them.
"""

from __future__ import annotations

import numpy as np

# (rows, cols) lists in PyTorch (out_features, in_features) order.
LLAMA7B_LAYER = [(4096, 4096)] * 4 + [(11008, 4096), (11008, 4096), (4096, 11008)]
VLA_MIX = [(256, 256)] * 50 + [(1024, 1024)] * 50 + [(1024, 4096)] * 50 + [(2048, 8192)] * 50
MLP70B = [(8192, 28672)] * 8

WORKLOADS = {
    # name: (shapes, dtype, sigma, seed)
    "fp32_256x1024": ([(256, 1024)], "f32", 1.0, 1),
    "bf16_64x128x512": ([(128, 512)] * 64, "bf16", 0.02, 2),
    "llama7b_layer": (LLAMA7B_LAYER, "bf16", 0.02, 3),
    "vla_mix_200": (VLA_MIX, "bf16", 0.02, 4),
    "mlp70b_8x8192x28672": (MLP70B, "bf16", 0.02, 5),
}


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    # NaN stays NaN (not produced by the generators, kept for completeness)
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), x, out)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def gaussian(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    """float32 N(0, sigma^2) draw, rounded to bf16 when dtype == 'bf16'."""
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    return bf16_round(x) if dtype == "bf16" else x


def workload(name: str, count: int | None = None):
    """Matrices of a named workload, drawn in list order from its seed.

    Returns (list of float32 arrays holding the exact input values, dtype).
    ``count`` limits how many matrices are drawn (the first ``count``).
    """
    shapes, dtype, sigma, seed = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    shapes = shapes if count is None else shapes[:count]
    return [gaussian(rng, s, sigma, dtype) for s in shapes], dtype


def step_inputs(name: str):
    """Gradients and parameters of a named workload for the Muon step.

    The gradients are the first draw from the workload's seed (so they equal
    ``workload(name)`` matrix for matrix), the parameters the second draw.
    Returns (G, W, dtype) as lists of float32 arrays holding the exact input
    values.
    """
    shapes, dtype, sigma, seed = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    G = [gaussian(rng, s, sigma, dtype) for s in shapes]
    W = [gaussian(rng, s, sigma, dtype) for s in shapes]
    return G, W, dtype


def signed_selection(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """One entry of +-1 per row of the short side, in distinct columns; else 0.

    Exact in bf16 and fp16.  Its rows (or columns) are orthonormal.
    """
    m, n = min(rows, cols), max(rows, cols)
    X = np.zeros((m, n), np.float32)
    cols_ = rng.permutation(n)[:m]
    X[np.arange(m), cols_] = rng.choice(np.array([-1.0, 1.0], np.float32), size=m)
    return X if rows <= cols else X.T.copy()


def permuted_blocks(rng: np.random.Generator, rows: int, cols: int, nblocks: int,
                    sigma: float, dtype: str):
    """A matrix Pr . blockdiag(B_1..B_k) . Pc with Gaussian blocks.

    Returns (M, row_perm, col_perm, row_slices, col_slices): ``M[r, c]`` is
    nonzero only where row_perm[r] and col_perm[c] fall in the same block.
    Block k occupies rows row_slices[k] and columns col_slices[k] of the
    unpermuted block-diagonal matrix D, and M = D[row_perm][:, col_perm].
    """
    rb = np.linspace(0, rows, nblocks + 1).astype(int)
    cb = np.linspace(0, cols, nblocks + 1).astype(int)
    D = np.zeros((rows, cols), np.float32)
    rs, cs = [], []
    for k in range(nblocks):
        r0, r1, c0, c1 = rb[k], rb[k + 1], cb[k], cb[k + 1]
        D[r0:r1, c0:c1] = gaussian(rng, (r1 - r0, c1 - c0), sigma, dtype)
        rs.append(slice(r0, r1))
        cs.append(slice(c0, c1))
    rp = rng.permutation(rows)
    cp = rng.permutation(cols)
    return D[rp][:, cp].copy(), rp, cp, rs, cs
