"""Per-head projections around absorbed MLA attention. TEST INFRASTRUCTURE ONLY.

Attention over the shared MLA latent ("The Shared Memory Ceiling", section
"The Broader Context: Building a Custom sm_120 Verify Kernel") works in the
512-wide latent space. A head's query enters it through that head's key
up-projection and its output leaves it through the value up-projection:

    q_lat[m, h, :]  = q_nope[m, h, :] . W_UK[h]      W_UK[h]: [128, 512]
    o_head[m, h, :] = out_lat[m, h, :] . W_UV[h]     W_UV[h]: [512, 128]

Both are y[m, h, :] = x[m, h, :] . W[h]; computed here in fp64 with one matrix
product per head (a library primitive used as a step).
"""
from __future__ import annotations

import numpy as np


def head_project(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x [M, H, K], w [H, K, N] -> y [M, H, N] in float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    M, H, K = x.shape
    assert w.shape[:2] == (H, K)
    y = np.empty((M, H, w.shape[2]))
    for h in range(H):
        y[:, h, :] = x[:, h, :] @ w[h]
    return y
