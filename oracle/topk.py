"""Top-k index selection, the plain definition. TEST INFRASTRUCTURE ONLY.

"The SMEM Ceiling", section "The Problem Space: Sparse Decode on Blackwell":
during decode each token attends only to a sparse set of earlier tokens that
an index-selection (top-k) step picks. Only the selection itself is built
here (the scores that a trained indexer would produce are inputs):

    for each row r with n_r = row_lens[r] candidate positions (all of the row
    when row_lens is None) and k_r = min(k, n_r):
        order positions p < n_r by (score[r, p] descending, p ascending), where
        scores compare by the IEEE-754 total order of float32 restricted to
        numbers (-0.0 < +0.0; -inf lowest) and every NaN ranks below every
        number;
        take the first k_r positions, sort them ascending, pad with -1 to k.

The tie rule makes the selected set unique; ascending order is the order the
sparse attention call expects its index lists in.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def order_key(scores: np.ndarray) -> np.ndarray:
    """uint64 keys whose natural order is the ranking order of float32 scores."""
    bits = np.asarray(scores, dtype=np.float32).view(np.uint32).astype(np.uint64)
    neg = (bits >> 31) == 1
    key = np.where(neg, (~bits) & 0xFFFFFFFF, bits | 0x80000000)
    return np.where(np.isnan(np.asarray(scores, dtype=np.float32)), 0, key)


def select_topk(scores: np.ndarray, k: int, row_lens: Optional[np.ndarray] = None) -> np.ndarray:
    """scores [R, L] float32 -> indices [R, k] int32 (ascending, -1 padded)."""
    scores = np.asarray(scores, dtype=np.float32)
    R, L = scores.shape
    out = np.full((R, k), -1, dtype=np.int32)
    for r in range(R):
        n = L if row_lens is None else int(min(max(int(row_lens[r]), 0), L))
        kk = min(k, n)
        if kk == 0:
            continue
        key = order_key(scores[r, :n])
        pos = np.arange(n)
        # lexsort sorts by its last key first: inverted score key ascending (= score
        # descending), then position ascending
        ranked = np.lexsort((pos, np.uint64(0xFFFFFFFF) - key))
        out[r, :kk] = np.sort(ranked[:kk])
    return out
