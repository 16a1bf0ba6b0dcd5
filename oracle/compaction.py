"""Post-verify KV compaction, the plain definition. TEST INFRASTRUCTURE ONLY.

"The Shared Memory Ceiling", section "The Broader Context: Building a Custom
sm_120 Verify Kernel", names the plan as a verify kernel plus "defrag" and says
nothing more about the second step. The plainest reading, taken here: once the
verifier has accepted a path of draft tokens, the cache rows of the accepted
drafts are moved to the front of the draft region, in path order, so that the
next decoding step sees prefix + accepted tokens as one contiguous run.

For sequence b with T draft slots, prefix P_b = kv_lens[b] - T, n_b =
num_accepted[b] clamped to [0, T] and accepted draft indices a_0 .. a_{n_b-1}:

    for i < n_b:   row(P_b + i)  <-  row(P_b + a_i)      (c_kv and k_rope)
    new_kv_lens[b] = max(P_b + n_b, 0)

kv_lens[b] is first clamped to [0, max_kv_len] (when given), as the kernels do.

All sources are read before any destination is written, so overlapping moves
(a_i >= i always holds for a root-to-node path, but any order is allowed) are
well defined. A move whose source or destination position is outside
[0, kv_lens[b]), whose draft index is outside [0, T), or whose physical row is
absent (page-table entry < 0 or past the cache) is skipped.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _phys(b: int, p: int, kv_seq_stride: int, page_table: Optional[np.ndarray], page_size: int,
          kv_rows: int) -> int:
    """Physical row of logical position p of sequence b, or -1 when absent."""
    if page_table is None:
        r = b * kv_seq_stride + p
    else:
        page = int(page_table[b, p // page_size])
        if page < 0:
            return -1
        r = page * page_size + p % page_size
    return r if 0 <= r < kv_rows else -1


def compact_kv(c_kv: np.ndarray, k_rope: np.ndarray, kv_lens: np.ndarray, accepted: np.ndarray,
               num_accepted: np.ndarray, T: int, *, kv_seq_stride: int = 0,
               page_table: Optional[np.ndarray] = None, page_size: int = 0,
               max_kv_len: Optional[int] = None):
    """Returns (c_kv', k_rope', new_kv_lens); the inputs are not modified.

    c_kv [rows, 512], k_rope [rows, 64] (any dtype, copied bit for bit),
    kv_lens [B], accepted [B, T] draft indices, num_accepted [B].
    """
    c_out = np.array(c_kv, copy=True)
    r_out = np.array(k_rope, copy=True)
    B = len(kv_lens)
    rows = c_kv.shape[0]
    new_lens = np.zeros(B, dtype=np.int32)
    for b in range(B):
        kv = int(kv_lens[b])
        kv = max(kv, 0)
        if max_kv_len is not None:
            kv = min(kv, int(max_kv_len))
        n = min(max(int(num_accepted[b]), 0), T)
        P = kv - T
        moves = []
        for i in range(n):
            a = int(accepted[b, i])
            if not (0 <= a < T):
                continue
            src, dst = P + a, P + i
            if not (0 <= src < kv and 0 <= dst < kv):
                continue
            rs = _phys(b, src, kv_seq_stride, page_table, page_size, rows)
            rd = _phys(b, dst, kv_seq_stride, page_table, page_size, rows)
            if rs < 0 or rd < 0:
                continue
            moves.append((rd, c_kv[rs].copy(), k_rope[rs].copy()))  # read every source first
        for rd, cv, kr in moves:
            c_out[rd] = cv
            r_out[rd] = kr
        new_lens[b] = max(P + n, 0)
    return c_out, r_out, new_lens
