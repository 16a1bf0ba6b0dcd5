"""Pure-Python brute force for tiny inputs — TEST INFRASTRUCTURE ONLY.

One query head at a time, every sum with math.fsum: score every visible key,
subtract the max, exponentiate, normalise, weight the latent rows ("The Shared
Memory Ceiling", section "Technical Deep Dive: Why Shared Memory Matters").
It exists to pin ``oracle.definition`` independently of numpy's matrix
products; it never runs on anything but a handful of rows.
"""
from __future__ import annotations

import math


def attend_one(q_lat, q_rope, keys_lat, keys_rope, scale):
    """q_lat [512], q_rope [64] (sequences of floats); keys_* lists of rows. -> (out list, lse)."""
    n = len(keys_lat)
    if n == 0:
        return [0.0] * len(q_lat), -math.inf
    scores = []
    for p in range(n):
        dot = math.fsum(float(a) * float(c) for a, c in zip(q_lat, keys_lat[p]))
        dot_r = math.fsum(float(a) * float(c) for a, c in zip(q_rope, keys_rope[p]))
        scores.append(float(scale) * math.fsum([dot, dot_r]))
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    l = math.fsum(w)
    out = [math.fsum(w[p] * float(keys_lat[p][d]) for p in range(n)) / l for d in range(len(q_lat))]
    return out, m + math.log(l)


def visible(kv_len, T, t, mask_row):
    prefix = kv_len - T
    vis = [p for p in range(max(prefix, 0))]
    for j in range(T):
        ok = (j <= t) if mask_row is None else (int(mask_row[j]) != 0)
        if ok and 0 <= prefix + j < kv_len:
            vis.append(prefix + j)
    return vis


def verify(q_lat, q_rope, lookup, kv_lens, T, tree_mask=None, indices=None, scale=1.0):
    """Brute-force verify (dense when ``indices`` is None, sparse otherwise).

    ``lookup(b, p)`` returns (c_kv row, k_rope row) for logical position p of
    sequence b, or None when that key's row does not exist (the key is then not
    attended). Returns nested lists out[b][t][h][d] and lse[b][t][h].
    """
    B = len(q_lat)
    out, lse = [], []
    for b in range(B):
        ob, lb = [], []
        for t in range(T):
            if indices is None:
                pos = visible(int(kv_lens[b]), T, t, None if tree_mask is None else tree_mask[b][t])
            else:
                pos = [int(i) for i in indices[b][t] if 0 <= int(i) < int(kv_lens[b])]
            rows = [r for r in (lookup(b, p) for p in pos) if r is not None]
            kl = [r[0] for r in rows]
            kr = [r[1] for r in rows]
            ot, lt = [], []
            for h in range(len(q_lat[b][t])):
                o, s = attend_one(q_lat[b][t][h], q_rope[b][t][h], kl, kr, scale)
                ot.append(o)
                lt.append(s)
            ob.append(ot)
            lb.append(lt)
        out.append(ob)
        lse.append(lb)
    return out, lse
