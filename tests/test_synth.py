"""Seeded generator checks (CPU): structure, reproducibility and bf16 encoding."""
import math
import os

import numpy as np
import pytest
import torch

from speculative_decode_verify_mla_amd import synth
from speculative_decode_verify_mla_amd.synth import Spec, generate


def test_bf16_rounding_matches_torch():
    """RNE float32 -> bf16, pinned to torch's own conversion (ties, subnormals, infinities)."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(10000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 10000),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 1e-40, -3e-39], dtype=np.float32),
        # exact ties: low 16 bits 0x8000 with even and odd upper halves
        np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32).view(np.float32),
    ])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_nan_stays_nan():
    assert np.isnan(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


@pytest.mark.parametrize("i", [1, 2, 4])
def test_reproducible(i):
    a, b = synth.config(i), synth.config(i)
    for f in ("q_lat", "q_rope", "kv_lens", "tree_mask"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    np.testing.assert_array_equal(a.c_kv[:100], b.c_kv[:100])


def test_tree_parents_and_masks():
    rng = np.random.default_rng(3)
    for T in (1, 2, 16, 64):
        p = synth.random_tree_parents(rng, T)
        assert p[0] == -1
        assert all(-1 <= p[i] <= i - 1 for i in range(1, T))
        vis = synth.tree_visibility(p)
        for i in range(T):
            assert vis[i, i] == 1
            assert not vis[i, i + 1:].any()  # only ancestors (lower index) and self
            # ancestor-closed: whatever i sees, its parent's set is contained
            if p[i] >= 0:
                assert np.all(vis[i] >= vis[p[i]])
                assert vis[i].sum() == vis[p[i]].sum() + 1
            else:
                assert vis[i].sum() == 1


def test_config_shapes():
    w1 = synth.config(1)
    assert w1.q_lat.shape == (1, 4, 16, 512) and w1.c_kv.shape == (132, 512)
    assert w1.kv_lens.tolist() == [132] and w1.mask_for_kernel is None
    assert np.array_equal(w1.tree_mask[0], np.tril(np.ones((4, 4), np.uint8)))
    w2 = synth.config(2)
    assert w2.q_lat.shape == (1, 16, 64, 512) and w2.kv_lens.tolist() == [4096 + 16]
    assert w2.scale == pytest.approx(1 / math.sqrt(192), rel=1e-7)


def test_paged_structure():
    w = synth.config(4)
    assert w.B == 8 and w.T == 8 and w.H == 64 and w.page_size == 64
    prefix = w.kv_lens - w.T
    assert np.all(prefix >= 1024) and np.all(prefix < 32768)
    n_pages = (w.kv_lens + 63) // 64
    used = np.concatenate([w.page_table[b, : n_pages[b]] for b in range(w.B)])
    assert sorted(used.tolist()) == list(range(int(n_pages.sum())))  # a permutation of the pool
    for b in range(w.B):
        assert np.all(w.page_table[b, n_pages[b]:] == -1)
    assert w.kv_rows == int(n_pages.sum()) * 64


def test_sparse_structure():
    spec = Spec("sp", B=3, T=2, H=8, layout="sparse", cache_len=5000, topk=300)
    w = generate(spec, seed=1)
    assert w.indices.shape == (3, 2, 300)
    for b in range(3):
        for t in range(2):
            idx = w.indices[b, t]
            assert np.all(np.diff(idx) > 0) and idx[0] >= 0 and idx[-1] < 5000
    # exactly the selected rows are materialised
    expect = sorted({b * 5000 + int(i) for b in range(3) for i in np.unique(w.indices[b])})
    assert w.row_ids.tolist() == expect


def test_poison_rows_are_nan_and_unread_region():
    spec = Spec("pp", B=2, T=3, H=2, layout="paged", prefix=[70, 5], page_size=64)
    w = generate(spec, seed=2, poison=True)
    vals = synth.bf16_bits_to_f32(w.c_kv)
    assert np.isnan(vals[w.poison_rows]).all()
    for b in range(2):
        for p in range(int(w.kv_lens[b])):
            r = int(w.page_table[b, p // 64]) * 64 + p % 64
            assert not np.isnan(vals[r]).any()


def test_naive_guard_matches_the_pages():
    """bench.py's naive-kernel column ("fits" / "n/a" in the prefix sweep) uses the
    pages' guard arithmetic: tests/golden/naive_score_row.txt holds the printed
    formula's constants and the values they give."""
    import bench
    path = os.path.join(os.path.dirname(__file__), "golden", "naive_score_row.txt")
    g = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            g[k] = int(v)
    assert bench.naive_score_row_bytes(0) == (g["dl"] + g["dr"]) * 4
    assert 65536 * 4 == g["score_row_only_bytes_at_65536"]
    assert bench.naive_row_fits(g["largest_kv_len_within_guard"], g["guard_bytes"])
    assert not bench.naive_row_fits(g["first_kv_len_over_guard"], g["guard_bytes"])
    # on MI355X (160 KiB of LDS per CU) the same row fits up to 40,384 keys
    assert bench.naive_row_fits(40384, 163840) and not bench.naive_row_fits(40385, 163840)
