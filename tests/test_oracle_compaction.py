"""Pins of the compaction oracle (oracle/compaction.py) against what its
definition fixes: a hand-worked example, simultaneous-read semantics, the
attention it preserves, paged = contiguous, and the skip rules."""
import numpy as np
import pytest

import oracle
from speculative_decode_verify_mla_amd import synth


def _cache(rows, seed=0):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 1 << 16, size=(rows, 512), dtype=np.uint16)
    r = rng.integers(0, 1 << 16, size=(rows, 64), dtype=np.uint16)
    return c, r


def test_worked_example():
    # T = 4 draft slots after a 6-token prefix (kv_len 10); drafts 1 and 3 accepted:
    # row 6 <- row 7, row 7 <- row 9; rows 0..5 and 8, 9 unchanged; new length 8.
    c, r = _cache(10)
    c2, r2, lens = oracle.compact_kv(c, r, np.array([10]), np.array([[1, 3, -1, -1]]),
                                     np.array([2]), 4, kv_seq_stride=10)
    exp_c = c.copy()
    exp_c[6], exp_c[7] = c[7], c[9]
    exp_r = r.copy()
    exp_r[6], exp_r[7] = r[7], r[9]
    assert np.array_equal(c2, exp_c) and np.array_equal(r2, exp_r)
    assert lens.tolist() == [8]


def test_moves_read_every_source_first():
    # accepted 1, 2, 3 shifts the run down by one: row 7 receives the ORIGINAL row 8
    c, r = _cache(10, 1)
    c2, _, lens = oracle.compact_kv(c, r, np.array([10]), np.array([[1, 2, 3, 0]]),
                                    np.array([3]), 4, kv_seq_stride=10)
    assert np.array_equal(c2[6:9], c[7:10]) and np.array_equal(c2[9], c[9])
    assert lens.tolist() == [9]


def test_identity_path_changes_only_lengths():
    c, r = _cache(40, 2)
    acc = np.tile(np.arange(8), (2, 1))
    c2, r2, lens = oracle.compact_kv(c, r, np.array([20, 17]), acc, np.array([5, 8]), 8,
                                     kv_seq_stride=20)
    assert np.array_equal(c2, c) and np.array_equal(r2, r)
    assert lens.tolist() == [17, 17]


def test_attention_over_compacted_cache_equals_masked_original():
    """A query over prefix + accepted drafts sees the same keys before and after."""
    spec = synth.Spec("cmp", B=1, T=8, H=4, layout="contig", prefix=50)
    w = synth.generate(spec, seed=3)
    parents = synth.random_tree_parents(np.random.default_rng(5), 8)
    node = 6
    path = []
    while node >= 0:
        path.append(node)
        node = parents[node]
    path = path[::-1]  # root-to-node: increasing draft indices
    acc = np.full((1, 8), -1)
    acc[0, :len(path)] = path
    c2, r2, lens = oracle.compact_kv(w.c_kv, w.k_rope, w.kv_lens, acc, np.array([len(path)]), 8,
                                     kv_seq_stride=w.kv_seq_stride)
    P = int(w.kv_lens[0]) - 8
    f = synth.bf16_bits_to_f64
    q_lat, q_rope = f(w.q_lat[0, 0]), f(w.q_rope[0, 0])
    before = np.concatenate([np.arange(P), P + np.asarray(path)])
    o1, l1 = oracle.attend(q_lat, q_rope, f(w.c_kv[before]), f(w.k_rope[before]), w.scale)
    after = np.arange(int(lens[0]))
    o2, l2 = oracle.attend(q_lat, q_rope, f(c2[after]), f(r2[after]), w.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_paged_equals_contiguous():
    rng = np.random.default_rng(7)
    B, T, page = 3, 6, 64
    lens = np.array([100, 64 * 3 + 6, 7])
    stride = 256
    c, r = _cache(B * stride, 8)
    acc = np.stack([np.sort(rng.choice(T, size=T, replace=False)) for _ in range(B)])
    nacc = np.array([3, 6, 2])
    c_ref, r_ref, l_ref = oracle.compact_kv(c, r, lens, acc, nacc, T, kv_seq_stride=stride)
    # the same logical sequences stored in permuted 64-row pages
    pages_per = stride // page
    perm = rng.permutation(B * pages_per)
    pt = perm.reshape(B, pages_per)
    cp = np.zeros_like(c)
    rp = np.zeros_like(r)
    for b in range(B):
        for k in range(pages_per):
            cp[pt[b, k] * page:(pt[b, k] + 1) * page] = c[b * stride + k * page:b * stride + (k + 1) * page]
            rp[pt[b, k] * page:(pt[b, k] + 1) * page] = r[b * stride + k * page:b * stride + (k + 1) * page]
    c_p, r_p, l_p = oracle.compact_kv(cp, rp, lens, acc, nacc, T, page_table=pt, page_size=page)
    assert np.array_equal(l_p, l_ref)
    for b in range(B):
        for k in range(pages_per):
            sl = slice(b * stride + k * page, b * stride + (k + 1) * page)
            ps = slice(pt[b, k] * page, (pt[b, k] + 1) * page)
            assert np.array_equal(c_p[ps], c_ref[sl]) and np.array_equal(r_p[ps], r_ref[sl])


@pytest.mark.parametrize("case", ["bad_index", "too_many", "short_sequence", "absent_page"])
def test_skip_rules(case):
    c, r = _cache(64, 9)
    T = 4
    if case == "bad_index":      # draft indices outside [0, T) move nothing
        c2, _, lens = oracle.compact_kv(c, r, np.array([20]), np.array([[5, -2, 2, 9]]),
                                        np.array([4]), T, kv_seq_stride=64)
        exp = c.copy()
        exp[18] = c[18]  # i=2 <- a=2: a no-op move
        assert np.array_equal(c2, exp) and lens.tolist() == [20]
    elif case == "too_many":     # num_accepted is clamped to T
        c2, _, lens = oracle.compact_kv(c, r, np.array([20]), np.array([[0, 1, 2, 3]]),
                                        np.array([99]), T, kv_seq_stride=64)
        assert np.array_equal(c2, c) and lens.tolist() == [20]
    elif case == "short_sequence":  # kv_len < T: draft positions below 0 do not exist
        c2, _, lens = oracle.compact_kv(c, r, np.array([2]), np.array([[2, 3, 0, 0]]),
                                        np.array([2]), T, kv_seq_stride=64)
        # P = -2: move 0 (dst -2) skipped; move 1: dst -1 skipped
        assert np.array_equal(c2, c) and lens.tolist() == [0]
    else:                         # a page-table hole: moves touching it are skipped
        pt = np.array([[0, -1]])
        c2, _, lens = oracle.compact_kv(c, r, np.array([66]), np.array([[3, 0, 0, 0]]),
                                        np.array([1]), T, page_table=pt, page_size=64)
        # P = 62, move 0: src 65 is in the absent page -> skipped
        assert np.array_equal(c2, c) and lens.tolist() == [63]
