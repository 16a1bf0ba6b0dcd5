"""Pins for the fp64 oracle (CPU only).

The pages print no worked numbers for the attention itself, so the oracle is
pinned by things other than itself: pure-Python brute force, a textbook
attention routine (torch SDPA in float64), closed forms (single key, uniform
scores, a two-key case with known weights), and invariants (split/stream
consistency, logit shift, head and page permutations, chain = tree with chain
parents, sparse arange = dense, argmax limit). Each check is chosen so that a
dropped rope term, a wrong sign, a shifted mask index or a transposed operand
fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce
from speculative_decode_verify_mla_amd import synth
from speculative_decode_verify_mla_amd.synth import Spec, generate, bf16_bits_to_f64
from tests._util import run_oracle, oracle_inputs

DL, DR = 512, 64


def _lookup_fn(w):
    d = oracle_inputs(w)
    c, k = d["c_kv"], d["k_rope"]
    if w.row_ids is not None:
        where = {int(r): i for i, r in enumerate(w.row_ids)}
    else:
        where = None

    def phys(b, p):
        if w.page_table is not None:
            return int(w.page_table[b][p // w.page_size]) * w.page_size + p % w.page_size
        return b * w.kv_seq_stride + p

    def lookup(b, p):
        r = phys(b, p)
        i = r if where is None else where[r]
        return c[i].tolist(), k[i].tolist()

    return lookup


TINY = [
    Spec("tiny_chain", B=1, T=3, H=2, layout="contig", prefix=5, tree="chain", pass_null_mask=True),
    Spec("tiny_tree", B=2, T=4, H=3, layout="contig", prefix=[7, 11], tree="random"),
    Spec("tiny_paged", B=2, T=2, H=2, layout="paged", prefix=[9, 3], page_size=4),
    Spec("tiny_sparse", B=2, T=2, H=2, layout="sparse", cache_len=20, topk=6),
    Spec("tiny_sparse_paged", B=1, T=2, H=2, layout="sparse", cache_len=16, topk=5,
         paged_sparse=True, page_size=4),
]


@pytest.mark.parametrize("spec", TINY, ids=lambda s: s.name)
def test_oracle_matches_bruteforce(spec):
    w = generate(spec, seed=101)
    out, lse = run_oracle(w)
    d = oracle_inputs(w)
    bo, bl = bruteforce.verify(
        d["q_lat"].tolist(), d["q_rope"].tolist(), _lookup_fn(w), w.kv_lens, w.T,
        tree_mask=None if w.mask_for_kernel is None else w.mask_for_kernel.tolist(),
        indices=None if w.indices is None else w.indices.tolist(), scale=w.scale)
    np.testing.assert_allclose(out, np.asarray(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.asarray(bl), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_matches_torch_sdpa_fp64(seed):
    """Library special case: SDPA with K=[c_kv|k_rope], V=c_kv and the boolean tree mask."""
    spec = Spec("sdpa", B=1, T=6, H=4, layout="contig", prefix=37)
    w = generate(spec, seed=seed)
    out, lse = run_oracle(w)
    d = oracle_inputs(w)
    kv_len = int(w.kv_lens[0])
    K = torch.from_numpy(np.concatenate([d["c_kv"][:kv_len], d["k_rope"][:kv_len]], axis=1))
    V = torch.from_numpy(d["c_kv"][:kv_len])
    Q = torch.from_numpy(np.concatenate([d["q_lat"][0], d["q_rope"][0]], axis=2))  # [T,H,576]
    allowed = torch.ones(w.T, kv_len, dtype=torch.bool)
    allowed[:, kv_len - w.T:] = torch.from_numpy(w.tree_mask[0].astype(bool))
    for h in range(w.H):
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[:, h][None, None], K[None, None], V[None, None],
            attn_mask=allowed[None, None], scale=w.scale)[0, 0]
        np.testing.assert_allclose(out[0, :, h], ref.numpy(), rtol=0, atol=1e-12)
        scores = (Q[:, h] @ K.T) * w.scale
        scores = scores.masked_fill(~allowed, -math.inf)
        np.testing.assert_allclose(lse[0, :, h], torch.logsumexp(scores, dim=1).numpy(),
                                   rtol=0, atol=1e-12)


def test_single_key_gives_that_row():
    """kv_len = 1, T = 1: out is the c_kv row exactly and lse is the lone score."""
    rng = np.random.default_rng(5)
    ql, qr = rng.standard_normal((1, 1, 3, DL)), rng.standard_normal((1, 1, 3, DR))
    c, k = rng.standard_normal((1, DL)), rng.standard_normal((1, DR))
    out, lse = oracle.verify_dense(ql, qr, c, k, np.array([1]), None, 0.3, kv_seq_stride=1)
    for h in range(3):
        assert np.array_equal(out[0, 0, h], c[0])
        s = 0.3 * (ql[0, 0, h] @ c[0] + qr[0, 0, h] @ k[0])
        assert abs(lse[0, 0, h] - s) < 1e-12


def test_uniform_scores_give_mean_and_log_count():
    """q = 0: out = mean of the visible rows, lse = ln |V|, with |V| = P + depth(t) + 1."""
    spec = Spec("uni", B=2, T=5, H=2, layout="contig", prefix=[13, 4])
    w = generate(spec, seed=9)
    d = oracle_inputs(w)
    ql = np.zeros_like(d["q_lat"])
    qr = np.zeros_like(d["q_rope"])
    out, lse = oracle.verify_dense(ql, qr, d["c_kv"], d["k_rope"], w.kv_lens, w.tree_mask, w.scale,
                                   kv_seq_stride=w.kv_seq_stride)
    for b in range(w.B):
        P = int(w.kv_lens[b]) - w.T
        for t in range(w.T):
            depth, j = 0, int(w.parents[b, t])
            while j >= 0:
                depth, j = depth + 1, int(w.parents[b, j])
            n = P + depth + 1
            vis = list(range(P)) + [P + j for j in range(w.T) if w.tree_mask[b, t, j]]
            assert len(vis) == n
            mean = d["c_kv"][b * w.kv_seq_stride + np.asarray(vis)].mean(axis=0)
            for h in range(w.H):
                np.testing.assert_allclose(out[b, t, h], mean, atol=1e-12, rtol=0)
                assert abs(lse[b, t, h] - math.log(n)) < 1e-12


def test_two_key_closed_form():
    """Scores 0 and ln 3 (scale 1): weights 1/4 and 3/4, lse = ln 4."""
    q_lat = np.zeros((1, DL))
    q_rope = np.zeros((1, DR))
    q_rope[0, 0] = math.log(3.0)
    k_lat = np.zeros((2, DL))
    k_lat[0, 0], k_lat[1, 1] = 8.0, -4.0
    k_rope = np.zeros((2, DR))
    k_rope[1, 0] = 1.0  # key 1 scores ln 3, key 0 scores 0
    out, lse = oracle.attend(q_lat, q_rope, k_lat, k_rope, 1.0)
    assert abs(lse[0] - math.log(4.0)) < 1e-15
    assert abs(out[0, 0] - 2.0) < 1e-15 and abs(out[0, 1] + 3.0) < 1e-15
    assert np.all(out[0, 2:] == 0)


@pytest.mark.parametrize("bounds_fn", [
    lambda n: [0, n],
    lambda n: [0, 1, n],
    lambda n: [0, n // 3, n // 3, 2 * n // 3, n],  # includes an empty chunk
    lambda n: list(range(0, n, 7)) + [n],
])
def test_chunked_combine_equals_full(bounds_fn):
    rng = np.random.default_rng(3)
    n = 50
    ql, qr = rng.standard_normal((4, DL)), rng.standard_normal((4, DR))
    kl, kr = rng.standard_normal((n, DL)), rng.standard_normal((n, DR))
    o, l = oracle.attend(ql, qr, kl, kr, 0.07)
    oc, lc = oracle.attend_chunked(ql, qr, kl, kr, 0.07, bounds_fn(n))
    np.testing.assert_allclose(oc, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lc, l, atol=1e-12, rtol=0)


@pytest.mark.parametrize("tile", [1, 8, 64, 1000])
def test_streaming_equals_full(tile):
    rng = np.random.default_rng(4)
    n = 70
    ql, qr = rng.standard_normal((3, DL)), rng.standard_normal((3, DR))
    kl, kr = rng.standard_normal((n, DL)), rng.standard_normal((n, DR))
    kl[40] *= 4.0  # a late, large score forces a rescale
    o, l = oracle.attend(ql, qr, kl, kr, 0.2)
    os_, ls = oracle.attend_streaming(ql, qr, kl, kr, 0.2, tile)
    np.testing.assert_allclose(os_, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(ls, l, atol=1e-12, rtol=0)


def test_rope_shift_invariance():
    """With k_rope[:, 0] = 1, adding c to q_rope[..., 0] keeps out and adds scale*c to lse."""
    spec = Spec("shift", B=1, T=4, H=3, layout="contig", prefix=20)
    w = generate(spec, seed=12)
    d = oracle_inputs(w)
    d["k_rope"][:, 0] = 1.0
    a = oracle.verify_dense(d["q_lat"], d["q_rope"], d["c_kv"], d["k_rope"], w.kv_lens,
                            w.tree_mask, w.scale, kv_seq_stride=w.kv_seq_stride)
    qr2 = d["q_rope"].copy()
    qr2[..., 0] += 2.5
    b = oracle.verify_dense(d["q_lat"], qr2, d["c_kv"], d["k_rope"], w.kv_lens,
                            w.tree_mask, w.scale, kv_seq_stride=w.kv_seq_stride)
    np.testing.assert_allclose(b[0], a[0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(b[1], a[1] + w.scale * 2.5, atol=1e-12, rtol=0)
    # and the rope term is live: changing q_rope elsewhere moves the result
    qr3 = d["q_rope"].copy()
    qr3[..., 1] += 2.5
    c = oracle.verify_dense(d["q_lat"], qr3, d["c_kv"], d["k_rope"], w.kv_lens,
                            w.tree_mask, w.scale, kv_seq_stride=w.kv_seq_stride)
    assert np.abs(c[1] - a[1]).max() > 1e-3


def test_head_permutation():
    spec = Spec("perm", B=1, T=3, H=5, layout="contig", prefix=17)
    w = generate(spec, seed=13)
    d = oracle_inputs(w)
    a_out, a_lse = run_oracle(w)
    perm = np.array([3, 0, 4, 1, 2])
    out, lse = oracle.verify_dense(d["q_lat"][:, :, perm], d["q_rope"][:, :, perm], d["c_kv"],
                                   d["k_rope"], w.kv_lens, w.tree_mask, w.scale,
                                   kv_seq_stride=w.kv_seq_stride)
    np.testing.assert_array_equal(out, a_out[:, :, perm])
    np.testing.assert_array_equal(lse, a_lse[:, :, perm])


def test_paged_equals_contiguous():
    """The paged workload's logical contents, laid out contiguously, give the same result."""
    spec = Spec("pg", B=3, T=4, H=2, layout="paged", prefix=[70, 5, 130], page_size=64)
    w = generate(spec, seed=14)
    out_p, lse_p = run_oracle(w)
    d = oracle_inputs(w)
    stride = int(w.kv_lens.max())
    c = np.zeros((w.B * stride, DL))
    k = np.zeros((w.B * stride, DR))
    for b in range(w.B):
        for p in range(int(w.kv_lens[b])):
            r = int(w.page_table[b, p // 64]) * 64 + p % 64
            c[b * stride + p], k[b * stride + p] = d["c_kv"][r], d["k_rope"][r]
    out_c, lse_c = oracle.verify_dense(d["q_lat"], d["q_rope"], c, k, w.kv_lens, w.tree_mask,
                                       w.scale, kv_seq_stride=stride)
    np.testing.assert_array_equal(out_p, out_c)
    np.testing.assert_array_equal(lse_p, lse_c)


def test_chain_mask_equals_chain_parents_and_null():
    spec = Spec("ch", B=1, T=5, H=2, layout="contig", prefix=9, tree="chain")
    w = generate(spec, seed=15)
    vis = synth.tree_visibility(synth.chain_parents(5))
    assert np.array_equal(vis, np.tril(np.ones((5, 5), dtype=np.uint8)))
    a = run_oracle(w, mask_override=w.tree_mask)
    b = run_oracle(w, mask_override=None)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_mask_is_applied_as_given():
    """Hiding one draft key changes exactly the tokens that saw it."""
    spec = Spec("mk", B=1, T=4, H=2, layout="contig", prefix=6, tree="chain")
    w = generate(spec, seed=16)
    m = w.tree_mask.copy()
    a = run_oracle(w, mask_override=m)
    m2 = m.copy()
    m2[0, 3, 1] = 0
    b = run_oracle(w, mask_override=m2)
    assert np.array_equal(a[0][0, :3], b[0][0, :3])
    assert np.abs(a[1][0, 3] - b[1][0, 3]).min() > 0


def test_sparse_arange_equals_dense_t1():
    spec = Spec("dense1", B=2, T=1, H=3, layout="contig", prefix=[30, 12])
    w = generate(spec, seed=17)
    d = oracle_inputs(w)
    dense = oracle.verify_dense(d["q_lat"], d["q_rope"], d["c_kv"], d["k_rope"], w.kv_lens,
                                w.tree_mask, w.scale, kv_seq_stride=w.kv_seq_stride)
    K = int(w.kv_lens.max())
    idx = np.full((2, 1, K), -1, dtype=np.int32)
    for b in range(2):
        idx[b, 0, : w.kv_lens[b]] = np.arange(w.kv_lens[b])
    sparse = oracle.verify_sparse(d["q_lat"], d["q_rope"], d["c_kv"], d["k_rope"], w.kv_lens,
                                  idx, w.scale, kv_seq_stride=w.kv_seq_stride)
    np.testing.assert_allclose(sparse[0], dense[0], atol=1e-13, rtol=0)
    np.testing.assert_allclose(sparse[1], dense[1], atol=1e-13, rtol=0)


def test_sparse_subset_equals_gathered_dense():
    spec = Spec("sp", B=1, T=2, H=2, layout="sparse", cache_len=40, topk=9)
    w = generate(spec, seed=18)
    out, lse = run_oracle(w)
    d = oracle_inputs(w)
    order = {int(r): i for i, r in enumerate(w.row_ids)}
    for t in range(2):
        rows = [order[int(p)] for p in w.indices[0, t]]
        o, l = oracle.attend(d["q_lat"][0, t], d["q_rope"][0, t], d["c_kv"][rows],
                             d["k_rope"][rows], w.scale)
        np.testing.assert_allclose(out[0, t], o, atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse[0, t], l, atol=1e-13, rtol=0)


def test_argmax_limit():
    """A query aligned with one key at a large gain returns that key's row."""
    rng = np.random.default_rng(19)
    kl, kr = rng.standard_normal((30, DL)), rng.standard_normal((30, DR))
    ql = (50.0 * kl[11])[None]
    qr = np.zeros((1, DR))
    out, _ = oracle.attend(ql, qr, kl, kr, 1.0)
    np.testing.assert_allclose(out[0], kl[11], atol=1e-9, rtol=0)


def test_empty_visible_set():
    out, lse = oracle.attend(np.ones((2, DL)), np.ones((2, DR)), np.zeros((0, DL)),
                             np.zeros((0, DR)), 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_sparse_out_of_range_indices_select_nothing():
    spec = Spec("oor", B=1, T=1, H=2, layout="sparse", cache_len=30, topk=5)
    w = generate(spec, seed=20)
    out, lse = run_oracle(w)
    idx2 = w.indices.copy()
    idx2 = np.concatenate([idx2, np.array([[[-1, 30, 1 << 20]]], dtype=np.int32)], axis=2)
    d = oracle_inputs(w)
    out2, lse2 = oracle.verify_sparse(d["q_lat"], d["q_rope"], d["c_kv"], d["k_rope"], w.kv_lens,
                                      idx2, w.scale, kv_seq_stride=w.kv_seq_stride,
                                      row_ids=w.row_ids)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def _with_bad_pages(w, bad):
    """Copy of paged workload w whose page_table entries (b, i) in ``bad`` are
    replaced: -1 (no page) or a page index past the pool."""
    import dataclasses
    pt = w.page_table.copy()
    pool_pages = w.kv_rows // w.page_size
    for (b, i), kind in bad.items():
        pt[b, i] = -1 if kind == "neg" else pool_pages + 3
    return dataclasses.replace(w, page_table=pt)


def test_absent_pages_match_bruteforce():
    """Keys on a page-table entry that is negative or past the pool are not
    attended: the oracle against brute force told the same rule per key."""
    w = generate(Spec("tiny_bad_pages", B=2, T=2, H=2, layout="paged", prefix=[13, 6],
                      page_size=4), seed=61)
    w = _with_bad_pages(w, {(0, 1): "neg", (0, 3): "past", (1, 0): "neg"})
    d = oracle_inputs(w)
    got_out, got_lse = oracle.verify_dense(d["q_lat"], d["q_rope"], d["c_kv"], d["k_rope"],
                                           w.kv_lens, w.tree_mask, w.scale,
                                           page_table=w.page_table, page_size=w.page_size,
                                           kv_rows=w.kv_rows)
    c, k = d["c_kv"], d["k_rope"]

    def lookup(b, p):
        r = int(w.page_table[b][p // w.page_size]) * w.page_size + p % w.page_size
        if r < 0 or r >= w.kv_rows:
            return None
        return c[r].tolist(), k[r].tolist()

    ref_out, ref_lse = bruteforce.verify(d["q_lat"].tolist(), d["q_rope"].tolist(), lookup,
                                         w.kv_lens, w.T, tree_mask=w.tree_mask, scale=w.scale)
    assert np.abs(got_out - np.array(ref_out)).max() < 1e-12
    assert np.abs(got_lse - np.array(ref_lse)).max() < 1e-12


def test_absent_prefix_page_equals_sparse_over_the_rest():
    """A one-token dense call whose second prefix page is absent equals a sparse
    call over exactly the remaining visible positions (an independent route to
    the same key set)."""
    import dataclasses
    w = generate(Spec("t1_bad_page", B=1, T=1, H=3, layout="paged", prefix=[11], page_size=4),
                 seed=62)
    w = _with_bad_pages(w, {(0, 1): "neg"})
    d = oracle_inputs(w)
    out_d, lse_d = oracle.verify_dense(d["q_lat"], d["q_rope"], d["c_kv"], d["k_rope"], w.kv_lens,
                                       w.tree_mask, w.scale, page_table=w.page_table,
                                       page_size=w.page_size, kv_rows=w.kv_rows)
    keep = np.array([p for p in range(int(w.kv_lens[0])) if p // 4 != 1], dtype=np.int32)
    out_s, lse_s = oracle.verify_sparse(d["q_lat"], d["q_rope"], d["c_kv"], d["k_rope"], w.kv_lens,
                                        keep[None, None, :], w.scale, page_table=w.page_table,
                                        page_size=w.page_size, kv_rows=w.kv_rows)
    assert np.abs(out_d - out_s).max() < 1e-12 and np.abs(lse_d - lse_s).max() < 1e-12
    # and differs from the call that reads all 12 keys
    full = dataclasses.replace(w, page_table=generate(
        Spec("t1_bad_page", B=1, T=1, H=3, layout="paged", prefix=[11], page_size=4),
        seed=62).page_table)
    assert np.abs(run_oracle(full)[1] - lse_d).max() > 1e-6


def test_sparse_absent_rows_are_skipped():
    """Sparse over a paged cache: an index on an absent page selects nothing,
    like an index past kv_len; the rest are attended (brute force)."""
    w = generate(Spec("sp_bad_page", B=1, T=2, H=2, layout="sparse", cache_len=16, topk=6,
                      paged_sparse=True, page_size=4), seed=63)
    import dataclasses
    pt = w.page_table.copy()
    pt[0, 2] = -1
    idx = w.indices.copy()
    idx[0, 1, -1] = 40  # past kv_len
    w = dataclasses.replace(w, page_table=pt, indices=idx)
    d = oracle_inputs(w)
    got_out, got_lse = run_oracle(w)
    where = {int(r): i for i, r in enumerate(w.row_ids)}

    def lookup(b, p):
        r = int(pt[b][p // 4]) * 4 + p % 4
        if r < 0 or r >= w.kv_rows:
            return None
        return d["c_kv"][where[r]].tolist(), d["k_rope"][where[r]].tolist()

    ref_out, ref_lse = bruteforce.verify(d["q_lat"].tolist(), d["q_rope"].tolist(), lookup,
                                         w.kv_lens, w.T, indices=idx.tolist(), scale=w.scale)
    assert np.abs(got_out - np.array(ref_out)).max() < 1e-12
    assert np.abs(got_lse - np.array(ref_lse)).max() < 1e-12
