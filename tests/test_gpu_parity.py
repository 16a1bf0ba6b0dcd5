"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: |out - oracle|_inf <= 1e-2 (bf16 output) and |lse - oracle|_inf <= 1e-3.
Every case prints its name, seed and shape before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import speculative_decode_verify_mla_amd as mv
from speculative_decode_verify_mla_amd import synth
from speculative_decode_verify_mla_amd.synth import Spec, generate
from tests._util import run_oracle, oracle_inputs

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3


def _announce(tag, w):
    print(f"[case] {tag} seed={w.seed} B={w.B} T={w.T} H={w.H} layout={w.layout} "
          f"kv_lens={w.kv_lens.tolist()[:8]} topk={w.topk}", flush=True)


def _dev(w):
    from tests._gpu import DeviceWorkload
    return DeviceWorkload(w)


def _check(out, lse, ref_out, ref_lse, tag=""):
    assert np.isfinite(out).all(), f"{tag}: non-finite output"
    assert np.isfinite(lse).all(), f"{tag}: non-finite lse"
    e_out = np.abs(out - ref_out).max()
    e_lse = np.abs(lse - ref_lse).max()
    rel = math.sqrt(((out - ref_out) ** 2).mean() / max(((ref_out) ** 2).mean(), 1e-300))
    print(f"   {tag}: max|dout|={e_out:.3e} max|dlse|={e_lse:.3e} rel_rms(out)={rel:.3e}", flush=True)
    assert e_out <= OUT_TOL, f"{tag}: out error {e_out}"
    assert e_lse <= LSE_TOL, f"{tag}: lse error {e_lse}"


SMALL = [
    Spec("contig_ragged_rows", B=2, T=5, H=40, layout="contig", prefix=[300, 777]),
    Spec("contig_chain_h16", B=1, T=4, H=16, layout="contig", prefix=1000, tree="chain",
         pass_null_mask=True),
    Spec("contig_t64", B=1, T=64, H=8, layout="contig", prefix=200),
    Spec("contig_t1", B=3, T=1, H=64, layout="contig", prefix=[5, 64, 4000]),
    Spec("paged_small", B=3, T=8, H=64, layout="paged", prefix=[100, 1000, 3000]),
    Spec("paged_p128", B=2, T=3, H=32, layout="paged", prefix=[700, 190], page_size=128),
    # ragged batches: the device split plan gives long sequences many splits,
    # short ones one (written directly), and a sequence with no prefix at all
    Spec("contig_skewed", B=4, T=3, H=64, layout="contig", prefix=[0, 9000, 40, 700]),
    Spec("paged_skewed", B=6, T=4, H=32, layout="paged", prefix=[5000, 1, 130, 2500, 64, 12000]),
    Spec("sparse_small", B=4, T=2, H=64, layout="sparse", cache_len=5000, topk=300),
    Spec("sparse_h32_k70", B=2, T=3, H=32, layout="sparse", cache_len=900, topk=70),
    Spec("sparse_paged", B=2, T=2, H=64, layout="sparse", cache_len=3000, topk=200,
         paged_sparse=True),
    # groups of at most 32 rows: one wave computes, three only load
    Spec("paged_t2_h16", B=3, T=2, H=16, layout="paged", prefix=[50, 900, 4100]),
    Spec("contig_t1_h8", B=2, T=1, H=8, layout="contig", prefix=[129, 3000]),
    Spec("sparse_paged_h16", B=2, T=2, H=16, layout="sparse", cache_len=2000, topk=150,
         paged_sparse=True),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_small_parity(gpu_lib, spec, splits):
    w = generate(spec, seed=7)
    _announce(f"{spec.name} splits={splits}", w)
    ref = run_oracle(w)
    d = _dev(w)
    d.run(num_splits=splits)
    _check(*d.results(), *ref, tag=spec.name)


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5, 6])
def test_config_parity(gpu_lib, i):
    w = synth.config(i)
    _announce(f"config{i}", w)
    d = _dev(w)
    d.run()
    out, lse = d.results()
    ref = run_oracle(w)
    _check(out, lse, *ref, tag=f"config{i}")


def test_paged_poison_does_not_leak(gpu_lib):
    spec = Spec("poison", B=3, T=8, H=64, layout="paged", prefix=[100, 1000, 2500])
    w = generate(spec, seed=11, poison=True)
    _announce("paged poison", w)
    d = _dev(w)
    d.run()
    _check(*d.results(), *run_oracle(w), tag="poison")


def test_contig_poison_past_kv_len(gpu_lib):
    spec = Spec("ragged_poison", B=3, T=4, H=64, layout="contig", prefix=[70, 1500, 300])
    w = generate(spec, seed=12, poison=True)
    _announce("contig poison", w)
    d = _dev(w)
    d.run()
    _check(*d.results(), *run_oracle(w), tag="contig_poison")


def test_single_key_is_exact(gpu_lib):
    """kv_len = 1, T = 1: out equals the c_kv row bit for bit; lse is the lone score."""
    spec = Spec("one", B=1, T=1, H=64, layout="contig", prefix=0)
    w = generate(spec, seed=13)
    _announce("single key", w)
    d = _dev(w)
    d.run()
    out, lse = d.results()
    row = synth.bf16_bits_to_f64(w.c_kv[0])
    assert np.array_equal(out[0, 0], np.broadcast_to(row, out[0, 0].shape))
    _check(out, lse, *run_oracle(w), tag="single")


def test_uniform_scores_give_mean(gpu_lib):
    spec = Spec("uni", B=1, T=6, H=64, layout="contig", prefix=333)
    w = generate(spec, seed=14)
    w.q_lat[:] = 0
    w.q_rope[:] = 0
    _announce("uniform", w)
    d = _dev(w)
    d.run()
    out, lse = d.results()
    ref_out, ref_lse = run_oracle(w)
    _check(out, lse, ref_out, ref_lse, tag="uniform")
    P = int(w.kv_lens[0]) - w.T
    for t in range(w.T):
        n = P + int(w.tree_mask[0, t].sum())
        assert np.abs(lse[0, t] - math.log(n)).max() < 1e-5


def test_splits_agree(gpu_lib):
    spec = Spec("splits", B=1, T=8, H=64, layout="contig", prefix=3000)
    w = generate(spec, seed=15)
    _announce("splits agree", w)
    d = _dev(w)
    res = []
    for s in (1, 2, 3, 7, 0):
        d.run(num_splits=s)
        res.append(d.results())
    ref = run_oracle(w)
    for o, l in res:
        _check(o, l, *ref, tag="split")
        assert np.abs(l - res[0][1]).max() < 2e-4


def test_paged_equals_contiguous_bitwise(gpu_lib):
    """Split boundaries are logical positions, so paging must not change a single bit."""
    spec = Spec("pg", B=2, T=8, H=64, layout="paged", prefix=[900, 2000])
    w = generate(spec, seed=16)
    _announce("paged vs contiguous", w)
    d = _dev(w)
    d.run(num_splits=4)
    o_p, l_p = d.results()
    stride = int(w.kv_lens.max())
    c = np.zeros((w.B * stride, 512), np.uint16)
    k = np.zeros((w.B * stride, 64), np.uint16)
    for b in range(w.B):
        for p in range(int(w.kv_lens[b])):
            r = int(w.page_table[b, p // 64]) * 64 + p % 64
            c[b * stride + p], k[b * stride + p] = w.c_kv[r], w.k_rope[r]
    import dataclasses
    wc = dataclasses.replace(w, layout="contig", c_kv=c, k_rope=k, kv_rows=w.B * stride,
                             kv_seq_stride=stride, page_table=None, page_size=0,
                             spec=dataclasses.replace(spec, layout="contig"))
    dc = _dev(wc)
    dc.run(num_splits=4)
    o_c, l_c = dc.results()
    assert np.array_equal(o_p, o_c) and np.array_equal(l_p, l_c)


def test_sparse_arange_matches_dense(gpu_lib):
    """Sparse indices 0..kv_len-1 select the same keys as the dense call: the
    two outputs agree to one bf16 rounding of the largest |out| and the lse to
    1e-5, and each meets the bar against the oracle."""
    spec = Spec("dense1", B=2, T=1, H=64, layout="contig", prefix=[1000, 1500])
    w = generate(spec, seed=17)
    _announce("sparse arange vs dense", w)
    d = _dev(w)
    d.run(num_splits=1)
    o_d, l_d = d.results()
    K = int(w.kv_lens.max())
    idx = np.full((2, 1, K), -1, np.int32)
    for b in range(2):
        idx[b, 0, : w.kv_lens[b]] = np.arange(w.kv_lens[b])
    d.indices = torch.from_numpy(idx).to(d.device)
    import dataclasses
    d.w = dataclasses.replace(w, layout="sparse", indices=idx, topk=K)
    d.run(num_splits=1)
    o_s, l_s = d.results()
    assert np.abs(o_s - o_d).max() <= 2 ** -8 * max(np.abs(o_d).max(), 1e-3)
    assert np.abs(l_s - l_d).max() < 1e-5
    ref_out, ref_lse = run_oracle(w)
    _check(o_d, l_d, ref_out, ref_lse, tag="dense")
    _check(o_s, l_s, ref_out, ref_lse, tag="sparse arange")


def test_deterministic(gpu_lib):
    w = synth.config(2)
    _announce("determinism", w)
    d = _dev(w)
    d.run()
    a = d.results()
    d.run()
    b = d.results()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_phases_equal_one_call(gpu_lib):
    spec = Spec("ph", B=2, T=4, H=64, layout="contig", prefix=[2000, 4000])
    w = generate(spec, seed=18)
    _announce("phases", w)
    d = _dev(w)
    d.run(num_splits=5)
    a = d.results()
    d.out.zero_()
    d.lse.zero_()
    d.run(num_splits=5, phase=mv.binding.PHASE_PARTIAL)
    d.run(num_splits=5, phase=mv.binding.PHASE_COMBINE)
    b = d.results()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_late_large_score_takes_exact_second_pass(gpu_lib):
    """A key far past the first tile scores ~100 nats above the rest: the result is
    that key's row (argmax limit), reached through the split's exact second pass."""
    spec = Spec("argmax", B=1, T=2, H=64, layout="contig", prefix=900)
    w = generate(spec, seed=19)
    j = 700
    kv = synth.bf16_bits_to_f32(w.c_kv[j])
    # q = c * c_kv[j] for every head of token 0: score about c*|c_kv[j]|^2*scale
    c = 100.0 / (float(kv.astype(np.float64) @ kv) * w.scale)
    w.q_lat[0, 0, :] = synth.f32_to_bf16_bits(np.broadcast_to(c * kv, (w.H, 512)).copy())
    _announce("late large score", w)
    d = _dev(w)
    for s in (1, 0):
        d.run(num_splits=s)
        out, lse = d.results()
        ref_out, ref_lse = run_oracle(w)
        _check(out, lse, ref_out, ref_lse, tag=f"argmax splits={s}")
        assert np.abs(out[0, 0] - synth.bf16_bits_to_f64(w.c_kv[j])).max() < 1e-2


def test_sparse_late_large_score_takes_exact_second_pass(gpu_lib):
    """The sparse path's second pass: the key at position 450 of token 0's index
    list (8th 64-key tile) scores ~100 nats above the rest, more than the 2^96
    a tile may grow past the exponent reference set by the split's first tile.
    The split runs again, its first tile's indices fetched anew; the result is
    that key's row, for one split, the automatic plan and three splits."""
    spec = Spec("argmax_sparse", B=1, T=2, H=64, layout="sparse", cache_len=3000, topk=600)
    w = generate(spec, seed=31)
    j = int(w.indices[0, 0, 450])
    m = int(np.searchsorted(w.row_ids, j))
    assert w.row_ids[m] == j
    kv = synth.bf16_bits_to_f32(w.c_kv[m])
    c = 100.0 / (float(kv.astype(np.float64) @ kv) * w.scale)
    w.q_lat[0, 0, :] = synth.f32_to_bf16_bits(np.broadcast_to(c * kv, (w.H, 512)).copy())
    _announce("sparse late large score", w)
    ref_out, ref_lse = run_oracle(w)
    d = _dev(w)
    for s in (1, 0, 3):
        d.run(num_splits=s)
        out, lse = d.results()
        _check(out, lse, ref_out, ref_lse, tag=f"sparse argmax splits={s}")
        assert np.abs(out[0, 0] - synth.bf16_bits_to_f64(w.c_kv[m])).max() < 1e-2


def test_ragged_batch_with_empty_sequence(gpu_lib):
    """kv_lens of 0 in a batch: that sequence's rows are out = 0, lse = -inf; the
    device split plan still balances the others and they match the oracle."""
    spec = Spec("ragged_empty", B=4, T=4, H=64, layout="paged", prefix=[3000, 200, 8000, 50])
    w = generate(spec, seed=16)
    w.kv_lens[1] = 0
    _announce("ragged with an empty sequence", w)
    d = _dev(w)
    ref_out, ref_lse = run_oracle(w)
    for splits in (0, 2):
        d.run(num_splits=splits)
        out, lse = d.results()
        assert np.all(out[1] == 0.0) and np.all(lse[1] == -np.inf)
        assert np.all(ref_lse[1] == -np.inf)
        keep = [0, 2, 3]
        _check(out[keep], lse[keep], ref_out[keep], ref_lse[keep], tag=f"ragged_empty s={splits}")


def test_ragged_batch_equals_single_sequences(gpu_lib):
    """Each sequence of a skewed batch gives the same result as when it is run
    alone (the split plan only changes how keys are grouped, within tolerance)."""
    spec = Spec("skew", B=3, T=2, H=64, layout="contig", prefix=[6000, 100, 2000])
    w = generate(spec, seed=17)
    _announce("ragged vs single", w)
    d = _dev(w)
    d.run()
    out, lse = d.results()
    ref_out, ref_lse = run_oracle(w)
    _check(out, lse, ref_out, ref_lse, tag="skew batch")
    for b in range(w.B):
        sub = generate(Spec(f"skew{b}", B=1, T=2, H=64, layout="contig",
                            prefix=int(w.kv_lens[b]) - w.T), seed=17)
        # same rows as sequence b of the batch
        sub.q_lat[:] = w.q_lat[b:b + 1]
        sub.q_rope[:] = w.q_rope[b:b + 1]
        r0 = b * w.kv_seq_stride
        n = int(w.kv_lens[b])
        sub.c_kv[:n] = w.c_kv[r0:r0 + n]
        sub.k_rope[:n] = w.k_rope[r0:r0 + n]
        sub.tree_mask[:] = w.tree_mask[b:b + 1]
        ds = _dev(sub)
        ds.run()
        o1, l1 = ds.results()
        assert np.abs(l1[0] - lse[b]).max() < 2e-4
        assert np.abs(o1[0] - out[b]).max() <= OUT_TOL


@pytest.mark.parametrize("layout", ["contig", "paged"])
def test_batch_wider_than_a_wave(gpu_lib, layout):
    """More sequences than a wave has lanes (80 > 64): the device split plan
    scans the batch lane-strided; ragged lengths, including an empty prefix and
    prefixes shorter and longer than one tile, all match the oracle."""
    rng = np.random.default_rng(21)
    prefix = [int(x) for x in rng.integers(0, 600, size=80)]
    prefix[3] = 0
    prefix[70] = 2500  # one long sequence among many short ones
    spec = Spec(f"wide_{layout}", B=80, T=2, H=16, layout=layout, prefix=prefix)
    w = generate(spec, seed=21)
    _announce(f"batch of 80, {layout}", w)
    ref_out, ref_lse = run_oracle(w)
    d = _dev(w)
    for splits in (0, 3):
        d.run(num_splits=splits)
        _check(*d.results(), ref_out, ref_lse, tag=f"wide {layout} s={splits}")


def test_sparse_leading_padding(gpu_lib):
    """Sorted index lists whose -1 padding comes first and fills whole 64-key
    tiles: rows see their first visible key only after several empty tiles (the
    exponent reference is set mid-split), and with several splits the first
    ones hold no key at all (weight 0 in the combine)."""
    spec = Spec("sparse_lead", B=3, T=2, H=64, layout="sparse", cache_len=4000, topk=400)
    w = generate(spec, seed=23)
    idx = w.indices.copy()
    drop = {(0, 0): 150, (0, 1): 330, (1, 0): 64, (2, 1): 399}  # entries replaced by -1
    for (b, t), n in drop.items():
        idx[b, t, :n] = -1
        idx[b, t] = np.sort(idx[b, t])
    import dataclasses
    w = dataclasses.replace(w, indices=idx)
    _announce("sparse with leading padding", w)
    ref_out, ref_lse = run_oracle(w)
    d = _dev(w)
    for splits in (0, 1, 3, 7):
        d.run(num_splits=splits)
        _check(*d.results(), ref_out, ref_lse, tag=f"sparse_lead s={splits}")


def test_absent_pages_and_out_of_range_indices(gpu_lib):
    """Page-table entries that are negative or point past the pool read as
    absent keys, and sparse indices at or past kv_lens[b] select nothing; the
    rows they would have named hold finite values, so a stray read shows."""
    import dataclasses
    spec = Spec("bad_pages", B=3, T=4, H=64, layout="paged", prefix=[700, 1500, 300])
    w = generate(spec, seed=24)
    pt = w.page_table.copy()
    pool = w.kv_rows // w.page_size
    pt[0, 2] = -1
    pt[1, 5] = pool + 7
    pt[1, 20] = -1
    w = dataclasses.replace(w, page_table=pt)
    _announce("absent pages", w)
    ref = run_oracle(w)
    d = _dev(w)
    for splits in (0, 1, 3):
        d.run(num_splits=splits)
        _check(*d.results(), *ref, tag=f"absent pages s={splits}")

    spec = Spec("sparse_short", B=3, T=2, H=64, layout="sparse", cache_len=5000, topk=300)
    w = generate(spec, seed=25)
    kv = w.kv_lens.copy()
    kv[0], kv[2] = 3000, 1234  # indices at or past these select nothing
    idx = w.indices.copy()
    idx[1, 0, -5:-1] = [5000, 5001, 7000, 1 << 30]  # past kv_len (5000); the list stays unsorted
    w = dataclasses.replace(w, kv_lens=kv, indices=idx)
    _announce("sparse indices past kv_lens", w)
    ref = run_oracle(w)
    d = _dev(w)
    for splits in (0, 1, 3):
        d.run(num_splits=splits)
        _check(*d.results(), *ref, tag=f"sparse past kv_len s={splits}")

    spec = Spec("sparse_paged_bad", B=2, T=2, H=64, layout="sparse", cache_len=3000, topk=200,
                paged_sparse=True)
    w = generate(spec, seed=26)
    pt = w.page_table.copy()
    pt[0, 3] = -1
    pt[1, 10] = w.kv_rows // w.page_size + 1
    w = dataclasses.replace(w, page_table=pt)
    _announce("sparse over absent pages", w)
    ref = run_oracle(w)
    d = _dev(w)
    for splits in (0, 3):
        d.run(num_splits=splits)
        _check(*d.results(), *ref, tag=f"sparse absent pages s={splits}")


def test_late_spikes_in_every_split_full_size(gpu_lib):
    """Workload 3 at full size with, in the last tile of every split, a key
    scoring ~40 nats above the rest for every row: every split's streaming
    softmax must move its exponent reference, and the result still matches the
    oracle."""
    import speculative_decode_verify_mla_amd as mv
    w = synth.config(3)
    tiles = -(-int(w.kv_lens[0]) // 64)
    dims = mv.binding.make_dims(batch=1, num_q=w.T, num_heads=w.H, max_kv_len=w.max_kv_len,
                                kv_rows=w.kv_rows, kv_seq_stride=w.kv_seq_stride)
    n = int(mv.plan(dims).num_splits)
    w, keys = synth.plant_late_spikes(w, [s * tiles // n for s in range(n + 1)], 40.0)
    assert len(keys) == n
    _announce("late spikes in every split", w)
    d = _dev(w)
    d.run()
    out, lse = d.results()
    ref_out, ref_lse = run_oracle(w)
    _check(out, lse, ref_out, ref_lse, tag="spiked config3")
    assert ref_lse.min() > 35.0  # the spikes dominate every row


def test_reference_rises_several_times_in_a_split(gpu_lib):
    """Keys scoring ~30, ~55 and ~80 nats above the rest at growing positions:
    each lies more than 2^32 above the exponent reference of the tiles before
    it, so the reference rises three times within one split (an exact
    power-of-two rescale of the accumulators each time), and with several
    splits some rise once; every result matches the oracle."""
    spec = Spec("three_rises", B=1, T=2, H=64, layout="contig", prefix=3000)
    w = generate(spec, seed=27)
    w.q_rope[..., 0] = synth.f32_to_bf16_bits(np.ones(w.q_rope[..., 0].shape, np.float32))
    for p, nats in ((200, 30.0), (900, 55.0), (2000, 80.0)):
        w.k_rope[p, 0] = synth.f32_to_bf16_bits(np.array([nats / w.scale], np.float32))[0]
    _announce("reference rises three times", w)
    ref_out, ref_lse = run_oracle(w)
    assert ref_lse.min() > 75.0
    d = _dev(w)
    for s in (1, 0, 3):
        d.run(num_splits=s)
        _check(*d.results(), ref_out, ref_lse, tag=f"three rises splits={s}")


@pytest.mark.parametrize("nats", [30.0, 100.0])
def test_partial_last_tile_large_score(gpu_lib, nats):
    """The sequence's last tile holds 18 keys (prefix 2,960, T = 2; the other
    46 read as absent). A key of that tile scores `nats` above the rest: 30
    raises the exponent reference at the tile's end, 100 sends the split to its
    second pass. Splits 1, automatic, 3 and 47 (one tile each: the last split
    is the partial tile alone) all match the oracle."""
    spec = Spec("partial_last_tile", B=1, T=2, H=64, layout="contig", prefix=2960)
    w = generate(spec, seed=33)
    assert int(w.kv_lens[0]) % 64 == 18
    w.q_rope[..., 0] = synth.f32_to_bf16_bits(np.ones(w.q_rope[..., 0].shape, np.float32))
    w.k_rope[2950, 0] = synth.f32_to_bf16_bits(np.array([nats / w.scale], np.float32))[0]
    _announce(f"partial last tile, {nats:g} nats", w)
    ref_out, ref_lse = run_oracle(w)
    assert ref_lse.min() > nats - 5.0
    d = _dev(w)
    for s in (1, 0, 3, 47):
        d.run(num_splits=s)
        _check(*d.results(), ref_out, ref_lse, tag=f"partial last tile {nats:g} splits={s}")


@pytest.mark.parametrize("layout", ["contig", "sparse"])
def test_many_splits_combine(gpu_lib, layout):
    """Groups of more than 32 splits (one sequence, or sparse tokens) combine in
    the wide kernel (every split's loads of 32 rows x 8 dims in flight at once,
    8 split groups summed in LDS). Split counts of 33..79 and a sequence
    shorter than the planned length (its last planned splits hold no key) all
    match the oracle."""
    import dataclasses
    if layout == "contig":
        spec = Spec("many_splits", B=1, T=2, H=64, layout="contig", prefix=5000)
        w = generate(spec, seed=28)
        _announce("wide combine, one sequence", w)
        d = _dev(w)
        ref = run_oracle(w)
        for splits in (33, 60, 65, 79):
            d.run(num_splits=splits)
            _check(*d.results(), *ref, tag=f"many splits s={splits}")
        # the same cache and plan, but the sequence is only 3000 keys long
        w2 = dataclasses.replace(w, kv_lens=np.array([3000], np.int32))
        d2 = _dev(w2)
        d2.w = dataclasses.replace(w2, max_kv_len=w.max_kv_len)
        ref2 = run_oracle(w2)
        d2.run(num_splits=79)
        _check(*d2.results(), *ref2, tag="many splits, shorter sequence")
    else:
        spec = Spec("many_splits_sparse", B=2, T=2, H=64, layout="sparse", cache_len=9000,
                    topk=3000)
        w = generate(spec, seed=29)
        _announce("wide combine, sparse", w)
        d = _dev(w)
        ref = run_oracle(w)
        for splits in (33, 47):
            d.run(num_splits=splits)
            _check(*d.results(), *ref, tag=f"sparse many splits s={splits}")


@pytest.mark.parametrize("layout", ["contig", "batch", "sparse"])
def test_combine_batches_of_17_to_24_splits(gpu_lib, layout):
    """The one-stage combine's 24-split body (groups of 17..24 splits) for all
    three record layouts: one sequence, a batch (records found through the
    split kernel's map) and sparse tokens."""
    if layout == "contig":
        w = generate(Spec("c24_one", B=1, T=3, H=64, layout="contig", prefix=1400), seed=34)
        splits = (17, 20, 22)
    elif layout == "batch":
        # a requested count cuts every sequence into chunks of one tile: 22 and 12 splits
        w = generate(Spec("c24_batch", B=2, T=3, H=40, layout="contig", prefix=[1400, 700]), seed=35)
        splits = (22,)
    else:
        # 22 index tiles per token, one per split
        w = generate(Spec("c24_sparse", B=2, T=2, H=64, layout="sparse", cache_len=4000, topk=1408),
                     seed=36)
        splits = (22,)
    _announce(f"combine of 17..24 splits, {layout}", w)
    ref = run_oracle(w)
    d = _dev(w)
    for s in splits:
        d.run(num_splits=s)
        _check(*d.results(), *ref, tag=f"{layout} splits={s}")
